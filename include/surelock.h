/*
 * surelock.h — C ABI of the SureLock decoding step on one AMD MI355X (gfx950).
 *
 * SureLock (arXiv 2602.06412, "Stopping Computation for Converged Tokens in
 * Masked Diffusion-LM Decoding") keeps, at every step of a masked diffusion LM
 * sampler, an active set A_t of positions that are still computed and a locked
 * set L_t of positions that are skipped.  A locked position no longer computes
 * its Q projection or FFN; its K/V stay in a per-layer cache so the active
 * queries still attend to it, and its posterior stays frozen (zhaoyang97
 * Paper-Notes, 方法详解: 整体框架 and 永久锁定机制).  A position locks once the step
 * divergence KL(p_t || p_{t-1}) is at most eps, optionally AND-ed with the
 * confidence gate 1 - max_v p_t(v) <= q_m (same notes, 锁定判据 and
 * 可选置信度门控).  Attention then costs O(M N d) and the FFN O(M d^2)
 * instead of O(N^2 d) and O(N d^2) (paperdance abstract; gist.science/nl §2,
 * Complexiteitsvermindering).
 *
 * Conventions shared by every entry point
 *  - All pointers are DEVICE pointers unless the comment says "host".  The
 *    caller allocates and owns every buffer, including workspaces; the library
 *    never allocates device memory, never frees, and keeps no pointer after a
 *    call returns.
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream).  The only host synchronisation happens when an `m_tot_host`
 *    pointer is given: the call then waits for the stream and stores the new
 *    active count there.
 *  - Arguments are checked on the host before anything is launched: a NULL
 *    required pointer, a non-positive size, an inconsistent size or an
 *    unsupported shape returns SL_ERR_INVALID / SL_ERR_UNSUPPORTED and launches
 *    nothing.  A failed launch returns SL_ERR_HIP; sl_last_error() gives the
 *    message (per thread).  No exception crosses the ABI.
 *  - Device contents (active lists, offsets) are trusted: an act_idx entry must
 *    lie in [0, N) and be strictly ascending within its sequence, and act_off
 *    must be non-decreasing with act_off[B] == M_tot.  sl_compact produces
 *    exactly such lists.
 *  - Element type: SL_BF16 (bfloat16 bit patterns, 2 bytes) or SL_F32
 *    (4 bytes) for weights, activations, K/V caches and logits; the type is the
 *    storage and MFMA operand type, accumulation is always fp32.
 *  - Active lists: act_idx[M_tot] holds positions within their own sequence
 *    (0..N-1), ascending; sequence b owns rows act_off[b] .. act_off[b+1]-1.
 *    Row m of a compact [M_tot][...] buffer is the active position
 *    (b, act_idx[m]); its row in a full [B*N][...] buffer is b*N + act_idx[m].
 *  - Inputs are assumed finite; NaN propagates and is not checked.
 */
#ifndef SURELOCK_H
#define SURELOCK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SL_OK = 0,
  SL_ERR_INVALID = 1,     /* bad argument: NULL pointer, size <= 0, inconsistent sizes */
  SL_ERR_UNSUPPORTED = 2, /* valid but not supported by these kernels (see each call) */
  SL_ERR_HIP = 3          /* a HIP runtime call or launch failed */
} sl_status;

typedef enum { SL_BF16 = 0, SL_F32 = 1 } sl_dtype;

typedef void* sl_stream; /* hipStream_t */

/* Human-readable name of a status code (static string). */
const char* sl_status_string(sl_status s);
/* Message of the last failing call on this host thread ("" if none). */
const char* sl_last_error(void);
/* Library version string. */
const char* sl_version(void);

/*
 * sl_compact — active set A_t from the lock mask (stream compaction).
 * A_t is every position not in L_t, kept in ascending order per sequence
 * (zhaoyang97 notes, 整体框架: active set vs locked set).
 *   locked   [B*N] uint8, 0 = active, nonzero = locked.
 *   act_idx  [B*N] capacity; receives the M_tot active positions.
 *   act_off  [B+1]; act_off[B] = M_tot.
 *   m_tot_host  host int32* or NULL: if given, the stream is synchronised and
 *               M_tot is stored there.
 * Limits: B >= 1, N >= 1, B*N < 2^31.
 */
sl_status sl_compact(const uint8_t* locked, int B, int N, int32_t* act_idx, int32_t* act_off,
                     int32_t* m_tot_host, sl_stream stream);

/*
 * sl_cache_scatter — write the fresh K/V rows of the active positions into a
 * layer's cache, leaving locked positions' cached rows untouched
 * (zhaoyang97 notes, 永久锁定机制: K^all[L_t] <- C.k[L_t]; gist.science/it §2:
 * K/V cached for every layer).
 *   k_cache, v_cache  [B][N][H][Dh] of `dtype`, updated in place.
 *   k_new, v_new      [M_tot][H][Dh] of `dtype`.
 * Limits: (H*Dh*elem_size) % 16 == 0.
 */
sl_status sl_cache_scatter(int dtype, void* k_cache, void* v_cache, const void* k_new,
                           const void* v_new, const int32_t* act_idx, const int32_t* act_off,
                           int B, int N, int M_tot, int H, int Dh, sl_stream stream);

/*
 * sl_attn_active — bidirectional attention of the M_tot active queries over
 * all N cached keys of their own sequence: o = softmax(q K^T * scale) V per
 * head, no mask.  Locked positions take part through their cached K/V
 * (zhaoyang97 notes, 永久锁定机制; cost O(M N d), paperdance abstract).
 *   q        [M_tot][H][Dh] of `dtype`, RoPE already applied.
 *   k_cache, v_cache [B][N][H][Dh] of `dtype`.
 *   key_excl [B*N] uint8 or NULL, 4-byte aligned: positions with a nonzero
 *            flag are not attended (the "no KV cache" ablation of the notes
 *            page, 消融实验: locked positions cannot be attended; pass the
 *            lock mask).  Every query row must keep at least one key.
 *   out      [M_tot][H*Dh] of `dtype`.
 *   ws       workspace of at least sl_attn_workspace_size(B, N, M_tot, H, Dh)
 *            bytes (any contents; used for split-KV partial results); that
 *            size serves every call with at most M_tot query rows.
 * Limits: Dh in {32, 64, 128}; N % 64 == 0.
 */
sl_status sl_attn_active(int dtype, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* act_off, const uint8_t* key_excl, int B, int N, int M_tot, int H,
                         int Dh, float scale, void* out, void* ws, size_t ws_bytes, sl_stream stream);
size_t sl_attn_workspace_size(int B, int N, int M_tot, int H, int Dh);

/* Lock rule parameters (zhaoyang97 notes, 锁定判据 and 可选置信度门控). */
typedef struct {
  float eps;     /* lock when KL <= eps; eps <= 0 disables locking; eps = +inf drops the KL
                    test (with the gate on: the notes page's confidence-gate-only ablation) */
  float gate_q;  /* quantile m in [0,1] of the gate u <= q_m(u); < 0 disables the gate */
  int mask_id;   /* [MASK] token id excluded from the argmax; -1 = none */
  int have_prev; /* 0 on the first step: no previous posterior, KL = +inf, nothing locks */
} sl_lock_params;

/*
 * sl_kl_lock — the vocabulary pass plus the lock update and compaction.
 * For every active row r (position (b, act_idx[r])):
 *   A = LSE(cur), p = softmax(cur); kl[r] = KL(p || softmax(prev)) (nats,
 *   +inf when have_prev == 0); u[r] = 1 - max_v p(v); lse[r] = A;
 *   argmax[r] = argmax over v != mask_id (lowest id on ties); conf[r] = p(argmax).
 * Then per sequence gate_thr[b] = the floor(m*(M_b-1))-th smallest u of its
 * active rows (lower nearest rank; +inf when the gate is off), and a position
 * locks, permanently, when cand (NULL = every active row) && have_prev &&
 * eps > 0 && kl <= eps && (gate off || u <= gate_thr[b])
 * (zhaoyang97 notes, 锁定判据 / 可选置信度门控 / 永久锁定机制; gist.science/it §2).
 * Finally the new active list is compacted from the updated mask.
 *   logits_cur, logits_prev [B*N][V] of `dtype`; only the active rows are read.
 *   cand     [B*N] uint8 or NULL.
 *   locked   [B*N] uint8, in/out (only 0 -> 1 transitions).
 *   kl, u, lse, conf [M_tot] float; argmax [M_tot] int32 (conf/argmax may be NULL).
 *   lse_pos  [B*N] float or NULL: also receives A at each active position b*N + act_idx[r].
 *   lse_prev [B*N] float or NULL: B = LSE(prev) at each active position, as an earlier call
 *            stored it in its lse_pos for these same previous logits.  The pass then reads
 *            prev only for sum_v p(v) (cur(v) - prev(v)), with KL = that sum - A + B: the
 *            identity the KL is computed from either way, without recomputing the previous
 *            posterior's normaliser (the pass that produced prev already did).  The caller
 *            keeps the pairing (two stores beside two logits buffers, as sl_state does);
 *            a stale lse_prev gives a wrong KL.  Must not alias lse_pos.
 *   gate_thr [B] float or NULL.
 *   new_act_idx [B*N] capacity, new_act_off [B+1] (may alias act_idx / act_off).
 *   ws       at least sl_kl_lock_workspace_size(B, N, M_tot, V) bytes (any contents); that size
 *            serves every call with at most M_tot active rows.
 * Limits: V % 8 == 0 (bf16) or V % 4 == 0 (f32); N <= 65536.
 */
sl_status sl_kl_lock(int dtype, const void* logits_cur, const void* logits_prev, int V,
                     const int32_t* act_idx, const int32_t* act_off, int B, int N, int M_tot,
                     const uint8_t* cand, const sl_lock_params* params, uint8_t* locked,
                     float* kl, float* u, float* lse, int32_t* argmax, float* conf,
                     const float* lse_prev, float* lse_pos, float* gate_thr,
                     int32_t* new_act_idx, int32_t* new_act_off,
                     int32_t* m_tot_host, void* ws, size_t ws_bytes, sl_stream stream);
size_t sl_kl_lock_workspace_size(int B, int N, int M_tot, int V);

/*
 * sl_kl_lock_noalloc — sl_kl_lock for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  Same arguments,
 * results and limits as sl_kl_lock, without ws / ws_bytes: the partial sums of the vocabulary
 * pass go to a 256 KiB device array inside the library (one per GPU, held until the process
 * ends), which covers every size sl_kl_lock accepts.  No allocation, no memset; nothing in the
 * array needs to start at zero.  Calls that overlap on one GPU (two streams at once) share that
 * array and race: serialise them.  Returns SL_ERR_UNSUPPORTED if a size ever needed more scratch.
 */
sl_status sl_kl_lock_noalloc(int dtype, const void* logits_cur, const void* logits_prev, int V,
                             const int32_t* act_idx, const int32_t* act_off, int B, int N, int M_tot,
                             const uint8_t* cand, const sl_lock_params* params, uint8_t* locked,
                             float* kl, float* u, float* lse, int32_t* argmax, float* conf,
                             const float* lse_prev, float* lse_pos, float* gate_thr,
                             int32_t* new_act_idx, int32_t* new_act_off,
                             int32_t* m_tot_host, sl_stream stream);

/*
 * sl_rope_table — cos/sin table of rotary position embeddings (rotate-half
 * form: pair j = (x_j, x_{j+Dh/2}) rotated by pos * theta^(-2j/Dh)), computed
 * on the device in double precision and stored as float pairs.
 *   table [n_pos][Dh/2][2] float (cos, sin).
 */
sl_status sl_rope_table(int n_pos, int head_dim, float theta, float* table, sl_stream stream);

/* Epilogues of sl_gemm. */
typedef enum {
  SL_EPI_QKV_ROPE = 0, /* q -> out0 [M][d]; RoPE on q and k; k, v -> caches out1/out2 at rows b*N+pos */
  SL_EPI_RESIDUAL = 1, /* out0 (fp32 [M][n_out]) += A W^T */
  SL_EPI_SWIGLU = 2,   /* out0 [M][n_out/2] = SiLU(A W0^T) * (A W1^T) */
  SL_EPI_LOGITS = 3    /* out0 rows b*N+pos of a [B*N][n_out] buffer = A W0^T */
} sl_epilogue;

/*
 * sl_gemm — the gathered-row projections of the active rows, C = A W^T with a
 * fused epilogue.  Only the M active rows are multiplied: locked rows skip
 * their Q projection and FFN (zhaoyang97 notes, 永久锁定机制; O(M d^2),
 * gist.science/nl §2).  sl_step calls the same kernels.
 *   A        [M][K] of `dtype` (compact active rows).
 *   w0,w1,w2 [n][K] weights: QKV_ROPE takes wq, wk, wv (n = d each, n_out = 3d);
 *            SWIGLU takes the gate and up matrices (n = n_out/2 each);
 *            RESIDUAL and LOGITS take w0 only (n = n_out).
 *   rope     [>=N][head_dim/2][2] from sl_rope_table (QKV_ROPE only).
 *   act_idx/act_off/B/N map compact rows to positions (QKV_ROPE, LOGITS).
 * Limits: K*elem_size % 128 == 0; n_out % 64 == 0; QKV_ROPE needs d % 128 == 0;
 * M*K*elem_size <= 4 GiB (A rows are addressed with 32-bit offsets).  Beyond
 * them the call returns SL_ERR_UNSUPPORTED and launches nothing.
 */
sl_status sl_gemm(int dtype, int epilogue, const void* A, int M, int K, int n_out, const void* w0,
                  const void* w1, const void* w2, void* out0, void* out1, void* out2,
                  const float* rope, int d, int head_dim, const int32_t* act_idx,
                  const int32_t* act_off, int B, int N, sl_stream stream);

/*
 * sl_gemm_plan — the launch sl_gemm would make for this shape: workgroup tile
 * rows x columns, the split-K factor (the residual epilogue alone splits K) and
 * the load path (*through_registers = 1: both operands' tiles go through vector
 * registers into LDS, used when few rows stream a wide weight matrix; 0: direct
 * global-to-LDS loads), chosen by the library's cost model.  through_registers
 * may be NULL.  Writes nothing on error.  No device work.  sl_step's residual
 * projections may split K differently: there the split-K partial sums go to
 * workspace planes that the fused residual reduce + RMSNorm adds up, which the
 * cost model prices below sl_gemm's fp32 atomics.
 */
sl_status sl_gemm_plan(int dtype, int epilogue, int M, int K, int n_out, int* tile_m, int* tile_n,
                       int* split_k, int* through_registers);

/* One layer's weights, each stored [out_features][in_features] row-major. */
typedef struct {
  const void* wq; /* [d][d] */
  const void* wk; /* [d][d] */
  const void* wv; /* [d][d] */
  const void* wo; /* [d][d] */
  const void* wg; /* [F][d] SwiGLU gate */
  const void* wu; /* [F][d] SwiGLU up */
  const void* wd; /* [d][F] down */
} sl_layer_weights;

typedef struct {
  int dtype;                       /* sl_dtype */
  int n_layers, d, n_heads, head_dim, ffn, vocab;
  float rms_eps;                   /* RMSNorm epsilon (unit gains, no biases) */
  const sl_layer_weights* layers;  /* HOST array [n_layers] of device pointers */
  const void* embed;               /* [V][d] or NULL (then the state gives h_in) */
  const void* lm_head;             /* [V][d] or NULL (then the step stops after the layers) */
  const float* rope;               /* [rope_n][Dh/2][2] from sl_rope_table */
  int rope_n;                      /* >= N */
} sl_model;

typedef struct {
  int B, N;
  int M_tot;             /* host: active rows in act_idx (from the last compaction) */
  int t;                 /* step index: logits[t%2] is written, logits[(t+1)%2] is p_{t-1} */
  int32_t* tok;          /* [B*N] token ids (needed with embed, or with unmask_k > 0) */
  uint8_t* cand;         /* [B*N] lock candidates (unmasked positions) or NULL = all */
  uint8_t* locked;       /* [B*N] lock mask, in/out */
  int32_t* act_idx;      /* [B*N] capacity: A_t in, A_{t+1} out (when locking) */
  int32_t* act_off;      /* [B+1] */
  void* k_cache;         /* [n_layers][B][N][H][Dh] */
  void* v_cache;         /* [n_layers][B][N][H][Dh] */
  const void* h_in;      /* [B*N][d] layer-0 input rows, or NULL to use embed[tok] */
  float* h_out;          /* [M_tot][d] fp32 final hidden rows (residual stream), or NULL */
  void* logits[2];       /* [B*N][V] each: double-buffered posterior store */
  float* kl;             /* [M_tot] per-row statistics of this step (may be NULL when */
  float* u;              /*  lm_head is NULL)                                          */
  float* lse;
  float* conf;
  int32_t* argmax;
  float* gate_thr;       /* [B] or NULL */
  int32_t* lock_step;    /* [B*N] or NULL: step at which each position locked */
  int32_t* m_tot_host;   /* host int32* or NULL: receives M_{t+1} (synchronises) */
  int32_t* t_dev;        /* device int32 or NULL: step index that lock_step records instead of t;
                            the step adds one to it when it runs the lock update */
  int kv_head_major;     /* 0: caches token-major [n_layers][B][N][H][Dh] (a position's K or V row
                            is one run of d elements); 1: head-major [n_layers][B][H][N][Dh] (a
                            head's keys are one run of N * Dh elements).  The cache-layout study of
                            gist.science/nl §5 (optimised cache layouts); sl_attn_active and
                            sl_cache_scatter take token-major caches. */
  float* lse_pos[2];     /* [B*N] float each, or both NULL: per-position LSE store beside logits[2].
                            Step t writes the LSE of each active row's logits to lse_pos[t%2], and
                            from t = 1 on takes the previous posterior's LSE from lse_pos[(t+1)%2]
                            instead of recomputing it from logits[(t+1)%2] (see sl_kl_lock).  Every
                            step that writes logits must then run the vocabulary pass: a step with
                            the LM head and do_lock = 0 is rejected. */
} sl_state;

typedef struct {
  float eps;      /* as sl_lock_params */
  float gate_q;
  int mask_id;
  int do_lock;    /* 0: stop after the logits (no vocabulary pass, no lock) */
  int unmask_k;   /* > 0: sampler unmasks this many [MASK] positions per sequence */
  int no_kv_cache; /* 0: SureLock (locked positions attended through their cached K/V);
                      1: the notes page's "no KV cache" ablation (消融实验): positions
                      locked before this step are not attended */
  int device_m;    /* 0: state->M_tot is the active count (as the last compaction left it).
                      1: the active count stays on the device: every kernel reads act_off[B]
                      and state->M_tot is only an upper bound on it (any earlier step's count
                      serves, since A_t only shrinks), which sizes the grids.  A step can then
                      be enqueued, or captured into a HIP graph and replayed, without the host
                      reading the count back; launches past the live count exit at once. */
  int fuse_head_kl; /* 1: the LM head's epilogue also computes, from the logits it stores, each
                       row's statistics over its column tiles against the previous posterior,
                       so the vocabulary pass does not read the current logits back (the
                       pages' fused-kernel direction, gist.science/nl §5); a short merge pass
                       then finishes the rows.  Used from the second step on (a previous
                       posterior must exist); same results as 0 up to the order of the fp32
                       additions. */
} sl_step_params;

/*
 * sl_step — one whole SureLock iteration:
 *   gather the active rows (embedding of tok, or h_in rows) -> for every layer:
 *   RMSNorm, fused QKV projection + RoPE with the K/V rows scattered into the
 *   layer cache, active-query attention over all N cached rows (over the active
 *   rows only with no_kv_cache), O projection
 *   + residual, RMSNorm, SwiGLU FFN + residual -> final RMSNorm, LM head
 *   writing logits rows b*N+pos of logits[t%2] -> sl_kl_lock against
 *   logits[(t+1)%2] -> optional sampler (the unmask_k most confident [MASK]
 *   positions per sequence take their argmax token and become candidates)
 *   -> compaction of A_{t+1} into act_idx/act_off.
 * Locked rows are never read or written by any stage except as cached K/V
 * (zhaoyang97 notes, 永久锁定机制: posterior frozen, K/V cached; gist.science/it
 * §2: block input frozen, K/V cached for every layer).  A_t within A_{t-1}
 * guarantees logits[(t+1)%2] holds p_{t-1} for every active row.
 *   ws: sl_step_workspace_size(...) bytes (any contents).  A workspace sized for
 *       the first step's M_tot serves every later step (M only shrinks): the size is
 *       the largest any step with at most M_tot rows needs.  Less is
 *       accepted down to the fixed buffers of the step; the O and down projections
 *       then accumulate their split-K partial sums with fp32 atomics instead of the
 *       partial-sum planes (same results up to the order of the additions); below
 *       that the call fails with SL_ERR_INVALID.
 * Limits: d % 128 == 0, ffn % 64 == 0, vocab % 128 == 0, head_dim in {32, 64, 128},
 * n_heads*head_dim == d, N % 64 == 0, N <= 65536, rope_n >= N, and
 * M_tot*max(d, ffn)*elem_size <= 4 GiB (the GEMMs' A operands).
 */
sl_status sl_step(const sl_model* model, sl_state* state, const sl_step_params* params,
                  void* ws, size_t ws_bytes, sl_stream stream);
/* The largest workspace any step with at most M_tot active rows needs.  Not
 * a per-row product: fewer rows can need more (the attention splits its keys,
 * and stores per-split partials, only when few query tiles would idle the chip). */
size_t sl_step_workspace_size(const sl_model* model, int B, int N, int M_tot);
/* The smallest workspace sl_step accepts for every step with at most M_tot active
 * rows: the fixed buffers only (split-K residual projections then use fp32 atomics). */
size_t sl_step_workspace_min(const sl_model* model, int B, int N, int M_tot);

/*
 * Measurement helpers (not part of the SureLock step): the ceilings this chip sustains, which
 * the step's roofline fractions are reported against beside the vendor figures.
 * sl_peak_mfma       `workgroups` x 4 waves, each running `iters` rounds of 4 independent
 *                    v_mfma_f32_32x32x16_bf16 on register operands; sl_peak_mfma_flops gives
 *                    the FLOPs of such a launch.  sink: device float[256], never written in
 *                    practice (it keeps the work alive).
 * sl_peak_stream     streams `bytes` (a multiple of 16) from src with 16-byte non-temporal loads,
 *                    each workgroup over one contiguous range; dst != NULL: copies them there,
 *                    dst == NULL: only reads.  sink as above.
 * sl_peak_gemm_loop  the LDS-to-MFMA loop of a 256 x 256 bf16 GEMM tile alone: `workgroups` x 4
 *                    waves (wave tile 128 x 128) over `tiles` k-tiles of 32, fragments from LDS;
 *                    with_loads != 0 adds the GEMM's per-k-tile direct global-to-LDS loads (from
 *                    src: device memory of at least 1 MiB, L2-resident), their waits and a
 *                    barrier.  sl_peak_gemm_loop_flops gives the FLOPs.  sink as above.
 * sl_peak_mfma_operands  sl_peak_mfma's loop on operands read from `operands` (device memory of
 *                    16 x 256 16-byte chunks, e.g. random bf16 values: the matrix cores' power, and
 *                    the clock the chip holds, depend on the operand bits), eight operand sets per
 *                    lane rotated between consecutive MFMAs; iters a multiple of 8, FLOPs as
 *                    sl_peak_mfma_flops.  clocks (device, 2 x workgroups entries, or NULL): per
 *                    workgroup the shader-clock cycles and the 100 MHz real-time ticks it took.
 * sl_gemm_clocked    sl_gemm (bf16; SL_EPI_SWIGLU with w0, w1, out0, or SL_EPI_LOGITS with w0,
 *                    out0, act_idx, act_off, B, N; the same launch plan) in a variant that records
 *                    per workgroup w < clock_slots, in clocks[4 w .. 4 w + 3]: shader-clock cycles
 *                    and 100 MHz real-time ticks of the workgroup, cycles of its k-tile loop, and the
 *                    K elements it multiplied.  Workgroups past the live rows leave their slots as
 *                    they were (the caller clears them).  Workgroup w of a launch is tile w of
 *                    sl_gemm_plan's grid (K splits: w = split * tiles + tile).
 */
sl_status sl_peak_mfma(int workgroups, int iters, float* sink, sl_stream stream);
double sl_peak_mfma_flops(int workgroups, int iters);
sl_status sl_peak_mfma_operands(int workgroups, int iters, const void* operands, float* sink,
                                unsigned long long* clocks, sl_stream stream);
sl_status sl_gemm_clocked(int epilogue, const void* A, int M, int K, int n_out, const void* w0, const void* w1,
                          void* out0, const int32_t* act_idx, const int32_t* act_off, int B, int N,
                          unsigned long long* clocks, int clock_slots, sl_stream stream);
sl_status sl_peak_stream(const void* src, void* dst, size_t bytes, int workgroups, float* sink, sl_stream stream);
sl_status sl_peak_gemm_loop(int workgroups, int tiles, int with_loads, const void* src, float* sink,
                            sl_stream stream);
double sl_peak_gemm_loop_flops(int workgroups, int tiles);

#ifdef __cplusplus
}
#endif
#endif /* SURELOCK_H */
