// Host-side launchers of the SureLock kernels (internal; the public ABI is include/surelock.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sl {

// Device-resident row count.  Every launcher below takes the row count M_tot
// from the host; when m_dev is given, M_tot is only a capacity (an upper bound
// that sizes grids, workspaces and strides) and the kernels process the first
// min(M_tot, *m_dev) rows, reading the count from device memory.  A step can
// then be launched, or captured in a graph, without the host knowing how many
// rows the previous step left active.
__device__ __forceinline__ int rows_live(int M_cap, const int32_t* m_dev) {
  return m_dev ? min(M_cap, *m_dev) : M_cap;
}

// Parameters of the lock / sampler tail that runs after the vocabulary pass.
struct TailParams {
  int B, N, M_tot;
  const int32_t* m_dev;  // device row count (M_tot is then a capacity), or NULL
  int32_t* t_dev;        // device step index for lock_step, advanced after the step, or NULL (use t)
  float eps, gate_q;
  int mask_id, have_prev;
  int t;                 // step index recorded in lock_step
  const int32_t* act_idx;
  const int32_t* act_off;
  const uint8_t* cand;   // may be NULL
  uint8_t* locked;
  int32_t* lock_step;    // may be NULL
  const float* kl;
  const float* u;
  const float* conf;     // may be NULL when unmask_k == 0
  const int32_t* argmax; // may be NULL when unmask_k == 0
  float* gate_thr;       // may be NULL
  int32_t* tok;          // sampler (unmask_k > 0)
  uint8_t* cand_out;     // sampler marks unmasked positions as candidates
  int unmask_k;
  int32_t* new_act_idx;
  int32_t* new_act_off;
};

struct KLRowParams {
  const void* cur;
  const void* prev;
  int V;
  float* kl;
  float* u;
  float* lse;
  int32_t* argmax;  // may be NULL
  float* conf;      // may be NULL
  const float* lse_prev;  // [B*N] per position: LSE of `prev` from the pass that produced it, or NULL
  float* lse_pos;         // [B*N] per position: receives this pass's LSE, or NULL
};

// Workspace of the vocabulary pass: per-segment partials of split rows.
size_t kl_part_bytes(int M_tot, int V, int elem_bytes);
constexpr int kKlPartBytes = 32;   // one stored row partial (8 words)
hipError_t launch_compact(const uint8_t* locked, int B, int N, int32_t* act_idx, int32_t* act_off,
                          hipStream_t s);
hipError_t launch_kl_lock(int dtype, const KLRowParams& rp, const TailParams& tp, float* part, hipStream_t s);
// The vocabulary pass when the LM head produced its statistics (EPI_LOGITS_KL): merge the n_vt
// column-tile partials of every row (klp as GemmArgs::klp, stride tp.M_tot), then the tail.
hipError_t launch_kl_merge_tail(int dtype, const KLRowParams& rp, const TailParams& tp, const float* klp, int n_vt,
                                hipStream_t s);

hipError_t launch_cache_scatter(int dtype, void* kc, void* vc, const void* kn, const void* vn,
                                const int32_t* act_idx, const int32_t* act_off, int B, int N,
                                int M_tot, int row_elems, hipStream_t s);

size_t attn_ws_bytes(int B, int N, int M_tot, int H, int Dh);
// key_excl: [B*N] flags or NULL; nonzero = that position is not attended.
hipError_t launch_attn(int dtype, const void* q, const void* kc, const void* vc,
                       const int32_t* act_off, const uint8_t* key_excl, int B, int N, int M_tot, int H, int Dh,
                       float scale, void* out, void* ws, hipStream_t s, const int32_t* m_dev = nullptr,
                       int kv_hm = 0);   // kv_hm: caches head-major [B][H][N][Dh] instead of [B][N][H][Dh]

hipError_t launch_rope_table(int n_pos, int Dh, float theta, float* table, hipStream_t s);

// Row gather / RMSNorm.
hipError_t launch_gather_norm(int dtype, const void* h_in, const void* embed, const int32_t* tok,
                              const int32_t* act_idx, const int32_t* act_off, int B, int N,
                              int M_tot, int d, float eps, float* h32, void* x, hipStream_t s,
                              const int32_t* m_dev = nullptr);
// Split-K residual: h32 += the nsplit partial planes of part, then x = RMSNorm(h32) in the
// storage type (x NULL: no norm).  d % 4 == 0, d <= kResidMaxD, 2 <= nsplit <= 8.
constexpr int kResidMaxD = 4096;
hipError_t launch_resid_norm(int dtype, const float* part, int nsplit, float* h32, int M_tot, int d, float eps,
                             void* x, hipStream_t s, const int32_t* m_dev = nullptr);
hipError_t launch_norm(int dtype, const float* h32, int M_tot, int d, float eps, void* x,
                       hipStream_t s, const int32_t* m_dev = nullptr);

// GEMM family: C[m][n] = sum_k A[m][k] * W[n][k] with fused epilogues.
enum EpiKind { EPI_QKV = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_LOGITS = 3, EPI_LOGITS_KL = 4 };
struct GemmArgs {
  const void* A;       // [M][K]
  int M, K;
  int Nv;              // virtual output columns
  // weights
  const void* w0;      // QKV: wq, SWIGLU: wg, else the only matrix
  const void* w1;      // QKV: wk, SWIGLU: wu
  const void* w2;      // QKV: wv
  // epilogue destinations
  void* out0;          // QKV: q [M][d]; RESID: h32 (float) [M][Nv]; SWIGLU: act [M][F]; LOGITS: logits [B*N][V]
  void* out1;          // QKV: k cache (one layer)
  void* out2;          // QKV: v cache (one layer)
  const float* rope;   // QKV: [rope_n][Dh/2][2]
  int d, Dh;           // QKV geometry
  const int32_t* act_idx;
  const int32_t* act_off;
  int B, N;
  int split_k;         // RESID only: K splits (set by the launcher)
  float* part;         // RESID split over K: [splits][M][Nv] fp32 partial sums written with plain stores
                       // (added into out0 by launch_resid_norm), or NULL: fp32 atomics into out0
  const int32_t* m_dev;  // device row count (M is then a capacity), or NULL
  // LOGITS_KL: the logits as LOGITS, plus each row's statistics over every tile of BN columns
  // against the previous posterior: klp[(n0 / BN) * M + m] (kPartWords floats each)
  const void* prev;      // [B*N][Nv] previous posterior, rows b*N + pos
  float* klp;
  int mask_id;           // id left out of the argmax (-1: none)
  int kv_hm;             // QKV: caches head-major [B][H][N][Dh] (0: token-major [B][N][H][Dh])
  // clock record (launch_gemm_clocked only): per workgroup w < clk_slots, clk[4w..4w+3] = shader-clock
  // cycles and 100 MHz real-time ticks of the whole workgroup, cycles of its k-tile loop, K elements it
  // multiplied (slots of workgroups past the live rows are left untouched)
  unsigned long long* clk;
  int clk_slots;
};
// nsplit (may be NULL) receives the number of K splits launched.
hipError_t launch_gemm(int dtype, EpiKind epi, const GemmArgs& a, hipStream_t s, int* nsplit = nullptr);
// launch_gemm with the clock record of GemmArgs::clk (bf16, SwiGLU or logits epilogue only).
hipError_t launch_gemm_clocked(EpiKind epi, const GemmArgs& a, hipStream_t s);
// Number of K splits launch_gemm runs for this shape when partial-sum planes are
// provided (GemmArgs::part set; 1 = none): the planes' workspace is sized from it.
int gemm_split(int dtype, EpiKind epi, int M, int K, int Nv);
int gemm_supported(int dtype, EpiKind epi, int Nv, int K, int d, int Dh);
// The GEMM addresses its A rows with 32-bit byte offsets: M * K * element bytes must stay within 4 GiB.
inline bool gemm_a_fits(long long M, long long K, int elem_bytes) { return M * K * elem_bytes <= (1LL << 32); }
// Tile (rows, columns), split-K and load path (1: through registers) the launcher
// picks for this shape; vb may be NULL.
void gemm_plan(int dtype, EpiKind epi, int M, int K, int Nv, int* bm, int* bn, int* split, int* vb);

}  // namespace sl
