// C ABI of the SureLock step: host-side argument checks, workspace layout and
// the per-step launch sequence.  Declarations and contracts: include/surelock.h.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/surelock.h"
#include "internal.hpp"

namespace {

thread_local char g_err[512] = "";

sl_status fail(sl_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

sl_status hip_check(hipError_t e, const char* what) {
  if (e == hipSuccess) return SL_OK;
  return fail(SL_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define SL_TRY(expr, what)                          \
  do {                                              \
    sl_status _st = hip_check((expr), (what));      \
    if (_st != SL_OK) return _st;                   \
  } while (0)

#define SL_REQUIRE(cond, code, ...)                 \
  do {                                              \
    if (!(cond)) return fail((code), __VA_ARGS__);  \
  } while (0)

inline size_t align256(size_t x) { return (x + 255) / 256 * 256; }
inline int elem_bytes(int dtype) { return dtype == SL_BF16 ? 2 : 4; }

// Column tiles of the LM head's plan at M rows when it also computes the row statistics
// (EPI_LOGITS_KL): one stored partial per (tile, row).
int head_kl_tiles(const sl_model* m, int M) {
  int bm = 0, bn = 0, sp = 0;
  sl::gemm_plan(m->dtype, sl::EPI_LOGITS_KL, M > 0 ? M : 1, m->d, m->vocab, &bm, &bn, &sp, nullptr);
  return bn > 0 ? m->vocab / bn : 0;
}

// Workspace layout of sl_step (contents need no initialisation).
struct StepLayout {
  size_t kl_part, h32, x, q, o, act, attn, total;
  StepLayout(const sl_model* m, int B, int N, int M_tot) {
    const int eb = elem_bytes(m->dtype);
    const size_t M = (size_t)(M_tot > 0 ? M_tot : 1);
    size_t off = 0;
    // the vocabulary pass's partials, or the fused LM head's per-tile row statistics
    size_t klb = m->lm_head ? sl::kl_part_bytes(M_tot, m->vocab, eb) : 256;
    if (m->lm_head) {
      const size_t fused = M * (size_t)head_kl_tiles(m, M_tot) * sl::kKlPartBytes;
      if (fused > klb) klb = fused;
    }
    kl_part = off; off += align256(klb);
    h32 = off; off += align256(M * m->d * 4);
    x = off; off += align256(M * m->d * eb);
    q = off; off += align256(M * m->d * eb);
    o = off; off += align256(M * m->d * eb);
    act = off; off += align256(M * m->ffn * eb);
    attn = off; off += align256(sl::attn_ws_bytes(B, N, M_tot, m->n_heads, m->head_dim));
    total = off;
  }
};

// Bytes of split-K partial sums the O and down projections need at M rows (their output
// width is d); 0 when neither splits or the row is too wide for the fused reduce.
size_t resid_part_bytes(const sl_model* m, int M) {
  if (M <= 0 || m->d > sl::kResidMaxD || m->d % 4) return 0;
  const int so = sl::gemm_split(m->dtype, sl::EPI_RESID, M, m->d, m->d);
  const int sd = sl::gemm_split(m->dtype, sl::EPI_RESID, M, m->ffn, m->d);
  const int sp = so > sd ? so : sd;
  return sp > 1 ? align256((size_t)sp * M * m->d * 4) : 0;
}

// The largest workspace any step with at most M_tot rows needs: the fixed regions, plus the
// split-K partial planes when with_part.  Neither is monotone in M: the attention splits its keys
// (and stores per-split partials) only when few query tiles leave the chip idle, and the
// launcher's split of the residual projections changes with M.
size_t step_ws_upto(const sl_model* m, int B, int N, int M_tot, bool with_part) {
  size_t best = 0;
  for (int M = 1; M <= (M_tot > 1 ? M_tot : 1); ++M) {
    const size_t b = StepLayout(m, B, N, M).total + (with_part ? resid_part_bytes(m, M) : 0);
    if (b > best) best = b;
  }
  return best;
}

sl_status check_dtype(int dtype) {
  SL_REQUIRE(dtype == SL_BF16 || dtype == SL_F32, SL_ERR_INVALID, "dtype %d is neither SL_BF16 nor SL_F32", dtype);
  return SL_OK;
}

sl_status check_model(const sl_model* m) {
  SL_REQUIRE(m, SL_ERR_INVALID, "model is NULL");
  sl_status st = check_dtype(m->dtype);
  if (st != SL_OK) return st;
  SL_REQUIRE(m->n_layers >= 1 && m->d > 0 && m->n_heads > 0 && m->head_dim > 0 && m->ffn > 0,
             SL_ERR_INVALID, "non-positive model dimension");
  SL_REQUIRE(m->n_heads * m->head_dim == m->d, SL_ERR_INVALID, "n_heads*head_dim (%d) != d (%d)",
             m->n_heads * m->head_dim, m->d);
  SL_REQUIRE(m->head_dim == 32 || m->head_dim == 64 || m->head_dim == 128, SL_ERR_UNSUPPORTED,
             "head_dim %d not in {32, 64, 128}", m->head_dim);
  SL_REQUIRE(m->d % 128 == 0, SL_ERR_UNSUPPORTED, "d %% 128 != 0 (d = %d)", m->d);
  SL_REQUIRE(m->ffn % 64 == 0, SL_ERR_UNSUPPORTED, "ffn %% 64 != 0 (ffn = %d)", m->ffn);
  SL_REQUIRE(m->layers, SL_ERR_INVALID, "layers is NULL");
  for (int l = 0; l < m->n_layers; ++l) {
    const sl_layer_weights& w = m->layers[l];
    SL_REQUIRE(w.wq && w.wk && w.wv && w.wo && w.wg && w.wu && w.wd, SL_ERR_INVALID,
               "layer %d has a NULL weight pointer", l);
  }
  SL_REQUIRE(m->rope && m->rope_n > 0, SL_ERR_INVALID, "rope table missing");
  if (m->lm_head) {
    SL_REQUIRE(m->vocab > 0 && m->vocab % 128 == 0, SL_ERR_UNSUPPORTED, "vocab %% 128 != 0 (vocab = %d)", m->vocab);
  }
  return SL_OK;
}

// Scratch memory of sl_kl_lock_noalloc: the vocabulary pass's per-segment partial sums live in this
// file-scope device array instead of a caller workspace.  Every (M_tot, V) needs at most
// M_tot * (segments per row) * 32 < 4096 * 32 bytes of partials (rows are split only while
// M_tot < 2048: into at most four below 768 rows, two from there on), so 256 KiB covers every
// size sl_kl_lock accepts.  Each device holds its own
// copy; host code reaches it only through the address hipGetSymbolAddress returns for the current
// device (the array's name on the host is not a device address).
constexpr size_t kNoAllocScratchBytes = 256 * 1024;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

// Device address of `scratch` on the current device, looked up once per device.
sl_status scratch_ptr(void** out) {
  int dev = -1;
  SL_TRY(hipGetDevice(&dev), "hipGetDevice");
  SL_REQUIRE(dev >= 0 && dev < kMaxDevices, SL_ERR_UNSUPPORTED, "device index %d >= %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    SL_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    SL_REQUIRE(p != nullptr, SL_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SL_OK;
}

}  // namespace

extern "C" {

const char* sl_status_string(sl_status s) {
  switch (s) {
    case SL_OK: return "SL_OK";
    case SL_ERR_INVALID: return "SL_ERR_INVALID";
    case SL_ERR_UNSUPPORTED: return "SL_ERR_UNSUPPORTED";
    case SL_ERR_HIP: return "SL_ERR_HIP";
  }
  return "SL_ERR_UNKNOWN";
}

const char* sl_last_error(void) { return g_err; }
const char* sl_version(void) { return "surelock-gfx950 0.1"; }

sl_status sl_compact(const uint8_t* locked, int B, int N, int32_t* act_idx, int32_t* act_off,
                     int32_t* m_tot_host, sl_stream stream) {
  g_err[0] = 0;
  SL_REQUIRE(locked && act_idx && act_off, SL_ERR_INVALID, "NULL pointer argument");
  SL_REQUIRE(B >= 1 && N >= 1, SL_ERR_INVALID, "B and N must be positive");
  SL_REQUIRE((long long)B * N < (1LL << 31), SL_ERR_UNSUPPORTED, "B*N too large");
  hipStream_t s = (hipStream_t)stream;
  SL_TRY(sl::launch_compact(locked, B, N, act_idx, act_off, s), "sl_compact launch");
  if (m_tot_host) {
    SL_TRY(hipMemcpyAsync(m_tot_host, act_off + B, 4, hipMemcpyDeviceToHost, s), "sl_compact copy");
    SL_TRY(hipStreamSynchronize(s), "sl_compact sync");
  }
  return SL_OK;
}

sl_status sl_cache_scatter(int dtype, void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                           const int32_t* act_idx, const int32_t* act_off, int B, int N, int M_tot,
                           int H, int Dh, sl_stream stream) {
  g_err[0] = 0;
  sl_status st = check_dtype(dtype);
  if (st != SL_OK) return st;
  SL_REQUIRE(k_cache && v_cache && act_off, SL_ERR_INVALID, "NULL pointer argument");
  SL_REQUIRE(B >= 1 && N >= 1 && H >= 1 && Dh >= 1 && M_tot >= 0, SL_ERR_INVALID, "bad size");
  SL_REQUIRE(M_tot == 0 || act_idx, SL_ERR_INVALID, "NULL act_idx");
  SL_REQUIRE((long long)M_tot <= (long long)B * N, SL_ERR_INVALID, "M_tot > B*N");
  SL_REQUIRE(M_tot == 0 || (k_new && v_new), SL_ERR_INVALID, "NULL k_new / v_new");
  SL_REQUIRE(((long long)H * Dh * elem_bytes(dtype)) % 16 == 0, SL_ERR_UNSUPPORTED, "row bytes %% 16 != 0");
  SL_TRY(sl::launch_cache_scatter(dtype, k_cache, v_cache, k_new, v_new, act_idx, act_off, B, N, M_tot,
                                  H * Dh, (hipStream_t)stream),
         "sl_cache_scatter launch");
  return SL_OK;
}

size_t sl_attn_workspace_size(int B, int N, int M_tot, int H, int Dh) {
  // The largest any call with at most M_tot rows needs: keys are split (and per-split partials
  // stored) only when few query tiles would leave the chip idle, so the need is not monotone in M_tot.
  // Splits need fewer than 64 workgroups of at most 128 queries: none from 8192 rows on.
  size_t best = sl::attn_ws_bytes(B, N, M_tot, H, Dh);
  const int top = M_tot < 8192 ? M_tot : 8192;
  for (int m = 1; m < top; ++m) {
    const size_t b = sl::attn_ws_bytes(B, N, m, H, Dh);
    if (b > best) best = b;
  }
  return best;
}

sl_status sl_attn_active(int dtype, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* act_off, const uint8_t* key_excl, int B, int N, int M_tot, int H,
                         int Dh, float scale, void* out, void* ws, size_t ws_bytes, sl_stream stream) {
  g_err[0] = 0;
  sl_status st = check_dtype(dtype);
  if (st != SL_OK) return st;
  SL_REQUIRE(k_cache && v_cache && act_off, SL_ERR_INVALID, "NULL pointer argument");
  SL_REQUIRE(B >= 1 && N >= 1 && H >= 1 && M_tot >= 0, SL_ERR_INVALID, "bad size");
  SL_REQUIRE((long long)M_tot <= (long long)B * N, SL_ERR_INVALID, "M_tot > B*N");
  SL_REQUIRE(M_tot == 0 || (q && out), SL_ERR_INVALID, "NULL q / out");
  SL_REQUIRE(Dh == 32 || Dh == 64 || Dh == 128, SL_ERR_UNSUPPORTED, "head_dim %d not in {32, 64, 128}", Dh);
  SL_REQUIRE(N % 64 == 0, SL_ERR_UNSUPPORTED, "N %% 64 != 0 (N = %d)", N);
  SL_REQUIRE((uintptr_t)key_excl % 4 == 0, SL_ERR_INVALID, "key_excl not 4-byte aligned");
  SL_REQUIRE(ws_bytes >= sl::attn_ws_bytes(B, N, M_tot, H, Dh) && ws, SL_ERR_INVALID,
             "workspace too small (%zu < %zu)", ws_bytes, sl::attn_ws_bytes(B, N, M_tot, H, Dh));
  SL_TRY(sl::launch_attn(dtype, q, k_cache, v_cache, act_off, key_excl, B, N, M_tot, H, Dh, scale, out, ws,
                         (hipStream_t)stream),
         "sl_attn_active launch");
  return SL_OK;
}

namespace {
// Segment partials one call with M_tot active rows needs, sized for whichever element type splits
// rows more.
size_t kl_ws_exact(int M_tot, int V) {
  const size_t p2 = sl::kl_part_bytes(M_tot, V, 2), p4 = sl::kl_part_bytes(M_tot, V, 4);
  return align256(p2 > p4 ? p2 : p4);
}
}  // namespace

size_t sl_kl_lock_workspace_size(int B, int N, int M_tot, int V) {
  // The largest any call with at most M_tot rows needs: rows split into more segments below 768
  // rows than above, and not at all from 2048 rows on, so the need is not monotone in M_tot.
  (void)B; (void)N;
  size_t best = kl_ws_exact(M_tot, V);
  const int top = M_tot < 2048 ? M_tot : 2047;
  for (int m = 1; m <= top; ++m) {
    const size_t b = kl_ws_exact(m, V);
    if (b > best) best = b;
  }
  return best;
}

sl_status sl_kl_lock(int dtype, const void* logits_cur, const void* logits_prev, int V,
                     const int32_t* act_idx, const int32_t* act_off, int B, int N, int M_tot,
                     const uint8_t* cand, const sl_lock_params* params, uint8_t* locked, float* kl,
                     float* u, float* lse, int32_t* argmax, float* conf, const float* lse_prev,
                     float* lse_pos, float* gate_thr, int32_t* new_act_idx, int32_t* new_act_off,
                     int32_t* m_tot_host, void* ws, size_t ws_bytes, sl_stream stream) {
  g_err[0] = 0;
  sl_status st = check_dtype(dtype);
  if (st != SL_OK) return st;
  SL_REQUIRE(params, SL_ERR_INVALID, "params is NULL");
  SL_REQUIRE(act_off && locked && new_act_idx && new_act_off && ws, SL_ERR_INVALID, "NULL pointer argument");
  SL_REQUIRE(M_tot == 0 || act_idx, SL_ERR_INVALID, "NULL act_idx");
  SL_REQUIRE(B >= 1 && N >= 1 && V > 0 && M_tot >= 0, SL_ERR_INVALID, "bad size");
  SL_REQUIRE((long long)M_tot <= (long long)B * N, SL_ERR_INVALID, "M_tot > B*N");
  SL_REQUIRE(N <= 65536, SL_ERR_UNSUPPORTED, "N > 65536");
  SL_REQUIRE(((long long)V * elem_bytes(dtype)) % 16 == 0, SL_ERR_UNSUPPORTED, "V*elem_size %% 16 != 0 (V = %d)", V);
  SL_REQUIRE(M_tot == 0 || (logits_cur && kl && u && lse), SL_ERR_INVALID, "NULL logits / kl / u / lse");
  SL_REQUIRE(M_tot == 0 || !params->have_prev || logits_prev, SL_ERR_INVALID, "NULL logits_prev");
  SL_REQUIRE(params->gate_q <= 1.f, SL_ERR_INVALID, "gate_q > 1");
  SL_REQUIRE(params->mask_id < V, SL_ERR_INVALID, "mask_id >= V");
  const size_t need = kl_ws_exact(M_tot, V);
  SL_REQUIRE(ws_bytes >= need, SL_ERR_INVALID, "workspace too small (%zu < %zu)", ws_bytes, need);
  SL_REQUIRE(!(lse_prev && lse_pos) || lse_prev != lse_pos, SL_ERR_INVALID,
             "lse_prev and lse_pos are the same buffer (keep two, as for the logits)");
  sl::KLRowParams rp{logits_cur, logits_prev, V, kl, u, lse, argmax, conf, lse_prev, lse_pos};
  sl::TailParams tp{};
  tp.B = B; tp.N = N; tp.M_tot = M_tot;
  tp.eps = params->eps; tp.gate_q = params->gate_q; tp.mask_id = params->mask_id;
  tp.have_prev = params->have_prev ? 1 : 0; tp.t = 0;
  tp.act_idx = act_idx; tp.act_off = act_off; tp.cand = cand; tp.locked = locked; tp.lock_step = nullptr;
  tp.kl = kl; tp.u = u; tp.conf = conf; tp.argmax = argmax; tp.gate_thr = gate_thr;
  tp.tok = nullptr; tp.cand_out = nullptr; tp.unmask_k = 0;
  tp.new_act_idx = new_act_idx; tp.new_act_off = new_act_off;
  char* w = (char*)ws;
  hipStream_t s = (hipStream_t)stream;
  SL_TRY(sl::launch_kl_lock(dtype, rp, tp, (float*)w, s), "sl_kl_lock launch");
  if (m_tot_host) {
    SL_TRY(hipMemcpyAsync(m_tot_host, new_act_off + B, 4, hipMemcpyDeviceToHost, s), "sl_kl_lock copy");
    SL_TRY(hipStreamSynchronize(s), "sl_kl_lock sync");
  }
  return SL_OK;
}

sl_status sl_kl_lock_noalloc(int dtype, const void* logits_cur, const void* logits_prev, int V,
                             const int32_t* act_idx, const int32_t* act_off, int B, int N, int M_tot,
                             const uint8_t* cand, const sl_lock_params* params, uint8_t* locked, float* kl,
                             float* u, float* lse, int32_t* argmax, float* conf, const float* lse_prev,
                             float* lse_pos, float* gate_thr, int32_t* new_act_idx, int32_t* new_act_off,
                             int32_t* m_tot_host, sl_stream stream) {
  g_err[0] = 0;
  SL_REQUIRE(B >= 1 && N >= 1 && V > 0 && M_tot >= 0, SL_ERR_INVALID, "bad size");
  const size_t need = kl_ws_exact(M_tot, V);
  SL_REQUIRE(need <= kNoAllocScratchBytes, SL_ERR_UNSUPPORTED,
             "sl_kl_lock_noalloc: %zu bytes of partial sums exceed its %zu-byte scratch", need, kNoAllocScratchBytes);
  void* ws = nullptr;
  sl_status st = scratch_ptr(&ws);
  if (st != SL_OK) return st;
  return sl_kl_lock(dtype, logits_cur, logits_prev, V, act_idx, act_off, B, N, M_tot, cand, params, locked, kl, u,
                    lse, argmax, conf, lse_prev, lse_pos, gate_thr, new_act_idx, new_act_off, m_tot_host, ws,
                    kNoAllocScratchBytes, stream);
}

sl_status sl_rope_table(int n_pos, int head_dim, float theta, float* table, sl_stream stream) {
  g_err[0] = 0;
  SL_REQUIRE(table, SL_ERR_INVALID, "table is NULL");
  SL_REQUIRE(n_pos > 0 && head_dim > 0 && head_dim % 2 == 0 && theta > 0.f, SL_ERR_INVALID, "bad size");
  SL_TRY(sl::launch_rope_table(n_pos, head_dim, theta, table, (hipStream_t)stream), "sl_rope_table launch");
  return SL_OK;
}

// Checks sl_gemm's arguments and fills g (M == 0 passes with nothing to launch).
static sl_status gemm_args(int dtype, int epilogue, const void* A, int M, int K, int n_out, const void* w0,
                           const void* w1, const void* w2, void* out0, void* out1, void* out2, const float* rope,
                           int d, int head_dim, const int32_t* act_idx, const int32_t* act_off, int B, int N,
                           sl::GemmArgs& g) {
  sl_status st = check_dtype(dtype);
  if (st != SL_OK) return st;
  SL_REQUIRE(epilogue >= SL_EPI_QKV_ROPE && epilogue <= SL_EPI_LOGITS, SL_ERR_INVALID, "bad epilogue %d", epilogue);
  SL_REQUIRE(M >= 0 && K > 0 && n_out > 0, SL_ERR_INVALID, "bad size");
  g = sl::GemmArgs{};
  g.M = 0;
  if (M == 0) return SL_OK;
  SL_REQUIRE(A && w0 && out0, SL_ERR_INVALID, "NULL pointer argument");
  const sl::EpiKind epi = (sl::EpiKind)epilogue;
  SL_REQUIRE(sl::gemm_supported(dtype, epi, n_out, K, d, head_dim), SL_ERR_UNSUPPORTED,
             "unsupported GEMM shape (K=%d, n_out=%d)", K, n_out);
  SL_REQUIRE(sl::gemm_a_fits(M, K, elem_bytes(dtype)), SL_ERR_UNSUPPORTED, "A operand of %d x %d exceeds 4 GiB", M, K);
  if (epi == sl::EPI_QKV) {
    SL_REQUIRE(w1 && w2 && out1 && out2 && rope && act_idx && act_off, SL_ERR_INVALID, "QKV needs wk, wv, caches, rope, act lists");
    SL_REQUIRE(n_out == 3 * d && d % 128 == 0 && head_dim > 0 && d % head_dim == 0 && head_dim % 2 == 0,
               SL_ERR_UNSUPPORTED, "QKV needs n_out = 3d, d %% 128 == 0");
  }
  if (epi == sl::EPI_SWIGLU) SL_REQUIRE(w1, SL_ERR_INVALID, "SwiGLU needs the up matrix");
  if (epi == sl::EPI_LOGITS) SL_REQUIRE(act_idx && act_off && B >= 1 && N >= 1, SL_ERR_INVALID, "LOGITS needs act lists");
  g.A = A; g.M = M; g.K = K; g.Nv = n_out; g.w0 = w0; g.w1 = w1; g.w2 = w2;
  g.out0 = out0; g.out1 = out1; g.out2 = out2; g.rope = rope; g.d = d; g.Dh = head_dim;
  g.act_idx = act_idx; g.act_off = act_off; g.B = B; g.N = N; g.split_k = 1;
  return SL_OK;
}

sl_status sl_gemm(int dtype, int epilogue, const void* A, int M, int K, int n_out, const void* w0,
                  const void* w1, const void* w2, void* out0, void* out1, void* out2, const float* rope,
                  int d, int head_dim, const int32_t* act_idx, const int32_t* act_off, int B, int N,
                  sl_stream stream) {
  g_err[0] = 0;
  sl::GemmArgs g;
  const sl_status st = gemm_args(dtype, epilogue, A, M, K, n_out, w0, w1, w2, out0, out1, out2, rope, d, head_dim,
                                 act_idx, act_off, B, N, g);
  if (st != SL_OK || g.M == 0) return st;
  SL_TRY(sl::launch_gemm(dtype, (sl::EpiKind)epilogue, g, (hipStream_t)stream), "sl_gemm launch");
  return SL_OK;
}

sl_status sl_gemm_clocked(int epilogue, const void* A, int M, int K, int n_out, const void* w0, const void* w1,
                          void* out0, const int32_t* act_idx, const int32_t* act_off, int B, int N,
                          unsigned long long* clocks, int clock_slots, sl_stream stream) {
  g_err[0] = 0;
  SL_REQUIRE(epilogue == SL_EPI_SWIGLU || epilogue == SL_EPI_LOGITS, SL_ERR_UNSUPPORTED,
             "sl_gemm_clocked takes the SwiGLU or logits epilogue");
  SL_REQUIRE(clocks && clock_slots > 0, SL_ERR_INVALID, "NULL clock record");
  sl::GemmArgs g;
  const sl_status st = gemm_args(SL_BF16, epilogue, A, M, K, n_out, w0, w1, nullptr, out0, nullptr, nullptr, nullptr,
                                 0, 0, act_idx, act_off, B, N, g);
  if (st != SL_OK || g.M == 0) return st;
  g.clk = clocks;
  g.clk_slots = clock_slots;
  SL_TRY(sl::launch_gemm_clocked((sl::EpiKind)epilogue, g, (hipStream_t)stream), "sl_gemm_clocked launch");
  return SL_OK;
}

sl_status sl_gemm_plan(int dtype, int epilogue, int M, int K, int n_out, int* tile_m, int* tile_n,
                       int* split_k, int* through_registers) {
  g_err[0] = 0;
  sl_status st = check_dtype(dtype);
  if (st != SL_OK) return st;
  SL_REQUIRE(tile_m && tile_n && split_k, SL_ERR_INVALID, "NULL output pointer");
  SL_REQUIRE(epilogue >= SL_EPI_QKV_ROPE && epilogue <= SL_EPI_LOGITS, SL_ERR_INVALID, "bad epilogue %d", epilogue);
  SL_REQUIRE(M > 0 && K > 0 && n_out > 0, SL_ERR_INVALID, "bad size");
  SL_REQUIRE(sl::gemm_supported(dtype, (sl::EpiKind)epilogue, n_out, K, 128, 2), SL_ERR_UNSUPPORTED,
             "unsupported GEMM shape (K=%d, n_out=%d)", K, n_out);
  sl::gemm_plan(dtype, (sl::EpiKind)epilogue, M, K, n_out, tile_m, tile_n, split_k, through_registers);
  return SL_OK;
}

size_t sl_step_workspace_size(const sl_model* model, int B, int N, int M_tot) {
  if (!model) return 0;
  return step_ws_upto(model, B, N, M_tot, true);
}

size_t sl_step_workspace_min(const sl_model* model, int B, int N, int M_tot) {
  if (!model) return 0;
  return step_ws_upto(model, B, N, M_tot, false);
}

sl_status sl_step(const sl_model* m, sl_state* st, const sl_step_params* p, void* ws, size_t ws_bytes,
                  sl_stream stream) {
  g_err[0] = 0;
  sl_status cs = check_model(m);
  if (cs != SL_OK) return cs;
  SL_REQUIRE(st && p, SL_ERR_INVALID, "state or params is NULL");
  const int B = st->B, N = st->N, M = st->M_tot;
  SL_REQUIRE(B >= 1 && N >= 1 && M >= 0 && (long long)M <= (long long)B * N, SL_ERR_INVALID,
             "bad B / N / M_tot (%d, %d, %d)", B, N, M);
  SL_REQUIRE(N % 64 == 0, SL_ERR_UNSUPPORTED, "N %% 64 != 0 (N = %d)", N);
  SL_REQUIRE(N <= 65536, SL_ERR_UNSUPPORTED, "N > 65536");
  SL_REQUIRE(m->rope_n >= N, SL_ERR_INVALID, "rope table has %d positions < N = %d", m->rope_n, N);
  SL_REQUIRE(st->locked && st->act_idx && st->act_off && st->k_cache && st->v_cache, SL_ERR_INVALID,
             "NULL state buffer");
  SL_REQUIRE(st->h_in || (m->embed && st->tok), SL_ERR_INVALID, "need h_in, or embed and tok");
  SL_REQUIRE(st->t >= 0, SL_ERR_INVALID, "t < 0");
  SL_REQUIRE(sl::gemm_a_fits(M, m->d > m->ffn ? m->d : m->ffn, elem_bytes(m->dtype)), SL_ERR_UNSUPPORTED,
             "M_tot = %d active rows exceed the GEMMs' 4 GiB A operand", M);
  const bool head = m->lm_head != nullptr;
  const bool lock = head && p->do_lock;
  // the LM head computes the vocabulary statistics in its epilogue (needs a previous posterior)
  const bool fuse = lock && p->fuse_head_kl && st->t > 0 && head_kl_tiles(m, M) > 0;
  if (head) SL_REQUIRE(st->logits[0] && st->logits[1], SL_ERR_INVALID, "logits buffers missing");
  if (lock) {
    SL_REQUIRE(st->kl && st->u && st->lse, SL_ERR_INVALID, "kl / u / lse missing");
    SL_REQUIRE(p->gate_q <= 1.f, SL_ERR_INVALID, "gate_q > 1");
    SL_REQUIRE(p->mask_id < m->vocab, SL_ERR_INVALID, "mask_id >= vocab");
  }
  const bool lse_store = st->lse_pos[0] && st->lse_pos[1];
  SL_REQUIRE(!(st->lse_pos[0] || st->lse_pos[1]) || lse_store, SL_ERR_INVALID, "only one lse_pos buffer");
  SL_REQUIRE(!lse_store || st->lse_pos[0] != st->lse_pos[1], SL_ERR_INVALID, "lse_pos buffers alias");
  SL_REQUIRE(!(lse_store && head && !lock), SL_ERR_INVALID,
             "with lse_pos set every step that writes logits must run the vocabulary pass (do_lock = 1)");
  if (lock && p->unmask_k > 0) {
    SL_REQUIRE(st->tok && st->cand && st->argmax && st->conf && p->mask_id >= 0, SL_ERR_INVALID,
               "sampler needs tok, cand, argmax, conf and a mask id");
  }
  const StepLayout L(m, B, N, M);
  SL_REQUIRE(ws && ws_bytes >= L.total, SL_ERR_INVALID, "workspace too small (%zu < %zu)", ws_bytes, L.total);
  // split-K partial sums of the residual projections go after the fixed regions when they fit
  // (a workspace of sl_step_workspace_size bytes always has room); otherwise fp32 atomics
  const size_t part_need = resid_part_bytes(m, M);
  float* part = (part_need > 0 && ws_bytes - L.total >= part_need) ? (float*)((char*)ws + L.total) : nullptr;

  hipStream_t s = (hipStream_t)stream;
  const int dt = m->dtype, eb = elem_bytes(dt);
  const int d = m->d, F = m->ffn, H = m->n_heads, Dh = m->head_dim;
  char* w = (char*)ws;
  float* h32 = st->h_out ? st->h_out : (float*)(w + L.h32);
  void* x = w + L.x;
  void* q = w + L.q;
  void* o = w + L.o;
  void* act = w + L.act;
  void* attn_ws = w + L.attn;
  const size_t cache_layer = (size_t)B * N * d * eb;
  const float scale = 1.f / sqrtf((float)Dh);
  // no-KV-cache ablation: the positions locked before this step are not attended
  const uint8_t* key_excl = p->no_kv_cache ? st->locked : nullptr;
  // device-resident row count: M is then a capacity, every kernel reads the live count act_off[B]
  const int32_t* m_dev = p->device_m ? st->act_off + B : nullptr;

  if (M > 0) {
    SL_TRY(sl::launch_gather_norm(dt, st->h_in, m->embed, st->tok, st->act_idx, st->act_off, B, N, M, d,
                                  m->rms_eps, h32, x, s, m_dev),
           "gather");
    for (int l = 0; l < m->n_layers; ++l) {
      const sl_layer_weights& W = m->layers[l];
      char* kc = (char*)st->k_cache + l * cache_layer;
      char* vc = (char*)st->v_cache + l * cache_layer;
      sl::GemmArgs g{};
      g.act_idx = st->act_idx; g.act_off = st->act_off; g.B = B; g.N = N; g.M = M; g.d = d; g.Dh = Dh;
      g.split_k = 1;
      g.m_dev = m_dev;
      g.kv_hm = st->kv_head_major ? 1 : 0;
      // QKV + RoPE + K/V scatter into the layer cache
      g.A = x; g.K = d; g.Nv = 3 * d; g.w0 = W.wq; g.w1 = W.wk; g.w2 = W.wv;
      g.out0 = q; g.out1 = kc; g.out2 = vc; g.rope = m->rope;
      SL_TRY(sl::launch_gemm(dt, sl::EPI_QKV, g, s), "qkv gemm");
      SL_TRY(sl::launch_attn(dt, q, kc, vc, st->act_off, key_excl, B, N, M, H, Dh, scale, o, attn_ws, s, m_dev,
                             st->kv_head_major ? 1 : 0),
             "attention");
      // O projection + residual, then the pre-FFN RMSNorm (fused with the partial sums' reduce
      // when the projection is split over K)
      int ns = 1;
      g.A = o; g.K = d; g.Nv = d; g.w0 = W.wo; g.w1 = g.w2 = nullptr; g.out0 = h32; g.part = part;
      SL_TRY(sl::launch_gemm(dt, sl::EPI_RESID, g, s, &ns), "o gemm");
      if (part && ns > 1)
        SL_TRY(sl::launch_resid_norm(dt, part, ns, h32, M, d, m->rms_eps, x, s, m_dev), "residual + norm");
      else
        SL_TRY(sl::launch_norm(dt, h32, M, d, m->rms_eps, x, s, m_dev), "norm");
      // SwiGLU FFN + residual, then the next block's RMSNorm (none after the last layer without a head)
      g.A = x; g.K = d; g.Nv = 2 * F; g.w0 = W.wg; g.w1 = W.wu; g.out0 = act; g.part = nullptr;
      SL_TRY(sl::launch_gemm(dt, sl::EPI_SWIGLU, g, s), "gate/up gemm");
      g.A = act; g.K = F; g.Nv = d; g.w0 = W.wd; g.w1 = nullptr; g.out0 = h32; g.part = part;
      SL_TRY(sl::launch_gemm(dt, sl::EPI_RESID, g, s, &ns), "down gemm");
      void* xn = (head || l + 1 < m->n_layers) ? x : nullptr;
      if (part && ns > 1)
        SL_TRY(sl::launch_resid_norm(dt, part, ns, h32, M, d, m->rms_eps, xn, s, m_dev), "residual + norm");
      else if (xn)
        SL_TRY(sl::launch_norm(dt, h32, M, d, m->rms_eps, xn, s, m_dev), "norm");
    }
    if (head) {
      sl::GemmArgs g{};
      g.act_idx = st->act_idx; g.act_off = st->act_off; g.B = B; g.N = N; g.M = M; g.d = d; g.Dh = Dh;
      g.split_k = 1;
      g.m_dev = m_dev;
      g.A = x; g.K = d; g.Nv = m->vocab; g.w0 = m->lm_head; g.out0 = st->logits[st->t & 1];
      if (fuse) {
        g.prev = st->logits[(st->t + 1) & 1];
        g.klp = (float*)(w + L.kl_part);
        g.mask_id = p->mask_id;
      }
      SL_TRY(sl::launch_gemm(dt, fuse ? sl::EPI_LOGITS_KL : sl::EPI_LOGITS, g, s), "lm head gemm");
    }
  }
  if (lock) {
    // with the per-position LSE store: this step's LSE goes to lse_pos[t%2], and the previous
    // posterior's is read from lse_pos[(t+1)%2], where step t-1 stored it
    sl::KLRowParams rp{st->logits[st->t & 1], st->logits[(st->t + 1) & 1], m->vocab, st->kl, st->u,
                       st->lse, st->argmax, st->conf,
                       (lse_store && st->t > 0) ? st->lse_pos[(st->t + 1) & 1] : nullptr,
                       lse_store ? st->lse_pos[st->t & 1] : nullptr};
    sl::TailParams tp{};
    tp.B = B; tp.N = N; tp.M_tot = M;
    tp.m_dev = m_dev; tp.t_dev = st->t_dev;
    tp.eps = p->eps; tp.gate_q = p->gate_q; tp.mask_id = p->mask_id; tp.have_prev = st->t > 0; tp.t = st->t;
    tp.act_idx = st->act_idx; tp.act_off = st->act_off; tp.cand = st->cand; tp.locked = st->locked;
    tp.lock_step = st->lock_step; tp.kl = st->kl; tp.u = st->u; tp.conf = st->conf; tp.argmax = st->argmax;
    tp.gate_thr = st->gate_thr; tp.tok = st->tok; tp.cand_out = st->cand;
    tp.unmask_k = p->unmask_k > 0 ? p->unmask_k : 0;
    tp.new_act_idx = st->act_idx; tp.new_act_off = st->act_off;
    if (fuse)
      SL_TRY(sl::launch_kl_merge_tail(dt, rp, tp, (const float*)(w + L.kl_part), head_kl_tiles(m, M), s),
             "kl merge + lock");
    else
      SL_TRY(sl::launch_kl_lock(dt, rp, tp, (float*)(w + L.kl_part), s), "kl lock");
    if (st->m_tot_host) {
      SL_TRY(hipMemcpyAsync(st->m_tot_host, st->act_off + B, 4, hipMemcpyDeviceToHost, s), "M copy");
      SL_TRY(hipStreamSynchronize(s), "M sync");
    }
  }
  return SL_OK;
}

}  // extern "C"
