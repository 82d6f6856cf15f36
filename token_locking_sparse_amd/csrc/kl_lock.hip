// Vocabulary pass, gate, permanent lock update, sampler tail and compaction.
//
// Per active row (one or a few workgroups per row): one streaming pass over
// the current and previous logits with an online (rescaled) log-sum-exp,
// giving LSE, the step KL(p_t || p_{t-1}), 1 - max p and the argmax
// (zhaoyang97 notes on SureLock, 锁定判据 and 可选置信度门控).  A second,
// single-workgroup kernel merges split rows and runs the tail: per-sequence
// gate quantile (radix select), monotone lock update, optional unmasking
// sampler and stream compaction of the next active set (same notes,
// 永久锁定机制; 整体框架).  The kernel boundary is the only hand-off between
// workgroups, so no device-wide fences are needed.
#include <float.h>
#include <math.h>

#include "common.hpp"
#include "internal.hpp"

namespace sl {

constexpr int kKLThreads = 256;
constexpr int kPartWords = 8;
constexpr int kTailThreads = 1024;

// ------------------------------------------------------------------ compaction
// Ascending positions with locked == 0 of B sequences of N, written with the
// whole workgroup: per round every thread tests one position, a wave ballot and
// mbcnt give the rank inside the wave, and the per-wave counts are prefix-summed
// through LDS.  s_w: LDS scratch of blockDim/64 ints.
__device__ void block_compact(const uint8_t* locked, int B, int N, int32_t* act_idx,
                              int32_t* act_off, int* s_w) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, nw = blockDim.x >> 6;
  const int total = B * N;
  int base = 0;
  for (int r0 = 0; r0 < total; r0 += blockDim.x) {
    const int i = r0 + tid;
    const bool act = (i < total) && (locked[i] == 0);
    const uint64_t bal = __ballot(act);
    const int lane_pre = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                   __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
    if (lane == 0) s_w[wid] = __popcll(bal);
    __syncthreads();
    int wpre = 0, tot = 0;
    for (int w = 0; w < nw; ++w) {
      const int c = s_w[w];
      wpre += (w < wid) ? c : 0;
      tot += c;
    }
    const int pos = base + wpre + lane_pre;
    if (i < total) {
      const int q = i / N, rr = i - q * N;
      if (act) act_idx[pos] = rr;
      if (rr == 0) act_off[q] = pos;
    }
    base += tot;
    __syncthreads();
  }
  if (tid == 0) act_off[B] = base;
}

__global__ void __launch_bounds__(1024) compact_kernel(const uint8_t* locked, int B, int N,
                                                       int32_t* act_idx, int32_t* act_off) {
  __shared__ int s_w[16];
  block_compact(locked, B, N, act_idx, act_off, s_w);
}

hipError_t launch_compact(const uint8_t* locked, int B, int N, int32_t* act_idx, int32_t* act_off,
                          hipStream_t s) {
  hipLaunchKernelGGL(compact_kernel, dim3(1), dim3(1024), 0, s, locked, B, N, act_idx, act_off);
  return hipGetLastError();
}

// ------------------------------------------------------------------ tail
struct TailShared {
  int w[16];
  uint32_t hist[256];
  int sel[2];
  float fv[16];
  int iv[32];
};

// k-th smallest (0-based) of the non-negative floats u[o0..o1), exact, by a
// 4-pass 8-bit radix select on their bit patterns (monotone for x >= 0).
__device__ float block_select_kth(const float* u, int o0, int o1, int k, TailShared& sh) {
  const int tid = threadIdx.x, lane = tid & 63;
  uint32_t prefix = 0, pmask = 0;
  int kk = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += blockDim.x) sh.hist[i] = 0;
    __syncthreads();
    for (int m = o0 + tid; m < o1; m += blockDim.x) {
      const uint32_t v = __float_as_uint(u[m]);
      if ((v & pmask) == prefix) atomicAdd(&sh.hist[(v >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      int c[4], ls = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) { c[j] = (int)sh.hist[4 * lane + j]; ls += c[j]; }
      int inc = ls;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(inc, o, 64);
        if (lane >= o) inc += t;
      }
      int ex = inc - ls;
      if (ex <= kk && kk < inc) {
        int run = ex, j = 0;
        while (run + c[j] <= kk) { run += c[j]; ++j; }
        sh.sel[0] = 4 * lane + j;
        sh.sel[1] = kk - run;
      }
    }
    __syncthreads();
    prefix |= ((uint32_t)sh.sel[0]) << shift;
    pmask |= 255u << shift;
    kk = sh.sel[1];
    __syncthreads();
  }
  return __uint_as_float(prefix);
}

// Gate quantile, lock update, optional sampler, compaction — one workgroup.
__device__ void tail_phase(const TailParams& p, TailShared& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, nw = blockDim.x >> 6;
  const bool gate = p.gate_q >= 0.f;
  const bool can_lock = p.eps > 0.f && p.have_prev;
  for (int b = 0; b < p.B; ++b) {
    const int o0 = p.act_off[b], o1 = p.act_off[b + 1];
    const int n = o1 - o0;
    float thr = INFINITY;
    if (gate && n > 0) {
      const int k = (int)floor((double)p.gate_q * (double)(n - 1));
      thr = block_select_kth(p.u, o0, o1, k, sh);
    }
    if (tid == 0 && p.gate_thr) p.gate_thr[b] = thr;
    if (can_lock) {
      for (int m = o0 + tid; m < o1; m += blockDim.x) {
        const int64_t g = (int64_t)b * p.N + p.act_idx[m];
        bool ok = (p.cand == nullptr) || (p.cand[g] != 0);
        ok = ok && (p.kl[m] <= p.eps);
        if (gate) ok = ok && (p.u[m] <= thr);
        if (ok) {
          p.locked[g] = 1;
          if (p.lock_step) p.lock_step[g] = p.t;
        }
      }
    }
    // Sampler: the unmask_k most confident [MASK] positions take their argmax.
    for (int r = 0; r < p.unmask_k; ++r) {
      float bc = -1.f;
      int bp = INT_MAX, bm = -1;
      for (int m = o0 + tid; m < o1; m += blockDim.x) {
        const int pos = p.act_idx[m];
        const int64_t g = (int64_t)b * p.N + pos;
        if (p.tok[g] != p.mask_id) continue;
        const float c = p.conf[m];
        if (c > bc || (c == bc && pos < bp)) { bc = c; bp = pos; bm = m; }
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const float oc = __shfl_xor(bc, o, 64);
        const int op = __shfl_xor(bp, o, 64), om = __shfl_xor(bm, o, 64);
        if (oc > bc || (oc == bc && op < bp)) { bc = oc; bp = op; bm = om; }
      }
      if (lane == 0) { sh.fv[wid] = bc; sh.iv[wid] = bp; sh.iv[16 + wid] = bm; }
      __syncthreads();
      if (tid == 0) {
        for (int w = 1; w < nw; ++w) {
          if (sh.fv[w] > bc || (sh.fv[w] == bc && sh.iv[w] < bp)) { bc = sh.fv[w]; bp = sh.iv[w]; bm = sh.iv[16 + w]; }
        }
        if (bm >= 0) {
          const int64_t g = (int64_t)b * p.N + bp;
          p.tok[g] = p.argmax[bm];
          p.cand_out[g] = 1;
        }
      }
      __syncthreads();
    }
  }
  __syncthreads();
  block_compact(p.locked, p.B, p.N, p.new_act_idx, p.new_act_off, sh.w);
}


// ------------------------------------------------------------------ row pass
struct Part {
  float ma, sa, ta;  // running max of cur (all ids), sum e^(a-ma), sum e^(a-ma) (a-b)
  float mb, sb;      // running max of prev, sum e^(b-mb)
  float best;        // max of cur over ids != mask
  int bidx;          // chunk holding `best` (lowest on ties)
};

__device__ __forceinline__ float scale_to(float m_old, float m_new) {
  return (m_old > -INFINITY) ? __builtin_amdgcn_exp2f((m_old - m_new) * kLog2e) : 0.f;
}

__device__ __forceinline__ Part combine(const Part& x, const Part& y) {
  Part r;
  r.ma = fmaxf(x.ma, y.ma);
  const float ex = scale_to(x.ma, r.ma), ey = scale_to(y.ma, r.ma);
  r.sa = x.sa * ex + y.sa * ey;
  r.ta = x.ta * ex + y.ta * ey;
  r.mb = fmaxf(x.mb, y.mb);
  const float fx = scale_to(x.mb, r.mb), fy = scale_to(y.mb, r.mb);
  r.sb = x.sb * fx + y.sb * fy;
  const bool take_y = (y.best > x.best) || (y.best == x.best && y.bidx < x.bidx);
  r.best = take_y ? y.best : x.best;
  r.bidx = take_y ? y.bidx : x.bidx;
  return r;
}

__device__ __forceinline__ Part shfl_part(const Part& x, int o) {
  Part r;
  r.ma = __shfl_xor(x.ma, o, 64); r.sa = __shfl_xor(x.sa, o, 64); r.ta = __shfl_xor(x.ta, o, 64);
  r.mb = __shfl_xor(x.mb, o, 64); r.sb = __shfl_xor(x.sb, o, 64);
  r.best = __shfl_xor(x.best, o, 64); r.bidx = __shfl_xor(x.bidx, o, 64);
  return r;
}

// Row statistics from a (combined) partial: with S_a = sum e^(a - max a),
// A = max a + ln S_a, max p = 1/S_a, KL = sum p (a - b) - A + B.
template <typename T, bool PREV>
__device__ void finish_row(const KLRowParams& rp, const Part& t, const char* crow, int C, int mask_id, int r) {
  constexpr int E = Chunk<T>::kElems;
  const float A = t.ma + logf(t.sa);
  rp.lse[r] = A;
  rp.u[r] = 1.f - 1.f / t.sa;
  if (PREV) rp.kl[r] = t.ta / t.sa - (t.ma - t.mb) - logf(t.sa / t.sb);
  else rp.kl[r] = INFINITY;
  // exact argmax inside the winning chunk (lowest id equal to the max, not the mask)
  int am = 0;
  if (t.bidx >= 0 && t.bidx < C) {   // always true for finite logits
    float a[E];
    Chunk<T>::unpack(ld16(crow + (size_t)t.bidx * 16), a);
    am = t.bidx * E;
    for (int j = E - 1; j >= 0; --j)
      if (a[j] == t.best && t.bidx * E + j != mask_id) am = t.bidx * E + j;
  }
  if (rp.argmax) rp.argmax[r] = am;
  if (rp.conf) rp.conf[r] = __expf(t.best - t.ma) / t.sa;
}

// Row pass: workgroup (row r, segment) streams its slice of the current and
// previous logits once.  With one segment per row it finishes the row itself;
// otherwise it stores its partial for the tail kernel.  No inter-workgroup
// communication happens inside this kernel.
template <typename T, bool PREV>
__global__ void __launch_bounds__(kKLThreads)
kl_rows_kernel(KLRowParams rp, TailParams tp, int n_seg, int seg_chunks, float* part) {
  constexpr int E = Chunk<T>::kElems;
  __shared__ Part s_part[kKLThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int r = blockIdx.x / n_seg, seg = blockIdx.x - r * n_seg;
  const int b = seq_of_row(tp.act_off, tp.B, r);
  const int64_t g = (int64_t)b * tp.N + tp.act_idx[r];
  const size_t rowbytes = (size_t)rp.V * sizeof(T);
  const char* crow = (const char*)rp.cur + g * rowbytes;
  const char* prow = (const char*)rp.prev + g * rowbytes;
  const int C = rp.V / E;
  const int c0 = seg * seg_chunks;
  const int c1 = min(C, c0 + seg_chunks);
  const int mask_id = tp.mask_id;

  Part acc;
  acc.ma = -INFINITY; acc.sa = 0.f; acc.ta = 0.f;
  acc.mb = -INFINITY; acc.sb = 0.f;
  acc.best = -INFINITY; acc.bidx = INT_MAX;

  for (int c = c0 + tid; c < c1; c += kKLThreads) {
    float a[E], bb[E];
    Chunk<T>::unpack(ld16(crow + (size_t)c * 16), a);
    if (PREV) Chunk<T>::unpack(ld16(prow + (size_t)c * 16), bb);
    float cm = a[0];
#pragma unroll
    for (int j = 1; j < E; ++j) cm = fmaxf(cm, a[j]);
    float cmn = cm;
    const int e0 = c * E;
    if ((unsigned)(mask_id - e0) < (unsigned)E) {
      cmn = -INFINITY;
#pragma unroll
      for (int j = 0; j < E; ++j)
        if (e0 + j != mask_id) cmn = fmaxf(cmn, a[j]);
    }
    if (cmn > acc.best) { acc.best = cmn; acc.bidx = c; }
    const float mnew = fmaxf(acc.ma, cm);
    const float sc = scale_to(acc.ma, mnew);
    acc.sa *= sc;
    acc.ta *= sc;
    acc.ma = mnew;
    const float ml = mnew * kLog2e;
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const float e = __builtin_amdgcn_exp2f(fmaf(a[j], kLog2e, -ml));
      acc.sa += e;
      if (PREV) acc.ta = fmaf(e, a[j] - bb[j], acc.ta);
    }
    if (PREV) {
      float bm = bb[0];
#pragma unroll
      for (int j = 1; j < E; ++j) bm = fmaxf(bm, bb[j]);
      const float mbn = fmaxf(acc.mb, bm);
      acc.sb *= scale_to(acc.mb, mbn);
      acc.mb = mbn;
      const float mbl = mbn * kLog2e;
#pragma unroll
      for (int j = 0; j < E; ++j) acc.sb += __builtin_amdgcn_exp2f(fmaf(bb[j], kLog2e, -mbl));
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc = combine(acc, shfl_part(acc, o));
  if (lane == 0) s_part[wid] = acc;
  __syncthreads();
  if (tid == 0) {
    Part t = s_part[0];
    for (int w = 1; w < kKLThreads / 64; ++w) t = combine(t, s_part[w]);
    if (n_seg == 1) {
      finish_row<T, PREV>(rp, t, crow, C, mask_id, r);
    } else {
      float* pp = part + ((size_t)r * n_seg + seg) * kPartWords;
      pp[0] = t.ma; pp[1] = t.sa; pp[2] = t.ta; pp[3] = t.mb; pp[4] = t.sb; pp[5] = t.best;
      pp[6] = __int_as_float(t.bidx);
    }
  }
}

// Tail kernel (one workgroup): merge the segment partials of every row (when a
// row was split), then gate quantile, lock update, sampler and compaction.
template <typename T, bool PREV>
__global__ void __launch_bounds__(kTailThreads)
kl_tail_kernel(KLRowParams rp, TailParams tp, int n_seg, const float* part) {
  __shared__ TailShared sh;
  if (n_seg > 1) {
    const int C = rp.V / Chunk<T>::kElems;
    const size_t rowbytes = (size_t)rp.V * sizeof(T);
    for (int r = threadIdx.x; r < tp.M_tot; r += blockDim.x) {
      const float* q = part + (size_t)r * n_seg * kPartWords;
      Part x;
      x.ma = q[0]; x.sa = q[1]; x.ta = q[2]; x.mb = q[3]; x.sb = q[4]; x.best = q[5];
      x.bidx = __float_as_int(q[6]);
      for (int s2 = 1; s2 < n_seg; ++s2) {
        const float* qs = q + s2 * kPartWords;
        Part y;
        y.ma = qs[0]; y.sa = qs[1]; y.ta = qs[2]; y.mb = qs[3]; y.sb = qs[4]; y.best = qs[5];
        y.bidx = __float_as_int(qs[6]);
        x = combine(x, y);
      }
      const int b = seq_of_row(tp.act_off, tp.B, r);
      const int64_t g = (int64_t)b * tp.N + tp.act_idx[r];
      finish_row<T, PREV>(rp, x, (const char*)rp.cur + g * rowbytes, C, tp.mask_id, r);
    }
    __syncthreads();
  }
  tail_phase(tp, sh);
}

static int kl_nseg(int M_tot, int V, int elem_bytes) {
  const int C = V * elem_bytes / 16;
  if (M_tot <= 0) return 1;
  const int want = (4096 + M_tot - 1) / M_tot;
  const int maxseg = C / (kKLThreads * 4) > 1 ? C / (kKLThreads * 4) : 1;
  int n = want < maxseg ? want : maxseg;
  return n < 1 ? 1 : n;
}

size_t kl_part_bytes(int M_tot, int V, int elem_bytes) {
  const int n_seg = kl_nseg(M_tot, V, elem_bytes);
  if (n_seg <= 1) return 256;
  return (size_t)(M_tot > 0 ? M_tot : 1) * n_seg * kPartWords * 4;
}

template <typename T, bool PREV>
static void kl_launch_t(const KLRowParams& rp, const TailParams& tp, float* part, hipStream_t s) {
  const int n_seg = kl_nseg(tp.M_tot, rp.V, sizeof(T));
  if (tp.M_tot > 0) {
    const int C = rp.V * (int)sizeof(T) / 16;
    const int seg_chunks = (C + n_seg - 1) / n_seg;
    hipLaunchKernelGGL((kl_rows_kernel<T, PREV>), dim3((unsigned)tp.M_tot * n_seg), dim3(kKLThreads), 0, s, rp, tp,
                       n_seg, seg_chunks, part);
  }
  hipLaunchKernelGGL((kl_tail_kernel<T, PREV>), dim3(1), dim3(kTailThreads), 0, s, rp, tp,
                     tp.M_tot > 0 ? n_seg : 1, (const float*)part);
}

hipError_t launch_kl_lock(int dtype, const KLRowParams& rp, const TailParams& tp, float* part, hipStream_t s) {
  const bool prev = tp.have_prev != 0;
  if (dtype == 0) {
    if (prev) kl_launch_t<bf16, true>(rp, tp, part, s);
    else kl_launch_t<bf16, false>(rp, tp, part, s);
  } else {
    if (prev) kl_launch_t<float, true>(rp, tp, part, s);
    else kl_launch_t<float, false>(rp, tp, part, s);
  }
  return hipGetLastError();
}

}  // namespace sl
