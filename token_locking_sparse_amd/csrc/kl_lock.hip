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

#include <type_traits>

#include "common.hpp"
#include "internal.hpp"
#include "klpart.hpp"

namespace sl {

// Workgroups of 4 waves: at the row pass's register use (under 96 VGPRs, 5 waves per SIMD) five of
// them fit a CU where two of 8 waves would leave a fifth of the wave slots empty.
constexpr int kKLThreads = 256;
constexpr int kTailThreads = 1024;

// ------------------------------------------------------------------ compaction
// Ascending positions with locked == 0 of B sequences of N.  Each round gives
// every thread `per` consecutive positions (4, 8 or 16, so that small totals
// still spread over every wave), read with one load; the per-thread counts are
// prefix-summed across the workgroup (DPP wave scan, then the wave totals
// through LDS), and each thread writes its run of active positions.  One
// division per thread and round locates its first position; later ones step.
// s_w: LDS scratch of blockDim/64 ints.
__device__ __forceinline__ int block_excl_scan(int c, int& total, int* s_w) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, nw = blockDim.x >> 6;
  const int inc = wave_incl_scan(c);
  if (lane == 63) s_w[wid] = inc;
  __syncthreads();
  int wpre = 0, tot = 0;
  for (int w = 0; w < nw; ++w) {
    const int x = s_w[w];
    wpre += (w < wid) ? x : 0;
    tot += x;
  }
  __syncthreads();   // s_w is reused by the next round
  total = tot;
  return wpre + inc - c;
}

// Flags f[i0 .. i0+per) with one load when aligned (per = 4, 8 or 16); bit j of
// the result: position i0 + j is in range and unlocked.
__device__ __forceinline__ uint32_t active_bits(const uint8_t* f, int i0, int per, int total) {
  uint32_t w[4] = {0xffffffffu, 0xffffffffu, 0xffffffffu, 0xffffffffu};   // past the end: locked
  const bool whole = i0 + per <= total && ((uintptr_t)(f + i0) & (per - 1)) == 0;
  if (whole && per == 16) {
    const u32x4 v = ld16(f + i0);
    w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
  } else if (whole && per == 8) {
    const uint2 v = *(const uint2*)(f + i0);
    w[0] = v.x; w[1] = v.y;
  } else if (whole) {
    w[0] = *(const uint32_t*)(f + i0);
  } else {
    for (int j = 0; j < per; ++j) {
      const uint32_t x = (i0 + j < total) ? (uint32_t)f[i0 + j] : 0xffu;
      w[j >> 2] = (w[j >> 2] & ~(0xffu << (8 * (j & 3)))) | (x << (8 * (j & 3)));
    }
  }
  uint32_t am = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j)
    am |= (((w[j >> 2] >> (8 * (j & 3))) & 0xffu) == 0u ? 1u : 0u) << j;
  return per == 16 ? am : am & ((1u << per) - 1u);
}

__device__ __forceinline__ void block_compact(const uint8_t* locked, int B, int N, int32_t* act_idx,
                                              int32_t* act_off, int* s_w) {
  const int tid = threadIdx.x, bd = blockDim.x;
  const int total = B * N;
  const int need = (total + bd - 1) / bd;
  const int per = need <= 4 ? 4 : (need <= 8 ? 8 : 16);
  int base = 0;
  for (int r0 = 0; r0 < total; r0 += per * bd) {
    const int i0 = r0 + per * tid;
    const uint32_t am = active_bits(locked, i0, per, total);
    int tot;
    int pos = base + block_excl_scan(__popc(am), tot, s_w);
    if (i0 < total) {
      int q = i0 / N, rr = i0 - q * N;
      for (int j = 0; j < per && i0 + j < total; ++j) {
        if (rr == 0) act_off[q] = pos;
        if ((am >> j) & 1u) act_idx[pos++] = rr;
        if (++rr == N) { rr = 0; ++q; }
      }
    }
    base += tot;
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
// Sequences whose gate quantile and lock update run side by side (a group of waves each).
constexpr int kSelGroups = 8;
constexpr int kGrpRegs = 16;   // values a thread of a group holds

struct TailShared {
  int w[16];
  uint32_t hist[3][256];   // radix-select histograms, used round-robin
  uint32_t mm[32];         // per-wave min / max of the select's values
  float fv[16];
  int iv[32];
  uint32_t ghist[kSelGroups][3][256];   // per-group histograms of the grouped select
  int gpass[kSelGroups];                 // digit passes each group needs
};

// Up to kRegSel values of a sequence per thread are held in registers; longer
// sequences are read from global memory on every pass.
constexpr int kRegSel = 4;
constexpr uint32_t kNoValue = 0xffffffffu;   // not a non-negative float's pattern

// One 8-bit digit of the radix select, run by every wave on the complete
// histogram h: find the bucket holding the kk-th value, extend the prefix and
// rebase kk.  All waves reach the same answer, so nothing is broadcast.
__device__ __forceinline__ void radix_digit(const uint32_t* h, int& kk, int shift, uint32_t& prefix,
                                            uint32_t& pmask) {
  const int lane = threadIdx.x & 63;
  int c[4], ls = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) { c[j] = (int)h[4 * lane + j]; ls += c[j]; }
  const int inc = wave_incl_scan(ls);
  const int ex = inc - ls;
  const bool mine = ex <= kk && kk < inc;   // exactly one lane
  int run = ex, j = 0;
  if (mine)
    while (j < 3 && run + c[j] <= kk) { run += c[j]; ++j; }
  const int src = __ffsll((unsigned long long)__ballot(mine)) - 1;
  const int bucket = __builtin_amdgcn_readlane(4 * lane + j, src);
  const int rem = __builtin_amdgcn_readlane(kk - run, src);
  prefix |= ((uint32_t)bucket) << shift;
  pmask |= 255u << shift;
  kk = rem;
}

// k-th smallest (0-based) of non-negative floats, exact, by a radix select on
// their bit patterns (monotone for x >= 0).  The values are either v[]
// (kNoValue = absent) or, when from_regs is false, u[o0..o1).  The high bits
// shared by the smallest and largest value are fixed first, so the 8-bit
// digit passes start at the first bit where the values differ (this also
// spreads the first histogram when the values cluster, as 1 - max p does).
// One barrier per pass: pass q counts into hist[q % 3] while clearing
// hist[(q + 1) % 3], whose last readers finished before the previous barrier.
__device__ float block_select_kth(const uint32_t (&v)[kRegSel], bool from_regs, const float* u, int o0,
                                  int o1, int k, TailShared& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, nw = blockDim.x >> 6;
  __syncthreads();   // earlier readers of sh.hist / sh.mm are done
  uint32_t lo = 0xffffffffu, hi = 0u;
  if (from_regs) {
#pragma unroll
    for (int i = 0; i < kRegSel; ++i)
      if (v[i] != kNoValue) { lo = min(lo, v[i]); hi = max(hi, v[i]); }
  } else {
    for (int m = o0 + tid; m < o1; m += blockDim.x) {
      const uint32_t x = __float_as_uint(u[m]);
      lo = min(lo, x); hi = max(hi, x);
    }
  }
  lo = wave_min_u32(lo);
  hi = wave_max_u32(hi);
  if (lane == 0) { sh.mm[wid] = lo; sh.mm[16 + wid] = hi; }
  for (int i = tid; i < 256; i += blockDim.x) sh.hist[0][i] = 0;
  __syncthreads();
  lo = 0xffffffffu; hi = 0u;
  for (int w = 0; w < nw; ++w) { lo = min(lo, sh.mm[w]); hi = max(hi, sh.mm[16 + w]); }
  if (lo == hi) return __uint_as_float(lo);
  const int free_bits = 32 - __clz((int)(lo ^ hi));   // bits below the shared prefix
  uint32_t pmask = free_bits >= 32 ? 0u : ~((1u << free_bits) - 1u);
  uint32_t prefix = lo & pmask;
  int kk = k;
  int shift = free_bits > 8 ? free_bits - 8 : 0;
  for (int q = 0;; ++q) {
    uint32_t* h = sh.hist[q % 3];
    if (from_regs) {
      // values sit densely in the first waves (kRegSel per thread); the rest skip
      if (wid * 64 * kRegSel < o1 - o0)
#pragma unroll
      for (int i = 0; i < kRegSel; ++i) {
        bool act = v[i] != kNoValue && (v[i] & pmask) == prefix;
        const uint32_t d = (v[i] >> shift) & 255u;
        // lanes sharing the first active lane's digit add once (values cluster)
        const unsigned long long m = __ballot(act);
        if (m != 0ull) {
          const int leader = __ffsll(m) - 1;
          const uint32_t dl = (uint32_t)__builtin_amdgcn_readlane((int)d, leader);
          const unsigned long long same = __ballot(act && d == dl);
          if (lane == leader) atomicAdd(&h[dl], (uint32_t)__popcll(same));
          act = act && d != dl;
        }
        if (act) atomicAdd(&h[d], 1u);
      }
    } else {
      for (int m = o0 + tid; m < o1; m += blockDim.x) {
        const uint32_t x = __float_as_uint(u[m]);
        if ((x & pmask) == prefix) atomicAdd(&h[(x >> shift) & 255u], 1u);
      }
    }
    for (int i = tid; i < 256; i += blockDim.x) sh.hist[(q + 1) % 3][i] = 0;
    __syncthreads();
    radix_digit(h, kk, shift, prefix, pmask);
    if (shift == 0) break;
    shift = shift > 8 ? shift - 8 : 0;
  }
  return __uint_as_float(prefix);
}

// Gate quantile and lock update of several sequences at once (B > 1, gate on): the workgroup's waves
// form min(B, kSelGroups) groups, each taking one sequence per round; a group holds up to kGrpRegs
// consecutive rows per thread in registers and runs the same radix select as block_select_kth on
// histograms of its own, every group advancing one digit per workgroup barrier.  Returns false
// (and does nothing) when a sequence does not fit its group's registers.
__device__ bool tail_select_lock_grouped(const TailParams& p, TailShared& sh, int t_now) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, nw = blockDim.x >> 6;
  const int G = p.B < kSelGroups ? p.B : kSelGroups;
  const int wpg = nw / G;                       // waves per group
  const int cap = wpg * 64 * kGrpRegs;
  for (int b = 0; b < p.B; ++b)
    if (p.act_off[b + 1] - p.act_off[b] > cap) return false;   // uniform: every thread reads the same
  const int g = wid / wpg, gt = tid - g * wpg * 64;   // group, thread within it
  const bool in_group = g < G;
  const bool can_lock = p.eps > 0.f && p.have_prev;
  for (int b0 = 0; b0 < p.B; b0 += G) {
    const int b = b0 + g;
    const bool live = in_group && b < p.B;
    int o0 = 0, o1 = 0;
    if (live) { o0 = p.act_off[b]; o1 = p.act_off[b + 1]; }
    const int n = o1 - o0;
    uint32_t uv[kGrpRegs];
    float kv[kGrpRegs];
    int pv[kGrpRegs];
#pragma unroll
    for (int i = 0; i < kGrpRegs; ++i) {
      const int m = o0 + gt * kGrpRegs + i;   // dense: only the group's first waves hold values
      const bool in = live && m < o1;
      uv[i] = in ? __float_as_uint(p.u[m]) : kNoValue;
      kv[i] = in ? p.kl[m] : INFINITY;
      pv[i] = in ? p.act_idx[m] : -1;
    }
    // the group's min and max, and the digit passes it needs
    uint32_t lo = 0xffffffffu, hi = 0u;
#pragma unroll
    for (int i = 0; i < kGrpRegs; ++i)
      if (uv[i] != kNoValue) { lo = min(lo, uv[i]); hi = max(hi, uv[i]); }
    lo = wave_min_u32(lo);
    hi = wave_max_u32(hi);
    __syncthreads();   // earlier readers of sh.mm / sh.ghist / sh.gpass are done
    if (lane == 0) { sh.mm[wid] = lo; sh.mm[16 + wid] = hi; }
    if (in_group)
      for (int i = gt; i < 256; i += wpg * 64) sh.ghist[g][0][i] = 0;
    __syncthreads();
    lo = 0xffffffffu; hi = 0u;
    if (in_group)
      for (int w = g * wpg; w < (g + 1) * wpg; ++w) { lo = min(lo, sh.mm[w]); hi = max(hi, sh.mm[16 + w]); }
    const bool sel = live && n > 0;
    const int k = sel ? (int)floor((double)p.gate_q * (double)(n - 1)) : 0;
    int free_bits = 0, passes = 0;
    uint32_t pmask = 0u, prefix = lo;
    if (sel && lo != hi) {
      free_bits = 32 - __clz((int)(lo ^ hi));
      pmask = free_bits >= 32 ? 0u : ~((1u << free_bits) - 1u);
      prefix = lo & pmask;
      passes = (free_bits + 7) / 8;
    }
    if (in_group && gt == 0) sh.gpass[g] = passes;
    __syncthreads();
    int max_pass = 0;
    for (int j = 0; j < G; ++j) max_pass = max(max_pass, sh.gpass[j]);
    int kk = k;
    int shift = free_bits > 8 ? free_bits - 8 : 0;
    for (int q = 0; q < max_pass; ++q) {
      const bool act = q < passes;   // uniform over the group
      uint32_t* h = sh.ghist[in_group ? g : 0][q % 3];
      if (act) {
#pragma unroll
        for (int i = 0; i < kGrpRegs; ++i) {
          bool a = uv[i] != kNoValue && (uv[i] & pmask) == prefix;
          const uint32_t d = (uv[i] >> shift) & 255u;
          // lanes sharing the first active lane's digit add once (values cluster)
          const unsigned long long m = __ballot(a);
          if (m != 0ull) {
            const int leader = __ffsll(m) - 1;
            const uint32_t dl = (uint32_t)__builtin_amdgcn_readlane((int)d, leader);
            const unsigned long long same = __ballot(a && d == dl);
            if (lane == leader) atomicAdd(&h[dl], (uint32_t)__popcll(same));
            a = a && d != dl;
          }
          if (a) atomicAdd(&h[d], 1u);
        }
      }
      if (in_group)
        for (int i = gt; i < 256; i += wpg * 64) sh.ghist[g][(q + 1) % 3][i] = 0;
      __syncthreads();
      if (act) {
        radix_digit(h, kk, shift, prefix, pmask);
        shift = shift > 8 ? shift - 8 : 0;
      }
    }
    const float thr = sel ? __uint_as_float(prefix) : INFINITY;
    if (live && gt == 0 && p.gate_thr) p.gate_thr[b] = thr;
    if (live && can_lock) {
      const int64_t gb = (int64_t)b * p.N;
      bool ok[kGrpRegs];
#pragma unroll
      for (int i = 0; i < kGrpRegs; ++i)
        ok[i] = pv[i] >= 0 && kv[i] <= p.eps && __uint_as_float(uv[i]) <= thr;
      if (p.cand) {
#pragma unroll
        for (int i = 0; i < kGrpRegs; ++i) ok[i] = ok[i] && (p.cand[gb + (ok[i] ? pv[i] : 0)] != 0);
      }
#pragma unroll
      for (int i = 0; i < kGrpRegs; ++i) {
        if (ok[i]) {
          p.locked[gb + pv[i]] = 1;
          if (p.lock_step) p.lock_step[gb + pv[i]] = t_now;
        }
      }
    }
  }
  __syncthreads();
  return true;
}

// Gate quantile, lock update, optional sampler, compaction — one workgroup.
// A sequence of at most kRegSel * blockDim active rows is read once into
// registers, kRegSel consecutive rows per thread (positions, u, KL, then the
// candidate flags), and its select and lock update run from there.
__device__ void tail_phase(const TailParams& p, TailShared& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, nw = blockDim.x >> 6;
  const int bd = blockDim.x;
  const bool gate = p.gate_q >= 0.f;
  const bool can_lock = p.eps > 0.f && p.have_prev;
  const int t_now = p.t_dev ? p.t_dev[0] : p.t;   // step index recorded in lock_step
  // several sequences with the gate: their selects and lock updates side by side
  const bool grouped = gate && p.B > 1 && tail_select_lock_grouped(p, sh, t_now);
  for (int b = 0; b < p.B; ++b) {
    const int o0 = p.act_off[b], o1 = p.act_off[b + 1];
    const int n = o1 - o0;
    if (grouped && p.unmask_k <= 0) break;   // nothing left per sequence
    if (!grouped) {   // select and lock update of this sequence alone
      const bool regs = n <= kRegSel * bd;
      uint32_t uv[kRegSel];
      float kv[kRegSel];
      int pv[kRegSel];
#pragma unroll
      for (int i = 0; i < kRegSel; ++i) {
        const int m = o0 + tid * kRegSel + i;   // dense: only the first waves hold values
        const bool in = regs && m < o1;
        uv[i] = in ? __float_as_uint(p.u[m]) : kNoValue;
        kv[i] = in ? p.kl[m] : INFINITY;
        pv[i] = in ? p.act_idx[m] : -1;
      }
      float thr = INFINITY;
      if (gate && n > 0) {
        const int k = (int)floor((double)p.gate_q * (double)(n - 1));
        thr = block_select_kth(uv, regs, p.u, o0, o1, k, sh);
      }
      if (tid == 0 && p.gate_thr) p.gate_thr[b] = thr;
      if (can_lock) {
        const int64_t gb = (int64_t)b * p.N;
        if (regs) {
          bool ok[kRegSel];
#pragma unroll
          for (int i = 0; i < kRegSel; ++i) {
            ok[i] = pv[i] >= 0 && kv[i] <= p.eps;
            if (gate) ok[i] = ok[i] && (__uint_as_float(uv[i]) <= thr);
          }
          if (p.cand) {
#pragma unroll
            for (int i = 0; i < kRegSel; ++i) ok[i] = ok[i] && (p.cand[gb + (ok[i] ? pv[i] : 0)] != 0);
          }
#pragma unroll
          for (int i = 0; i < kRegSel; ++i) {
            if (ok[i]) {
              p.locked[gb + pv[i]] = 1;
              if (p.lock_step) p.lock_step[gb + pv[i]] = t_now;
            }
          }
        } else {
          for (int m = o0 + tid; m < o1; m += bd) {
            const int64_t g = gb + p.act_idx[m];
            bool ok = (p.cand == nullptr) || (p.cand[g] != 0);
            ok = ok && (p.kl[m] <= p.eps);
            if (gate) ok = ok && (p.u[m] <= thr);
            if (ok) {
              p.locked[g] = 1;
              if (p.lock_step) p.lock_step[g] = t_now;
            }
          }
        }
      }
    }
    // Sampler: the unmask_k most confident [MASK] positions take their argmax.
    // It runs after the lock update, which reads the candidate flags it sets.
    __syncthreads();
    for (int r = 0; r < p.unmask_k; ++r) {
      float bc = -1.f;
      int bp = INT_MAX, bm = -1;
      for (int m = o0 + tid; m < o1; m += bd) {
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
// Lane (l - shift) within the row of 16, or the identity partial where that
// lane lies outside the row / the row is masked off (DPP, no LDS round trip).
template <int CTRL, int RM>
__device__ __forceinline__ Part dpp_part(const Part& x) {
  const int ninf = __float_as_int(-INFINITY);
  Part y;
  y.ma = __int_as_float(dpp_i<CTRL, RM>(ninf, __float_as_int(x.ma)));
  y.sa = __int_as_float(dpp_i<CTRL, RM>(0, __float_as_int(x.sa)));
  y.ta = __int_as_float(dpp_i<CTRL, RM>(0, __float_as_int(x.ta)));
  y.mb = __int_as_float(dpp_i<CTRL, RM>(ninf, __float_as_int(x.mb)));
  y.sb = __int_as_float(dpp_i<CTRL, RM>(0, __float_as_int(x.sb)));
  y.best = __int_as_float(dpp_i<CTRL, RM>(ninf, __float_as_int(x.best)));
  y.bidx = dpp_i<CTRL, RM>(INT_MAX, x.bidx);
  return y;
}

// Combine the partials of the 64 lanes (the same steps as wave_incl_scan);
// lane 63 ends with the wave's total, which is returned to every lane.
__device__ __forceinline__ Part wave_reduce_part(Part p) {
  p = combine(p, dpp_part<kRowShr1, 0xf>(p));
  p = combine(p, dpp_part<kRowShr2, 0xf>(p));
  p = combine(p, dpp_part<kRowShr4, 0xf>(p));
  p = combine(p, dpp_part<kRowShr8, 0xf>(p));
  p = combine(p, dpp_part<kRowBcast15, 0xa>(p));
  p = combine(p, dpp_part<kRowBcast31, 0xc>(p));
  Part t;
  t.ma = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p.ma), 63));
  t.sa = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p.sa), 63));
  t.ta = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p.ta), 63));
  t.mb = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p.mb), 63));
  t.sb = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p.sb), 63));
  t.best = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p.best), 63));
  t.bidx = __builtin_amdgcn_readlane(p.bidx, 63);
  return t;
}

// Exact argmax inside the 16-byte chunk `c` whose raw bits are `raw`: the
// lowest id equal to `best` that is not the mask, or INT_MAX when c < 0 (no
// finite maximum was seen).
template <typename T>
__device__ __forceinline__ int resolve_argmax(const u32x4& raw, int c, float best, int mask_id) {
  constexpr int E = Chunk<T>::kElems;
  if (c < 0 || c == INT_MAX) return INT_MAX;
  float a[E];
  Chunk<T>::unpack(raw, a);
  int am = INT_MAX;
#pragma unroll
  for (int j = E - 1; j >= 0; --j)
    if (a[j] == best && c * E + j != mask_id) am = c * E + j;
  return am;
}

constexpr int GroupChunks = 4;   // chunks per thread per streaming step of the row pass

// Lowest id != mask_id holding `best` in the argmax group g of a row (row bytes at `row`): its
// chunks g, g + kKLThreads, ... below c1.  INT_MAX when none does.  Every chunk is loaded before
// any is scanned.
template <typename T>
__device__ int resolve_group(const char* row, int g, int c1, float best, int mask_id) {
  u32x4 raw[GroupChunks];
#pragma unroll
  for (int u = 0; u < GroupChunks; ++u)
    if (g + u * kKLThreads < c1) raw[u] = ld16(row + (size_t)(g + u * kKLThreads) * 16);
#pragma unroll
  for (int u = 0; u < GroupChunks; ++u) {
    if (g + u * kKLThreads < c1) {
      const int id = resolve_argmax<T>(raw[u], g + u * kKLThreads, best, mask_id);
      if (id != INT_MAX) return id;   // chunks ascend: the first hit is the lowest id
    }
  }
  return INT_MAX;
}

__device__ __forceinline__ int wave_min_i32(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = min(v, __shfl_xor(v, o, 64));
  return v;
}

// KL(p || q) of a row from its (combined) partial: with S_a = sum e^(a - max a),
// A = max a + ln S_a and B the LSE of the previous logits,
// KL = sum p (a - b) - A + B.  PLSE: B is the partial's mb (known from the pass
// that produced the previous posterior); otherwise B = mb + ln S_b.
template <bool PREV, bool PLSE>
__device__ __forceinline__ float row_kl(const Part& t) {
  if (!PREV) return INFINITY;
  if (PLSE) return (t.ta / t.sa - logf(t.sa)) - (t.ma - t.mb);
  return t.ta / t.sa - (t.ma - t.mb) - logf(t.sa / t.sb);
}

// Row statistics from a (combined) partial whose `bidx` is the exact argmax
// (INT_MAX: none): A = max a + ln S_a, max p = 1/S_a, and the KL above.  g is
// the row's position b*N + pos (where the per-position LSE store takes A).
template <bool PREV, bool PLSE>
__device__ void finish_row(const KLRowParams& rp, const Part& t, int r, int g) {
  const float A = t.ma + logf(t.sa);
  rp.lse[r] = A;
  if (rp.lse_pos) rp.lse_pos[g] = A;
  rp.u[r] = 1.f - 1.f / t.sa;
  rp.kl[r] = row_kl<PREV, PLSE>(t);
  if (rp.argmax) rp.argmax[r] = t.bidx == INT_MAX ? 0 : t.bidx;
  if (rp.conf) rp.conf[r] = __expf(t.best - t.ma) / t.sa;
}

// Row pass: workgroup (row r, segment) streams its slice of the current and
// previous logits once.  With one segment per row it finishes the row itself;
// otherwise it stores its partial for the tail kernel.  No inter-workgroup
// communication happens inside this kernel.  PLSE (with PREV): the previous
// posterior's LSE comes from the pass that produced it (rp.lse_prev), so the
// previous logits enter only the sum p (a - b): no exponential, maximum or
// sum of their own.
template <typename T, bool PREV, bool PLSE>
__global__ void __launch_bounds__(kKLThreads)
kl_rows_kernel(KLRowParams rp, TailParams tp, int n_seg, int seg_chunks, float* part) {
  constexpr int E = Chunk<T>::kElems;
  __shared__ Part s_part[kKLThreads / 64];
  __shared__ int s_id[kKLThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int r = blockIdx.x / n_seg, seg = blockIdx.x - r * n_seg;
  if (r >= rows_live(tp.M_tot, tp.m_dev)) return;   // uniform over the workgroup, before any barrier
  const int b = seq_of_row(tp.act_off, tp.B, r);
  const int64_t g = (int64_t)b * tp.N + tp.act_idx[r];
  const float lse_b = PLSE ? rp.lse_prev[g] : 0.f;   // consumed after the streaming loop
  const size_t rowbytes = (size_t)rp.V * sizeof(T);
  const char* crow = (const char*)rp.cur + g * rowbytes;
  const char* prow = (const char*)rp.prev + g * rowbytes;
  const int C = rp.V / E;
  const int c0 = seg * seg_chunks;
  const int c1 = min(C, c0 + seg_chunks);
  const int mask_id = tp.mask_id;
  // chunk holding the [MASK] id (never matches when there is none): it is left
  // out of the argmax tracking in the streaming loops and folded in afterwards
  const int mask_chunk = mask_id >= 0 ? mask_id / E : -1;

  Part acc;
  acc.ma = -INFINITY; acc.sa = 0.f; acc.ta = 0.f;
  acc.mb = -INFINITY; acc.sb = 0.f;
  acc.best = -INFINITY; acc.bidx = INT_MAX;

  // Groups of U chunks per thread (strided by the workgroup size, so every load
  // instruction of the workgroup covers a contiguous 4 KB): U loads of each row
  // in flight, one running-max rescale per group.  Segments hold whole groups
  // except at the end of the row, where one last group loads only the chunks
  // below c1 (the others read as -inf and add nothing), so every thread keeps
  // U loads per row in flight to the end.  The argmax is tracked per group:
  // acc.best is the largest value seen over ids != mask_id, acc.bidx the first
  // chunk of the group that holds it; the exact id is found after the loop,
  // only by the threads whose value is the workgroup's maximum.
  constexpr int U = GroupChunks;
  constexpr uint32_t kNegInfBits = sizeof(T) == 2 ? 0xff80ff80u : 0xff800000u;   // -inf in every element
  int c = c0 + tid;
  auto group = [&](auto partial) {
    constexpr bool P = decltype(partial)::value;
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) ok[u] = !P || c + u * kKLThreads < c1;
    // past the end: the last chunk again (in bounds), read as -inf
    uint32_t off[U];
#pragma unroll
    for (int u = 0; u < U; ++u) off[u] = (uint32_t)(ok[u] ? c + u * kKLThreads : c1 - 1) * 16u;
    u32x4 ra[U], rb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) ra[u] = ld16_stream(crow + off[u]);
    if (PREV) {
#pragma unroll
      for (int u = 0; u < U; ++u) rb[u] = ld16_stream(prow + off[u]);
    }
    if (P) {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          ra[u][q] = ok[u] ? ra[u][q] : kNegInfBits;
          rb[u][q] = ok[u] ? rb[u][q] : kNegInfBits;
        }
    }
    float a[U][E];
#pragma unroll
    for (int u = 0; u < U; ++u) Chunk<T>::unpack(ra[u], a[u]);
    float cm[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      cm[u] = a[u][0];
#pragma unroll
      for (int j = 1; j < E; ++j) cm[u] = __builtin_fmaxf(cm[u], a[u][j]);
    }
    const float gm = __builtin_fmaxf(__builtin_fmaxf(cm[0], cm[1]), __builtin_fmaxf(cm[2], cm[3]));
    // the group's maximum over ids != mask_id: the [MASK] chunk, when it is one of the
    // group's, is left out here and handled after the loop
    float gx = gm;
    const unsigned mrel = (unsigned)(mask_chunk - c);
    if (mrel < (unsigned)(U * kKLThreads) && (mrel & (kKLThreads - 1)) == 0) {
      gx = -INFINITY;
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (mrel != (unsigned)(u * kKLThreads)) gx = __builtin_fmaxf(gx, cm[u]);
    }
    if (gx > acc.best) { acc.best = gx; acc.bidx = c; }   // strictly greater: the earliest group wins
    const float mnew = __builtin_fmaxf(acc.ma, gm);
    const float sc = scale_to(acc.ma, mnew);
    acc.sa *= sc;
    acc.ta *= sc;
    acc.ma = mnew;
    const float ml = mnew * kLog2e;
    if (PREV) {
      float b[U][E];
#pragma unroll
      for (int u = 0; u < U; ++u) Chunk<T>::unpack(rb[u], b[u]);
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int j = 0; j < E; ++j) {
          const float e = __builtin_amdgcn_exp2f(fmaf(a[u][j], kLog2e, -ml));
          acc.sa += e;
          // chunks past the row's end: e = 0, and their a - b (-inf - -inf) must not enter
          acc.ta = fmaf(e, ok[u] ? a[u][j] - b[u][j] : 0.f, acc.ta);
        }
      if (!PLSE) {
        float bm = -INFINITY;
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int j = 0; j < E; ++j) bm = __builtin_fmaxf(bm, b[u][j]);
        const float mbn = __builtin_fmaxf(acc.mb, bm);
        acc.sb *= scale_to(acc.mb, mbn);
        acc.mb = mbn;
        const float mbl = mbn * kLog2e;
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int j = 0; j < E; ++j) acc.sb += __builtin_amdgcn_exp2f(fmaf(b[u][j], kLog2e, -mbl));
      }
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int j = 0; j < E; ++j) acc.sa += __builtin_amdgcn_exp2f(fmaf(a[u][j], kLog2e, -ml));
    }
  };
  for (; c + (U - 1) * kKLThreads < c1; c += U * kKLThreads) group(std::false_type{});
  if (c < c1) group(std::true_type{});
  // the [MASK] chunk, if this thread streamed it: its largest value over the other ids
  float mbest = -INFINITY;
  u32x4 mraw = {0u, 0u, 0u, 0u};
  if (mask_chunk >= c0 && mask_chunk < c1 && (mask_chunk - c0) % kKLThreads == tid) {
    float a[E];
    mraw = ld16(crow + (size_t)mask_chunk * 16);
    Chunk<T>::unpack(mraw, a);
    for (int j = 0; j < E; ++j)
      if (mask_chunk * E + j != mask_id) mbest = __builtin_fmaxf(mbest, a[j]);
  }
  const float my_best = acc.best;
  const int my_grp = acc.bidx;
  acc.best = __builtin_fmaxf(acc.best, mbest);
  acc.bidx = INT_MAX;
  if (PLSE) { acc.mb = lse_b; acc.sb = 0.f; }   // the same on every lane: combine keeps it
  acc = wave_reduce_part(acc);
  if (lane == 0) s_part[wid] = acc;
  __syncthreads();
  // the workgroup's maximum; the threads holding it find the lowest id with that value
  float wbest = s_part[0].best;
#pragma unroll
  for (int w = 1; w < kKLThreads / 64; ++w) wbest = __builtin_fmaxf(wbest, s_part[w].best);
  int id = INT_MAX;
  if (wbest > -INFINITY) {
    if (my_best == wbest) id = resolve_group<T>(crow, my_grp, c1, wbest, mask_id);
    if (mbest == wbest) id = min(id, resolve_argmax<T>(mraw, mask_chunk, wbest, mask_id));
  }
  id = wave_min_i32(id);
  if (lane == 0) s_id[wid] = id;
  __syncthreads();
  if (tid == 0) {
    Part t = s_part[0];
    int tid_min = s_id[0];
    for (int w = 1; w < kKLThreads / 64; ++w) { t = combine(t, s_part[w]); tid_min = min(tid_min, s_id[w]); }
    t.best = wbest;
    t.bidx = tid_min;
    if (n_seg == 1) finish_row<PREV, PLSE>(rp, t, r, (int)g);
    else store_part(part + ((size_t)seg * tp.M_tot + r) * kPartWords, t, (int)g);
  }
}

// Tail kernel (one workgroup): merge the segment partials of every row (when a
// row was split), then gate quantile, lock update, sampler and compaction.
// The merge takes kMergeRows rows per thread per round and issues every
// partial load of the round before combining.
constexpr int kMaxSeg = 4;
constexpr int kMergeRows = 2;

// When the lock mask and the active rows fit in LDS, the tail issues every
// global load it needs (partials or row statistics, positions, lock and
// candidate flags) at once, and the select, lock update and compaction then
// run on the LDS copies; the lock mask is written back at the end.  Each
// dependent round trip to HBM costs microseconds, and the single workgroup
// would otherwise make four of them.
constexpr int kTailPos = 16 * kTailThreads;   // B*N held in LDS (16 flags per thread)
constexpr int kTailRowsPerThread = 8;
constexpr int kTailRows = kTailRowsPerThread * kTailThreads;
struct TailLds {
  uint8_t lk[kTailPos];   // lock flags, updated in place
  uint8_t cd[kTailPos];   // candidate flags
  float u[kTailRows];
  float kl[kTailRows];
  int32_t ai[kTailRows];
};

__device__ __forceinline__ u32x4 load_flags16(const uint8_t* f, int p0, int P, uint32_t fill) {
  if (((uintptr_t)f & 15) == 0 && p0 + 16 <= P) return ld16(f + p0);
  u32x4 w = {fill, fill, fill, fill};
  for (int j = 0; j < 16; ++j) {
    const uint32_t x = p0 + j < P ? (uint32_t)f[p0 + j] : (fill & 0xffu);
    w[j >> 2] = (w[j >> 2] & ~(0xffu << (8 * (j & 3)))) | (x << (8 * (j & 3)));
  }
  return w;
}

template <typename T, bool PREV, bool PLSE>
__device__ void tail_from_lds(const KLRowParams& rp, const TailParams& tp, int n_seg, const float* part,
                              TailShared& sh, TailLds& ls) {
  const int tid = threadIdx.x, bd = blockDim.x;
  const int P = tp.B * tp.N, Mt = rows_live(tp.M_tot, tp.m_dev), Mcap = tp.M_tot;
  const int p0 = 16 * tid;
  // every global load first
  const u32x4 lkv = load_flags16(tp.locked, p0, P, 0x01010101u);
  const u32x4 cdv = tp.cand ? load_flags16(tp.cand, p0, P, 0u) : u32x4{0x01010101u, 0x01010101u, 0x01010101u, 0x01010101u};
  int32_t ai[kTailRowsPerThread];
  float uu[kTailRowsPerThread], kk[kTailRowsPerThread];
#pragma unroll
  for (int j = 0; j < kTailRowsPerThread; ++j) {
    const int m = tid + j * bd;
    ai[j] = m < Mt ? tp.act_idx[m] : 0;
    if (n_seg == 1) {
      uu[j] = m < Mt ? rp.u[m] : 0.f;
      kk[j] = m < Mt ? rp.kl[m] : 0.f;
    }
  }
  Part x[kMergeRows][kMaxSeg];
  int gpos[kMergeRows];   // positions b*N + pos, carried by the first segment's partial
  if (n_seg > 1 && Mt > 0) {   // n_seg > 1 only when M_tot < kMergeRows * blockDim: one round
#pragma unroll
    for (int k = 0; k < kMergeRows; ++k) {
      const int r = min(tid + k * bd, Mt - 1);   // clamped: loads stay in bounds
#pragma unroll
      for (int s2 = 0; s2 < kMaxSeg; ++s2)
        if (s2 < n_seg) x[k][s2] = load_part(part + ((size_t)s2 * Mcap + r) * kPartWords, s2 == 0 ? &gpos[k] : nullptr);
    }
  }
  // LDS copies
  if (p0 < kTailPos) {
    *(u32x4*)(ls.lk + p0) = lkv;
    *(u32x4*)(ls.cd + p0) = cdv;
  }
#pragma unroll
  for (int j = 0; j < kTailRowsPerThread; ++j) {
    const int m = tid + j * bd;
    ls.ai[m] = ai[j];
    if (n_seg == 1) { ls.u[m] = uu[j]; ls.kl[m] = kk[j]; }
  }
  if (n_seg > 1 && Mt > 0) {
#pragma unroll
    for (int k = 0; k < kMergeRows; ++k) {
      Part t = x[k][0];
#pragma unroll
      for (int s2 = 1; s2 < kMaxSeg; ++s2)
        if (s2 < n_seg) t = combine(t, x[k][s2]);
      const int r = tid + k * bd;
      if (r < Mt) {
        finish_row<PREV, PLSE>(rp, t, r, gpos[k]);
        ls.u[r] = 1.f - 1.f / t.sa;
        ls.kl[r] = row_kl<PREV, PLSE>(t);
      }
    }
  }
  __syncthreads();
  TailParams q = tp;
  q.M_tot = Mt;
  q.m_dev = nullptr;
  q.locked = ls.lk;
  q.cand = tp.cand ? ls.cd : nullptr;
  q.u = ls.u;
  q.kl = ls.kl;
  q.act_idx = ls.ai;
  tail_phase(q, sh);
  __syncthreads();
  // write the lock mask back
  if (p0 < P) {
    if (((uintptr_t)tp.locked & 15) == 0 && p0 + 16 <= P) {
      st16(tp.locked + p0, *(const u32x4*)(ls.lk + p0));
    } else {
      for (int j = 0; j < 16 && p0 + j < P; ++j) tp.locked[p0 + j] = ls.lk[p0 + j];
    }
  }
}

template <typename T, bool PREV, bool PLSE>
__global__ void __launch_bounds__(kTailThreads)
kl_tail_kernel(KLRowParams rp, TailParams tp, int n_seg, const float* part) {
  __shared__ TailShared sh;
  __shared__ __attribute__((aligned(16))) TailLds ls;
  const int Mt = rows_live(tp.M_tot, tp.m_dev);   // tp.M_tot: capacity and stride of the partials
  if ((long)tp.B * tp.N <= kTailPos && tp.M_tot <= kTailRows && Mt > 0) {
    tail_from_lds<T, PREV, PLSE>(rp, tp, n_seg, part, sh, ls);
  } else {
    if (n_seg > 1 && Mt > 0) {
      const int bd = blockDim.x;
      for (int r0 = 0; r0 < Mt; r0 += kMergeRows * bd) {
        Part x[kMergeRows][kMaxSeg];
        int gpos[kMergeRows];
#pragma unroll
        for (int k = 0; k < kMergeRows; ++k) {
          const int r = min(r0 + (int)threadIdx.x + k * bd, Mt - 1);   // clamped: loads stay in bounds
#pragma unroll
          for (int s2 = 0; s2 < kMaxSeg; ++s2)
            if (s2 < n_seg)
              x[k][s2] = load_part(part + ((size_t)s2 * tp.M_tot + r) * kPartWords, s2 == 0 ? &gpos[k] : nullptr);
        }
#pragma unroll
        for (int k = 0; k < kMergeRows; ++k) {
          Part t = x[k][0];
#pragma unroll
          for (int s2 = 1; s2 < kMaxSeg; ++s2)
            if (s2 < n_seg) t = combine(t, x[k][s2]);
          const int r = r0 + (int)threadIdx.x + k * bd;
          if (r < Mt) finish_row<PREV, PLSE>(rp, t, r, gpos[k]);
        }
      }
      __syncthreads();
    }
    TailParams q = tp;
    q.M_tot = Mt;
    q.m_dev = nullptr;
    tail_phase(q, sh);
  }
  // advance the device step index once every use of it in this step is done
  if (tp.t_dev) {
    __syncthreads();
    if (threadIdx.x == 0) tp.t_dev[0] = tp.t_dev[0] + 1;
  }
}

// Segments per row: rows are split only while there are fewer than kSplitBelow of them, so that
// the tail merges every split row in one round (kMergeRows rows per thread): into kMaxSeg below
// kFourSegBelow rows, where fewer workgroups would leave CUs idle through the ends of the launch,
// and into two from there on.  Measured at N = 4096, V = 126464 (bf16, previous LSE from the
// store), two segments per row against four: 82.0 / 92.5 / 115.8 / 137.0 / 159.8 us against
// 81.9 / 95.0 / 117.2 / 141.8 / 161.6 us at 799 / 1024 / 1311 / 1639 / 1926 rows, three segments
// no better than four: half the partials for the one-workgroup tail to merge, and fewer, longer
// workgroups.  Partials then take at most 4 * 767 or 2 * 2047 < 4096 slots.  A segment is a whole
// number of thread groups (GroupChunks * kKLThreads chunks), so that only the row's last segment
// ends in a partial group.
constexpr int kSplitBelow = 2048;
constexpr int kFourSegBelow = 768;
struct KlSplit {
  int n_seg, seg_chunks;
};
static KlSplit kl_split(int M_tot, int V, int elem_bytes) {
  const int C = V * elem_bytes / 16;
  constexpr int G = GroupChunks * kKLThreads;
  int n = 1;
  if (M_tot > 0 && M_tot < kSplitBelow) {
    const int want = M_tot < kFourSegBelow ? kMaxSeg : 2;
    const int maxseg = C / G > 1 ? C / G : 1;
    n = want < maxseg ? want : maxseg;
    n = n < kMaxSeg ? n : kMaxSeg;
    n = n < 1 ? 1 : n;
  }
  int seg = (C + n - 1) / n;
  seg = (seg + G - 1) / G * G;
  if (seg <= 0) seg = G;
  n = (C + seg - 1) / seg;   // no empty segment after the rounding
  return KlSplit{n < 1 ? 1 : n, seg};
}
static int kl_nseg(int M_tot, int V, int elem_bytes) { return kl_split(M_tot, V, elem_bytes).n_seg; }
static_assert(kSplitBelow <= kMergeRows * kTailThreads, "split rows must merge in one tail round");

size_t kl_part_bytes(int M_tot, int V, int elem_bytes) {
  const int n_seg = kl_nseg(M_tot, V, elem_bytes);
  if (n_seg <= 1) return 256;
  return (size_t)(M_tot > 0 ? M_tot : 1) * n_seg * kPartWords * 4;
}

template <typename T, bool PREV, bool PLSE>
static void kl_launch_t(const KLRowParams& rp, const TailParams& tp, float* part, hipStream_t s) {
  const KlSplit sp = kl_split(tp.M_tot, rp.V, sizeof(T));
  const int n_seg = sp.n_seg;
  if (tp.M_tot > 0) {
    hipLaunchKernelGGL((kl_rows_kernel<T, PREV, PLSE>), dim3((unsigned)tp.M_tot * n_seg), dim3(kKLThreads), 0, s, rp,
                       tp, n_seg, sp.seg_chunks, part);
  }
  hipLaunchKernelGGL((kl_tail_kernel<T, PREV, PLSE>), dim3(1), dim3(kTailThreads), 0, s, rp, tp,
                     tp.M_tot > 0 ? n_seg : 1, (const float*)part);
}

// Merge of the LM head's per-tile row statistics (EPI_LOGITS_KL): one wave per row combines the
// row's n_vt partials (lane v takes tiles v, v + 64, ...; every load of a lane issued before use),
// then the row's statistics as the row pass would finish them.
constexpr int kMergeLoads = 8;

__global__ void __launch_bounds__(256)
kl_merge_kernel(KLRowParams rp, TailParams tp, int n_vt, const float* __restrict__ klp) {
  const int M_cap = tp.M_tot;
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (m >= rows_live(M_cap, tp.m_dev)) return;   // uniform over the wave
  // the row's position, for the per-position LSE store (loaded before the partials are combined)
  const int g = rp.lse_pos ? seq_of_row(tp.act_off, tp.B, m) * tp.N + tp.act_idx[m] : 0;
  Part acc = empty_part();
  for (int v0 = lane; v0 < n_vt; v0 += 64 * kMergeLoads) {
    Part x[kMergeLoads];
#pragma unroll
    for (int k = 0; k < kMergeLoads; ++k) {
      const int v = min(v0 + 64 * k, n_vt - 1);   // clamped: loads stay in bounds
      x[k] = load_part(klp + ((size_t)v * M_cap + m) * kPartWords);
    }
#pragma unroll
    for (int k = 0; k < kMergeLoads; ++k)
      if (v0 + 64 * k < n_vt) acc = combine(acc, x[k]);
  }
  acc = wave_reduce_part(acc);
  if (lane == 0) finish_row<true, false>(rp, acc, m, g);
}

template <typename T>
static void kl_merge_tail_t(const KLRowParams& rp, const TailParams& tp, const float* klp, int n_vt, hipStream_t s) {
  if (tp.M_tot > 0)
    hipLaunchKernelGGL(kl_merge_kernel, dim3((tp.M_tot + 3) / 4), dim3(256), 0, s, rp, tp, n_vt, klp);
  hipLaunchKernelGGL((kl_tail_kernel<T, true, false>), dim3(1), dim3(kTailThreads), 0, s, rp, tp, 1,
                     (const float*)nullptr);
}

hipError_t launch_kl_merge_tail(int dtype, const KLRowParams& rp, const TailParams& tp, const float* klp, int n_vt,
                                hipStream_t s) {
  if (!tp.have_prev || n_vt < 1) return hipErrorInvalidValue;
  if (dtype == 0) kl_merge_tail_t<bf16>(rp, tp, klp, n_vt, s);
  else kl_merge_tail_t<float>(rp, tp, klp, n_vt, s);
  return hipGetLastError();
}

hipError_t launch_kl_lock(int dtype, const KLRowParams& rp, const TailParams& tp, float* part, hipStream_t s) {
  const bool prev = tp.have_prev != 0;
  const bool plse = prev && rp.lse_prev != nullptr;
  if (dtype == 0) {
    if (plse) kl_launch_t<bf16, true, true>(rp, tp, part, s);
    else if (prev) kl_launch_t<bf16, true, false>(rp, tp, part, s);
    else kl_launch_t<bf16, false, false>(rp, tp, part, s);
  } else {
    if (plse) kl_launch_t<float, true, true>(rp, tp, part, s);
    else if (prev) kl_launch_t<float, true, false>(rp, tp, part, s);
    else kl_launch_t<float, false, false>(rp, tp, part, s);
  }
  return hipGetLastError();
}

}  // namespace sl
