// Gathered-row GEMMs of the active rows: C[m][n] = sum_k A[m][k] W[n][k].
//
// Only the M active rows are multiplied (zhaoyang97 notes on SureLock,
// 永久锁定机制: locked rows skip the Q projection and FFN; cost O(M d^2),
// gist.science/nl §2).  One MFMA kernel template (v_mfma_f32_32x32x16_bf16, or
// v_mfma_f32_32x32x2f32 for fp32 storage) over tile shapes, with fused
// epilogues applied straight from the accumulators:
//   EPI_QKV    RoPE on q and k, q to a compact buffer, k and v scattered into
//              the layer's cache rows b*N + pos (locked rows untouched);
//   EPI_RESID  h += C in the fp32 residual stream (atomic when split over K);
//   EPI_SWIGLU SiLU(gate) * up;
//   EPI_LOGITS logits written to rows b*N + pos of the posterior buffer;
//   EPI_LOGITS_KL the same, plus each row's posterior statistics over the tile's
//              columns against the previous posterior (the vocabulary pass done
//              in place, so the logits are not read back).
// Paired epilogues (RoPE halves, gate/up) use a "pair layout": in every wave's
// N-range the first half of the columns holds the first element of each pair
// and the second half its partner, so both land in the same lane and register.
#include <math.h>

#include <type_traits>

#include "common.hpp"
#include "internal.hpp"
#include "klpart.hpp"

namespace sl {


// Tile geometry.  RB = bytes of K per row per k-tile (64 or 128); a k-tile is
// staged in LDS as BM + BN rows of RB bytes, chunks placed by swz<RB> so the
// 16 rows of every fragment read hit 16 distinct bank slots.
template <typename T, int BM, int BN, int WM, int WN, int RB, int S>
struct GemmCfg {
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int FM = TM / 32, FN = TN / 32;
  static constexpr int CPR = RB / 16;                 // chunks per row
  static constexpr int KS = RB / 32;                  // MFMA k-steps per k-tile (32 bytes each)
  static constexpr int NW = WM * WN, NT = 64 * NW;     // waves and threads per workgroup
  static constexpr int ADma = BM * CPR / NT;            // direct loads per thread per k-tile
  static constexpr int BDma = BN * CPR / NT;
  static constexpr int StageBytes = (BM + BN) * RB;
  static_assert(RB == 64 || RB == 128, "row bytes");
  static_assert(NW == 4 || NW == 8, "four or eight waves");
  static_assert(FM >= 1 && FN >= 1 && TM % 32 == 0 && TN % 32 == 0, "wave tile");
  static_assert(ADma >= 1 && BDma >= 1 && BM * CPR % NT == 0 && BN * CPR % NT == 0, "load split");
  static_assert(S >= 2 && S * StageBytes <= 150 * 1024, "LDS budget");
  static_assert((S - 2) * (ADma + BDma) < 64, "vmcnt range");
};

__device__ __forceinline__ float silu_f(float g) {
  return g * __builtin_amdgcn_rcpf(1.f + __expf(-g));
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// 16 bytes from global memory straight into LDS: lane l of the wave writes
// bytes [16 l, 16 l + 16) after the wave-uniform LDS base.
__device__ __forceinline__ void dma16(const void* g, void* lds_base) {
  __builtin_amdgcn_global_load_lds((glb_void_t*)g, (lds_void_t*)lds_base, 16, 0, 0);
}

// s_waitcnt vmcnt(n) (gfx9 encoding: vmcnt bits [3:0] and [15:14]; others left at "no wait").
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier without a memory fence.  __syncthreads() adds a release
// fence, which makes the compiler drain every outstanding global load first
// (vmcnt(0)), including the direct loads of later k-tiles that are meant to
// stay in flight.  The main loop orders its LDS traffic itself: the stage it
// overwrites was last read by ds_reads whose results the MFMAs have consumed,
// and the tile it reads was waited for with wait_vmcnt before the barrier.
__device__ __forceinline__ void barrier_no_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <typename T, int EPI>
__device__ __forceinline__ const char* w_row_ptr(const GemmArgs& a, int vrow, int TN) {
  const size_t rb = (size_t)a.K * sizeof(T);
  if (EPI == EPI_QKV || EPI == EPI_SWIGLU) {
    const int wbase = vrow - vrow % TN;            // first virtual column of this wave range
    const int c = vrow % TN;
    const int pair = wbase / 2 + c % (TN / 2);
    const int half = c / (TN / 2);
    if (EPI == EPI_SWIGLU) return (const char*)(half ? a.w1 : a.w0) + (size_t)pair * rb;
    const int hd = a.d / 2, hh = a.Dh / 2;
    const int mat = pair / hd, gp = pair % hd;
    const int phys = (gp / hh) * a.Dh + half * hh + gp % hh;
    const void* w = mat == 0 ? a.w0 : (mat == 1 ? a.w1 : a.w2);
    return (const char*)w + (size_t)phys * rb;
  }
  return (const char*)a.w0 + (size_t)vrow * rb;
}

// 8 consecutive outputs of the storage type (one 16-byte store for bf16).
template <typename T>
__device__ __forceinline__ void store8(T* dst, const float* y) {
  if (sizeof(T) == 2) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16 lo = (bf16)y[2 * i], hi = (bf16)y[2 * i + 1];
      w[i] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
    st16(dst, w);
  } else {
    st16(dst, u32x4{__float_as_uint(y[0]), __float_as_uint(y[1]), __float_as_uint(y[2]), __float_as_uint(y[3])});
    st16((float*)dst + 4, u32x4{__float_as_uint(y[4]), __float_as_uint(y[5]), __float_as_uint(y[6]), __float_as_uint(y[7])});
  }
}

__device__ __forceinline__ void lds8(const float* p, float* y) {
  const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) { y[i] = a[i]; y[4 + i] = b[i]; }
}

// EPI_LOGITS_KL, one pass over PR rows of the fp32 tile (rows from mrow0): the logits as EPI_LOGITS,
// then, from the stored values a (rounded to the storage type, as a later pass would read them) and
// the previous posterior's b (prefetched into praw by logits_kl_prefetch), each row's statistics over this tile's BN
// columns: max a, sum e^(a - max a), sum e^(a - max a) (a - b), max b, sum e^(b - max b), and the
// largest a other than the [MASK] id with its lowest id.  A row's CPR chunks sit on CPR consecutive
// lanes (ids are consecutive, CPR divides 64); the lanes first agree on the row maxima, so the sums
// combine by plain additions.  grow[it] = the row b*N + pos of chunk it, or -1 past the live rows.
template <typename T, int BN, int LDW, int PR, int NT, int IT, int PW>
__device__ __forceinline__ void logits_kl_pass(const GemmArgs& a, const float* tile, int mrow0, int n0,
                                               const u32x4 (&praw)[IT][PW], const int32_t (&grow)[IT]) {
  constexpr int CPR = BN / 8;
  static_assert(CPR == 8 || CPR == 16 || CPR == 32, "fused statistics need BN in {64, 128, 256}");
  const int tid = threadIdx.x;
  const int vt = n0 / BN;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int id = tid + it * NT;
    if (grow[it] < 0) continue;   // uniform over the row's lanes
    const int r = id / CPR, c = (id % CPR) * 8;
    const int m = mrow0 + r;
    float y[8], bv[8];
    lds8(tile + r * LDW + c, y);
    store8<T>((T*)a.out0 + (size_t)grow[it] * a.Nv + n0 + c, y);
    if (sizeof(T) == 2) {
      Chunk<bf16>::unpack(praw[it][0], bv);
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = (float)(bf16)y[i];
    } else {
      Chunk<float>::unpack(praw[it][0], bv);
      Chunk<float>::unpack(praw[it][PW - 1], bv + 4);
    }
    float ma = y[0], mb = bv[0], best = -INFINITY;
    int bidx = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ma = fmaxf(ma, y[i]);
      mb = fmaxf(mb, bv[i]);
      if (y[i] > best && n0 + c + i != a.mask_id) { best = y[i]; bidx = n0 + c + i; }
    }
#pragma unroll
    for (int o = CPR / 2; o >= 1; o >>= 1) {
      ma = fmaxf(ma, __shfl_xor(ma, o, 64));
      mb = fmaxf(mb, __shfl_xor(mb, o, 64));
      const float ob = __shfl_xor(best, o, 64);
      const int oi = __shfl_xor(bidx, o, 64);
      if (ob > best || (ob == best && oi < bidx)) { best = ob; bidx = oi; }
    }
    const float mal = ma * kLog2e, mbl = mb * kLog2e;
    float sa = 0.f, ta = 0.f, sb = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float e = __builtin_amdgcn_exp2f(fmaf(y[i], kLog2e, -mal));
      sa += e;
      ta = fmaf(e, y[i] - bv[i], ta);
      sb += __builtin_amdgcn_exp2f(fmaf(bv[i], kLog2e, -mbl));
    }
#pragma unroll
    for (int o = CPR / 2; o >= 1; o >>= 1) {
      sa += __shfl_xor(sa, o, 64);
      ta += __shfl_xor(ta, o, 64);
      sb += __shfl_xor(sb, o, 64);
    }
    if (id % CPR == 0) {
      Part p;
      p.ma = ma; p.sa = sa; p.ta = ta; p.mb = mb; p.sb = sb; p.best = best; p.bidx = bidx;
      store_part(a.klp + ((size_t)vt * a.M + m) * kPartWords, p);
    }
  }
}

// The previous posterior's chunks of the PR rows from mrow0 that logits_kl_pass will use.
template <typename T, int BN, int PR, int NT, int IT, int PW>
__device__ __forceinline__ void logits_kl_prefetch(const GemmArgs& a, int mrow0, int n0, int Mr, u32x4 (&praw)[IT][PW],
                                                   int32_t (&grow)[IT]) {
  constexpr int CPR = BN / 8;
  const int tid = threadIdx.x;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int id = tid + it * NT;
    const int m = mrow0 + id / CPR;
    grow[it] = -1;
    if (id < PR * CPR && m < Mr) {
      const int b = seq_of_row(a.act_off, a.B, m);
      grow[it] = b * a.N + a.act_idx[m];
      const char* src = (const char*)((const T*)a.prev + (size_t)grow[it] * a.Nv + n0 + (id % CPR) * 8);
#pragma unroll
      for (int w = 0; w < PW; ++w) praw[it][w] = ld16(src + 16 * w);
    }
  }
}

// One pass of the epilogue over PR rows of the fp32 tile (rows from mrow0).
// Paired epilogues: output pair p of the tile takes its first element from
// tile column (p / (TN/2)) * TN + p % (TN/2) and its partner TN/2 further.
template <typename T, int EPI, int BN, int TN, int LDW, int PR, int NT>
__device__ __forceinline__ void epilogue_pass(const GemmArgs& a, const float* tile, int mrow0, int n0, int Mr) {
  const int tid = threadIdx.x;
  if (EPI == EPI_RESID) {
    if (a.split_k > 1 && a.part) {
      // this split's partial sums, plane blockIdx.z, with 16-byte stores
      constexpr int CPR = BN / 4;
      float* plane = a.part + (size_t)blockIdx.z * a.M * a.Nv;
      for (int id = tid; id < PR * CPR; id += NT) {
        const int r = id / CPR, c = (id % CPR) * 4;
        const int m = mrow0 + r;
        if (m < Mr) *(f32x4*)(plane + (size_t)m * a.Nv + n0 + c) = *(const f32x4*)(tile + r * LDW + c);
      }
    } else if (a.split_k > 1) {
      // fp32 atomics, consecutive lanes on consecutive floats of a row
      for (int id = tid; id < PR * BN; id += NT) {
        const int r = id / BN, c = id % BN;
        const int m = mrow0 + r;
        if (m < Mr) unsafeAtomicAdd((float*)a.out0 + (size_t)m * a.Nv + n0 + c, tile[r * LDW + c]);
      }
    } else {
      constexpr int CPR = BN / 4;
      for (int id = tid; id < PR * CPR; id += NT) {
        const int r = id / CPR, c = (id % CPR) * 4;
        const int m = mrow0 + r;
        if (m >= Mr) continue;
        float* h = (float*)a.out0 + (size_t)m * a.Nv + n0 + c;
        f32x4 y = *(const f32x4*)h;
        y += *(const f32x4*)(tile + r * LDW + c);
        *(f32x4*)h = y;
      }
    }
  } else if (EPI == EPI_LOGITS) {
    constexpr int CPR = BN / 8;
    for (int id = tid; id < PR * CPR; id += NT) {
      const int r = id / CPR, c = (id % CPR) * 8;
      const int m = mrow0 + r;
      if (m >= Mr) continue;
      const int b = seq_of_row(a.act_off, a.B, m);
      const size_t g = (size_t)b * a.N + a.act_idx[m];
      float y[8];
      lds8(tile + r * LDW + c, y);
      store8<T>((T*)a.out0 + g * a.Nv + n0 + c, y);
    }
  } else {
    constexpr int CPR = BN / 16;                  // 8-pair runs per row
    for (int id = tid; id < PR * CPR; id += NT) {
      const int r = id / CPR, p0 = (id % CPR) * 8;
      const int m = mrow0 + r;
      if (m >= Mr) continue;
      const int c1 = (p0 / (TN / 2)) * TN + p0 % (TN / 2);
      float x1[8], x2[8];
      lds8(tile + r * LDW + c1, x1);
      lds8(tile + r * LDW + c1 + TN / 2, x2);
      const int pair = n0 / 2 + p0;
      if (EPI == EPI_SWIGLU) {
        float y[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] = silu_f(x1[i]) * x2[i];
        store8<T>((T*)a.out0 + (size_t)m * (a.Nv / 2) + pair, y);
      } else {
        const int hd = a.d / 2, hh = a.Dh / 2;          // hh is a power of two
        const int mat = pair >= 2 * hd ? 2 : (pair >= hd ? 1 : 0);
        const int gp = pair - mat * hd;
        const int jj = gp & (hh - 1);
        const int col = (gp / hh) * a.Dh + jj;
        const int pos = a.act_idx[m];
        if (mat < 2) {
          const float* cs = a.rope + ((size_t)pos * hh + jj) * 2;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x4 t = *(const f32x4*)(cs + 4 * q);   // (cos, sin) of pairs 2q, 2q+1
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              const int i = 2 * q + e;
              const float c = t[2 * e], sn = t[2 * e + 1];
              const float u1 = x1[i] * c - x2[i] * sn, u2 = x2[i] * c + x1[i] * sn;
              x1[i] = u1;
              x2[i] = u2;
            }
          }
        }
        T* dst;
        int c0 = col;
        if (mat == 0) {
          dst = (T*)a.out0 + (size_t)m * a.d;
        } else if (a.kv_hm) {   // head-major cache: this head's row of Dh elements at (b, h, pos)
          const int b = seq_of_row(a.act_off, a.B, m);
          const int H = a.d / a.Dh, hd = col / a.Dh;
          dst = (T*)(mat == 1 ? a.out1 : a.out2) + (((size_t)b * H + hd) * a.N + pos) * a.Dh;
          c0 = col - hd * a.Dh;
        } else {
          const int b = seq_of_row(a.act_off, a.B, m);
          dst = (T*)(mat == 1 ? a.out1 : a.out2) + ((size_t)b * a.N + pos) * a.d;
        }
        store8<T>(dst + c0, x1);
        store8<T>(dst + c0 + hh, x2);
      }
    }
  }
}

// Calls f(integral_constant<int, I>) for I in [I0, I1).
template <int I0, int I1, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I0 < I1) {
    f(std::integral_constant<int, I0>{});
    static_for<I0 + 1, I1>(f);
  }
}

// A wave's direct load fills 1 KB = 1024/RB consecutive rows: lane l lands at
// row l/CPR, stored chunk l%CPR, so it fetches the logical chunk that the
// swizzle stores there.  S-stage pipeline: tile kt+S-1 is requested while tile
// kt is multiplied; one barrier per k-tile.
//
// VB (through registers): when few activation rows stream a large weight matrix
// once, the direct-to-LDS path is the limit: it moves HBM data to a CU markedly
// slower than ordinary vector loads (≈ 4.3 against ≈ 6 TB/s chip-wide).  With VB
// both operands' tiles are fetched with 16-byte vector loads (non-temporal for
// the weights) into a ring of S-1 register stages, each lane loading the 16
// bytes its direct load would have placed, and written to one of two LDS stages
// with ds_write before the k-tile's barrier.  The k-tile loop is unrolled by the
// ring so every register slot is static, and every load is unconditional (past
// the end it repeats the last tile into a slot that is never read): a
// conditional load, or a direct-to-LDS load in the same kernel, makes the
// compiler drain all loads before a slot is used.  Small LDS and register use
// let two workgroups share a CU.
//
// CLK (a measurement variant) records per workgroup the shader-clock cycles (s_memtime) and the
// 100 MHz real-time ticks (s_memrealtime) it took, and the cycles of its k-tile loop: their ratio is
// the clock the chip sustained under this load, and the loop's cycles against BM*BN*K*2 / 4096 (the
// FLOPs one CU's four matrix cores retire per cycle) its MFMA utilisation at that clock.
template <typename T, int BM, int BN, int WM, int WN, int RB, int S, int EPI, bool VB, bool CLK = false>
__global__ void __launch_bounds__(64 * WM * WN)
__attribute__((amdgpu_waves_per_eu(WM * WN / 4, 2)))
gemm_kernel(GemmArgs a, int MT, int NT, int k_iters_per_split) {
  using C = GemmCfg<T, BM, BN, WM, WN, RB, S>;
  constexpr int kStages = VB ? 2 : S;   // LDS stages
  __shared__ __attribute__((aligned(1024))) char smem[kStages * C::StageBytes];
  const int tid = threadIdx.x, lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: LDS bases stay scalar
  const int wm = wid / WN, wn = wid % WN;

  // workgroup -> tile.  Each XCD takes a contiguous range of the tile order (workgroups are dealt
  // to the 8 XCDs round-robin), and the order walks groups of up to 8 row tiles column by column,
  // so the workgroups an XCD runs at once cover a block of row and column tiles whose operand
  // slices they share through its L2.
  const int nb = MT * NT;
  int lid = blockIdx.x;
  if ((nb & 7) == 0) lid = (blockIdx.x & 7) * (nb >> 3) + (blockIdx.x >> 3);
  constexpr int kGroupRows = 8;
  const int grp = lid / (kGroupRows * NT), in_grp = lid - grp * (kGroupRows * NT);
  const int gm = min(kGroupRows, MT - grp * kGroupRows);
  const int bm = grp * kGroupRows + in_grp % gm, bn = in_grp / gm;
  const int m0 = bm * BM, n0 = bn * BN;
  const int Mr = rows_live(a.M, a.m_dev);   // rows to compute (a.M is their capacity and plane stride)
  if (m0 >= Mr) return;                     // uniform over the workgroup, before any barrier
  unsigned long long clk_c0 = 0, clk_r0 = 0, clk_m0 = 0, clk_m1 = 0;
  if constexpr (CLK) {
    clk_c0 = __builtin_amdgcn_s_memtime();
    clk_r0 = __builtin_amdgcn_s_memrealtime();
  }
  const int split = blockIdx.z;
  const int KI = a.K * (int)sizeof(T) / RB;
  const int kt0 = split * k_iters_per_split;
  const int kt1 = min(KI, kt0 + k_iters_per_split);

  // global sources of this thread's direct loads: lane l lands at tile row
  // r = group*(1024/RB) + l/CPR, stored position l%CPR, holding the logical
  // chunk that swz<RB> puts there (swz is an involution in the chunk index)
  const int lrow = lane / C::CPR, lpos = lane % C::CPR;
  const size_t arb = (size_t)a.K * sizeof(T);
  uint32_t aoff[C::ADma];
  const char* bp[C::BDma];
#pragma unroll
  for (int i = 0; i < C::ADma; ++i) {
    const int r = (i * C::NW + wid) * (1024 / RB) + lrow;
    aoff[i] = (uint32_t)((size_t)min(m0 + r, Mr - 1) * arb) + swz<RB>(r, lpos) * 16;
  }
#pragma unroll
  for (int i = 0; i < C::BDma; ++i) {
    const int r = (i * C::NW + wid) * (1024 / RB) + lrow;
    bp[i] = w_row_ptr<T, EPI>(a, n0 + r, C::TN) + swz<RB>(r, lpos) * 16;
  }
  const char* abase = (const char*)a.A;
  // direct loads j in [j0, j1) of k-tile kt into `stage` (A loads first, then B)
  auto issue = [&](int kt, int stage, int j0, int j1) {
    char* as = smem + stage * C::StageBytes;
    char* bs = as + BM * RB;
    const size_t off = (size_t)kt * RB;
#pragma unroll
    for (int j = 0; j < C::ADma + C::BDma; ++j) {
      if (j < j0 || j >= j1) continue;
      if (j < C::ADma) dma16(abase + aoff[j] + off, as + (j * C::NW + wid) * 1024);
      else dma16(bp[j - C::ADma] + off, bs + ((j - C::ADma) * C::NW + wid) * 1024);
    }
  };

  f32x16 acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // LDS byte offsets of this lane's fragment rows (chunk added per k-step)
  int arow[C::FM], brow[C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i) arow[i] = wm * C::TM + i * 32 + l32;
#pragma unroll
  for (int j = 0; j < C::FN; ++j) brow[j] = wn * C::TN + j * 32 + l32;

  constexpr int NDMA = C::ADma + C::BDma;
  constexpr int DPS = (NDMA + C::KS - 1) / C::KS;   // direct loads issued per k-step

  // Fragment reads of k-step ks of the k-tile at (as, bs) into register buffer buf.
  u32x4 fa[2][C::FM], fb[2][C::FN];
  auto frags = [&](const char* as, const char* bs, int ks, int buf) {
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
      const int r = arow[i];
      fa[buf][i] = *(const u32x4*)(as + r * RB + (swz<RB>(r, 2 * ks + hl) << 4));
    }
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      const int r = brow[j];
      fb[buf][j] = *(const u32x4*)(bs + r * RB + (swz<RB>(r, 2 * ks + hl) << 4));
    }
  };
  // The MFMAs of k-step ks (register buffer ks & 1), with the fragment reads issued just
  // before them spread between them.
  auto mfmas = [&](int ks, bool reads_follow) {
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j) Mfma<T>::run(acc[i][j], fa[ks & 1][i], fb[ks & 1][j]);
    if (reads_follow) {
      constexpr int NRD = C::FM + C::FN;
      constexpr int NM = C::FM * C::FN * (sizeof(T) == 2 ? 1 : 4);
#pragma unroll
      for (int g = 0; g < NRD; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, NM / NRD > 0 ? NM / NRD : 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // Multiply one k-tile held in LDS (A rows at `as`, B rows at `bs`) whose first k-step's
  // fragments are already in buffer 0; step(ks) issues that k-step's share of the loads in
  // flight.
  auto mma_tile = [&](const char* as, const char* bs, auto&& step) {
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      step(ks);
      if (ks + 1 < C::KS) frags(as, bs, ks + 1, (ks + 1) & 1);
      mfmas(ks, ks + 1 < C::KS);
    }
  };

  if constexpr (!VB) {
    static_assert(C::KS % 2 == 0, "the next tile's first fragments go to buffer 0");
#pragma unroll
    for (int st = 0; st < S - 1; ++st)
      if (kt0 + st < kt1) issue(kt0 + st, st, 0, NDMA);
    // Tile kt's fragments of its first k-step are read during the last k-step of tile kt - 1,
    // behind that step's barrier, so every k-tile starts with its MFMAs' operands in registers.
    if (kt0 < kt1) {
      if (kt0 + S - 2 < kt1) wait_vmcnt<(S - 2) * NDMA>();
      else wait_vmcnt<0>();
      barrier_no_fence();
      frags(smem, smem + BM * RB, 0, 0);
    }
    if constexpr (CLK) clk_m0 = __builtin_amdgcn_s_memtime();
    for (int kt = kt0; kt < kt1; ++kt) {
      const bool pre = kt + S - 1 < kt1;
      const int pre_stage = (kt + S - 1 - kt0) % S;
      const char* as = smem + ((kt - kt0) % S) * C::StageBytes;
      const char* bs = as + BM * RB;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        if (pre) issue(kt + S - 1, pre_stage, ks * DPS, (ks + 1) * DPS);
        if (ks + 1 < C::KS) {
          frags(as, bs, ks + 1, (ks + 1) & 1);
        } else {
          // tile kt + 1 has landed when at most the S - 2 later tiles are in flight; the
          // barrier also tells that every wave's reads of tile kt (the stage the next
          // k-tile's loads overwrite) are done.  After the last tile the reads fetch a stale
          // stage that nothing uses.
          __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));   // lgkmcnt(0)
          if (pre) wait_vmcnt<(S - 2) * NDMA>();
          else wait_vmcnt<0>();
          barrier_no_fence();
          const char* an = smem + ((kt + 1 - kt0) % S) * C::StageBytes;
          frags(an, an + BM * RB, 0, 0);
        }
        mfmas(ks, true);
      }
    }
  } else {
    constexpr int RS = S - 1;   // register stages
    u32x4 areg[RS][C::ADma], breg[RS][C::BDma];
    // weights first, then activations, for every tile: "tile kt landed" is one count
    auto vload = [&](int kt, int slot) {
#pragma unroll
      for (int j = 0; j < C::BDma; ++j) breg[slot][j] = ld16_stream(bp[j] + (size_t)kt * RB);
#pragma unroll
      for (int j = 0; j < C::ADma; ++j) areg[slot][j] = ld16(abase + aoff[j] + (size_t)kt * RB);
    };
    auto vtile = [&](const int kt, auto U) {
      constexpr int u = decltype(U)::value;
      wait_vmcnt<(S - 2) * NDMA>();   // tile kt landed; the S-2 later ones may be in flight
      // stage kt&1 was last read two k-tiles ago, which every wave finished before the
      // previous barrier
      char* as = smem + ((kt - kt0) & 1) * C::StageBytes;
      char* bs = as + BM * RB;
#pragma unroll
      for (int j = 0; j < C::ADma; ++j) st16(as + (j * C::NW + wid) * 1024 + lane * 16, areg[u][j]);
#pragma unroll
      for (int j = 0; j < C::BDma; ++j) st16(bs + (j * C::NW + wid) * 1024 + lane * 16, breg[u][j]);
      vload(min(kt + S - 1, kt1 - 1), u);
      __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));   // lgkmcnt(0): stores done
      barrier_no_fence();
      frags(as, bs, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      mma_tile(as, bs, [](int) {});
    };
#pragma unroll
    for (int st = 0; st < RS; ++st) vload(min(kt0 + st, kt1 - 1), st);
    if constexpr (CLK) clk_m0 = __builtin_amdgcn_s_memtime();
    int kb = kt0;
    for (; kb + RS <= kt1; kb += RS)
      static_for<0, RS>([&](auto U) { vtile(kb + decltype(U)::value, U); });
    static_for<0, RS - 1>([&](auto U) {
      if (kb + decltype(U)::value < kt1) vtile(kb + decltype(U)::value, U);
    });
  }
  if constexpr (CLK) clk_m1 = __builtin_amdgcn_s_memtime();
  __syncthreads();   // every wave is done with the pipeline's LDS

  // ---------------------------------------------------------------- epilogue
  // The accumulators go through LDS (an fp32 tile, rows padded to BN+8 floats so
  // that both half-waves of an MFMA store hit different banks), in row passes
  // when the tile is larger than the pipeline's LDS; then every thread handles
  // runs of 8 (4 for the residual) consecutive outputs with 16-byte accesses.
  constexpr int LDW = BN + 8;
  constexpr int SMEM = kStages * C::StageBytes;
  constexpr int PR = (BM * LDW * 4 <= SMEM) ? BM : (BM / 2 * LDW * 4 <= SMEM) ? BM / 2 : (BM / 4 * LDW * 4 <= SMEM) ? BM / 4 : 32;
  static_assert(PR >= 32 && PR % 32 == 0 && BM % PR == 0 && PR * LDW * 4 <= SMEM, "epilogue pass");
  float* tile = (float*)smem;
  // Writes the accumulators of rows [r_lo, r_lo + rows) of the tile into the fp32 LDS tile.
  auto stage_rows = [&](int r_lo, int rows) {
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
      const int rb = wm * C::TM + i * 32 - r_lo;   // first tile row of this MFMA block in the pass
      if (rb < 0 || rb >= rows) continue;
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          tile[(rb + (v >> 2) * 8 + 4 * hl + (v & 3)) * LDW + wn * C::TN + j * 32 + l32] = acc[i][j][v];
    }
  };
  if constexpr (EPI == EPI_LOGITS_KL) {
    // The previous posterior's chunks of the next row pass are loaded as soon as a pass has used its
    // own, so their latency overlaps the next pass's staging instead of stalling every wave of the CU.
    // Passes of at most 4 chunks per thread keep the prefetched registers within the budget.
    constexpr int KCPR = BN / 8, KPR = PR < 4 * C::NT / KCPR ? PR : 4 * C::NT / KCPR;
    constexpr int KIT = (KPR * KCPR + C::NT - 1) / C::NT, KPW = sizeof(T) == 2 ? 1 : 2;
    static_assert(BM % KPR == 0 && KPR % 32 == 0, "fused statistics pass");
    u32x4 praw[KIT][KPW];
    int32_t grow[KIT];   // b*N + pos < 2^31, or -1 past the live rows
    logits_kl_prefetch<T, BN, KPR, C::NT, KIT, KPW>(a, m0, n0, Mr, praw, grow);
    for (int r_lo = 0; r_lo < BM; r_lo += KPR) {
      stage_rows(r_lo, KPR);
      __syncthreads();
      logits_kl_pass<T, BN, LDW, KPR, C::NT, KIT, KPW>(a, tile, m0 + r_lo, n0, praw, grow);
      if (r_lo + KPR < BM) logits_kl_prefetch<T, BN, KPR, C::NT, KIT, KPW>(a, m0 + r_lo + KPR, n0, Mr, praw, grow);
      __syncthreads();
    }
  } else {
    for (int r_lo = 0; r_lo < BM; r_lo += PR) {
      stage_rows(r_lo, PR);
      __syncthreads();
      epilogue_pass<T, EPI, BN, C::TN, LDW, PR, C::NT>(a, tile, m0 + r_lo, n0, Mr);
      __syncthreads();
    }
  }
  if constexpr (CLK) {
    const unsigned long long c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
    const long w = (long)blockIdx.z * gridDim.x + blockIdx.x;
    if (tid == 0 && a.clk && w < a.clk_slots) {
      unsigned long long* o = a.clk + 4 * w;
      o[0] = c1 - clk_c0;
      o[1] = r1 - clk_r0;
      o[2] = clk_m1 - clk_m0;
      o[3] = (unsigned long long)(kt1 - kt0) * RB / sizeof(T);
    }
  }
}

// ------------------------------------------------------------------ dispatch
// K splits actually launched for a requested split: every split takes the same number of k-tiles.
static int splits_launched(int KI, int split) {
  const int kps = (KI + split - 1) / split;
  return (KI + kps - 1) / kps;
}

template <typename T, int BM, int BN, int WM, int WN, int RB, int S, bool VB = false, bool CLK = false>
static hipError_t run_cfg(EpiKind epi, const GemmArgs& a, hipStream_t s, int split) {
  const int MT = (a.M + BM - 1) / BM, NT = a.Nv / BN;
  const int KI = a.K * (int)sizeof(T) / RB;
  const int kps = (KI + split - 1) / split;
  const int nsplit = splits_launched(KI, split);
  GemmArgs b = a;
  b.split_k = nsplit;
  const dim3 grid(MT * NT, 1, nsplit), block(64 * WM * WN);
  if constexpr (CLK) {
    switch (epi) {
      case EPI_SWIGLU: hipLaunchKernelGGL((gemm_kernel<T, BM, BN, WM, WN, RB, S, EPI_SWIGLU, VB, true>), grid, block, 0, s, b, MT, NT, kps); break;
      case EPI_LOGITS: hipLaunchKernelGGL((gemm_kernel<T, BM, BN, WM, WN, RB, S, EPI_LOGITS, VB, true>), grid, block, 0, s, b, MT, NT, kps); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  switch (epi) {
    case EPI_QKV: hipLaunchKernelGGL((gemm_kernel<T, BM, BN, WM, WN, RB, S, EPI_QKV, VB>), grid, block, 0, s, b, MT, NT, kps); break;
    case EPI_RESID: hipLaunchKernelGGL((gemm_kernel<T, BM, BN, WM, WN, RB, S, EPI_RESID, VB>), grid, block, 0, s, b, MT, NT, kps); break;
    case EPI_SWIGLU: hipLaunchKernelGGL((gemm_kernel<T, BM, BN, WM, WN, RB, S, EPI_SWIGLU, VB>), grid, block, 0, s, b, MT, NT, kps); break;
    case EPI_LOGITS: hipLaunchKernelGGL((gemm_kernel<T, BM, BN, WM, WN, RB, S, EPI_LOGITS, VB>), grid, block, 0, s, b, MT, NT, kps); break;
    case EPI_LOGITS_KL:
      if constexpr (BN == 64 || BN == 128 || BN == 256)
        hipLaunchKernelGGL((gemm_kernel<T, BM, BN, WM, WN, RB, S, EPI_LOGITS_KL, VB>), grid, block, 0, s, b, MT, NT, kps);
      else
        return hipErrorInvalidValue;
      break;
  }
  return hipGetLastError();
}

// Tile shapes (4 or 8 waves; RB = k-tile row bytes; S = stages) and their
// measured sustained rate per CU in multiply-adds per microsecond (bf16,
// calibrated on the 4096 / 12288 projections at M = 64 .. 1024 on MI355X,
// weights rotated over copies larger than the Infinity Cache); occ =
// workgroups one CU holds at once, cap = chip-wide weight streaming rate.
struct TileCfg { int BM, BN, RB, S; float rate; int occ; float cap; bool vb; };
constexpr int kNumCfgs = 12;
constexpr float kStreamCapBytesPerUs = 5.0e6f;  // weight streaming from HBM by direct-to-LDS loads
static const TileCfg kCfgs[kNumCfgs] = {
    {256, 256, 64, 4, 2.35e6f, 1, kStreamCapBytesPerUs, false},   // 0: eight waves 2x4, wave tile 128x64
    {256, 128, 128, 3, 2.17e6f, 1, kStreamCapBytesPerUs, false},  // 1: eight waves 4x2, wave tile 64x64
    {128, 256, 128, 3, 2.13e6f, 1, kStreamCapBytesPerUs, false},  // 2: eight waves 2x4, wave tile 64x64
    {128, 128, 128, 3, 1.55e6f, 1, kStreamCapBytesPerUs, false},  // 3: four waves, wave tile 64x64
    {128, 64, 128, 4, 1.25e6f, 1, kStreamCapBytesPerUs, false},   // 4: four waves 4x1, wave tile 32x64
    {256, 192, 64, 4, 1.90e6f, 1, kStreamCapBytesPerUs, false},   // 5: four waves, wave tile 128x96 (256 tiles at M = 1024, N = 12288)
    {128, 384, 64, 4, 1.87e6f, 1, kStreamCapBytesPerUs, false},   // 6: four waves, wave tile 64x192
    {64, 128, 128, 6, 1.06e6f, 1, kStreamCapBytesPerUs, false},   // 7: four waves 1x4, wave tile 64x32: weight streaming at small M
    {64, 64, 128, 8, 0.82e6f, 1, kStreamCapBytesPerUs, false},    // 8: four waves 2x2, wave tile 32x32: weight streaming at small M
    {64, 128, 128, 6, 1.06e6f, 2, 6.0e6f, true},                  // 9: as 7, through registers (VB), two per CU
    // 96-wide wave tiles: 12288 columns make 128 column tiles of 96 (256 tiles at 256 rows) and 64 of
    // 192 (256 tiles at 512 rows), where 128-wide tiles leave a quarter of the CUs idle
    {128, 96, 128, 4, 1.30e6f, 1, kStreamCapBytesPerUs, false},   // 10: four waves 4x1, wave tile 32x96
    {128, 192, 128, 3, 1.80e6f, 1, kStreamCapBytesPerUs, false},  // 11: four waves 2x2, wave tile 64x96
};
constexpr int kCUs = 256;
constexpr float kCuBytesPerUs = 4.2e4f;        // what one CU pulls from HBM (latency bound)
constexpr float kCuLoadBytesPerUs = 5.5e4f;    // what one CU loads of both operands, L2 hits included
constexpr float kLoadLatencyUs = 1.0f;          // what a workgroup's S-1 tiles in flight amortise
constexpr float kAtomicBytesPerUs = 1.5e6f;     // fp32 atomic adds of split-K partials
constexpr float kPartBytesPerUs = 3.0e6f;       // partial-sum planes beyond the first (store, then read back)
constexpr float kLaunchUs = 2.0f;

// Estimated time of a launch: the compute of the most loaded CU, or streaming
// the weights, whichever is longer.  The resident workgroups keep
// (S-1) weight tiles (BN x RB bytes each) in flight, and each CU pulls at most
// kCuBytesPerUs, so few workgroups stream slower than the chip can.  Split-K adds
// its atomic traffic, or, when the caller provides partial-sum planes that the
// residual reduce + RMSNorm sums (part), the extra planes it stores and reads back.
static float est_us(const GemmArgs& a, int eb, int c, int split, bool part) {
  const TileCfg& g = kCfgs[c];
  const long MT = (a.M + g.BM - 1) / g.BM, NT = a.Nv / g.BN;
  const long blocks = MT * NT * split;
  const long slots = (long)g.occ * kCUs;
  const long per_cu = (blocks + kCUs - 1) / kCUs;   // tiles per CU (shared when occ > 1)
  const float comp = (float)per_cu * g.BM * g.BN * ((float)a.K / split) / g.rate;
  const long resident = blocks < slots ? blocks : slots;
  const long cus = blocks < kCUs ? blocks : kCUs;
  float bw = (float)resident * (g.S - 1) * g.BN * g.RB / kLoadLatencyUs;
  if (bw > (float)cus * kCuBytesPerUs) bw = (float)cus * kCuBytesPerUs;
  if (bw > g.cap) bw = g.cap;
  float mem = (float)a.Nv * a.K * eb / bw;
  // each tile also loads its BM activation rows (rows past M repeat the last one), and one
  // CU loads both operands at a bounded rate: at few rows, 128-row tiles load twice the bytes
  const float cu_load = (float)per_cu * (g.BM + g.BN) * ((float)a.K * eb / split) / kCuLoadBytesPerUs;
  if (cu_load > mem) mem = cu_load;
  const float atom = split <= 1 ? 0.f
                     : part ? (float)a.M * a.Nv * 4.f * (split - 1) / kPartBytesPerUs
                            : (float)a.M * a.Nv * 4.f * split / kAtomicBytesPerUs;
  return (comp > mem ? comp : mem) + atom + kLaunchUs;
}

static void pick_cfg(const GemmArgs& a, EpiKind epi, int eb, bool part, int& cfg, int& split) {
  float best = 3.4e38f;
  cfg = -1; split = 1;
  for (int c = 0; c < kNumCfgs; ++c) {
    const TileCfg& g = kCfgs[c];
    if (a.Nv % g.BN || (a.K * eb) % g.RB) continue;
    if (g.vb && eb != 2) continue;   // the register path is calibrated for bf16 only
    if (epi == EPI_LOGITS_KL && g.BN != 64 && g.BN != 128 && g.BN != 256) continue;   // lane groups of a row
    const int KI = a.K * eb / g.RB;
    for (int sp = 1; sp <= 8; sp *= 2) {
      if (sp > 1 && (epi != EPI_RESID || KI / sp < 8 || g.vb)) break;   // the register path streams whole K
      const float t = est_us(a, eb, c, sp, part && epi == EPI_RESID);
      if (t < best) { best = t; cfg = c; split = sp; }
    }
  }
}

int gemm_supported(int dtype, EpiKind epi, int Nv, int K, int d, int Dh) {
  const int eb = dtype == 0 ? 2 : 4;
  if ((K * eb) % 128) return 0;   // every config then has a valid k-tile
  if (Nv % 64) return 0;          // config 4 then tiles the columns
  if (epi == EPI_QKV && (d % 128 || Dh % 2)) return 0;
  return 1;
}

template <typename T, bool CLK = false>
static hipError_t launch_t(EpiKind epi, const GemmArgs& a, hipStream_t s, int* nsplit) {
  int c, split;
  pick_cfg(a, epi, (int)sizeof(T), a.part != nullptr, c, split);
  if (nsplit) *nsplit = c >= 0 ? splits_launched(a.K * (int)sizeof(T) / kCfgs[c].RB, split) : 1;
  switch (c) {
    case 0: return run_cfg<T, 256, 256, 2, 4, 64, 4, false, CLK>(epi, a, s, split);
    case 1: return run_cfg<T, 256, 128, 4, 2, 128, 3, false, CLK>(epi, a, s, split);
    case 2: return run_cfg<T, 128, 256, 2, 4, 128, 3, false, CLK>(epi, a, s, split);
    case 3: return run_cfg<T, 128, 128, 2, 2, 128, 3, false, CLK>(epi, a, s, split);
    case 4: return run_cfg<T, 128, 64, 4, 1, 128, 4, false, CLK>(epi, a, s, split);
    case 5: return run_cfg<T, 256, 192, 2, 2, 64, 4, false, CLK>(epi, a, s, split);
    case 6: return run_cfg<T, 128, 384, 2, 2, 64, 4, false, CLK>(epi, a, s, split);
    case 7: return run_cfg<T, 64, 128, 1, 4, 128, 6, false, CLK>(epi, a, s, split);
    case 8: return run_cfg<T, 64, 64, 2, 2, 128, 8, false, CLK>(epi, a, s, split);
    case 9: return run_cfg<T, 64, 128, 1, 4, 128, 6, true, CLK>(epi, a, s, split);
    case 10: return run_cfg<T, 128, 96, 4, 1, 128, 4, false, CLK>(epi, a, s, split);
    case 11: return run_cfg<T, 128, 192, 2, 2, 128, 3, false, CLK>(epi, a, s, split);
  }
  return hipErrorInvalidValue;
}

void gemm_plan(int dtype, EpiKind epi, int M, int K, int Nv, int* bm, int* bn, int* split, int* vb) {
  GemmArgs a{};
  a.M = M; a.K = K; a.Nv = Nv;
  int c, sp;
  pick_cfg(a, epi, dtype == 0 ? 2 : 4, false, c, sp);
  *bm = c >= 0 ? kCfgs[c].BM : 0;
  *bn = c >= 0 ? kCfgs[c].BN : 0;
  *split = c >= 0 ? sp : 0;
  if (vb) *vb = c >= 0 && kCfgs[c].vb ? 1 : 0;
}

int gemm_split(int dtype, EpiKind epi, int M, int K, int Nv) {
  GemmArgs a{};
  a.M = M; a.K = K; a.Nv = Nv;
  const int eb = dtype == 0 ? 2 : 4;
  int c, sp;
  pick_cfg(a, epi, eb, true, c, sp);
  return c >= 0 ? splits_launched(K * eb / kCfgs[c].RB, sp) : 1;
}

hipError_t launch_gemm_clocked(EpiKind epi, const GemmArgs& a, hipStream_t s) {
  if (epi != EPI_SWIGLU && epi != EPI_LOGITS) return hipErrorInvalidValue;
  if (a.M <= 0) return hipSuccess;
  return launch_t<bf16, true>(epi, a, s, nullptr);
}

hipError_t launch_gemm(int dtype, EpiKind epi, const GemmArgs& a, hipStream_t s, int* nsplit) {
  if (nsplit) *nsplit = 1;
  if (a.M <= 0) return hipSuccess;
  return dtype == 0 ? launch_t<bf16>(epi, a, s, nsplit) : launch_t<float>(epi, a, s, nsplit);
}

}  // namespace sl
