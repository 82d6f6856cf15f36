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
//   EPI_LOGITS logits written to rows b*N + pos of the posterior buffer.
// Paired epilogues (RoPE halves, gate/up) use a "pair layout": in every wave's
// N-range the first half of the columns holds the first element of each pair
// and the second half its partner, so both land in the same lane and register.
#include <math.h>

#include "common.hpp"
#include "internal.hpp"

namespace sl {

constexpr int kGemmThreads = 256;
constexpr int kRowBytes = 128;   // bytes of K per row per stage (64 bf16 / 32 fp32)

template <typename T, int BM, int BN, int WM, int WN>
struct GemmCfg {
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int FM = TM / 32, FN = TN / 32;
  static constexpr int ALoads = BM * 8 / kGemmThreads;
  static constexpr int BLoads = BN * 8 / kGemmThreads;
  static constexpr int StageBytes = (BM + BN) * kRowBytes;
  static_assert(WM * WN == 4, "four waves");
  static_assert(FM >= 1 && FN >= 1 && TM % 32 == 0 && TN % 32 == 0, "wave tile");
  static_assert(ALoads >= 1 && BLoads >= 1, "load split");
};

__device__ __forceinline__ int gswz(int row, int c) { return c ^ (row & 7); }

__device__ __forceinline__ float silu_f(float g) { return g / (1.f + __expf(-g)); }

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

template <typename T, int BM, int BN, int WM, int WN, int EPI>
__global__ void __launch_bounds__(kGemmThreads)
gemm_kernel(GemmArgs a, int MT, int NT, int k_iters_per_split) {
  using C = GemmCfg<T, BM, BN, WM, WN>;
  __shared__ __attribute__((aligned(16))) char smem[2 * C::StageBytes];
  __shared__ int s_pos[BM];
  __shared__ int s_glob[BM];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, hl = lane >> 5, l32 = lane & 31;
  const int wm = wid / WN, wn = wid % WN;

  // workgroup -> tile; tiles sharing a weight tile are consecutive and sit on one XCD
  const int nb = MT * NT;
  int lid = blockIdx.x;
  if ((nb & 7) == 0) lid = (blockIdx.x & 7) * (nb >> 3) + (blockIdx.x >> 3);
  const int bm = lid % MT, bn = lid / MT;
  const int m0 = bm * BM, n0 = bn * BN;
  const int split = blockIdx.z;
  const int KI = a.K * (int)sizeof(T) / kRowBytes;
  const int kt0 = split * k_iters_per_split;
  const int kt1 = min(KI, kt0 + k_iters_per_split);

  if (EPI == EPI_QKV || EPI == EPI_LOGITS) {
    for (int r = tid; r < BM; r += kGemmThreads) {
      const int m = min(m0 + r, a.M - 1);
      const int b = seq_of_row(a.act_off, a.B, m);
      const int pos = a.act_idx[m];
      s_pos[r] = pos;
      s_glob[r] = b * a.N + pos;
    }
  }

  // global source pointers of this thread's 16-byte chunks
  const char* ap[C::ALoads];
  const char* bp[C::BLoads];
  const size_t arb = (size_t)a.K * sizeof(T);
#pragma unroll
  for (int i = 0; i < C::ALoads; ++i) {
    const int id = tid + i * kGemmThreads;
    const int r = id >> 3, c = id & 7;
    ap[i] = (const char*)a.A + (size_t)min(m0 + r, a.M - 1) * arb + c * 16;
  }
#pragma unroll
  for (int i = 0; i < C::BLoads; ++i) {
    const int id = tid + i * kGemmThreads;
    const int r = id >> 3, c = id & 7;
    bp[i] = w_row_ptr<T, EPI>(a, n0 + r, C::TN) + c * 16;
  }
  u32x4 ra[C::ALoads], rb[C::BLoads];
  auto gload = [&](int kt) {
    const size_t off = (size_t)kt * kRowBytes;
#pragma unroll
    for (int i = 0; i < C::ALoads; ++i) ra[i] = ld16(ap[i] + off);
#pragma unroll
    for (int i = 0; i < C::BLoads; ++i) rb[i] = ld16(bp[i] + off);
  };
  auto lstore = [&](int stage) {
    char* as = smem + stage * C::StageBytes;
    char* bs = as + BM * kRowBytes;
#pragma unroll
    for (int i = 0; i < C::ALoads; ++i) {
      const int id = tid + i * kGemmThreads;
      const int r = id >> 3, c = id & 7;
      st16(as + r * kRowBytes + gswz(r, c) * 16, ra[i]);
    }
#pragma unroll
    for (int i = 0; i < C::BLoads; ++i) {
      const int id = tid + i * kGemmThreads;
      const int r = id >> 3, c = id & 7;
      st16(bs + r * kRowBytes + gswz(r, c) * 16, rb[i]);
    }
  };

  f32x16 acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  if (kt0 < kt1) {
    gload(kt0);
    lstore(0);
  }
  __syncthreads();
  for (int kt = kt0; kt < kt1; ++kt) {
    const int stage = (kt - kt0) & 1;
    if (kt + 1 < kt1) gload(kt + 1);
    const char* as = smem + stage * C::StageBytes;
    const char* bs = as + BM * kRowBytes;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4 fa[C::FM], fb[C::FN];
#pragma unroll
      for (int i = 0; i < C::FM; ++i) {
        const int r = wm * C::TM + i * 32 + l32;
        fa[i] = *(const u32x4*)(as + r * kRowBytes + gswz(r, 2 * ks + hl) * 16);
      }
#pragma unroll
      for (int j = 0; j < C::FN; ++j) {
        const int r = wn * C::TN + j * 32 + l32;
        fb[j] = *(const u32x4*)(bs + r * kRowBytes + gswz(r, 2 * ks + hl) * 16);
      }
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) Mfma<T>::run(acc[i][j], fa[i], fb[j]);
    }
    if (kt + 1 < kt1) lstore(stage ^ 1);
    __syncthreads();
  }

  // ---------------------------------------------------------------- epilogues
#pragma unroll
  for (int i = 0; i < C::FM; ++i) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int lr = wm * C::TM + i * 32 + (v >> 2) * 8 + 4 * hl + (v & 3);
      const int m = m0 + lr;
      if (m >= a.M) continue;
      if (EPI == EPI_RESID) {
        float* h = (float*)a.out0 + (size_t)m * a.Nv + n0 + wn * C::TN + l32;
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
          if (a.split_k > 1) unsafeAtomicAdd(h + j * 32, acc[i][j][v]);
          else h[j * 32] += acc[i][j][v];
        }
      } else if (EPI == EPI_LOGITS) {
        T* o = (T*)a.out0 + (size_t)s_glob[lr] * a.Nv + n0 + wn * C::TN + l32;
#pragma unroll
        for (int j = 0; j < C::FN; ++j) o[j * 32] = from_f32<T>(acc[i][j][v]);
      } else {
        const int pbase = (n0 + wn * C::TN) / 2 + l32;
#pragma unroll
        for (int j = 0; j < C::FN / 2; ++j) {
          const float x1 = acc[i][j][v], x2 = acc[i][j + C::FN / 2][v];
          const int pair = pbase + j * 32;
          if (EPI == EPI_SWIGLU) {
            const int F = a.Nv / 2;
            ((T*)a.out0)[(size_t)m * F + pair] = from_f32<T>(silu_f(x1) * x2);
          } else {
            const int hd = a.d / 2, hh = a.Dh / 2;
            const int mat = pair / hd, gp = pair % hd;
            const int jj = gp % hh;
            const int col = (gp / hh) * a.Dh + jj;
            float y1 = x1, y2 = x2;
            if (mat < 2) {
              const float2 cs = *(const float2*)(a.rope + ((size_t)s_pos[lr] * hh + jj) * 2);
              y1 = x1 * cs.x - x2 * cs.y;
              y2 = x2 * cs.x + x1 * cs.y;
            }
            T* dst;
            if (mat == 0) dst = (T*)a.out0 + (size_t)m * a.d;
            else dst = (T*)(mat == 1 ? a.out1 : a.out2) + (size_t)s_glob[lr] * a.d;
            dst[col] = from_f32<T>(y1);
            dst[col + hh] = from_f32<T>(y2);
          }
        }
      }
    }
  }
}

// ------------------------------------------------------------------ dispatch
struct TileCfg { int BM, BN; };

template <typename T, int BM, int BN, int WM, int WN>
static hipError_t run_cfg(EpiKind epi, const GemmArgs& a, hipStream_t s, int split) {
  const int MT = (a.M + BM - 1) / BM, NT = a.Nv / BN;
  const int KI = a.K * (int)sizeof(T) / kRowBytes;
  const int kps = (KI + split - 1) / split;
  const int nsplit = (KI + kps - 1) / kps;
  GemmArgs b = a;
  b.split_k = nsplit;
  const dim3 grid(MT * NT, 1, nsplit), block(kGemmThreads);
  switch (epi) {
    case EPI_QKV: hipLaunchKernelGGL((gemm_kernel<T, BM, BN, WM, WN, EPI_QKV>), grid, block, 0, s, b, MT, NT, kps); break;
    case EPI_RESID: hipLaunchKernelGGL((gemm_kernel<T, BM, BN, WM, WN, EPI_RESID>), grid, block, 0, s, b, MT, NT, kps); break;
    case EPI_SWIGLU: hipLaunchKernelGGL((gemm_kernel<T, BM, BN, WM, WN, EPI_SWIGLU>), grid, block, 0, s, b, MT, NT, kps); break;
    case EPI_LOGITS: hipLaunchKernelGGL((gemm_kernel<T, BM, BN, WM, WN, EPI_LOGITS>), grid, block, 0, s, b, MT, NT, kps); break;
  }
  return hipGetLastError();
}

// Tile shapes: 0 = 256x256 (wave 128x128), 1 = 128x128 (64x64), 2 = 128x64 (32x64, waves 4x1).
static const TileCfg kCfgs[3] = {{256, 256}, {128, 128}, {128, 64}};

static int pick_cfg(const GemmArgs& a) {
  // largest tile that still gives >= 256 workgroups; else the one with the most tiles
  int best = -1;
  for (int c = 0; c < 3; ++c) {
    if (a.Nv % kCfgs[c].BN) continue;
    const long tiles = (long)((a.M + kCfgs[c].BM - 1) / kCfgs[c].BM) * (a.Nv / kCfgs[c].BN);
    if (tiles >= 256) return c;
    best = c;
  }
  return best;
}

int gemm_supported(int dtype, EpiKind epi, int Nv, int K, int d, int Dh) {
  const int eb = dtype == 0 ? 2 : 4;
  if ((K * eb) % kRowBytes) return 0;
  if (Nv % 64) return 0;
  if (epi == EPI_QKV && (d % 128 || Dh % 2)) return 0;
  return 1;
}

template <typename T>
static hipError_t launch_t(EpiKind epi, const GemmArgs& a, hipStream_t s) {
  const int c = pick_cfg(a);
  if (c < 0) return hipErrorInvalidValue;
  const int BM = kCfgs[c].BM, BN = kCfgs[c].BN;
  const long tiles = (long)((a.M + BM - 1) / BM) * (a.Nv / BN);
  int split = 1;
  if (epi == EPI_RESID) {
    const int KI = a.K * (int)sizeof(T) / kRowBytes;
    while (tiles * split * 2 <= 512 && KI / (split * 2) >= 8) split *= 2;
  }
  if (c == 0) return run_cfg<T, 256, 256, 2, 2>(epi, a, s, split);
  if (c == 1) return run_cfg<T, 128, 128, 2, 2>(epi, a, s, split);
  return run_cfg<T, 128, 64, 4, 1>(epi, a, s, split);
}

hipError_t launch_gemm(int dtype, EpiKind epi, const GemmArgs& a, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  return dtype == 0 ? launch_t<bf16>(epi, a, s) : launch_t<float>(epi, a, s);
}

}  // namespace sl
