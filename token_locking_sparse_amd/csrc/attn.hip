// Active-query attention: the M active queries of a sequence attend over all
// N positions of that sequence, locked ones through their cached K/V
// (zhaoyang97 notes on SureLock, 永久锁定机制: K^all[L_t] <- C.k[L_t]); cost
// O(M N d) instead of O(N^2 d) (paperdance abstract).
//
// One workgroup = 4 waves x 32 query rows of one (sequence, head), looping
// over 64-key tiles staged in LDS (double-buffered).  Scores are computed
// transposed, S^T = K Q^T, so each lane owns one query row and the online
// softmax statistics stay in registers; the output is produced transposed too,
// O^T = V^T P^T, with V stored transposed in LDS and P fed straight from the
// score registers.  For bf16 the LDS order of keys inside each group of 16 is
// permuted (quads 1 and 2 swapped) so that a lane's eight P values line up with
// eight consecutive V^T entries.  Few query tiles => the keys are split over
// several workgroups and a second kernel merges the partial softmaxes.
#include <math.h>

#include "common.hpp"
#include "internal.hpp"

namespace sl {

constexpr int kAttnThreads = 256;
constexpr int kBQ = 128;   // query rows per workgroup (32 per wave)
constexpr int kBKV = 64;   // keys per tile

template <typename T, int Dh>
struct AttnCfg {
  static constexpr int E = 16 / (int)sizeof(T);        // elements per 16-byte chunk
  static constexpr int KC = Dh / E;                     // chunks per K row
  static constexpr int VC = kBKV / E;                   // chunks per V^T row
  static constexpr int KBytes = kBKV * Dh * (int)sizeof(T);
  static constexpr int VBytes = Dh * kBKV * (int)sizeof(T);
  static constexpr int Stage = KBytes + VBytes;
  static constexpr int EpiBytes = 4 * 32 * (Dh + 1) * 4;
  static constexpr int Smem = (2 * Stage > EpiBytes) ? 2 * Stage : EpiBytes;
  static constexpr int nKK = Dh / (2 * E);              // QK^T fragments per key subtile
  static constexpr int nPV = kBKV / (2 * E);            // PV fragments per key tile
  static constexpr int KLoads = kBKV * KC / kAttnThreads;
  static constexpr int VTasks = (kBKV / 2) * KC;        // (key pair, d chunk)
  static constexpr int VLoads = (VTasks + kAttnThreads - 1) / kAttnThreads;
  static_assert(KLoads >= 1 && kBKV * KC % kAttnThreads == 0, "K tile split");
};


// LDS position of key k (0..63) of a tile inside V^T rows.
template <typename T>
__device__ __forceinline__ int vpos(int k) {
  if (sizeof(T) == 4) return k;
  const int r = k & 15, quad = r >> 2;
  const int q2 = (quad == 1) ? 2 : (quad == 2 ? 1 : quad);
  return (k & ~15) + 4 * q2 + (r & 3);
}

// Locate query tile `slot` of the ragged sequences: returns b (or -1) and the
// first row of the tile.
__device__ __forceinline__ int find_tile(const int32_t* act_off, int B, int slot, int& row0, int& row_end) {
  int s = slot;
  for (int b = 0; b < B; ++b) {
    const int o0 = act_off[b], o1 = act_off[b + 1];
    const int nt = (o1 - o0 + kBQ - 1) / kBQ;
    if (s < nt) { row0 = o0 + s * kBQ; row_end = o1; return b; }
    s -= nt;
  }
  return -1;
}

template <typename T, int Dh>
__global__ void __launch_bounds__(kAttnThreads)
attn_kernel(const T* __restrict__ q, const T* __restrict__ kc, const T* __restrict__ vc,
            const int32_t* __restrict__ act_off, int B, int N, int H, float scale_log2,
            int nsplit, int tiles_per_split, T* __restrict__ out, float* __restrict__ part_o,
            float* __restrict__ part_ml, int M_tot) {
  using C = AttnCfg<T, Dh>;
  constexpr int E = C::E;
  __shared__ __attribute__((aligned(16))) char smem[C::Smem];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, hl = lane >> 5, l32 = lane & 31;
  const int h = blockIdx.y, split = blockIdx.z;
  int row0 = 0, row_end = 0;
  const int b = find_tile(act_off, B, blockIdx.x, row0, row_end);
  if (b < 0) return;
  const int n_tiles_total = N / kBKV;
  const int t_begin = split * tiles_per_split;
  const int t_end = min(n_tiles_total, t_begin + tiles_per_split);
  const int HD = H * Dh;

  // query fragments (B operand of S^T = K Q^T): lane owns query row q0 + l32
  const int wrow0 = row0 + wid * 32;
  const bool wave_live = wrow0 < row_end;
  const int my_row = min(wrow0 + l32, row_end - 1);
  u32x4 qf[C::nKK];
  {
    const char* qr = (const char*)(q + (size_t)my_row * HD + (size_t)h * Dh);
#pragma unroll
    for (int kk = 0; kk < C::nKK; ++kk) qf[kk] = ld16(qr + (2 * kk + hl) * 16);
  }

  const char* kbase = (const char*)(kc + ((size_t)b * N * H + h) * Dh);
  const char* vbase = (const char*)(vc + ((size_t)b * N * H + h) * Dh);
  const size_t krow_stride = (size_t)HD * sizeof(T);

  u32x4 kreg[C::KLoads];
  u32x4 vreg[C::VLoads][2];
  auto gload = [&](int tile) {
    const int key0 = tile * kBKV;
#pragma unroll
    for (int i = 0; i < C::KLoads; ++i) {
      const int id = tid + i * kAttnThreads;
      const int kr = id / C::KC, c = id % C::KC;
      kreg[i] = ld16(kbase + (size_t)(key0 + kr) * krow_stride + c * 16);
    }
#pragma unroll
    for (int i = 0; i < C::VLoads; ++i) {
      const int id = tid + i * kAttnThreads;
      if (id < C::VTasks) {
        const int kp = id % (kBKV / 2), dc = id / (kBKV / 2);
        vreg[i][0] = ld16(vbase + (size_t)(key0 + 2 * kp) * krow_stride + dc * 16);
        vreg[i][1] = ld16(vbase + (size_t)(key0 + 2 * kp + 1) * krow_stride + dc * 16);
      }
    }
  };
  auto lstore = [&](int stage) {
    char* ks = smem + stage * C::Stage;
    char* vs = ks + C::KBytes;
#pragma unroll
    for (int i = 0; i < C::KLoads; ++i) {
      const int id = tid + i * kAttnThreads;
      const int kr = id / C::KC, c = id % C::KC;
      st16(ks + kr * (Dh * (int)sizeof(T)) + swz<Dh * (int)sizeof(T)>(kr, c) * 16, kreg[i]);
    }
#pragma unroll
    for (int i = 0; i < C::VLoads; ++i) {
      const int id = tid + i * kAttnThreads;
      if (id < C::VTasks) {
        const int kp = id % (kBKV / 2), dc = id / (kBKV / 2);
        const int p = vpos<T>(2 * kp);          // keys 2kp, 2kp+1 stay adjacent
        const int pc = (p * (int)sizeof(T)) >> 4, po = (p * (int)sizeof(T)) & 15;
        if (sizeof(T) == 2) {
          const uint32_t* a0 = (const uint32_t*)&vreg[i][0];
          const uint32_t* a1 = (const uint32_t*)&vreg[i][1];
#pragma unroll
          for (int j = 0; j < E; ++j) {
            const int d = dc * E + j;
            const uint32_t x0 = (j & 1) ? (a0[j >> 1] >> 16) : (a0[j >> 1] & 0xffffu);
            const uint32_t x1 = (j & 1) ? (a1[j >> 1] & 0xffff0000u) : (a1[j >> 1] << 16);
            *(uint32_t*)(vs + d * (kBKV * 2) + (swz<kBKV * 2>(d, pc) << 4) + po) = x0 | x1;
          }
        } else {
          const uint32_t* a0 = (const uint32_t*)&vreg[i][0];
          const uint32_t* a1 = (const uint32_t*)&vreg[i][1];
#pragma unroll
          for (int j = 0; j < E; ++j) {
            const int d = dc * E + j;
            uint2 pr; pr.x = a0[j]; pr.y = a1[j];
            *(uint2*)(vs + d * (kBKV * 4) + (swz<kBKV * 4>(d, pc) << 4) + po) = pr;
          }
        }
      }
    }
  };

  f32x16 oacc[Dh / 32];
#pragma unroll
  for (int i = 0; i < Dh / 32; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[i][v] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  if (t_begin < t_end) {
    gload(t_begin);
    lstore(0);
  }
  __syncthreads();
  for (int t = t_begin; t < t_end; ++t) {
    const int stage = (t - t_begin) & 1;
    if (t + 1 < t_end) gload(t + 1);
    if (wave_live) {
      const char* ks = smem + stage * C::Stage;
      const char* vs = ks + C::KBytes;
      f32x16 s[2];
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
        for (int v = 0; v < 16; ++v) s[sub][v] = 0.f;
        const int kr = sub * 32 + l32;
#pragma unroll
        for (int kk = 0; kk < C::nKK; ++kk) {
          const u32x4 a = *(const u32x4*)(ks + kr * (Dh * (int)sizeof(T)) + swz<Dh * (int)sizeof(T)>(kr, 2 * kk + hl) * 16);
          Mfma<T>::run(s[sub], a, qf[kk]);
        }
      }
      // online softmax in log2 units; lane pair (l, l^32) shares a query row
      float mx = -INFINITY;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[sub][v]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * scale_log2;
      const float m_new = fmaxf(m_run, mx);
      const float alpha = (m_run > -INFINITY) ? __builtin_amdgcn_exp2f(m_run - m_new) : 0.f;
      m_run = m_new;
      float ls = 0.f;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float pv = __builtin_amdgcn_exp2f(fmaf(s[sub][v], scale_log2, -m_new));
          s[sub][v] = pv;
          ls += pv;
        }
      l_run = l_run * alpha + ls;
#pragma unroll
      for (int i = 0; i < Dh / 32; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[i][v] *= alpha;
      // O^T += V^T P^T
#pragma unroll
      for (int ks2 = 0; ks2 < C::nPV; ++ks2) {
        constexpr int FPS = 16 / E;  // fragments per 32-key subtile
        const int sub = ks2 / FPS, r0 = (ks2 % FPS) * E;
        u32x4 pb;
        if (sizeof(T) == 2) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bf16 lo = (bf16)s[sub][r0 + 2 * i], hi = (bf16)s[sub][r0 + 2 * i + 1];
            pb[i] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) pb[i] = __float_as_uint(s[sub][r0 + i]);
        }
#pragma unroll
        for (int dt = 0; dt < Dh / 32; ++dt) {
          const int d = dt * 32 + l32;
          const u32x4 a = *(const u32x4*)(vs + d * (kBKV * (int)sizeof(T)) + (swz<kBKV * (int)sizeof(T)>(d, 2 * ks2 + hl) << 4));
          Mfma<T>::run(oacc[dt], a, pb);
        }
      }
    }
    if (t + 1 < t_end) lstore(stage ^ 1);
    __syncthreads();
  }

  // epilogue: stage O (query-major) through LDS, then write rows with 16-byte stores
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const bool final_out = (nsplit == 1);
  const float inv = (final_out && l_tot > 0.f) ? 1.f / l_tot : 1.f;
  float* ep = (float*)smem + wid * 32 * (Dh + 1);
  // (all waves passed the last barrier of the loop, so the K/V stages are free)
#pragma unroll
  for (int dt = 0; dt < Dh / 32; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int d = dt * 32 + (v >> 2) * 8 + 4 * hl + (v & 3);
      ep[l32 * (Dh + 1) + d] = oacc[dt][v] * inv;
    }
  __syncthreads();
  if (wave_live) {
    const int nrow = min(32, row_end - wrow0);
    if (final_out) {
      constexpr int CPR = Dh / E;  // 16-byte chunks per output row
      for (int id = lane; id < 32 * CPR; id += 64) {
        const int rr = id / CPR, c = id % CPR;
        if (rr < nrow) {
          const float* src = ep + rr * (Dh + 1) + c * E;
          u32x4 w;
          if (sizeof(T) == 2) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const bf16 lo = (bf16)src[2 * i], hi = (bf16)src[2 * i + 1];
              w[i] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
            }
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) w[i] = __float_as_uint(src[i]);
          }
          st16((char*)(out + (size_t)(wrow0 + rr) * HD + (size_t)h * Dh) + c * 16, w);
        }
      }
    } else {
      constexpr int CPR = Dh / 4;
      for (int id = lane; id < 32 * CPR; id += 64) {
        const int rr = id / CPR, c = id % CPR;
        if (rr < nrow) {
          const float* src = ep + rr * (Dh + 1) + c * 4;
          u32x4 w;
#pragma unroll
          for (int i = 0; i < 4; ++i) w[i] = __float_as_uint(src[i]);
          st16(part_o + (((size_t)split * M_tot + wrow0 + rr) * H + h) * Dh + c * 4, w);
        }
      }
      if (hl == 0 && l32 < nrow) {
        float* ml = part_ml + (((size_t)split * M_tot + wrow0 + l32) * H + h) * 2;
        ml[0] = m_run;
        ml[1] = l_tot;
      }
    }
  }
}

// Merge the split-KV partial softmaxes: one wave per (row, head).
template <typename T, int Dh>
__global__ void __launch_bounds__(256)
attn_combine_kernel(const float* __restrict__ part_o, const float* __restrict__ part_ml, int nsplit,
                    int M_tot, int H, T* __restrict__ out) {
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (w >= M_tot * H) return;
  const int m = w / H, h = w % H;
  float mx = -INFINITY;
  for (int s = 0; s < nsplit; ++s) mx = fmaxf(mx, part_ml[(((size_t)s * M_tot + m) * H + h) * 2]);
  float L = 0.f;
  float acc[(Dh + 63) / 64];
#pragma unroll
  for (int i = 0; i < (Dh + 63) / 64; ++i) acc[i] = 0.f;
  for (int s = 0; s < nsplit; ++s) {
    const float* ml = part_ml + (((size_t)s * M_tot + m) * H + h) * 2;
    const float wgt = (ml[0] > -INFINITY) ? __builtin_amdgcn_exp2f(ml[0] - mx) : 0.f;
    L += ml[1] * wgt;
    const float* po = part_o + (((size_t)s * M_tot + m) * H + h) * Dh;
#pragma unroll
    for (int i = 0; i < (Dh + 63) / 64; ++i) {
      const int d = lane + 64 * i;
      if (d < Dh) acc[i] += po[d] * wgt;
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
  for (int i = 0; i < (Dh + 63) / 64; ++i) {
    const int d = lane + 64 * i;
    if (d < Dh) out[(size_t)m * H * Dh + (size_t)h * Dh + d] = from_f32<T>(acc[i] * inv);
  }
}

static void attn_plan(int B, int N, int M_tot, int H, int& slots, int& nsplit, int& tps) {
  slots = (M_tot + kBQ - 1) / kBQ + B;
  const int tiles = N / kBKV;
  const int blocks = ((M_tot + kBQ - 1) / kBQ) * H;   // useful workgroups without a split
  nsplit = 1;
  while (blocks * nsplit < 512 && nsplit * 2 <= tiles / 2) nsplit *= 2;
  tps = (tiles + nsplit - 1) / nsplit;
}

size_t attn_ws_bytes(int B, int N, int M_tot, int H, int Dh) {
  int slots, nsplit, tps;
  attn_plan(B, N, M_tot, H, slots, nsplit, tps);
  if (nsplit == 1) return 256;
  return (size_t)nsplit * M_tot * H * (Dh + 2) * 4 + 256;
}

template <typename T, int Dh>
static hipError_t attn_launch_t(const void* q, const void* kc, const void* vc, const int32_t* act_off,
                                int B, int N, int M_tot, int H, float scale, void* out, void* ws,
                                hipStream_t s) {
  int slots, nsplit, tps;
  attn_plan(B, N, M_tot, H, slots, nsplit, tps);
  float* part_o = (float*)ws;
  float* part_ml = part_o + (size_t)nsplit * M_tot * H * Dh;
  const float sl2 = scale * kLog2e;
  hipLaunchKernelGGL((attn_kernel<T, Dh>), dim3(slots, H, nsplit), dim3(kAttnThreads), 0, s,
                     (const T*)q, (const T*)kc, (const T*)vc, act_off, B, N, H, sl2, nsplit, tps,
                     (T*)out, part_o, part_ml, M_tot);
  if (nsplit > 1) {
    const int waves = M_tot * H;
    hipLaunchKernelGGL((attn_combine_kernel<T, Dh>), dim3((waves + 3) / 4), dim3(256), 0, s, part_o,
                       part_ml, nsplit, M_tot, H, (T*)out);
  }
  return hipGetLastError();
}

hipError_t launch_attn(int dtype, const void* q, const void* kc, const void* vc,
                       const int32_t* act_off, int B, int N, int M_tot, int H, int Dh, float scale,
                       void* out, void* ws, hipStream_t s) {
  if (M_tot <= 0) return hipSuccess;
  if (dtype == 0) {
    if (Dh == 128) return attn_launch_t<bf16, 128>(q, kc, vc, act_off, B, N, M_tot, H, scale, out, ws, s);
    if (Dh == 64) return attn_launch_t<bf16, 64>(q, kc, vc, act_off, B, N, M_tot, H, scale, out, ws, s);
    if (Dh == 32) return attn_launch_t<bf16, 32>(q, kc, vc, act_off, B, N, M_tot, H, scale, out, ws, s);
  } else {
    if (Dh == 128) return attn_launch_t<float, 128>(q, kc, vc, act_off, B, N, M_tot, H, scale, out, ws, s);
    if (Dh == 64) return attn_launch_t<float, 64>(q, kc, vc, act_off, B, N, M_tot, H, scale, out, ws, s);
    if (Dh == 32) return attn_launch_t<float, 32>(q, kc, vc, act_off, B, N, M_tot, H, scale, out, ws, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace sl
