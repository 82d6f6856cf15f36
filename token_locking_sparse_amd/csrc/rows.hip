// Row kernels of the active set: gather of the layer-0 input, RMSNorm, the
// K/V cache scatter and the RoPE table.
//
// Gather: the active rows A_t form a compact list (zhaoyang97 notes on
// SureLock, 整体框架); their layer-0 input is the embedding of the current
// token or a given hidden row.  Locked rows are never read.
#include <math.h>

#include "common.hpp"
#include "internal.hpp"

namespace sl {

// One wave per row: x = h / sqrt(mean(h^2) + eps) in the GEMM operand type TO,
// from a row of TI (the fp32 residual stream, or the storage-type input of the
// gather, which is also copied into the fp32 residual stream).  A row of up to
// kRowElems elements is read once into registers (all loads in flight
// together); wider rows are read twice.
constexpr int kRowElems = 8192;

// 4 or 8 floats -> the output type with one or two 16-byte (or one 8-byte) stores
__device__ __forceinline__ void store_x(bf16* dst, const float* f, int n) {
  if (n == 8) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
    st16(dst, w);
  } else {
    uint2 w;
    w.x = pack_bf16x2(f[0], f[1]);
    w.y = pack_bf16x2(f[2], f[3]);
    *reinterpret_cast<uint2*>(dst) = w;
  }
}
__device__ __forceinline__ void store_x(float* dst, const float* f, int n) {
  st16(dst, u32x4{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3])});
  if (n == 8)
    st16(dst + 4, u32x4{__float_as_uint(f[4]), __float_as_uint(f[5]), __float_as_uint(f[6]), __float_as_uint(f[7])});
}

template <typename TI, typename TO, bool H32>
__device__ __forceinline__ void norm_row(const TI* __restrict__ src, int d, float eps, float* __restrict__ h32row,
                                         TO* __restrict__ xrow, int lane) {
  constexpr int E = Chunk<TI>::kElems;
  constexpr int kRowChunks = kRowElems / (64 * E);   // 16-byte chunks per lane
  const int nc = d / E;
  if (nc <= 64 * kRowChunks) {
    u32x4 v[kRowChunks];
#pragma unroll
    for (int k = 0; k < kRowChunks; ++k)
      if (lane + 64 * k < nc) v[k] = ld16(src + (lane + 64 * k) * E);
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < kRowChunks; ++k)
      if (lane + 64 * k < nc) {
        float f[E];
        Chunk<TI>::unpack(v[k], f);
#pragma unroll
        for (int j = 0; j < E; ++j) ss = fmaf(f[j], f[j], ss);
      }
    ss = wave_sum(ss);
    const float r = 1.f / sqrtf(ss / (float)d + eps);
#pragma unroll
    for (int k = 0; k < kRowChunks; ++k)
      if (lane + 64 * k < nc) {
        const int c = lane + 64 * k;
        float f[E], y[E];
        Chunk<TI>::unpack(v[k], f);
        if (H32) store_x(h32row + c * E, f, E);
#pragma unroll
        for (int j = 0; j < E; ++j) y[j] = f[j] * r;
        store_x(xrow + c * E, y, E);
      }
    return;
  }
  float ss = 0.f;
  for (int c = lane; c < nc; c += 64) {
    float f[E];
    Chunk<TI>::unpack(ld16(src + c * E), f);
#pragma unroll
    for (int j = 0; j < E; ++j) ss = fmaf(f[j], f[j], ss);
  }
  ss = wave_sum(ss);
  const float r = 1.f / sqrtf(ss / (float)d + eps);
  for (int c = lane; c < nc; c += 64) {
    float f[E], y[E];
    Chunk<TI>::unpack(ld16(src + c * E), f);
    if (H32) store_x(h32row + c * E, f, E);
#pragma unroll
    for (int j = 0; j < E; ++j) y[j] = f[j] * r;
    store_x(xrow + c * E, y, E);
  }
}

// Gather of the layer-0 input of the active rows (embedding of the current
// token, or a given hidden row) into the fp32 residual stream, plus its RMSNorm.
template <typename T>
__global__ void __launch_bounds__(256)
gather_norm_kernel(const T* __restrict__ h_in, const T* __restrict__ embed, const int32_t* __restrict__ tok,
                   const int32_t* __restrict__ act_idx, const int32_t* __restrict__ act_off, int B, int N,
                   int M_tot, int d, float eps, float* __restrict__ h32, T* __restrict__ x,
                   const int32_t* __restrict__ m_dev) {
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (m >= rows_live(M_tot, m_dev)) return;
  const int b = seq_of_row(act_off, B, m);
  const int64_t g = (int64_t)b * N + act_idx[m];
  const T* src = h_in ? h_in + g * d : embed + (int64_t)tok[g] * d;
  norm_row<T, T, true>(src, d, eps, h32 + (size_t)m * d, x + (size_t)m * d, lane);
}

template <typename T>
__global__ void __launch_bounds__(256)
norm_kernel(const float* __restrict__ h32, int M_tot, int d, float eps, T* __restrict__ x,
            const int32_t* __restrict__ m_dev) {
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (m >= rows_live(M_tot, m_dev)) return;
  norm_row<float, T, false>(h32 + (size_t)m * d, d, eps, nullptr, x + (size_t)m * d, lane);
}

hipError_t launch_gather_norm(int dtype, const void* h_in, const void* embed, const int32_t* tok,
                              const int32_t* act_idx, const int32_t* act_off, int B, int N,
                              int M_tot, int d, float eps, float* h32, void* x, hipStream_t s,
                              const int32_t* m_dev) {
  if (M_tot <= 0) return hipSuccess;
  const dim3 grid((M_tot + 3) / 4), block(256);
  if (dtype == 0)
    hipLaunchKernelGGL(gather_norm_kernel<bf16>, grid, block, 0, s, (const bf16*)h_in, (const bf16*)embed,
                       tok, act_idx, act_off, B, N, M_tot, d, eps, h32, (bf16*)x, m_dev);
  else
    hipLaunchKernelGGL(gather_norm_kernel<float>, grid, block, 0, s, (const float*)h_in, (const float*)embed,
                       tok, act_idx, act_off, B, N, M_tot, d, eps, h32, (float*)x, m_dev);
  return hipGetLastError();
}

// Residual update of a projection split over K, fused with the next RMSNorm:
// h[m] += sum of the S partial planes, then x[m] = h[m] / sqrt(mean(h[m]^2) + eps)
// in the GEMM operand type (skipped when x is NULL).  One workgroup per row;
// each thread takes four 16-byte chunks of the row (d <= 4096), and every load
// of its chunks (the residual and all S partials) is issued before any is used.
// Chunks past the row end re-read the last chunk (in bounds) and are not stored.
constexpr int kResidThreads = 256, kResidCPT = kResidMaxD / 4 / kResidThreads;

template <typename T, int S>
__global__ void __launch_bounds__(kResidThreads)
resid_norm_kernel(const float* __restrict__ part, float* __restrict__ h32, int M_tot, int d, float eps,
                  T* __restrict__ x, const int32_t* __restrict__ m_dev) {
  const int m = blockIdx.x, tid = threadIdx.x;
  if (m >= rows_live(M_tot, m_dev)) return;   // uniform over the workgroup
  const int nc = d / 4;
  float* hrow = h32 + (size_t)m * d;
  f32x4 acc[kResidCPT], pv[S][kResidCPT];
#pragma unroll
  for (int k = 0; k < kResidCPT; ++k) {
    const int c = min(tid + kResidThreads * k, nc - 1);
    acc[k] = *(const f32x4*)(hrow + 4 * c);
#pragma unroll
    for (int sp = 0; sp < S; ++sp) pv[sp][k] = *(const f32x4*)(part + ((size_t)sp * M_tot + m) * d + 4 * c);
  }
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < kResidCPT; ++k) {
    const int c = tid + kResidThreads * k;
#pragma unroll
    for (int sp = 0; sp < S; ++sp) acc[k] += pv[sp][k];
    if (c < nc) {
      *(f32x4*)(hrow + 4 * c) = acc[k];
#pragma unroll
      for (int j = 0; j < 4; ++j) ss = fmaf(acc[k][j], acc[k][j], ss);
    }
  }
  if (!x) return;   // uniform: a kernel argument
  __shared__ float red[kResidThreads / kWave];
  ss = wave_sum(ss);
  if ((tid & (kWave - 1)) == 0) red[tid / kWave] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < kResidThreads / kWave; ++w) tot += red[w];
  const float r = 1.f / sqrtf(tot / (float)d + eps);
  T* xrow = x + (size_t)m * d;
#pragma unroll
  for (int k = 0; k < kResidCPT; ++k) {
    const int c = tid + kResidThreads * k;
    if (c < nc) {
      float y[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) y[j] = acc[k][j] * r;
      store_x(xrow + 4 * c, y, 4);
    }
  }
}

template <typename T>
static hipError_t resid_norm_t(const float* part, int nsplit, float* h32, int M_tot, int d, float eps, T* x,
                               hipStream_t s, const int32_t* m_dev) {
  const dim3 grid(M_tot), block(kResidThreads);
  switch (nsplit) {
    case 2: hipLaunchKernelGGL((resid_norm_kernel<T, 2>), grid, block, 0, s, part, h32, M_tot, d, eps, x, m_dev); break;
    case 3: hipLaunchKernelGGL((resid_norm_kernel<T, 3>), grid, block, 0, s, part, h32, M_tot, d, eps, x, m_dev); break;
    case 4: hipLaunchKernelGGL((resid_norm_kernel<T, 4>), grid, block, 0, s, part, h32, M_tot, d, eps, x, m_dev); break;
    case 5: hipLaunchKernelGGL((resid_norm_kernel<T, 5>), grid, block, 0, s, part, h32, M_tot, d, eps, x, m_dev); break;
    case 6: hipLaunchKernelGGL((resid_norm_kernel<T, 6>), grid, block, 0, s, part, h32, M_tot, d, eps, x, m_dev); break;
    case 7: hipLaunchKernelGGL((resid_norm_kernel<T, 7>), grid, block, 0, s, part, h32, M_tot, d, eps, x, m_dev); break;
    case 8: hipLaunchKernelGGL((resid_norm_kernel<T, 8>), grid, block, 0, s, part, h32, M_tot, d, eps, x, m_dev); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_resid_norm(int dtype, const float* part, int nsplit, float* h32, int M_tot, int d, float eps,
                             void* x, hipStream_t s, const int32_t* m_dev) {
  if (M_tot <= 0) return hipSuccess;
  if (d % 4 || d > kResidMaxD || d < 4) return hipErrorInvalidValue;
  return dtype == 0 ? resid_norm_t<bf16>(part, nsplit, h32, M_tot, d, eps, (bf16*)x, s, m_dev)
                    : resid_norm_t<float>(part, nsplit, h32, M_tot, d, eps, (float*)x, s, m_dev);
}

hipError_t launch_norm(int dtype, const float* h32, int M_tot, int d, float eps, void* x, hipStream_t s,
                       const int32_t* m_dev) {
  if (M_tot <= 0) return hipSuccess;
  const dim3 grid((M_tot + 3) / 4), block(256);
  if (dtype == 0) hipLaunchKernelGGL(norm_kernel<bf16>, grid, block, 0, s, h32, M_tot, d, eps, (bf16*)x, m_dev);
  else hipLaunchKernelGGL(norm_kernel<float>, grid, block, 0, s, h32, M_tot, d, eps, (float*)x, m_dev);
  return hipGetLastError();
}

// K/V scatter: row m of the compact lists goes to cache row b*N + act_idx[m].
__global__ void __launch_bounds__(256)
scatter_kernel(char* __restrict__ kc, char* __restrict__ vc, const char* __restrict__ kn,
               const char* __restrict__ vn, const int32_t* __restrict__ act_idx,
               const int32_t* __restrict__ act_off, int B, int N, int M_tot, int row_chunks) {
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= (int64_t)M_tot * row_chunks) return;
  const int m = (int)(id / row_chunks), c = (int)(id % row_chunks);
  const int b = seq_of_row(act_off, B, m);
  const int64_t g = (int64_t)b * N + act_idx[m];
  const size_t rb = (size_t)row_chunks * 16;
  st16(kc + g * rb + c * 16, ld16(kn + (size_t)m * rb + c * 16));
  st16(vc + g * rb + c * 16, ld16(vn + (size_t)m * rb + c * 16));
}

hipError_t launch_cache_scatter(int dtype, void* kc, void* vc, const void* kn, const void* vn,
                                const int32_t* act_idx, const int32_t* act_off, int B, int N,
                                int M_tot, int row_elems, hipStream_t s) {
  if (M_tot <= 0) return hipSuccess;
  const int row_chunks = row_elems * (dtype == 0 ? 2 : 4) / 16;
  const int64_t total = (int64_t)M_tot * row_chunks;
  hipLaunchKernelGGL(scatter_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, (char*)kc,
                     (char*)vc, (const char*)kn, (const char*)vn, act_idx, act_off, B, N, M_tot, row_chunks);
  return hipGetLastError();
}

// RoPE table: pair j of position p rotates by p * theta^(-2j/Dh), evaluated in double.
__global__ void rope_table_kernel(int n_pos, int half, int Dh, double theta, float* table) {
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= (int64_t)n_pos * half) return;
  const int p = (int)(id / half), j = (int)(id % half);
  const double inv = pow(theta, -(2.0 * j) / (double)Dh);
  double sv, cv;
  sincos((double)p * inv, &sv, &cv);
  table[2 * id] = (float)cv;
  table[2 * id + 1] = (float)sv;
}

hipError_t launch_rope_table(int n_pos, int Dh, float theta, float* table, hipStream_t s) {
  const int half = Dh / 2;
  const int64_t total = (int64_t)n_pos * half;
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, n_pos, half,
                     Dh, (double)theta, table);
  return hipGetLastError();
}

}  // namespace sl
