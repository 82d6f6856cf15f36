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

// One wave per row.  The residual stream h32 is fp32; x = h / sqrt(mean(h^2)+eps)
// is stored in the GEMM operand type.
template <typename T>
__global__ void __launch_bounds__(256)
gather_norm_kernel(const T* __restrict__ h_in, const T* __restrict__ embed, const int32_t* __restrict__ tok,
                   const int32_t* __restrict__ act_idx, const int32_t* __restrict__ act_off, int B, int N,
                   int M_tot, int d, float eps, float* __restrict__ h32, T* __restrict__ x) {
  constexpr int E = 16 / (int)sizeof(T);
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (m >= M_tot) return;
  const int b = seq_of_row(act_off, B, m);
  const int64_t g = (int64_t)b * N + act_idx[m];
  const T* src = h_in ? h_in + g * d : embed + (int64_t)tok[g] * d;
  const int nc = d / E;
  float ss = 0.f;
  for (int c = lane; c < nc; c += 64) {
    float f[E];
    Chunk<T>::unpack(ld16(src + c * E), f);
#pragma unroll
    for (int j = 0; j < E; ++j) ss = fmaf(f[j], f[j], ss);
  }
  ss = wave_sum(ss);
  const float r = 1.f / sqrtf(ss / (float)d + eps);
  for (int c = lane; c < nc; c += 64) {
    float f[E];
    Chunk<T>::unpack(ld16(src + c * E), f);
    float* hp = h32 + (size_t)m * d + c * E;
    T* xp = x + (size_t)m * d + c * E;
#pragma unroll
    for (int j = 0; j < E; ++j) { hp[j] = f[j]; xp[j] = from_f32<T>(f[j] * r); }
  }
}

template <typename T>
__global__ void __launch_bounds__(256)
norm_kernel(const float* __restrict__ h32, int M_tot, int d, float eps, T* __restrict__ x) {
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (m >= M_tot) return;
  const float* hp = h32 + (size_t)m * d;
  const int nc = d / 4;
  float ss = 0.f;
  for (int c = lane; c < nc; c += 64) {
    const f32x4 v = *(const f32x4*)(hp + 4 * c);
#pragma unroll
    for (int j = 0; j < 4; ++j) ss = fmaf(v[j], v[j], ss);
  }
  ss = wave_sum(ss);
  const float r = 1.f / sqrtf(ss / (float)d + eps);
  T* xp = x + (size_t)m * d;
  for (int c = lane; c < nc; c += 64) {
    const f32x4 v = *(const f32x4*)(hp + 4 * c);
#pragma unroll
    for (int j = 0; j < 4; ++j) xp[4 * c + j] = from_f32<T>(v[j] * r);
  }
}

hipError_t launch_gather_norm(int dtype, const void* h_in, const void* embed, const int32_t* tok,
                              const int32_t* act_idx, const int32_t* act_off, int B, int N,
                              int M_tot, int d, float eps, float* h32, void* x, hipStream_t s) {
  if (M_tot <= 0) return hipSuccess;
  const dim3 grid((M_tot + 3) / 4), block(256);
  if (dtype == 0)
    hipLaunchKernelGGL(gather_norm_kernel<bf16>, grid, block, 0, s, (const bf16*)h_in, (const bf16*)embed,
                       tok, act_idx, act_off, B, N, M_tot, d, eps, h32, (bf16*)x);
  else
    hipLaunchKernelGGL(gather_norm_kernel<float>, grid, block, 0, s, (const float*)h_in, (const float*)embed,
                       tok, act_idx, act_off, B, N, M_tot, d, eps, h32, (float*)x);
  return hipGetLastError();
}

hipError_t launch_norm(int dtype, const float* h32, int M_tot, int d, float eps, void* x, hipStream_t s) {
  if (M_tot <= 0) return hipSuccess;
  const dim3 grid((M_tot + 3) / 4), block(256);
  if (dtype == 0) hipLaunchKernelGGL(norm_kernel<bf16>, grid, block, 0, s, h32, M_tot, d, eps, (bf16*)x);
  else hipLaunchKernelGGL(norm_kernel<float>, grid, block, 0, s, h32, M_tot, d, eps, (float*)x);
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
