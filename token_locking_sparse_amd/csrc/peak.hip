// Measurement helpers: the dense bf16 MFMA rate and the HBM streaming rates this
// chip sustains.  They give the measured ceilings that the step's roofline
// fractions are also reported against, beside the vendor figures (2.5 PFLOP/s,
// 8 TB/s).  Not part of the SureLock step.
#include "../../include/surelock.h"
#include "common.hpp"

namespace sl {

// Every wave runs `iters` rounds of kChains independent v_mfma_f32_32x32x16_bf16
// on register operands (no memory traffic), so the matrix cores are the only
// limit.  The operands depend on the thread id and the result is stored under a
// condition that never holds, so nothing is folded away.
constexpr int kPeakChains = 4;

__global__ void __launch_bounds__(256) mfma_peak_kernel(int iters, float* sink) {
  const uint32_t t = threadIdx.x + 1;
  u32x4 a = {0x3f803f80u ^ t, 0x3f003f00u, 0x3e803e80u, 0x3f803f80u};
  u32x4 b = {0x3f003f00u, 0x3f803f80u ^ t, 0x3e003e00u, 0x3f003f00u};
  f32x16 acc[kPeakChains];
#pragma unroll
  for (int c = 0; c < kPeakChains; ++c)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[c][v] = 0.f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < kPeakChains; ++c) Mfma<bf16>::run(acc[c], a, b);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kPeakChains; ++c)
#pragma unroll
    for (int v = 0; v < 16; ++v) s += acc[c][v];
  if (s == 1234.5f) sink[threadIdx.x] = s;
}

// The same loop on operands read from memory: eight A and eight B fragments per lane (16-byte chunk
// (2 i) * 256 + t and (2 i + 1) * 256 + t of `ops` for set i, thread t), rotated so that consecutive
// MFMAs of a chain multiply different values.  The matrix cores' power, and with it the clock the chip
// sustains, depends on the operand bits: random bf16 operands hold it well below what constant ones
// do.  clocks[2 w], clocks[2 w + 1] (w < nclk) receive the shader-clock cycles (s_memtime) and the
// 100 MHz real-time ticks (s_memrealtime) that workgroup w took.
constexpr int kOperandSets = 8;

__global__ void __launch_bounds__(256)
mfma_operand_kernel(int iters, const u32x4* __restrict__ ops, float* sink, unsigned long long* clocks, int nclk) {
  const unsigned long long c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  const int t = threadIdx.x;
  u32x4 a[kOperandSets], b[kOperandSets];
#pragma unroll
  for (int i = 0; i < kOperandSets; ++i) {
    a[i] = ops[(2 * i) * 256 + t];
    b[i] = ops[(2 * i + 1) * 256 + t];
  }
  f32x16 acc[kPeakChains];
#pragma unroll
  for (int c = 0; c < kPeakChains; ++c)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[c][v] = 0.f;
  for (int i = 0; i < iters; i += kOperandSets) {
#pragma unroll
    for (int u = 0; u < kOperandSets; ++u)
#pragma unroll
      for (int c = 0; c < kPeakChains; ++c)
        Mfma<bf16>::run(acc[c], a[(u + c) % kOperandSets], b[(u + 3 * c + 1) % kOperandSets]);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kPeakChains; ++c)
#pragma unroll
    for (int v = 0; v < 16; ++v) s += acc[c][v];
  if (s == 1234.5f) sink[t] = s;
  const unsigned long long c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  if (clocks && t == 0 && (int)blockIdx.x < nclk) {
    clocks[2 * blockIdx.x] = c1 - c0;
    clocks[2 * blockIdx.x + 1] = r1 - r0;
  }
}

// Streaming copy (16-byte non-temporal loads and stores, each workgroup on a
// contiguous range) and streaming read (the loads summed into a register).
constexpr int kStreamThreads = 256, kStreamUnroll = 8;

__global__ void __launch_bounds__(kStreamThreads)
stream_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst, size_t n16, size_t per_block, float* sink) {
  const size_t b0 = (size_t)blockIdx.x * per_block;
  const size_t b1 = b0 + per_block < n16 ? b0 + per_block : n16;
  uint32_t acc = 0;
  for (size_t i0 = b0 + threadIdx.x; i0 < b1; i0 += (size_t)kStreamThreads * kStreamUnroll) {
    u32x4 v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) {
      const size_t i = i0 + (size_t)u * kStreamThreads;
      v[u] = i < b1 ? __builtin_nontemporal_load(src + i) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) {
      const size_t i = i0 + (size_t)u * kStreamThreads;
      if (dst) {
        if (i < b1) __builtin_nontemporal_store(v[u], dst + i);
      } else {
        acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
      }
    }
  }
  if (acc == 0x9e3779b9u) sink[threadIdx.x] = (float)acc;
}

// The LDS-to-MFMA loop of a 256 x 256 GEMM tile on its own: 4 waves (one per SIMD), wave
// tile 128 x 128 (16 accumulators of v_mfma_f32_32x32x16_bf16), 64-byte k-tile rows swizzled
// as the GEMM's, the next k-step's 8 fragments read between the current step's 16 MFMAs.
// LOADS adds what the GEMM's k-tile loop adds around it: per k-tile 8 direct global-to-LDS
// loads of 1 KB per wave into a spare 4-stage ring (from a 1 MiB L2-resident source), the wait
// for the loads of three tiles back, and a workgroup barrier.  The gap between the two rates
// and the GEMM's own is what operand latency from beyond the L2 costs.
typedef __attribute__((address_space(3))) void peak_lds_t;
typedef __attribute__((address_space(1))) void peak_glb_t;

template <bool LOADS>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_loop_kernel(int tiles, const u32x4* __restrict__ src, float* sink) {
  __shared__ __attribute__((aligned(1024))) char lds[160 * 1024];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, hl = lane >> 5, l32 = lane & 31;
  const int wm = wid >> 1, wn = wid & 1;
  for (int i = tid; i < 32 * 1024 / 16; i += 256)
    ((u32x4*)lds)[i] = u32x4{0x3f803f80u ^ (uint32_t)i, 0x3f003f00u, 0x3e803e80u, 0x3f803f80u};
  __syncthreads();
  const char* as = lds;
  const char* bs = lds + 16384;
  char* ring = lds + 32768;                                     // 4 stages of 32 KB
  const u32x4* gsrc = src + (size_t)(blockIdx.x & 31) * (32 * 1024 / 16);
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  u32x4 fa[2][4], fb[2][4];
  auto rd = [&](int ks, int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wm * 128 + i * 32 + l32;
      fa[buf][i] = *(const u32x4*)(as + r * 64 + (swz<64>(r, 2 * (ks & 1) + hl) << 4));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = wn * 128 + j * 32 + l32;
      fb[buf][j] = *(const u32x4*)(bs + r * 64 + (swz<64>(r, 2 * (ks & 1) + hl) << 4));
    }
  };
  auto issue = [&](int t, int j0, int j1) {
    char* st = ring + (t & 3) * 32768;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < j0 || j >= j1) continue;
      __builtin_amdgcn_global_load_lds((peak_glb_t*)(gsrc + (j * 4 + wid) * 64 + lane),
                                       (peak_lds_t*)(st + (j * 4 + wid) * 1024), 16, 0, 0);
    }
  };
  if (LOADS) { issue(0, 0, 8); issue(1, 0, 8); issue(2, 0, 8); }
  rd(0, 0);
  for (int t = 0; t < tiles; ++t) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      if (LOADS) issue(t + 3, ks * 4, ks * 4 + 4);
      if (LOADS && ks == 1) {
        __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));              // lgkmcnt(0)
        __builtin_amdgcn_s_waitcnt((16 & 15) | ((16 >> 4) << 14) | (7 << 4) | (15 << 8));  // vmcnt(16)
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
      }
      rd(ks + 1, (ks + 1) & 1);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) Mfma<bf16>::run(acc[i][j], fa[ks & 1][i], fb[ks & 1][j]);
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) s += acc[i][j][v];
  if (s == 1234.5f) sink[tid] = s + (float)ring[tid];
}

}  // namespace sl

extern "C" {

sl_status sl_peak_mfma(int workgroups, int iters, float* sink, sl_stream stream) {
  if (workgroups <= 0 || iters <= 0 || !sink) return SL_ERR_INVALID;
  hipLaunchKernelGGL(sl::mfma_peak_kernel, dim3(workgroups), dim3(256), 0, (hipStream_t)stream, iters, sink);
  return hipGetLastError() == hipSuccess ? SL_OK : SL_ERR_HIP;
}

double sl_peak_mfma_flops(int workgroups, int iters) {
  return (double)workgroups * 4 /* waves */ * iters * sl::kPeakChains * 2.0 * 32 * 32 * 16;
}

sl_status sl_peak_mfma_operands(int workgroups, int iters, const void* operands, float* sink,
                                unsigned long long* clocks, sl_stream stream) {
  if (workgroups <= 0 || iters <= 0 || iters % sl::kOperandSets || !operands || !sink) return SL_ERR_INVALID;
  hipLaunchKernelGGL(sl::mfma_operand_kernel, dim3(workgroups), dim3(256), 0, (hipStream_t)stream, iters,
                     (const sl::u32x4*)operands, sink, clocks, clocks ? workgroups : 0);
  return hipGetLastError() == hipSuccess ? SL_OK : SL_ERR_HIP;
}

sl_status sl_peak_stream(const void* src, void* dst, size_t bytes, int workgroups, float* sink, sl_stream stream) {
  if (!src || !sink || bytes < 16 || bytes % 16 || workgroups <= 0) return SL_ERR_INVALID;
  const size_t n16 = bytes / 16;
  const size_t per_block = (n16 + workgroups - 1) / workgroups;
  hipLaunchKernelGGL(sl::stream_kernel, dim3(workgroups), dim3(sl::kStreamThreads), 0, (hipStream_t)stream,
                     (const sl::u32x4*)src, (sl::u32x4*)dst, n16, per_block, sink);
  return hipGetLastError() == hipSuccess ? SL_OK : SL_ERR_HIP;
}

sl_status sl_peak_gemm_loop(int workgroups, int tiles, int with_loads, const void* src, float* sink,
                            sl_stream stream) {
  if (workgroups <= 0 || tiles <= 0 || !sink || (with_loads && !src)) return SL_ERR_INVALID;
  if (with_loads)
    hipLaunchKernelGGL(sl::gemm_loop_kernel<true>, dim3(workgroups), dim3(256), 0, (hipStream_t)stream, tiles,
                       (const sl::u32x4*)src, sink);
  else
    hipLaunchKernelGGL(sl::gemm_loop_kernel<false>, dim3(workgroups), dim3(256), 0, (hipStream_t)stream, tiles,
                       (const sl::u32x4*)src, sink);
  return hipGetLastError() == hipSuccess ? SL_OK : SL_ERR_HIP;
}

double sl_peak_gemm_loop_flops(int workgroups, int tiles) {
  return (double)workgroups * 256.0 * 256.0 * 32.0 * 2.0 * tiles;
}

}  // extern "C"
