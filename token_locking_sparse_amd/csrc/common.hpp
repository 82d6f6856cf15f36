// Device-side building blocks shared by the SureLock kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sl {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ------------------------------------------------------------------ element conversions
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }

// Two floats -> two bf16 (round to nearest even) in one 32-bit word, low half first.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t x = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2_t));
}

// 16-byte chunk -> float values (8 for bf16, 4 for f32).
template <typename T> struct Chunk;
template <> struct Chunk<bf16> {
  static constexpr int kElems = 8;
  __device__ static __forceinline__ void unpack(const u32x4& c, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) { f[2 * i] = bf16_lo(c[i]); f[2 * i + 1] = bf16_hi(c[i]); }
  }
};
template <> struct Chunk<float> {
  static constexpr int kElems = 4;
  __device__ static __forceinline__ void unpack(const u32x4& c, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(c[i]);
  }
};

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }
// Streaming read of data used once (non-temporal hint: do not keep it in the caches).
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// ------------------------------------------------------------------ MFMA traits
// A 16-byte fragment per lane per operand.  For bf16 one fragment feeds one
// v_mfma_f32_32x32x16_bf16 (lane l: row l%32, k = 8*(l/32) + 0..7).  For f32 one
// fragment feeds four v_mfma_f32_32x32x2f32 (lane l: row l%32, k = l/32, element
// j of the fragment in the j-th instruction).  Both operands use the same k
// assignment, so the contraction is exact either way.  Output (both): lane l,
// register v holds row (v/4)*8 + 4*(l/32) + v%4, column l%32.
template <typename T> struct Mfma;
template <> struct Mfma<bf16> {
  __device__ static __forceinline__ void run(f32x16& acc, const u32x4& a, const u32x4& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
  }
};
template <> struct Mfma<float> {
  __device__ static __forceinline__ void run(f32x16& acc, const u32x4& a, const u32x4& b) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[j]), __uint_as_float(b[j]), acc, 0, 0, 0);
  }
};

// ------------------------------------------------------------------ LDS swizzle
// LDS tiles are rows of RB bytes made of 16-byte chunks.  A 128-bit LDS read is
// served 16 lanes at a time over 64 four-byte banks (256 bytes), so the 16
// rows a fragment read touches must put their chunks in 16 distinct slots of
// a 256-byte window: chunk c of `row` is stored at position
// c ^ ((row / max(1, 256/RB)) & (min(RB/16, 16) - 1)).
template <int RB>
__device__ __forceinline__ int swz(int row, int c) {
  constexpr int W = RB >= 256 ? 1 : 256 / RB;
  constexpr int CPR = RB / 16;
  constexpr int MASK = (CPR < 16 ? CPR : 16) - 1;
  return c ^ ((row / W) & MASK);
}

// ------------------------------------------------------------------ wave / block reductions
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// DPP wave primitives (no LDS round trip).  Within each row of 16 lanes the
// row_shr:1,2,4,8 steps form an inclusive scan; row_bcast:15 then adds row 0's
// (row 2's) total to row 1 (row 3), and row_bcast:31 adds lane 31's running
// total to rows 2 and 3.  Lanes whose source lies outside the row keep `old`.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_i(int old, int v) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, ROW_MASK, 0xf, false);
}
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143;

// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += dpp_i<kRowShr1, 0xf>(0, v);
  v += dpp_i<kRowShr2, 0xf>(0, v);
  v += dpp_i<kRowShr4, 0xf>(0, v);
  v += dpp_i<kRowShr8, 0xf>(0, v);
  v += dpp_i<kRowBcast15, 0xa>(0, v);
  v += dpp_i<kRowBcast31, 0xc>(0, v);
  return v;
}
// Minimum / maximum over the 64 lanes, returned to every lane.
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  const int id = (int)0xffffffffu;
  v = min(v, (uint32_t)dpp_i<kRowShr1, 0xf>(id, (int)v));
  v = min(v, (uint32_t)dpp_i<kRowShr2, 0xf>(id, (int)v));
  v = min(v, (uint32_t)dpp_i<kRowShr4, 0xf>(id, (int)v));
  v = min(v, (uint32_t)dpp_i<kRowShr8, 0xf>(id, (int)v));
  v = min(v, (uint32_t)dpp_i<kRowBcast15, 0xa>(id, (int)v));
  v = min(v, (uint32_t)dpp_i<kRowBcast31, 0xc>(id, (int)v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)dpp_i<kRowShr1, 0xf>(0, (int)v));
  v = max(v, (uint32_t)dpp_i<kRowShr2, 0xf>(0, (int)v));
  v = max(v, (uint32_t)dpp_i<kRowShr4, 0xf>(0, (int)v));
  v = max(v, (uint32_t)dpp_i<kRowShr8, 0xf>(0, (int)v));
  v = max(v, (uint32_t)dpp_i<kRowBcast15, 0xa>(0, (int)v));
  v = max(v, (uint32_t)dpp_i<kRowBcast31, 0xc>(0, (int)v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Row of a compact active list -> its sequence: largest b with act_off[b] <= m.
__device__ __forceinline__ int seq_of_row(const int32_t* act_off, int B, int m) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (act_off[mid] <= m) lo = mid; else hi = mid - 1;
  }
  return lo;
}

}  // namespace sl
