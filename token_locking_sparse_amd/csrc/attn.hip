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
__device__ __forceinline__ int find_tile(const int32_t* act_off, int B, int slot, int& row0, int& row_end,
                                         int bq = kBQ) {
  int s = slot;
  for (int b = 0; b < B; ++b) {
    const int o0 = act_off[b], o1 = act_off[b + 1];
    const int nt = (o1 - o0 + bq - 1) / bq;
    if (s < nt) { row0 = o0 + s * bq; row_end = o1; return b; }
    s -= nt;
  }
  return -1;
}

// Key exclusion (the no-KV-cache ablation: positions that may not be attended).
// Score register v of a lane holds key 8 (v / 4) + 4 hl + v % 4 of its 32-key
// subtile, so the lane needs four 4-byte words of the flags: word g covers keys
// 8 g + 4 hl .. + 3.  Excluded keys get a score of -inf.
__device__ __forceinline__ uint32_t excl_word(const uint8_t* excl_row, int key0, int sub, int g, int hl) {
  return *(const uint32_t*)(excl_row + key0 + 32 * sub + 8 * g + 4 * hl);
}
__device__ __forceinline__ void mask_scores(f32x16& s, const uint32_t* w) {
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if ((w[g] >> (8 * r)) & 0xffu) s[4 * g + r] = -INFINITY;
}

template <typename T, int Dh, bool EXCL>
__global__ void __launch_bounds__(kAttnThreads)
attn_kernel(const T* __restrict__ q, const T* __restrict__ kc, const T* __restrict__ vc,
            const int32_t* __restrict__ act_off, const uint8_t* __restrict__ key_excl, int B, int N, int H,
            float scale_log2,
            int nsplit, int tiles_per_split, T* __restrict__ out, float* __restrict__ part_o,
            float* __restrict__ part_ml, int M_tot, int kv_hm) {
  using C = AttnCfg<T, Dh>;
  constexpr int E = C::E;
  __shared__ __attribute__((aligned(16))) char smem[C::Smem];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, hl = lane >> 5, l32 = lane & 31;
  // Flat grid of slots * H * nsplit workgroups.  Workgroups are dealt to the 8
  // XCDs round-robin; when H % 8 == 0 every (slot, split) of a head is placed
  // on the same XCD, so that head's K/V is fetched from HBM once per XCD and
  // then served from that XCD's L2.
  const int per_head = gridDim.x / H;   // slots * nsplit
  int h, rest;
  if ((H & 7) == 0) {
    const int bid = blockIdx.x, xcd = bid & 7, k = bid >> 3;
    h = xcd + 8 * (k / per_head);
    rest = k % per_head;
  } else {
    h = blockIdx.x / per_head;
    rest = blockIdx.x % per_head;
  }
  const int split = rest % nsplit, slot = rest / nsplit;
  int row0 = 0, row_end = 0;
  const int b = find_tile(act_off, B, slot, row0, row_end);
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

  // token-major cache [B][N][H][Dh]: a head's key rows are Dh-element slices HD apart;
  // head-major [B][H][N][Dh]: they are contiguous
  const size_t kv0 = kv_hm ? ((size_t)b * H + h) * N * Dh : ((size_t)b * N * H + h) * Dh;
  const char* kbase = (const char*)(kc + kv0);
  const char* vbase = (const char*)(vc + kv0);
  const size_t krow_stride = (size_t)(kv_hm ? Dh : HD) * sizeof(T);
  const uint8_t* excl_row = EXCL ? key_excl + (size_t)b * N : nullptr;

  u32x4 kreg[C::KLoads];
  u32x4 vreg[C::VLoads][2];
  uint32_t mw[2][4];   // exclusion words of the tile being loaded, per 32-key subtile
  auto gload = [&](int tile) {
    const int key0 = tile * kBKV;
    if constexpr (EXCL) {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int g = 0; g < 4; ++g) mw[sub][g] = excl_word(excl_row, key0, sub, g, hl);
    }
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
    uint32_t mcur[2][4];
    if constexpr (EXCL) {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int g = 0; g < 4; ++g) mcur[sub][g] = mw[sub][g];
    }
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
        if constexpr (EXCL) mask_scores(s[sub], mcur[sub]);
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
      // every key so far excluded: the scores are all -inf and P is 0
      const float m_ref = m_new > -INFINITY ? m_new : 0.f;
      float ls = 0.f;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float pv = __builtin_amdgcn_exp2f(fmaf(s[sub][v], scale_log2, -m_ref));
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

// ------------------------------------------------------------------ bf16, Dh = 128
// Same decomposition (4 waves x 32 queries, 64-key tiles, S^T = K Q^T, online
// softmax per lane, O^T = V^T P^T), but K and V reach LDS by direct
// global->LDS loads in their natural [key][d] layout, double-buffered with one
// barrier per tile, and the V^T operand is read with the LDS transpose read
// (ds_read_b64_tr_b16).  In each 16-lane group that instruction hands lane i,
// element j, the (i % 4)-th 16-bit value read by lane 4 j + i / 4; so when lane
// s of the group reads the 4 values V[kb + s / 4][d0 + 4 (s % 4) ...], lane i
// receives V[kb .. kb + 3][d0 + i]: four consecutive keys of one column, as
// the MFMA A operand wants.  Two such reads give a lane its 8 k-slots; their
// key bases follow the key order of the S^T accumulator (lane half hl holds
// keys 16 m + 4 hl + {0..3} and 16 m + 8 + 4 hl + {0..3} of k-step m), so P^T
// goes from the score registers to the B operand unpermuted.
// LDS layouts (row = one key, 16 chunks of 16 bytes): K chunk c at position
// c ^ (row & 15) (conflict-free 16-byte fragment reads); V chunk c at position
// c ^ 4 (row & 3), which spreads the 16 (row, chunk) pairs one half-wave of a
// transpose read touches over the 16 positions.
constexpr int kTrDh = 128;
constexpr int kTrRB = kTrDh * 2;                 // bytes per key row
constexpr int kTrMergeWave = 64 * (kTrDh / 2) + 2 * 64;   // floats a wave hands over: O^T, m, l

// Shape of one workgroup of the bf16 / Dh = 128 kernel: QW query waves (32
// queries each) x G key groups (group g takes the BKV-key tiles t = g mod G),
// double-buffered per group.
template <int QW, int G, int BKV>
struct TrCfg {
  static constexpr int kThreads = 64 * QW * G;
  static constexpr int kBQ = 32 * QW;
  static constexpr int kTile = BKV * kTrRB;            // one K or V tile
  static constexpr int kStage = 2 * kTile;             // K + V of one group's tile
  static constexpr int kPipe = 2 * G * kStage;
  static constexpr int kMerge = (G - 1) * QW * kTrMergeWave * 4;
  static constexpr int kEpi = QW * 32 * (kTrDh + 4) * 4;
  static constexpr int kSmem = kPipe > kMerge ? (kPipe > kEpi ? kPipe : kEpi) : (kMerge > kEpi ? kMerge : kEpi);
  static constexpr int kDma = kTile / (64 * QW * 16);  // direct loads per thread per K (or V) tile
  static_assert(kThreads == 512 && kDma >= 1 && kTile % (64 * QW * 16) == 0 && BKV % 32 == 0, "shape");
  static_assert(kBKV % BKV == 0, "split plan counts kBKV-key tiles");
  static_assert(kSmem <= 160 * 1024, "LDS");
};

typedef __attribute__((address_space(3))) void attn_lds_t;
typedef __attribute__((address_space(1))) void attn_glb_t;
typedef short attn_v4s __attribute__((ext_vector_type(4)));
typedef attn_v4s __attribute__((address_space(3))) attn_lds_v4s;

__device__ __forceinline__ int vswz(int row, int c) { return c ^ (4 * (row & 3)); }

__device__ __forceinline__ uint2 lds_tr16(const char* p) {
  const attn_v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((attn_lds_v4s*)(attn_lds_t*)p);
  return __builtin_bit_cast(uint2, r);
}

template <int QW, int G, int BKV, bool EXCL>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_tr_kernel(const bf16* __restrict__ q, const bf16* __restrict__ kc, const bf16* __restrict__ vc,
               const int32_t* __restrict__ act_off, const uint8_t* __restrict__ key_excl, int B, int N, int H,
               float scale_log2, int nsplit,
               int tiles_per_split, bf16* __restrict__ out, float* __restrict__ part_o,
               float* __restrict__ part_ml, int M_tot, int kv_hm) {
  using C = TrCfg<QW, G, BKV>;
  constexpr int Dh = kTrDh, E = 8, nKK = Dh / 16;
  __shared__ __attribute__((aligned(1024))) char smem[C::kSmem];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, hl = lane >> 5, l32 = lane & 31;
  const int grp = wid / QW, wq = wid % QW;   // key group; query block of the wave
  const int per_head = gridDim.x / H;
  int h, rest;
  if ((H & 7) == 0) {   // all workgroups of a head on one XCD (see attn_kernel)
    const int bid = blockIdx.x, xcd = bid & 7, k = bid >> 3;
    h = xcd + 8 * (k / per_head);
    rest = k % per_head;
  } else {
    h = blockIdx.x / per_head;
    rest = blockIdx.x % per_head;
  }
  const int split = rest % nsplit, slot = rest / nsplit;
  int row0 = 0, row_end = 0;
  const int b = find_tile(act_off, B, slot, row0, row_end, C::kBQ);
  if (b < 0) return;   // uniform over the workgroup
  // the split plan counts kBKV-key tiles; this kernel walks BKV-key tiles
  constexpr int TR = kBKV / BKV;
  const int t_begin = split * tiles_per_split * TR;
  const int t_end = min(N / kBKV, (split + 1) * tiles_per_split) * TR;
  const int HD = H * Dh;

  const int wrow0 = row0 + wq * 32;
  const bool wave_live = wrow0 < row_end;
  const int my_row = min(wrow0 + l32, row_end - 1);
  u32x4 qf[nKK];
  {
    const char* qr = (const char*)(q + (size_t)my_row * HD + (size_t)h * Dh);
#pragma unroll
    for (int kk = 0; kk < nKK; ++kk) qf[kk] = ld16(qr + (2 * kk + hl) * 16);
  }

  // direct-load sources: load j of wave wq of a group fills LDS bytes [(QW j + wq) KB, +1 KB)
  // of its tile = key rows 4 (QW j + wq) + lane / 16, stored position lane % 16
  // key row stride and the head's first row: token-major [B][N][H][Dh] or head-major [B][H][N][Dh]
  const size_t krow = (size_t)(kv_hm ? Dh : HD) * 2;
  const size_t kv0 = kv_hm ? ((size_t)b * H + h) * N * Dh : ((size_t)b * N * H + h) * Dh;
  const char* kb0 = (const char*)(kc + kv0);
  const char* vb0 = (const char*)(vc + kv0);
  uint32_t koff[C::kDma], voff[C::kDma];
#pragma unroll
  for (int j = 0; j < C::kDma; ++j) {
    const int r = 4 * (QW * j + wq) + (lane >> 4), pos = lane & 15;
    koff[j] = (uint32_t)(r * krow) + swz<kTrRB>(r, pos) * 16;
    voff[j] = (uint32_t)(r * krow) + vswz(r, pos) * 16;
  }
  auto stage_base = [&](int stage) { return smem + (stage * G + grp) * C::kStage; };
  constexpr int NS = BKV / 32;   // 32-key subtiles of a tile
  const uint8_t* excl_row = EXCL ? key_excl + (size_t)b * N : nullptr;
  uint32_t mw[NS][4];            // exclusion words of the tile issued last, per subtile
  auto issue = [&](int tile, int stage) {
    if constexpr (EXCL) {
#pragma unroll
      for (int sub = 0; sub < NS; ++sub)
#pragma unroll
        for (int g = 0; g < 4; ++g) mw[sub][g] = excl_word(excl_row, tile * BKV, sub, g, hl);
    }
    char* ks = stage_base(stage);
    char* vs = ks + C::kTile;
    const size_t t0 = (size_t)tile * BKV * krow;
#pragma unroll
    for (int j = 0; j < C::kDma; ++j)
      __builtin_amdgcn_global_load_lds((attn_glb_t*)(kb0 + t0 + koff[j]), (attn_lds_t*)(ks + (QW * j + wq) * 1024), 16, 0, 0);
#pragma unroll
    for (int j = 0; j < C::kDma; ++j)
      __builtin_amdgcn_global_load_lds((attn_glb_t*)(vb0 + t0 + voff[j]), (attn_lds_t*)(vs + (QW * j + wq) * 1024), 16, 0, 0);
  };

  // transpose-read offsets inside a V tile: this lane of its 16-lane group reads
  // key row kb + s / 4 at column d0 + 4 (s % 4)
  const int g16 = lane >> 4, s16 = lane & 15;
  const int tr_dhalf = 16 * (g16 & 1);            // d0 within the 32-wide d-tile
  const int tr_khalf = 4 * (g16 >> 1);            // 4 hl
  // Per-lane byte offsets of every LDS read of a tile, fixed across tiles: the swizzles depend on the
  // key row only through row % 16 (K) and row % 4 (V), which the lane fixes, so what remains per read
  // (32-key subtile, 16-key k-step, second half of the transpose pair) is a constant immediate.
  // K fragment kk: row l32 (+ 32 sub), chunk (2 kk + hl) ^ (l32 % 16).
  uint32_t kofs[nKK];
#pragma unroll
  for (int kk = 0; kk < nKK; ++kk) kofs[kk] = l32 * kTrRB + swz<kTrRB>(l32, 2 * kk + hl) * 16;
  // V^T d-tile dt: row tr_khalf + s16 / 4 (+ 16 m, + 8 for the second read), column
  // 32 dt + tr_dhalf + 4 (s16 % 4), chunk placed by vswz of that row.
  uint32_t vofs[Dh / 32];
#pragma unroll
  for (int dt = 0; dt < Dh / 32; ++dt) {
    const int kr = tr_khalf + (s16 >> 2), d = 32 * dt + tr_dhalf + 4 * (s16 & 3);
    vofs[dt] = kr * kTrRB + vswz(kr, d >> 3) * 16 + (d & 7) * 2;
  }
  f32x16 oacc[Dh / 32];
#pragma unroll
  for (int i = 0; i < Dh / 32; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[i][v] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // iteration it: group g takes tile t_begin + 2 it + g (if inside the range)
  const int n_it = (t_end - t_begin + G - 1) / G;
  auto own_tile = [&](int it) { return t_begin + it * G + grp; };
  if (n_it > 0 && own_tile(0) < t_end) issue(own_tile(0), 0);
  for (int it = 0; it < n_it; ++it) {
    const int stage = it & 1;
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));   // vmcnt(0): this thread's loads of the tile landed
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();                  // everyone's landed; the other stage is free again
    asm volatile("" ::: "memory");
    uint32_t mcur[NS][4];
    if constexpr (EXCL) {
#pragma unroll
      for (int sub = 0; sub < NS; ++sub)
#pragma unroll
        for (int g = 0; g < 4; ++g) mcur[sub][g] = mw[sub][g];
    }
    if (it + 1 < n_it && own_tile(it + 1) < t_end) issue(own_tile(it + 1), stage ^ 1);
    if (!wave_live || own_tile(it) >= t_end) continue;
    const char* ks = stage_base(stage);
    const char* vs = ks + C::kTile;
    f32x16 sc[NS];
#pragma unroll
    for (int sub = 0; sub < NS; ++sub) {
#pragma unroll
      for (int v = 0; v < 16; ++v) sc[sub][v] = 0.f;
#pragma unroll
      for (int kk = 0; kk < nKK; ++kk) {
        const u32x4 a = *(const u32x4*)(ks + kofs[kk] + sub * 32 * kTrRB);
        Mfma<bf16>::run(sc[sub], a, qf[kk]);
      }
      if constexpr (EXCL) mask_scores(sc[sub], mcur[sub]);
    }
    // Online softmax with a lazily moved reference: the row's reference m_run
    // only moves when the tile max exceeds it by more than kLazy (log2 units),
    // so P <= 2^kLazy and the accumulators are rescaled only on those tiles.
    constexpr float kLazy = 8.f;
    float mx = -INFINITY;
#pragma unroll
    for (int sub = 0; sub < NS; ++sub)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sc[sub][v]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * scale_log2;
    const bool move = mx > m_run + kLazy;          // also true on the first tile
    const float m_new = move ? mx : m_run;
    const float alpha = (move && m_run > -INFINITY) ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
    if (__ballot(move && m_run > -INFINITY)) {     // wave-uniform: rare after the first tiles
#pragma unroll
      for (int i = 0; i < Dh / 32; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[i][v] *= alpha;
    }
    m_run = m_new;
    // every key so far excluded: the scores are all -inf and P is 0
    const float m_ref = m_new > -INFINITY ? m_new : 0.f;
    float ls = 0.f;
#pragma unroll
    for (int sub = 0; sub < NS; ++sub)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float pv = __builtin_amdgcn_exp2f(fmaf(sc[sub][v], scale_log2, -m_ref));
        sc[sub][v] = pv;
        ls += pv;
      }
    l_run = l_run * alpha + ls;
    // O^T += V^T P^T, k-step m covers keys 16 m .. 16 m + 15 of the tile
#pragma unroll
    for (int m = 0; m < BKV / 16; ++m) {
      const int sub = m >> 1, r0 = (m & 1) * 8;
      u32x4 pb;
#pragma unroll
      for (int i = 0; i < 4; ++i) pb[i] = pack_bf16x2(sc[sub][r0 + 2 * i], sc[sub][r0 + 2 * i + 1]);
#pragma unroll
      for (int dt = 0; dt < Dh / 32; ++dt) {
        const uint2 x0 = lds_tr16(vs + vofs[dt] + 16 * m * kTrRB);
        const uint2 x1 = lds_tr16(vs + vofs[dt] + (16 * m + 8) * kTrRB);
        u32x4 a;
        a[0] = x0.x; a[1] = x0.y; a[2] = x1.x; a[3] = x1.y;
        Mfma<bf16>::run(oacc[dt], a, pb);
      }
    }
  }
  __syncthreads();   // stages free

  // groups 1 .. G-1 hand their partials (O^T registers in runs of four, m, l) to the group-0
  // wave of the same queries, which merges the online softmaxes
  if (grp > 0) {
    float* mg = (float*)smem + ((grp - 1) * QW + wq) * kTrMergeWave;
#pragma unroll
    for (int dt = 0; dt < Dh / 32; ++dt)
#pragma unroll
      for (int vb = 0; vb < 4; ++vb)
        *(f32x4*)(mg + ((dt * 4 + vb) * 64 + lane) * 4) =
            f32x4{oacc[dt][4 * vb], oacc[dt][4 * vb + 1], oacc[dt][4 * vb + 2], oacc[dt][4 * vb + 3]};
    mg[64 * (Dh / 2) + lane] = m_run;
    mg[64 * (Dh / 2) + 64 + lane] = l_run;
  }
  __syncthreads();
  if (grp == 0) {
    for (int g2 = 1; g2 < G; ++g2) {
      const float* mg = (const float*)smem + ((g2 - 1) * QW + wq) * kTrMergeWave;
      const float m_o = mg[64 * (Dh / 2) + lane], l_o = mg[64 * (Dh / 2) + 64 + lane];
      const float m_new = fmaxf(m_run, m_o);
      const float a0 = m_run > -INFINITY ? __builtin_amdgcn_exp2f(m_run - m_new) : 0.f;
      const float a1 = m_o > -INFINITY ? __builtin_amdgcn_exp2f(m_o - m_new) : 0.f;
#pragma unroll
      for (int dt = 0; dt < Dh / 32; ++dt)
#pragma unroll
        for (int vb = 0; vb < 4; ++vb) {
          const f32x4 o = *(const f32x4*)(mg + ((dt * 4 + vb) * 64 + lane) * 4);
#pragma unroll
          for (int r = 0; r < 4; ++r) oacc[dt][4 * vb + r] = oacc[dt][4 * vb + r] * a0 + o[r] * a1;
        }
      l_run = l_run * a0 + l_o * a1;
      m_run = m_new;
    }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const int nrow = min(32, row_end - wrow0);
  if (nsplit == 1) {
    // the normalised bf16 output, staged through LDS as a row-major fp32 tile so that every store
    // writes 16 consecutive bytes of a row (measured faster than 8-byte stores from the registers).
    // Rows of Dh + 4 floats: a lane's run of four columns is one 16-byte write, and the 16 lanes a
    // 16-byte access serves at a time (rows l32 .. l32 + 15) start on 16 distinct 4-bank groups.
    constexpr int LDE = Dh + 4;
    __syncthreads();   // merge area free for the output staging
    const float inv = l_tot > 0.f ? 1.f / l_tot : 1.f;
    float* ep = (float*)smem + wq * 32 * LDE;
    if (grp == 0) {
#pragma unroll
      for (int dt = 0; dt < Dh / 32; ++dt)
#pragma unroll
        for (int vb = 0; vb < 4; ++vb)
          *(f32x4*)(ep + l32 * LDE + dt * 32 + vb * 8 + 4 * hl) =
              f32x4{oacc[dt][4 * vb] * inv, oacc[dt][4 * vb + 1] * inv, oacc[dt][4 * vb + 2] * inv,
                    oacc[dt][4 * vb + 3] * inv};
    }
    __syncthreads();
    if (grp == 0 && wave_live) {
      constexpr int CPR = Dh / E;
      for (int id = lane; id < 32 * CPR; id += 64) {
        const int rr = id / CPR, c = id % CPR;
        if (rr < nrow) {
          const float* src = ep + rr * LDE + c * E;
          const f32x4 y0 = *(const f32x4*)src, y1 = *(const f32x4*)(src + 4);
          u32x4 w;
          w[0] = pack_bf16x2(y0[0], y0[1]);
          w[1] = pack_bf16x2(y0[2], y0[3]);
          w[2] = pack_bf16x2(y1[0], y1[1]);
          w[3] = pack_bf16x2(y1[2], y1[3]);
          st16((char*)(out + (size_t)(wrow0 + rr) * HD + (size_t)h * Dh) + c * 16, w);
        }
      }
    }
  } else if (grp == 0 && wave_live && l32 < nrow) {
    // this split's fp32 partial straight from the registers: lane (l32, hl) holds, for d-tile dt
    // and register run vb, O^T[d0 .. d0 + 3][query l32] with d0 = 32 dt + 8 vb + 4 hl
    float* prow = part_o + (((size_t)split * M_tot + wrow0 + l32) * H + h) * Dh;
#pragma unroll
    for (int dt = 0; dt < Dh / 32; ++dt)
#pragma unroll
      for (int vb = 0; vb < 4; ++vb)
        *(f32x4*)(prow + 32 * dt + 8 * vb + 4 * hl) =
            f32x4{oacc[dt][4 * vb], oacc[dt][4 * vb + 1], oacc[dt][4 * vb + 2], oacc[dt][4 * vb + 3]};
    if (hl == 0) {
      float* ml = part_ml + (((size_t)split * M_tot + wrow0 + l32) * H + h) * 2;
      ml[0] = m_run;
      ml[1] = l_tot;
    }
  }
}

// Merge the split-KV partial softmaxes: one wave per (row, head).  Splits are
// taken eight at a time, every load of a batch issued before any is used (one
// memory round trip per batch instead of one per split), with a running max
// across batches.
constexpr int kCombineBatch = 8;

template <typename T, int Dh>
__global__ void __launch_bounds__(256)
attn_combine_kernel(const float* __restrict__ part_o, const float* __restrict__ part_ml, int nsplit,
                    int M_tot, int H, T* __restrict__ out, const int32_t* __restrict__ m_dev) {
  constexpr int PER = (Dh + 63) / 64;   // output elements per lane
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (w >= rows_live(M_tot, m_dev) * H) return;   // M_tot: capacity and stride of the partials
  const int m = w / H, h = w % H;
  const size_t stride_ml = (size_t)M_tot * H * 2, stride_o = (size_t)M_tot * H * Dh;
  const float* ml0 = part_ml + ((size_t)m * H + h) * 2;
  const float* po0 = part_o + ((size_t)m * H + h) * Dh;
  float mx = -INFINITY, L = 0.f;
  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  for (int s0 = 0; s0 < nsplit; s0 += kCombineBatch) {
    float ms[kCombineBatch], ls[kCombineBatch], os[kCombineBatch][PER];
#pragma unroll
    for (int k = 0; k < kCombineBatch; ++k) {
      const int sidx = min(s0 + k, nsplit - 1);   // clamped: loads stay in bounds
      ms[k] = ml0[sidx * stride_ml];
      ls[k] = ml0[sidx * stride_ml + 1];
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int d = lane + 64 * i;
        os[k][i] = d < Dh ? po0[sidx * stride_o + d] : 0.f;
      }
    }
    float bm = mx;
#pragma unroll
    for (int k = 0; k < kCombineBatch; ++k)
      if (s0 + k < nsplit) bm = fmaxf(bm, ms[k]);
    const float rescale = (mx > -INFINITY) ? __builtin_amdgcn_exp2f(mx - bm) : 0.f;
    L *= rescale;
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] *= rescale;
#pragma unroll
    for (int k = 0; k < kCombineBatch; ++k) {
      const float wgt = (s0 + k < nsplit && ms[k] > -INFINITY) ? __builtin_amdgcn_exp2f(ms[k] - bm) : 0.f;
      L += ls[k] * wgt;
#pragma unroll
      for (int i = 0; i < PER; ++i) acc[i] += os[k][i] * wgt;
    }
    mx = bm;
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int d = lane + 64 * i;
    if (d < Dh) out[(size_t)m * H * Dh + (size_t)h * Dh + d] = from_f32<T>(acc[i] * inv);
  }
}

// Launch plan.  bq = queries per workgroup; shape 1 (bf16, head dim 128 only)
// = 64-query workgroups with four key groups, for when 128-query workgroups
// would leave the chip half idle and 64-query ones need no key split.  Splitting the keys over workgroups costs a
// second pass over fp32 partials (several us), so it is used only when the
// query tiles alone leave most of the chip idle.  Then each key group's run of
// keys is the latency chain: the transposed-score kernels split only down to
// 128 keys per key group, and for N <= 512 take shape 1 (four key groups of at
// most 128 keys) with no split and no merge pass.  Measured at 32 heads and
// M <= 64: N = 512, 13.4-14.3 us against 16.6-17.9 us split four ways;
// N = 1024, 15.2-17.1 us split four ways against 16.2-18.6 us split eight ways.
// Shape 1 only when its workgroups fit in one wave of the chip: at 32 heads and
// M = 768 its 384 workgroups take 37-39 us against 25-26 us for shape 0's 192.
struct AttnPlan { int bq, shape, slots, nsplit, tps; };

static AttnPlan attn_plan(int B, int N, int M_tot, int H, bool tr) {
  AttnPlan p{};
  const int tiles = N / kBKV;
  p.bq = kBQ;
  p.shape = 0;
  const int b64 = ((M_tot + 63) / 64) * H;   // 64-query workgroups
  if (tr && ((M_tot + kBQ - 1) / kBQ) * H < 256 && b64 >= 64 && b64 <= 256) { p.bq = 64; p.shape = 1; }
  const int blocks = ((M_tot + p.bq - 1) / p.bq) * H;   // useful workgroups without a split
  p.nsplit = 1;
  if (blocks < 64) {
    if (tr && N <= 4 * 128) {
      p.bq = 64;
      p.shape = 1;
    } else {
      const int G = tr ? 2 : 1;   // key groups of shape 0
      while (blocks * p.nsplit < 256 && p.nsplit * 2 <= tiles / 2 && (!tr || N / (2 * p.nsplit * G) >= 128))
        p.nsplit *= 2;
    }
  }
  p.tps = (tiles + p.nsplit - 1) / p.nsplit;
  p.slots = (M_tot + p.bq - 1) / p.bq + B;
  return p;
}

size_t attn_ws_bytes(int B, int N, int M_tot, int H, int Dh) {
  const AttnPlan p0 = attn_plan(B, N, M_tot, H, false), p1 = attn_plan(B, N, M_tot, H, Dh == kTrDh);
  const int nsplit = p0.nsplit > p1.nsplit ? p0.nsplit : p1.nsplit;
  if (nsplit == 1) return 256;
  return (size_t)nsplit * M_tot * H * (Dh + 2) * 4 + 256;
}

template <typename T, int Dh, bool EXCL>
static hipError_t attn_launch_t(const void* q, const void* kc, const void* vc, const int32_t* act_off,
                                const uint8_t* key_excl, int B, int N, int M_tot, int H, float scale, void* out,
                                void* ws, hipStream_t s, const int32_t* m_dev, int kv_hm) {
  const bool tr = sizeof(T) == 2 && Dh == kTrDh;
  const AttnPlan p = attn_plan(B, N, M_tot, H, tr);
  const int nsplit = p.nsplit, tps = p.tps;
  float* part_o = (float*)ws;
  float* part_ml = part_o + (size_t)nsplit * M_tot * H * Dh;
  const float sl2 = scale * kLog2e;
  const dim3 grid(p.slots * H * nsplit);
  if (tr && p.shape == 0)
    hipLaunchKernelGGL((attn_tr_kernel<4, 2, 64, EXCL>), grid, dim3(512), 0, s, (const bf16*)q, (const bf16*)kc,
                       (const bf16*)vc, act_off, key_excl, B, N, H, sl2, nsplit, tps, (bf16*)out, part_o, part_ml,
                       M_tot, kv_hm);
  else if (tr)
    hipLaunchKernelGGL((attn_tr_kernel<2, 4, 32, EXCL>), grid, dim3(512), 0, s, (const bf16*)q, (const bf16*)kc,
                       (const bf16*)vc, act_off, key_excl, B, N, H, sl2, nsplit, tps, (bf16*)out, part_o, part_ml,
                       M_tot, kv_hm);
  else
    hipLaunchKernelGGL((attn_kernel<T, Dh, EXCL>), grid, dim3(kAttnThreads), 0, s, (const T*)q, (const T*)kc,
                       (const T*)vc, act_off, key_excl, B, N, H, sl2, nsplit, tps, (T*)out, part_o, part_ml, M_tot, kv_hm);
  if (nsplit > 1) {
    const int waves = M_tot * H;
    hipLaunchKernelGGL((attn_combine_kernel<T, Dh>), dim3((waves + 3) / 4), dim3(256), 0, s, part_o,
                       part_ml, nsplit, M_tot, H, (T*)out, m_dev);
  }
  return hipGetLastError();
}

template <typename T, int Dh>
static hipError_t attn_launch_excl(const void* q, const void* kc, const void* vc, const int32_t* act_off,
                                   const uint8_t* key_excl, int B, int N, int M_tot, int H, float scale, void* out,
                                   void* ws, hipStream_t s, const int32_t* m_dev, int kv_hm) {
  return key_excl ? attn_launch_t<T, Dh, true>(q, kc, vc, act_off, key_excl, B, N, M_tot, H, scale, out, ws, s, m_dev,
                                               kv_hm)
                  : attn_launch_t<T, Dh, false>(q, kc, vc, act_off, nullptr, B, N, M_tot, H, scale, out, ws, s,
                                                m_dev, kv_hm);
}

hipError_t launch_attn(int dtype, const void* q, const void* kc, const void* vc,
                       const int32_t* act_off, const uint8_t* key_excl, int B, int N, int M_tot, int H, int Dh,
                       float scale, void* out, void* ws, hipStream_t s, const int32_t* m_dev, int kv_hm) {
  if (M_tot <= 0) return hipSuccess;
  if (dtype == 0) {
    if (Dh == 128) return attn_launch_excl<bf16, 128>(q, kc, vc, act_off, key_excl, B, N, M_tot, H, scale, out, ws, s, m_dev, kv_hm);
    if (Dh == 64) return attn_launch_excl<bf16, 64>(q, kc, vc, act_off, key_excl, B, N, M_tot, H, scale, out, ws, s, m_dev, kv_hm);
    if (Dh == 32) return attn_launch_excl<bf16, 32>(q, kc, vc, act_off, key_excl, B, N, M_tot, H, scale, out, ws, s, m_dev, kv_hm);
  } else {
    if (Dh == 128) return attn_launch_excl<float, 128>(q, kc, vc, act_off, key_excl, B, N, M_tot, H, scale, out, ws, s, m_dev, kv_hm);
    if (Dh == 64) return attn_launch_excl<float, 64>(q, kc, vc, act_off, key_excl, B, N, M_tot, H, scale, out, ws, s, m_dev, kv_hm);
    if (Dh == 32) return attn_launch_excl<float, 32>(q, kc, vc, act_off, key_excl, B, N, M_tot, H, scale, out, ws, s, m_dev, kv_hm);
  }
  return hipErrorInvalidValue;
}

}  // namespace sl
