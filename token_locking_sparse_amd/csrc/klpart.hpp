// Partial statistics of a slice of one posterior row, shared by the vocabulary
// pass and the LM-head epilogue that computes them in place: online
// (rescaled) sums of the current and previous logits, from which LSE, the step
// KL(p_t || p_{t-1}), 1 - max p and the argmax follow (zhaoyang97 notes on
// SureLock, 锁定判据 and 可选置信度门控).  Slices combine associatively.
#pragma once

#include <math.h>

#include "common.hpp"

namespace sl {

struct Part {
  float ma, sa, ta;  // running max of cur (all ids), sum e^(a-ma), sum e^(a-ma) (a-b)
  float mb, sb;      // running max of prev, sum e^(b-mb); when the previous posterior's LSE is
                     // known from the pass that produced it: mb = that LSE, sb unused (0)
  float best;        // max of cur over ids != mask
  int bidx;          // where `best` is (lowest on ties): its 16-byte chunk while a row is
                     // streamed, its exact id once resolved (and in every stored partial)
};

constexpr int kPartWords = 8;   // words of a stored partial (kKlPartBytes of the launchers)

// The partial of no element (the identity of combine).
__device__ __forceinline__ Part empty_part() {
  Part p;
  p.ma = -INFINITY; p.sa = 0.f; p.ta = 0.f;
  p.mb = -INFINITY; p.sb = 0.f;
  p.best = -INFINITY; p.bidx = 0x7fffffff;
  return p;
}

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

// Segment partials: 8 words per (segment, row), segment-major, so the tail
// reads one segment of consecutive rows with consecutive lanes.  The eighth
// word carries an int beside the partial (the vocabulary pass: the row's
// position b*N + pos).
__device__ __forceinline__ void store_part(float* pp, const Part& t, int word7 = 0) {
  f32x4 x0, x1;
  x0[0] = t.ma; x0[1] = t.sa; x0[2] = t.ta; x0[3] = t.mb;
  x1[0] = t.sb; x1[1] = t.best; x1[2] = __int_as_float(t.bidx); x1[3] = __int_as_float(word7);
  reinterpret_cast<f32x4*>(pp)[0] = x0;
  reinterpret_cast<f32x4*>(pp)[1] = x1;
}
__device__ __forceinline__ Part load_part(const float* pp, int* word7 = nullptr) {
  const f32x4 x0 = reinterpret_cast<const f32x4*>(pp)[0];
  const f32x4 x1 = reinterpret_cast<const f32x4*>(pp)[1];
  Part t;
  t.ma = x0[0]; t.sa = x0[1]; t.ta = x0[2]; t.mb = x0[3];
  t.sb = x1[0]; t.best = x1[1]; t.bidx = __float_as_int(x1[2]);
  if (word7) *word7 = __float_as_int(x1[3]);
  return t;
}

}  // namespace sl
