// Per-chunk helpers shared by the chunk-parallel kernels (forward summary and
// backward gradients): block boundaries of the cumulative log-decay and the
// Neumann inverse of a 16 x 16 leaf.
#pragma once

#include "mma.h"

namespace muir {

// Largest per-channel log-decay over one 16-token leaf for which the leaf's
// pair factors exp(Lam_r - Lam_i) are formed as exp(Lam_r - B) * exp(B - Lam_i)
// (B: the leaf's start boundary).  Both factors and every product of them
// then stay within [e^-80, e^80], inside the fp32 and bf16 exponent range;
// above it the leaf uses the per-pair factors directly.
constexpr float LEAF_SAFE_RANGE = 80.f;

// Leaf inverse on one wave: T = (I + A)^-1 = (I - A)(I + A^2)(I + A^4)(I + A^8)
// for a strictly lower 16 x 16 A (A^16 = 0), fp32 MFMA throughout, in
// registers.  A arrives in both lane layouts: a_acc[i] = A[4g+i][c] (the
// accumulator layout, g = lane/16, c = lane%16) and a_tr[i] = A[c][4g+i].
// Every factor is a polynomial in A, so they all commute: each power P is
// carried in both layouts, P^2 = P P in the accumulator layout and
// (P^2)^T = P^T P^T in the other come from the same two operands swapped,
// and T <- T + P^2 T takes P^2 as the left operand.  Returns T in the
// accumulator layout.
__device__ __forceinline__ f32x4 neumann16(f32x4 a_acc, f32x4 a_tr) {
  typedef MM<float> MF;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int c = lane & 15;
  f32x4 t;
#pragma unroll
  for (int i = 0; i < 4; ++i) t[i] = (4 * g + i == c ? 1.f : 0.f) - a_acc[i];
  f32x4 pa = a_acc, pt = a_tr;
#pragma unroll
  for (int step = 0; step < 3; ++step) {
    const f32x4 qt = MF::mma(pa, pt, zero4());                     // A^(2^(step+1)), other layout
    const f32x4 qa = step < 2 ? MF::mma(pt, pa, zero4()) : zero4(); // the same, accumulator layout
    t = MF::mma(qt, t, t);                                         // T (I + A^(2^(step+1)))
    pa = qa;
    pt = qt;
  }
  return t;
}

}  // namespace muir
