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
// for a strictly lower 16 x 16 A held in sA ([16][17] fp32).  sP is a work
// tile.  On return the lane's T elements (rows 4*(lane/16)+i, column lane%16)
// are returned and also left in sT.  fp32 MFMA throughout.
__device__ __forceinline__ f32x4 neumann16(float (*sA)[17], float (*sP)[17], float (*sT)[17]) {
  typedef MM<float> MF;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int c = lane & 15;
  f32x4 t, p;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * g + i;
    p[i] = sA[r][c];
    t[i] = (r == c ? 1.f : 0.f) - p[i];
    sP[r][c] = p[i];
    sT[r][c] = t[i];
  }
#pragma unroll 1
  for (int step = 0; step < 3; ++step) {
    f32x4 a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = sP[c][4 * g + i];
      b[i] = sP[4 * g + i][c];
    }
    p = MF::mma(a, b, zero4());  // A^(2^(step+1))
#pragma unroll
    for (int i = 0; i < 4; ++i) sP[4 * g + i][c] = p[i];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = sT[c][4 * g + i];
      b[i] = sP[4 * g + i][c];
    }
    t = MF::mma(a, b, t);  // T (I + A^(2^(step+1)))
#pragma unroll
    for (int i = 0; i < 4; ++i) sT[4 * g + i][c] = t[i];
  }
  return t;
}

}  // namespace muir
