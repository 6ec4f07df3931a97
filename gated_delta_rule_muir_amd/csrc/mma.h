// 16x16 tile products over a 16-long contraction, in either compute type.
//
// A fragment holds, per lane l, four values along the contraction index
// k = 4*(l/16) + i (i < 4) for row/column (l % 16) -- the same placement as
// the rows of an accumulator tile, so an accumulator converts to an operand
// of the next product without moving data between lanes.
//   bf16: one v_mfma_f32_16x16x16_bf16 (fp32 accumulate); mma2 sums two such
//         products in one v_mfma_f32_16x16x32_bf16
//   fp32: four v_mfma_f32_16x16x4_f32; sub-step i contracts k in {i, 4+i, 8+i, 12+i}
#pragma once

#include "device_common.h"

namespace muir {

template <typename TC> struct MM;

template <> struct MM<uint16_t> {
  typedef i16x4 frag;
  static __device__ __forceinline__ frag from_f32(f32x4 v) { return pack4(v); }
  static __device__ __forceinline__ frag load(const uint16_t* p) { return load_bf16x4(p); }
  static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) { return mma16_bf16(a, b, c); }
  // c + A1 B1 + A2 B2 (two contraction tiles in one 32-deep product)
  static __device__ __forceinline__ f32x4 mma2(frag a1, frag b1, frag a2, frag b2, f32x4 c) {
    return mma32_bf16(a1, b1, a2, b2, c);
  }
  static __device__ __forceinline__ uint16_t cvt(float x) { return f32_to_bf16(x); }
  static __device__ __forceinline__ float to_f32(uint16_t x) { return bf16_to_f32(x); }
};

template <> struct MM<float> {
  typedef f32x4 frag;
  static __device__ __forceinline__ frag from_f32(f32x4 v) { return v; }
  static __device__ __forceinline__ frag load(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
  static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    c = mma4_f32(a[0], b[0], c);
    c = mma4_f32(a[1], b[1], c);
    c = mma4_f32(a[2], b[2], c);
    c = mma4_f32(a[3], b[3], c);
    return c;
  }
  static __device__ __forceinline__ f32x4 mma2(frag a1, frag b1, frag a2, frag b2, f32x4 c) {
    return mma(a2, b2, mma(a1, b1, c));
  }
  static __device__ __forceinline__ float cvt(float x) { return x; }
  static __device__ __forceinline__ float to_f32(float x) { return x; }
};

}  // namespace muir
