// Device-side helpers shared by the Muir HIP kernels (gfx950 only).
//
// MFMA lane layouts used throughout (wave64; checked on hardware):
//   v_mfma_f32_16x16x16_bf16  A: lane l holds row (l%16), k = 4*(l/16)+i, i<4
//                             B: lane l holds col (l%16), k = 4*(l/16)+i, i<4
//                             D: lane l holds row 4*(l/16)+i, col (l%16), i<4
//   v_mfma_f32_16x16x4_f32    A: lane l holds row (l%16), k = l/16
//                             B: lane l holds col (l%16), k = l/16
//                             D: as above.
// The accumulator layout of a 16x16 tile (4 consecutive rows per lane) is the
// operand layout of a 16x16x16 product whose contraction runs over those rows,
// which lets results feed the next product without a shuffle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace muir {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// ---- bf16 storage helpers (raw 16-bit patterns) ------------------------------

__device__ __forceinline__ float bf16_to_f32(uint16_t x) {
  return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

// Round-to-nearest-even fp32 -> bf16 (gfx950 converts in hardware,
// v_cvt_pk_bf16_f32, two values per instruction).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Element loads from an input tensor of either dtype.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p, size_t i) { return p[i]; }
  static __device__ __forceinline__ void store(float* p, size_t i, float v) { p[i] = v; }
};
template <> struct Elem<uint16_t> {
  static __device__ __forceinline__ float load(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
  static __device__ __forceinline__ void store(uint16_t* p, size_t i, float v) { p[i] = f32_to_bf16(v); }
};

// Element access through a workgroup-uniform base pointer and a 32-bit element
// index: the address is formed as scalar base + 32-bit vector offset, so no
// per-lane 64-bit address arithmetic is needed.  The caller keeps
// index * sizeof(T) below 2^32.
template <typename T> __device__ __forceinline__ const T* at(const T* base, uint32_t i) {
  return reinterpret_cast<const T*>(reinterpret_cast<const char*>(base) + i * static_cast<uint32_t>(sizeof(T)));
}
template <typename T> __device__ __forceinline__ T* at(T* base, uint32_t i) {
  return reinterpret_cast<T*>(reinterpret_cast<char*>(base) + i * static_cast<uint32_t>(sizeof(T)));
}
template <typename T> __device__ __forceinline__ float ldv(const T* base, uint32_t i) {
  return Elem<T>::load(at(base, i), 0);
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Four consecutive elements of a compute type as one raw word (8 or 16 bytes).
template <typename TC> struct Raw4;
template <> struct Raw4<uint16_t> { typedef uint2 type; };
template <> struct Raw4<float> { typedef uint4 type; };

// Converted in pairs: a whole-vector conversion compiles to one conversion per
// value plus byte permutes to merge them, a pairwise one to one per two values.
__device__ __forceinline__ i16x4 pack4(f32x4 v) {
  u32x2 r = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  return __builtin_bit_cast(i16x4, r);
}

// Load 4 consecutive elements (16-byte aligned for fp32, 8-byte for bf16).
__device__ __forceinline__ f32x4 load4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ f32x4 load4(const uint16_t* p) {
  uint2 r = *reinterpret_cast<const uint2*>(p);
  f32x4 o;
  o[0] = __uint_as_float(r.x << 16);
  o[1] = __uint_as_float(r.x & 0xffff0000u);
  o[2] = __uint_as_float(r.y << 16);
  o[3] = __uint_as_float(r.y & 0xffff0000u);
  return o;
}
__device__ __forceinline__ void store4(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }
__device__ __forceinline__ void store4(uint16_t* p, f32x4 v) {
  *reinterpret_cast<i16x4*>(p) = pack4(v);
}

// ---- MFMA wrappers -----------------------------------------------------------

// acc += A(16x16 bf16) * B(16x16 bf16); operands packed as 4 bf16 per lane.
__device__ __forceinline__ f32x4 mma16_bf16(i16x4 a, i16x4 b, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, acc, 0, 0, 0);
}

// acc += A1 B1 + A2 B2 for two 16-deep bf16 products as ONE 32-deep product
// (v_mfma_f32_16x16x32_bf16, whose lane l holds contraction slots
// 8*(l/16) + i, i < 8): both operands take the first pair's four values in
// slots 0-3 and the second pair's in slots 4-7, so the slots match up and the
// sum is the same.  On gfx950 the 32-deep product issues in the same time as
// one 16-deep product.
__device__ __forceinline__ f32x4 mma32_bf16(i16x4 a1, i16x4 b1, i16x4 a2, i16x4 b2, f32x4 acc) {
  const i16x8 a = __builtin_shufflevector(a1, a2, 0, 1, 2, 3, 4, 5, 6, 7);
  const i16x8 b = __builtin_shufflevector(b1, b2, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                 acc, 0, 0, 0);
}

// acc += A(16x4 f32) * B(4x16 f32); one value per lane.
__device__ __forceinline__ f32x4 mma4_f32(float a, float b, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
}

__device__ __forceinline__ i16x4 load_bf16x4(const uint16_t* p) {
  return *reinterpret_cast<const i16x4*>(p);
}

__device__ __forceinline__ f32x4 zero4() {
  f32x4 z = {0.f, 0.f, 0.f, 0.f};
  return z;
}

// Sum over each row of 16 lanes (the result in all 16), with DPP moves:
// quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror.
template <int CTRL> __device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float sum16(float v) {
  v += dpp_mov<0xB1>(v);
  v += dpp_mov<0x4E>(v);
  v += dpp_mov<0x141>(v);
  v += dpp_mov<0x140>(v);
  return v;
}

// Reductions over the 64 lanes of a wave.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

}  // namespace muir
