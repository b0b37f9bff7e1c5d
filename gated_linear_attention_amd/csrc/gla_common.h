// Device-side helpers shared by the GLA kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gla {

constexpr float kLog2e = 1.4426950408889634f;

// A log-gate at or below -128 ln 2 (a multiplier g <= 2^-128, under the
// smallest normal fp32) is taken as g = 0 exactly: the gate resets the state
// (the previous state is multiplied by zero). -inf is the canonical reset.
// Exponentials of sums that contain such a gate are never formed: the scans
// treat it as 0 and cut every decay product that spans it.
constexpr float kResetLn = -88.72283906f;
__device__ __forceinline__ bool is_reset(float l) { return l <= kResetLn; }
// exp(l), with every reset gate exactly 0.
__device__ __forceinline__ float gate_exp(float l) { return is_reset(l) ? 0.f : expf(l); }

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

// bf16 is stored as the upper 16 bits of a binary32; widening is a shift.
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Round-to-nearest-even narrowing of a finite or infinite float to bf16 bits;
// NaN maps to a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two bf16 (lo element first) packed in one 32-bit word.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return f32_to_bf16_bits(a) | (f32_to_bf16_bits(b) << 16);
}

// Split x into hi + lo with hi = bf16(x) and lo = bf16(x - hi): the pair holds
// about 16 significant bits, so products hi*y + lo*y on the bf16 matrix cores
// keep fp32-level accuracy (x - hi is exact in fp32).
__device__ __forceinline__ void split_bf16(float x, uint32_t &hi, uint32_t &lo) {
  hi = f32_to_bf16_bits(x);
  lo = f32_to_bf16_bits(x - bf16_bits_to_f32(hi));
}

// Two floats to packed bf16 (round to nearest even) with one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// hi/lo split of two floats at once: returns packed bf16 pairs hi = bf16(x),
// lo = bf16(x - hi) (element 0 in the low half).
__device__ __forceinline__ void split_pk_bf16(float a, float b, uint32_t &hi, uint32_t &lo) {
  hi = cvt_pk_bf16(a, b);
  const float ha = __uint_as_float(hi << 16), hb = __uint_as_float(hi & 0xffff0000u);
  lo = cvt_pk_bf16(a - ha, b - hb);
}

// 2^x on the hardware exp unit (v_exp_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Load element i of a bf16 or fp32 array as float.
template <typename T> __device__ __forceinline__ float load_as_f32(const T *p, size_t i);
template <> __device__ __forceinline__ float load_as_f32<float>(const float *p, size_t i) {
  return p[i];
}
template <> __device__ __forceinline__ float load_as_f32<uint16_t>(const uint16_t *p, size_t i) {
  return bf16_bits_to_f32(p[i]);
}

// Load four consecutive elements (16-byte aligned fp32, 8-byte aligned bf16) as floats.
__device__ __forceinline__ f32x4 load4_as_f32(const float *p) {
  return *reinterpret_cast<const f32x4 *>(p);
}
__device__ __forceinline__ f32x4 load4_as_f32(const uint16_t *p) {
  const u32x2 w = *reinterpret_cast<const u32x2 *>(p);
  return f32x4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
               __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u)};
}

// Store a float as fp32 or bf16.
template <typename T> __device__ __forceinline__ void store_from_f32(T *p, size_t i, float x);
template <> __device__ __forceinline__ void store_from_f32<float>(float *p, size_t i, float x) {
  p[i] = x;
}
template <> __device__ __forceinline__ void store_from_f32<uint16_t>(uint16_t *p, size_t i, float x) {
  p[i] = (uint16_t)f32_to_bf16_bits(x);
}

// Store four consecutive floats as fp32 (one 16-byte store) or bf16 (8 bytes).
__device__ __forceinline__ void store4_from_f32(float *p, const f32x4 &x) {
  *reinterpret_cast<f32x4 *>(p) = x;
}
__device__ __forceinline__ void store4_from_f32(uint16_t *p, const f32x4 &x) {
  u32x2 w;
  w.x = cvt_pk_bf16(x[0], x[1]);
  w.y = cvt_pk_bf16(x[2], x[3]);
  *reinterpret_cast<u32x2 *>(p) = w;
}

}  // namespace gla
