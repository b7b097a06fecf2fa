// Device helpers: storage-format conversions used by the kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace mla {

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// float -> bfloat16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two floats -> packed bfloat16 pair (lo in bits 0-15, hi in 16-31), round
// to nearest even: one v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t bf16x2_bits(float lo, float hi) {
  typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f2;
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 b2;
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){lo, hi}, b2));
}

// Splits the pair (x0, x1) into bf16 parts h + l with x = h + l + O(2^-16 x):
// h = bf16(x), l = bf16(x - h); returns the packed pairs.
__device__ __forceinline__ void split_bf16x2(float x0, float x1, uint32_t& h, uint32_t& l) {
  h = bf16x2_bits(x0, x1);
  l = bf16x2_bits(x0 - __uint_as_float(h << 16), x1 - __uint_as_float(h & 0xffff0000u));
}

// OCP e4m3fn byte -> float: 1 sign, 4 exponent bits (bias 7), 3 mantissa
// bits, exponent 0 subnormal, S.1111.111 NaN, no infinities.
__device__ __forceinline__ float e4m3fn_to_f32(uint32_t b) {
  const uint32_t sign = (b & 0x80u) << 24;
  const uint32_t e = (b >> 3) & 0xfu;
  const uint32_t m = b & 0x7u;
  if (e == 0xfu && m == 0x7u) return __uint_as_float(0x7fc00000u);
  if (e == 0) return __uint_as_float(sign | __float_as_uint((float)m * 0x1p-9f));
  return __uint_as_float(sign | ((e + 120u) << 23) | (m << 20));
}

// OCP e8m0 scale byte -> 2^(E - 127); 0xff is NaN.
// OCP e2m1 (fp4): sign, 2 exponent bits (bias 1), 1 mantissa bit; exponent 0
// is subnormal (m / 2).  Magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.
__device__ __forceinline__ float e2m1_to_f32(uint32_t c) {
  const uint32_t e = (c >> 1) & 3u, m = c & 1u;
  const float mag = e == 0 ? 0.5f * (float)m : (1.f + 0.5f * (float)m) * (float)(1u << (e - 1));
  return (c & 8u) ? -mag : mag;
}

__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
  if (e == 0xffu) return __uint_as_float(0x7fc00000u);
  if (e == 0) return 0x1p-127f;
  return __uint_as_float(e << 23);
}

}  // namespace mla
