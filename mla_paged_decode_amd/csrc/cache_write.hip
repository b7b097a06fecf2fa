// Cache append: store new tokens' [latent | RoPE key] rows into the paged
// cache in its row format.
//
// One wave per row.  f32 and bf16 rows are converted value by value (bf16:
// round to nearest, ties to even).  The fp8 row (the GLM-4.7-Flash model
// record, ENGINE KERNEL CONSTRAINTS item (2): 512 e4m3 values, RoPE dims
// included, then one e8m0 scale byte per 32 values, 528 B) is quantised per
// block of 32 values: the scale is 2^(E-127) with E the smallest exponent
// for which the block's largest magnitude is at most 448 (the largest e4m3fn
// value), and each value / scale is rounded to the nearest e4m3fn value,
// ties to the even code.  Both steps are exact integer and power-of-two
// operations, so the stored bytes do not depend on rounding order.  Lane l
// owns values 8l..8l+7: four lanes make a block, whose maximum is two
// shuffles away, and the lane's eight codes are one 8-byte store.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "device_common.h"
#include "internal.h"

namespace mla {
namespace {

constexpr int kRowsPerBlock = 4;  // one wave per row

// Smallest E in [0, 254] with amax <= 448 * 2^(E - 127); 127 for amax = 0.
// With amax = 1.m * 2^(ea - 127) and 448 = 1.75 * 2^8 that is ea - 8 when
// 1.m <= 1.75 (mantissa field <= 0x600000), else ea - 7.
__device__ __forceinline__ uint32_t e8m0_exponent(float amax) {
  if (!(amax > 0.f)) return 127u;
  const uint32_t u = __float_as_uint(amax);
  const int ea = (int)(u >> 23);
  if (ea == 0) return 0u;  // below 2^-126: 448 * 2^-127 already covers it
  const int e = ea - 8 + ((u & 0x7fffffu) > 0x600000u ? 1 : 0);
  return (uint32_t)min(max(e, 0), 254);
}

// e4m3fn code of x, |x| <= 448 and finite: nearest value, ties to the even
// code (the code's last bit is the mantissa's); the sign bit is x's.
__device__ __forceinline__ uint32_t e4m3fn_encode(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fabsf(x);
  uint32_t code;
  if (a < 0x1p-6f) {
    // Subnormal range, steps of 2^-9: codes 0..7, and 8 (= 2^-6, the
    // smallest normal) when rounding carries.
    code = (uint32_t)__builtin_rintf(a * 512.f);
  } else {
    const int e = (int)(__float_as_uint(a) >> 23) - 127;  // floor(log2 a), -6..8
    uint32_t m = (uint32_t)__builtin_rintf(ldexpf(a, 3 - e));  // 8..16, steps of 2^(e-3)
    int ee = e;
    if (m == 16u) {
      m = 8u;
      ++ee;
    }
    code = ((uint32_t)(ee + 7) << 3) | (m - 8u);
  }
  return code | sign;
}

// Value of a finite, positive e4m3fn code (exact in float32).
__device__ __forceinline__ float e4m3fn_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 0xfu, m = c & 7u;
  return e == 0 ? ldexpf((float)m, -9) : ldexpf((float)(8u + m), (int)e - 10);
}

// fp4 block scale: the smallest positive e4m3fn value s with amax <= 6 s
// (6 s is exact in float32); 0x7E (448) if none, 0x38 (1.0) for amax = 0.
// The search starts at the e4m3 code nearest to amax / 6 and moves by whole
// codes, so the comparison, not the rounding of amax / 6, decides.
__device__ __forceinline__ uint32_t fp4_scale_code(float amax) {
  if (!(amax > 0.f)) return 0x38u;
  const float t = fminf(amax * (1.f / 6.f), 448.f);
  int c = (int)(e4m3fn_encode(t) & 0x7fu);
  c = max(c, 1);
  while (c > 1 && amax <= 6.f * e4m3fn_value((uint32_t)(c - 1))) --c;
  while (c < 126 && amax > 6.f * e4m3fn_value((uint32_t)c)) ++c;
  return (uint32_t)c;
}

// e2m1 code of x: nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6 (ties to the even
// code, magnitudes past 6 saturate), sign bit from x.
__device__ __forceinline__ uint32_t e2m1_encode(float x) {
  const float a = fabsf(x);
  const uint32_t code = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) + (a >= 3.5f) + (a > 5.f);
  return code | ((__float_as_uint(x) >> 28) & 8u);
}

template <int FMT>
__global__ __launch_bounds__(64 * kRowsPerBlock) void cache_write_kernel(CacheWriteArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (r >= a.n_rows) return;
  const int64_t slot = a.slots[r];
  if (slot < 0 || slot >= a.n_slots) return;  // skipped row
  const int n = a.n_vals;
  uint8_t* dst = a.pool + slot * a.row_bytes;
  const float* rf = static_cast<const float*>(a.rows) + r * n;
  const uint16_t* rb = static_cast<const uint16_t*>(a.rows) + r * n;
  auto value = [&](int i) -> float { return a.rows_f32 ? rf[i] : bf16_bits_to_f32(rb[i]); };

  if constexpr (FMT == kF32) {
    for (int i = lane; i < n; i += 64) reinterpret_cast<float*>(dst)[i] = value(i);
  } else if constexpr (FMT == kBF16) {
    for (int i = lane; i < n; i += 64)
      reinterpret_cast<uint16_t*>(dst)[i] = a.rows_f32 ? (uint16_t)f32_to_bf16_bits(rf[i]) : rb[i];
  } else if constexpr (FMT == kFP4) {
    // n == 512: lane l holds values 8l..8l+7, half of 16-value block l / 2;
    // its eight codes are one 4-byte store, and even lanes store the scale.
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = value(8 * lane + i);
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    const uint32_t sc = fp4_scale_code(amax);
    const float s = e4m3fn_value(sc);
    uint32_t packed = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) packed |= e2m1_encode(v[i] / s) << (4 * i);
    *reinterpret_cast<uint32_t*>(dst + 4 * lane) = packed;
    if ((lane & 1) == 0) dst[n / 2 + (lane >> 1)] = (uint8_t)sc;
  } else {
    // n == 512: lane l holds values 8l..8l+7 of block l / 4.
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = value(8 * lane + i);
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    amax = fmaxf(amax, __shfl_xor(amax, 2));
    const uint32_t E = e8m0_exponent(amax);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo |= e4m3fn_encode(ldexpf(v[i], 127 - (int)E)) << (8 * i);
      hi |= e4m3fn_encode(ldexpf(v[4 + i], 127 - (int)E)) << (8 * i);
    }
    *reinterpret_cast<uint2*>(dst + 8 * lane) = make_uint2(lo, hi);
    if ((lane & 3) == 0) dst[n + (lane >> 2)] = (uint8_t)E;
  }
}

}  // namespace

hipError_t launch_cache_write(const CacheWriteArgs& a, hipStream_t s) {
  if (a.n_rows == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((a.n_rows + kRowsPerBlock - 1) / kRowsPerBlock);
  switch (a.fmt) {
    case kF32: cache_write_kernel<kF32><<<blocks, 64 * kRowsPerBlock, 0, s>>>(a); break;
    case kBF16: cache_write_kernel<kBF16><<<blocks, 64 * kRowsPerBlock, 0, s>>>(a); break;
    case kFP8: cache_write_kernel<kFP8><<<blocks, 64 * kRowsPerBlock, 0, s>>>(a); break;
    case kFP4: cache_write_kernel<kFP4><<<blocks, 64 * kRowsPerBlock, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mla
