// Query absorption and value up-projection on the matrix cores.
//
// Both are per-head GEMMs with the head's slice of kv_b_proj
// ([d_nope + d_v][d_latent], row-major, bf16):
//   absorb:   q_lat[n][c] = sum_k q[n][k] * W[k][c]          (K = d_nope)
//   out_proj: out[n][v]   = sum_c o[n][c] * W[d_nope + v][c] (K = d_latent)
// with v_mfma_f32_16x16x32_bf16 (A: row l%16, k 8g..8g+7; B: column l%16,
// k 8g..8g+7; C: column l%16, rows 4g..4g+3; g = lane / 16).
//
// absorb: the weight's contiguous dimension is the output column, so a
// 64-column weight tile is staged in LDS and read k-major with
// ds_read_b64_tr_b16.  bf16 q times bf16 W is exact in fp32.
// out_proj: weight rows are contiguous along K and load straight into the B
// operand.  The fp32 latent input is split into hi + lo bf16 parts, so the
// products are exact to ~16 significant bits; accumulation is fp32.
//
// Workgroup: 4 waves x 16 tokens, one head, a 64-wide block of output
// columns.  grid = (ceil(N / 64), out_cols / 64, H).
#include "device_common.h"
#include "internal.h"

namespace mla {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr int kWaves = 4;
constexpr int kTokPerWg = 16 * kWaves;
constexpr int kCols = 64;                 // output columns per workgroup
constexpr int kMaxNope = 512;
constexpr int kWRow = kCols * 2 + 16;     // LDS row stride (bytes) of the weight tile

__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

__device__ __forceinline__ uint32_t pack2(uint32_t lo, uint32_t hi) { return lo | (hi << 16); }

template <bool kOutF32, int NKS>  // NKS = d_nope / 32
__global__ __launch_bounds__(64 * kWaves) void absorb_mfma_kernel(ProjArgs a) {
  __shared__ __attribute__((aligned(16))) char w_tile[kMaxNope * kWRow];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, li = lane & 15;
  const int h = blockIdx.z, c0 = blockIdx.y * kCols;
  const int n0 = blockIdx.x * kTokPerWg + wave * 16;
  const uint16_t* w = static_cast<const uint16_t*>(a.w) + (int64_t)h * (a.dn + a.dv) * a.dc;

  const int n = n0 + li;
  const bool n_ok = n < a.N;
  const int qw = a.dn + a.dr, ow = a.dc + a.dr;
  const uint16_t* q = static_cast<const uint16_t*>(a.in) + ((int64_t)(n_ok ? n : 0) * a.H + h) * qw;
  // This wave's query operands, all loads issued before the weight tile's.
  bf16x8 qa[NKS];
  const bf16x8 zero = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) qa[ks] = n_ok ? load_bf16x8(q + 32 * ks + 8 * g) : zero;

  // Stage W[0:dn][c0:c0+64]: 8 chunks of 16 B per row.
  for (int i = threadIdx.x; i < a.dn * 8; i += 64 * kWaves) {
    const int k = i >> 3, ch = i & 7;
    *reinterpret_cast<uint4*>(w_tile + k * kWRow + 16 * ch) =
        *reinterpret_cast<const uint4*>(w + (int64_t)k * a.dc + c0 + 8 * ch);
  }
  __syncthreads();

  f32x4 acc[kCols / 16];
#pragma unroll
  for (int cb = 0; cb < kCols / 16; ++cb) acc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    const char* rows = w_tile + (32 * ks + 8 * g + (li >> 2)) * kWRow + 8 * (li & 3);
#pragma unroll
    for (int cb = 0; cb < kCols / 16; ++cb) {
      const bf16x4 b0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(rows + 32 * cb));
      const bf16x4 b1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(rows + 4 * kWRow + 32 * cb));
      const bf16x8 wb = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
      acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ks], wb, acc[cb], 0, 0, 0);
    }
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int nn = n0 + 4 * g + i;
    if (nn >= a.N) continue;
    const int64_t base = ((int64_t)nn * a.H + h) * ow + c0 + li;
#pragma unroll
    for (int cb = 0; cb < kCols / 16; ++cb) {
      if (kOutF32) static_cast<float*>(a.out)[base + 16 * cb] = acc[cb][i];
      else static_cast<uint16_t*>(a.out)[base + 16 * cb] = (uint16_t)f32_to_bf16_bits(acc[cb][i]);
    }
  }
  // The RoPE part of the query is copied unchanged by the first column block.
  if (blockIdx.y == 0) {
    for (int i = lane; i < 16 * a.dr; i += 64) {
      const int nn = n0 + i / a.dr, k = i % a.dr;
      if (nn >= a.N) continue;
      const int64_t r = (int64_t)nn * a.H + h;
      const uint16_t v = static_cast<const uint16_t*>(a.in)[r * qw + a.dn + k];
      if (kOutF32) static_cast<float*>(a.out)[r * ow + a.dc + k] = bf16_bits_to_f32(v);
      else static_cast<uint16_t*>(a.out)[r * ow + a.dc + k] = v;
    }
  }
}

constexpr int kMaxLatent = 512;
constexpr int kVRow = kMaxLatent * 2 + 16;  // LDS row stride (bytes): 16 rows hit distinct banks

template <int NKS>  // NKS = d_latent / 32
__global__ __launch_bounds__(64 * kWaves) void out_proj_mfma_kernel(ProjArgs a) {
  __shared__ __attribute__((aligned(16))) char w_tile[kCols * kVRow];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, li = lane & 15;
  const int h = blockIdx.z, v0 = blockIdx.y * kCols;
  const int n0 = blockIdx.x * kTokPerWg + wave * 16;
  const int n = n0 + li;
  const bool n_ok = n < a.N;
  const float* o = static_cast<const float*>(a.in) + ((int64_t)(n_ok ? n : 0) * a.H + h) * a.dc;
  const uint16_t* w = static_cast<const uint16_t*>(a.w) + ((int64_t)h * (a.dn + a.dv) + a.dn + v0) * a.dc;

  // This wave's latent operands (fp32 -> hi + lo bf16), loads issued first.
  float4 raw[NKS][2];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    if (n_ok) {
      raw[ks][0] = *reinterpret_cast<const float4*>(o + 32 * ks + 8 * g);
      raw[ks][1] = *reinterpret_cast<const float4*>(o + 32 * ks + 8 * g + 4);
    } else {
      raw[ks][0] = raw[ks][1] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  // Stage W_UV rows v0..v0+63 (K-contiguous) into LDS.
  const int chunks = a.dc / 8;
  for (int i = threadIdx.x; i < kCols * chunks; i += 64 * kWaves) {
    const int r = i / chunks, ch = i % chunks;
    *reinterpret_cast<uint4*>(w_tile + r * kVRow + 16 * ch) =
        *reinterpret_cast<const uint4*>(w + (int64_t)r * a.dc + 8 * ch);
  }
  __syncthreads();

  f32x4 acc[kCols / 16];
#pragma unroll
  for (int vb = 0; vb < kCols / 16; ++vb) acc[vb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    const float x[8] = {raw[ks][0].x, raw[ks][0].y, raw[ks][0].z, raw[ks][0].w,
                        raw[ks][1].x, raw[ks][1].y, raw[ks][1].z, raw[ks][1].w};
    uint32_t hb[8], lb[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      hb[i] = f32_to_bf16_bits(x[i]);
      lb[i] = f32_to_bf16_bits(x[i] - bf16_bits_to_f32(hb[i]));
    }
    const bf16x8 ah = __builtin_bit_cast(bf16x8, make_uint4(pack2(hb[0], hb[1]), pack2(hb[2], hb[3]),
                                                            pack2(hb[4], hb[5]), pack2(hb[6], hb[7])));
    const bf16x8 al = __builtin_bit_cast(bf16x8, make_uint4(pack2(lb[0], lb[1]), pack2(lb[2], lb[3]),
                                                            pack2(lb[4], lb[5]), pack2(lb[6], lb[7])));
#pragma unroll
    for (int vb = 0; vb < kCols / 16; ++vb) {
      const bf16x8 wb = *reinterpret_cast<const bf16x8*>(w_tile + (16 * vb + li) * kVRow + 64 * ks + 16 * g);
      acc[vb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, wb, acc[vb], 0, 0, 0);
      acc[vb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, wb, acc[vb], 0, 0, 0);
    }
  }
  float* out = static_cast<float*>(a.out);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int nn = n0 + 4 * g + i;
    if (nn >= a.N) continue;
    const int64_t base = ((int64_t)nn * a.H + h) * a.dv + v0 + li;
#pragma unroll
    for (int vb = 0; vb < kCols / 16; ++vb) out[base + 16 * vb] = acc[vb][i];
  }
}

}  // namespace

bool absorb_mfma_supported(const ProjArgs& a) {
  return !a.in_f32 && !a.w_f32 && a.dc % kCols == 0 && a.dn % 32 == 0 && a.dn <= kMaxNope && a.dr % 16 == 0;
}

bool out_proj_mfma_supported(const ProjArgs& a) {
  return !a.w_f32 && a.dv % kCols == 0 && a.dc % 32 == 0 && a.dc <= kMaxLatent;
}

hipError_t launch_absorb_mfma(const ProjArgs& a, hipStream_t s) {
  const dim3 grid((a.N + kTokPerWg - 1) / kTokPerWg, a.dc / kCols, a.H);
  switch (a.dn / 32) {
#define MLA_CASE(K)                                                                   \
  case K:                                                                             \
    if (a.out_f32) absorb_mfma_kernel<true, K><<<grid, 64 * kWaves, 0, s>>>(a);       \
    else absorb_mfma_kernel<false, K><<<grid, 64 * kWaves, 0, s>>>(a);                \
    break;
    MLA_CASE(1) MLA_CASE(2) MLA_CASE(3) MLA_CASE(4) MLA_CASE(5) MLA_CASE(6) MLA_CASE(7) MLA_CASE(8)
    MLA_CASE(9) MLA_CASE(10) MLA_CASE(11) MLA_CASE(12) MLA_CASE(13) MLA_CASE(14) MLA_CASE(15) MLA_CASE(16)
#undef MLA_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_out_proj_mfma(const ProjArgs& a, hipStream_t s) {
  const dim3 grid((a.N + kTokPerWg - 1) / kTokPerWg, a.dv / kCols, a.H);
  switch (a.dc / 32) {
#define MLA_CASE(K) \
  case K: out_proj_mfma_kernel<K><<<grid, 64 * kWaves, 0, s>>>(a); break;
    MLA_CASE(1) MLA_CASE(2) MLA_CASE(3) MLA_CASE(4) MLA_CASE(5) MLA_CASE(6) MLA_CASE(7) MLA_CASE(8)
    MLA_CASE(9) MLA_CASE(10) MLA_CASE(11) MLA_CASE(12) MLA_CASE(13) MLA_CASE(14) MLA_CASE(15) MLA_CASE(16)
#undef MLA_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mla
