// Query absorption and value up-projection on the matrix cores.
//
// Both are per-head GEMMs with the head's slice of kv_b_proj
// ([d_nope + d_v][d_latent], row-major, bf16):
//   absorb:   q_lat[n][c] = sum_k q[n][k] * W[k][c]          (K = d_nope)
//   out_proj: out[n][v]   = sum_c o[n][c] * W[d_nope + v][c] (K = d_latent)
// with v_mfma_f32_16x16x32_bf16 (A: row l%16, k 8g..8g+7; B: column l%16,
// k 8g..8g+7; C: column l%16, rows 4g..4g+3; g = lane / 16).
//
// absorb: the weight's contiguous dimension is the output column, so the
// workgroup's d_nope x 64 weight tile is staged in LDS (all loads issued
// before the first store) and read k-major with ds_read_b64_tr_b16.  bf16 q
// times bf16 W is exact in fp32.
// out_proj: weight rows are contiguous along K and load straight from
// memory into the B operand.  The fp32 latent input is split into hi + lo
// bf16 parts, so the products are exact to ~16 significant bits;
// accumulation is fp32.
//
// Decode batches are small (tens to hundreds of tokens), so the cost is
// reading the weights: workgroups are small (16 tokens, one head, 64 output
// columns, one wave per 16 columns) to spread those reads over the chip.
// grid = (ceil(N / 16), out_cols / 64, H).
#include "device_common.h"
#include "internal.h"

namespace mla {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

constexpr int kWaves = 4;
constexpr int kTok = 16;                  // tokens per workgroup
constexpr int kCols = 16 * kWaves;        // output columns per workgroup
constexpr int kMaxNope = 512;
constexpr int kWRow = kCols * 2 + 16;     // LDS row stride (bytes) of the weight tile

__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

template <bool kOutF32, int NKS>  // NKS = d_nope / 32
__global__ __launch_bounds__(64 * kWaves) void absorb_mfma_kernel(ProjArgs a) {
  constexpr int kRows = 32 * NKS;               // d_nope
  constexpr int kChunks = kRows * (kCols / 8);  // 16-B chunks of the weight tile
  constexpr int kPer = (kChunks + 64 * kWaves - 1) / (64 * kWaves);
  __shared__ __attribute__((aligned(16))) char w_tile[kRows * kWRow];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, li = lane & 15;
  const int h = blockIdx.z, c0 = blockIdx.y * kCols;
  const int n0 = blockIdx.x * kTok;
  const uint16_t* w = static_cast<const uint16_t*>(a.w) + (int64_t)h * (a.dn + a.dv) * a.dc;

  // Weight tile W[0:dn][c0:c0+64] and the query operands: every load is
  // issued before the first one is waited for.
  u32x4 wt[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = j * 64 * kWaves + threadIdx.x;
    if (i < kChunks) wt[j] = *reinterpret_cast<const u32x4*>(w + (int64_t)(i >> 3) * a.dc + c0 + 8 * (i & 7));
  }
  const int n = n0 + li;
  const bool n_ok = n < a.N;
  const int qw = a.dn + a.dr, ow = a.dc + a.dr;
  const uint16_t* q = static_cast<const uint16_t*>(a.in) + ((int64_t)(n_ok ? n : 0) * a.H + h) * qw;
  bf16x8 qa[NKS];
  const bf16x8 zero = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    qa[ks] = load_bf16x8(q + 32 * ks + 8 * g);  // padding tokens read token 0 ...
    if (!n_ok) qa[ks] = zero;                   // ... and use zeros
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = j * 64 * kWaves + threadIdx.x;
    if (i < kChunks) *reinterpret_cast<u32x4*>(w_tile + (i >> 3) * kWRow + 16 * (i & 7)) = wt[j];
  }
  __syncthreads();

  // This wave's 16 columns c0 + 16 * wave + li.
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    const char* rows = w_tile + (32 * ks + 8 * g + (li >> 2)) * kWRow + 32 * wave + 8 * (li & 3);
    const bf16x4 b0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)rows);
    const bf16x4 b1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(rows + 4 * kWRow));
    const bf16x8 wb = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ks], wb, acc, 0, 0, 0);
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int nn = n0 + 4 * g + i;
    if (nn >= a.N) continue;
    const int64_t o = ((int64_t)nn * a.H + h) * ow + c0 + 16 * wave + li;
    if (kOutF32) static_cast<float*>(a.out)[o] = acc[i];
    else static_cast<uint16_t*>(a.out)[o] = (uint16_t)f32_to_bf16_bits(acc[i]);
  }
  // The RoPE part of the query is copied unchanged by the first column block.
  if (blockIdx.y == 0) {
    for (int i = threadIdx.x; i < kTok * a.dr; i += 64 * kWaves) {
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

template <int NKS>  // NKS = d_latent / 32
__global__ __launch_bounds__(64 * kWaves) void out_proj_mfma_kernel(ProjArgs a) {
  constexpr int kStep = NKS;  // k-steps of latent operands in flight (all of them)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, li = lane & 15;
  const int h = blockIdx.z, v = blockIdx.y * kCols + 16 * wave + li;
  const int n0 = blockIdx.x * kTok;
  const int n = n0 + li;
  const bool n_ok = n < a.N;
  const float* o = static_cast<const float*>(a.in) + ((int64_t)(n_ok ? n : 0) * a.H + h) * a.dc;
  const uint16_t* w = static_cast<const uint16_t*>(a.w) + ((int64_t)h * (a.dn + a.dv) + a.dn + v) * a.dc;

  // B operand: this lane's weight row (value column v), all of K.
  bf16x8 wb[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) wb[ks] = load_bf16x8(w + 32 * ks + 8 * g);

  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k0 = 0; k0 < NKS; k0 += kStep) {
    float4 raw[kStep][2];
#pragma unroll
    for (int j = 0; j < kStep && k0 + j < NKS; ++j) {
      // Padding tokens read token 0 (no branch around the loads) and use zeros.
      raw[j][0] = *reinterpret_cast<const float4*>(o + 32 * (k0 + j) + 8 * g);
      raw[j][1] = *reinterpret_cast<const float4*>(o + 32 * (k0 + j) + 8 * g + 4);
      if (!n_ok) raw[j][0] = raw[j][1] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int j = 0; j < kStep && k0 + j < NKS; ++j) {
      const float x[8] = {raw[j][0].x, raw[j][0].y, raw[j][0].z, raw[j][0].w,
                          raw[j][1].x, raw[j][1].y, raw[j][1].z, raw[j][1].w};
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) split_bf16x2(x[2 * i], x[2 * i + 1], hw[i], lw[i]);
      const bf16x8 ah = __builtin_bit_cast(bf16x8, make_uint4(hw[0], hw[1], hw[2], hw[3]));
      const bf16x8 al = __builtin_bit_cast(bf16x8, make_uint4(lw[0], lw[1], lw[2], lw[3]));
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, wb[k0 + j], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, wb[k0 + j], acc, 0, 0, 0);
    }
  }
  float* out = static_cast<float*>(a.out);
  const int vc = blockIdx.y * kCols + 16 * wave + li;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int nn = n0 + 4 * g + i;
    if (nn < a.N) out[((int64_t)nn * a.H + h) * a.dv + vc] = acc[i];
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
  const dim3 grid((a.N + kTok - 1) / kTok, a.dc / kCols, a.H);
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
  const dim3 grid((a.N + kTok - 1) / kTok, a.dv / kCols, a.H);
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
