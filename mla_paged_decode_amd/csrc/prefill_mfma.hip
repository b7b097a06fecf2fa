// Prefill K/V rebuild on the matrix cores (gfx950): per head h and cached
// token t, the rows of kv_b_proj times the latent,
//   [k_t ; v_t] = W[h] c_t,   W[h] = [W_UK[h] ; W_UV[h]]  ((d_nope + d_v) x d_latent),
// as v_mfma_f32_16x16x32_bf16 products with fp32 accumulation.
//
// Workgroup = 4 waves over one (sequence, head), 64 output rows of W[h]
// (16 per wave, held in registers as the B operand for the whole
// workgroup) and up to 8 blocks of 16 tokens.  Per block the latent rows
// are decoded from the cache row into a bf16 tile in LDS (the A operand).
// bf16, fp8 and fp4 latents are exact in bf16; an f32 latent is split into
// bf16 hi + lo parts, two products per k-step, as the fp32 projections do.
#include <cmath>

#include "decode_common.h"
#include "device_common.h"
#include "internal.h"

namespace mla {
namespace {

using mfma::bf16x8;
using mfma::f32x4;

constexpr int kTokBlk = 16;    // tokens per MFMA row block
constexpr int kBlocks = 8;     // token blocks per workgroup
constexpr int kWaves = 4;
constexpr int kCols = 16 * kWaves;  // output rows of W[h] per workgroup

// Value i of a quantised row (fp8: e4m3 x e8m0 per 32; fp4: e2m1 x e4m3 per
// 16); n = d_latent + d_rope.
template <int FMT>
__device__ __forceinline__ float quant_value(const uint8_t* row, int i, int n) {
  if constexpr (FMT == kFP8) {
    return e4m3fn_to_f32(row[i]) * e8m0_to_f32(row[n + i / 32]);
  } else {
    const uint32_t code = (row[i >> 1] >> (4 * (i & 1))) & 0xfu;
    return e2m1_to_f32(code) * e4m3fn_to_f32(row[n / 2 + i / 16]);
  }
}

template <int FMT>
__device__ __forceinline__ float any_value(const uint8_t* row, int i, int n) {
  if constexpr (FMT == kF32) return reinterpret_cast<const float*>(row)[i];
  else if constexpr (FMT == kBF16) return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(row)[i]);
  else return quant_value<FMT>(row, i, n);
}

template <int FMT, int NKS>  // NKS = d_latent / 32
__global__ __launch_bounds__(64 * kWaves) void prefill_expand_mfma_kernel(PrefillArgs a) {
  constexpr int kDc = 32 * NKS;
  constexpr int kRowB = kDc * 2 + 16;  // LDS row stride (bytes) of the bf16 tile
  constexpr bool kSplit = FMT == kF32;
  __shared__ __attribute__((aligned(16))) char hi_tile[kTokBlk * kRowB];
  __shared__ __attribute__((aligned(16))) char lo_tile[kSplit ? kTokBlk * kRowB : 16];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, g = lane >> 4, li = lane & 15;
  const int b = blockIdx.z / a.H, h = blockIdx.z % a.H;
  const int col = blockIdx.y * kCols + 16 * wave + li;  // row of W[h], < d_nope + d_v
  const int L = (int)min((int64_t)max(a.seq_lens[b], 0), a.Lcap);
  const int t_begin = blockIdx.x * kTokBlk * kBlocks;
  if (t_begin >= L) return;  // uniform
  const int t_end = min(L, t_begin + kTokBlk * kBlocks);
  const int nv = a.dc + a.dr;

  const uint16_t* w = static_cast<const uint16_t*>(a.w) + ((int64_t)h * (a.dn + a.dv) + col) * a.dc;
  bf16x8 wb[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
    wb[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(w + 32 * ks + 8 * g));

  for (int t0 = t_begin; t0 < t_end; t0 += kTokBlk) {
    // bf16 tile of the block's latent rows (rows past the end are zero)
    for (int idx = tid; idx < kTokBlk * (kDc / 8); idx += 64 * kWaves) {
      const int r = idx / (kDc / 8), c8 = idx % (kDc / 8), t = t0 + r;
      uint4 hv = make_uint4(0u, 0u, 0u, 0u), lv = make_uint4(0u, 0u, 0u, 0u);
      if (t < t_end) {
        const int page = a.block_table[(int64_t)b * a.max_blocks + t / a.P];
        const uint8_t* row = a.pool + ((int64_t)page * a.P + (t % a.P)) * a.row_bytes;
        if constexpr (FMT == kBF16) {
          hv = *reinterpret_cast<const uint4*>(row + 16 * c8);
        } else {
          float x[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) x[j] = any_value<FMT>(row, 8 * c8 + j, nv);
          uint32_t hw[4], lw[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if constexpr (kSplit) split_bf16x2(x[2 * j], x[2 * j + 1], hw[j], lw[j]);
            else hw[j] = bf16x2_bits(x[2 * j], x[2 * j + 1]), lw[j] = 0u;  // exact in bf16
          }
          hv = make_uint4(hw[0], hw[1], hw[2], hw[3]);
          lv = make_uint4(lw[0], lw[1], lw[2], lw[3]);
        }
      }
      *reinterpret_cast<uint4*>(hi_tile + r * kRowB + 16 * c8) = hv;
      if constexpr (kSplit) *reinterpret_cast<uint4*>(lo_tile + r * kRowB + 16 * c8) = lv;
    }
    // the shared RoPE keys, once per token: head 0, first column group
    if (h == 0 && blockIdx.y == 0)
      for (int idx = tid; idx < kTokBlk * a.dr; idx += 64 * kWaves) {
        const int r = idx / a.dr, i = idx % a.dr, t = t0 + r;
        if (t < t_end) {
          const int page = a.block_table[(int64_t)b * a.max_blocks + t / a.P];
          const uint8_t* row = a.pool + ((int64_t)page * a.P + (t % a.P)) * a.row_bytes;
          a.kr[((int64_t)b * a.Lcap + t) * a.dr + i] = any_value<FMT>(row, a.dc + i, nv);
        }
      }
    __syncthreads();

    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    const char* hrow = hi_tile + li * kRowB + 16 * g;
    const char* lrow = lo_tile + (kSplit ? li * kRowB + 16 * g : 0);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const bf16x8 ah = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(hrow + 64 * ks));
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, wb[ks], acc, 0, 0, 0);
      if constexpr (kSplit) {
        const bf16x8 al = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(lrow + 64 * ks));
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, wb[ks], acc, 0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 4 * g + i;
      if (t < t_end) {
        const int64_t tok = ((int64_t)b * a.Lcap + t) * a.H + h;
        if (col < a.dn) a.kn[tok * a.dn + col] = acc[i];
        else a.v[tok * a.dv + (col - a.dn)] = acc[i];
      }
    }
    __syncthreads();  // the tile is rewritten by the next block
  }
}

template <int FMT>
hipError_t launch_fmt(const PrefillArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((a.Lcap + kTokBlk * kBlocks - 1) / (kTokBlk * kBlocks)),
                  (unsigned)((a.dn + a.dv) / kCols), (unsigned)(a.B * a.H));
  switch (a.dc / 32) {
#define MLA_CASE(K) \
  case K: prefill_expand_mfma_kernel<FMT, K><<<grid, 64 * kWaves, 0, s>>>(a); break;
    MLA_CASE(1) MLA_CASE(2) MLA_CASE(3) MLA_CASE(4) MLA_CASE(5) MLA_CASE(6) MLA_CASE(7) MLA_CASE(8)
    MLA_CASE(9) MLA_CASE(10) MLA_CASE(11) MLA_CASE(12) MLA_CASE(13) MLA_CASE(14) MLA_CASE(15) MLA_CASE(16)
#undef MLA_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

bool prefill_expand_mfma_supported(const PrefillArgs& a) {
  return !a.w_f32 && a.dc % 32 == 0 && a.dc <= 512 && (a.dn + a.dv) % kCols == 0 && a.dr % 4 == 0;
}

hipError_t launch_prefill_expand_mfma(const PrefillArgs& a, int fmt, hipStream_t s) {
  if (!prefill_expand_mfma_supported(a)) return hipErrorInvalidValue;
  switch (fmt) {
    case kF32: return launch_fmt<kF32>(a, s);
    case kBF16: return launch_fmt<kBF16>(a, s);
    case kFP8: return launch_fmt<kFP8>(a, s);
    case kFP4: return launch_fmt<kFP4>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mla
