// Unabsorbed MLA prefill over the paged latent cache, fp32 on the vector ALUs.
//
// A chunk of Sq new tokens per sequence (already appended, the last Sq of
// the L cached tokens) attends causally to the whole cache in the
// unabsorbed form of multi-head latent attention (DeepSeek-V2 MLA, as the
// GLM-4.7-Flash model record uses it): per head h the no-RoPE key and the
// value of every cached token are rebuilt through kv_b_proj,
//   k_t = [W_UK[h] c_t , k^R_t],   v_t = W_UV[h] c_t,
// and query i (position L - Sq + i) runs softmax attention over t <= its
// position.  Two kernels:
//   1. prefill_expand_kernel: per (32-token block, sequence, head) the
//      latent rows are decoded to fp32 into LDS and multiplied by the head's
//      kv_b_proj rows; K (no-RoPE part), the shared RoPE key and V go to the
//      workspace as fp32;
//   2. prefill_attn_kernel: one wave per (query token, head); a 64-token
//      block's scores (one token per lane), an online-softmax update, and
//      the value rows accumulated with each lane owning 4 output columns.
// Every product is an fp32 FMA; this is the full-precision first path of the
// prefill, not a matrix-core one.
#include <cmath>

#include "device_common.h"
#include "internal.h"

namespace mla {
namespace {

constexpr int kExpandTok = 32;       // tokens per expand workgroup
constexpr int kExpandThreads = 256;
constexpr int kMaxLatent = 512;      // d_latent at most
constexpr int kMaxQk = 256;          // d_nope + d_rope at most
constexpr int kMaxV = 256;           // d_v at most
constexpr float kLn2 = 0.693147180559945309f;

// Value i of a stored row (f32, bf16, fp8 e4m3 + e8m0 per 32, fp4 e2m1 +
// e4m3 per 16); n = d_latent + d_rope values per row.
template <int FMT>
__device__ __forceinline__ float row_value(const uint8_t* row, int i, int n) {
  if constexpr (FMT == kF32) {
    return reinterpret_cast<const float*>(row)[i];
  } else if constexpr (FMT == kBF16) {
    return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(row)[i]);
  } else if constexpr (FMT == kFP8) {
    return e4m3fn_to_f32(row[i]) * e8m0_to_f32(row[n + i / 32]);
  } else {
    const uint32_t code = (row[i >> 1] >> (4 * (i & 1))) & 0xfu;
    return e2m1_to_f32(code) * e4m3fn_to_f32(row[n / 2 + i / 16]);
  }
}

__device__ __forceinline__ const uint8_t* cache_row(const PrefillArgs& a, int b, int t) {
  const int page = a.block_table[(int64_t)b * a.max_blocks + t / a.P];
  return a.pool + ((int64_t)page * a.P + (t % a.P)) * a.row_bytes;
}

template <int FMT>
__global__ __launch_bounds__(kExpandThreads) void prefill_expand_kernel(PrefillArgs a) {
  __shared__ float sC[kExpandTok][kMaxLatent];
  const int b = blockIdx.y, h = blockIdx.z;
  const int t0 = blockIdx.x * kExpandTok;
  // Lengths past the table's capacity are clamped to it: no read or write
  // leaves the sequence's block-table row or workspace slots.
  const int L = (int)min((int64_t)max(a.seq_lens[b], 0), a.Lcap);
  if (t0 >= L) return;  // the whole workgroup: t0 and L are uniform
  const int n = min(kExpandTok, L - t0);
  const int nv = a.dc + a.dr;
  const int tid = threadIdx.x;
  for (int idx = tid; idx < kExpandTok * a.dc; idx += kExpandThreads) {
    const int tk = idx / a.dc, c = idx % a.dc;
    sC[tk][c] = tk < n ? row_value<FMT>(cache_row(a, b, t0 + tk), c, nv) : 0.f;
  }
  if (h == 0)
    for (int idx = tid; idx < n * a.dr; idx += kExpandThreads) {
      const int tk = idx / a.dr, i = idx % a.dr;
      a.kr[((int64_t)b * a.Lcap + t0 + tk) * a.dr + i] = row_value<FMT>(cache_row(a, b, t0 + tk), a.dc + i, nv);
    }
  __syncthreads();

  const int nout = a.dn + a.dv;
  for (int j = tid; j < nout; j += kExpandThreads) {
    float acc[kExpandTok];
#pragma unroll
    for (int tk = 0; tk < kExpandTok; ++tk) acc[tk] = 0.f;
    const int64_t w0 = ((int64_t)h * nout + j) * a.dc;
    for (int c = 0; c < a.dc; c += 4) {
      float w[4];
      if (a.w_f32) {
        const float4 v = *reinterpret_cast<const float4*>(static_cast<const float*>(a.w) + w0 + c);
        w[0] = v.x, w[1] = v.y, w[2] = v.z, w[3] = v.w;
      } else {
        const uint2 v = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.w) + w0 + c);
        w[0] = bf16_bits_to_f32(v.x & 0xffffu), w[1] = bf16_bits_to_f32(v.x >> 16);
        w[2] = bf16_bits_to_f32(v.y & 0xffffu), w[3] = bf16_bits_to_f32(v.y >> 16);
      }
#pragma unroll
      for (int tk = 0; tk < kExpandTok; ++tk) {
        const float4 x = *reinterpret_cast<const float4*>(&sC[tk][c]);
        acc[tk] = fmaf(w[0], x.x, fmaf(w[1], x.y, fmaf(w[2], x.z, fmaf(w[3], x.w, acc[tk]))));
      }
    }
#pragma unroll
    for (int tk = 0; tk < kExpandTok; ++tk) {
      if (tk >= n) break;
      const int64_t tok = ((int64_t)b * a.Lcap + t0 + tk) * a.H + h;
      if (j < a.dn) a.kn[tok * a.dn + j] = acc[tk];
      else a.v[tok * a.dv + (j - a.dn)] = acc[tk];
    }
  }
}

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__global__ __launch_bounds__(64) void prefill_attn_kernel(PrefillArgs a) {
  __shared__ float sq[kMaxQk];
  __shared__ float sp[64];
  const int bq = blockIdx.x, h = blockIdx.y;
  const int b = bq / a.Sq, i = bq % a.Sq;
  const int lane = threadIdx.x;
  const int L = (int)min((int64_t)max(a.seq_lens[b], 0), a.Lcap);
  const int last = L - a.Sq + i;  // visible positions t <= last
  const int nqk = a.dn + a.dr;
  const int64_t qoff = ((int64_t)bq * a.H + h) * nqk;
  for (int d = lane; d < nqk; d += 64)
    sq[d] = a.q_f32 ? static_cast<const float*>(a.q)[qoff + d]
                    : bf16_bits_to_f32(static_cast<const uint16_t*>(a.q)[qoff + d]);
  __syncthreads();

  float o[kMaxV / 64] = {0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;  // base-2 running maximum and sum
  for (int t0 = 0; t0 <= last; t0 += 64) {
    const int t = t0 + lane;
    float s = -INFINITY;
    if (t <= last) {
      const float* kn = a.kn + (((int64_t)b * a.Lcap + t) * a.H + h) * a.dn;
      const float* kr = a.kr + ((int64_t)b * a.Lcap + t) * a.dr;
      float dot = 0.f;
      for (int d = 0; d < a.dn; ++d) dot = fmaf(sq[d], kn[d], dot);
      for (int d = 0; d < a.dr; ++d) dot = fmaf(sq[a.dn + d], kr[d], dot);
      s = dot * a.scale_log2;
    }
    const float m_new = fmaxf(m, wave_max(s));  // finite: t0 <= last
    const float alpha = m == -INFINITY ? 0.f : exp2f(m - m_new);
    const float p = t <= last ? exp2f(s - m_new) : 0.f;
    l = l * alpha + wave_sum(p);
#pragma unroll
    for (int k = 0; k < kMaxV / 64; ++k) o[k] *= alpha;
    sp[lane] = p;
    __syncthreads();
    const int nt = min(64, last + 1 - t0);
    for (int tt = 0; tt < nt; ++tt) {
      const float pt = sp[tt];
      const float* vr = a.v + (((int64_t)b * a.Lcap + t0 + tt) * a.H + h) * a.dv;
#pragma unroll
      for (int k = 0; k < kMaxV / 64; ++k) {
        const int d = lane + 64 * k;
        if (d < a.dv) o[k] = fmaf(pt, vr[d], o[k]);
      }
    }
    __syncthreads();  // sp is rewritten by the next block
    m = m_new;
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  float* dst = a.out + ((int64_t)bq * a.H + h) * a.dv;
#pragma unroll
  for (int k = 0; k < kMaxV / 64; ++k) {
    const int d = lane + 64 * k;
    if (d < a.dv) dst[d] = o[k] * inv;
  }
  if (a.lse && lane == 0) a.lse[(int64_t)bq * a.H + h] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
}

}  // namespace

bool prefill_supported(int dc, int dr, int dn, int dv) {
  return dc >= 4 && dc <= kMaxLatent && dc % 4 == 0 && dn + dr <= kMaxQk && dv <= kMaxV;
}

hipError_t launch_prefill(const PrefillArgs& a, int fmt, hipStream_t s) {
  if (a.B == 0 || a.Sq == 0) return hipSuccess;
  const dim3 eg((unsigned)((a.Lcap + kExpandTok - 1) / kExpandTok), (unsigned)a.B, (unsigned)a.H);
  switch (fmt) {
    case kF32: prefill_expand_kernel<kF32><<<eg, kExpandThreads, 0, s>>>(a); break;
    case kBF16: prefill_expand_kernel<kBF16><<<eg, kExpandThreads, 0, s>>>(a); break;
    case kFP8: prefill_expand_kernel<kFP8><<<eg, kExpandThreads, 0, s>>>(a); break;
    case kFP4: prefill_expand_kernel<kFP4><<<eg, kExpandThreads, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  prefill_attn_kernel<<<dim3((unsigned)(a.B * a.Sq), (unsigned)a.H), 64, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mla
