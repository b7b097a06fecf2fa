// Unabsorbed MLA prefill over the paged latent cache: the fp32 vector-ALU
// kernels, and the launcher (which takes the matrix-core kernels of
// prefill_mfma.hip where they apply: the K/V rebuild for bf16 weights, the
// attention for 256-wide keys and values).
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
//   2. prefill_attn_kernel: per (16 queries, head) a workgroup walks the
//      keys in blocks of 16 staged in LDS once for all 16 queries: one score
//      per thread, an online-softmax update per query, and each thread
//      accumulating 16 output columns of its query.
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

// Attention: a workgroup takes 16 consecutive queries of one (sequence,
// head) and walks the keys in blocks of 16, staged in LDS once for all 16
// queries.  Thread (qi, k) = (tid / 16, tid % 16) scores query qi against
// key k of the block, then owns output columns 16k .. 16k + 15 of query qi.
constexpr int kQB = 16;      // queries per workgroup
constexpr int kKB = 16;      // keys per block
constexpr int kRow = 260;    // LDS row stride in floats: float4 rows 4 banks apart

__device__ __forceinline__ float group16_max(float v) {
  for (int o = 8; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float group16_sum(float v) {
  for (int o = 8; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__global__ __launch_bounds__(kQB * kKB) void prefill_attn_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) float sQ[kQB][kRow];
  __shared__ __attribute__((aligned(16))) float sK[kKB][kRow];
  __shared__ __attribute__((aligned(16))) float sV[kKB][kRow];
  __shared__ float sP[kQB][kKB + 1];
  const int tid = threadIdx.x;
  const int h = blockIdx.y;
  const int nqb = (a.Sq + kQB - 1) / kQB;
  const int b = blockIdx.x / nqb, i0 = (blockIdx.x % nqb) * kQB;
  const int L = (int)min((int64_t)max(a.seq_lens[b], 0), a.Lcap);
  const int nqk = a.dn + a.dr;
  for (int idx = tid; idx < kQB * nqk; idx += kQB * kKB) {
    const int r = idx / nqk, d = idx % nqk, i = i0 + r;
    const int64_t off = (((int64_t)b * a.Sq + i) * a.H + h) * nqk + d;
    float x = 0.f;
    if (i < a.Sq) x = a.q_f32 ? static_cast<const float*>(a.q)[off] : bf16_bits_to_f32(static_cast<const uint16_t*>(a.q)[off]);
    sQ[r][d] = x;
  }
  const int qi = tid >> 4, k = tid & 15;
  const int my_last = L - a.Sq + i0 + qi;  // this query sees t <= my_last
  const int blk_last = min(L - 1, L - a.Sq + min(i0 + kQB, a.Sq) - 1);  // the block's last visible key
  float o[16];
#pragma unroll
  for (int c = 0; c < 16; ++c) o[c] = 0.f;
  float m = -INFINITY, l = 0.f;  // base 2, the same in the 16 threads of a query
  const int nk4 = nqk / 4, nv4 = a.dv / 4;
  for (int t0 = 0; t0 <= blk_last; t0 += kKB) {
    __syncthreads();  // the previous block's readers are done (and the queries are in)
    for (int idx = tid; idx < kKB * nk4; idx += kQB * kKB) {
      const int r = idx / nk4, c4 = idx % nk4, t = t0 + r;
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
      if (t <= blk_last)
        x = 4 * c4 < a.dn ? reinterpret_cast<const float4*>(a.kn + (((int64_t)b * a.Lcap + t) * a.H + h) * a.dn)[c4]
                          : reinterpret_cast<const float4*>(a.kr + ((int64_t)b * a.Lcap + t) * a.dr)[c4 - a.dn / 4];
      *reinterpret_cast<float4*>(&sK[r][4 * c4]) = x;
    }
    for (int idx = tid; idx < kKB * nv4; idx += kQB * kKB) {
      const int r = idx / nv4, c4 = idx % nv4, t = t0 + r;
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
      if (t <= blk_last) x = reinterpret_cast<const float4*>(a.v + (((int64_t)b * a.Lcap + t) * a.H + h) * a.dv)[c4];
      *reinterpret_cast<float4*>(&sV[r][4 * c4]) = x;
    }
    __syncthreads();

    const int t = t0 + k;
    float d0 = 0.f, d1 = 0.f, d2 = 0.f, d3 = 0.f;
#pragma unroll 4
    for (int c4 = 0; c4 < nk4; ++c4) {
      const float4 x = *reinterpret_cast<const float4*>(&sQ[qi][4 * c4]);
      const float4 y = *reinterpret_cast<const float4*>(&sK[k][4 * c4]);
      d0 = fmaf(x.x, y.x, d0), d1 = fmaf(x.y, y.y, d1), d2 = fmaf(x.z, y.z, d2), d3 = fmaf(x.w, y.w, d3);
    }
    const float sc = t <= my_last ? ((d0 + d1) + (d2 + d3)) * a.scale_log2 : -INFINITY;
    const float m_new = fmaxf(m, group16_max(sc));
    float alpha = 1.f, p = 0.f;
    if (m_new != -INFINITY) {  // uniform over the query's 16 threads
      alpha = m == -INFINITY ? 0.f : exp2f(m - m_new);
      p = sc == -INFINITY ? 0.f : exp2f(sc - m_new);
    }
    l = l * alpha + group16_sum(p);
    m = m_new;
    sP[qi][k] = p;
#pragma unroll
    for (int c = 0; c < 16; ++c) o[c] *= alpha;
    __syncthreads();  // P of the block is in LDS

#pragma unroll 4
    for (int tt = 0; tt < kKB; ++tt) {
      const float pt = sP[qi][tt];
      const float4* vr = reinterpret_cast<const float4*>(&sV[tt][16 * k]);
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) {
        const float4 y = vr[c4];
        o[4 * c4 + 0] = fmaf(pt, y.x, o[4 * c4 + 0]);
        o[4 * c4 + 1] = fmaf(pt, y.y, o[4 * c4 + 1]);
        o[4 * c4 + 2] = fmaf(pt, y.z, o[4 * c4 + 2]);
        o[4 * c4 + 3] = fmaf(pt, y.w, o[4 * c4 + 3]);
      }
    }
  }
  const int i = i0 + qi;
  if (i >= a.Sq) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  float* dst = a.out + (((int64_t)b * a.Sq + i) * a.H + h) * a.dv;
#pragma unroll
  for (int c = 0; c < 16; ++c)
    if (16 * k + c < a.dv) dst[16 * k + c] = o[c] * inv;
  if (a.lse && k == 0) a.lse[((int64_t)b * a.Sq + i) * a.H + h] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
}

}  // namespace

bool prefill_supported(int dc, int dr, int dn, int dv) {
  return dc >= 4 && dc <= kMaxLatent && dc % 4 == 0 && dn + dr <= kMaxQk && dv <= kMaxV;
}

hipError_t launch_prefill(const PrefillArgs& a, int fmt, hipStream_t s) {
  if (a.B == 0 || a.Sq == 0) return hipSuccess;
  const dim3 eg((unsigned)((a.Lcap + kExpandTok - 1) / kExpandTok), (unsigned)a.B, (unsigned)a.H);
  if (prefill_expand_mfma_supported(a)) {
    const hipError_t e = launch_prefill_expand_mfma(a, fmt, s);
    if (e != hipSuccess) return e;
  } else switch (fmt) {
    case kF32: prefill_expand_kernel<kF32><<<eg, kExpandThreads, 0, s>>>(a); break;
    case kBF16: prefill_expand_kernel<kBF16><<<eg, kExpandThreads, 0, s>>>(a); break;
    case kFP8: prefill_expand_kernel<kFP8><<<eg, kExpandThreads, 0, s>>>(a); break;
    case kFP4: prefill_expand_kernel<kFP4><<<eg, kExpandThreads, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (prefill_attn_mfma_supported(a)) return launch_prefill_attn_mfma(a, s);
  const unsigned qblocks = (unsigned)((a.Sq + kQB - 1) / kQB);
  prefill_attn_kernel<<<dim3((unsigned)a.B * qblocks, (unsigned)a.H), kQB * kKB, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mla
