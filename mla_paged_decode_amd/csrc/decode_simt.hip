// Split-KV paged MLA decode on the vector ALUs, fp32 throughout.
//
// This is the full-precision path: every cache format is decoded to fp32,
// scores and the value accumulation use fp32 FMAs.  It serves the fp32 cache
// and acts as an independent second kernel for the matrix-core path's tests.
//
// Workgroup = 256 threads = (16 query rows) x (16 tokens per inner tile) for
// the scores; the same threads own 2 latent columns x 16 rows of the output
// accumulator.  grid = (work units, ceil(R / 16)).
//
// Sparse top-k mode (DecodeArgs::sparse_sq > 0): a unit covers slots of a
// (sequence, query token) pair's index list instead of token positions; slot
// t names the cached token topk[b][t], and slots whose entry is negative or
// beyond the query's causal limit are masked (padding).  The page-gather
// and masking are the only differences.
#include <cmath>

#include "device_common.h"
#include "internal.h"
#include "schedule.h"

namespace mla {
namespace {

constexpr int kRows = 16;
constexpr int kTok = 16;
constexpr int kThreads = 256;
constexpr int kMaxVals = 576;            // d_latent + d_rope at most
constexpr int kStride = kMaxVals + 1;    // odd stride: conflict-free columns
constexpr float kLn2 = 0.693147180559945309f;

__device__ __forceinline__ const uint8_t* row_ptr(const DecodeArgs& a, int b, int t) {
  const int page = a.block_table[(int64_t)b * a.max_blocks + t / a.P];
  return a.pool + ((int64_t)page * a.P + (t % a.P)) * a.row_bytes;
}

// Decode the tile's tokens into sK as fp32; zero the rest.  pos[k] is the
// cached position of tile token k, or -1 (no token: past the unit's end, or
// a masked slot of a sparse index list).
template <int FMT>
__device__ void load_tile(const DecodeArgs& a, int b, const int* pos, float (*sK)[kStride]) {
  const int n = a.dc + a.dr;
  if constexpr (FMT == kF32) {
    const int per_row = n / 4;
    for (int idx = threadIdx.x; idx < kTok * per_row; idx += kThreads) {
      const int tk = idx / per_row, c = idx % per_row;
      const int t = pos[tk];
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (t >= 0) v = *reinterpret_cast<const float4*>(row_ptr(a, b, t) + 16 * c);
      sK[tk][4 * c + 0] = v.x;
      sK[tk][4 * c + 1] = v.y;
      sK[tk][4 * c + 2] = v.z;
      sK[tk][4 * c + 3] = v.w;
    }
  } else if constexpr (FMT == kBF16) {
    const int per_row = n / 8;
    for (int idx = threadIdx.x; idx < kTok * per_row; idx += kThreads) {
      const int tk = idx / per_row, c = idx % per_row;
      const int t = pos[tk];
      uint4 v = make_uint4(0, 0, 0, 0);
      if (t >= 0) v = *reinterpret_cast<const uint4*>(row_ptr(a, b, t) + 16 * c);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sK[tk][8 * c + 2 * i + 0] = bf16_bits_to_f32(w[i] & 0xffffu);
        sK[tk][8 * c + 2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
      }
    }
  } else if constexpr (FMT == kFP4) {
    // 32 e2m1 values per 16-byte chunk (value 2i in the low nibble of byte
    // i), two 16-value blocks with an e4m3fn scale each.
    const int per_row = n / 32;
    for (int idx = threadIdx.x; idx < kTok * per_row; idx += kThreads) {
      const int tk = idx / per_row, c = idx % per_row;
      const int t = pos[tk];
      uint4 v = make_uint4(0, 0, 0, 0);
      float s0 = 0.f, s1 = 0.f;
      if (t >= 0) {
        const uint8_t* row = row_ptr(a, b, t);
        v = *reinterpret_cast<const uint4*>(row + 16 * c);
        s0 = e4m3fn_to_f32(row[n / 2 + 2 * c]);
        s1 = e4m3fn_to_f32(row[n / 2 + 2 * c + 1]);
      }
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float sc = i < 2 ? s0 : s1;  // values 32c .. 32c+15, then 32c+16 .. 32c+31
          sK[tk][32 * c + 8 * i + k] = (t >= 0) ? e2m1_to_f32((w[i] >> (4 * k)) & 0xfu) * sc : 0.f;
        }
    }
  } else {
    // 16 e4m3 values per 16-byte chunk, all inside one 32-value scale block.
    const int per_row = n / 16;
    for (int idx = threadIdx.x; idx < kTok * per_row; idx += kThreads) {
      const int tk = idx / per_row, c = idx % per_row;
      const int t = pos[tk];
      uint4 v = make_uint4(0, 0, 0, 0);
      float scale = 0.f;
      if (t >= 0) {
        const uint8_t* row = row_ptr(a, b, t);
        v = *reinterpret_cast<const uint4*>(row + 16 * c);
        scale = e8m0_to_f32(row[n + c / 2]);
      }
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int k = 0; k < 4; ++k)
          sK[tk][16 * c + 4 * i + k] = (t >= 0) ? e4m3fn_to_f32((w[i] >> (8 * k)) & 0xffu) * scale : 0.f;
    }
  }
}

template <int FMT>
__global__ __launch_bounds__(kThreads) void decode_simt_kernel(DecodeArgs a) {
  __shared__ float sQ[kRows][kStride];
  __shared__ float sK[kTok][kStride];
  __shared__ float sP[kRows][kTok + 1];
  __shared__ float sRow[kRows];
  __shared__ int sPos[kTok];

  const int n = a.dc + a.dr;
  const int row0 = blockIdx.y * kRows;
  const int nrows = min(kRows, a.R - row0);
  const int tid = threadIdx.x;
  const int my_r = tid >> 4, my_t = tid & 15;

  for_each_unit(a, [&](int b, int L, int t0, int t1, int64_t slot) {
    __syncthreads();  // the previous unit's readers of sQ / sRow are done
    for (int idx = tid; idx < kRows * n; idx += kThreads) {
      const int r = idx / n, k = idx % n;
      float v = 0.f;
      if (r < nrows) {
        const int64_t off = ((int64_t)b * a.R + row0 + r) * n + k;
        v = a.q_f32 ? static_cast<const float*>(a.q_abs)[off]
                    : bf16_bits_to_f32(static_cast<const uint16_t*>(a.q_abs)[off]);
      }
      sQ[r][k] = v;
    }
    const bool row_ok = my_r < nrows;
    // Sparse: pair b is query token jq of sequence sb; its slots name tokens.
    const int sb = a.sparse_sq ? b / a.sparse_sq : b;
    const int jq = a.sparse_sq ? b % a.sparse_sq : 0;
    const int sparse_visible = a.sparse_sq ? max(a.seq_lens[sb], 0) - a.sparse_sq + jq : 0;
    const int j = row_ok ? (row0 + my_r) / a.H : 0;
    const int last_visible = L - a.Sq + j;  // query j sees tokens [0, last_visible]

    float m = -INFINITY, l = 0.f;
    float acc[2][kRows];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < kRows; ++r) acc[i][r] = 0.f;

    for (int tt0 = t0; tt0 < t1; tt0 += kTok) {
      __syncthreads();  // sK / sP / sRow / sPos are free; sQ is written
      if (tid < kTok) {
        const int t = tt0 + tid;
        int p = -1;
        if (t < t1) {
          if (!a.sparse_sq) {
            p = t;
          } else {
            p = a.topk[(int64_t)b * a.topk_width + t];
            if (p < 0 || p > sparse_visible) p = -1;
          }
        }
        sPos[tid] = p;
      }
      __syncthreads();
      load_tile<FMT>(a, sb, sPos, sK);
      __syncthreads();
      float s = 0.f;
      for (int k = 0; k < n; ++k) s = fmaf(sQ[my_r][k], sK[my_t][k], s);
      s *= a.scale_log2;
      const int t = sPos[my_t];
      const bool valid = row_ok && t >= 0 && (a.sparse_sq || t <= last_visible);
      if (!valid) s = -INFINITY;
      float tmax = s;
#pragma unroll
      for (int o = 8; o >= 1; o >>= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, o, 16));
      const float m_new = fmaxf(m, tmax);
      float alpha = 1.f, p = 0.f;
      if (m_new != -INFINITY) {
        alpha = exp2f(m - m_new);
        p = valid ? exp2f(s - m_new) : 0.f;
      }
      float psum = p;
#pragma unroll
      for (int o = 8; o >= 1; o >>= 1) psum += __shfl_xor(psum, o, 16);
      l = l * alpha + psum;
      m = m_new;
      sP[my_r][my_t] = p;
      if (my_t == 0) sRow[my_r] = alpha;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int d = tid + i * kThreads;
        if (d < a.dc) {
#pragma unroll
          for (int r = 0; r < kRows; ++r) acc[i][r] *= sRow[r];
          for (int tk = 0; tk < kTok; ++tk) {
            const float v = sK[tk][d];
#pragma unroll
            for (int r = 0; r < kRows; ++r) acc[i][r] = fmaf(sP[r][tk], v, acc[i][r]);
          }
        }
      }
    }
    __syncthreads();  // all readers of the alphas in sRow are done
    if (my_t == 0) {
      sRow[my_r] = l > 0.f ? 1.f / l : 0.f;
      if (row_ok) a.part_lse[slot * a.R + row0 + my_r] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int d = tid + i * kThreads;
      if (d < a.dc) {
        for (int r = 0; r < nrows; ++r)
          a.part_o[(slot * a.R + row0 + r) * a.dc + d] = acc[i][r] * sRow[r];
      }
    }
  });
}

}  // namespace

hipError_t launch_decode_simt(const DecodeArgs& a, int fmt, hipStream_t s) {
  const unsigned units = a.num_splits > 0 ? (unsigned)(a.B * a.num_splits) : (unsigned)a.workers;
  const dim3 grid(units, (a.R + kRows - 1) / kRows);
  switch (fmt) {
    case kF32: decode_simt_kernel<kF32><<<grid, kThreads, 0, s>>>(a); break;
    case kBF16: decode_simt_kernel<kBF16><<<grid, kThreads, 0, s>>>(a); break;
    case kFP4: decode_simt_kernel<kFP4><<<grid, kThreads, 0, s>>>(a); break;
    default: decode_simt_kernel<kFP8><<<grid, kThreads, 0, s>>>(a); break;
  }
  return hipGetLastError();
}

}  // namespace mla
