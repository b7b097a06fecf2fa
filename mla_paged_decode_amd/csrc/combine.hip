// Split-KV planning and the log-sum-exp merge of partial results.
//
// Partials over disjoint token sets s, each normalised (o_s) with its
// log-sum-exp lse_s, merge exactly into the result over their union:
//   lse = log sum_s exp(lse_s),   o = sum_s exp(lse_s - lse) * o_s.
// Parts with lse_s = -inf carry no weight; if every part is empty the row
// has no visible token and gets o = 0, lse = -inf.
#include <cmath>

#include "internal.h"
#include "schedule.h"

namespace mla {
namespace {

constexpr int kPlanThreads = 1024;

// tile_start[b] = sum over b' < b of ceil(max(L_b', 0) / kPlanTile).
__global__ __launch_bounds__(kPlanThreads) void plan_kernel(const int32_t* __restrict__ lens, int B,
                                                            int32_t* __restrict__ tile_start) {
  __shared__ int32_t s[kPlanThreads];
  const int tid = threadIdx.x;
  const int per = (B + kPlanThreads - 1) / kPlanThreads;
  const int b0 = min(B, tid * per), b1 = min(B, b0 + per);
  int32_t sum = 0;
  for (int b = b0; b < b1; ++b) sum += (max(lens[b], 0) + kPlanTile - 1) / kPlanTile;
  s[tid] = sum;
  __syncthreads();
  for (int off = 1; off < kPlanThreads; off <<= 1) {
    const int32_t v = tid >= off ? s[tid - off] : 0;
    __syncthreads();
    s[tid] += v;
    __syncthreads();
  }
  int32_t run = s[tid] - sum;
  for (int b = b0; b < b1; ++b) {
    tile_start[b] = run;
    run += (max(lens[b], 0) + kPlanTile - 1) / kPlanTile;
  }
  if (tid == kPlanThreads - 1) tile_start[B] = s[tid];
}

constexpr int kCombineThreads = 128;  // x 4 values = one 512-wide latent row per pass
constexpr int kMaxParts = 4096;       // partial slots one sequence can have
constexpr int kUnroll = 16;           // partial rows in flight per thread

__device__ __forceinline__ float block_reduce(float v, float* red, bool is_max) {
  for (int o = 32; o >= 1; o >>= 1) {
    const float u = __shfl_xor(v, o);
    v = is_max ? fmaxf(v, u) : v + u;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();  // red[] free
  if (lane == 0) red[wave] = v;
  __syncthreads();
  v = red[0];
  for (int w = 1; w < kCombineThreads / 64; ++w) v = is_max ? fmaxf(v, red[w]) : v + red[w];
  return v;
}

// One workgroup per (sequence, query row).  The slots' log-sum-exps are
// read in parallel and reduced in LDS; then each thread sums 4 consecutive
// values of the partial rows with kUnroll independent 16-byte loads in
// flight.
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(DecodeArgs a) {
  __shared__ float s_w[kMaxParts];
  __shared__ int32_t s_slot[kMaxParts];
  __shared__ float red[kCombineThreads / 64];
  const int b = blockIdx.x / a.R;
  const int row = blockIdx.x % a.R;
  const int tid = threadIdx.x;

  // Candidate parts: uniform mode, splits 0..S-1 (slot b*S + s); balanced
  // mode, workers g0..g1 (slot g + b), skipping workers with no tiles.
  int64_t g0 = 0, n = 0;
  int64_t N = 0, G = a.workers;
  if (a.num_splits > 0) {
    n = a.num_splits;
  } else {
    const int64_t ts = a.tile_start[b], te = a.tile_start[b + 1];
    N = a.tile_start[a.B];
    if (ts < te) {
      g0 = worker_of_tile(ts, N, G);
      n = worker_of_tile(te - 1, N, G) - g0 + 1;
    }
  }
  for (int64_t i = tid; i < n; i += kCombineThreads) {
    int64_t slot;
    bool ok = true;
    if (a.num_splits > 0) {
      slot = (int64_t)b * a.num_splits + i;
    } else {
      const int64_t g = g0 + i;
      ok = worker_tile_begin(g, N, G) < worker_tile_begin(g + 1, N, G);
      slot = g + b;
    }
    s_slot[i] = ok ? (int32_t)slot : -1;
  }
  __syncthreads();

  // The first kUnroll partial rows are requested before their weights are
  // known; the log-sum-exps are read meanwhile.
  const float* po = a.part_o + (int64_t)row * a.dc;
  const int64_t slot_stride = (int64_t)a.R * a.dc;
  const int d4 = tid;  // this thread's 4 values (first pass)
  const bool d_ok = d4 < a.dc / 4;
  float4 pre[kUnroll];
#pragma unroll
  for (int j = 0; j < kUnroll; ++j) {
    const int32_t sl = j < n ? s_slot[j] : -1;
    pre[j] = d_ok && sl >= 0 ? reinterpret_cast<const float4*>(po + sl * slot_stride)[d4]
                             : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float m = -INFINITY;
  for (int64_t i = tid; i < n; i += kCombineThreads) {
    const int32_t sl = s_slot[i];
    const float l = sl >= 0 ? a.part_lse[(int64_t)sl * a.R + row] : -INFINITY;
    s_w[i] = l;
    m = fmaxf(m, l);
  }
  m = block_reduce(m, red, true);
  const int64_t out_row = (int64_t)b * a.R + row;
  if (m == -INFINITY) {
    for (int d = tid; d < a.dc; d += kCombineThreads) a.o[out_row * a.dc + d] = 0.f;
    if (a.lse && tid == 0) a.lse[out_row] = -INFINITY;
    return;
  }
  float z = 0.f;
  for (int64_t i = tid; i < n; i += kCombineThreads) {
    const float w = s_w[i] == -INFINITY ? 0.f : expf(s_w[i] - m);
    s_w[i] = w;
    z += w;
  }
  z = block_reduce(z, red, false);  // also orders the s_w writes before the reads below
  const float inv = 1.f / z;
  // Rows with zero weight (no visible token in that part, or a worker
  // without tiles) are selected away, never multiplied.
  auto accumulate = [&](float4& c, float w, const float4& p) {
    const bool use = w != 0.f;
    c.x = fmaf(w, use ? p.x : 0.f, c.x);
    c.y = fmaf(w, use ? p.y : 0.f, c.y);
    c.z = fmaf(w, use ? p.z : 0.f, c.z);
    c.w = fmaf(w, use ? p.w : 0.f, c.w);
  };
  for (int dd = d4; dd < a.dc / 4; dd += kCombineThreads) {
    float4 acc[2] = {make_float4(0.f, 0.f, 0.f, 0.f), make_float4(0.f, 0.f, 0.f, 0.f)};
    int64_t i0 = 0;
    if (dd == d4) {
#pragma unroll
      for (int j = 0; j < kUnroll; ++j) accumulate(acc[j & 1], j < n ? s_w[j] : 0.f, pre[j]);
      i0 = kUnroll;
    }
    for (; i0 < n; i0 += kUnroll) {
      float4 p[kUnroll];
#pragma unroll
      for (int j = 0; j < kUnroll; ++j) {
        const int32_t sl = i0 + j < n ? s_slot[i0 + j] : -1;
        p[j] = sl >= 0 ? reinterpret_cast<const float4*>(po + sl * slot_stride)[dd] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int j = 0; j < kUnroll; ++j) accumulate(acc[j & 1], i0 + j < n ? s_w[i0 + j] : 0.f, p[j]);
    }
    reinterpret_cast<float4*>(a.o + out_row * a.dc)[dd] =
        make_float4((acc[0].x + acc[1].x) * inv, (acc[0].y + acc[1].y) * inv,
                    (acc[0].z + acc[1].z) * inv, (acc[0].w + acc[1].w) * inv);
  }
  if (a.lse && tid == 0) a.lse[out_row] = m + logf(z);
}

// Merge for the tiled partial layout of the matrix-core kernel.  One
// workgroup per (sequence, 16-row block, 4 column blocks of 16): thread t
// owns column block 4*blockIdx.z + t/64 and lane l = t%64, i.e. column
// 16d + l%16 of rows 16w + 4(l/16) + i, i = 0..3, which are one float4 of
// every partial.  Per-row maxima and sums over the parts are reduced in LDS;
// weights are computed in LDS for chunks of kChunk parts.
constexpr int kTiledThreads = 256;
constexpr int kChunk = 128;

__global__ __launch_bounds__(kTiledThreads) void combine_tiled_kernel(DecodeArgs a) {
  __shared__ int32_t s_slot[kMaxParts];
  __shared__ float s_red[kTiledThreads];
  __shared__ float s_m[16], s_z[16];
  __shared__ float s_wt[kChunk][16];
  const int b = blockIdx.x, w = blockIdx.y;
  const int tid = threadIdx.x;
  const int row_blocks = (a.R + 15) / 16;
  const int kdb = a.dc / 16;
  const int d = 4 * blockIdx.z + tid / 64;
  const int lane = tid & 63, g = lane >> 4, li = lane & 15;

  int64_t g0 = 0, n = 0;
  int64_t N = 0, G = a.workers;
  if (a.num_splits > 0) {
    n = a.num_splits;
  } else {
    const int64_t ts = a.tile_start[b], te = a.tile_start[b + 1];
    N = a.tile_start[a.B];
    if (ts < te) {
      g0 = worker_of_tile(ts, N, G);
      n = worker_of_tile(te - 1, N, G) - g0 + 1;
    }
  }
  for (int64_t i = tid; i < n; i += kTiledThreads) {
    int64_t slot;
    bool ok = true;
    if (a.num_splits > 0) {
      slot = (int64_t)b * a.num_splits + i;
    } else {
      const int64_t gg = g0 + i;
      ok = worker_tile_begin(gg, N, G) < worker_tile_begin(gg + 1, N, G);
      slot = gg + b;
    }
    s_slot[i] = ok ? (int32_t)slot : -1;
  }
  __syncthreads();

  // Per-row maximum and sum: thread t covers row t%16 and parts t/16, +16, ...
  const int rr = tid & 15, r_glob = 16 * w + rr;
  float pm = -INFINITY;
  for (int64_t i = tid >> 4; i < n; i += kTiledThreads / 16) {
    const int32_t sl = s_slot[i];
    if (sl >= 0 && r_glob < a.R) pm = fmaxf(pm, a.part_lse[(int64_t)sl * a.R + r_glob]);
  }
  s_red[tid] = pm;
  __syncthreads();
  if (tid < 16) {
    float m = -INFINITY;
    for (int k = 0; k < kTiledThreads / 16; ++k) m = fmaxf(m, s_red[tid + 16 * k]);
    s_m[tid] = m;
  }
  __syncthreads();
  float pz = 0.f;
  const float mr = s_m[rr];
  if (mr != -INFINITY)
    for (int64_t i = tid >> 4; i < n; i += kTiledThreads / 16) {
      const int32_t sl = s_slot[i];
      if (sl >= 0 && r_glob < a.R) {
        const float l = a.part_lse[(int64_t)sl * a.R + r_glob];
        pz += l == -INFINITY ? 0.f : expf(l - mr);
      }
    }
  s_red[tid] = pz;
  __syncthreads();
  if (tid < 16) {
    float z = 0.f;
    for (int k = 0; k < kTiledThreads / 16; ++k) z += s_red[tid + 16 * k];
    s_z[tid] = z;
    const int r = 16 * w + tid;
    if (a.lse && blockIdx.z == 0 && r < a.R)
      a.lse[(int64_t)b * a.R + r] = s_m[tid] == -INFINITY ? -INFINITY : s_m[tid] + logf(z);
  }
  __syncthreads();

  const float* po = a.part_o + ((int64_t)w * kdb + d) * 256 + lane * 4;
  const int64_t slot_stride = (int64_t)row_blocks * kdb * 256;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int64_t c0 = 0; c0 < n; c0 += kChunk) {
    const int64_t cn = min((int64_t)kChunk, n - c0);
    // Weights of this chunk: e^(lse - m) / z, zero for empty parts.
    for (int k = tid; k < kChunk * 16; k += kTiledThreads) {
      const int i = k >> 4, r = k & 15, rg = 16 * w + r;
      float wt = 0.f;
      if (i < cn && rg < a.R) {
        const int32_t sl = s_slot[c0 + i];
        if (sl >= 0 && s_m[r] != -INFINITY) {
          const float l = a.part_lse[(int64_t)sl * a.R + rg];
          wt = l == -INFINITY ? 0.f : expf(l - s_m[r]) / s_z[r];
        }
      }
      s_wt[i][r] = wt;
    }
    __syncthreads();
    for (int i0 = 0; i0 < cn; i0 += kUnroll) {
      float4 p[kUnroll];
#pragma unroll
      for (int j = 0; j < kUnroll; ++j) {
        const int32_t sl = i0 + j < cn ? s_slot[c0 + i0 + j] : -1;
        p[j] = sl >= 0 ? *reinterpret_cast<const float4*>(po + sl * slot_stride) : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int j = 0; j < kUnroll; ++j) {
        if (i0 + j >= cn) break;
        const float* wt = s_wt[i0 + j] + 4 * g;
        // zero-weight parts may hold stale data: select, never multiply
        acc.x = fmaf(wt[0], wt[0] != 0.f ? p[j].x : 0.f, acc.x);
        acc.y = fmaf(wt[1], wt[1] != 0.f ? p[j].y : 0.f, acc.y);
        acc.z = fmaf(wt[2], wt[2] != 0.f ? p[j].z : 0.f, acc.z);
        acc.w = fmaf(wt[3], wt[3] != 0.f ? p[j].w : 0.f, acc.w);
      }
    }
    __syncthreads();  // s_wt is rewritten by the next chunk
  }
  const float v[4] = {acc.x, acc.y, acc.z, acc.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 16 * w + 4 * g + i;
    if (r < a.R) a.o[((int64_t)b * a.R + r) * a.dc + 16 * d + li] = v[i];
  }
}

}  // namespace

hipError_t launch_plan(const DecodeArgs& a, hipStream_t s) {
  plan_kernel<<<1, kPlanThreads, 0, s>>>(a.seq_lens, a.B, a.tile_start);
  return hipGetLastError();
}

hipError_t launch_combine(const DecodeArgs& a, hipStream_t s) {
  if ((int64_t)a.B * a.R == 0) return hipSuccess;
  if (a.part_tiled) {
    if (a.dc % 64) return hipErrorInvalidValue;
    const dim3 grid((unsigned)a.B, (unsigned)((a.R + 15) / 16), (unsigned)(a.dc / 64));
    combine_tiled_kernel<<<grid, kTiledThreads, 0, s>>>(a);
  } else {
    combine_kernel<<<dim3((unsigned)((int64_t)a.B * a.R)), kCombineThreads, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace mla
