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

constexpr int kCombineThreads = 256;
constexpr int kMaxParts = 4096;  // partial slots one sequence can have

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
// read in parallel, reduced in LDS, and the partial rows are then summed
// with independent loads.
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
  float m = -INFINITY;
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
    const float l = ok ? a.part_lse[slot * a.R + row] : -INFINITY;
    s_w[i] = l;
    s_slot[i] = (int32_t)slot;
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
  for (int d = tid; d < a.dc; d += kCombineThreads) {
    // Partial values are loaded without waiting for the weights; slots of
    // workers that had no tiles may hold stale data and are selected away.
    float acc0 = 0.f, acc1 = 0.f, acc2 = 0.f, acc3 = 0.f;
    int64_t i = 0;
    for (; i + 4 <= n; i += 4) {
      float p[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) p[j] = a.part_o[((int64_t)s_slot[i + j] * a.R + row) * a.dc + d];
      const float w0 = s_w[i], w1 = s_w[i + 1], w2 = s_w[i + 2], w3 = s_w[i + 3];
      acc0 = fmaf(w0, w0 != 0.f ? p[0] : 0.f, acc0);
      acc1 = fmaf(w1, w1 != 0.f ? p[1] : 0.f, acc1);
      acc2 = fmaf(w2, w2 != 0.f ? p[2] : 0.f, acc2);
      acc3 = fmaf(w3, w3 != 0.f ? p[3] : 0.f, acc3);
    }
    for (; i < n; ++i) {
      const float p = a.part_o[((int64_t)s_slot[i] * a.R + row) * a.dc + d];
      const float w = s_w[i];
      acc0 = fmaf(w, w != 0.f ? p : 0.f, acc0);
    }
    a.o[out_row * a.dc + d] = ((acc0 + acc1) + (acc2 + acc3)) * inv;
  }
  if (a.lse && tid == 0) a.lse[out_row] = m + logf(z);
}

}  // namespace

hipError_t launch_plan(const DecodeArgs& a, hipStream_t s) {
  plan_kernel<<<1, kPlanThreads, 0, s>>>(a.seq_lens, a.B, a.tile_start);
  return hipGetLastError();
}

hipError_t launch_combine(const DecodeArgs& a, hipStream_t s) {
  const int64_t blocks = (int64_t)a.B * a.R;
  if (blocks == 0) return hipSuccess;
  combine_kernel<<<dim3((unsigned)blocks), kCombineThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mla
