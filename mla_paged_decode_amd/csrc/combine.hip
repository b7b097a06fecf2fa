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

// One workgroup per (sequence, query row).
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(DecodeArgs a) {
  const int b = blockIdx.x / a.R;
  const int row = blockIdx.x % a.R;
  int64_t g0 = 0, g1 = -1;  // balanced: worker range; uniform: split range
  if (a.num_splits > 0) {
    g0 = 0;
    g1 = a.num_splits - 1;
  } else {
    const int64_t ts = a.tile_start[b], te = a.tile_start[b + 1];
    if (ts < te) {
      const int64_t N = a.tile_start[a.B], G = a.workers;
      g0 = worker_of_tile(ts, N, G);
      g1 = worker_of_tile(te - 1, N, G);
    }
  }
  auto slot_of = [&](int64_t g, int64_t* slot) -> bool {
    if (a.num_splits > 0) {
      *slot = (int64_t)b * a.num_splits + g;
      return true;
    }
    const int64_t N = a.tile_start[a.B], G = a.workers;
    if (worker_tile_begin(g, N, G) >= worker_tile_begin(g + 1, N, G)) return false;
    *slot = g + b;
    return true;
  };

  float M = -INFINITY;
  for (int64_t g = g0; g <= g1; ++g) {
    int64_t slot;
    if (slot_of(g, &slot)) M = fmaxf(M, a.part_lse[slot * a.R + row]);
  }
  const int64_t out_row = (int64_t)b * a.R + row;
  if (M == -INFINITY) {
    for (int d = threadIdx.x; d < a.dc; d += kCombineThreads) a.o[out_row * a.dc + d] = 0.f;
    if (a.lse && threadIdx.x == 0) a.lse[out_row] = -INFINITY;
    return;
  }
  float z = 0.f;
  float acc[2] = {0.f, 0.f};
  for (int64_t g = g0; g <= g1; ++g) {
    int64_t slot;
    if (!slot_of(g, &slot)) continue;
    const float ls = a.part_lse[slot * a.R + row];
    if (ls == -INFINITY) continue;
    const float w = expf(ls - M);
    z += w;
    const float* po = a.part_o + (slot * a.R + row) * a.dc;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int d = threadIdx.x + i * kCombineThreads;
      if (d < a.dc) acc[i] = fmaf(w, po[d], acc[i]);
    }
  }
  const float inv = 1.f / z;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int d = threadIdx.x + i * kCombineThreads;
    if (d < a.dc) a.o[out_row * a.dc + d] = acc[i] * inv;
  }
  if (a.lse && threadIdx.x == 0) a.lse[out_row] = M + logf(z);
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
