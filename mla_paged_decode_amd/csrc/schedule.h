// Split-KV work units: which token ranges of which sequences a workgroup
// handles, and which workspace slot receives each partial result.
//
// Uniform mode (num_splits = S >= 1): grid.x = B * S; workgroup x handles
// chunk s = x % S of sequence b = x / S, tokens [s*c, min((s+1)*c, L)) with
// c = ceil(L / S); its partial goes to slot x.  Every slot is written, empty
// chunks included (lse = -inf).
//
// Balanced mode (num_splits = 0): every sequence is cut into tiles of
// kPlanTile tokens; tile_start[b] is the exclusive prefix sum of tile counts
// and N = tile_start[B].  Worker g of G owns the concatenated tiles
// [g*N/G, (g+1)*N/G), which may span several sequences; its partial for
// sequence b goes to slot g + b (unique, < G + B).
#pragma once

#include "internal.h"

namespace mla {

__device__ __forceinline__ int64_t worker_tile_begin(int64_t g, int64_t N, int64_t G) {
  return g * N / G;
}

// Largest worker whose range starts at or before tile t (its range holds t).
__device__ __forceinline__ int64_t worker_of_tile(int64_t t, int64_t N, int64_t G) {
  return ((t + 1) * G - 1) / N;
}

// Largest b in [0, B] with tile_start[b] <= t.
__device__ __forceinline__ int seq_of_tile(const int32_t* ts, int B, int64_t t) {
  int lo = 0, hi = B;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (ts[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Calls f(b, L, t0, t1, slot) for each unit of this workgroup, uniformly
// across the workgroup.
template <class F>
__device__ __forceinline__ void for_each_unit(const DecodeArgs& a, F&& f) {
  if (a.num_splits > 0) {
    const int S = a.num_splits;
    const int b = blockIdx.x / S, s = blockIdx.x % S;
    const int L = max(a.seq_lens[b], 0);
    const int chunk = (L + S - 1) / S;
    const int t0 = min(L, s * chunk);
    const int t1 = min(L, t0 + chunk);
    f(b, L, t0, t1, (int64_t)blockIdx.x);
    return;
  }
  const int64_t G = a.workers, N = a.tile_start[a.B];
  const int64_t g = blockIdx.x;
  const int64_t tb = worker_tile_begin(g, N, G), te = worker_tile_begin(g + 1, N, G);
  if (tb >= te) return;
  for (int b = seq_of_tile(a.tile_start, a.B, tb); b < a.B && a.tile_start[b] < te; ++b) {
    const int64_t s0 = max(tb, (int64_t)a.tile_start[b]);
    const int64_t s1 = min(te, (int64_t)a.tile_start[b + 1]);
    if (s0 >= s1) continue;
    const int L = max(a.seq_lens[b], 0);
    const int t0 = (int)((s0 - a.tile_start[b]) * kPlanTile);
    const int t1 = (int)min((int64_t)L, (s1 - a.tile_start[b]) * kPlanTile);
    f(b, L, t0, t1, g + b);
  }
}

}  // namespace mla
