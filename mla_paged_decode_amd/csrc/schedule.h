// Split-KV work units: which token ranges of which sequences a workgroup
// handles, and which workspace slot receives each partial result.
//
// Uniform mode (num_splits = S >= 1): grid.x = B * S; workgroup x handles
// chunk s = x % S of sequence b = x / S, tokens [s*c, min((s+1)*c, L)) with
// c = ceil(L / S) rounded up to a multiple of kPlanTile; its partial goes to
// slot x.  Every slot is written, empty
// chunks included (lse = -inf).
//
// In both modes a unit starts at a multiple of kPlanTile tokens.
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

// Balanced-mode plan computed by one workgroup: ts[b] = sum over b' < b of
// ceil(max(L_b', 0) / kPlanTile), ts[B] = total, written to `ts` (LDS or
// global).  `scan` is LDS scratch of blockDim.x ints.  If lens_out is not
// null, max(lens[b], 0) is also stored there.  Contains barriers: every
// thread of the workgroup must call it.
__device__ __forceinline__ void block_plan(const int32_t* lens, int B, int32_t* ts, int32_t* scan,
                                           int32_t* lens_out = nullptr) {
  const int nt = blockDim.x, tid = threadIdx.x;
  const int per = (B + nt - 1) / nt;
  const int b0 = min(B, tid * per), b1 = min(B, b0 + per);
  int32_t sum = 0;
  for (int b = b0; b < b1; ++b) {
    const int32_t L = max(lens[b], 0);
    if (lens_out) lens_out[b] = L;
    sum += (L + kPlanTile - 1) / kPlanTile;
  }
  scan[tid] = sum;
  __syncthreads();
  for (int off = 1; off < nt; off <<= 1) {
    const int32_t v = tid >= off ? scan[tid - off] : 0;
    __syncthreads();
    scan[tid] += v;
    __syncthreads();
  }
  int32_t run = scan[tid] - sum;
  for (int b = b0; b < b1; ++b) {
    ts[b] = run;
    run += (max(lens[b], 0) + kPlanTile - 1) / kPlanTile;
  }
  if (tid == nt - 1) ts[B] = scan[tid];
  __syncthreads();
}

// One work unit: tokens [t0, t1) of sequence b (length L), partial -> slot.
struct Unit {
  int b, L, t0, t1;
  int64_t slot;
};

// Walks this workgroup's units with a single loop body at the call site:
//   UnitIter it(a); Unit u; while (it.next(a, u)) { ... }
// All lanes of the workgroup see the same sequence of units.
struct UnitIter {
  const int32_t* ts;    // tile_start[0..B] (global memory or LDS)
  const int32_t* lens;  // sequence lengths (global memory, or clamped copies in LDS)
  int b;                // next sequence to consider (balanced) / done flag (uniform)
  int64_t tb, te;       // this worker's tile range (balanced)

  __device__ __forceinline__ UnitIter(const DecodeArgs& a, const int32_t* tile_start, const int32_t* seq_lens)
      : ts(tile_start), lens(seq_lens) {
    if (a.num_splits > 0) {
      b = 0;
      tb = te = 0;
    } else {
      const int64_t G = a.workers, N = ts[a.B], g = blockIdx.x;
      tb = worker_tile_begin(g, N, G);
      te = worker_tile_begin(g + 1, N, G);
      b = tb < te ? seq_of_tile(ts, a.B, tb) : a.B;
    }
  }

  __device__ __forceinline__ bool next(const DecodeArgs& a, Unit& u) {
    if (a.num_splits > 0) {
      if (b) return false;
      b = 1;
      const int S = a.num_splits;
      u.b = blockIdx.x / S;
      const int s = blockIdx.x % S;
      u.L = max(lens[u.b], 0);
      const int chunk = ((u.L + S - 1) / S + kPlanTile - 1) / kPlanTile * kPlanTile;
      u.t0 = min(u.L, s * chunk);
      u.t1 = min(u.L, u.t0 + chunk);
      u.slot = blockIdx.x;
      return true;
    }
    for (; b < a.B && ts[b] < te; ++b) {
      const int64_t s0 = max(tb, (int64_t)ts[b]);
      const int64_t s1 = min(te, (int64_t)ts[b + 1]);
      if (s0 >= s1) continue;
      u.b = b;
      u.L = max(lens[b], 0);
      u.t0 = (int)((s0 - ts[b]) * kPlanTile);
      u.t1 = (int)min((int64_t)u.L, (s1 - ts[b]) * kPlanTile);
      u.slot = (int64_t)blockIdx.x + b;
      ++b;
      return true;
    }
    return false;
  }
};

// Calls f(b, L, t0, t1, slot) for each unit of this workgroup.
template <class F>
__device__ __forceinline__ void for_each_unit(const DecodeArgs& a, F&& f) {
  UnitIter it(a, a.tile_start, a.seq_lens);
  Unit u;
  while (it.next(a, u)) f(u.b, u.L, u.t0, u.t1, u.slot);
}

}  // namespace mla
