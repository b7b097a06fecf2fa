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
// kPlanTile tokens, preceded by c virtual tiles (none for an empty sequence)
// that stand for what starting another sequence costs a worker (its queries
// are loaded and its tile stream restarts).  tile_start[b] is the exclusive
// prefix sum of these counts, N = tile_start[B] and c = tile_start[B + 1].
// Worker g of G owns the concatenated positions [g*N/G, (g+1)*N/G), which
// may span several sequences; the real tiles among them are its units, and
// its partial for sequence b goes to slot g + b (unique, < G + B).  A worker
// whose positions in b are all virtual has no unit there.  c is
// kUnitCostTiles, or 0 when, without it, every sequence would start exactly
// where a worker starts (no worker would cross into another sequence, and the
// virtual tiles would only unbalance the split).  Worker g runs on the
// workgroup given by balanced_worker().
#pragma once

#include "internal.h"

namespace mla {

// Virtual positions at the start of a sequence that spans [ts, te).
__device__ __forceinline__ int64_t plan_lead(int64_t ts, int64_t te, int32_t c) { return te > ts ? c : 0; }

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

// Whether some worker's range starts exactly at position p (0 < p < N0) of
// a plan over N0 positions and G workers: worker starts are floor(g*N0/G),
// so p is one iff the first multiple of N0 at or above p*G is below (p+1)*G.
__device__ __forceinline__ bool starts_worker(int64_t p, int64_t N0, int64_t G) {
  const uint64_t pg = (uint64_t)p * (uint64_t)G;
  const uint64_t r = pg < (1ull << 32) && N0 < (1ll << 32) ? (uint32_t)pg % (uint32_t)N0 : pg % (uint64_t)N0;
  return r == 0 || (uint64_t)N0 - r < (uint64_t)G;
}

// Balanced-mode plan computed by one workgroup for G workers: tile_start
// as described above (B + 2 values), written to `ts` (LDS or global).
// `scan` is LDS scratch of blockDim.x 64-bit values.  If lens_out is not
// null, max(lens[b], 0) is also stored there.  Contains barriers: every
// thread of the workgroup must call it.
__device__ __forceinline__ void block_plan(const int32_t* lens, int B, int G, int32_t* ts, int64_t* scan,
                                           int32_t* lens_out = nullptr) {
  const int nt = blockDim.x, tid = threadIdx.x;
  const int per = (B + nt - 1) / nt;
  const int b0 = min(B, tid * per), b1 = min(B, b0 + per);
  // Counts packed as tiles + (non-empty sequences << 32).
  auto count = [](int32_t L) -> int64_t { return L > 0 ? ((L + kPlanTile - 1) / kPlanTile) + (1ll << 32) : 0; };
  int64_t sum = 0;
  for (int b = b0; b < b1; ++b) {
    const int32_t L = max(lens[b], 0);
    if (lens_out) lens_out[b] = L;
    sum += count(L);
  }
  scan[tid] = sum;
  __syncthreads();
  for (int off = 1; off < nt; off <<= 1) {
    const int64_t v = tid >= off ? scan[tid - off] : 0;
    __syncthreads();
    scan[tid] += v;
    __syncthreads();
  }
  const int64_t total = scan[nt - 1];
  const int64_t N0 = total & 0xffffffffll;  // real tiles
  // Does any sequence start strictly inside a worker's range of the plan
  // without virtual tiles?
  bool crossing = false;
  int64_t run = scan[tid] - sum;
  for (int b = b0; b < b1; ++b) {
    const int64_t p = run & 0xffffffffll;
    if (lens[b] > 0 && p > 0) crossing |= !starts_worker(p, N0, G);
    run += count(max(lens[b], 0));
  }
  const int32_t c = __syncthreads_or(crossing) ? kUnitCostTiles : 0;
  run = scan[tid] - sum;
  for (int b = b0; b < b1; ++b) {
    ts[b] = (int32_t)((run & 0xffffffffll) + c * (run >> 32));
    run += count(max(lens[b], 0));
  }
  if (tid == nt - 1) {
    ts[B] = (int32_t)(N0 + c * (total >> 32));
    ts[B + 1] = c;
  }
  __syncthreads();
}

// Worker index of this workgroup in balanced mode (defined below).
__device__ __forceinline__ int balanced_worker(int G);

// The same plan computed by one wave, for B <= 64 * kPlanPerLane, without
// barriers: lane l handles sequences [l * per, (l + 1) * per).  Also stores
// in *first the sequence holding this workgroup's first position (the
// largest b with ts[b] <= that position).  Every lane of the wave must call
// it; the caller synchronises the workgroup afterwards.
constexpr int kPlanPerLane = kMaxInKernelPlan / 64;
__device__ __forceinline__ void wave_plan(const int32_t* lens, int B, int G, int32_t* ts, int32_t* lens_out,
                                          int32_t* first, int worker = -1) {
  const int lane = threadIdx.x & 63;
  const int per = (B + 63) / 64;
  const int b0 = lane * per;
  // The lane's lengths are loaded together (indices clamped into [0, B), the
  // extra values masked afterwards), so the plan waits one memory round trip.
  int32_t L[kPlanPerLane];
  int32_t tiles = 0, ne = 0;
#pragma unroll
  for (int i = 0; i < kPlanPerLane; ++i) L[i] = lens[min(b0 + i, B - 1)];
#pragma unroll
  for (int i = 0; i < kPlanPerLane; ++i) {
    L[i] = i < per && b0 + i < B ? max(L[i], 0) : 0;
    tiles += (L[i] + kPlanTile - 1) / kPlanTile;
    ne += L[i] > 0;
  }
  int32_t st = tiles, sn = ne;  // inclusive prefix sums over lanes
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t u = __shfl_up(st, off), v = __shfl_up(sn, off);
    if (lane >= off) {
      st += u;
      sn += v;
    }
  }
  const int32_t N0 = __shfl(st, 63), Bn = __shfl(sn, 63);
  bool crossing = false;
  int32_t p = st - tiles;
#pragma unroll
  for (int i = 0; i < kPlanPerLane; ++i) {
    if (L[i] > 0 && p > 0) crossing |= !starts_worker(p, N0, G);
    p += (L[i] + kPlanTile - 1) / kPlanTile;
  }
  const int32_t c = __any(crossing) ? kUnitCostTiles : 0;
  const int64_t N = (int64_t)N0 + (int64_t)c * Bn;
  const int64_t tb = worker_tile_begin(worker >= 0 ? worker : balanced_worker(G), N, G);
  p = st - tiles;
  int32_t q = sn - ne;
  int32_t cand = -1;
#pragma unroll
  for (int i = 0; i < kPlanPerLane; ++i) {
    const int b = b0 + i;
    if (i < per && b < B) {
      const int32_t t = p + c * q;
      ts[b] = t;
      if (lens_out) lens_out[b] = L[i];
      if (t <= tb) cand = b;
    }
    p += (L[i] + kPlanTile - 1) / kPlanTile;
    q += L[i] > 0;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) cand = max(cand, __shfl_xor(cand, off));
  if (lane == 63) {
    ts[B] = (int32_t)N;
    ts[B + 1] = c;
  }
  if (lane == 0) *first = N <= tb ? B : cand;
}

// Balanced-mode worker index of this workgroup.  Workgroups are dispatched
// round-robin over the 8 XCDs, each with its own L2, so workers are numbered
// XCD-major: the workgroups of one XCD own one contiguous run of tiles, and
// a sequence split over several of them has its queries read into one L2.
__device__ __forceinline__ int balanced_worker(int G) {
  constexpr int kXcds = 8;
  const int x = blockIdx.x;
  return G % kXcds == 0 ? (x % kXcds) * (G / kXcds) + x / kXcds : x;
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
  const int32_t* ts;    // tile_start[0..B+1] (global memory or LDS)
  const int32_t* lens;  // sequence lengths (global memory, or clamped copies in LDS)
  int b;                // next sequence to consider (balanced) / done flag (uniform)
  int g;                // worker index (balanced)
  int32_t c;            // virtual tiles at the start of each sequence (balanced)
  int64_t tb, te;       // this worker's tile range (balanced)

  // first_b >= 0: the sequence holding this worker's first position, known
  // from the plan (otherwise it is searched for).
  __device__ __forceinline__ UnitIter(const DecodeArgs& a, const int32_t* tile_start, const int32_t* seq_lens,
                                      int first_b = -1)
      : ts(tile_start), lens(seq_lens) {
    if (a.num_splits > 0) {
      b = 0;
      g = 0;
      c = 0;
      tb = te = 0;
    } else {
      g = balanced_worker(a.workers);
      c = ts[a.B + 1];
      const int64_t G = a.workers, N = ts[a.B];
      tb = worker_tile_begin(g, N, G);
      te = worker_tile_begin(g + 1, N, G);
      b = tb < te ? (first_b >= 0 ? first_b : seq_of_tile(ts, a.B, tb)) : a.B;
    }
  }

  __device__ __forceinline__ bool next(const DecodeArgs& a, Unit& u) {
    if (a.num_splits > 0) {
      if (b) return false;
      b = 1;
      const int S = a.num_splits;
      u.b = blockIdx.x / S;
      const int s = blockIdx.x % S;
      u.L = a.sparse_sq ? a.topk_width : max(lens[u.b], 0);  // sparse: slots of the index list
      const int chunk = ((u.L + S - 1) / S + kPlanTile - 1) / kPlanTile * kPlanTile;
      u.t0 = min(u.L, s * chunk);
      u.t1 = min(u.L, u.t0 + chunk);
      u.slot = blockIdx.x;
      return true;
    }
    for (; b < a.B && ts[b] < te; ++b) {
      const int64_t first = ts[b] + plan_lead(ts[b], ts[b + 1], c);  // first real tile
      const int64_t s0 = max(tb, first);
      const int64_t s1 = min(te, (int64_t)ts[b + 1]);
      if (s0 >= s1) continue;
      u.b = b;
      u.L = max(lens[b], 0);
      u.t0 = (int)((s0 - first) * kPlanTile);
      u.t1 = (int)min((int64_t)u.L, (s1 - first) * kPlanTile);
      u.slot = (int64_t)g + b;
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
