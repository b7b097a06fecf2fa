// Dynamically scheduled split-KV paged MLA decode on the CDNA4 matrix cores
// (bf16 cache, balanced split), and the merge of its partial results.
//
// The arithmetic per tile is the static kernel's (decode_mfma.hip): 32 cached
// tokens staged in LDS, S^T = Tile . Q^T and O += P . Tile[:, :d_c] on
// v_mfma_f32_16x16x32_bf16, online softmax in the base-2 domain.  What
// differs is who computes which tile.  A static split gives every worker an
// equal share, but the chip does not serve the workers equally fast (on
// MI355X the workgroups of some XCDs finish tens of microseconds after the
// others, and which ones changes from run to run).  Here the balanced plan
// (schedule.h) only decides which sequences a worker visits; the tiles of a
// sequence are handed out at run time, kDynClaimTiles at a time, from a
// per-sequence counter, to whichever of its visitors asks next, and a worker
// whose planned sequences are used up steals into the sequence with the
// most unclaimed tiles.  Every visit that computed at least one tile writes
// one normalised partial with its log-sum-exp, and the merge kernel combines
// the visits of each sequence (the log-sum-exp rule of combine.hip).
//
// Per-sequence counters (the workspace's counter region, zero between calls):
//   claimed   chunks handed out by the counter, times kDynClaimTiles
//   permits   steal visits admitted (at most kDynStealParts count)
//   pcount    parts of the last call, for the merge kernel
// The planned visitors of sequence b are the workers whose plan ranges
// overlap its tiles; visitor k (in plan order) starts with chunk k and writes
// partial slot base(b) + k, with no atomic; the counter hands out the chunks
// after those of the planned visitors; a steal visit with permit p writes
// slot base(b) + nvis + p.  base(b) = b * (1 + kDynStealParts) + (the first
// planned visitor of b): the planned visitors of b are at most
// base(b + 1) - base(b) - kDynStealParts, so every sequence's slots fit below
// the next sequence's base, and workers + B * (1 + kDynStealParts) slots hold
// them all.  Every visit writes its slot: a normalised partial and its
// log-sum-exp, or a log-sum-exp of -inf if the sequence had no tile left for
// it.  The last workgroup to finish (a grid-wide exit counter) sets pcount =
// planned visitors + admitted steals and zeroes the other counters, so the
// next call, eager or replayed from a graph, starts from zero without a
// clearing step.
//
// Roles inside a workgroup.  Wave 0 issues the counter atomics; their results
// come back through the vector-memory counter, which the compiler tracks and
// waits on.  Waves 1..NW-1 issue the tiles' direct-to-LDS transfers, which
// are inline assembly counted by hand.  Keeping the two apart lets each wave
// wait for exactly what it needs.  Every wave computes 16 query rows.
//
// The claim pipeline.  The claim for a sequence's next chunk is issued when
// the first tile of the current chunk is issued (step s); wave 0 publishes
// the result in LDS at step s + 1 and every wave reads it at step s + 2, while
// the current chunk still has tiles to issue (kDynClaimTiles >= 4).  Only a
// short chunk (the end of a sequence) waits for its successor's claim.
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "decode_common.h"
#include "device_common.h"
#include "internal.h"
#include "schedule.h"
#include "staging_bf16.h"

namespace mla {
namespace {

using namespace mfma;

static_assert(kDynClaimTiles >= 4, "the claim pipeline needs a chunk of four tiles to hide a claim");

constexpr int kMaxSteals = 8;                        // steal visits per worker
constexpr int kMinStealTiles = 2 * kDynClaimTiles;   // unclaimed tiles that make a steal worth its start-up

struct SeqCtr {
  uint32_t claimed, unused, permits, pcount;
};

__device__ __forceinline__ uint32_t ctr_add(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ctr_load(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void ctr_store(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// First partial slot of sequence b; ts is the balanced plan (B + 2 values).
__device__ __forceinline__ int64_t first_visitor(const int32_t* ts, int B, int G, int b);
__device__ __forceinline__ int64_t part_base(const int32_t* ts, int B, int G, int b) {
  return (int64_t)b * (1 + kDynStealParts) + first_visitor(ts, B, G, b);
}

// The planned visitors of sequence b: the workers whose plan ranges overlap
// its real tiles, first_visitor(b) .. first_visitor(b) + planned_visitors(b) - 1.
__device__ __forceinline__ int64_t first_visitor(const int32_t* ts, int B, int G, int b) {
  const int64_t N = ts[B];
  const int64_t first = ts[b] + plan_lead(ts[b], ts[b + 1], ts[B + 1]);
  return N > 0 ? worker_of_tile(min(first, N - 1), N, G) : 0;
}

// Workers with a non-empty plan range among workers 0 .. x - 1: all of them
// when there are at least as many positions as workers, else floor(x N / G)
// (each position then starts exactly one non-empty range).
__device__ __forceinline__ int64_t nonempty_workers(int64_t x, int64_t N, int64_t G) {
  return N >= G ? x : x * N / G;
}

__device__ __forceinline__ int planned_visitors(const int32_t* ts, int B, int G, int b) {
  const int64_t N = ts[B];
  const int64_t first = ts[b] + plan_lead(ts[b], ts[b + 1], ts[B + 1]);
  if (first >= ts[b + 1]) return 0;  // no real tiles
  return (int)(nonempty_workers(worker_of_tile(ts[b + 1] - 1, N, G) + 1, N, G) -
               nonempty_workers(worker_of_tile(first, N, G), N, G));
}

// Index of planned visitor g among the planned visitors of b.
__device__ __forceinline__ int visitor_index(const int32_t* ts, int B, int G, int b, int g) {
  const int64_t N = ts[B];
  return (int)(nonempty_workers(g, N, G) - nonempty_workers(first_visitor(ts, B, G, b), N, G));
}

__device__ __forceinline__ int64_t part_cap(const int32_t* ts, int B, int G, int b) {
  const int64_t end = b + 1 < B ? part_base(ts, B, G, b + 1) : (int64_t)G + (int64_t)B * (1 + kDynStealParts);
  return end - part_base(ts, B, G, b);
}

template <bool HILO, int NW>
__global__ __launch_bounds__(64 * NW) void decode_dyn_kernel(DecodeArgs a) {
  using G = Geo<kBF16>;
  constexpr int NBUF = 2;
  constexpr int NL = NW - 1;  // loader waves
  using Dma = DmaStaging<NL>;
  constexpr int M = Dma::kMinOps;  // transfers each loader wave issues per tile, at least
  static_assert(M < 64, "one tile's transfers must fit the 6-bit vector-memory counter");
  __shared__ __attribute__((aligned(16))) char tiles_mem[NBUF * G::kTileBytes];
  __shared__ int32_t s_ts[kMaxInKernelPlan + 2];
  __shared__ int32_t s_lens[kMaxInKernelPlan];
  __shared__ int32_t s_first;
  __shared__ int32_t s_sink[64];  // destination of L2 prefetch loads, never read
  // [0] claim result, [1] steal target, [2] steal permit, [3] last-exit flag
  __shared__ int32_t s_msg[4];
  lds_char* const tiles = (lds_char*)tiles_mem;
  uint32_t* const exit_ctr = a.ctr;
  SeqCtr* const ctr = reinterpret_cast<SeqCtr*>(a.ctr + 4);

  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);  // scalar: branches on it are uniform
  const int g = lane >> 4;
  const int li = lane & 15;
  const int row = wave * 16 + li;
  const bool row_ok = row < a.R;
  const bool loader = wave > 0;
  const int lw = max(wave - 1, 0);  // index among the loader waves
  const int Gw = a.workers;
  const int gw = blockIdx.x;  // worker index: workgroups in dispatch order, round-robin over the XCDs

  // Pull the block table into L2 while the plan is computed.
  {
    const int64_t lines = ((int64_t)a.B * a.max_blocks * 4 + 127) / 128;
    const int64_t first = ((int64_t)blockIdx.x * NW + uniform(wave)) * 64;
    if (first < lines)
      dma4_vaddr((const char*)a.block_table + 128 * min(first + lane, lines - 1), (lds_char*)s_sink);
  }
  if (threadIdx.x < 64) wave_plan(a.seq_lens, a.B, Gw, s_ts, s_lens, &s_first, gw);
  __syncthreads();
  if (blockIdx.x == 0)  // publish the plan for the merge kernel
    for (int i = threadIdx.x; i <= a.B + 1; i += 64 * NW) a.tile_start[i] = s_ts[i];

  // (LDS values are read into scalar registers: the whole schedule is uniform
  // over the workgroup, and the page lookups must stay scalar loads.)
  const int64_t N = uniform(s_ts[a.B]);
  const int64_t tb = worker_tile_begin(gw, N, Gw), te = worker_tile_begin(gw + 1, N, Gw);
  const int32_t lead_c = uniform(s_ts[a.B + 1]);
  int vb = tb < te ? uniform(s_first) : a.B;  // next planned sequence to consider
  int steals = 0;
  Dma dma;
  dma.init();

  for (;;) {
    // ---- the next visit: a planned sequence, else a steal ----
    int b = -1;
    while (vb < a.B) {
      const int64_t t0 = uniform(s_ts[vb]), t1 = uniform(s_ts[vb + 1]);
      if (t0 >= te) break;
      const int64_t f = t0 + plan_lead(t0, t1, lead_c);
      const bool overlap = max(tb, f) < min(te, t1);
      ++vb;
      if (overlap) {
        b = vb - 1;
        break;
      }
    }
    wait_vmcnt_lgkm0<0>();
    lds_barrier();  // the previous visit's readers of the ring and of s_msg are done
    int permit = -1;
    if (b < 0) {
      if (steals >= kMaxSteals) break;
      if (wave == 0) {
        // The sequence with the most unclaimed tiles that still admits a visit.
        uint64_t key = 0;
        for (int i = lane; i < a.B; i += 64) {
          const uint32_t nt_i = (uint32_t)(s_lens[i] + kTile - 1) / kTile;
          const uint32_t cl = ctr_load(&ctr[i].claimed) + (uint32_t)planned_visitors(s_ts, a.B, Gw, i) * kDynClaimTiles;
          const uint32_t pm = ctr_load(&ctr[i].permits);
          const uint32_t rem = cl < nt_i ? nt_i - cl : 0u;
          const uint64_t k = pm < (uint32_t)kDynStealParts && rem > 0 ? ((uint64_t)rem << 32) | (uint32_t)i : 0;
          key = k > key ? k : key;
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
          const uint64_t o = __shfl_xor(key, off);
          key = o > key ? o : key;
        }
        if (lane == 0) {
          int tgt = -1, p = -1;
          if ((key >> 32) >= (uint64_t)kMinStealTiles) {
            const int cand = (int)(uint32_t)key;
            p = (int)ctr_add(&ctr[cand].permits, 1);
            tgt = p < kDynStealParts ? cand : -1;
          }
          s_msg[1] = tgt;
          s_msg[2] = p;
        }
      }
      wait_lgkm0();
      lds_barrier();
      b = uniform(s_msg[1]);
      if (b < 0) break;
      permit = uniform(s_msg[2]);
      ++steals;
    }
    b = uniform(b);
    const int L = uniform(s_lens[b]);
    const int nt = uniform((L + kTile - 1) / kTile);
    // The planned visitors of b take chunks 0 .. nvis - 1 without a claim (the
    // first chunk of visitor k is chunk k) and the partial slots base(b) + k;
    // the counter hands out the chunks after them, and a steal visit writes
    // slot base(b) + nvis + its permit.
    const int nvis = uniform(planned_visitors(s_ts, a.B, Gw, b));
    const int claim_base = nvis * kDynClaimTiles;
    const int slot_k = permit < 0 ? uniform(visitor_index(s_ts, a.B, Gw, b, gw)) : nvis + permit;
    const int64_t slot = part_base(s_ts, a.B, Gw, b) + slot_k;
    const bool slot_ok = slot_k < part_cap(s_ts, a.B, Gw, b);
    int c0 = permit < 0 ? slot_k * kDynClaimTiles : nt;
    if (c0 >= nt) {  // no chunk of its own: claim one, waited for
      if (threadIdx.x == 0) s_msg[0] = claim_base + (int)ctr_add(&ctr[b].claimed, kDynClaimTiles);
      wait_lgkm0();
      lds_barrier();
      c0 = uniform(s_msg[0]);
    }
    if (c0 >= nt) {  // nothing left: the visit's slot says so
      if (slot_ok && g == 0 && row_ok) a.part_lse[slot * a.R + row] = -INFINITY;
      continue;
    }

    // ---- queries in the B-operand layout (as the static kernel) ----
    bf16x8 qh[G::kKs], ql[HILO ? G::kKs : 1];
    {
      const int64_t qoff = ((int64_t)b * a.R + (row_ok ? row : 0)) * G::kVals + 8 * g;
      auto put = [&](int ks, const float (&x)[8]) __attribute__((always_inline)) {
        uint32_t hw[4], lwd[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v0 = row_ok ? x[2 * i] : 0.f, v1 = row_ok ? x[2 * i + 1] : 0.f;
          if constexpr (HILO) split_bf16x2(v0, v1, hw[i], lwd[i]);
          else hw[i] = bf16x2_bits(v0, v1);
        }
        qh[ks] = __builtin_bit_cast(bf16x8, u32x4{hw[0], hw[1], hw[2], hw[3]});
        if constexpr (HILO) ql[ks] = __builtin_bit_cast(bf16x8, u32x4{lwd[0], lwd[1], lwd[2], lwd[3]});
      };
      if (uniform(a.q_f32)) {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(a.q_abs) + qoff);
        float4 raw[G::kKs][2];
#pragma unroll
        for (int ks = 0; ks < G::kKs; ++ks) {
          raw[ks][0] = p[8 * ks];
          raw[ks][1] = p[8 * ks + 1];
        }
#pragma unroll
        for (int ks = 0; ks < G::kKs; ++ks) {
          const float4 u = raw[ks][0], w = raw[ks][1];
          const float x[8] = {u.x, u.y, u.z, u.w, w.x, w.y, w.z, w.w};
          put(ks, x);
        }
      } else {
        const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q_abs) + qoff);
        uint4 raw[G::kKs];
#pragma unroll
        for (int ks = 0; ks < G::kKs; ++ks) raw[ks] = p[4 * ks];
#pragma unroll
        for (int ks = 0; ks < G::kKs; ++ks) {
          const uint32_t uw[4] = {raw[ks].x, raw[ks].y, raw[ks].z, raw[ks].w};
          float x[8];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            x[2 * i] = bf16_bits_to_f32(uw[i] & 0xffffu);
            x[2 * i + 1] = bf16_bits_to_f32(uw[i] >> 16);
          }
          put(ks, x);
        }
      }
    }
#pragma unroll
    for (int ks = 0; ks < G::kKs; ++ks) {
      asm volatile("" : "+a"(qh[ks]));
      if constexpr (HILO) asm volatile("" : "+a"(ql[ks]));
    }

    // ---- tile stream state (uniform) ----
    const const_i32_ptr bt = (const_i32_ptr)(a.block_table) + (int64_t)b * a.max_blocks;
    int cur_hi = uniform(min(c0 + kDynClaimTiles, nt));
    int nxt_lo = 0, nxt_hi = 0;
    bool have_nxt = false, exhausted = false;
    int claim_age = -1;  // steps since the claim in flight was issued; -1: none
    int iss = c0;        // next sequence tile to issue; -1: not known yet
    bool iss_first = true;  // `iss` is the first tile of a claimed chunk
    int n_issued = 0;
    int buf_t0 = 0, buf_t1 = 0;  // sequence tile held by ring buffer 0 / 1
    uint32_t claim_res = 0;  // wave 0: the claim in flight
    TilePages pg_next{};
    if (loader) pg_next = tile_pages(a, bt, uniform(iss) * kTile, L);

    // (The state updates below are written without branches on purpose:
    // conditional stores to different flags get merged by the optimiser into
    // a store through a selected address, which moves the flags to private
    // memory, and every reload of them would then wait for all transfers in
    // flight.)
    auto apply_claim = [&](int c) __attribute__((always_inline)) {
      c = uniform(c) + claim_base;
      const bool got = c < nt;  // a claim is only in flight while not exhausted
      exhausted = !got;
      have_nxt = got;
      nxt_lo = c;
      nxt_hi = uniform(min(c + kDynClaimTiles, nt));
      claim_age = -1;
      const bool resume = iss < 0 && got;  // the stream was waiting for this chunk
      iss = resume ? nxt_lo : iss;
      cur_hi = resume ? nxt_hi : cur_hi;
      have_nxt = have_nxt && !resume;
      iss_first = resume || iss_first;
      if (resume && loader) pg_next = tile_pages(a, bt, uniform(iss) * kTile, L);
    };
    // Issue tile `iss` into ring buffer `slot`; start the next claim if it is
    // the first tile of a claimed chunk; advance and look up the next pages.
    auto issue = [&](int slot) __attribute__((always_inline)) {
      if (loader) {
        const TilePages tp{uniform(pg_next.tt0), uniform(pg_next.pg0), uniform(pg_next.pg1)};
        dma.load_compact(tile_src(a, tp, L), tiles + slot * G::kTileBytes, lw);
      }
      buf_t1 = slot ? iss : buf_t1;
      buf_t0 = slot ? buf_t0 : iss;
      ++n_issued;
      const bool claim = iss_first && !exhausted && claim_age < 0;
      if (claim && threadIdx.x == 0) claim_res = ctr_add(&ctr[b].claimed, kDynClaimTiles);
      claim_age = claim ? 0 : claim_age;
      ++iss;
      const bool end = iss >= cur_hi;
      const bool sw = end && have_nxt;
      iss = sw ? nxt_lo : (end ? -1 : iss);
      cur_hi = sw ? nxt_hi : cur_hi;
      have_nxt = have_nxt && !sw;
      iss_first = sw;
      if (iss >= 0 && loader) pg_next = tile_pages(a, bt, uniform(iss) * kTile, L);
    };

    // Prologue: the chunk's first tile (and second, if it has one); a rolled
    // loop, so that the transfer code is not inlined once more.
#pragma unroll 1
    for (int k = 0; k < NBUF && iss >= 0; ++k) issue(k);
    claim_age = claim_age == 0 ? 1 : claim_age;  // the prologue counts as step -1

    const int j_q = row_ok ? row / a.H : 0;
    const int last_visible = L - a.Sq + j_q;
    f32x4 acc[G::kDb];
#pragma unroll
    for (int d = 0; d < G::kDb; ++d) acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, lsum = 0.f;

    // One pipeline step before computing visit tile `it`: the buffer of tile
    // it - 1 is free once every wave is past barrier A; tile it + 1 is issued
    // into it; the loaders wait for their part of tile it; barrier B.
    auto step = [&](int it) __attribute__((always_inline)) {
      wait_lgkm0();
      lds_barrier();  // A
      if (claim_age >= 2) apply_claim(s_msg[0]);
      if (n_issued == it + 1) {
        if (iss < 0 && claim_age == 1) {  // the stream needs the claim in flight now
          if (threadIdx.x == 0) s_msg[0] = (int)claim_res;
          wait_lgkm0();
          lds_barrier();
          apply_claim(s_msg[0]);
        }
        if (iss >= 0) issue((it + 1) & 1);
      }
      // The loaders wait for their part of tile it and for the page lookups
      // just issued (the compute's LDS reads are counted by the same lgkm
      // counter, which the compiler can only use at zero while scalar loads
      // are in flight).
      if (loader) {
        if (n_issued > it + 1) wait_vmcnt_lgkm0<M>();
        else wait_vmcnt_lgkm0<0>();
      }
      if (claim_age == 1 && threadIdx.x == 0) s_msg[0] = (int)claim_res;  // published, read at step it + 1
      wait_lgkm0();
      lds_barrier();  // B
      if (claim_age >= 0) ++claim_age;
    };

    constexpr float kHeadroom = 64.f;
    auto tile = [&](int it, auto rescale_tag) __attribute__((always_inline)) -> bool {
      constexpr bool kRescale = decltype(rescale_tag)::value;
      const lds_char* buf = tiles + (it & 1) * G::kTileBytes;
      const int tt0 = uniform((it & 1) ? buf_t1 : buf_t0) * kTile;

      constexpr int kQkAhead = HILO ? 2 : 3;
      f32x4 sc[2][2];
#pragma unroll
      for (int tb2 = 0; tb2 < 2; ++tb2) sc[tb2][0] = sc[tb2][1] = f32x4{0.f, 0.f, 0.f, 0.f};
      const lds_char* lat_base[2][2];
      const lds_char* rope_base[2][2];
#pragma unroll
      for (int tb2 = 0; tb2 < 2; ++tb2) {
        const int tok = tb2 * 16 + li;
        const int xs = swz(tok);
        const int flip = 64 * (xs >> 2);
        const lds_char* bl = buf + tok * G::kLatRow + 16 * (g ^ (xs & 3));
        const lds_char* br = buf + G::kRopeBase + tok * G::kRopeRow + 16 * (g ^ (xs & 3));
        lat_base[tb2][0] = bl + flip;
        lat_base[tb2][1] = bl - flip;
        rope_base[tb2][0] = br + flip;
        rope_base[tb2][1] = br - flip;
      }
      auto tile_a = [&](int ks, int tb2) {
        const lds_char* p = ks < G::kKsLat ? lat_base[tb2][ks & 1] + 64 * ks
                                           : rope_base[tb2][ks & 1] + 64 * (ks - G::kKsLat);
        return *(const lds_bf16x8*)p;
      };
      bf16x8 ta[kQkAhead][2];
#pragma unroll
      for (int k = 0; k < kQkAhead; ++k) {
        ta[k][0] = tile_a(k, 0);
        ta[k][1] = tile_a(k, 1);
      }
#pragma unroll
      for (int ks = 0; ks < G::kKs; ++ks) {
        const bf16x8 a0 = ta[ks % kQkAhead][0], a1 = ta[ks % kQkAhead][1];
        if (ks + kQkAhead < G::kKs) {
          ta[ks % kQkAhead][0] = tile_a(ks + kQkAhead, 0);
          ta[ks % kQkAhead][1] = tile_a(ks + kQkAhead, 1);
        }
        f32x4& c0r = sc[0][ks & 1];
        f32x4& c1r = sc[1][ks & 1];
        c0r = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qh[ks], c0r, 0, 0, 0);
        c1r = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qh[ks], c1r, 0, 0, 0);
        if constexpr (HILO) {
          c0r = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, ql[ks], c0r, 0, 0, 0);
          c1r = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, ql[ks], c1r, 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      const f32x4 s[2] = {sc[0][0] + sc[0][1], sc[1][0] + sc[1][1]};

      float sv[2][4];
      float mx = -INFINITY;
#pragma unroll
      for (int tb2 = 0; tb2 < 2; ++tb2)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = tt0 + tb2 * 16 + 4 * g + i;
          const bool ok = row_ok && t <= last_visible;  // last_visible < L
          sv[tb2][i] = ok ? s[tb2][i] * a.scale_log2 : -INFINITY;
          mx = fmaxf(mx, sv[tb2][i]);
        }
      mx = max_over_rows(mx);
      if constexpr (kRescale) {
        const bool raise = mx > m + 8.f;
        if (__any(raise)) {
          const float m_new = raise ? mx : m;
          const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m - m_new);
          lsum *= alpha;
          m = m_new;
          float al[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * g + i);
#pragma unroll
          for (int d = 0; d < G::kDb; ++d)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[d][i] *= al[i];
        }
      } else {
        if (__any(m != -INFINITY && mx > m + kHeadroom)) return false;
        m = m == -INFINITY ? mx : m;
      }
      float psum = 0.f;
      uint32_t pk[4], pl[4];
#pragma unroll
      for (int tb2 = 0; tb2 < 2; ++tb2)
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          const float e0 = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv[tb2][i] - m);
          const float e1 = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv[tb2][i + 1] - m);
          psum += e0 + e1;
          if constexpr (HILO) split_bf16x2(e0, e1, pk[2 * tb2 + i / 2], pl[2 * tb2 + i / 2]);
          else pk[2 * tb2 + i / 2] = bf16x2_bits(e0, e1);
        }
      psum = sum_over_rows(psum);
      lsum += psum;
      const bf16x8 pa = __builtin_bit_cast(bf16x8, make_uint4(pk[0], pk[1], pk[2], pk[3]));
      bf16x8 pa_lo = pa;
      if constexpr (HILO) pa_lo = __builtin_bit_cast(bf16x8, make_uint4(pl[0], pl[1], pl[2], pl[3]));

      const lds_char* vbase[2][4];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int tok = 16 * half + 4 * g + (li >> 2);
        const int xs = swz(tok);
        const int h = (li & 3) >> 1;
        const lds_char* b0 = buf + tok * G::kLatRow + 16 * (h ^ (xs & 1)) + 8 * (li & 1);
#pragma unroll
        for (int r = 0; r < 4; ++r) vbase[half][r] = b0 + 32 * (r ^ (xs >> 1));
      }
      auto tile_v = [&](int d) {
        const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vbase[0][d & 3] + 128 * (d >> 2)));
        const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vbase[1][d & 3] + 128 * (d >> 2)));
        return __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
      };
      constexpr int kPrefetch = HILO ? 4 : 8;
      bf16x8 vq[kPrefetch];
#pragma unroll
      for (int d = 0; d < kPrefetch; ++d) vq[d] = tile_v(d);
#pragma unroll
      for (int d = 0; d < G::kDb; ++d) {
        const bf16x8 vb2 = vq[d % kPrefetch];
        if (d + kPrefetch < G::kDb) vq[d % kPrefetch] = tile_v(d + kPrefetch);
        acc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vb2, acc[d], 0, 0, 0);
        if constexpr (HILO) acc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_lo, vb2, acc[d], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      return true;
    };

    int it = 0;
    for (; it < n_issued; ++it) {
      step(it);
      if (!tile(it, std::false_type{})) break;
    }
    if (it < n_issued) {  // tile `it` is synchronised but not yet computed
      tile(it, std::true_type{});
      for (++it; it < n_issued; ++it) {
        step(it);
        tile(it, std::true_type{});
      }
    }

    // ---- the visit's partial: normalised rows and their log-sum-exp ----
    if (slot_ok) {
      const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
      float inv_r[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) inv_r[i] = __shfl(inv, 4 * g + i);
      if (g == 0 && row_ok) a.part_lse[slot * a.R + row] = lsum > 0.f ? (m + log2f(lsum)) * kLn2 : -INFINITY;
      const int row_blocks = (a.R + 15) / 16;
      if (wave < row_blocks && wave * 16 + 4 * g < a.R) {
        float* dst = a.part_o + ((slot * row_blocks + wave) * G::kDb * 64 + lane) * 4;
#pragma unroll
        for (int d = 0; d < G::kDb; ++d)
          *reinterpret_cast<float4*>(dst + 256 * d) =
              make_float4(acc[d][0] * inv_r[0], acc[d][1] * inv_r[1], acc[d][2] * inv_r[2], acc[d][3] * inv_r[3]);
      }
    }
  }

  // ---- exit: the last workgroup resets the counters for the next call ----
  wait_vmcnt_lgkm0<0>();
  __syncthreads();
  if (threadIdx.x == 0) {
    // Relaxed: every counter operation of this workgroup was an atomic whose
    // result has come back, so it has been performed where every workgroup
    // sees it; no other data passes between workgroups in this kernel (the
    // partials reach the merge kernel through the kernel boundary).  An
    // acquire-release here would write back and invalidate the XCD's L2 at
    // every workgroup's exit, under the workgroups still streaming.
    const uint32_t prev = ctr_add(exit_ctr, 1u);
    s_msg[3] = prev == gridDim.x - 1 ? 1 : 0;
  }
  __syncthreads();
  if (s_msg[3]) {
    for (int i = threadIdx.x; i < a.B; i += 64 * NW) {
      const uint32_t pm = ctr_load(&ctr[i].permits);
      ctr_store(&ctr[i].pcount, (uint32_t)planned_visitors(s_ts, a.B, Gw, i) + min(pm, (uint32_t)kDynStealParts));
      ctr_store(&ctr[i].claimed, 0u);
      ctr_store(&ctr[i].permits, 0u);
    }
    if (threadIdx.x == 0) ctr_store(exit_ctr, 0u);
  }
}

// ---------------------------------------------------------------- merge --
//
// One workgroup per (sequence, 16-row block, DW column blocks of 16).  The
// sequence's P parts are the slots base(b) + [0, P) (P = pcount).  Work items
// are (part, column block) pairs; wave w takes items w, w + 4, ..., and lane
// l of a wave owns column 16d + l%16 of rows 16rb + 4(l/16) + i, i = 0..3 (one
// float4 of a partial in the tiled layout).  All the workgroup's partial
// loads and log-sum-exp loads are issued before the first weight is needed,
// so a batch costs one memory round trip; per-row maximum and sum come from
// the log-sum-exps in LDS.
constexpr int kMergeThreads = 256;
constexpr int kMergeWaves = kMergeThreads / 64;
constexpr int kMergeBatch = 32;   // items in flight per lane
constexpr int kMergeMaxParts = kMfmaWorkersBf16 + 2 * (1 + kDynStealParts) + 8;

template <int DW>
__global__ __launch_bounds__(kMergeThreads) void combine_dyn_kernel(DecodeArgs a) {
  __shared__ float s_lse[kMergeMaxParts][16];
  __shared__ float s_red[2][kMergeThreads];
  __shared__ float s_m[16], s_z[16];
  __shared__ float4 s_acc[kMergeWaves][DW][64];
  const int b = blockIdx.x, rb = blockIdx.y;
  const int d0 = blockIdx.z * DW;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4;
  const int row_blocks = (a.R + 15) / 16;
  const int kdb = a.dc / 16;
  const SeqCtr* ctr = reinterpret_cast<const SeqCtr*>(a.ctr + 4);
  const int64_t base = part_base(a.tile_start, a.B, a.workers, b);
  const int P = (int)min(min((int64_t)ctr_load(&ctr[b].pcount), part_cap(a.tile_start, a.B, a.workers, b)),
                         (int64_t)kMergeMaxParts);
  const bool lane_rows = 16 * rb + 4 * g < a.R;  // lanes holding only padding rows load nothing
  const int64_t slot_stride = (int64_t)row_blocks * kdb * 256;
  const float* po = a.part_o + (int64_t)rb * kdb * 256 + lane * 4;
  const int items = P * DW;

  // First batch of partial rows, requested before the log-sum-exps.
  float4 pv[kMergeBatch];
  auto load_batch = [&](int i0) {
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      const int item = i0 + wave + kMergeWaves * j;
      const int p = item / DW, dd = item % DW;
      pv[j] = item < items && lane_rows
                  ? *reinterpret_cast<const float4*>(po + (base + p) * slot_stride + (int64_t)(d0 + dd) * 256)
                  : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  load_batch(0);
  for (int k = tid; k < P * 16; k += kMergeThreads) {
    const int p = k >> 4, r = k & 15, rg = 16 * rb + r;
    s_lse[p][r] = rg < a.R ? a.part_lse[(base + p) * a.R + rg] : -INFINITY;
  }
  __syncthreads();
  // Per-row maximum, then sum of e^(lse - max): thread t takes row t % 16.
  const int rr = tid & 15;
  float pm = -INFINITY;
  for (int p = tid >> 4; p < P; p += kMergeThreads / 16) pm = fmaxf(pm, s_lse[p][rr]);
  s_red[0][tid] = pm;
  __syncthreads();
  if (tid < 16) {
    float mm = -INFINITY;
    for (int k = 0; k < kMergeThreads / 16; ++k) mm = fmaxf(mm, s_red[0][tid + 16 * k]);
    s_m[tid] = mm;
  }
  __syncthreads();
  const float mr = s_m[rr];
  float pz = 0.f;
  if (mr != -INFINITY)
    for (int p = tid >> 4; p < P; p += kMergeThreads / 16) {
      const float l = s_lse[p][rr];
      pz += l == -INFINITY ? 0.f : __expf(l - mr);
    }
  s_red[1][tid] = pz;
  __syncthreads();
  if (tid < 16) {
    float z = 0.f;
    for (int k = 0; k < kMergeThreads / 16; ++k) z += s_red[1][tid + 16 * k];
    s_z[tid] = z;
    const int r = 16 * rb + tid;
    if (a.lse && blockIdx.z == 0 && r < a.R) a.lse[(int64_t)b * a.R + r] = s_m[tid] == -INFINITY ? -INFINITY : s_m[tid] + logf(z);
  }
  __syncthreads();
  float mrow[4], izrow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    mrow[i] = s_m[4 * g + i];
    izrow[i] = s_z[4 * g + i] > 0.f ? 1.f / s_z[4 * g + i] : 0.f;
  }
  float4 acc[DW];
#pragma unroll
  for (int dd = 0; dd < DW; ++dd) acc[dd] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int i0 = 0; i0 < items; i0 += kMergeWaves * kMergeBatch) {
    if (i0 > 0) load_batch(i0);
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      const int item = i0 + wave + kMergeWaves * j;
      if (item >= items) break;
      const int p = item / DW, dd = item % DW;
      const float v[4] = {pv[j].x, pv[j].y, pv[j].z, pv[j].w};
      float r[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float l = s_lse[p][4 * g + i];
        const float w = l == -INFINITY || mrow[i] == -INFINITY ? 0.f : __expf(l - mrow[i]) * izrow[i];
        r[i] = w != 0.f ? w * v[i] : 0.f;  // zero-weight parts are selected away, never multiplied
      }
#pragma unroll
      for (int x = 0; x < DW; ++x)
        if (x == dd) {
          acc[x].x += r[0];
          acc[x].y += r[1];
          acc[x].z += r[2];
          acc[x].w += r[3];
        }
    }
  }
#pragma unroll
  for (int dd = 0; dd < DW; ++dd) s_acc[wave][dd][lane] = acc[dd];
  __syncthreads();
  for (int k = tid; k < DW * 64; k += kMergeThreads) {
    const int dd = k >> 6, l = k & 63, gg = l >> 4, c = l & 15;
    float4 s = s_acc[0][dd][l];
#pragma unroll
    for (int w = 1; w < kMergeWaves; ++w) {
      const float4 o = s_acc[w][dd][l];
      s.x += o.x;
      s.y += o.y;
      s.z += o.z;
      s.w += o.w;
    }
    const float v[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * rb + 4 * gg + i;
      if (r < a.R) a.o[((int64_t)b * a.R + r) * a.dc + 16 * (d0 + dd) + c] = v[i];
    }
  }
}

// One to four waves (up to 64 query rows): more would leave too few
// registers per wave for the queries and the accumulators.
template <bool HILO>
hipError_t launch_dyn_nw(const DecodeArgs& a, int nw, hipStream_t s) {
  const unsigned grid = (unsigned)a.workers;
  switch (nw) {
    case 2: decode_dyn_kernel<HILO, 2><<<grid, 128, 0, s>>>(a); break;
    case 3: decode_dyn_kernel<HILO, 3><<<grid, 192, 0, s>>>(a); break;
    case 4: decode_dyn_kernel<HILO, 4><<<grid, 256, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

bool decode_dyn_supported(int fmt, int dc, int dr, int R, int q_f32, int num_splits, int B) {
  const int nw = std::max(2, (R + 15) / 16);
  (void)q_f32;
  return fmt == kBF16 && dc == 512 && dr == kDr && num_splits == 0 && B >= 1 && B <= kDynMaxB && nw <= 4;
}

hipError_t launch_combine_dyn(const DecodeArgs& a, hipStream_t s) {
  // Column blocks per workgroup from the parts a sequence is expected to
  // have: many parts share one column block over four waves; few parts take
  // several column blocks per workgroup.
  const int kdb = a.dc / 16;
  const int64_t parts = ((int64_t)a.workers + a.B - 1) / a.B + 1;
  const int dw = parts >= 32 ? 1 : parts >= 8 ? 2 : 4;
  const dim3 grid((unsigned)a.B, (unsigned)((a.R + 15) / 16), (unsigned)(kdb / dw));
  switch (dw) {
    case 1: combine_dyn_kernel<1><<<grid, kMergeThreads, 0, s>>>(a); break;
    case 2: combine_dyn_kernel<2><<<grid, kMergeThreads, 0, s>>>(a); break;
    default: combine_dyn_kernel<4><<<grid, kMergeThreads, 0, s>>>(a); break;
  }
  return hipGetLastError();
}

hipError_t launch_decode_dyn(const DecodeArgs& a, hipStream_t s) {
  if (!decode_dyn_supported(kBF16, a.dc, a.dr, a.R, a.q_f32, a.num_splits, a.B) || !a.ctr ||
      a.workers != kMfmaWorkersBf16 || a.dc / 16 % 4)
    return hipErrorInvalidValue;
  const int nw = std::max(2, (a.R + 15) / 16);
  return a.q_f32 ? launch_dyn_nw<true>(a, nw, s) : launch_dyn_nw<false>(a, nw, s);
}

}  // namespace mla
