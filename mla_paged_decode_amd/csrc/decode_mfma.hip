// Split-KV paged MLA decode on the CDNA4 matrix cores (gfx950).
//
// Every head of a sequence reads the same latent row, so per tile of 32
// cached tokens the work is two dense products over one LDS-resident tile:
//   S^T [32 tok x 16 rows] = Tile [32 x (d_c+d_r)] . Q^T      (QK^T)
//   O   [16 rows x d_c]   += P [16 x 32 tok] . Tile[:, :d_c]   (PV)
// with v_mfma_f32_16x16x32_bf16.  One wave owns 16 query rows (rows are
// (query token, head) pairs), keeps its queries in registers in the MFMA
// B-operand layout, and accumulates its 16 x d_c output in registers.
//
// Operand layouts of v_mfma_f32_16x16x32_bf16 (lane l, g = l / 16):
//   A: row l%16, k = 8g..8g+7     B: column l%16, k = 8g..8g+7
//   C: column l%16, rows 4g..4g+3
// QK^T puts tokens on the A side, so the C tile of S^T gives lane l the
// scores of query row l%16 for tokens 4g..4g+3 (+16 for the second token
// block): exactly the A-operand (P) layout of PV when PV's k index runs over
// tokens {4g..4g+3, 16+4g..16+4g+3}.  PV's B operand (value column d, those 8
// tokens) is read from the token-major tile with ds_read_b64_tr_b16, whose
// 16-lane groups turn four 4-value row pieces into four column pieces.
//
// Precision: with fp32 queries each query is split q = hi + lo into two bf16
// numbers and QK^T runs twice (the cache operand is exact in bf16), which
// keeps the scores at ~16 significant bits; P is split the same way and PV
// also runs twice; all accumulation is fp32.  bf16 queries take a single pass
// with P rounded once to bf16.
//
// Tile staging.  bf16 rows go from HBM straight into LDS with 16-byte
// direct-to-LDS loads, NBUF-1 tiles ahead of the one being computed; their
// completion is tracked with explicit vmcnt waits and the hand-off between
// waves uses an LDS-only barrier, so later tiles stay in flight.  fp8 rows
// (e4m3 + e8m0 per 32 values) are loaded into registers one tile ahead and
// decoded to bf16 on the way into LDS (both conversions are exact).
//
// LDS tile layout: the latent part of the 32 rows (region A) and the RoPE
// part (region B) are stored separately, so that a region-A row is exactly
// one direct-to-LDS instruction (64 lanes x 16 B).  16-byte chunks within a
// row are XOR-swizzled by the token index so that the 16-token b128 reads of
// QK^T and the 4-token transposed reads of PV hit distinct banks.
#include <cmath>
#include <type_traits>

#include "decode_common.h"
#include "staging_bf16.h"
#include "device_common.h"
#include "internal.h"
#include "merge_fused.h"
#include "schedule.h"

namespace mla {
namespace {

using namespace mfma;

// fp8 tiles are loaded into registers, decoded to bf16 and stored to LDS.
template <int NW>
struct Fp8Staging {
  using G = Geo<kFP8>;
  static constexpr int kThreads = 64 * NW;
  static constexpr int kSrc = kTile * G::kSrcChunks;  // 16-value chunks per tile
  static constexpr int kPer = (kSrc + kThreads - 1) / kThreads;
  uint4 v[kPer];
  uint32_t s[kPer];

  __device__ __forceinline__ void load(const DecodeArgs& a, const TileSrc& ts) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int q = j * kThreads + threadIdx.x;
      const int tok = min(q / G::kSrcChunks, kTile - 1);
      const int c = q % G::kSrcChunks;
      const int kk = min(tok, ts.n - 1);
      const uint8_t* p = (const uint8_t*)(uintptr_t)((kk < ts.kb ? ts.base0 : ts.base1) + (uint64_t)(kk * (int)a.row_bytes));
      if (q < kSrc) {
        v[j] = *reinterpret_cast<const uint4*>(p + 16 * c);
        s[j] = p[G::kVals + c / 2];
      }
    }
  }

  __device__ __forceinline__ void store(lds_char* buf) const {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int q = j * kThreads + threadIdx.x;
      if (q >= kSrc) continue;
      const int tok = q / G::kSrcChunks;
      const int c = q % G::kSrcChunks;
      // 16 e4m3 values -> 16 bf16 (two LDS chunks), times 2^(E-127).
      const float scale = e8m0_to_f32(s[j]);
      const uint32_t w[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
      uint32_t o[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], false);
        const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], true);
        o[2 * i + 0] = pack_bf16(lo[0] * scale, lo[1] * scale);
        o[2 * i + 1] = pack_bf16(hi[0] * scale, hi[1] * scale);
      }
      const int c0 = 2 * c;  // first bf16 chunk of these 16 values
      lds_char* d0 = c0 < G::kLatChunks ? buf + lds_off(tok, c0, G::kLatRow)
                                        : buf + G::kRopeBase + lds_off(tok, c0 - G::kLatChunks, G::kRopeRow);
      lds_char* d1 = c0 < G::kLatChunks ? buf + lds_off(tok, c0 + 1, G::kLatRow)
                                        : buf + G::kRopeBase + lds_off(tok, c0 + 1 - G::kLatChunks, G::kRopeRow);
      *(lds_u32x4*)d0 = u32x4{o[0], o[1], o[2], o[3]};
      *(lds_u32x4*)d1 = u32x4{o[4], o[5], o[6], o[7]};
    }
  }
};

// Staging interface over the two formats.  kDepth tiles are in flight ahead
// of the one being computed: issue() starts a tile's transfer into its ring
// buffer, finish() completes it from registers (fp8), wait(n) blocks until
// this wave's part of the oldest outstanding tile has landed when n younger
// tiles have been issued after it (and all its LDS operations are done).
template <int FMT, int NW, int NBUF>
struct Staging;

// bf16: a tile's transfer is issued as soon as its ring buffer is free
// (kEarlyIssue), before waiting for the tile about to be computed, so that
// up to NBUF - 1 tiles per workgroup are in flight while it waits.
template <int NW, int NBUF>
struct Staging<kBF16, NW, NBUF> {
  static constexpr int kDepth = NBUF - 1;
  static constexpr bool kEarlyIssue = true;
  DmaStaging<NW> dma;
  __device__ __forceinline__ void init() { dma.init(); }
  __device__ __forceinline__ void issue(const DecodeArgs&, const TileSrc& ts, lds_char* buf) { dma.load(ts, buf); }
  __device__ __forceinline__ void issue_gather(const DecodeArgs& a, const Gather& gt, lds_char* buf) {
    dma.load_gather(gt, a.pool, buf);
  }
  __device__ __forceinline__ void finish(lds_char*) {}
  // Every wave issues at least kMinOps transfers per tile, so allowing
  // younger * kMinOps outstanding leaves only younger tiles in flight.
  __device__ __forceinline__ void wait(int younger) {
    constexpr int M = DmaStaging<NW>::kMinOps;
    if (younger >= 3) wait_vmcnt_lgkm0<(3 * M < 64 ? 3 * M : 0)>();
    else if (younger == 2) wait_vmcnt_lgkm0<(2 * M < 64 ? 2 * M : 0)>();
    else if (younger == 1) wait_vmcnt_lgkm0<M>();
    else wait_vmcnt_lgkm0<0>();
  }
};

template <int NW, int NBUF>
struct Staging<kFP8, NW, NBUF> {
  static_assert(NBUF == 2, "fp8 tiles are staged through registers, one ahead");
  static constexpr int kDepth = 1;
  static constexpr bool kEarlyIssue = false;
  Fp8Staging<NW> f;
  __device__ __forceinline__ void init() {}
  __device__ __forceinline__ void issue(const DecodeArgs& a, const TileSrc& ts, lds_char*) { f.load(a, ts); }
  __device__ __forceinline__ void finish(lds_char* buf) { f.store(buf); }
  __device__ __forceinline__ void wait(int) { wait_vmcnt_lgkm0<0>(); }
};

// FUSE: balanced plan computed in the kernel, with the merge done by the
// last workgroup to finish each sequence (merge_fused.h): sequences with one
// part are written to o and lse directly.
template <int FMT, bool HILO, int NW, int NBUF, bool SPARSE = false, bool FUSE = false>
__global__ __launch_bounds__(64 * NW) void decode_mfma_kernel(DecodeArgs a) {
  using G = Geo<FMT>;
  static_assert(!FUSE || (FMT == kBF16 && !SPARSE), "the fused merge is built for the dense bf16 kernel");
  __shared__ __attribute__((aligned(16))) char tiles_mem[NBUF * G::kTileBytes];
  __shared__ int32_t s_ts[kMaxInKernelPlan + 2];
  __shared__ int32_t s_lens[kMaxInKernelPlan];
  __shared__ int32_t s_first;
  __shared__ int32_t s_last[2];
  __shared__ int32_t s_sink[64];  // destination of L2 prefetch loads, never read
  lds_char* const tiles = (lds_char*)tiles_mem;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4;          // lane group
  const int li = lane & 15;         // index within the group
  const int row = wave * 16 + li;   // this lane's query row (B / P side)
  const bool row_ok = row < a.R;

  // Pull the block table into L2 while the plan is computed, so that the
  // page lookups after it hit in L2: one 4-byte load per 128-byte line,
  // spread over all workgroups.
  {
    const int64_t lines = ((int64_t)a.B * a.max_blocks * 4 + 127) / 128;
    const int64_t first = ((int64_t)blockIdx.x * NW + uniform(wave)) * 64;
    if (first < lines)
      dma4_vaddr((const char*)a.block_table + 128 * min(first + lane, lines - 1), (lds_char*)s_sink);
  }
  const int32_t* ts = a.tile_start;
  if (a.num_splits == 0 && a.plan_in_kernel) {
    if (threadIdx.x < 64) wave_plan(a.seq_lens, a.B, a.workers, s_ts, s_lens, &s_first);
    __syncthreads();
    if (blockIdx.x == 0)  // publish the plan for the merge kernel
      for (int i = threadIdx.x; i <= a.B + 1; i += 64 * NW) a.tile_start[i] = s_ts[i];
    ts = s_ts;
    if constexpr (FUSE) zero_empty_sequences(a, s_lens, a.workers);
  }
  // FUSE: sequences of this worker with several parts whose arrival is
  // counted at the end (only the first and the last unit can be such: a
  // sequence between them lies wholly in this worker's range).
  int pend0 = -1, pend1 = -1;
  using St = Staging<FMT, NW, NBUF>;
  constexpr int D = St::kDepth;
  St st;
  st.init();
  UnitIter unit_it(a, ts, ts == s_ts ? s_lens : a.seq_lens, ts == s_ts ? s_first : -1);
  // Units are walked one ahead: with early issue, the first tile of the next
  // unit is transferred while the last tile of the current one is computed,
  // so a worker's tile stream does not stall where it crosses into another
  // sequence.  `ring` is the buffer of the unit's tile 0; `pre` says whether
  // that tile is already in flight when the unit starts.
  Unit unit, nxt;
  // (uniform(): the loop is the same for every lane, and its carried values
  // must stay in scalar registers.)
  bool have = uniform(unit_it.next(a, unit));
  bool have_next = have && uniform(unit_it.next(a, nxt));
  int ring = 0;
  bool pre = false, first_unit = true;
  while (have) {
    // The unit is the same for the whole workgroup: keep it in scalar
    // registers so page lookups below are scalar loads.
    const int b = uniform(unit.b), L = uniform(unit.L), t0 = uniform(unit.t0), t1 = uniform(unit.t1);
    const int64_t slot = unit.slot;

    // Unless the unit's first tile is already in flight, its queries are
    // loaded first and its first tiles are issued after them: transfers
    // complete in order, so queries requested after the tiles would only
    // arrive with the last of them (measured: tiles issued first land later
    // too, the start-up burst then being slower).  With early issue every
    // ring buffer is free here, so kPro = NBUF tiles start at once (one more
    // than in the loop).
    const int ntiles = uniform((t1 - t0 + kTile - 1) / kTile);
    // Sparse: b is a (sequence, query token) pair whose tokens are the ones
    // its index list names; query token b % sparse_sq sees positions up to
    // L - Sq + j of sequence b / sparse_sq.
    const int sb = SPARSE ? uniform(b / a.sparse_sq) : b;
    const int sparse_limit =
        SPARSE ? uniform(max(((const_i32_ptr)a.seq_lens)[sb], 0) - a.sparse_sq + b % a.sparse_sq) : 0;
    const const_i32_ptr list = (const_i32_ptr)(a.topk) + (SPARSE ? (int64_t)b * a.topk_width : 0);
    const const_i32_ptr bt = (const_i32_ptr)(a.block_table) + (int64_t)sb * a.max_blocks;
    Gather gnext;                      // sparse: rows of the next tile to issue, looked up one tile early
    uint32_t mask_slot[2] = {0u, 0u};  // sparse: visible-slot mask of the tile in ring buffer 0 / 1
    static_assert(!SPARSE || NBUF == 2, "sparse masks are kept for a 2-deep ring");
    constexpr int kPro = St::kEarlyIssue ? NBUF : D;
    auto ring_buf = [&](int i) { return tiles + ((ring + i) % NBUF) * G::kTileBytes; };
    TilePages pages_next;  // pages of the next tile to issue, looked up one tile early
    TilePages pages_pro[kPro];
    int issued = 0;        // tiles of this unit issued so far
    if (ntiles > 0) {
      if (pre) {
        issued = 1;  // tile 0 is in flight; tile 1 follows once the ring slot is free
      } else {
        if (!first_unit) {
          wait_vmcnt_lgkm0<0>();
          lds_barrier();  // the previous unit's readers of the ring are done
        }
        if constexpr (!SPARSE) {
#pragma unroll
          for (int x = 0; x < kPro; ++x)
            if (x < ntiles) pages_pro[x] = tile_pages(a, bt, t0 + x * kTile, t1);
        }
        issued = min(kPro, ntiles);
      }
      if constexpr (!SPARSE) {
        if (issued < ntiles) pages_next = tile_pages(a, bt, t0 + issued * kTile, t1);
      }
    }
    // First tile of the next unit (pages looked up now, issued after this
    // unit's last tile).
    bool ahead = false, ahead_done = false;
    int n_t1 = 0;
    TilePages pages_ahead;
    if constexpr (St::kEarlyIssue) {
      if (have_next && ntiles > 0) {
        const int n_b = uniform(nxt.b), n_t0 = uniform(nxt.t0);
        n_t1 = uniform(nxt.t1);
        if (n_t1 > n_t0) {
          ahead = true;
          pages_ahead = tile_pages(a, (const_i32_ptr)(a.block_table) + (int64_t)n_b * a.max_blocks, n_t0, n_t1);
        }
      }
    }

    // ---- queries in the B-operand layout: column = row, k = 8g..8g+7 ----
    // Every load of the row is issued before the first conversion, so the
    // queries cost one memory round trip.  Padding rows read row 0 (always
    // in bounds) and are zeroed after the load, which keeps the loads free of
    // divergent branches; the dtype test is uniform and outside the loads.
    bf16x8 qh[G::kKs], ql[HILO ? G::kKs : 1];
    {
      const int64_t qoff = ((int64_t)b * a.R + (row_ok ? row : 0)) * G::kVals + 8 * g;
      auto put = [&](int ks, const float (&x)[8]) __attribute__((always_inline)) {
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v0 = row_ok ? x[2 * i] : 0.f, v1 = row_ok ? x[2 * i + 1] : 0.f;
          if constexpr (HILO) split_bf16x2(v0, v1, hw[i], lw[i]);
          else hw[i] = bf16x2_bits(v0, v1);
        }
        qh[ks] = __builtin_bit_cast(bf16x8, u32x4{hw[0], hw[1], hw[2], hw[3]});
        if constexpr (HILO) ql[ks] = __builtin_bit_cast(bf16x8, u32x4{lw[0], lw[1], lw[2], lw[3]});
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
    // The queries are only ever read as the MFMA B operand, which may come
    // from AGPRs: keeping them there leaves the VGPRs to tile operands.
#pragma unroll
    for (int ks = 0; ks < G::kKs; ++ks) {
      asm volatile("" : "+a"(qh[ks]));
      if constexpr (HILO) asm volatile("" : "+a"(ql[ks]));
    }
    if (ntiles > 0 && !pre) {
      if constexpr (SPARSE) {
#pragma unroll
        for (int x = 0; x < kPro; ++x)
          if (x < ntiles) {
            const Gather gx = gather_lookup(a, list, bt, t0 + x * kTile, t1, sparse_limit);
            st.issue_gather(a, gx, ring_buf(x));
            mask_slot[(ring + x) & 1] = gx.mask;
          }
        if (issued < ntiles) gnext = gather_lookup(a, list, bt, t0 + issued * kTile, t1, sparse_limit);
      } else {
#pragma unroll
        for (int x = 0; x < kPro; ++x)
          if (x < ntiles) st.issue(a, tile_src(a, pages_pro[x], t1), ring_buf(x));
      }
    }
    const int j_q = row_ok ? row / a.H : 0;
    const int last_visible = L - a.Sq + j_q;

    f32x4 acc[G::kDb];
#pragma unroll
    for (int d = 0; d < G::kDb; ++d) acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, lsum = 0.f;

    if (ntiles > 0) st.finish(ring_buf(0));  // fp8: first tile from registers to LDS

    // One pipeline step before computing tile `it`.  Early issue: once every
    // wave is done with tile it-1, start tile it+D into its buffer (unless
    // the prologue did), then wait for tile it.  Otherwise (fp8, staged
    // through registers one tile ahead): wait for tile it, then start
    // loading tile it+1 into registers.
    auto sync_issue = [&](int it) __attribute__((always_inline)) {
      const int x = it + D;
      if constexpr (St::kEarlyIssue) {
        wait_lgkm0();
        lds_barrier();  // everyone finished tile it-1: its buffer is free
        if (issued <= x && issued < ntiles) {
          if constexpr (SPARSE) {
            st.issue_gather(a, gnext, ring_buf(issued));
            mask_slot[(ring + issued) & 1] = gnext.mask;
            ++issued;
            if (issued < ntiles) gnext = gather_lookup(a, list, bt, t0 + issued * kTile, t1, sparse_limit);
          } else {
            st.issue(a, tile_src(a, pages_next, t1), ring_buf(issued));
            ++issued;
            if (issued < ntiles) pages_next = tile_pages(a, bt, t0 + issued * kTile, t1);
          }
        } else if (ahead && !ahead_done && issued <= x) {
          st.issue(a, tile_src(a, pages_ahead, n_t1), ring_buf(ntiles));
          ahead_done = true;
        }
        st.wait(issued - 1 - it + (ahead_done ? 1 : 0));  // this wave's part of tile `it` landed
        lds_barrier();                                    // everyone's did
      } else {
        st.wait(min(D - 1, ntiles - 1 - it));
        lds_barrier();  // everyone's part of tile `it` landed; everyone finished tile it-1
        if (x < ntiles) {
          st.issue(a, tile_src(a, pages_next, t1), ring_buf(x));
          if (x + 1 < ntiles) pages_next = tile_pages(a, bt, t0 + (x + 1) * kTile, t1);
        }
      }
    };
    auto finish_next = [&](int it) __attribute__((always_inline)) {
      if (D == 1 && it + 1 < ntiles) st.finish(ring_buf(it + 1));
    };

    // Online softmax with a reference maximum m per row (base-2 domain).
    // m is set by the first tile with a visible token and then kept while
    // the scores stay below m + kHeadroom: P = 2^(s - m) < 2^kHeadroom is
    // far from overflowing bf16 / fp32, and P, the denominator and the
    // accumulator all use the same m, so the result does not depend on it.
    // The accumulator is zero while m = -inf, so setting m then needs no
    // rescale.  A tile whose scores exceed m + kHeadroom (rare: a score
    // ~44 nats above every earlier one) sends the wave to the loop below,
    // which rescales the accumulator; keeping that out of the main loop
    // lets the accumulators stay in the matrix-core registers.
    constexpr float kHeadroom = 64.f;
    // Returns false (having changed nothing) if tile `it` needs a rescale
    // and kRescale is false.
    auto tile = [&](int it, auto rescale_tag) __attribute__((always_inline)) -> bool {
      constexpr bool kRescale = decltype(rescale_tag)::value;
      const lds_char* buf = ring_buf(it);
      const int tt0 = t0 + it * kTile;

      // ---- S^T = Tile . Q^T for two 16-token blocks ----
      // Lane reads chunk 4ks+g of token tb*16+li.  With x = swz(token),
      // (4ks+g)^x = 4(ks ^ (x>>2)) + (g ^ (x&3)), so the address is a per-lane
      // base (one for even, one for odd ks) plus the immediate 64*ks.
      // Operands are prefetched kQkAhead k-steps ahead (LDS latency is several
      // MFMA issue slots); the scheduling fences keep the compiler from
      // hoisting every LDS read of the unrolled loop.  Even and odd k-steps
      // accumulate separately, so four independent MFMA chains are in flight.
      constexpr int kQkAhead = HILO ? 2 : 3;
      f32x4 sc[2][2];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) sc[tb][0] = sc[tb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
      const lds_char* lat_base[2][2];
      const lds_char* rope_base[2][2];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const int tok = tb * 16 + li;
        const int xs = swz(tok);
        const int flip = 64 * (xs >> 2);
        const lds_char* bl = buf + tok * G::kLatRow + 16 * (g ^ (xs & 3));
        const lds_char* br = buf + G::kRopeBase + tok * G::kRopeRow + 16 * (g ^ (xs & 3));
        lat_base[tb][0] = bl + flip;
        lat_base[tb][1] = bl - flip;
        rope_base[tb][0] = br + flip;
        rope_base[tb][1] = br - flip;
      }
      auto tile_a = [&](int ks, int tb) {
        const lds_char* p = ks < G::kKsLat ? lat_base[tb][ks & 1] + 64 * ks
                                           : rope_base[tb][ks & 1] + 64 * (ks - G::kKsLat);
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
        f32x4& c0 = sc[0][ks & 1];
        f32x4& c1 = sc[1][ks & 1];
        c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qh[ks], c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qh[ks], c1, 0, 0, 0);
        if constexpr (HILO) {
          c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, ql[ks], c0, 0, 0, 0);
          c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, ql[ks], c1, 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      const f32x4 s[2] = {sc[0][0] + sc[0][1], sc[1][0] + sc[1][1]};


      float sv[2][4];
      float mx = -INFINITY;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = tt0 + tb * 16 + 4 * g + i;
          const bool ok = SPARSE ? row_ok && ((mask_slot[(ring + it) & 1] >> (tb * 16 + 4 * g + i)) & 1u)
                                 : row_ok && t < t1 && t <= last_visible;
          sv[tb][i] = ok ? s[tb][i] * a.scale_log2 : -INFINITY;
          mx = fmaxf(mx, sv[tb][i]);
        }
      mx = max_over_rows(mx);
      if constexpr (kRescale) {
        const bool raise = mx > m + 8.f;  // also true when m = -inf < mx
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
      // With fp32 queries P is also split into hi + lo bf16 parts, so PV keeps
      // ~16 significant bits of the weights; otherwise P is rounded once.
      float psum = 0.f;
      uint32_t pk[4], pl[4];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          const float e0 = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv[tb][i] - m);
          const float e1 = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv[tb][i + 1] - m);
          psum += e0 + e1;
          if constexpr (HILO) split_bf16x2(e0, e1, pk[2 * tb + i / 2], pl[2 * tb + i / 2]);
          else pk[2 * tb + i / 2] = bf16x2_bits(e0, e1);
        }
      psum = sum_over_rows(psum);
      lsum += psum;
      const bf16x8 pa = __builtin_bit_cast(bf16x8, make_uint4(pk[0], pk[1], pk[2], pk[3]));
      bf16x8 pa_lo = pa;
      if constexpr (HILO) pa_lo = __builtin_bit_cast(bf16x8, make_uint4(pl[0], pl[1], pl[2], pl[3]));

      // ---- O += P . V, V read transposed from the tile ----
      // Column block d needs two transposed reads (tokens 4g+li/4 and 16 more)
      // of bf16 chunk 2d + h (h = (li&3)>>1), byte 8*(li&1).  With x =
      // swz(token), (2d+h)^x = 2(4(d>>2) + ((d&3) ^ (x>>1))) + (h ^ (x&1)):
      // one per-lane base per (d&3, half) plus the immediate 128*(d>>2).
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
      // Sparse mode: a padding slot's row (whatever it holds, NaN bytes
      // included) must contribute nothing, and a zero weight cannot cancel a
      // NaN, so its values are zeroed in the operand.  Element j of the lane's
      // operand is token 4g + j (j < 4) or 16 + 4g + j - 4 of the tile.
      u32x4 vkeep = {~0u, ~0u, ~0u, ~0u};
      if constexpr (SPARSE) {
        const uint32_t msk = mask_slot[(ring + it) & 1];
        uint32_t k[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int ta = (i < 2 ? 0 : 16) + 4 * g + (2 * i) % 4;
          k[i] = (((msk >> ta) & 1u) ? 0x0000ffffu : 0u) | (((msk >> (ta + 1)) & 1u) ? 0xffff0000u : 0u);
        }
        vkeep = u32x4{k[0], k[1], k[2], k[3]};
      }
      auto tile_v = [&](int d) {
        const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vbase[0][d & 3] + 128 * (d >> 2)));
        const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vbase[1][d & 3] + 128 * (d >> 2)));
        const bf16x8 v = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
        if constexpr (SPARSE) return __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, v) & vkeep);
        else return v;
      };
      constexpr int kPrefetch = HILO ? 4 : 8;
      bf16x8 vq[kPrefetch];
#pragma unroll
      for (int d = 0; d < kPrefetch; ++d) vq[d] = tile_v(d);
#pragma unroll
      for (int d = 0; d < G::kDb; ++d) {
        const bf16x8 vb = vq[d % kPrefetch];
        if (d + kPrefetch < G::kDb) vq[d % kPrefetch] = tile_v(d + kPrefetch);
        acc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vb, acc[d], 0, 0, 0);
        if constexpr (HILO) acc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_lo, vb, acc[d], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }

      return true;
    };

    int it = 0;
    for (; it < ntiles; ++it) {
      sync_issue(it);
      if (!tile(it, std::false_type{})) break;
      finish_next(it);
    }
    if (it < ntiles) {  // tile `it` is synchronised but not yet computed
      tile(it, std::true_type{});
      finish_next(it);
      for (++it; it < ntiles; ++it) {
        sync_issue(it);
        tile(it, std::true_type{});
        finish_next(it);
      }
    }

    // ---- normalise and write this unit's partial ----
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    float inv_r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) inv_r[i] = __shfl(inv, 4 * g + i);
    const float lse_row = lsum > 0.f ? (m + log2f(lsum)) * kLn2 : -INFINITY;
    const int row_blocks = (a.R + 15) / 16;
    bool direct = false;
    if constexpr (FUSE) {
      direct = uniform(part_range(ts, a.B, a.workers, b).n) == 1;
      if (!direct) {
        if (pend0 < 0) pend0 = b;
        else pend1 = b;
      }
    }
    if (direct) {  // the only part: the result itself, rows of o
      if (a.lse && g == 0 && row_ok) a.lse[(int64_t)b * a.R + row] = lse_row;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = wave * 16 + 4 * g + i;
        if (r < a.R) {
          float* dst = a.o + ((int64_t)b * a.R + r) * a.dc + li;
#pragma unroll
          for (int d = 0; d < G::kDb; ++d) dst[16 * d] = acc[d][i] * inv_r[i];
        }
      }
    } else {
      if (g == 0 && row_ok) a.part_lse[slot * a.R + row] = lse_row;
      // Tiled partial layout: the lane's four rows of column block d are one
      // 16-byte store, and a wave's store instruction writes 1 KB contiguously.
      if (wave < row_blocks && wave * 16 + 4 * g < a.R) {  // lanes with only padding rows skip
        float* dst = a.part_o + ((slot * row_blocks + wave) * G::kDb * 64 + lane) * 4;
#pragma unroll
        for (int d = 0; d < G::kDb; ++d)
          *reinterpret_cast<float4*>(dst + 256 * d) =
              make_float4(acc[d][0] * inv_r[0], acc[d][1] * inv_r[1], acc[d][2] * inv_r[2], acc[d][3] * inv_r[3]);
      }
    }
    ring = uniform((ring + ntiles) % NBUF);
    pre = uniform(ahead_done);
    first_unit = false;
    unit = nxt;
    have = have_next;
    have_next = have && uniform(unit_it.next(a, nxt));
  }
  wait_vmcnt_lgkm0<0>();  // no transfer into LDS outlives the workgroup
  if constexpr (FUSE) {
    if (pend0 >= 0) {
      const int pend[2] = {pend0, pend1};
      // Every wave's partial stores are visible at agent scope before the
      // arrival is counted.
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      __syncthreads();
      if (threadIdx.x == 0) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          s_last[k] = 0;
          if (pend[k] >= 0) {
            const int n = part_range(ts, a.B, a.workers, pend[k]).n;
            s_last[k] = __hip_atomic_fetch_add(arrival_counter(a, pend[k]), 1u, __ATOMIC_ACQ_REL,
                                               __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(n - 1);
          }
        }
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        if (s_last[k]) {  // this workgroup completed the sequence: merge it
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
          merge_sequence<G::kDb>(a, ts, pend[k], NW, wave, lane);
          if (threadIdx.x == 0)
            __hip_atomic_store(arrival_counter(a, pend[k]), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
  }
}

template <int FMT, bool HILO>
hipError_t launch_nw(const DecodeArgs& a, int nw, hipStream_t s) {
  const unsigned units = a.num_splits > 0 ? (unsigned)(a.B * a.num_splits) : (unsigned)a.workers;
  constexpr int NBUF = FMT == kBF16 ? kRingBf16 : 2;
  if (a.fuse_merge) {
    if constexpr (FMT == kBF16) {
      if (nw == 2 && a.num_splits == 0 && a.plan_in_kernel && a.ctr) {
        decode_mfma_kernel<FMT, HILO, 2, NBUF, false, true><<<units, 128, 0, s>>>(a);
        return hipGetLastError();
      }
    }
    return hipErrorInvalidValue;
  }
  switch (nw) {
#define MLA_CASE(N) \
  case N: decode_mfma_kernel<FMT, HILO, N, NBUF><<<units, 64 * N, 0, s>>>(a); break;
    MLA_CASE(2) MLA_CASE(3) MLA_CASE(4)
    MLA_CASE(5) MLA_CASE(6) MLA_CASE(7) MLA_CASE(8)
#undef MLA_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Waves per workgroup: one per 16 query rows, at least two so that small
// row counts still have two waves staging tiles.
int waves_for(int R) { return max(2, (R + 15) / 16); }

template <bool HILO>
hipError_t launch_sparse_nw(const DecodeArgs& a, int nw, hipStream_t s) {
  const unsigned units = (unsigned)(a.B * a.num_splits);
  switch (nw) {
    case 2: decode_mfma_kernel<kBF16, HILO, 2, 2, true><<<units, 128, 0, s>>>(a); break;
    case 3: decode_mfma_kernel<kBF16, HILO, 3, 2, true><<<units, 192, 0, s>>>(a); break;
    case 4: decode_mfma_kernel<kBF16, HILO, 4, 2, true><<<units, 256, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

// fp32 (hi + lo) queries need twice the query registers, which limits them
// to four waves.
bool decode_mfma_supported(int fmt, int dc, int dr, int R, int q_f32) {
  if (decode_fp8_rows_supported(fmt, dc, dr, R, q_f32)) return true;
  if (dr != kDr) return false;
  if (!((fmt == kBF16 && dc == 512) || (fmt == kFP8 && dc == 448))) return false;
  const int nw = waves_for(R);
  return nw <= (q_f32 ? 4 : 8);
}

// The fused merge is offered where sequences have few parts: its merging
// workgroup reads every other part itself (a merge kernel spreads that over
// the chip), so it needs at least one sequence per five workers.
bool decode_fused_merge_supported(int fmt, int dc, int dr, int R, int num_splits, int B, int workers) {
  return fmt == kBF16 && dc == 512 && dr == kDr && waves_for(R) == 2 && num_splits == 0 && B >= 1 &&
         B <= kMaxInKernelPlan && 5 * B >= workers;
}

bool decode_mfma_sparse_supported(int fmt, int dc, int dr, int R, int topk_width) {
  return fmt == kBF16 && dc == 512 && dr == kDr && R <= 64 && topk_width % kTile == 0 && kRingBf16 == 2;
}

hipError_t launch_decode_mfma_sparse(const DecodeArgs& a, hipStream_t s) {
  if (a.num_splits < 1 || !decode_mfma_sparse_supported(kBF16, a.dc, a.dr, a.R, a.topk_width))
    return hipErrorInvalidValue;
  const int nw = waves_for(a.R);
  return a.q_f32 ? launch_sparse_nw<true>(a, nw, s) : launch_sparse_nw<false>(a, nw, s);
}

hipError_t launch_decode_mfma(const DecodeArgs& a, int fmt, hipStream_t s) {
  if (decode_fp8_rows_supported(fmt, a.dc, a.dr, a.R, a.q_f32)) return launch_decode_fp8_rows(a, fmt, s);
  const int nw = waves_for(a.R);
  if (nw > (a.q_f32 ? 4 : 8)) return hipErrorInvalidValue;
  if (fmt == kBF16) return a.q_f32 ? launch_nw<kBF16, true>(a, nw, s) : launch_nw<kBF16, false>(a, nw, s);
  if (fmt == kFP8) return a.q_f32 ? launch_nw<kFP8, true>(a, nw, s) : launch_nw<kFP8, false>(a, nw, s);
  return hipErrorInvalidValue;
}

}  // namespace mla
