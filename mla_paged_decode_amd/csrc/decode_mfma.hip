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
// keeps the scores at ~16 significant bits; P is rounded once to bf16; all
// accumulation is fp32.  bf16 queries take a single pass.
//
// Tile staging: the next tile's rows are loaded into registers (16-byte,
// coalesced along each row) while the current tile is computed, then stored
// to the other LDS buffer.  fp8 rows (e4m3 + e8m0 per 32 values) are decoded
// to bf16 on the way; both conversions are exact.  Rows of the LDS tile are
// 16-byte-chunk XOR-swizzled so that the 16-token b128 reads of QK^T and the
// 4-token transposed reads of PV hit distinct banks.
#include <cmath>

#include "device_common.h"
#include "internal.h"
#include "schedule.h"

namespace mla {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr int kTile = 32;      // tokens per tile
constexpr int kDr = 64;        // RoPE dims
constexpr float kLn2 = 0.693147180559945309f;

// LDS tile: the latent part of the 32 rows (region A, d_c values per row)
// and the RoPE part (region B, 64 values per row) are stored separately, so
// that region A rows are a whole number of 1 KB / 896 B and a direct-to-LDS
// instruction moves exactly one token's latent row.
template <int FMT>
struct Geo {
  static constexpr int kDc = FMT == kBF16 ? 512 : 448;      // latent width
  static constexpr int kVals = kDc + kDr;                   // values per row
  static constexpr int kKs = kVals / 32;                    // QK k-steps
  static constexpr int kKsLat = kDc / 32;                   // ... over the latent
  static constexpr int kDb = kDc / 16;                      // PV column blocks
  static constexpr int kLatChunks = kDc / 8;                // 16-B bf16 chunks per latent row
  static constexpr int kLatRow = kLatChunks * 16;           // region A row stride
  static constexpr int kRopeRow = kDr * 2;                  // region B row stride (8 chunks)
  static constexpr int kRopeBase = kTile * kLatRow;         // region B offset in the tile
  static constexpr int kTileBytes = kRopeBase + kTile * kRopeRow;
  static constexpr int kSrcChunks = kVals / 16;             // stored fp8 16-value chunks per row
};

// Swizzle of 16-B chunk index within a row: a permutation of 0..7 on the
// token's low 3 bits such that 8 consecutive tokens get 8 distinct values
// and each 4 consecutive tokens get 4 distinct chunk pairs.
__device__ __forceinline__ int swz(int tok) { return ((tok & 3) << 1) | ((tok >> 2) & 1); }

// Byte offset of 16-B chunk `chunk` of token `tok` in a region with the
// given row stride (rows are a multiple of 8 chunks).
__device__ __forceinline__ int lds_off(int tok, int chunk, int row_bytes) {
  return tok * row_bytes + 16 * (chunk ^ swz(tok));
}

// Hide a value from loop-invariant code motion: address arithmetic is
// recomputed where it is used instead of being held in registers.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// Physical pages of one 32-token tile: tokens [tt0, tt1) of the current
// sequence lie in logical pages p0 .. p0+2 at most (page_block >= 16).
// Loaded with scalar loads, so the vector-memory counter only tracks the
// tile data itself.
struct TilePages {
  int tt0, tt1, p0, pg0, pg1, pg2;
};

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// The block table is read-only during the call: reading it through the
// constant address space lets the compiler use scalar loads.
typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;

__device__ __forceinline__ TilePages tile_pages(const DecodeArgs& a, const_i32_ptr bt, int tt0, int t1) {
  TilePages r;
  r.tt0 = tt0;
  r.tt1 = min(tt0 + kTile, t1);
  r.p0 = tt0 >> a.P_log2;
  const int p1 = (r.tt1 - 1) >> a.P_log2;
  r.pg0 = uniform(bt[r.p0]);
  r.pg1 = uniform(bt[min(r.p0 + 1, p1)]);
  r.pg2 = uniform(bt[min(r.p0 + 2, p1)]);
  // Pin the fields in scalar registers so the struct never lives in memory
  // (a dynamically indexed copy would add waits on the transfer counter).
  asm volatile("" : "+s"(r.tt0), "+s"(r.tt1), "+s"(r.p0), "+s"(r.pg0), "+s"(r.pg1), "+s"(r.pg2));
  return r;
}

// Row index (page * P + slot) of tile token k; tokens past the end repeat
// the last valid one.
__device__ __forceinline__ int64_t tile_row(const DecodeArgs& a, TilePages tp, int k) {
  const int t = min(tp.tt0 + k, tp.tt1 - 1);
  const int pi = (t >> a.P_log2) - tp.p0;  // 0, 1 or 2
  const int page = tp.pg0 + (pi >= 1 ? tp.pg1 - tp.pg0 : 0) + (pi >= 2 ? tp.pg2 - tp.pg1 : 0);
  return (int64_t)page * a.P + (t & (a.P - 1));
}

// s_waitcnt vmcnt(N) lgkmcnt(0) (gfx9 encoding: vmcnt[3:0], expcnt[6:4],
// lgkmcnt[11:8], vmcnt[5:4] in bits 15:14).
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (0x7 << 4) | ((N >> 4) << 14));
}

// Workgroup barrier for LDS hand-off only.  The caller has already waited
// for its own LDS operations and tile transfers; unlike __syncthreads() this
// does not drain the tile transfers still in flight for later tiles.  The
// signal fences keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// One 16-byte direct-to-LDS load per lane: the wave's 64 chunks land at
// lds + 16 * lane.  Issued as inline assembly so that the compiler does not
// treat the pending LDS write as aliasing every LDS read (which would make
// it drain all transfers before reading the current tile); completion is
// tracked explicitly with wait_vmcnt_lgkm0.
__device__ __forceinline__ void dma16(const void* src, const char* lds) {
  const uint32_t lds_addr = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)lds);
  uint32_t saved;
  // m0 holds the LDS destination of the transfer; its previous value is
  // restored afterwards.
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(lds_addr)
      : "memory");
}

// bf16 tiles go straight from HBM to LDS with 16-byte direct-to-LDS loads.
// A wave instruction fills 64 consecutive 16-B LDS chunks from per-lane
// sources: instruction k < 32 is token k's latent row (lane = swizzled
// chunk, 1 KB contiguous in HBM); the 4 instructions after it carry the
// RoPE parts of 8 tokens each.  Wave w issues latent rows w, w+NW, ... and
// RoPE groups w, w+NW, ...; every wave issues at least kMinOps of them.
template <int NW>
struct DmaStaging {
  using G = Geo<kBF16>;
  static constexpr int kRopeInst = kTile * 8 / 64;  // 4
  static constexpr int kMinOps = kTile / NW + kRopeInst / NW;

  __device__ __forceinline__ static void load(const DecodeArgs& a, TilePages tp, char* buf) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll 1
    for (int k = wave; k < kTile; k += NW) {
      const uint8_t* src = a.pool + tile_row(a, tp, k) * a.row_bytes + 16 * (lane ^ swz(k));
      dma16(src, buf + G::kLatRow * k);
    }
#pragma unroll 1
    for (int r = wave; r < kRopeInst; r += NW) {
      const int tok = 8 * r + (lane >> 3);
      const uint8_t* src = a.pool + tile_row(a, tp, tok) * a.row_bytes + 2 * G::kDc + 16 * ((lane & 7) ^ swz(tok));
      dma16(src, buf + G::kRopeBase + 1024 * r);
    }
  }
};

// fp8 tiles are loaded into registers, decoded to bf16 and stored to LDS.
template <int NW>
struct Fp8Staging {
  using G = Geo<kFP8>;
  static constexpr int kThreads = 64 * NW;
  static constexpr int kSrc = kTile * G::kSrcChunks;  // 16-value chunks per tile
  static constexpr int kPer = (kSrc + kThreads - 1) / kThreads;
  uint4 v[kPer];
  uint32_t s[kPer];

  __device__ __forceinline__ void load(const DecodeArgs& a, TilePages tp) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int q = j * kThreads + threadIdx.x;
      const int tok = min(q / G::kSrcChunks, kTile - 1);
      const int c = q % G::kSrcChunks;
      const uint8_t* p = a.pool + tile_row(a, tp, tok) * a.row_bytes;
      if (q < kSrc) {
        v[j] = *reinterpret_cast<const uint4*>(p + 16 * c);
        s[j] = p[G::kVals + c / 2];
      }
    }
  }

  __device__ __forceinline__ void store(char* buf) const {
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
      char* d0 = c0 < G::kLatChunks ? buf + lds_off(tok, c0, G::kLatRow)
                                    : buf + G::kRopeBase + lds_off(tok, c0 - G::kLatChunks, G::kRopeRow);
      char* d1 = c0 < G::kLatChunks ? buf + lds_off(tok, c0 + 1, G::kLatRow)
                                    : buf + G::kRopeBase + lds_off(tok, c0 + 1 - G::kLatChunks, G::kRopeRow);
      *reinterpret_cast<uint4*>(d0) = make_uint4(o[0], o[1], o[2], o[3]);
      *reinterpret_cast<uint4*>(d1) = make_uint4(o[4], o[5], o[6], o[7]);
    }
  }
};

// Staging interface over the two formats.  kDepth tiles are in flight ahead
// of the one being computed: issue(x) starts tile x's transfer into its ring
// buffer, finish(x) completes it from registers (fp8), wait(n) blocks until
// this wave's part of the oldest outstanding tile has landed when n younger
// tiles have been issued after it.
template <int FMT, int NW, int NBUF>
struct Staging;

template <int NW, int NBUF>
struct Staging<kBF16, NW, NBUF> {
  static constexpr int kDepth = NBUF - 1;
  __device__ __forceinline__ void issue(const DecodeArgs& a, TilePages tp, char* buf) {
    DmaStaging<NW>::load(a, tp, buf);
  }
  __device__ __forceinline__ void finish(char*) {}
  __device__ __forceinline__ void wait(int younger) {
    constexpr int M = DmaStaging<NW>::kMinOps;
    if (younger >= 2) wait_vmcnt_lgkm0<(NBUF >= 4 ? 2 * M : 0)>();
    else if (younger == 1) wait_vmcnt_lgkm0<(NBUF >= 3 ? M : 0)>();
    else wait_vmcnt_lgkm0<0>();
  }
};

template <int NW, int NBUF>
struct Staging<kFP8, NW, NBUF> {
  static_assert(NBUF == 2, "fp8 tiles are staged through registers, one ahead");
  static constexpr int kDepth = 1;
  Fp8Staging<NW> f;
  __device__ __forceinline__ void issue(const DecodeArgs& a, TilePages tp, char*) { f.load(a, tp); }
  __device__ __forceinline__ void finish(char* buf) { f.store(buf); }
  __device__ __forceinline__ void wait(int) { wait_vmcnt_lgkm0<0>(); }
};

template <int FMT, bool HILO, int NW, int NBUF>
__global__ __launch_bounds__(64 * NW) void decode_mfma_kernel(DecodeArgs a) {
  using G = Geo<FMT>;
  __shared__ __attribute__((aligned(16))) char tiles[NBUF][G::kTileBytes];
  __shared__ int32_t s_ts[kMaxInKernelPlan + 1];
  __shared__ int32_t s_scan[64 * NW];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4;          // lane group
  const int li = lane & 15;         // index within the group
  const int row = wave * 16 + li;   // this lane's query row (B / P side)
  const bool row_ok = row < a.R;

  const int32_t* ts = a.tile_start;
  if (a.num_splits == 0 && a.plan_in_kernel) {
    block_plan(a.seq_lens, a.B, s_ts, s_scan);
    if (blockIdx.x == 0)  // publish the plan for the merge kernel
      for (int i = threadIdx.x; i <= a.B; i += 64 * NW) a.tile_start[i] = s_ts[i];
    ts = s_ts;
  }
  UnitIter unit_it(a, ts);
  Unit unit;
  while (unit_it.next(a, unit)) {
    // The unit is the same for the whole workgroup: keep it in scalar
    // registers so page lookups below are scalar loads.
    const int b = uniform(unit.b), L = uniform(unit.L), t0 = uniform(unit.t0), t1 = uniform(unit.t1);
    const int64_t slot = a.num_splits > 0 ? (int64_t)blockIdx.x : (int64_t)blockIdx.x + b;
    // ---- queries in the B-operand layout: column = row, k = 8g..8g+7 ----
    bf16x8 qh[G::kKs], ql[HILO ? G::kKs : 1];
    {
      const int64_t qoff = ((int64_t)b * a.R + (row_ok ? row : 0)) * G::kVals + 8 * g;
#pragma unroll
      for (int ks = 0; ks < G::kKs; ++ks) {
        float x[8];
        if (a.q_f32) {
          const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(a.q_abs) + qoff + 32 * ks);
          const float4 u = p[0], w = p[1];
          x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w; x[4] = w.x; x[5] = w.y; x[6] = w.z; x[7] = w.w;
        } else {
          const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q_abs) + qoff + 32 * ks);
          const uint32_t uw[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            x[2 * i] = bf16_bits_to_f32(uw[i] & 0xffffu);
            x[2 * i + 1] = bf16_bits_to_f32(uw[i] >> 16);
          }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float v = row_ok ? x[i] : 0.f;
          const uint32_t hb = f32_to_bf16_bits(v);
          qh[ks][i] = __builtin_bit_cast(__bf16, (uint16_t)hb);
          if constexpr (HILO) {
            const float r = v - bf16_bits_to_f32(hb);
            ql[ks][i] = __builtin_bit_cast(__bf16, (uint16_t)f32_to_bf16_bits(r));
          }
        }
      }
    }
    const int j_q = row_ok ? row / a.H : 0;
    const int last_visible = L - a.Sq + j_q;

    f32x4 acc[G::kDb];
#pragma unroll
    for (int d = 0; d < G::kDb; ++d) acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, lsum = 0.f;

    const int ntiles = (t1 - t0 + kTile - 1) / kTile;
    const const_i32_ptr bt = (const_i32_ptr)(a.block_table) + (int64_t)b * a.max_blocks;
    using St = Staging<FMT, NW, NBUF>;
    constexpr int D = St::kDepth;
    St st;
    TilePages tp_next;  // pages of the next tile to issue, loaded one tile early
    if (ntiles > 0) {
      wait_vmcnt_lgkm0<0>();
      lds_barrier();  // the previous unit's readers of the ring are done
#pragma unroll
      for (int x = 0; x < D; ++x)
        if (x < ntiles) st.issue(a, tile_pages(a, bt, t0 + x * kTile, t1), tiles[x]);
      if (D < ntiles) tp_next = tile_pages(a, bt, t0 + D * kTile, t1);
      st.finish(tiles[0]);
    }

    for (int it = 0; it < ntiles; ++it) {
      st.wait(min(D - 1, ntiles - 1 - it));  // this wave's part of tile `it` landed
      lds_barrier();                          // everyone's did; everyone finished tile it-1
      const int x = it + D;                   // goes into the buffer tile it-1 used
      if (x < ntiles) {
        st.issue(a, tp_next, tiles[x % NBUF]);
        if (x + 1 < ntiles) tp_next = tile_pages(a, bt, t0 + (x + 1) * kTile, t1);
      }
      const char* buf = tiles[it % NBUF];
      const int tt0 = t0 + it * kTile;

      // ---- S^T = Tile . Q^T for two 16-token blocks ----
      // Lane reads chunk 4ks+g of token tb*16+li.  With x = swz(token),
      // (4ks+g)^x = 4(ks ^ (x>>2)) + (g ^ (x&3)), so the address is a per-lane
      // base (one for even, one for odd ks) plus the immediate 64*ks.
      // Operands are prefetched one k-step ahead; the scheduling fences keep
      // the compiler from hoisting every LDS read of the unrolled loop.
      f32x4 s[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      const char* lat_base[2][2];
      const char* rope_base[2][2];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const int tok = tb * 16 + li;
        const int x = swz(tok);
        const int flip = 64 * (x >> 2);
        const char* bl = buf + tok * G::kLatRow + 16 * (g ^ (x & 3));
        const char* br = buf + G::kRopeBase + tok * G::kRopeRow + 16 * (g ^ (x & 3));
        lat_base[tb][0] = bl + flip;
        lat_base[tb][1] = bl - flip;
        rope_base[tb][0] = br + flip;
        rope_base[tb][1] = br - flip;
      }
      auto tile_a = [&](int ks, int tb) {
        const char* p = ks < G::kKsLat ? lat_base[tb][ks & 1] + 64 * ks
                                       : rope_base[tb][ks & 1] + 64 * (ks - G::kKsLat);
        return *reinterpret_cast<const bf16x8*>(p);
      };
      bf16x8 ta0 = tile_a(0, 0), ta1 = tile_a(0, 1);
#pragma unroll
      for (int ks = 0; ks < G::kKs; ++ks) {
        bf16x8 tn0 = ta0, tn1 = ta1;
        if (ks + 1 < G::kKs) {
          tn0 = tile_a(ks + 1, 0);
          tn1 = tile_a(ks + 1, 1);
        }
        s[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ta0, qh[ks], s[0], 0, 0, 0);
        s[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ta1, qh[ks], s[1], 0, 0, 0);
        if constexpr (HILO) {
          s[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ta0, ql[ks], s[0], 0, 0, 0);
          s[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ta1, ql[ks], s[1], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        ta0 = tn0;
        ta1 = tn1;
      }

      // ---- online softmax for row `row` over tokens tt0 + {4g+i, 16+4g+i} ----
      // m is a reference maximum that is only raised when a row's scores
      // exceed it by more than 2^8 (base-2 domain): P = 2^(s - m) then stays
      // below 256, and P, the denominator and the accumulator all use the
      // same m, so the result is unchanged while the rescale of the
      // accumulator is skipped on almost every tile.
      float sv[2][4];
      float mx = -INFINITY;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = tt0 + tb * 16 + 4 * g + i;
          const bool ok = row_ok && t < t1 && t <= last_visible;
          sv[tb][i] = ok ? s[tb][i] * a.scale_log2 : -INFINITY;
          mx = fmaxf(mx, sv[tb][i]);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const bool raise = mx > m + 8.f;  // also true when m = -inf < mx
      if (__any(raise)) {
        const float m_new = raise ? mx : m;
        const float alpha = m_new == -INFINITY ? 1.f : exp2f(m - m_new);
        lsum *= alpha;
        m = m_new;
        float al[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * g + i);
#pragma unroll
        for (int d = 0; d < G::kDb; ++d) {
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[d][i] *= al[i];
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      float psum = 0.f;
      uint32_t pk[4];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          const float e0 = m == -INFINITY ? 0.f : exp2f(sv[tb][i] - m);
          const float e1 = m == -INFINITY ? 0.f : exp2f(sv[tb][i + 1] - m);
          psum += e0 + e1;
          pk[2 * tb + i / 2] = pack_bf16(e0, e1);
        }
      psum += __shfl_xor(psum, 16);
      psum += __shfl_xor(psum, 32);
      lsum += psum;
      const bf16x8 pa = __builtin_bit_cast(bf16x8, make_uint4(pk[0], pk[1], pk[2], pk[3]));

      // ---- O += P . V, V read transposed from the tile ----
      // Column block d needs two transposed reads (tokens 4g+li/4 and 16 more)
      // of bf16 chunk 2d + h (h = (li&3)>>1), byte 8*(li&1).  With x =
      // swz(token), (2d+h)^x = 2(4(d>>2) + ((d&3) ^ (x>>1))) + (h ^ (x&1)):
      // one per-lane base per (d&3, half) plus the immediate 128*(d>>2).
      const char* vbase[2][4];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int tok = 16 * half + 4 * g + (li >> 2);
        const int x = swz(tok);
        const int h = (li & 3) >> 1;
        const char* b0 = buf + tok * G::kLatRow + 16 * (h ^ (x & 1)) + 8 * (li & 1);
#pragma unroll
        for (int r = 0; r < 4; ++r) vbase[half][r] = b0 + 32 * (r ^ (x >> 1));
      }
      auto tile_v = [&](int d) {
        const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vbase[0][d & 3] + 128 * (d >> 2)));
        const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vbase[1][d & 3] + 128 * (d >> 2)));
        return __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
      };
      constexpr int kPrefetch = 4;
      bf16x8 vq[kPrefetch];
#pragma unroll
      for (int d = 0; d < kPrefetch; ++d) vq[d] = tile_v(d);
#pragma unroll
      for (int d = 0; d < G::kDb; ++d) {
        const bf16x8 vb = vq[d % kPrefetch];
        if (d + kPrefetch < G::kDb) vq[d % kPrefetch] = tile_v(d + kPrefetch);
        acc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vb, acc[d], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }

      if (D == 1 && it + 1 < ntiles) st.finish(tiles[(it + 1) % NBUF]);
    }

    // ---- normalise and write this unit's partial ----
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    float inv_r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) inv_r[i] = __shfl(inv, 4 * g + i);
    if (g == 0 && row_ok)
      a.part_lse[slot * a.R + row] = lsum > 0.f ? (m + log2f(lsum)) * kLn2 : -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wave * 16 + 4 * g + i;
      if (r < a.R) {
        float* dst = a.part_o + (slot * a.R + r) * G::kDc + li;
#pragma unroll
        for (int d = 0; d < G::kDb; ++d) dst[16 * d] = acc[d][i] * inv_r[i];
      }
    }
  }
}

template <int FMT, bool HILO>
hipError_t launch_nw(const DecodeArgs& a, int nw, hipStream_t s) {
  const unsigned units = a.num_splits > 0 ? (unsigned)(a.B * a.num_splits) : (unsigned)a.workers;
  constexpr int NBUF = FMT == kBF16 ? kRingBf16 : 2;
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

}  // namespace

// Query rows per workgroup: one wave per 16 rows; fp32 (hi + lo) queries
// need twice the query registers, which limits them to four waves.
bool decode_mfma_supported(int fmt, int dc, int dr, int R, int q_f32) {
  if (dr != kDr) return false;
  if (!((fmt == kBF16 && dc == 512) || (fmt == kFP8 && dc == 448))) return false;
  const int nw = waves_for(R);
  return nw <= (q_f32 ? 4 : 8);
}

hipError_t launch_decode_mfma(const DecodeArgs& a, int fmt, hipStream_t s) {
  const int nw = waves_for(a.R);
  if (nw > (a.q_f32 ? 4 : 8)) return hipErrorInvalidValue;
  if (fmt == kBF16) return a.q_f32 ? launch_nw<kBF16, true>(a, nw, s) : launch_nw<kBF16, false>(a, nw, s);
  if (fmt == kFP8) return a.q_f32 ? launch_nw<kFP8, true>(a, nw, s) : launch_nw<kFP8, false>(a, nw, s);
  return hipErrorInvalidValue;
}

}  // namespace mla
