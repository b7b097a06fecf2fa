// Tile geometry and the direct-to-LDS staging of bf16 cache rows, shared by
// the matrix-core decode kernels (static and dynamically scheduled).
//
// LDS tile layout: the latent part of the 32 rows (region A) and the RoPE
// part (region B) are stored separately, so that a region-A row is exactly
// one direct-to-LDS instruction (64 lanes x 16 B).  16-byte chunks within a
// row are XOR-swizzled by the token index so that the 16-token b128 reads of
// QK^T and the 4-token transposed reads of PV hit distinct banks.
#pragma once

#include "decode_common.h"

namespace mla {
namespace mfma {

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

// bf16 tiles go straight from HBM to LDS.  A wave instruction fills 64
// consecutive 16-B LDS chunks: one token's latent row (lane = swizzled
// chunk, 1 KB contiguous in HBM), or the RoPE parts of 8 tokens.  Latent rows
// are handed out in groups of 8 tokens (group i = tokens 8i..8i+7, so that a
// row's swizzle only depends on its place in the group): wave w issues groups
// w, w+NW, ... and RoPE instructions w, w+NW, ...
template <int NW>
struct DmaStaging {
  using G = Geo<kBF16>;
  static constexpr int kRowBytes = 2 * G::kVals;
  static constexpr int kGroups = kTile / 8;
  static constexpr int kRopeInst = kTile * 8 / 64;
  // Fewest transfer instructions any wave issues per tile.
  static constexpr int kMinOps = 8 * (kGroups / NW) + kRopeInst / NW;

  // Per-lane source offsets for a whole tile in one page, relative to the
  // row of the group's first token: row j's swizzled latent chunk, and the
  // RoPE chunk of token lane/8.
  uint32_t lat_off[8];
  uint32_t rope_off;

  __device__ __forceinline__ void init() {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int j = 0; j < 8; ++j) lat_off[j] = j * kRowBytes + 16 * (lane ^ swz(j));
    const int t = lane >> 3;
    rope_off = t * kRowBytes + 2 * G::kDc + 16 * ((lane & 7) ^ swz(t));
  }

  __device__ __forceinline__ void load(const TileSrc& ts, lds_char* buf) const {
    load(ts, buf, uniform(threadIdx.x >> 6));
  }

  // As above, for loader wave `wave` of NW (the wave's index among the
  // waves that share the transfers).
  __device__ __forceinline__ void load(const TileSrc& ts, lds_char* buf, int wave) const {
    wave = uniform(wave);
    if (ts.n == kTile && ts.kb >= kTile) {  // whole tile, one page: rows are consecutive
#pragma unroll
      for (int i = 0; i < (kGroups + NW - 1) / NW; ++i) {
        const int grp = wave + NW * i;
        if (NW * i + NW <= kGroups || grp < kGroups)
          dma16x8((const void*)(uintptr_t)(ts.base0 + (uint64_t)(8 * kRowBytes) * grp), lat_off,
                  buf + G::kLatRow * 8 * grp);
      }
#pragma unroll
      for (int i = 0; i < (kRopeInst + NW - 1) / NW; ++i) {
        const int r = wave + NW * i;
        if (NW * i + NW <= kRopeInst || r < kRopeInst)
          dma16((const void*)(uintptr_t)(ts.base0 + (uint64_t)(8 * kRowBytes) * r), rope_off,
                buf + G::kRopeBase + 1024 * r);
      }
      return;
    }
    // Last tile of a unit, or a tile across two pages of 16 tokens.
    load_rows(ts, buf, wave);
  }

  // Gathered rows (sparse mode): one latent transfer per token and the
  // RoPE parts of 8 tokens per transfer, as on the per-row path below; the
  // wave's groups are unrolled with uniform conditions so that the row table
  // is indexed by constants.
  __device__ __forceinline__ void load_gather(const Gather& gt, const uint8_t* pool, lds_char* buf) const {
    const int lane = threadIdx.x & 63;
    const int wave = uniform(threadIdx.x >> 6);
    const uint64_t base = (uint64_t)(uintptr_t)pool;
#pragma unroll
    for (int grp = 0; grp < kGroups; ++grp) {
      if (grp % NW != wave) continue;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int k = 8 * grp + j;
        dma16((const void*)(uintptr_t)(base + (uint64_t)gt.phys[k] * kRowBytes), 16u * (lane ^ swz(j)),
              buf + G::kLatRow * k);
      }
    }
#pragma unroll
    for (int r = 0; r < kRopeInst; ++r) {
      if (r % NW != wave) continue;
      const int t = lane >> 3;  // token 8r + t
      uint32_t ph = gt.phys[8 * r];
#pragma unroll
      for (int x = 1; x < 8; ++x) ph = t == x ? gt.phys[8 * r + x] : ph;
      const uint64_t addr = base + (uint64_t)ph * kRowBytes + 2 * G::kDc + 16 * ((lane & 7) ^ swz(t));
      dma16_vaddr((const void*)(uintptr_t)addr, buf + G::kRopeBase + 1024 * r);
    }
  }

  // As load(), with the per-row path as a rolled loop: one row address is
  // live at a time, so a single loader wave does not need 32 scalar register
  // pairs for them (the per-row path only serves the last tile of a sequence
  // and tiles across two 16-token pages).
  __device__ __forceinline__ void load_compact(const TileSrc& ts, lds_char* buf, int wave) const {
    wave = uniform(wave);
    if (ts.n == kTile && ts.kb >= kTile) {
      load(ts, buf, wave);
      return;
    }
    const int lane = threadIdx.x & 63;
#pragma unroll 1
    for (int grp = wave; grp < kGroups; grp += NW) {
#pragma unroll 1
      for (int j = 0; j < 8; ++j) {
        const int k = 8 * grp + j;
        dma16(tile_row_ptr(ts, k, kRowBytes), 16u * (lane ^ swz(j)), buf + G::kLatRow * k);
      }
    }
#pragma unroll 1
    for (int r = wave; r < kRopeInst; r += NW) {
      const int t = lane >> 3;
      const int kk = min(8 * r + t, ts.n - 1);
      const int kk_hi = min(8 * r + 7, ts.n - 1);
      const uint64_t base = kk_hi < ts.kb ? ts.base0 : ts.base1;
      const uint32_t off = (uint32_t)(kk * kRowBytes) + 2 * G::kDc + 16 * ((lane & 7) ^ swz(t));
      dma16((const void*)(uintptr_t)base, off, buf + G::kRopeBase + 1024 * r);
    }
  }

  __device__ __forceinline__ void load_rows(const TileSrc& ts, lds_char* buf, int wave) const {
    wave = uniform(wave);
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < (kGroups + NW - 1) / NW; ++i) {
      const int grp = wave + NW * i;
      if (NW * i + NW <= kGroups || grp < kGroups) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int k = 8 * grp + j;
          dma16(tile_row_ptr(ts, k, kRowBytes), 16u * (lane ^ swz(j)), buf + G::kLatRow * k);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < (kRopeInst + NW - 1) / NW; ++i) {
      const int r = wave + NW * i;
      if (NW * i + NW <= kRopeInst || r < kRopeInst) {
        // Tokens 8r..8r+7 share a page: the 16-token page boundary of
        // page_block 16 falls between groups, and clamping to n - 1 moves
        // a whole group below it.
        const int t = lane >> 3;
        const int kk = min(8 * r + t, ts.n - 1);
        const int kk_hi = min(8 * r + 7, ts.n - 1);
        const uint64_t base = kk_hi < ts.kb ? ts.base0 : ts.base1;
        const uint32_t off = (uint32_t)(kk * kRowBytes) + 2 * G::kDc + 16 * ((lane & 7) ^ swz(t));
        dma16((const void*)(uintptr_t)base, off, buf + G::kRopeBase + 1024 * r);
      }
    }
  }
};


}  // namespace mfma
}  // namespace mla
