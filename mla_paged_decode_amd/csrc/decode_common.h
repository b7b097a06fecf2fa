// Device helpers shared by the matrix-core decode kernels: operand types,
// the LDS chunk swizzle, tile addressing through the block table, explicit
// wait counters, the LDS-only barrier and direct-to-LDS loads.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_common.h"
#include "internal.h"

namespace mla {
namespace mfma {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
// The block table is read-only during a call: reading it through the
// constant address space lets the compiler use scalar loads.
typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;

constexpr int kTile = 32;      // tokens per tile
constexpr int kDr = 64;        // RoPE dims
constexpr float kLn2 = 0.693147180559945309f;

// Swizzle of 16-B chunk index within a row: a permutation of 0..7 on the
// token's low 3 bits such that 8 consecutive tokens get 8 distinct values
// and each 4 consecutive tokens get 4 distinct chunk pairs.
__device__ __forceinline__ int swz(int tok) { return ((tok & 3) << 1) | ((tok >> 2) & 1); }

// Byte offset of 16-B chunk `chunk` of token `tok` in a region with the
// given row stride (rows are a multiple of 8 chunks).
__device__ __forceinline__ int lds_off(int tok, int chunk, int row_bytes) {
  return tok * row_bytes + 16 * (chunk ^ swz(tok));
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) { return bf16x2_bits(lo, hi); }

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Maximum and sum over the four 16-lane rows of a wave at each lane's
// position in its row (what x op shfl_xor(x, 16) op shfl_xor(x, 32) gives),
// with gfx950's row-swap permutes: VALU operations instead of LDS permutes.
// After a swap of x with itself, every lane holds its own row's value and
// its partner row's (rows r and r ^ 1, then halves h and h ^ 1), so the
// results equal the shuffle forms exactly (both operations commute).
__device__ __forceinline__ float max_over_rows(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
// Maximum and sum over the 16 lanes of each row, every lane of the row
// getting the row's result, with DPP lane moves on the VALU instead of LDS
// permutes: swaps within quads (lanes 1 0 3 2, then 2 3 0 1), then the
// half-row mirror (lane i of 8 takes 7 - i) and the row mirror (i of 16
// takes 15 - i), each pairing two already-reduced groups.  The sum's order
// of additions differs from a xor butterfly's.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float max_in_row(float x) {
  x = fmaxf(x, dpp_move<0xB1>(x));
  x = fmaxf(x, dpp_move<0x4E>(x));
  x = fmaxf(x, dpp_move<0x141>(x));
  return fmaxf(x, dpp_move<0x140>(x));
}
__device__ __forceinline__ float sum_in_row(float x) {
  x += dpp_move<0xB1>(x);
  x += dpp_move<0x4E>(x);
  x += dpp_move<0x141>(x);
  return x + dpp_move<0x140>(x);
}
__device__ __forceinline__ float sum_over_rows(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Source of one tile: tokens [tt0, tt0 + n) of the current sequence.  Work
// units start at multiples of kTile tokens and page_block is a power of two
// >= 16, so the tile lies in one page (page_block >= 32) or two (16).  Tile
// token k is read from row kk = min(k, n - 1) (tokens past the end repeat the
// last valid one, so every row read holds finite values), at
//   (kk < kb ? base0 : base1) + kk * row_bytes.
// All fields are wave-uniform and live in scalar registers.
struct TileSrc {
  int n, kb;
  uint64_t base0, base1;
};

// Physical pages of one tile, looked up (scalar loads) one tile before they
// are used, so that the lookup latency overlaps the wait for the tile before.
struct TilePages {
  int tt0, pg0, pg1;
};

__device__ __forceinline__ TilePages tile_pages(const DecodeArgs& a, const_i32_ptr bt, int tt0, int t1) {
  const int n = min(kTile, t1 - tt0);
  return TilePages{tt0, bt[tt0 >> a.P_log2], bt[(tt0 + n - 1) >> a.P_log2]};
}

__device__ __forceinline__ TileSrc tile_src(const DecodeArgs& a, const TilePages& tp, int t1) {
  TileSrc r;
  r.n = min(kTile, t1 - tp.tt0);
  const int s0 = tp.tt0 & (a.P - 1);
  r.kb = a.P - s0;
  const uint64_t pool = (uint64_t)(uintptr_t)a.pool;
  r.base0 = pool + (uint64_t)((int64_t)uniform(tp.pg0) * a.P + s0) * (uint64_t)a.row_bytes;
  r.base1 = pool + (uint64_t)((int64_t)uniform(tp.pg1) * a.P - r.kb) * (uint64_t)a.row_bytes;
  asm volatile("" : "+s"(r.n), "+s"(r.kb), "+s"(r.base0), "+s"(r.base1));
  return r;
}

// Address of the row holding tile token k (wave-uniform k).
__device__ __forceinline__ const uint8_t* tile_row_ptr(const TileSrc& ts, int k, int64_t row_bytes) {
  const int kk = min(k, ts.n - 1);
  return (const uint8_t*)(uintptr_t)((kk < ts.kb ? ts.base0 : ts.base1) + (uint64_t)(kk * (int)row_bytes));
}

// Sparse top-k mode: a tile is 32 consecutive slots of a query's index list;
// slot k names the cached token list[tt0 + k].  Its physical rows are looked
// up one tile ahead with scalar loads (counted by lgkmcnt, so the tile
// transfers' vmcnt accounting is untouched).  Slots that are padding (< 0,
// past the causal limit, or past the unit's end) read row 0 of the pool,
// always in bounds, and are cleared in `mask`.
struct Gather {
  uint32_t phys[kTile];  // physical row (page * P + offset) per slot
  uint32_t mask;         // bit k: slot k names a visible token
};

__device__ __forceinline__ Gather gather_lookup(const DecodeArgs& a, const_i32_ptr list, const_i32_ptr bt, int tt0,
                                                int t1, int limit) {
  Gather g;
  int32_t p[kTile];
#pragma unroll
  for (int k = 0; k < kTile; ++k) p[k] = list[tt0 + k];  // in bounds: the list width is a multiple of 32
  g.mask = 0;
#pragma unroll
  for (int k = 0; k < kTile; ++k) {
    const bool ok = tt0 + k < t1 && p[k] >= 0 && p[k] <= limit;
    g.mask |= (uint32_t)ok << k;
    p[k] = ok ? p[k] : 0;
  }
#pragma unroll
  for (int k = 0; k < kTile; ++k) {
    const int32_t pg = bt[p[k] >> a.P_log2];
    g.phys[k] = (g.mask >> k) & 1 ? (uint32_t)(pg * a.P + (p[k] & (a.P - 1))) : 0u;
  }
  return g;
}

// s_waitcnt vmcnt(N) lgkmcnt(0) (gfx9 encoding: vmcnt[3:0], expcnt[6:4],
// lgkmcnt[11:8], vmcnt[5:4] in bits 15:14).
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (0x7 << 4) | ((N >> 4) << 14));
}

// s_waitcnt vmcnt(N) alone: the scalar loads in flight (page lookups for a
// later tile) are not waited for.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// s_waitcnt lgkmcnt(0): this wave's LDS reads have completed.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x3 << 14)); }

// Workgroup barrier for LDS hand-off only.  The caller has already waited
// for its own LDS operations and tile transfers; unlike __syncthreads() this
// does not drain the tile transfers still in flight for later tiles.  The
// signal fences keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// One 16-byte direct-to-LDS load per lane from sbase + voff: the wave's 64
// chunks land at lds + 16 * lane.  Issued as inline assembly so that the
// compiler does not treat the pending LDS write as aliasing every LDS read
// (which would make it drain all transfers before reading the current
// tile); completion is tracked explicitly with wait_vmcnt_lgkm0.  m0 holds
// the LDS destination during the instruction and is restored afterwards.
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, const lds_char* lds) {
  const uint32_t lds_addr = uniform((uint32_t)(uintptr_t)lds);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(sbase), "s"(lds_addr)
      : "memory");
}

// As dma16, with a full 64-bit address per lane.
__device__ __forceinline__ void dma16_vaddr(const void* src, const lds_char* lds) {
  const uint32_t lds_addr = uniform((uint32_t)(uintptr_t)lds);
  uint32_t saved;
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

// One 4-byte direct-to-LDS load per lane from a full 64-bit address: the
// wave's 64 dwords land at lds + 4 * lane.  Used to pull lines into L2
// ahead of their use (the LDS words written are never read).
__device__ __forceinline__ void dma4_vaddr(const void* src, const lds_char* lds) {
  const uint32_t lds_addr = uniform((uint32_t)(uintptr_t)lds);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(lds_addr)
      : "memory");
}

// Eight direct-to-LDS loads of one wave: lane l loads 16 B from
// sbase + voff[j] into lds + 1024 * j + 16 * l, for j = 0..7.
__device__ __forceinline__ void dma16x8(const void* sbase, const uint32_t (&voff)[8], const lds_char* lds) {
  const uint32_t lds_addr = uniform((uint32_t)(uintptr_t)lds);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %10\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %9\n\t"
      "s_add_u32 m0, m0, 0x400\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %9\n\t"
      "s_add_u32 m0, m0, 0x400\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %3, %9\n\t"
      "s_add_u32 m0, m0, 0x400\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %4, %9\n\t"
      "s_add_u32 m0, m0, 0x400\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %5, %9\n\t"
      "s_add_u32 m0, m0, 0x400\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %6, %9\n\t"
      "s_add_u32 m0, m0, 0x400\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %7, %9\n\t"
      "s_add_u32 m0, m0, 0x400\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %8, %9\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "v"(voff[3]), "v"(voff[4]), "v"(voff[5]), "v"(voff[6]),
        "v"(voff[7]), "s"(sbase), "s"(lds_addr)
      : "memory", "scc");
}

}  // namespace mfma
}  // namespace mla
