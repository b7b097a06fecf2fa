// Split-KV paged MLA decode for the quantised caches on the matrix cores
// (gfx950), for up to 128 query rows per sequence (several query tokens per
// sequence, as in a multi-token-prediction verify step).
//
// The fp8 row is 528 B: 512 e4m3 values (448 latent, then 64 RoPE) and 16
// e8m0 scales, one per 32 values (the GLM-4.7-Flash model record, ENGINE
// KERNEL CONSTRAINTS item (2)).  The fp4 row is 288 B (the same record's
// fp4 variant): 512 e2m1 codes and 32 e4m3 scales, one per 16 values.
//
// Two kernels.  decode_fp8_mx_kernel (fp8 rows, at most five row blocks)
// runs QK^T on the MX-scaled fp8 matrix cores: a cache row with its e8m0
// scales is exactly the A operand of v_mfma_scale_f32_16x16x128_f8f6f4, read
// from the raw rows in LDS, and the bf16 queries are split into fp8 hi + lo
// operands with their own scales.  Only V (the latent values) is decoded to
// bf16, by the waves that own no query rows, a tile ahead of PV.
//
// decode_fp8_kernel (fp4 rows, and fp8 rows with six to eight row blocks)
// decodes whole rows to bf16.  Per tile of 32 tokens:
//   1. the raw rows (one contiguous block when the tile lies in one page) go
//      from HBM to an LDS ring with direct-to-LDS loads, kRaw - 1 tiles
//      ahead of the one being computed;
//   2. all waves decode the raw tile into a bf16 tile, which is exact: an
//      e4m3 value times 2^(E-127) has 4 significant bits, an e2m1 value
//      times an e4m3 scale at most 6, and bf16 holds 8;
//   3. QK^T and PV run on v_mfma_f32_16x16x32_bf16 with the operand layouts
//      and swizzled bf16 tile of the bf16 kernel.  QK^T and the softmax are
//      split by 16-row blocks (one per wave); PV is split by column blocks,
//      each wave covering all rows, with P handed over through LDS.
// Up to four row blocks a workgroup has four waves, else eight.  One
// workgroup runs per CU (256 balanced workers); with at most two row blocks
// two run per CU (512 workers, a shallower ring, at most 256 registers per
// wave).  The per-tile cost is bound by LDS instructions (about 8 cycles per
// wave instruction), which the column split keeps to one transposed read
// per V chunk per tile.
//
// Online softmax, the rescale-free main loop and the partial layout follow
// the bf16 kernel: per row a reference maximum kept while scores stay
// within 2^64 of it; a tile that would exceed it sends the workgroup to a
// second loop that rescales.  Partials use the tiled matrix-core layout.
#include <cmath>
#include <type_traits>

#include "decode_common.h"
#include "device_common.h"
#include "internal.h"
#include "schedule.h"

namespace mla {
namespace {

using namespace mfma;

constexpr int kDc = 448;                       // latent width of the fp8 row
constexpr int kVals = kDc + kDr;               // 512 values per row
constexpr int kKs = kVals / 32;                // 16 QK k-steps
constexpr int kKsLat = kDc / 32;               // 14 over the latent
constexpr int kDb = kDc / 16;                  // 28 PV column blocks
// Stored row of each format: fp8 528 B (512 e4m3, then 16 e8m0 scales), fp4
// 288 B (256 B of e2m1 pairs, value 2i in the low nibble of byte i, then 32
// e4m3 scales, one per 16 values).
template <int FMT>
struct RawRow {
  static constexpr int kRowBytes = FMT == kFP8 ? kVals + kVals / 32 : kVals / 2 + kVals / 16;  // 528 / 288
  static constexpr int kChunksPerRow = kRowBytes / 16;      // 33 / 18 16-B chunks
  static constexpr int kRawChunks = kTile * kChunksPerRow;  // per tile
  static constexpr int kRawInst = (kRawChunks + 63) / 64;   // 17 / 9 wave loads per tile
  static constexpr int kRawBuf = kRawInst * 1024;           // raw buffer stride
};
// Raw ring depth: 4 buffers (3 tiles in flight) for one workgroup per CU;
// with at most two row blocks two workgroups share a CU, each with 2
// buffers (1 tile in flight), so that every SIMD has two waves.
template <int RB>
constexpr int raw_depth() { return RB <= 2 ? 2 : 4; }
// Converted bf16 tile, as in the bf16 kernel: latent rows (56 chunks) then
// the RoPE rows (8 chunks), chunks XOR-swizzled by token.
constexpr int kLatRow = kDc * 2;                   // 896
constexpr int kRopeRow = kDr * 2;                  // 128
constexpr int kRopeBase = kTile * kLatRow;         // 28672
constexpr int kTileBytes = kRopeBase + kTile * kRopeRow;  // 32768

// Raw tile loads: wave w issues instructions w, w + NW, ...; instruction k
// covers chunks 64k .. 64k + 63 of the tile (row q / kChunksPerRow, chunk
// q % kChunksPerRow).
template <int FMT, int NW>
struct RawStaging {
  using RR = RawRow<FMT>;
  static constexpr int kRowBytes = RR::kRowBytes, kRawChunks = RR::kRawChunks, kRawInst = RR::kRawInst;
  static constexpr int kMinOps = kRawInst / NW;  // fewest loads any wave issues per tile

  __device__ __forceinline__ static void load(const TileSrc& ts, lds_char* buf) {
    const int lane = threadIdx.x & 63;
    const int wave = uniform(threadIdx.x >> 6);
    if (ts.n == kTile && ts.kb >= kTile) {  // whole tile in one page: one contiguous block
#pragma unroll
      for (int i = 0; i < (kRawInst + NW - 1) / NW; ++i) {
        const int k = wave + NW * i;
        if (NW * i + NW <= kRawInst || k < kRawInst) {
          const int q = min(64 * k + lane, kRawChunks - 1);
          dma16((const void*)(uintptr_t)ts.base0, 16u * q, buf + 1024 * k);
        }
      }
      return;
    }
    // Last tile of a unit (rows past its end repeat the last valid one), or
    // a tile across two pages of 16 tokens.
#pragma unroll
    for (int i = 0; i < (kRawInst + NW - 1) / NW; ++i) {
      const int k = wave + NW * i;
      if (NW * i + NW <= kRawInst || k < kRawInst) {
        const int q = min(64 * k + lane, kRawChunks - 1);
        const int row = min(q / RR::kChunksPerRow, ts.n - 1), c = q % RR::kChunksPerRow;
        const uint64_t base = row < ts.kb ? ts.base0 : ts.base1;
        dma16_vaddr((const void*)(uintptr_t)(base + (uint64_t)(row * kRowBytes + 16 * c)), buf + 1024 * k);
      }
    }
  }

  // Gathered rows (sparse mode): lane j < 32 of a table register holds the
  // physical row of slot j, and each lane fetches its chunk's row from that
  // table with a cross-lane permute.
  __device__ __forceinline__ static void load_gather(const Gather& gt, const uint8_t* pool, lds_char* buf) {
    const int lane = threadIdx.x & 63;
    const int wave = uniform(threadIdx.x >> 6);
    int table = 0;
#pragma unroll
    for (int j = 0; j < kTile; ++j) table = lane == j ? (int)gt.phys[j] : table;
#pragma unroll
    for (int i = 0; i < (kRawInst + NW - 1) / NW; ++i) {
      const int k = wave + NW * i;
      if (NW * i + NW <= kRawInst || k < kRawInst) {
        const int q = min(64 * k + lane, kRawChunks - 1);
        const int row = q / RR::kChunksPerRow, c = q % RR::kChunksPerRow;
        const uint32_t phys = (uint32_t)__builtin_amdgcn_ds_bpermute(row << 2, table);
        dma16_vaddr(pool + (uint64_t)phys * kRowBytes + 16 * c, buf + 1024 * k);
      }
    }
  }
};

typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
typedef int i32x8 __attribute__((ext_vector_type(8)));

// ---- fp8 rows on the MX-scaled fp8 matrix cores (QK^T) ----
// v_mfma_scale_f32_16x16x128_f8f6f4 with both operands e4m3: lane l of a wave
// (g = l / 16) holds row or column l % 16 of its operand, with K values
// 16g .. 16g+15 in bytes 0..15 and 64+16g .. 64+16g+15 in bytes 16..31 (as
// measured on gfx950), and its scale register holds the e8m0 scale of K block
// g (values 32g .. 32g+31); the product is
//   D[i][j] = sum_k A[i][k] 2^(sa(i, k/32) - 127) B[k][j] 2^(sb(j, k/32) - 127),
// returned in the layout of the bf16 16x16x32 instruction.  A cache row's 512
// values with one e8m0 scale per 32 of them are exactly such an operand, read
// straight from the raw rows in LDS.  The bf16 queries are split into two
// such operands, hi + lo, each with its own block scales: hi holds the four
// leading significant bits of every value, lo the next four of the residual,
// so the two products sum to the bf16 query's scores up to about 2^-8 of each
// 32-value block's largest magnitude.

// e8m0 exponent for a block whose largest magnitude is b: the smallest e with
// b / 2^e <= 448 (the largest e4m3 value), at least -127.
__device__ __forceinline__ int mx_exp(float b) {
  if (!(b > 0.f)) return -127;
  int E;
  const float f = frexpf(b, &E);  // b = f 2^E, f in [0.5, 1); 448 = 0.875 2^9
  return max(f > 0.875f ? E - 8 : E - 9, -127);
}

// The scale this lane supplies: block g's e8m0 code.  Blocks 0 and 3 are the
// lane's own halves (g = 0: first half, g = 3: second); block 1 is the first
// half of group 2 (lane l + 16 for g = 1), block 2 the second half of group 1
// (lane l - 16 for g = 2).  A scale register holds four codes, one per byte;
// the instruction's op_sel picks the byte (as measured on gfx950).
__device__ __forceinline__ int mx_scale_code(int e0, int e1, int lane) {
  const int c0 = e0 + 127, c1 = e1 + 127;
  const int up = __shfl(c0, (lane + 16) & 63);
  const int dn = __shfl(c1, (lane + 48) & 63);
  const int g = lane >> 4;
  return g == 0 ? c0 : g == 1 ? up : g == 2 ? dn : c1;
}

// One scaled fp8 product with the scales of K step KS (byte KS of both
// scale registers); mfma_mx picks KS at compile time once loops are unrolled.
template <int KS>
__device__ __forceinline__ f32x4 mfma_mx_step(const i32x8& a, const i32x8& b, f32x4 c, uint32_t sa, uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, KS, (int)sa, KS, (int)sb);
}
__device__ __forceinline__ f32x4 mfma_mx(int ks, const i32x8& a, const i32x8& b, f32x4 c, uint32_t sa, uint32_t sb) {
  switch (ks) {
    case 0: return mfma_mx_step<0>(a, b, c, sa, sb);
    case 1: return mfma_mx_step<1>(a, b, c, sa, sb);
    case 2: return mfma_mx_step<2>(a, b, c, sa, sb);
    default: return mfma_mx_step<3>(a, b, c, sa, sb);
  }
}

// One query row's bf16 values as this lane's hi and lo B operands for the 4
// K steps of a 512-value row (all lanes of the wave take part).
struct MxQuery {
  i32x8 hi[kVals / 128], lo[kVals / 128];
  uint32_t sh, sl;  // byte ks: the scale of K step ks
};

__device__ __forceinline__ void mx_query(const uint16_t* row, bool row_ok, int lane, MxQuery& mq) {
  const int g = lane >> 4;
  mq.sh = mq.sl = 0u;
#pragma unroll
  for (int ks = 0; ks < kVals / 128; ++ks) {
    // this lane's 32 values: j < 16 from K 16g + j, j >= 16 from 64 + 16g + j - 16
    u32x4 w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int off = 128 * ks + (i < 2 ? 0 : 64) + 16 * g + 8 * (i & 1);
      w[i] = row_ok ? *reinterpret_cast<const u32x4*>(row + off) : u32x4{0u, 0u, 0u, 0u};
    }
    auto val = [&](int j) {
      const uint32_t d = w[j >> 3][(j & 7) >> 1];
      return __uint_as_float((j & 1) ? (d & 0xFFFF0000u) : (d << 16));
    };
    // e4m3 codes of four values scaled by 2^-e (clamped to the e4m3 range)
    auto code4 = [&](int e, float (&x)[4]) {
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = __builtin_amdgcn_fmed3f(ldexpf(x[i], -e), -448.f, 448.f);
      const int c = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
      return __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], c, true);
    };
    // values 4k..4k+3 minus their hi codes c (block exponent e)
    auto residual4 = [&](int k, int e, int c, float (&r)[4]) {
      const f32x2 d0 = __builtin_amdgcn_cvt_pk_f32_fp8(c, false);
      const f32x2 d1 = __builtin_amdgcn_cvt_pk_f32_fp8(c, true);
      r[0] = val(4 * k + 0) - ldexpf(d0[0], e);
      r[1] = val(4 * k + 1) - ldexpf(d0[1], e);
      r[2] = val(4 * k + 2) - ldexpf(d1[0], e);
      r[3] = val(4 * k + 3) - ldexpf(d1[1], e);
    };
    // hi: block maxima over this lane's halves and lane l ^ 16's
    float m0 = 0.f, m1 = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      m0 = fmaxf(m0, fabsf(val(j)));
      m1 = fmaxf(m1, fabsf(val(16 + j)));
    }
    m0 = fmaxf(m0, __shfl_xor(m0, 16));
    m1 = fmaxf(m1, __shfl_xor(m1, 16));
    const int e0 = mx_exp(m0), e1 = mx_exp(m1);
    float r0 = 0.f, r1 = 0.f;  // residual block maxima
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int e = k < 4 ? e0 : e1;
      float x[4] = {val(4 * k), val(4 * k + 1), val(4 * k + 2), val(4 * k + 3)};
      const int c = code4(e, x);
      mq.hi[ks][k] = c;
      float r[4];
      residual4(k, e, c, r);
      const float rm = fmaxf(fmaxf(fabsf(r[0]), fabsf(r[1])), fmaxf(fabsf(r[2]), fabsf(r[3])));
      if (k < 4) r0 = fmaxf(r0, rm);
      else r1 = fmaxf(r1, rm);
    }
    mq.sh |= (uint32_t)mx_scale_code(e0, e1, lane) << (8 * ks);
    // lo: the residuals (recomputed from the hi codes) with their own scales
    r0 = fmaxf(r0, __shfl_xor(r0, 16));
    r1 = fmaxf(r1, __shfl_xor(r1, 16));
    const int f0 = mx_exp(r0), f1 = mx_exp(r1);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      float r[4];
      residual4(k, k < 4 ? e0 : e1, mq.hi[ks][k], r);
      mq.lo[ks][k] = code4(k < 4 ? f0 : f1, r);
    }
    mq.sl |= (uint32_t)mx_scale_code(f0, f1, lane) << (8 * ks);
    __builtin_amdgcn_sched_barrier(0);  // one K step's temporaries at a time
  }
}

// One fp8 unit: 16 values v (chunk c of 32 of token tok's row) with their
// e8m0 scale code, decoded exactly into bf16 chunks 2c and 2c + 1 of the
// tile (zeros if zero).
__device__ __forceinline__ void fp8_convert(u32x4 v, uint32_t scale_code, lds_char* tile, int tok, int c,
                                            bool zero) {
  // e4m3 * 2^(E-127) is exact in bf16: one scaled conversion per pair of
  // values (checked bit for bit on gfx950 for every finite code and scale
  // exponents 2^-27 .. 2^28)
  const float scale = e8m0_to_f32(scale_code);
  uint32_t o[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i + 0] = zero ? 0u : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[i], scale, false));
    o[2 * i + 1] = zero ? 0u : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[i], scale, true));
  }
  const int c0 = 2 * c;  // first bf16 chunk of these 16 values
  lds_char* d0 = c0 < kDc / 8 ? tile + lds_off(tok, c0, kLatRow)
                              : tile + kRopeBase + lds_off(tok, c0 - kDc / 8, kRopeRow);
  lds_char* d1 = c0 < kDc / 8 ? tile + lds_off(tok, c0 + 1, kLatRow)
                              : tile + kRopeBase + lds_off(tok, c0 + 1 - kDc / 8, kRopeRow);
  *(lds_u32x4*)d0 = u32x4{o[0], o[1], o[2], o[3]};
  *(lds_u32x4*)d1 = u32x4{o[4], o[5], o[6], o[7]};
}
__device__ __forceinline__ void fp8_unit(const lds_char* src, lds_char* tile, int tok, int c, bool zero) {
  const u32x4 v = *(const lds_u32x4*)(src + 16 * c);
  fp8_convert(v, (uint32_t)(uint8_t)src[kVals + (c >> 1)], tile, tok, c, zero);
}

// fp8 rows for the MX path: only the latent values (V) go to the bf16 tile,
// 28 units of 16 values per token, over NTHR threads numbered from tid.  All
// of a thread's raw reads are issued before the first conversion, so that
// the LDS latency is paid once per tile.
template <bool SPARSE, int NTHR>
__device__ __forceinline__ void decode_v_fp8(const lds_char* raw, lds_char* tile, uint32_t vis, int tid) {
  constexpr int kRowBytes = RawRow<kFP8>::kRowBytes;
  constexpr int kPerTok = kDc / 16;
  constexpr int kUnits = kTile * kPerTok;
  constexpr int kIter = (kUnits + NTHR - 1) / NTHR;
  u32x4 v[kIter];
  uint32_t sc[kIter];
#pragma unroll
  for (int i = 0; i < kIter; ++i) {
    const int u = min(tid + i * NTHR, kUnits - 1);
    const int tok = u / kPerTok, c = u - tok * kPerTok;
    const lds_char* src = raw + tok * kRowBytes;
    v[i] = *(const lds_u32x4*)(src + 16 * c);
    sc[i] = (uint32_t)(uint8_t)src[kVals + (c >> 1)];
  }
#pragma unroll
  for (int i = 0; i < kIter; ++i) {
    const int u = tid + i * NTHR;
    if (u < kUnits) {
      const int tok = u / kPerTok, c = u - tok * kPerTok;
      fp8_convert(v[i], sc[i], tile, tok, c, SPARSE && !((vis >> tok) & 1u));
    }
  }
}

// Decode a raw tile into the bf16 tile: unit u = (token u / 32, value chunk
// u % 32 of 16 values), spread over all threads of the workgroup.
// In sparse mode a slot outside `vis` (padding) is written as zeros, so that
// whatever its gathered row holds, its P = 0 weight multiplies a finite value.
template <int FMT, int NW, bool SPARSE>
__device__ __forceinline__ void decode_tile(const lds_char* raw, lds_char* tile, uint32_t vis) {
  constexpr int kRowBytes = RawRow<FMT>::kRowBytes;
  for (int u = threadIdx.x; u < kTile * 32; u += 64 * NW) {
    const int tok = u >> 5, c = u & 31;
    const lds_char* src = raw + tok * kRowBytes;
    const bool zero = SPARSE && !((vis >> tok) & 1u);
    if constexpr (FMT == kFP4) {
      // 16 e2m1 codes (8 bytes) and their e4m3 scale.  The hardware converts
      // a byte's two codes (low nibble first) with a unit scale; an e2m1 value
      // times an e4m3 scale has at most 6 significant bits, so the bf16 value
      // is the upper half of the exact fp32 product.
      const u32x2 v = *(const lds_u32x2*)(src + 8 * c);
      const float scale = e4m3fn_to_f32((uint32_t)(uint8_t)src[kVals / 2 + c]);
      const f32x2 p[8] = {__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v[0], 1.0f, 0),
                          __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v[0], 1.0f, 1),
                          __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v[0], 1.0f, 2),
                          __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v[0], 1.0f, 3),
                          __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v[1], 1.0f, 0),
                          __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v[1], 1.0f, 1),
                          __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v[1], 1.0f, 2),
                          __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v[1], 1.0f, 3)};
      uint32_t o[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        o[i] = zero ? 0u
                    : __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, p[i][1] * scale),
                                            __builtin_bit_cast(uint32_t, p[i][0] * scale), 0x07060302u);
      const int c0 = 2 * c;
      lds_char* d0 = c0 < kDc / 8 ? tile + lds_off(tok, c0, kLatRow)
                                  : tile + kRopeBase + lds_off(tok, c0 - kDc / 8, kRopeRow);
      lds_char* d1 = c0 < kDc / 8 ? tile + lds_off(tok, c0 + 1, kLatRow)
                                  : tile + kRopeBase + lds_off(tok, c0 + 1 - kDc / 8, kRopeRow);
      *(lds_u32x4*)d0 = u32x4{o[0], o[1], o[2], o[3]};
      *(lds_u32x4*)d1 = u32x4{o[4], o[5], o[6], o[7]};
      continue;
    }
    fp8_unit(src, tile, tok, c, zero);
  }
}

// Waves split the work two ways.  Wave w < RB owns query rows 16w..16w+15
// for QK^T and the softmax (its queries stay in registers); every wave owns
// the PV column blocks [w*kDb/NW, (w+1)*kDb/NW) for all RB row blocks.  P
// goes from the row owners to all waves through LDS, so each transposed V
// read feeds RB MFMAs and every V column block is read once per tile.
//
// Sparse mode (SPARSE): a unit is one (sequence, query token) pair and its
// tiles are 32 consecutive slots of that query's index list, gathered as in
// the bf16 kernel's sparse mode; the slots' visibility masks ride with the
// raw ring in LDS.
template <int FMT, int NW, int RB, bool SPARSE = false>
__global__ __launch_bounds__(64 * NW, raw_depth<RB>() == 2 ? 2 : 1) void decode_fp8_kernel(DecodeArgs a) {
  constexpr int kRawBuf = RawRow<FMT>::kRawBuf;
  constexpr int kRaw = raw_depth<RB>();
  using Raw = RawStaging<FMT, NW>;
  static_assert(RB >= 1 && RB <= NW, "row blocks are owned by distinct waves");
  constexpr int kCols = (kDb + NW - 1) / NW;  // most column blocks a wave owns
  __shared__ __attribute__((aligned(16))) char tile_mem[kTileBytes];
  __shared__ __attribute__((aligned(16))) char raw_mem[kRaw * kRawBuf];
  __shared__ __attribute__((aligned(16))) char p_mem[RB * 64 * 16];  // P per row block, A-operand layout
  __shared__ __attribute__((aligned(16))) float s_row[RB][16];       // per row: rescale factor, then 1/sum
  __shared__ __attribute__((aligned(16))) int32_t s_flag[8];         // per row block: 0, 1 rescaled, 2 overflow
  __shared__ int32_t s_ts[kMaxInKernelPlan + 2];
  __shared__ int32_t s_lens[kMaxInKernelPlan];
  __shared__ int32_t s_first;
  __shared__ uint32_t s_mask[kRaw];  // sparse: visible-slot mask per raw ring buffer
  lds_char* const tile = (lds_char*)tile_mem;
  lds_char* const raws = (lds_char*)raw_mem;
  lds_char* const pbuf = (lds_char*)p_mem;

  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int li = lane & 15;
  const int row_blocks = (a.R + 15) / 16;
  const bool owner = wave < RB;
  const int row = wave * 16 + li;  // the owner's query row for this lane (B / P side)
  const bool row_ok = owner && row < a.R;
  const int c_begin = wave * kDb / NW;
  const int c_count = (wave + 1) * kDb / NW - c_begin;

  const int32_t* ts = a.tile_start;
  if (a.num_splits == 0 && a.plan_in_kernel) {
    if (threadIdx.x < 64) wave_plan(a.seq_lens, a.B, a.workers, s_ts, s_lens, &s_first);
    __syncthreads();
    if (blockIdx.x == 0)  // publish the plan for the merge kernel
      for (int i = threadIdx.x; i <= a.B + 1; i += 64 * NW) a.tile_start[i] = s_ts[i];
    ts = s_ts;
  }
  constexpr int D = kRaw - 1;  // raw tiles in flight ahead of the one being decoded
  UnitIter unit_it(a, ts, ts == s_ts ? s_lens : a.seq_lens, ts == s_ts ? s_first : -1);
  Unit unit;
  while (unit_it.next(a, unit)) {
    const int b = uniform(unit.b), L = uniform(unit.L), t0 = uniform(unit.t0), t1 = uniform(unit.t1);
    const int64_t slot = unit.slot;
    const int ntiles = uniform((t1 - t0 + kTile - 1) / kTile);
    // Sparse: unit b is query token b % sparse_sq of sequence b / sparse_sq,
    // which sees positions up to L - Sq + j of that sequence.
    const int sb = SPARSE ? uniform(b / a.sparse_sq) : b;
    const int sparse_limit =
        SPARSE ? uniform(max(((const_i32_ptr)a.seq_lens)[sb], 0) - a.sparse_sq + b % a.sparse_sq) : 0;
    const const_i32_ptr list = (const_i32_ptr)(a.topk) + (SPARSE ? (int64_t)b * a.topk_width : 0);
    const const_i32_ptr bt = (const_i32_ptr)(a.block_table) + (int64_t)sb * a.max_blocks;
    // Issue the raw rows of tile x (sparse: gathered, with its mask).
    auto issue = [&](int x, const TilePages& tp, const Gather& gt) __attribute__((always_inline)) {
      if constexpr (SPARSE) {
        Raw::load_gather(gt, a.pool, raws + (x % kRaw) * kRawBuf);
        if (threadIdx.x == 0) s_mask[x % kRaw] = gt.mask;
      } else {
        Raw::load(tile_src(a, tp, t1), raws + (x % kRaw) * kRawBuf);
      }
    };

    // ---- queries (bf16, B-operand layout) of the owned row block ----
    // Loaded and waited for before any tile transfer, so that later waits
    // on the transfers are not mixed up with the query loads.
    bf16x8 q[kKs];
    {
      const uint16_t* src = static_cast<const uint16_t*>(a.q_abs) + ((int64_t)b * a.R + (row_ok ? row : 0)) * kVals + 8 * g;
#pragma unroll
      for (int ks = 0; ks < kKs; ++ks) {
        q[ks] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
        if (row_ok) q[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(src + 32 * ks));
      }
    }
    wait_vmcnt_lgkm0<0>();

    f32x4 acc[RB][kCols];
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
      for (int d = 0; d < kCols; ++d) acc[r][d] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, lsum = 0.f;  // the owner's row statistics (base 2)

    TilePages pages_next;
    Gather gnext;  // sparse: rows of the next tile to issue, looked up one tile early
    if (ntiles > 0) {
      lds_barrier();  // the previous unit's readers of the tile, ring and P are done
#pragma unroll
      for (int x = 0; x < D; ++x)
        if (x < ntiles) {
          if constexpr (SPARSE) issue(x, pages_next, gather_lookup(a, list, bt, t0 + x * kTile, t1, sparse_limit));
          else issue(x, tile_pages(a, bt, t0 + x * kTile, t1), gnext);
        }
      if (D < ntiles) {
        if constexpr (SPARSE) gnext = gather_lookup(a, list, bt, t0 + D * kTile, t1, sparse_limit);
        else pages_next = tile_pages(a, bt, t0 + D * kTile, t1);
      }
    }

    // One pipeline step: tile `it` has landed in the ring (everyone's part),
    // the transfer of tile it + D starts into the buffer tile it-1 used, and
    // tile `it` is decoded into the bf16 tile once everyone is done with
    // tile it-1.
    auto step = [&](int it) __attribute__((always_inline)) {
      const int younger = min(D - 1, ntiles - 1 - it);
      constexpr int M = Raw::kMinOps;
      if (younger >= 2) wait_vmcnt_lgkm0<2 * M>();
      else if (younger == 1) wait_vmcnt_lgkm0<M>();
      else wait_vmcnt_lgkm0<0>();
      lds_barrier();  // tile `it` landed; everyone finished tile it-1
      const int x = it + D;
      if (x < ntiles) {
        issue(x, pages_next, gnext);
        if (x + 1 < ntiles) {
          if constexpr (SPARSE) gnext = gather_lookup(a, list, bt, t0 + (x + 1) * kTile, t1, sparse_limit);
          else pages_next = tile_pages(a, bt, t0 + (x + 1) * kTile, t1);
        }
      }
      decode_tile<FMT, NW, SPARSE>(raws + (it % kRaw) * kRawBuf, tile, SPARSE ? s_mask[it % kRaw] : ~0u);
      wait_lgkm0();
      lds_barrier();  // the bf16 tile is complete
    };

    // Per row a reference maximum m, set by the first tile with a visible
    // token.  The main loop keeps it while scores stay below m + 64 (P
    // cannot overflow, and P, the sum and the accumulators share m); a tile
    // beyond that is redone by the second loop, which raises m when a score
    // exceeds it by 8 and rescales the accumulators of that row block.
    constexpr float kHeadroom = 64.f;
    auto compute = [&](int it, auto rescale_tag) __attribute__((always_inline)) -> bool {
      constexpr bool kRescale = decltype(rescale_tag)::value;
      const float m_save = m, lsum_save = lsum;
      if (owner) {
        const int tt0 = t0 + it * kTile;
        // ---- S^T = Tile . Q^T for the two token blocks ----
        f32x4 s[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
        const lds_char* lat_base[2][2];
        const lds_char* rope_base[2][2];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          const int tok = tb * 16 + li;
          const int xs = swz(tok);
          const int flip = 64 * (xs >> 2);
          const lds_char* bl = tile + tok * kLatRow + 16 * (g ^ (xs & 3));
          const lds_char* br = tile + kRopeBase + tok * kRopeRow + 16 * (g ^ (xs & 3));
          lat_base[tb][0] = bl + flip;
          lat_base[tb][1] = bl - flip;
          rope_base[tb][0] = br + flip;
          rope_base[tb][1] = br - flip;
        }
        auto tile_a = [&](int ks, int tb) {
          const lds_char* p = ks < kKsLat ? lat_base[tb][ks & 1] + 64 * ks : rope_base[tb][ks & 1] + 64 * (ks - kKsLat);
          return *(const lds_bf16x8*)p;
        };
        constexpr int kAhead = NW > 4 ? 2 : 3;  // two waves per SIMD: half the registers
        bf16x8 ta[kAhead][2];
#pragma unroll
        for (int k = 0; k < kAhead; ++k) {
          ta[k][0] = tile_a(k, 0);
          ta[k][1] = tile_a(k, 1);
        }
#pragma unroll
        for (int ks = 0; ks < kKs; ++ks) {
          const bf16x8 a0 = ta[ks % kAhead][0], a1 = ta[ks % kAhead][1];
          if (ks + kAhead < kKs) {
            ta[ks % kAhead][0] = tile_a(ks + kAhead, 0);
            ta[ks % kAhead][1] = tile_a(ks + kAhead, 1);
          }
          s[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, q[ks], s[0], 0, 0, 0);
          s[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, q[ks], s[1], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }

        // ---- online softmax of the owned rows ----
        const int last_visible = L - a.Sq + (row_ok ? row / a.H : 0);
        const uint32_t vis = SPARSE ? s_mask[it % kRaw] : ~0u;
        float sv[2][4], mx = -INFINITY;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = tt0 + tb * 16 + 4 * g + i;
            const bool ok = SPARSE ? row_ok && ((vis >> (tb * 16 + 4 * g + i)) & 1u)
                                   : row_ok && t < t1 && t <= last_visible;
            sv[tb][i] = ok ? s[tb][i] * a.scale_log2 : -INFINITY;
            mx = fmaxf(mx, sv[tb][i]);
          }
        mx = max_over_rows(mx);
        int flag = 0;
        if constexpr (kRescale) {
          const bool raise = mx > m + 8.f;  // also true when m = -inf < mx
          if (__any(raise)) {
            const float m_new = raise ? mx : m;
            const float alpha = m == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m - m_new);
            lsum *= alpha;
            m = m_new;
            if (g == 0) s_row[wave][li] = alpha;
            flag = 1;
          }
        } else {
          if (__any(m != -INFINITY && mx > m + kHeadroom)) flag = 2;
          else m = m == -INFINITY ? mx : m;
        }
        if (flag != 2) {
          float psum = 0.f;
          uint32_t pk[4];
#pragma unroll
          for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int i = 0; i < 4; i += 2) {
              const float e0 = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv[tb][i] - m);
              const float e1 = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv[tb][i + 1] - m);
              psum += e0 + e1;
              pk[2 * tb + i / 2] = pack_bf16(e0, e1);
            }
          psum = sum_over_rows(psum);
          lsum += psum;
          *(lds_u32x4*)(pbuf + (wave * 64 + lane) * 16) = u32x4{pk[0], pk[1], pk[2], pk[3]};
        }
        if (lane == 0) s_flag[wave] = flag;
      }
      wait_lgkm0();
      lds_barrier();  // P, flags and rescale factors of every row block are in LDS

      int flags[RB];
#pragma unroll
      for (int r = 0; r < RB; ++r) flags[r] = uniform(s_flag[r]);
      if constexpr (!kRescale) {
        bool over = false;
#pragma unroll
        for (int r = 0; r < RB; ++r) over = over || flags[r] == 2;
        if (over) {  // every wave sees the same flags: redo this tile in the second loop
          m = m_save;
          lsum = lsum_save;
          return false;
        }
      } else {
#pragma unroll
        for (int r = 0; r < RB; ++r)
          if (flags[r] == 1) {
            const f32x4 al4 = *(const lds_f32x4*)(&s_row[r][4 * g]);
            const float4 al = make_float4(al4[0], al4[1], al4[2], al4[3]);
#pragma unroll
            for (int d = 0; d < kCols; ++d) {
              acc[r][d][0] *= al.x;
              acc[r][d][1] *= al.y;
              acc[r][d][2] *= al.z;
              acc[r][d][3] *= al.w;
            }
          }
      }
      bf16x8 pa[RB];
#pragma unroll
      for (int r = 0; r < RB; ++r) pa[r] = *(const lds_bf16x8*)(pbuf + (r * 64 + lane) * 16);

      // ---- O[:, own columns] += P . V, each V read feeding every row block ----
      const lds_char* vbase[2][4];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int tok = 16 * half + 4 * g + (li >> 2);
        const int xs = swz(tok);
        const int h = (li & 3) >> 1;
        const lds_char* b0 = tile + tok * kLatRow + 16 * (h ^ (xs & 1)) + 8 * (li & 1);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) vbase[half][rr] = b0 + 32 * (rr ^ (xs >> 1));
      }
      auto tile_v = [&](int c) {
        const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vbase[0][c & 3] + 128 * (c >> 2)));
        const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vbase[1][c & 3] + 128 * (c >> 2)));
        return __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
      };
      constexpr int kPrefetch = NW > 4 ? 2 : kCols < 4 ? kCols : 4;
      bf16x8 vq[kPrefetch];
#pragma unroll
      for (int d = 0; d < kPrefetch; ++d) vq[d] = tile_v(c_begin + min(d, c_count - 1));
#pragma unroll
      for (int d = 0; d < kCols; ++d) {
        if (d < c_count) {
          const bf16x8 vb = vq[d % kPrefetch];
          if (d + kPrefetch < kCols) vq[d % kPrefetch] = tile_v(c_begin + min(d + kPrefetch, c_count - 1));
#pragma unroll
          for (int r = 0; r < RB; ++r) acc[r][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[r], vb, acc[r][d], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      return true;
    };

    int it = 0;
    for (; it < ntiles; ++it) {
      step(it);
      if (!compute(it, std::false_type{})) break;
    }
    if (it < ntiles) {  // tile `it` is decoded but not yet computed
      compute(it, std::true_type{});
      for (++it; it < ntiles; ++it) {
        step(it);
        compute(it, std::true_type{});
      }
    }

    // ---- normalise and write this unit's partials (tiled layout) ----
    if (owner) {
      if (g == 0) {
        s_row[wave][li] = lsum > 0.f ? 1.f / lsum : 0.f;
        if (row_ok) a.part_lse[slot * a.R + row] = lsum > 0.f ? (m + log2f(lsum)) * kLn2 : -INFINITY;
      }
    }
    wait_lgkm0();
    lds_barrier();  // every row's 1/sum is in LDS
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      if (r * 16 + 4 * g >= a.R) continue;  // lanes holding only padding rows
      const f32x4 inv4 = *(const lds_f32x4*)(&s_row[r][4 * g]);
      const float4 inv = make_float4(inv4[0], inv4[1], inv4[2], inv4[3]);
      float* dst = a.part_o + ((slot * row_blocks + r) * kDb * 64 + lane) * 4;
#pragma unroll
      for (int d = 0; d < kCols; ++d)
        if (d < c_count)
          *reinterpret_cast<float4*>(dst + 256 * (c_begin + d)) =
              make_float4(acc[r][d][0] * inv.x, acc[r][d][1] * inv.y, acc[r][d][2] * inv.z, acc[r][d][3] * inv.w);
    }
  }
}


// ---- fp8 rows with at most five row blocks: the MX kernel ----
// Eight waves, one workgroup per CU.  Waves 0..RB-1 own the query row
// blocks: per tile they run QK^T on the MX-scaled fp8 matrix cores straight
// from the raw rows in the ring, then the online softmax, and hand P to the
// other waves through LDS.  Those (the workers) decode the tile's latent
// values (V) to bf16.  Every wave runs PV over its share of the column blocks
// one tile behind the scores.  A step has one barrier: in step s the owners
// score tile s + 1 while the workers decode it, and every wave accumulates
// tile s, so both kinds of matrix work and the conversions overlap on every
// SIMD.  P, the bf16 V tile and the rescale factors are double-buffered by
// tile parity.  Measured on 64 sequences x 4 query tokens x 20 heads of 16k
// fp8 tokens: 310 us against 403 us for the bf16-decoding kernel.
//
// Softmax: per row a reference maximum m, raised when a tile's scores exceed
// it by more than 8 (the row's sum and accumulators are then scaled by
// 2^(m_old - m_new)), so P = 2^(s - m) <= 2^8 always fits bf16.
constexpr int kMxWaves = 8;
constexpr int kMxMaxRowBlocks = 5;
constexpr int kMxStage = 16896;  // one owner's staged queries: hi, lo (8 KB each), scales
typedef __attribute__((address_space(3))) i32x8 lds_i32x8;

// PV column blocks of row owner w: waves w and w + 4 share a SIMD, so an
// owner sharing its SIMD with another owner (whose QK^T is the largest matrix
// job of a step) takes one column block, the others three; the workers split
// the rest.  With five row blocks this evens the matrix work of the SIMDs.
template <int RB>
constexpr int mx_owner_cols(int w) { return (w + 4 < RB || (w >= 4 && w - 4 < RB)) ? 1 : 3; }
template <int RB>
constexpr int mx_owner_cols_before(int w) {
  int t = 0;
  for (int v = 0; v < w && v < RB; ++v) t += mx_owner_cols<RB>(v);
  return t;
}

template <int RB, bool SPARSE>
__global__ __launch_bounds__(64 * kMxWaves, 1) void decode_fp8_mx_kernel(DecodeArgs a) {
  constexpr int NW = kMxWaves;
  constexpr int kRowBytes = RawRow<kFP8>::kRowBytes;
  constexpr int kRawBuf = RawRow<kFP8>::kRawBuf;
  constexpr int kRaw = 4;  // ring buffers: three tiles in flight (four measured no faster)
  constexpr int D = kRaw - 1;
  constexpr int kWk = NW - RB;                       // workers
  constexpr int kOC = 3;                             // most PV column blocks of an owner
  constexpr int kOTotal = mx_owner_cols_before<RB>(RB);  // of all owners
  constexpr int kWTotal = kDb - kOTotal;             // ... and of all workers
  constexpr int kWC = (kWTotal + kWk - 1) / kWk;     // most column blocks a worker owns
  constexpr int kSteps = kVals / 128;          // K steps of QK^T
  using Raw = RawStaging<kFP8, NW>;
  static_assert(RB >= 1 && RB <= kMxMaxRowBlocks, "row blocks");
  static_assert(4 * kMxStage <= kRaw * kRawBuf && (kMxMaxRowBlocks - 4) * kMxStage <= 2 * kRopeBase,
                "staged queries fit the ring and V buffers");
  __shared__ __attribute__((aligned(16))) char v_mem[2][kRopeBase];   // bf16 V tiles
  __shared__ __attribute__((aligned(16))) char raw_mem[kRaw * kRawBuf];
  __shared__ __attribute__((aligned(16))) char p_mem[2][RB * 64 * 16];  // P per row block, A-operand layout
  __shared__ __attribute__((aligned(16))) float s_alpha[2][RB][16];     // per row: the tile's rescale factor
  __shared__ __attribute__((aligned(16))) float s_inv[RB][16];          // per row: 1 / sum
  __shared__ int32_t s_flag[2][RB];                                     // per row block: rescaled in the tile
  __shared__ int32_t s_ts[kMaxInKernelPlan + 2];
  __shared__ int32_t s_lens[kMaxInKernelPlan];
  __shared__ int32_t s_first;
  __shared__ uint32_t s_mask[kRaw];  // sparse: visible-slot mask per raw ring buffer
  lds_char* const raws = (lds_char*)raw_mem;

  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int li = lane & 15;
  const int row_blocks = (a.R + 15) / 16;
  const bool owner = wave < RB;
  const int row = wave * 16 + li;  // the owner's query row for this lane
  const bool row_ok = owner && row < a.R;

  const int32_t* ts = a.tile_start;
  if (a.num_splits == 0 && a.plan_in_kernel) {
    if (threadIdx.x < 64) wave_plan(a.seq_lens, a.B, a.workers, s_ts, s_lens, &s_first);
    __syncthreads();
    if (blockIdx.x == 0)  // publish the plan for the merge kernel
      for (int i = threadIdx.x; i <= a.B + 1; i += 64 * NW) a.tile_start[i] = s_ts[i];
    ts = s_ts;
  }
  UnitIter unit_it(a, ts, ts == s_ts ? s_lens : a.seq_lens, ts == s_ts ? s_first : -1);

  // The unit loop of one role (owner or worker); both roles pass the same
  // barriers.
  auto run = [&](auto owner_tag) __attribute__((always_inline)) {
    constexpr bool kOwner = decltype(owner_tag)::value;
    const int wk = wave - RB;  // worker index
    constexpr int kC = kOwner ? kOC : kWC;  // accumulator column blocks
    int c_begin, c_count;
    if constexpr (kOwner) {
      c_begin = 0;
      c_count = 0;
      for (int v = 0; v < RB; ++v) {  // wave-uniform
        if (v < wave) c_begin += mx_owner_cols<RB>(v);
        if (v == wave) c_count = mx_owner_cols<RB>(v);
      }
    } else {
      c_begin = kOTotal + wk * kWTotal / kWk;
      c_count = kOTotal + (wk + 1) * kWTotal / kWk - c_begin;
    }
    Unit unit;
    while (unit_it.next(a, unit)) {
      const int b = uniform(unit.b), L = uniform(unit.L), t0 = uniform(unit.t0), t1 = uniform(unit.t1);
      const int64_t slot = unit.slot;
      const int ntiles = uniform((t1 - t0 + kTile - 1) / kTile);
      const int sb = SPARSE ? uniform(b / a.sparse_sq) : b;
      const int sparse_limit =
          SPARSE ? uniform(max(((const_i32_ptr)a.seq_lens)[sb], 0) - a.sparse_sq + b % a.sparse_sq) : 0;
      const const_i32_ptr list = (const_i32_ptr)(a.topk) + (SPARSE ? (int64_t)b * a.topk_width : 0);
      const const_i32_ptr bt = (const_i32_ptr)(a.block_table) + (int64_t)sb * a.max_blocks;
      auto issue = [&](int x, const TilePages& tp, const Gather& gt) __attribute__((always_inline)) {
        if constexpr (SPARSE) {
          Raw::load_gather(gt, a.pool, raws + (x % kRaw) * kRawBuf);
          if (threadIdx.x == 0) s_mask[x % kRaw] = gt.mask;
        } else {
          Raw::load(tile_src(a, tp, t1), raws + (x % kRaw) * kRawBuf);
        }
      };

      // Queries as fp8 hi + lo operands, made before any tile transfer.
      // They pass through LDS (the ring and V buffers are free between
      // units), so that the registers holding them during the tile loop are
      // not also tied up by the arithmetic that made them.
      MxQuery mq;
      if constexpr (kOwner) {
        MxQuery made;
        mx_query(static_cast<const uint16_t*>(a.q_abs) + ((int64_t)b * a.R + (row_ok ? row : 0)) * kVals, row_ok,
                 lane, made);
        lds_char* const st = wave < 4 ? raws + wave * kMxStage : (lds_char*)v_mem + (wave - 4) * kMxStage;
#pragma unroll
        for (int ks = 0; ks < kSteps; ++ks) {
          *(lds_i32x8*)(st + (ks * 64 + lane) * 32) = made.hi[ks];
          *(lds_i32x8*)(st + 8192 + (ks * 64 + lane) * 32) = made.lo[ks];
        }
        *(lds_u32x2*)(st + 16384 + lane * 8) = u32x2{made.sh, made.sl};
        asm volatile("" ::: "memory");
#pragma unroll
        for (int ks = 0; ks < kSteps; ++ks) {
          mq.hi[ks] = *(const lds_i32x8*)(st + (ks * 64 + lane) * 32);
          mq.lo[ks] = *(const lds_i32x8*)(st + 8192 + (ks * 64 + lane) * 32);
        }
        const u32x2 sc = *(const lds_u32x2*)(st + 16384 + lane * 8);
        mq.sh = sc[0];
        mq.sl = sc[1];
      }
      wait_vmcnt_lgkm0<0>();

      f32x4 acc[RB][kC];
#pragma unroll
      for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int d = 0; d < kC; ++d) acc[r][d] = f32x4{0.f, 0.f, 0.f, 0.f};
      float m = -INFINITY, lsum = 0.f;  // the owner's row statistics (base 2)

      TilePages pages_next;
      Gather gnext;
      lds_barrier();  // the queries' staging and the previous unit's readers of P are done
      if (ntiles > 0) {
#pragma unroll
        for (int x = 0; x < D; ++x)
          if (x < ntiles) {
            if constexpr (SPARSE) issue(x, pages_next, gather_lookup(a, list, bt, t0 + x * kTile, t1, sparse_limit));
            else issue(x, tile_pages(a, bt, t0 + x * kTile, t1), gnext);
          }
        if (D < ntiles) {
          if constexpr (SPARSE) gnext = gather_lookup(a, list, bt, t0 + D * kTile, t1, sparse_limit);
          else pages_next = tile_pages(a, bt, t0 + D * kTile, t1);
        }
      }

      // Owners: scores of tile x, online softmax, P into LDS.
      auto score = [&](int x) __attribute__((always_inline)) {
        const lds_char* const raw = raws + (x % kRaw) * kRawBuf;
        const int pb = x & 1;
        const lds_char* rowp[2] = {raw + li * kRowBytes + 16 * g, raw + (16 + li) * kRowBytes + 16 * g};
        // the token's scale of block g of every K step, one per byte
        uint32_t ska[2];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          const u32x4 sc = *(const lds_u32x4*)(rowp[tb] - 16 * g + kVals);
          const uint32_t sel = (uint32_t)g | ((uint32_t)(g + 4) << 8);
          ska[tb] = __builtin_amdgcn_perm(__builtin_amdgcn_perm(sc[3], sc[2], sel),
                                          __builtin_amdgcn_perm(sc[1], sc[0], sel), 0x05040100u);
        }
        auto load_k = [&](int ks, int tb) {
          const u32x4 x0 = *(const lds_u32x4*)(rowp[tb] + 128 * ks);
          const u32x4 x1 = *(const lds_u32x4*)(rowp[tb] + 128 * ks + 64);
          return i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3], (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
        };
        // S^T = K . Q^T, one accumulation chain per token block.  The next
        // step's K rows are requested before this step's products, so they
        // arrive while those run; the empty asm statements keep the steps
        // apart (the compiler would otherwise read all K rows first and run
        // out of registers).
        f32x4 s[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
        i32x8 ka[2] = {load_k(0, 0), load_k(0, 1)};
#pragma unroll
        for (int ks = 0; ks < kSteps; ++ks) {
          i32x8 kn[2];
          if (ks + 1 < kSteps) {
            kn[0] = load_k(ks + 1, 0);
            kn[1] = load_k(ks + 1, 1);
          }
#pragma unroll
          for (int tb = 0; tb < 2; ++tb) {
            s[tb] = mfma_mx(ks, ka[tb], mq.hi[ks], s[tb], ska[tb], mq.sh);
            s[tb] = mfma_mx(ks, ka[tb], mq.lo[ks], s[tb], ska[tb], mq.sl);
          }
          if (ks + 1 < kSteps) {
            asm volatile("" ::"v"(s[0]), "v"(s[1]) : "memory");
            ka[0] = kn[0];
            ka[1] = kn[1];
          }
        }
        // online softmax of the owned rows
        const int tt0 = t0 + x * kTile;
        const int last_visible = L - a.Sq + (row_ok ? row / a.H : 0);
        const uint32_t vis = SPARSE ? s_mask[x % kRaw] : ~0u;
        // a tile that every row sees whole (the usual case) needs no token mask
        const bool whole = !SPARSE && tt0 + kTile <= t1 && tt0 + kTile - 1 <= L - a.Sq;
        float sv[2][4], mx = -INFINITY;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = tt0 + tb * 16 + 4 * g + i;
            const bool ok = whole ? row_ok
                            : SPARSE ? row_ok && ((vis >> (tb * 16 + 4 * g + i)) & 1u)
                                     : row_ok && t < t1 && t <= last_visible;
            sv[tb][i] = ok ? s[tb][i] * a.scale_log2 : -INFINITY;
            mx = fmaxf(mx, sv[tb][i]);
          }
        mx = max_over_rows(mx);
        const bool raise = mx > m + 8.f;  // also true when m = -inf < mx
        const int flag = __any(raise) ? 1 : 0;
        float alpha = 1.f;
        if (flag) {
          const float m_new = raise ? mx : m;
          alpha = m == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m - m_new);
          lsum *= alpha;
          m = m_new;
        }
        float psum = 0.f;
        uint32_t pk[4];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int i = 0; i < 4; i += 2) {
            const float e0 = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv[tb][i] - m);
            const float e1 = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv[tb][i + 1] - m);
            psum += e0 + e1;
            pk[2 * tb + i / 2] = pack_bf16(e0, e1);
          }
        psum = sum_over_rows(psum);
        lsum += psum;
        *(lds_u32x4*)((lds_char*)p_mem[pb] + (wave * 64 + lane) * 16) = u32x4{pk[0], pk[1], pk[2], pk[3]};
        if (g == 0) s_alpha[pb][wave][li] = alpha;
        if (lane == 0) s_flag[pb][wave] = flag;
      };

      // Rescale, then O[:, own column blocks] += P . V for tile x.  Lane l
      // reads V rows 4(l/16) + (l%16)/4 and 16 more of each column block
      // transposed (ds_read_tr16_b64), as the B operand.
      auto pv = [&](int x) __attribute__((always_inline)) {
        const int pb = x & 1;
        // P is requested before the branches on the rescale flags, so its
        // LDS round trip overlaps theirs.
        bf16x8 pa[RB];
#pragma unroll
        for (int r = 0; r < RB; ++r) pa[r] = *(const lds_bf16x8*)((const lds_char*)p_mem[pb] + (r * 64 + lane) * 16);
#pragma unroll
        for (int r = 0; r < RB; ++r)
          if (uniform(s_flag[pb][r])) {
            const f32x4 al4 = *(const lds_f32x4*)(&s_alpha[pb][r][4 * g]);
#pragma unroll
            for (int d = 0; d < kC; ++d) {
              acc[r][d][0] *= al4[0];
              acc[r][d][1] *= al4[1];
              acc[r][d][2] *= al4[2];
              acc[r][d][3] *= al4[3];
            }
          }
        const int tok = 4 * g + (li >> 2);  // and tok + 16 (same swizzle)
        const int xs = swz(tok);
        const lds_char* const vb0 =
            (const lds_char*)v_mem[pb] + tok * kLatRow + 16 * (((li & 3) >> 1) ^ (xs & 1)) + 8 * (li & 1);
#pragma unroll
        for (int d = 0; d < kC; ++d) {
          if (d < c_count) {
            const int c = c_begin + d;
            const lds_char* const p0 = vb0 + 32 * ((c & 3) ^ (xs >> 1)) + 128 * (c >> 2);
            const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p0);
            const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p0 + 16 * kLatRow));
            const bf16x8 vb = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
            for (int r = 0; r < RB; ++r)
              acc[r][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[r], vb, acc[r][d], 0, 0, 0);
          }
        }
      };

      // Step s: tile s + 1 has landed (every wave's part); the transfer of
      // tile s + 1 + D starts into the buffer tile s used; owners score tile
      // s + 1, workers decode tile s + 1 and accumulate tile s.
      constexpr int M = Raw::kMinOps;                // loads per wave per tile ...
      constexpr int kExtra = Raw::kRawInst % NW;     // ... one more for waves below this
      for (int s = -1; s < ntiles; ++s) {
        const int x = s + 1;
        if (x < ntiles) {
          const int younger = min(D - 1, ntiles - 1 - x);  // tiles issued after x
          static_assert(D <= 4, "wait cases below");
          if (wave < kExtra) {
            if (younger >= 3) wait_vmcnt_lgkm0<3 * (M + 1)>();
            else if (younger == 2) wait_vmcnt_lgkm0<2 * (M + 1)>();
            else if (younger == 1) wait_vmcnt_lgkm0<M + 1>();
            else wait_vmcnt_lgkm0<0>();
          } else {
            if (younger >= 3) wait_vmcnt_lgkm0<3 * M>();
            else if (younger == 2) wait_vmcnt_lgkm0<2 * M>();
            else if (younger == 1) wait_vmcnt_lgkm0<M>();
            else wait_vmcnt_lgkm0<0>();
          }
        } else {
          wait_lgkm0();
        }
        lds_barrier();  // tile x landed; step s - 1 is done everywhere
        const int xn = x + D;
        if (xn < ntiles) {
          issue(xn, pages_next, gnext);
          if (xn + 1 < ntiles) {
            if constexpr (SPARSE) gnext = gather_lookup(a, list, bt, t0 + (xn + 1) * kTile, t1, sparse_limit);
            else pages_next = tile_pages(a, bt, t0 + (xn + 1) * kTile, t1);
          }
        }
        // Owners score first (their scores gate the next step), the other
        // waves accumulate first (their V decode is needed only next step):
        // measured 2% faster than both roles accumulating last.
        if constexpr (kOwner) {
          if (x < ntiles) score(x);
          if (s >= 0) pv(s);
        } else {
          if (s >= 0) pv(s);
          if (x < ntiles)
            decode_v_fp8<SPARSE, 64 * kWk>(raws + (x % kRaw) * kRawBuf, (lds_char*)v_mem[x & 1],
                                          SPARSE ? s_mask[x % kRaw] : ~0u, threadIdx.x - 64 * RB);
        }
      }

      // ---- normalise and write this unit's partials (tiled layout) ----
      if constexpr (kOwner) {
        if (g == 0) {
          s_inv[wave][li] = lsum > 0.f ? 1.f / lsum : 0.f;
          if (row_ok) a.part_lse[slot * a.R + row] = lsum > 0.f ? (m + log2f(lsum)) * kLn2 : -INFINITY;
        }
      }
      wait_lgkm0();
      lds_barrier();  // every row's 1/sum is in LDS
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        if (r * 16 + 4 * g >= a.R) continue;  // lanes holding only padding rows
        const f32x4 inv4 = *(const lds_f32x4*)(&s_inv[r][4 * g]);
        float* dst = a.part_o + ((slot * row_blocks + r) * kDb * 64 + lane) * 4;
#pragma unroll
        for (int d = 0; d < kC; ++d)
          if (d < c_count)
            *reinterpret_cast<float4*>(dst + 256 * (c_begin + d)) =
                make_float4(acc[r][d][0] * inv4[0], acc[r][d][1] * inv4[1], acc[r][d][2] * inv4[2],
                            acc[r][d][3] * inv4[3]);
      }
    }
  };
  if (owner) run(std::true_type{});
  else run(std::false_type{});
}
}  // namespace

// fp8 rows with at most five row blocks: the eight-wave MX kernel, one
// workgroup per CU.  Otherwise (fp4 rows, or six to eight row blocks) the
// kernel that decodes whole rows to bf16: up to four row blocks four waves,
// of which the first RB own row blocks (one workgroup per CU, a whole SIMD's
// registers per wave, for three or four row blocks; two workgroups per CU for
// one or two); five to eight row blocks eight waves, two per SIMD.  All waves
// split the PV columns, which keeps the SIMDs' matrix work close to even.
// Measured on 64 sequences of 16k fp8 tokens with one query token: two
// waves per workgroup and two workgroups per CU 302 us, four waves 231 us.
static bool rows_mx(int fmt, int R) { return fmt == kFP8 && (R + 15) / 16 <= kMxMaxRowBlocks; }
int fp8_rows_workers(int fmt, int R) { return !rows_mx(fmt, R) && (R + 15) / 16 <= 2 ? 512 : 256; }

bool decode_fp8_rows_supported(int fmt, int dc, int dr, int R, int q_f32) {
  return (fmt == kFP8 || fmt == kFP4) && dc == kDc && dr == kDr && !q_f32 && R >= 1 && R <= 128;
}

template <bool SPARSE>
hipError_t launch_mx(const DecodeArgs& a, unsigned units, hipStream_t s) {
  switch ((a.R + 15) / 16) {
#define MLA_CASE(N) \
  case N:           \
    decode_fp8_mx_kernel<N, SPARSE><<<units, 64 * kMxWaves, 0, s>>>(a); \
    break;
    MLA_CASE(1) MLA_CASE(2) MLA_CASE(3) MLA_CASE(4) MLA_CASE(5)
#undef MLA_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_rows(const DecodeArgs& a, hipStream_t s) {
  const unsigned units = a.num_splits > 0 ? (unsigned)(a.B * a.num_splits) : (unsigned)a.workers;
  if (rows_mx(FMT, a.R)) return launch_mx<false>(a, units, s);
  switch ((a.R + 15) / 16) {
#define MLA_CASE(N) \
  case N:           \
    decode_fp8_kernel<FMT, (N <= 4 ? 4 : 8), N><<<units, 64 * (N <= 4 ? 4 : 8), 0, s>>>(a); \
    break;
    MLA_CASE(1) MLA_CASE(2) MLA_CASE(3) MLA_CASE(4) MLA_CASE(5) MLA_CASE(6) MLA_CASE(7) MLA_CASE(8)
#undef MLA_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode_fp8_rows(const DecodeArgs& a, int fmt, hipStream_t s) {
  if (fmt == kFP4) return launch_rows<kFP4>(a, s);
  if (fmt == kFP8) return launch_rows<kFP8>(a, s);
  return hipErrorInvalidValue;
}

// Sparse mode: each index list is read in whole 32-slot tiles.
bool decode_fp8_rows_sparse_supported(int fmt, int dc, int dr, int R, int q_f32, int topk_width) {
  return decode_fp8_rows_supported(fmt, dc, dr, R, q_f32) && topk_width % kTile == 0;
}

// Sparse units are short (one query token's list chunk), so with one or two
// row blocks the two-workgroups-per-CU kernel keeps more of them in flight
// than the MX kernel's one per CU (fp8 MTP batch, 512 units: 252 us against
// 361 us).
template <int FMT>
hipError_t launch_rows_sparse(const DecodeArgs& a, hipStream_t s) {
  const unsigned units = (unsigned)(a.B * a.num_splits);
  if (rows_mx(FMT, a.R) && (a.R + 15) / 16 > 2) return launch_mx<true>(a, units, s);
  switch ((a.R + 15) / 16) {
#define MLA_CASE(N) \
  case N:           \
    decode_fp8_kernel<FMT, (N <= 4 ? 4 : 8), N, true><<<units, 64 * (N <= 4 ? 4 : 8), 0, s>>>(a); \
    break;
    MLA_CASE(1) MLA_CASE(2) MLA_CASE(3) MLA_CASE(4) MLA_CASE(5) MLA_CASE(6) MLA_CASE(7) MLA_CASE(8)
#undef MLA_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode_fp8_rows_sparse(const DecodeArgs& a, int fmt, hipStream_t s) {
  if (a.num_splits < 1 || !decode_fp8_rows_sparse_supported(fmt, a.dc, a.dr, a.R, a.q_f32, a.topk_width))
    return hipErrorInvalidValue;
  if (fmt == kFP4) return launch_rows_sparse<kFP4>(a, s);
  if (fmt == kFP8) return launch_rows_sparse<kFP8>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace mla
