// Prefill K/V rebuild on the matrix cores (gfx950): per head h and cached
// token t, the rows of kv_b_proj times the latent,
//   [k_t ; v_t] = W[h] c_t,   W[h] = [W_UK[h] ; W_UV[h]]  ((d_nope + d_v) x d_latent),
// as v_mfma_f32_16x16x32_bf16 products with fp32 accumulation.
//
// Two kernels.  prefill_expand_gemm_kernel (bf16 cache with a 512-wide
// latent or fp8 cache with a 448-wide one, d_nope + d_v a multiple of 64 up
// to 448) tiles the product as a GEMM over
// 128 tokens x all output rows; it is defined further down.  Otherwise
// prefill_expand_mfma_kernel: a workgroup of 4 waves over one (sequence,
// head), 64 output rows of W[h] (16 per wave, held in registers as the B
// operand for the whole workgroup) and up to 8 blocks of 16 tokens.  Per
// block the latent rows are decoded from the cache row into a bf16 tile in
// LDS (the A operand).  bf16, fp8 and fp4 latents are exact in bf16; an f32
// latent is split into bf16 hi + lo parts, two products per k-step, as the
// fp32 projections do.  Both accumulate over the latent in the same order,
// so on a bf16 cache they give the same bits.
#include <algorithm>
#include <cmath>

#include "decode_common.h"
#include "device_common.h"
#include "internal.h"

namespace mla {
namespace {

using mfma::bf16x8;
using mfma::f32x4;

constexpr int kTokBlk = 16;    // tokens per MFMA row block
constexpr int kBlocks = 8;     // token blocks per workgroup
constexpr int kWaves = 4;
constexpr int kCols = 16 * kWaves;  // output rows of W[h] per workgroup

// Value i of a quantised row (fp8: e4m3 x e8m0 per 32; fp4: e2m1 x e4m3 per
// 16); n = d_latent + d_rope.
template <int FMT>
__device__ __forceinline__ float quant_value(const uint8_t* row, int i, int n) {
  if constexpr (FMT == kFP8) {
    return e4m3fn_to_f32(row[i]) * e8m0_to_f32(row[n + i / 32]);
  } else {
    const uint32_t code = (row[i >> 1] >> (4 * (i & 1))) & 0xfu;
    return e2m1_to_f32(code) * e4m3fn_to_f32(row[n / 2 + i / 16]);
  }
}

template <int FMT>
__device__ __forceinline__ float any_value(const uint8_t* row, int i, int n) {
  if constexpr (FMT == kF32) return reinterpret_cast<const float*>(row)[i];
  else if constexpr (FMT == kBF16) return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(row)[i]);
  else return quant_value<FMT>(row, i, n);
}

template <int FMT, int NKS>  // NKS = d_latent / 32
__global__ __launch_bounds__(64 * kWaves) void prefill_expand_mfma_kernel(PrefillArgs a) {
  constexpr int kDc = 32 * NKS;
  constexpr int kRowB = kDc * 2 + 16;  // LDS row stride (bytes) of the bf16 tile
  constexpr bool kSplit = FMT == kF32;
  __shared__ __attribute__((aligned(16))) char hi_tile[kTokBlk * kRowB];
  __shared__ __attribute__((aligned(16))) char lo_tile[kSplit ? kTokBlk * kRowB : 16];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, g = lane >> 4, li = lane & 15;
  const int b = blockIdx.z / a.H, h = blockIdx.z % a.H;
  const int col = blockIdx.y * kCols + 16 * wave + li;  // row of W[h], < d_nope + d_v
  const int L = (int)min((int64_t)max(a.seq_lens[b], 0), a.Lcap);
  const int t_begin = blockIdx.x * kTokBlk * kBlocks;
  if (t_begin >= L) return;  // uniform
  const int t_end = min(L, t_begin + kTokBlk * kBlocks);
  const int nv = a.dc + a.dr;

  const uint16_t* w = static_cast<const uint16_t*>(a.w) + ((int64_t)h * (a.dn + a.dv) + col) * a.dc;
  bf16x8 wb[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
    wb[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(w + 32 * ks + 8 * g));

  // bf16 cache: the rows of the next two blocks are in flight while a block
  // is computed.  A 16-token block (its start is a multiple of 16, and
  // page_block is a power of two >= 16) lies in one page: one scalar page
  // lookup per block, all made up front.  Thread t carries 16-byte chunk
  // t % (kDc / 8) of rows t / (kDc / 8) + (256 / (kDc / 8)) j of each block.
  constexpr int kChunksPerRow = kDc / 8;
  constexpr int kRowsPerPass = 64 * kWaves / kChunksPerRow;
  constexpr int kRawPer = kTokBlk / kRowsPerPass;  // chunks per thread and block
  constexpr int kAhead = 2;
  const bool pipelined = FMT == kBF16 && (64 * kWaves) % kChunksPerRow == 0 && kRowsPerPass <= kTokBlk;
  if constexpr (FMT == kBF16) {
    if (pipelined) {
      const int nblk = (t_end - t_begin + kTokBlk - 1) / kTokBlk;
      const int32_t* bt = a.block_table + (int64_t)b * a.max_blocks;
      int pg[kBlocks];
#pragma unroll
      for (int k = 0; k < kBlocks; ++k) pg[k] = k < nblk ? bt[(t_begin + k * kTokBlk) / a.P] : 0;
      const int c8 = tid % kChunksPerRow, r0 = tid / kChunksPerRow;
      uint4 raw[kAhead + 1][kRawPer];
      auto load = [&](int k, uint4 (&dst)[kRawPer]) __attribute__((always_inline)) {
        const int t0 = t_begin + k * kTokBlk;
        const uint8_t* base = a.pool + ((int64_t)pg[k] * a.P + (t0 & (a.P - 1))) * a.row_bytes + 16 * c8;
#pragma unroll
        for (int j = 0; j < kRawPer; ++j)  // rows past the sequence stay inside the block's page
          dst[j] = *reinterpret_cast<const uint4*>(base + (int64_t)(r0 + kRowsPerPass * j) * a.row_bytes);
      };
#pragma unroll
      for (int k = 0; k < kAhead; ++k)
        if (k < nblk) load(k, raw[k]);
#pragma unroll
      for (int k = 0; k < kBlocks; ++k) {
        if (k >= nblk) break;
        const int t0 = t_begin + k * kTokBlk;
        if (k + kAhead < nblk) load(k + kAhead, raw[(k + kAhead) % (kAhead + 1)]);
#pragma unroll
        for (int j = 0; j < kRawPer; ++j) {
          const int r = r0 + kRowsPerPass * j;
          *reinterpret_cast<uint4*>(hi_tile + r * kRowB + 16 * c8) =
              t0 + r < t_end ? raw[k % (kAhead + 1)][j] : make_uint4(0u, 0u, 0u, 0u);
        }
        if (h == 0 && blockIdx.y == 0)  // the shared RoPE keys, once per token
          for (int idx = tid; idx < kTokBlk * a.dr; idx += 64 * kWaves) {
            const int r = idx / a.dr, i = idx % a.dr, t = t0 + r;
            if (t < t_end) {
              const uint8_t* row = a.pool + ((int64_t)pg[k] * a.P + (t & (a.P - 1))) * a.row_bytes;
              a.kr[((int64_t)b * a.Lcap + t) * a.dr + i] = any_value<FMT>(row, a.dc + i, nv);
            }
          }
        __syncthreads();
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
        const char* hrow = hi_tile + li * kRowB + 16 * g;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const bf16x8 ah = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(hrow + 64 * ks));
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, wb[ks], acc, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = t0 + 4 * g + i;
          if (t < t_end) {
            const int64_t tok = ((int64_t)b * a.Lcap + t) * a.H + h;
            if (col < a.dn) a.kn[tok * a.dn + col] = acc[i];
            else a.v[tok * a.dv + (col - a.dn)] = acc[i];
          }
        }
        __syncthreads();  // the tile is rewritten by the next block
      }
      return;
    }
  }
  for (int t0 = t_begin; t0 < t_end; t0 += kTokBlk) {
    // bf16 tile of the block's latent rows (rows past the end are zero)
    for (int idx = tid; idx < kTokBlk * (kDc / 8); idx += 64 * kWaves) {
      const int r = idx / (kDc / 8), c8 = idx % (kDc / 8), t = t0 + r;
      uint4 hv = make_uint4(0u, 0u, 0u, 0u), lv = make_uint4(0u, 0u, 0u, 0u);
      if (t < t_end) {
        const int page = a.block_table[(int64_t)b * a.max_blocks + t / a.P];
        const uint8_t* row = a.pool + ((int64_t)page * a.P + (t % a.P)) * a.row_bytes;
        if constexpr (FMT == kBF16) {
          hv = *reinterpret_cast<const uint4*>(row + 16 * c8);
        } else if constexpr (FMT == kFP8) {
          // 8 e4m3 codes and their block's e8m0 scale: one scaled conversion
          // per pair, exact in bf16 (the decode kernels use the same one)
          const uint2 raw = *reinterpret_cast<const uint2*>(row + 8 * c8);
          const float sc = e8m0_to_f32(row[nv + c8 / 4]);
          hv = make_uint4(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.x, sc, false)),
                          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.x, sc, true)),
                          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.y, sc, false)),
                          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.y, sc, true)));
        } else if constexpr (FMT == kFP4) {
          // 8 e2m1 codes (value 2i in the low nibble of byte i) and their
          // block's e4m3 scale: an e2m1 value times an e4m3 scale has at most
          // 6 significant bits, so the bf16 value is the upper half of the
          // exact fp32 product
          const uint32_t w = *reinterpret_cast<const uint32_t*>(row + 4 * c8);
          const float sc = e4m3fn_to_f32(row[nv / 2 + c8 / 2]);
          const auto p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
          const auto p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
          const auto p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
          const auto p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
          auto hi2 = [&](float x0, float x1) {
            return __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, x1 * sc), __builtin_bit_cast(uint32_t, x0 * sc),
                                         0x07060302u);
          };
          hv = make_uint4(hi2(p0[0], p0[1]), hi2(p1[0], p1[1]), hi2(p2[0], p2[1]), hi2(p3[0], p3[1]));
        } else {
          float x[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) x[j] = any_value<FMT>(row, 8 * c8 + j, nv);
          uint32_t hw[4], lw[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if constexpr (kSplit) split_bf16x2(x[2 * j], x[2 * j + 1], hw[j], lw[j]);
            else hw[j] = bf16x2_bits(x[2 * j], x[2 * j + 1]), lw[j] = 0u;  // exact in bf16
          }
          hv = make_uint4(hw[0], hw[1], hw[2], hw[3]);
          lv = make_uint4(lw[0], lw[1], lw[2], lw[3]);
        }
      }
      *reinterpret_cast<uint4*>(hi_tile + r * kRowB + 16 * c8) = hv;
      if constexpr (kSplit) *reinterpret_cast<uint4*>(lo_tile + r * kRowB + 16 * c8) = lv;
    }
    // the shared RoPE keys, once per token: head 0, first column group
    if (h == 0 && blockIdx.y == 0)
      for (int idx = tid; idx < kTokBlk * a.dr; idx += 64 * kWaves) {
        const int r = idx / a.dr, i = idx % a.dr, t = t0 + r;
        if (t < t_end) {
          const int page = a.block_table[(int64_t)b * a.max_blocks + t / a.P];
          const uint8_t* row = a.pool + ((int64_t)page * a.P + (t % a.P)) * a.row_bytes;
          a.kr[((int64_t)b * a.Lcap + t) * a.dr + i] = any_value<FMT>(row, a.dc + i, nv);
        }
      }
    __syncthreads();

    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    const char* hrow = hi_tile + li * kRowB + 16 * g;
    const char* lrow = lo_tile + (kSplit ? li * kRowB + 16 * g : 0);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const bf16x8 ah = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(hrow + 64 * ks));
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, wb[ks], acc, 0, 0, 0);
      if constexpr (kSplit) {
        const bf16x8 al = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(lrow + 64 * ks));
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, wb[ks], acc, 0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 4 * g + i;
      if (t < t_end) {
        const int64_t tok = ((int64_t)b * a.Lcap + t) * a.H + h;
        if (col < a.dn) a.kn[tok * a.dn + col] = acc[i];
        else a.v[tok * a.dv + (col - a.dn)] = acc[i];
      }
    }
    __syncthreads();  // the tile is rewritten by the next block
  }
}

// Causal attention of the chunk on the matrix cores, for 256-wide keys
// (d_nope + d_rope) and values.  A workgroup of 4 waves takes 64
// consecutive queries of one (sequence, head), 16 per wave, and walks the
// keys in blocks of 32 staged in LDS once for all of them.  Every fp32
// operand is split into bf16 hi + lo and each product takes three MFMAs
// (hi.hi + hi.lo + lo.hi), which keeps the result at fp32-level accuracy:
//   S^T = K Q^T: A = K rows (LDS), B = the wave's queries (registers);
//   online softmax per query (lane li = query, 8 keys per lane);
//   O += P V with P from registers (the S^T layout is PV's A layout) and V
//   read from its key-major LDS tile with transposing loads.
// Two workgroups share a CU (69 KB of LDS and at most 256 registers each),
// so that each SIMD has a second wave to run while the first one waits.
constexpr int kAQ = 16;        // queries per wave
constexpr int kAKeys = 32;     // keys per block
constexpr int kAD = 256;       // key and value width
constexpr int kKRowB = kAD * 2 + 16;      // K tile row stride (bytes)
constexpr int kVRowB = kAD * 2 + 32;      // V tile row stride (bytes): 4 rows land 32 B apart in the banks

__device__ __forceinline__ bf16x8 lds_b8(const char* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

// The rebuild for a bf16 cache with a 512-wide latent (or an fp8 cache with
// a 448-wide one, decoded exactly to bf16 when staged), tiled as a GEMM per
// (sequence, head): a workgroup of 8 waves computes 128 tokens x all
// N = d_nope + d_v output rows of W[h], so each latent row is read once per
// head (the kernel above reads it once per 64 output rows) and W[h] once per
// 128 tokens.  K = d_latent goes in chunks of 64: the chunk's latent rows
// (128 x 64) and W rows (N x 64) are staged in LDS (rows padded to 144 B, so
// the 16 lanes of an operand read hit distinct banks), the next chunk's are
// loaded into registers meanwhile.  Wave w takes tokens 64 (w % 2) .. +63
// (four 16-row blocks) and output rows (w / 2) N / 4 .. +N / 4 (NCB 16-row
// blocks).  XCD-aware order: the tiles of one (sequence, head) are
// consecutive on one XCD, which keeps W[h] in its L2.
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t gemm_u4;  // a native vector, kept in registers
constexpr int kGTok = 128;              // tokens per workgroup
constexpr int kGKc = 64;                // K chunk
constexpr int kGRowB = kGKc * 2 + 16;   // LDS row stride (bytes)
constexpr int kGWaves = 8;
constexpr int kGThreads = 64 * kGWaves;

template <int FMT, int NCB>  // bf16 or fp8 rows; 16-row blocks of W per wave: N = 64 NCB
__global__ __launch_bounds__(kGThreads) void prefill_expand_gemm_kernel(PrefillArgs a, int tiles) {
  static_assert(FMT == kBF16 || FMT == kFP8, "row formats");
  constexpr int N = 64 * NCB;
  constexpr int kDc = FMT == kBF16 ? 512 : 448;  // the latent width of the row format
  constexpr int kVB = FMT == kBF16 ? 2 : 1;      // stored bytes per value
  constexpr int kChunks = kDc / kGKc;
  constexpr int kAUnits = kGTok * (kGKc / 8);               // 16-B units of a latent chunk
  constexpr int kWUnits = N * (kGKc / 8);                   // ... of a W chunk
  static_assert(kAUnits == 2 * kGThreads, "two latent units per thread");
  constexpr int kWPer = kWUnits / kGThreads;
  static_assert(kAUnits % kGThreads == 0 && kWUnits % kGThreads == 0, "staging");
  __shared__ __attribute__((aligned(16))) char a_tile[kGTok * kGRowB];
  __shared__ __attribute__((aligned(16))) char w_tile[N * kGRowB];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, g = lane >> 4, li = lane & 15;
  const int x8 = blockIdx.x % 8, k = blockIdx.x / 8;
  const int u = 8 * (k / tiles) + x8;  // (sequence, head) unit
  if (u >= a.B * a.H) return;
  const int b = u / a.H, h = u % a.H;
  const int L = (int)min((int64_t)max(a.seq_lens[b], 0), a.Lcap);
  const int t0 = (k % tiles) * kGTok;
  if (t0 >= L) return;  // uniform

  // Latent rows of this thread's two staging units: tokens t0 + tid / 8 and
  // 64 more, values 8 (tid % 8) .. + 7 of each chunk (tokens past L read the
  // sequence's first row and are zeroed in LDS).  fp8 values are decoded
  // exactly to bf16 when staged, with their block's e8m0 scale.
  const int32_t* bt = a.block_table + (int64_t)b * a.max_blocks;
  const int u8 = tid % (kGKc / 8);
  auto row_of = [&](int un, uint32_t& m) __attribute__((always_inline)) {
    const int t = t0 + un / (kGKc / 8);
    m = t < L ? 0xffffffffu : 0u;
    const int tt = t < L ? t : 0;
    return a.pool + ((int64_t)bt[tt / a.P] * a.P + (tt & (a.P - 1))) * a.row_bytes;
  };
  uint32_t am0, am1;
  const uint8_t* const arow0 = row_of(tid, am0);
  const uint8_t* const arow1 = row_of(tid + kGThreads, am1);
  const uint16_t* wh = static_cast<const uint16_t*>(a.w) + (int64_t)h * (a.dn + a.dv) * kDc;
  // A unit of chunk c: 8 values (16 B of bf16, or 8 fp8 codes and the scale
  // code of their 32-value block).
  typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t gemm_u2;
  struct AUnit {
    gemm_u4 v;       // bf16
    gemm_u2 q;       // fp8 codes
    uint32_t sc;     // fp8 scale code
  };
  auto load_a = [&](const uint8_t* row, int c, AUnit& x) __attribute__((always_inline)) {
    if constexpr (FMT == kBF16) {
      x.v = *reinterpret_cast<const gemm_u4*>(row + kVB * (kGKc * c + 8 * u8));
    } else {
      x.q = *reinterpret_cast<const gemm_u2*>(row + kGKc * c + 8 * u8);
      x.sc = row[a.dc + a.dr + (kGKc * c + 8 * u8) / 32];
    }
  };
  auto bf16_of = [&](const AUnit& x) __attribute__((always_inline)) -> gemm_u4 {
    if constexpr (FMT == kBF16) {
      return x.v;
    } else {
      const float sc = e8m0_to_f32(x.sc);
      return gemm_u4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.q[0], sc, false)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.q[0], sc, true)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.q[1], sc, false)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.q[1], sc, true))};
    }
  };
  AUnit ra0, ra1;
  gemm_u4 rw[kWPer];
  // The shared RoPE keys, once per token (head 0).
  if (h == 0)
    for (int idx = tid; idx < kGTok * a.dr; idx += kGThreads) {
      const int r = idx / a.dr, i = idx % a.dr, t = t0 + r;
      if (t < L) {
        const uint8_t* row = a.pool + ((int64_t)bt[t / a.P] * a.P + (t & (a.P - 1))) * a.row_bytes;
        a.kr[((int64_t)b * a.Lcap + t) * a.dr + i] = any_value<FMT>(row, kDc + i, kDc + a.dr);
      }
    }

  const int th = wave & 1, cq = wave >> 1;
  f32x4 acc[4][NCB];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < NCB; ++c) acc[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};
  load_a(arow0, 0, ra0);
  load_a(arow1, 0, ra1);
#pragma unroll
  for (int j = 0; j < kWPer; ++j) {
    const int un = tid + kGThreads * j;
    rw[j] = *reinterpret_cast<const gemm_u4*>(wh + (int64_t)(un / (kGKc / 8)) * kDc + 8 * (un % (kGKc / 8)));
  }
  for (int c = 0; c < kChunks; ++c) {
    if (c > 0) __syncthreads();  // the previous chunk's readers are done
    {  // tokens past L are zeros
      const int u0 = tid, u1 = tid + kGThreads;
      *reinterpret_cast<gemm_u4*>(a_tile + (u0 / (kGKc / 8)) * kGRowB + 16 * (u0 % (kGKc / 8))) = bf16_of(ra0) & am0;
      *reinterpret_cast<gemm_u4*>(a_tile + (u1 / (kGKc / 8)) * kGRowB + 16 * (u1 % (kGKc / 8))) = bf16_of(ra1) & am1;
    }
#pragma unroll
    for (int j = 0; j < kWPer; ++j) {
      const int un = tid + kGThreads * j;  // kWUnits is a multiple of the thread count
      *reinterpret_cast<gemm_u4*>(w_tile + (un / (kGKc / 8)) * kGRowB + 16 * (un % (kGKc / 8))) = rw[j];
    }
    __syncthreads();
    if (c + 1 < kChunks) {  // the next chunk is in flight during this chunk's products
      load_a(arow0, c + 1, ra0);
      load_a(arow1, c + 1, ra1);
#pragma unroll
      for (int j = 0; j < kWPer; ++j) {
        const int un = tid + kGThreads * j;
        rw[j] = *reinterpret_cast<const gemm_u4*>(wh + (int64_t)(un / (kGKc / 8)) * kDc + kGKc * (c + 1) +
                                                8 * (un % (kGKc / 8)));
      }
    }
#pragma unroll
    for (int ks = 0; ks < kGKc / 32; ++ks) {
      bf16x8 av[4], bv[NCB];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        av[r] = lds_b8(a_tile + (64 * th + 16 * r + li) * kGRowB + 64 * ks + 16 * g);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
        bv[cb] = lds_b8(w_tile + (N / 4 * cq + 16 * cb + li) * kGRowB + 64 * ks + 16 * g);
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
          acc[r][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[r], bv[cb], acc[r][cb], 0, 0, 0);
    }
  }
  // C layout: lane (li, g) holds output row (of W) 16 cb + li for tokens 4g .. 4g + 3.
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 64 * th + 16 * r + 4 * g + i;
      if (t >= L) continue;
      const int64_t tok = ((int64_t)b * a.Lcap + t) * a.H + h;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const int n = N / 4 * cq + 16 * cb + li;
        if (n < a.dn) a.kn[tok * a.dn + n] = acc[r][cb][i];
        else a.v[tok * a.dv + (n - a.dn)] = acc[r][cb][i];
      }
    }
}


__global__ __launch_bounds__(64 * kWaves, 2) void prefill_attn_mfma_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) char kh[kAKeys * kKRowB];
  __shared__ __attribute__((aligned(16))) char kl[kAKeys * kKRowB];
  __shared__ __attribute__((aligned(16))) char vh_t[kAKeys * kVRowB];
  __shared__ __attribute__((aligned(16))) char vl_t[kAKeys * kVRowB];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, g = lane >> 4, li = lane & 15;
  const int nqb = (a.Sq + kAQ * kWaves - 1) / (kAQ * kWaves);
  // XCD-aware order (workgroups go round-robin over the 8 XCDs, each with its
  // own L2): the nqb query blocks of one (sequence, head, key split) read the
  // same keys and values, so they run on one XCD, one after another in its
  // dispatch order, and share its L2.  Unit u = (b * H + h) * splits + split
  // goes to XCD u % 8.
  int h, split, b, qb;
  {
    const int x8 = blockIdx.x % 8, k = blockIdx.x / 8;
    const int u = 8 * (k / nqb) + x8;
    if (u >= a.B * a.H * a.splits) return;  // no barrier precedes this
    qb = k % nqb;
    split = u % a.splits;
    h = (u / a.splits) % a.H;
    b = u / (a.splits * a.H);
  }
  const int iw = qb * kAQ * kWaves + kAQ * wave;  // the wave's first query
  const int L = (int)min((int64_t)max(a.seq_lens[b], 0), a.Lcap);
  const int ig_end = min(a.Sq, (qb + 1) * kAQ * kWaves);
  // Keys the workgroup's queries see: [0, n_keys); this split takes
  // [k_begin, blk_last] of them, a whole number of key blocks.  The split
  // boundaries come from the sequence's L keys (what its last query sees),
  // so every query block of the sequence cuts the keys at the same places
  // and the blocks' reads of a split coincide in L2.
  const int n_keys = max(0, min(L, L - a.Sq + ig_end));
  const int chunk = ((L + a.splits - 1) / a.splits + kAKeys - 1) / kAKeys * kAKeys;
  const int k_begin = split * chunk;
  const int blk_last = min(n_keys, k_begin + chunk) - 1;  // this split's last key

  // A operand: query row iw + li, dims 32 ks + 8 g .. + 7, as hi and lo.
  bf16x8 qh[kAD / 32], ql[kAD / 32];
  {
    const int i = iw + li;
    const int64_t off = (((int64_t)b * a.Sq + min(i, a.Sq - 1)) * a.H + h) * kAD;
#pragma unroll
    for (int ks = 0; ks < kAD / 32; ++ks) {
      float x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int64_t e = off + 32 * ks + 8 * g + j;
        x[j] = a.q_f32 ? static_cast<const float*>(a.q)[e] : bf16_bits_to_f32(static_cast<const uint16_t*>(a.q)[e]);
        if (i >= a.Sq) x[j] = 0.f;
      }
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) split_bf16x2(x[2 * j], x[2 * j + 1], hw[j], lw[j]);
      qh[ks] = __builtin_bit_cast(bf16x8, make_uint4(hw[0], hw[1], hw[2], hw[3]));
      ql[ks] = __builtin_bit_cast(bf16x8, make_uint4(lw[0], lw[1], lw[2], lw[3]));
    }
  }

  f32x4 o[kAD / 16];
#pragma unroll
  for (int d = 0; d < kAD / 16; ++d) o[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;  // query iw + li's running maximum and sum (base 2)

  // A block's K and V rows are loaded into registers one block ahead, so
  // that their transfer overlaps the previous block's products: thread tid
  // holds K chunks (key r, dims 4c .. 4c + 3) for idx = tid + 256 j and V
  // chunks (keys 2 rp, 2 rp + 1, dims 4c .. 4c + 3) likewise.
  constexpr int kKPer = kAKeys * (kAD / 4) / (64 * kWaves);        // 8
  float4 kx[kKPer], vx[kKPer];
  auto load_block = [&](int t0) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kKPer; ++j) {
      const int idx = tid + 64 * kWaves * j;
      const int r = idx / (kAD / 4), c = idx % (kAD / 4), t = min(t0 + r, blk_last);
      kx[j] = 4 * c < a.dn ? reinterpret_cast<const float4*>(a.kn + (((int64_t)b * a.Lcap + t) * a.H + h) * a.dn)[c]
                           : reinterpret_cast<const float4*>(a.kr + ((int64_t)b * a.Lcap + t) * a.dr)[c - a.dn / 4];
    }
#pragma unroll
    for (int j = 0; j < kKPer; ++j) {
      const int idx = tid + 64 * kWaves * j;
      const int r = idx / (kAD / 4), c = idx % (kAD / 4), t = min(t0 + r, blk_last);
      vx[j] = reinterpret_cast<const float4*>(a.v + (((int64_t)b * a.Lcap + t) * a.H + h) * a.dv)[c];
    }
  };
  if (k_begin <= blk_last) load_block(k_begin);

  for (int t0 = k_begin; t0 <= blk_last; t0 += kAKeys) {
    __syncthreads();  // the previous block's readers are done
    // K rows (hi, lo) and V transposed (hi, lo) into LDS; keys past the
    // workgroup's last visible one were loaded clamped and are zeroed here.
#pragma unroll
    for (int j = 0; j < kKPer; ++j) {
      const int idx = tid + 64 * kWaves * j;
      const int r = idx / (kAD / 4), c = idx % (kAD / 4);
      const float4 x = t0 + r <= blk_last ? kx[j] : make_float4(0.f, 0.f, 0.f, 0.f);
      uint32_t h0, l0, h1, l1;
      split_bf16x2(x.x, x.y, h0, l0);
      split_bf16x2(x.z, x.w, h1, l1);
      *reinterpret_cast<uint2*>(kh + r * kKRowB + 8 * c) = make_uint2(h0, h1);
      *reinterpret_cast<uint2*>(kl + r * kKRowB + 8 * c) = make_uint2(l0, l1);
    }
#pragma unroll
    for (int j = 0; j < kKPer; ++j) {
      const int idx = tid + 64 * kWaves * j;
      const int r = idx / (kAD / 4), c = idx % (kAD / 4);
      const float4 x = t0 + r <= blk_last ? vx[j] : make_float4(0.f, 0.f, 0.f, 0.f);
      uint32_t h0, l0, h1, l1;
      split_bf16x2(x.x, x.y, h0, l0);
      split_bf16x2(x.z, x.w, h1, l1);
      *reinterpret_cast<uint2*>(vh_t + r * kVRowB + 8 * c) = make_uint2(h0, h1);
      *reinterpret_cast<uint2*>(vl_t + r * kVRowB + 8 * c) = make_uint2(l0, l1);
    }
    __syncthreads();
    if (t0 + kAKeys <= blk_last) load_block(t0 + kAKeys);  // in flight during this block's products

    // S^T = K Q^T: K rows are the A operand (LDS), the wave's queries the B
    // operand (registers), so lane (li, g) gets query iw + li's scores for
    // keys t0 + 16 nt + 4 g + r.  Those are exactly PV's A operand (P, row li)
    // in the key order the transposing V reads use, so P stays in registers.
    // The two key halves' products alternate (two independent accumulation
    // chains), and each k-step's K operands are read one step ahead.
    f32x4 sc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    {
      constexpr int kAhead = 1;
      const char* krh[2] = {kh + li * kKRowB + 16 * g, kh + (16 + li) * kKRowB + 16 * g};
      const char* krl[2] = {kl + li * kKRowB + 16 * g, kl + (16 + li) * kKRowB + 16 * g};
      bf16x8 kbh[kAhead][2], kbl[kAhead][2];
#pragma unroll
      for (int k = 0; k < kAhead; ++k)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) kbh[k][nt] = lds_b8(krh[nt] + 64 * k), kbl[k][nt] = lds_b8(krl[nt] + 64 * k);
#pragma unroll
      for (int ks = 0; ks < kAD / 32; ++ks) {
        bf16x8 bh[2], bl[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) bh[nt] = kbh[ks % kAhead][nt], bl[nt] = kbl[ks % kAhead][nt];
        if (ks + kAhead < kAD / 32) {
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) {
            kbh[ks % kAhead][nt] = lds_b8(krh[nt] + 64 * (ks + kAhead));
            kbl[ks % kAhead][nt] = lds_b8(krl[nt] + 64 * (ks + kAhead));
          }
        }
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) sc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bh[nt], qh[ks], sc[nt], 0, 0, 0);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) sc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bl[nt], qh[ks], sc[nt], 0, 0, 0);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) sc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bh[nt], ql[ks], sc[nt], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // Online softmax of query iw + li (base 2; every lane group holds the
    // query's m and l, the reductions run over the 4 groups).
    const int last = L - a.Sq + iw + li;  // the query's last visible key
    float sv[2][4], mx = -INFINITY;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sv[nt][r] = t0 + 16 * nt + 4 * g + r <= last ? sc[nt][r] * a.scale_log2 : -INFINITY;
        mx = fmaxf(mx, sv[nt][r]);
      }
    mx = mfma::max_over_rows(mx);
    const float m_new = fmaxf(m, mx);
    float al = 1.f, ps = 0.f;
    uint32_t pkh[4], pkl[4];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int r = 0; r < 4; r += 2) {
        float e0 = 0.f, e1 = 0.f;
        if (m_new != -INFINITY) {
          e0 = sv[nt][r] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv[nt][r] - m_new);
          e1 = sv[nt][r + 1] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv[nt][r + 1] - m_new);
        }
        ps += e0 + e1;
        split_bf16x2(e0, e1, pkh[2 * nt + r / 2], pkl[2 * nt + r / 2]);
      }
    if (m_new != -INFINITY) al = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - m_new);
    ps = mfma::sum_over_rows(ps);
    l = l * al + ps;
    m = m_new;
    // O's rows are queries 4 g + r: their rescale factors come from lanes
    // 4 g + r (only when some query's maximum moved).
    if (__any(al != 1.f)) {
      float alr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) alr[r] = __shfl(al, 4 * g + r);
#pragma unroll
      for (int d = 0; d < kAD / 16; ++d)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[d][r] *= alr[r];
    }
    const bf16x8 pah = __builtin_bit_cast(bf16x8, make_uint4(pkh[0], pkh[1], pkh[2], pkh[3]));
    const bf16x8 pal = __builtin_bit_cast(bf16x8, make_uint4(pkl[0], pkl[1], pkl[2], pkl[3]));

    // O += P V.  B operand of column block d: V is key-major in LDS and read
    // transposed (ds_read_b64_tr_b16): lane li of group g reads the 4 values
    // of row 4 g + li / 4 (and 16 rows on), columns 16 d + 4 (li % 4) .. + 3,
    // and the 16-lane transpose hands it column 16 d + li of keys 4 g .. 4 g + 3
    // and 16 + 4 g .. 16 + 4 g + 3: the order of P's keys above.
    const int vrow = 4 * g + (li >> 2), vcol = 8 * (li & 3);  // bytes within the column block
    auto v8 = [&](const char* t, int d) {
      const char* p0 = t + vrow * kVRowB + 32 * d + vcol;
      typedef __attribute__((address_space(3))) mfma::bf16x4 lds_b4;
      const mfma::bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_b4*)(p0));
      const mfma::bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_b4*)(p0 + 16 * kVRowB));
      return __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    // (V operands read one column block ahead)
    constexpr int kVAhead = 1;
    bf16x8 vbh[kVAhead], vbl[kVAhead];
#pragma unroll
    for (int d = 0; d < kVAhead; ++d) vbh[d] = v8(vh_t, d), vbl[d] = v8(vl_t, d);
#pragma unroll
    for (int d = 0; d < kAD / 16; ++d) {
      const bf16x8 vh = vbh[d % kVAhead], vl = vbl[d % kVAhead];
      if (d + kVAhead < kAD / 16) vbh[d % kVAhead] = v8(vh_t, d + kVAhead), vbl[d % kVAhead] = v8(vl_t, d + kVAhead);
      o[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pah, vh, o[d], 0, 0, 0);
      o[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pah, vl, o[d], 0, 0, 0);
      o[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pal, vh, o[d], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // out[query iw + 4 g + r][16 d + li] = O / l and its lse (lane li = 0);
  // with several splits, this split's normalised partial and lse instead.
  // Query q's m and l live in lane q (every group).
  const float inv_q = l > 0.f ? 1.f / l : 0.f;
  const float ls_q = l > 0.f ? (m + log2f(l)) * 0.693147180559945309f : -INFINITY;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = iw + 4 * g + r;
    const float inv = __shfl(inv_q, 4 * g + r);
    const float ls = __shfl(ls_q, 4 * g + r);
    if (i >= a.Sq) continue;
    const int64_t row = ((int64_t)b * a.Sq + i) * a.H + h;
    if (a.splits == 1) {
      float* dst = a.out + row * a.dv;
#pragma unroll
      for (int d = 0; d < kAD / 16; ++d) dst[16 * d + li] = o[d][r] * inv;
      if (a.lse && li == 0) a.lse[row] = ls;
    } else {
      float* dst = a.part_o + (row * a.splits + split) * a.dv;
#pragma unroll
      for (int d = 0; d < kAD / 16; ++d) dst[16 * d + li] = o[d][r] * inv;
      if (li == 0) a.part_lse[row * a.splits + split] = ls;
    }
  }
}

// Merge of the key splits (log-sum-exp rule): one workgroup per (query,
// head), thread d owns output column d.
__global__ __launch_bounds__(kAD) void prefill_merge_kernel(PrefillArgs a) {
  const int64_t row = (int64_t)blockIdx.x * a.H + blockIdx.y;
  const float* lse = a.part_lse + row * a.splits;
  float mx = -INFINITY;
  for (int s = 0; s < a.splits; ++s) mx = fmaxf(mx, lse[s]);
  float z = 0.f, acc = 0.f;
  const int d = threadIdx.x;
  if (mx != -INFINITY)
    for (int s = 0; s < a.splits; ++s) {
      const float w = lse[s] == -INFINITY ? 0.f : expf(lse[s] - mx);
      z += w;
      if (d < a.dv) acc = fmaf(w, a.part_o[(row * a.splits + s) * a.dv + d], acc);
    }
  if (d < a.dv) a.out[row * a.dv + d] = z > 0.f ? acc / z : 0.f;
  if (a.lse && d == 0) a.lse[row] = z > 0.f ? mx + logf(z) : -INFINITY;
}

template <int FMT>
hipError_t launch_fmt(const PrefillArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((a.Lcap + kTokBlk * kBlocks - 1) / (kTokBlk * kBlocks)),
                  (unsigned)((a.dn + a.dv) / kCols), (unsigned)(a.B * a.H));
  switch (a.dc / 32) {
#define MLA_CASE(K) \
  case K: prefill_expand_mfma_kernel<FMT, K><<<grid, 64 * kWaves, 0, s>>>(a); break;
    MLA_CASE(1) MLA_CASE(2) MLA_CASE(3) MLA_CASE(4) MLA_CASE(5) MLA_CASE(6) MLA_CASE(7) MLA_CASE(8)
    MLA_CASE(9) MLA_CASE(10) MLA_CASE(11) MLA_CASE(12) MLA_CASE(13) MLA_CASE(14) MLA_CASE(15) MLA_CASE(16)
#undef MLA_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

bool prefill_attn_mfma_supported(const PrefillArgs& a) {
  return a.dn + a.dr == kAD && a.dv == kAD && a.dn % 4 == 0;
}

// The split count minimises the rounds of the grid per unit of work over
// 256 slots (ties go to fewer splits), with at least 128 keys of capacity
// per split.  Two workgroups run per CU (512 at once on MI355X), but the
// per-split costs (partials, the merge) make a 256-slot model pick better
// on the benchmark's chunks: 4 splits of 4 x 4,096 keys measured 933-937 us
// for the call, against 995-1,002 us with 2 and 963-982 us with 8.
int prefill_attn_splits(int B, int Sq, int H, int64_t Lcap, int dn, int dr, int dv) {
  if (dn + dr != kAD || dv != kAD || dn % 4) return 1;
  constexpr int kSlots = 256;
  const int64_t wgs = (int64_t)B * ((Sq + kAQ * kWaves - 1) / (kAQ * kWaves)) * H;
  const int smax = (int)std::max<int64_t>(1, std::min<int64_t>(16, Lcap / 128));
  int best = 1;
  double best_cost = 1e30;
  for (int sp = 1; sp <= smax; ++sp) {
    const double cost = (double)((wgs * sp + kSlots - 1) / kSlots) / sp;
    if (cost < best_cost - 1e-9) best_cost = cost, best = sp;
  }
  return best;
}

hipError_t launch_prefill_attn_mfma(const PrefillArgs& a, hipStream_t s) {
  if (!prefill_attn_mfma_supported(a) || a.splits < 1 || (a.splits > 1 && (!a.part_o || !a.part_lse)))
    return hipErrorInvalidValue;
  const int64_t qb = (a.Sq + kAQ * kWaves - 1) / (kAQ * kWaves);
  const int64_t units = (int64_t)a.B * a.H * a.splits;
  const int64_t grid = 8 * qb * ((units + 7) / 8);
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  prefill_attn_mfma_kernel<<<dim3((unsigned)grid), 64 * kWaves, 0, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  prefill_merge_kernel<<<dim3((unsigned)(a.B * a.Sq), (unsigned)a.H), kAD, 0, s>>>(a);
  return hipGetLastError();
}

bool prefill_expand_mfma_supported(const PrefillArgs& a) {
  return !a.w_f32 && a.dc % 32 == 0 && a.dc <= 512 && (a.dn + a.dv) % kCols == 0 && a.dr % 4 == 0;
}

hipError_t launch_prefill_expand_mfma(const PrefillArgs& a, int fmt, hipStream_t s) {
  if (!prefill_expand_mfma_supported(a)) return hipErrorInvalidValue;
  const int n = a.dn + a.dv;
  const bool gemm_rows = (fmt == kBF16 && a.dc == 512) || (fmt == kFP8 && a.dc == 448 && a.dr == 64);
  if (gemm_rows && a.dr % 4 == 0 && n % 64 == 0 && n / 64 >= 1 && n / 64 <= 7) {
    const int64_t tiles = (a.Lcap + kGTok - 1) / kGTok;
    const int64_t units = (int64_t)a.B * a.H;
    const int64_t grid = 8 * tiles * ((units + 7) / 8);
    if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
    switch (n / 64) {
#define MLA_CASE(K)                                                                                          \
  case K:                                                                                                    \
    if (fmt == kBF16) prefill_expand_gemm_kernel<kBF16, K><<<dim3((unsigned)grid), kGThreads, 0, s>>>(a, (int)tiles); \
    else prefill_expand_gemm_kernel<kFP8, K><<<dim3((unsigned)grid), kGThreads, 0, s>>>(a, (int)tiles);              \
    break;
      MLA_CASE(1) MLA_CASE(2) MLA_CASE(3) MLA_CASE(4) MLA_CASE(5) MLA_CASE(6) MLA_CASE(7)
#undef MLA_CASE
    }
    return hipGetLastError();
  }
  switch (fmt) {
    case kF32: return launch_fmt<kF32>(a, s);
    case kBF16: return launch_fmt<kBF16>(a, s);
    case kFP8: return launch_fmt<kFP8>(a, s);
    case kFP4: return launch_fmt<kFP4>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mla
