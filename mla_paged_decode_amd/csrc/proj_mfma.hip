// Query absorption and value up-projection on the matrix cores.
//
// Both are per-head GEMMs with the head's slice of kv_b_proj
// ([d_nope + d_v][d_latent], row-major, bf16):
//   absorb:   q_lat[n][c] = sum_k q[n][k] * W[k][c]          (K = d_nope)
//   out_proj: out[n][v]   = sum_c o[n][c] * W[d_nope + v][c] (K = d_latent)
// with v_mfma_f32_16x16x32_bf16 (A: row l%16, k 8g..8g+7; B: column l%16,
// k 8g..8g+7; C: column l%16, rows 4g..4g+3; g = lane / 16).
//
// absorb: the weight's contiguous dimension is the output column, so the
// workgroup's d_nope x 64 weight tile is staged in LDS (all loads issued
// before the first store) and read k-major with ds_read_b64_tr_b16; the
// queries (the A operand all four waves share) are staged in LDS too.  bf16
// q times bf16 W is exact in fp32.
// out_proj: weight rows are contiguous along K and load straight from
// memory into the B operand.  The fp32 latent input is split into hi + lo
// bf16 parts, so the products are exact to ~16 significant bits;
// accumulation is fp32.
//
// Decode batches are small (tens to hundreds of tokens): the weights are
// read once per step and the cost is memory latency.  A workgroup covers one
// head, 64 output columns (one wave per 16) and one or more 16-token blocks,
// keeping its weight slice (LDS or registers) across its blocks.  The grid is
// one round of workgroups (three per CU), and a workgroup requests its
// weights and the inputs of up to four (absorb) or two (out_proj) token
// blocks before it waits for any of them: one memory round trip.
// The grid is one-dimensional and XCD-aware (proj_cell below).
#include <algorithm>

#include "device_common.h"
#include "internal.h"

namespace mla {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

constexpr int kWaves = 4;
constexpr int kTok = 16;                  // tokens per workgroup
constexpr int kCols = 16 * kWaves;        // output columns per workgroup
constexpr int kMaxNope = 512;
constexpr int kMaxRope = 64;            // d_rope (the host accepts 64 only)
constexpr int kWRow = kCols * 2 + 16;     // LDS row stride (bytes) of the weight tile

__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

// Workgroups are dispatched round-robin over the 8 XCDs, each with its own L2.
// The grid is one-dimensional.  The H x col_groups (head, column group)
// pairs are dealt to the XCDs in contiguous runs of equal length (XCD x takes
// pairs [x U / 8, (x + 1) U / 8), U = H col_groups, a head's pairs being
// consecutive), and an XCD's workgroups take its pairs one after another, the
// token groups of a pair together.  A head's weight slice and its tokens'
// inputs thus come from HBM once per XCD holding one of its pairs (one or
// two XCDs once a run is at least a head long) and are then shared in that
// L2, and no XCD holds more than ceil(U / 8) pairs.  (Whole heads per XCD,
// head h on XCD h % 8, left 3 heads on some XCDs and 2 on others at 20
// heads, and the launch took as long as the busiest XCD.)
constexpr int kXcds = 8;
struct ProjCell {
  int h, col_group, tok_group;
  bool valid;
};
__device__ __forceinline__ ProjCell proj_cell(int col_groups, int tok_groups, int H) {
  const int L = blockIdx.x;
  const int x = L % kXcds, k = L / kXcds;
  const int U = H * col_groups;
  const int u = x * U / kXcds + k / tok_groups;
  return ProjCell{u / col_groups, u % col_groups, k % tok_groups, u < (x + 1) * U / kXcds};
}
// The most (head, column group) pairs an XCD holds.
int pairs_per_xcd(int col_groups, int H) { return (H * col_groups + kXcds - 1) / kXcds; }
// Grid size for proj_cell: 8 x (the most pairs an XCD holds) x token groups.
unsigned proj_grid(int col_groups, int tok_groups, int H) {
  return (unsigned)(kXcds * pairs_per_xcd(col_groups, H) * tok_groups);
}
// At most `per_cu` workgroups per CU on the busiest XCD (32 CUs): fewer,
// larger token groups when an XCD holds many pairs.
void cap_token_groups(ProjArgs& a, int col_groups, unsigned& gx, int per_cu) {
  const int nblk = (a.N + kTok - 1) / kTok;
  const int cap = std::max(1, 32 * per_cu / pairs_per_xcd(col_groups, a.H));
  if ((int)gx <= cap) return;
  a.tok_blocks = (nblk + cap - 1) / cap;
  gx = (unsigned)((nblk + a.tok_blocks - 1) / a.tok_blocks);
}

template <bool kOutF32, int NKS>  // NKS = d_nope / 32
__global__ __launch_bounds__(64 * kWaves) void absorb_mfma_kernel(ProjArgs a) {
  constexpr int kRows = 32 * NKS;               // d_nope
  constexpr int kChunks = kRows * (kCols / 8);  // 16-B chunks of the weight tile
  constexpr int kPer = (kChunks + 64 * kWaves - 1) / (64 * kWaves);
  // Token blocks whose queries are staged together (fewer for wide d_nope,
  // to keep the LDS of three workgroups per CU).
  constexpr int kBlk = NKS <= 8 ? 4 : 2;
  constexpr int kQRow = kRows * 2 + 16;          // LDS row stride (bytes) of the query tile
  constexpr int kQChunks = kBlk * kTok * (kRows / 8);
  constexpr int kQPer = (kQChunks + 64 * kWaves - 1) / (64 * kWaves);
  __shared__ __attribute__((aligned(16))) char w_tile[kRows * kWRow];
  __shared__ __attribute__((aligned(16))) char q_tile[kBlk * kTok * kQRow];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, li = lane & 15;
  const ProjCell cell = proj_cell(a.dc / kCols, a.tok_groups, a.H);
  if (!cell.valid) return;
  const int h = cell.h, c0 = cell.col_group * kCols;
  const int n0 = cell.tok_group * kTok * a.tok_blocks;
  const uint16_t* w = static_cast<const uint16_t*>(a.w) + (int64_t)h * (a.dn + a.dv) * a.dc;
  const int qw = a.dn + a.dr, ow = a.dc + a.dr;
  const uint16_t* qin = static_cast<const uint16_t*>(a.in);
  const bool rope_wg = cell.col_group == 0;
  constexpr int kRopePer = kTok * kMaxRope / (64 * kWaves);
  const int nb_end = min(a.N, n0 + kTok * a.tok_blocks);

  // The weight tile W[0:dn][c0:c0+64] and the d_nope part of kBlk token
  // blocks' queries (the A operand every wave shares) go through LDS: the
  // workgroup loads each once, and every load is issued before the first one
  // is waited for, so the workgroup waits one memory round trip.  Indices
  // past a tile are clamped, not branched around (padding tokens read the
  // last token; their products are never stored).
  u32x4 wt[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = min(j * 64 * kWaves + (int)threadIdx.x, kChunks - 1);
    wt[j] = *reinterpret_cast<const u32x4*>(w + (int64_t)(i >> 3) * a.dc + c0 + 8 * (i & 7));
  }
  bool first = true;
  for (int nc = n0; nc < nb_end; nc += kTok * kBlk) {
    u32x4 qt[kQPer];
#pragma unroll
    for (int j = 0; j < kQPer; ++j) {
      const int i = min(j * 64 * kWaves + (int)threadIdx.x, kQChunks - 1);
      const int n = min(nc + i / (kRows / 8), a.N - 1);  // token (block-major, 16 per block)
      qt[j] = *reinterpret_cast<const u32x4*>(qin + ((int64_t)n * a.H + h) * qw + 8 * (i % (kRows / 8)));
    }
    // The RoPE part of the query is copied by the first column group: thread
    // t holds values t, t + 256, ... of each block's kTok x d_rope part.
    uint16_t ra[kBlk][kRopePer];
    if (rope_wg) {
#pragma unroll
      for (int k = 0; k < kBlk; ++k)
#pragma unroll
        for (int u = 0; u < kRopePer; ++u) {
          const int i = min(u * 64 * kWaves + (int)threadIdx.x, kTok * a.dr - 1);
          const int nn = min(nc + k * kTok + i / a.dr, a.N - 1);
          ra[k][u] = qin[((int64_t)nn * a.H + h) * qw + a.dn + i % a.dr];
        }
    }
    __builtin_amdgcn_sched_barrier(0);  // all loads issued before the first is waited for
    if (!first) __syncthreads();        // the previous blocks' readers of q_tile are done
    if (first) {
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int i = j * 64 * kWaves + threadIdx.x;
        if (i < kChunks) *reinterpret_cast<u32x4*>(w_tile + (i >> 3) * kWRow + 16 * (i & 7)) = wt[j];
      }
      first = false;
    }
#pragma unroll
    for (int j = 0; j < kQPer; ++j) {
      const int i = j * 64 * kWaves + threadIdx.x;
      if (i < kQChunks)
        *reinterpret_cast<u32x4*>(q_tile + (i / (kRows / 8)) * kQRow + 16 * (i % (kRows / 8))) = qt[j];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kBlk; ++k) {
      const int nb = nc + k * kTok;
      if (nb >= nb_end) break;
      // This wave's 16 columns c0 + 16 * wave + li; A rows are tokens.
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
      const char* qrow = q_tile + (k * kTok + li) * kQRow + 16 * g;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const bf16x8 qa = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qrow + 64 * ks));
        const char* rows = w_tile + (32 * ks + 8 * g + (li >> 2)) * kWRow + 32 * wave + 8 * (li & 3);
        const bf16x4 b0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)rows);
        const bf16x4 b1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(rows + 4 * kWRow));
        const bf16x8 wb = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa, wb, acc, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int nn = nb + 4 * g + i;
        if (nn >= a.N) continue;
        const int64_t o = ((int64_t)nn * a.H + h) * ow + c0 + 16 * wave + li;
        if (kOutF32) static_cast<float*>(a.out)[o] = acc[i];
        else static_cast<uint16_t*>(a.out)[o] = (uint16_t)f32_to_bf16_bits(acc[i]);
      }
      if (rope_wg) {
#pragma unroll
        for (int u = 0; u < kRopePer; ++u) {
          const int i = u * 64 * kWaves + threadIdx.x;
          const int nn = nb + i / a.dr, kk = i % a.dr;
          if (i >= kTok * a.dr || nn >= a.N) continue;
          const int64_t r = (int64_t)nn * a.H + h;
          if (kOutF32) static_cast<float*>(a.out)[r * ow + a.dc + kk] = bf16_bits_to_f32(ra[k][u]);
          else static_cast<uint16_t*>(a.out)[r * ow + a.dc + kk] = ra[k][u];
        }
      }
    }
  }
}

constexpr int kMaxLatent = 512;

// out_proj: NW waves of 16 value columns each, NB token blocks whose rows
// are requested together with the weights (one memory round trip).
template <int NKS, int NW, int NB>  // NKS = d_latent / 32
__global__ __launch_bounds__(64 * NW, NW == 4 ? 3 : 1) void out_proj_mfma_kernel(ProjArgs a) {
  // The token block's fp32 latent rows (16 x d_latent) are the A operand of
  // all the waves.  They are staged once per workgroup in LDS and read back
  // per k-step, instead of each wave holding all of them in registers.
  constexpr int kC = 16 * NW;  // value columns per workgroup
  constexpr int kDc = 32 * NKS;
  constexpr int kRow = kDc * 4 + 16;  // LDS row stride: rows start 16 B apart in the bank cycle
  constexpr int kQuads = kDc / 4;     // float4 per row
  constexpr int kChunks = kTok * kQuads;
  constexpr int kPer = (kChunks + 64 * NW - 1) / (64 * NW);
  __shared__ __attribute__((aligned(16))) char o_tile[kTok * kRow];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, li = lane & 15;
  const ProjCell cell = proj_cell(a.dv / kC, a.tok_groups, a.H);
  if (!cell.valid) return;
  const int h = cell.h, v = cell.col_group * kC + 16 * wave + li;
  const int n0 = cell.tok_group * kTok * a.tok_blocks;
  const uint16_t* w = static_cast<const uint16_t*>(a.w) + ((int64_t)h * (a.dn + a.dv) + a.dn + v) * a.dc;

  // B operand: this lane's weight row (value column v), all of K, kept for
  // every token block of the workgroup.
  bf16x8 wb[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) wb[ks] = load_bf16x8(w + 32 * ks + 8 * g);

  // Latent rows of token block nb: thread t loads quads t, t + 64 NW, ...
  // (indices clamped, not branched around; padding tokens read token 0).
  float4 st[NB][kPer];
  auto load_rows = [&](int nb, float4 (&dst)[kPer]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int i = min(j * 64 * NW + (int)threadIdx.x, kChunks - 1);
      const int n = nb + i / kQuads;
      dst[j] = reinterpret_cast<const float4*>(static_cast<const float*>(a.in) +
                                               ((int64_t)(n < a.N ? n : 0) * a.H + h) * a.dc)[i % kQuads];
    }
  };

  float* out = static_cast<float*>(a.out);
  const int nb_end = min(a.N, n0 + kTok * a.tok_blocks);
  for (int nc = n0; nc < nb_end; nc += kTok * NB) {
#pragma unroll
    for (int k = 0; k < NB; ++k)
      if (nc + k * kTok < nb_end) load_rows(nc + k * kTok, st[k]);
    __builtin_amdgcn_sched_barrier(0);  // weights and rows requested before the first wait
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const int nb = nc + k * kTok;
      if (nb >= nb_end) break;
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int i = j * 64 * NW + threadIdx.x;
        if (i < kChunks) {
          const int r = i / kQuads;
          *reinterpret_cast<float4*>(o_tile + r * kRow + 16 * (i % kQuads)) =
              nb + r < a.N ? st[k][j] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
      __syncthreads();
      // hi and lo products in two accumulation chains, added at the end
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f}, acl = f32x4{0.f, 0.f, 0.f, 0.f};
      const char* arow = o_tile + li * kRow + 32 * g;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const float4 x0 = *reinterpret_cast<const float4*>(arow + 128 * ks);
        const float4 x1 = *reinterpret_cast<const float4*>(arow + 128 * ks + 16);
        const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) split_bf16x2(x[2 * i], x[2 * i + 1], hw[i], lw[i]);
        const bf16x8 ah = __builtin_bit_cast(bf16x8, make_uint4(hw[0], hw[1], hw[2], hw[3]));
        const bf16x8 al = __builtin_bit_cast(bf16x8, make_uint4(lw[0], lw[1], lw[2], lw[3]));
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, wb[ks], acc, 0, 0, 0);
        acl = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, wb[ks], acl, 0, 0, 0);
      }
      acc += acl;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int nn = nb + 4 * g + i;
        if (nn < a.N) out[((int64_t)nn * a.H + h) * a.dv + v] = acc[i];
      }
      __syncthreads();  // the tile is rewritten for the next block
    }
  }
}

// 16-token blocks per workgroup: about `target` workgroups, so that small batches
// get one block each and batches of hundreds of tokens a few, with every
// workgroup's weight slice loaded once for all of them.
int token_blocks(int N, int col_groups, int H, unsigned& grid_x, int target) {
  const int nblk = (N + kTok - 1) / kTok;
  int tb = (int)std::max<int64_t>(1, (int64_t)nblk * col_groups * H / target);
  tb = std::min(tb, nblk);
  const int gx = (nblk + tb - 1) / tb;
  grid_x = (unsigned)gx;
  return (nblk + gx - 1) / gx;
}

}  // namespace

bool absorb_mfma_supported(const ProjArgs& a) {
  return !a.in_f32 && !a.w_f32 && a.dc % kCols == 0 && a.dn % 32 == 0 && a.dn <= kMaxNope && a.dr % 16 == 0 && a.dr <= kMaxRope;
}

bool out_proj_mfma_supported(const ProjArgs& a) {
  return !a.w_f32 && a.dv % kCols == 0 && a.dc % 32 == 0 && a.dc <= kMaxLatent;
}

hipError_t launch_absorb_mfma(const ProjArgs& args, hipStream_t s) {
  ProjArgs a = args;
  unsigned gx;
  // One round of workgroups: three fit per CU (53 KB of LDS and 160 VGPRs
  // with d_nope = 192), and a workgroup's token blocks (up to four) cost one
  // memory round trip together.
  a.tok_blocks = token_blocks(a.N, a.dc / kCols, a.H, gx, 768);
  cap_token_groups(a, a.dc / kCols, gx, 3);
  a.tok_groups = (int)gx;
  const dim3 grid(proj_grid(a.dc / kCols, a.tok_groups, a.H));
  switch (a.dn / 32) {
#define MLA_CASE(K)                                                                   \
  case K:                                                                             \
    if (a.out_f32) absorb_mfma_kernel<true, K><<<grid, 64 * kWaves, 0, s>>>(a);       \
    else absorb_mfma_kernel<false, K><<<grid, 64 * kWaves, 0, s>>>(a);                \
    break;
    MLA_CASE(1) MLA_CASE(2) MLA_CASE(3) MLA_CASE(4) MLA_CASE(5) MLA_CASE(6) MLA_CASE(7) MLA_CASE(8)
    MLA_CASE(9) MLA_CASE(10) MLA_CASE(11) MLA_CASE(12) MLA_CASE(13) MLA_CASE(14) MLA_CASE(15) MLA_CASE(16)
#undef MLA_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_out_proj_mfma(const ProjArgs& args, hipStream_t s) {
  ProjArgs a = args;
  unsigned gx;
  // One round of workgroups (three per CU at 164 VGPRs); a workgroup's rows
  // of two token blocks cost one memory round trip together.  (Eight-wave
  // workgroups with four blocks, one per CU, halve the L2 traffic but
  // measured slower at 256 tokens: 18.2-20.9 us against 15.9-18.7 us.)
  a.tok_blocks = token_blocks(a.N, a.dv / kCols, a.H, gx, 768);
  cap_token_groups(a, a.dv / kCols, gx, 3);
  a.tok_groups = (int)gx;
  const dim3 grid(proj_grid(a.dv / kCols, a.tok_groups, a.H));
  switch (a.dc / 32) {
#define MLA_CASE(K) \
  case K: out_proj_mfma_kernel<K, kWaves, 2><<<grid, 64 * kWaves, 0, s>>>(a); break;
    MLA_CASE(1) MLA_CASE(2) MLA_CASE(3) MLA_CASE(4) MLA_CASE(5) MLA_CASE(6) MLA_CASE(7) MLA_CASE(8)
    MLA_CASE(9) MLA_CASE(10) MLA_CASE(11) MLA_CASE(12) MLA_CASE(13) MLA_CASE(14) MLA_CASE(15) MLA_CASE(16)
#undef MLA_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mla
