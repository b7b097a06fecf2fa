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
// before the first store) and read k-major with ds_read_b64_tr_b16.  bf16 q
// times bf16 W is exact in fp32.
// out_proj: weight rows are contiguous along K and load straight from
// memory into the B operand.  The fp32 latent input is split into hi + lo
// bf16 parts, so the products are exact to ~16 significant bits;
// accumulation is fp32.
//
// Decode batches are small (tens to hundreds of tokens): the weights are
// read once per step and the cost is memory latency.  A workgroup covers one
// head, 64 output columns (one wave per 16) and one or more 16-token blocks,
// keeping its weight slice (LDS or registers) across its blocks; blocks per
// workgroup are chosen for about 1024 (absorb) or 512 (out_proj) workgroups,
// one block for small batches.  Every load of a block is issued before the first one is waited
// for, and the next block's inputs before this block's products.
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
// The grid is one-dimensional and every workgroup of head h lands on XCD
// h % 8, so a head's weight slice and its tokens' inputs come from HBM once
// and are then shared in that L2 by the head's token and column blocks (a
// grid over (tokens, columns, heads) fetched them once per XCD that ran any
// of them, up to 8 times).  XCDs with fewer heads get idle workgroups.
constexpr int kXcds = 8;
struct ProjCell {
  int h, col_group, tok_group;
  bool valid;
};
__device__ __forceinline__ ProjCell proj_cell(int col_groups, int tok_groups, int H) {
  const int L = blockIdx.x;
  const int x = L % kXcds, k = L / kXcds;
  const int per_head = col_groups * tok_groups;
  const int h = x + kXcds * (k / per_head), r = k % per_head;
  return ProjCell{h, r % col_groups, r / col_groups, h < H};
}
// Grid size for proj_cell: 8 x (the most heads an XCD gets) x cells per head.
unsigned proj_grid(int col_groups, int tok_groups, int H) {
  return (unsigned)(kXcds * ((H + kXcds - 1) / kXcds) * col_groups * tok_groups);
}
// At most `per_cu` workgroups per CU on the busiest XCD (32 CUs): fewer,
// larger token groups when the heads do not spread evenly over the XCDs.
void cap_token_groups(ProjArgs& a, int col_groups, unsigned& gx, int per_cu) {
  const int nblk = (a.N + kTok - 1) / kTok;
  const int cap = std::max(1, 32 * per_cu / (((a.H + kXcds - 1) / kXcds) * col_groups));
  if ((int)gx <= cap) return;
  a.tok_blocks = (nblk + cap - 1) / cap;
  gx = (unsigned)((nblk + a.tok_blocks - 1) / a.tok_blocks);
}

template <bool kOutF32, int NKS>  // NKS = d_nope / 32
__global__ __launch_bounds__(64 * kWaves) void absorb_mfma_kernel(ProjArgs a) {
  constexpr int kRows = 32 * NKS;               // d_nope
  constexpr int kChunks = kRows * (kCols / 8);  // 16-B chunks of the weight tile
  constexpr int kPer = (kChunks + 64 * kWaves - 1) / (64 * kWaves);
  __shared__ __attribute__((aligned(16))) char w_tile[kRows * kWRow];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, li = lane & 15;
  const ProjCell cell = proj_cell(a.dc / kCols, a.tok_groups, a.H);
  if (!cell.valid) return;
  const int h = cell.h, c0 = cell.col_group * kCols;
  const int n0 = cell.tok_group * kTok * a.tok_blocks;
  const uint16_t* w = static_cast<const uint16_t*>(a.w) + (int64_t)h * (a.dn + a.dv) * a.dc;

  // Weight tile W[0:dn][c0:c0+64] and the query operands: every load is
  // issued before the first one is waited for.
  // (Indices past the tile are clamped, not branched around, so that the
  // loads are issued back to back.)
  u32x4 wt[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = min(j * 64 * kWaves + (int)threadIdx.x, kChunks - 1);
    wt[j] = *reinterpret_cast<const u32x4*>(w + (int64_t)(i >> 3) * a.dc + c0 + 8 * (i & 7));
  }
  const int qw = a.dn + a.dr, ow = a.dc + a.dr;
  const bf16x8 zero = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
  // Query operands of a token block (padding tokens read token 0, no branch
  // around the loads, and use zeros).  The first column block also copies
  // the RoPE part of the query: thread t holds values t, t + 256, ... of the
  // block's kTok x d_rope part, loaded with the query operands.
  constexpr int kRopePer = kTok * kMaxRope / (64 * kWaves);
  const uint16_t* qin = static_cast<const uint16_t*>(a.in);
  const bool rope_wg = cell.col_group == 0;
  auto load_q = [&](int nb, bf16x8 (&qv)[NKS], uint16_t (&rv)[kRopePer]) __attribute__((always_inline)) {
    const int n = nb + li;
    const uint16_t* q = qin + ((int64_t)(n < a.N ? n : 0) * a.H + h) * qw;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qv[ks] = load_bf16x8(q + 32 * ks + 8 * g);
    if (rope_wg) {
#pragma unroll
      for (int u = 0; u < kRopePer; ++u) {
        const int i = min(u * 64 * kWaves + (int)threadIdx.x, kTok * a.dr - 1);
        const int nn = min(nb + i / a.dr, a.N - 1);
        rv[u] = qin[((int64_t)nn * a.H + h) * qw + a.dn + i % a.dr];
      }
    }
  };
  bf16x8 qa[NKS];
  uint16_t ra[kRopePer];
  load_q(n0, qa, ra);
  __builtin_amdgcn_sched_barrier(0);  // all loads issued before the first is waited for
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = j * 64 * kWaves + threadIdx.x;
    if (i < kChunks) *reinterpret_cast<u32x4*>(w_tile + (i >> 3) * kWRow + 16 * (i & 7)) = wt[j];
  }
  __syncthreads();

  // The workgroup's token blocks share the weight tile; the next block's
  // queries are requested before this block's products.
  const int nb_end = min(a.N, n0 + kTok * a.tok_blocks);
  for (int nb = n0; nb < nb_end; nb += kTok) {
    bf16x8 qn[NKS];
    uint16_t rn[kRopePer];
    if (nb + kTok < nb_end) load_q(nb + kTok, qn, rn);
    if (nb + li >= a.N) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) qa[ks] = zero;
    }
    // This wave's 16 columns c0 + 16 * wave + li.
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const char* rows = w_tile + (32 * ks + 8 * g + (li >> 2)) * kWRow + 32 * wave + 8 * (li & 3);
      const bf16x4 b0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)rows);
      const bf16x4 b1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(rows + 4 * kWRow));
      const bf16x8 wb = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ks], wb, acc, 0, 0, 0);
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
        const int nn = nb + i / a.dr, k = i % a.dr;
        if (i >= kTok * a.dr || nn >= a.N) continue;
        const int64_t r = (int64_t)nn * a.H + h;
        if (kOutF32) static_cast<float*>(a.out)[r * ow + a.dc + k] = bf16_bits_to_f32(ra[u]);
        else static_cast<uint16_t*>(a.out)[r * ow + a.dc + k] = ra[u];
      }
    }
    if (nb + kTok < nb_end) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) qa[ks] = qn[ks];
      if (rope_wg) {
#pragma unroll
        for (int u = 0; u < kRopePer; ++u) ra[u] = rn[u];
      }
    }
  }
}

constexpr int kMaxLatent = 512;

template <int NKS>  // NKS = d_latent / 32
__global__ __launch_bounds__(64 * kWaves) void out_proj_mfma_kernel(ProjArgs a) {
  // The token block's fp32 latent rows (16 x d_latent) are the A operand of
  // all four waves.  They are staged once per workgroup in LDS and read back
  // per k-step, instead of each wave holding all of them in registers: that
  // keeps the kernel near 120 VGPRs, four workgroups per CU.  The next
  // block's rows are requested before this block's products.
  constexpr int kDc = 32 * NKS;
  constexpr int kRow = kDc * 4 + 16;  // LDS row stride: rows start 16 B apart in the bank cycle
  constexpr int kQuads = kDc / 4;     // float4 per row
  constexpr int kChunks = kTok * kQuads;
  constexpr int kPer = (kChunks + 64 * kWaves - 1) / (64 * kWaves);
  __shared__ __attribute__((aligned(16))) char o_tile[kTok * kRow];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, li = lane & 15;
  const ProjCell cell = proj_cell(a.dv / kCols, a.tok_groups, a.H);
  if (!cell.valid) return;
  const int h = cell.h, v = cell.col_group * kCols + 16 * wave + li;
  const int n0 = cell.tok_group * kTok * a.tok_blocks;
  const uint16_t* w = static_cast<const uint16_t*>(a.w) + ((int64_t)h * (a.dn + a.dv) + a.dn + v) * a.dc;

  // B operand: this lane's weight row (value column v), all of K, kept for
  // every token block of the workgroup.
  bf16x8 wb[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) wb[ks] = load_bf16x8(w + 32 * ks + 8 * g);

  // Latent rows of token block nb: thread t loads quads t, t + 256, ...
  // (indices clamped, not branched around; padding tokens read token 0).
  float4 st[kPer];
  auto load_rows = [&](int nb) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int i = min(j * 64 * kWaves + (int)threadIdx.x, kChunks - 1);
      const int n = nb + i / kQuads;
      st[j] = reinterpret_cast<const float4*>(static_cast<const float*>(a.in) +
                                              ((int64_t)(n < a.N ? n : 0) * a.H + h) * a.dc)[i % kQuads];
    }
  };
  load_rows(n0);
  __builtin_amdgcn_sched_barrier(0);  // weights and rows requested before the first wait

  float* out = static_cast<float*>(a.out);
  const int nb_end = min(a.N, n0 + kTok * a.tok_blocks);
  for (int nb = n0; nb < nb_end; nb += kTok) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int i = j * 64 * kWaves + threadIdx.x;
      if (i < kChunks) {
        const int r = i / kQuads;
        *reinterpret_cast<float4*>(o_tile + r * kRow + 16 * (i % kQuads)) =
            nb + r < a.N ? st[j] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    __syncthreads();
    if (nb + kTok < nb_end) load_rows(nb + kTok);
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
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
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, wb[ks], acc, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int nn = nb + 4 * g + i;
      if (nn < a.N) out[((int64_t)nn * a.H + h) * a.dv + v] = acc[i];
    }
    __syncthreads();  // the tile is rewritten for the next block
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
  // about 1024 workgroups: at 88 VGPRs and 27 KB of LDS five fit per CU, and
  // fewer blocks per workgroup measured faster (at 256 tokens, 2 blocks:
  // 17.6 us; 4 blocks: 19.5 us)
  a.tok_blocks = token_blocks(a.N, a.dc / kCols, a.H, gx, 1024);
  cap_token_groups(a, a.dc / kCols, gx, 5);
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
  a.tok_blocks = token_blocks(a.N, a.dv / kCols, a.H, gx, 512);
  cap_token_groups(a, a.dv / kCols, gx, 4);
  a.tok_groups = (int)gx;
  const dim3 grid(proj_grid(a.dv / kCols, a.tok_groups, a.H));
  switch (a.dc / 32) {
#define MLA_CASE(K) \
  case K: out_proj_mfma_kernel<K><<<grid, 64 * kWaves, 0, s>>>(a); break;
    MLA_CASE(1) MLA_CASE(2) MLA_CASE(3) MLA_CASE(4) MLA_CASE(5) MLA_CASE(6) MLA_CASE(7) MLA_CASE(8)
    MLA_CASE(9) MLA_CASE(10) MLA_CASE(11) MLA_CASE(12) MLA_CASE(13) MLA_CASE(14) MLA_CASE(15) MLA_CASE(16)
#undef MLA_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mla
