// Split-KV planning and the log-sum-exp merge of partial results.
//
// Partials over disjoint token sets s, each normalised (o_s) with its
// log-sum-exp lse_s, merge exactly into the result over their union:
//   lse = log sum_s exp(lse_s),   o = sum_s exp(lse_s - lse) * o_s.
// Parts with lse_s = -inf carry no weight; if every part is empty the row
// has no visible token and gets o = 0, lse = -inf.
#include <cmath>

#include "internal.h"
#include "schedule.h"

namespace mla {
namespace {

constexpr int kPlanThreads = 1024;

// The balanced plan (schedule.h) for batches too large for the decode
// kernel to plan itself.
__global__ __launch_bounds__(kPlanThreads) void plan_kernel(const int32_t* __restrict__ lens, int B, int G,
                                                            int32_t* __restrict__ tile_start) {
  __shared__ int64_t s[kPlanThreads];
  block_plan(lens, B, G, tile_start, s);
}

constexpr int kCombineThreads = 128;  // x 4 values = one 512-wide latent row per pass
constexpr int kMaxParts = 4096;       // partial slots one sequence can have
constexpr int kUnroll = 8;            // partial rows in flight per thread

__device__ __forceinline__ float block_reduce(float v, float* red, bool is_max) {
  for (int o = 32; o >= 1; o >>= 1) {
    const float u = __shfl_xor(v, o);
    v = is_max ? fmaxf(v, u) : v + u;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();  // red[] free
  if (lane == 0) red[wave] = v;
  __syncthreads();
  v = red[0];
  for (int w = 1; w < kCombineThreads / 64; ++w) v = is_max ? fmaxf(v, red[w]) : v + red[w];
  return v;
}

// One workgroup per (sequence, query row).  The slots' log-sum-exps are
// read in parallel and reduced in LDS; then each thread sums 4 consecutive
// values of the partial rows with kUnroll independent 16-byte loads in
// flight.
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(DecodeArgs a) {
  __shared__ float s_w[kMaxParts];
  __shared__ int32_t s_slot[kMaxParts];
  __shared__ float red[kCombineThreads / 64];
  const int b = blockIdx.x / a.R;
  const int row = blockIdx.x % a.R;
  const int tid = threadIdx.x;

  // Candidate parts: uniform mode, splits 0..S-1 (slot b*S + s); balanced
  // mode, the workers g0..g1 that own real tiles of the sequence (slot
  // g + b), skipping workers with no positions at all.
  int64_t g0 = 0, n = 0;
  int64_t N = 0, G = a.workers;
  if (a.num_splits > 0) {
    n = a.num_splits;
  } else {
    const int64_t te = a.tile_start[b + 1];
    const int64_t ts = a.tile_start[b] + plan_lead(a.tile_start[b], te, a.tile_start[a.B + 1]);  // first real tile
    N = a.tile_start[a.B];
    if (ts < te) {
      g0 = worker_of_tile(ts, N, G);
      n = worker_of_tile(te - 1, N, G) - g0 + 1;
    }
  }
  for (int64_t i = tid; i < n; i += kCombineThreads) {
    int64_t slot;
    bool ok = true;
    if (a.num_splits > 0) {
      slot = (int64_t)b * a.num_splits + i;
    } else {
      const int64_t g = g0 + i;
      ok = worker_tile_begin(g, N, G) < worker_tile_begin(g + 1, N, G);
      slot = g + b;
    }
    s_slot[i] = ok ? (int32_t)slot : -1;
  }
  __syncthreads();

  // The first kUnroll partial rows are requested before their weights are
  // known; the log-sum-exps are read meanwhile.
  const float* po = a.part_o + (int64_t)row * a.dc;
  const int64_t slot_stride = (int64_t)a.R * a.dc;
  const int d4 = tid;  // this thread's 4 values (first pass)
  const bool d_ok = d4 < a.dc / 4;
  float4 pre[kUnroll];
#pragma unroll
  for (int j = 0; j < kUnroll; ++j) {
    const int32_t sl = j < n ? s_slot[j] : -1;
    pre[j] = d_ok && sl >= 0 ? reinterpret_cast<const float4*>(po + sl * slot_stride)[d4]
                             : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float m = -INFINITY;
  for (int64_t i = tid; i < n; i += kCombineThreads) {
    const int32_t sl = s_slot[i];
    const float l = sl >= 0 ? a.part_lse[(int64_t)sl * a.R + row] : -INFINITY;
    s_w[i] = l;
    m = fmaxf(m, l);
  }
  m = block_reduce(m, red, true);
  const int64_t out_row = (int64_t)b * a.R + row;
  if (m == -INFINITY) {
    for (int d = tid; d < a.dc; d += kCombineThreads) a.o[out_row * a.dc + d] = 0.f;
    if (a.lse && tid == 0) a.lse[out_row] = -INFINITY;
    return;
  }
  float z = 0.f;
  for (int64_t i = tid; i < n; i += kCombineThreads) {
    const float w = s_w[i] == -INFINITY ? 0.f : expf(s_w[i] - m);
    s_w[i] = w;
    z += w;
  }
  z = block_reduce(z, red, false);  // also orders the s_w writes before the reads below
  const float inv = 1.f / z;
  // Rows with zero weight (no visible token in that part, or a worker
  // without tiles) are selected away, never multiplied.
  auto accumulate = [&](float4& c, float w, const float4& p) {
    const bool use = w != 0.f;
    c.x = fmaf(w, use ? p.x : 0.f, c.x);
    c.y = fmaf(w, use ? p.y : 0.f, c.y);
    c.z = fmaf(w, use ? p.z : 0.f, c.z);
    c.w = fmaf(w, use ? p.w : 0.f, c.w);
  };
  for (int dd = d4; dd < a.dc / 4; dd += kCombineThreads) {
    float4 acc[2] = {make_float4(0.f, 0.f, 0.f, 0.f), make_float4(0.f, 0.f, 0.f, 0.f)};
    int64_t i0 = 0;
    if (dd == d4) {
#pragma unroll
      for (int j = 0; j < kUnroll; ++j) accumulate(acc[j & 1], j < n ? s_w[j] : 0.f, pre[j]);
      i0 = kUnroll;
    }
    for (; i0 < n; i0 += kUnroll) {
      float4 p[kUnroll];
#pragma unroll
      for (int j = 0; j < kUnroll; ++j) {
        const int32_t sl = i0 + j < n ? s_slot[i0 + j] : -1;
        p[j] = sl >= 0 ? reinterpret_cast<const float4*>(po + sl * slot_stride)[dd] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int j = 0; j < kUnroll; ++j) accumulate(acc[j & 1], i0 + j < n ? s_w[i0 + j] : 0.f, p[j]);
    }
    reinterpret_cast<float4*>(a.o + out_row * a.dc)[dd] =
        make_float4((acc[0].x + acc[1].x) * inv, (acc[0].y + acc[1].y) * inv,
                    (acc[0].z + acc[1].z) * inv, (acc[0].w + acc[1].w) * inv);
  }
  if (a.lse && tid == 0) a.lse[out_row] = m + logf(z);
}

// Merge for the tiled partial layout of the matrix-core kernel.  One
// workgroup per (sequence, 16-row block, DPW column blocks of 16).  Lane l of
// a wave owns column 16d + l%16 of rows 16w + 4(l/16) + i, i = 0..3, which
// are one float4 of every partial.  With DPW >= 4 each wave takes DPW/4
// column blocks and all the parts; with DPW < 4, 4/DPW waves share a column
// block, split its parts and are summed in LDS at the end.  Parts are
// processed in chunks of kChunk: a first pass over the chunks' log-sum-exps
// gives each row's maximum and sum (merged online across chunks), a second
// pass weights and sums the partial rows.  With one chunk (the usual case)
// the second pass reuses the slots and weights already in LDS, and the
// first partial rows are requested with the first log-sum-exps.
constexpr int kTiledThreads = 256;
constexpr int kTiledWaves = kTiledThreads / 64;
constexpr int kChunk = 64;

// 32-bit forms of the balanced-split worker ranges (tile counts < 2^22,
// workers <= 1024).
__device__ __forceinline__ int64_t tiles_begin(int64_t g, int64_t N, int64_t G) {
  return N < (1 << 22) ? (int64_t)((uint32_t)(g * N) / (uint32_t)G) : worker_tile_begin(g, N, G);
}
__device__ __forceinline__ int64_t worker_of(int64_t t, int64_t N, int64_t G) {
  return N < (1 << 22) && G <= 1024 ? (int64_t)((uint32_t)((t + 1) * G - 1) / (uint32_t)N) : worker_of_tile(t, N, G);
}

template <int DPW>
__global__ __launch_bounds__(kTiledThreads, 4) void combine_tiled_kernel(DecodeArgs a) {
  constexpr int kShare = DPW >= kTiledWaves ? 1 : kTiledWaves / DPW;  // waves per column block
  constexpr int kDW = DPW >= kTiledWaves ? DPW / kTiledWaves : 1;     // column blocks per wave
  __shared__ int32_t s_slot[kChunk];
  __shared__ float s_lse[kChunk][16];  // log-sum-exps, then weights
  __shared__ float s_red[kTiledThreads];
  __shared__ float s_m[16], s_z[16];
  __shared__ float4 s_acc[kTiledWaves][64];
  const int b = blockIdx.x, w = blockIdx.y;
  const int tid = threadIdx.x;
  const int row_blocks = (a.R + 15) / 16;
  const int kdb = a.dc / 16;
  const int wave = tid >> 6, lane = tid & 63, g = lane >> 4, li = lane & 15;
  const int d0 = DPW * blockIdx.z + (wave / kShare) * kDW;  // this wave's first column block
  const int share = wave % kShare;                         // ... and its share of the parts

  int64_t g0 = 0, n = 0;
  int64_t N = 0, G = a.workers;
  if (a.num_splits > 0) {
    n = a.num_splits;
  } else {
    const int64_t te = a.tile_start[b + 1];
    const int64_t ts = a.tile_start[b] + plan_lead(a.tile_start[b], te, a.tile_start[a.B + 1]);  // first real tile
    N = a.tile_start[a.B];
    if (ts < te) {
      g0 = worker_of_tile(ts, N, G);
      n = worker_of_tile(te - 1, N, G) - g0 + 1;
    }
  }
  // Slots and log-sum-exps of parts [c0, c0 + kChunk) into LDS; `between`
  // runs once the slots are known, before the log-sum-exps are read.
  auto load_chunk = [&](int64_t c0, auto&& between) {
    __syncthreads();  // previous chunk's readers are done
    for (int t = tid; t < kChunk; t += kTiledThreads) {
      const int64_t i = c0 + t;
      int32_t slot = -1;
      if (i < n) {
        if (a.num_splits > 0) {
          slot = (int32_t)((int64_t)b * a.num_splits + i);
        } else {
          const int64_t gg = g0 + i;
          if (tiles_begin(gg, N, G) < tiles_begin(gg + 1, N, G)) slot = (int32_t)(gg + b);
        }
      }
      s_slot[t] = slot;
    }
    __syncthreads();
    between();
    for (int k = tid; k < kChunk * 16; k += kTiledThreads) {
      const int i = k >> 4, r = k & 15, rg = 16 * w + r;
      const int32_t sl = s_slot[i];
      s_lse[i][r] = sl >= 0 && rg < a.R ? a.part_lse[(int64_t)sl * a.R + rg] : -INFINITY;
    }
    __syncthreads();
  };

  const int64_t slot_stride = (int64_t)row_blocks * kdb * 256;
  const bool lane_rows = 16 * w + 4 * g < a.R;  // lanes holding only padding rows load nothing
  auto part_ptr = [&](int d) { return a.part_o + ((int64_t)w * kdb + d) * 256 + lane * 4; };
  // Parts of a chunk handled by this wave: share, share + kShare, ...,
  // loaded kBatch at a time.
  // kBatch partial loads per lane in flight: 8 keeps the kernel under 128
  // VGPRs, so four of its 4-wave workgroups fit on a CU and a grid of about
  // 1024 workgroups runs in one round (16 needed about 190 VGPRs, two
  // workgroups per CU and two rounds).
  constexpr int kPer = kChunk / kShare;
  constexpr int kBatch = 8 < kPer ? 8 : kPer;  // divides kPer
  float4 p[kBatch];
  auto load_parts = [&](int64_t c0, int j0, int d) {
    const float* po = part_ptr(d);
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int i = share + kShare * (j0 + j);
      const int32_t sl = c0 + i < n && lane_rows ? s_slot[i] : -1;
      p[j] = sl >= 0 ? *reinterpret_cast<const float4*>(po + sl * slot_stride) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };

  // Pass 1: per-row maximum and sum (thread t: row t%16, parts t/16, +16, ...).
  const int rr = tid & 15;
  float m_run = -INFINITY, z_run = 0.f;
  for (int64_t c0 = 0; c0 < n; c0 += kChunk) {
    load_chunk(c0, [&] { if (c0 == 0) load_parts(0, 0, d0); });
    float pm = -INFINITY;
    for (int i = tid >> 4; i < kChunk; i += kTiledThreads / 16) pm = fmaxf(pm, s_lse[i][rr]);
    s_red[tid] = pm;
    __syncthreads();
    if (tid < 16) {
      float m = -INFINITY;
      for (int k = 0; k < kTiledThreads / 16; ++k) m = fmaxf(m, s_red[tid + 16 * k]);
      s_m[tid] = m;
    }
    __syncthreads();
    const float mc = s_m[rr];
    float pz = 0.f;
    if (mc != -INFINITY)
      for (int i = tid >> 4; i < kChunk; i += kTiledThreads / 16) {
        const float l = s_lse[i][rr];
        pz += l == -INFINITY ? 0.f : __expf(l - mc);
      }
    __syncthreads();  // s_m read above
    s_red[tid] = pz;
    __syncthreads();
    if (tid < 16) {
      float z = 0.f;
      for (int k = 0; k < kTiledThreads / 16; ++k) z += s_red[tid + 16 * k];
      const float m_new = fmaxf(m_run, mc);
      z_run = (m_run == -INFINITY ? 0.f : z_run * __expf(m_run - m_new)) + (mc == -INFINITY ? 0.f : z * __expf(mc - m_new));
      m_run = m_new;
    }
  }
  __syncthreads();
  if (tid < 16) {
    s_m[tid] = m_run;
    s_z[tid] = z_run;
    const int r = 16 * w + tid;
    if (a.lse && blockIdx.z == 0 && r < a.R) a.lse[(int64_t)b * a.R + r] = m_run == -INFINITY ? -INFINITY : m_run + logf(z_run);
  }

  // Pass 2: weights e^(lse - m) / z, zero for empty parts; zero-weight parts
  // may hold stale data and are selected away, never multiplied.
  auto to_weights = [&]() {
    __syncthreads();  // s_m, s_z and the chunk's log-sum-exps are complete
    for (int k = tid; k < kChunk * 16; k += kTiledThreads) {
      const int i = k >> 4, r = k & 15;
      const float l = s_lse[i][r];
      s_lse[i][r] = l == -INFINITY || s_m[r] == -INFINITY ? 0.f : __expf(l - s_m[r]) / s_z[r];
    }
    __syncthreads();
  };
  float4 acc[kDW];
#pragma unroll
  for (int dd = 0; dd < kDW; ++dd) acc[dd] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int64_t c0 = 0; c0 < n; c0 += kChunk) {
    if (c0 > 0 || n > kChunk) load_chunk(c0, [] {});  // pass 1 left the last chunk in LDS
    to_weights();
#pragma unroll
    for (int dd = 0; dd < kDW; ++dd) {
      for (int j0 = 0; j0 < kPer && c0 + share + kShare * j0 < n; j0 += kBatch) {
        if (c0 > 0 || j0 > 0 || dd > 0) load_parts(c0, j0, d0 + dd);
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          const int i = share + kShare * (j0 + j);
          const float* wt = s_lse[i < kChunk ? i : 0] + 4 * g;
          const bool valid = c0 + i < n;
          const float pv[4] = {p[j].x, p[j].y, p[j].z, p[j].w};
          float r[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const float wk = valid ? wt[k] : 0.f;
            r[k] = wk != 0.f ? wk * pv[k] : 0.f;
          }
          acc[dd].x += r[0]; acc[dd].y += r[1]; acc[dd].z += r[2]; acc[dd].w += r[3];
        }
      }
    }
  }
  if constexpr (kShare > 1) {
    s_acc[wave][lane] = acc[0];
    __syncthreads();
    if (share != 0) return;
#pragma unroll
    for (int k = 1; k < kShare; ++k) {
      const float4 o = s_acc[wave + k][lane];
      acc[0].x += o.x; acc[0].y += o.y; acc[0].z += o.z; acc[0].w += o.w;
    }
  }
#pragma unroll
  for (int dd = 0; dd < kDW; ++dd) {
    const float v[4] = {acc[dd].x, acc[dd].y, acc[dd].z, acc[dd].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * w + 4 * g + i;
      if (r < a.R) a.o[((int64_t)b * a.R + r) * a.dc + 16 * (d0 + dd) + li] = v[i];
    }
  }
}


// Merge for the tiled partial layout when sequences have few parts.  One
// wave per (sequence, 16-row block, kStreamCols 16-column blocks); lane l
// holds column l % 16 of rows 4(l/16) .. +3 of every part (one float4 per
// column block), so each lane merges its own four rows without any exchange:
// the parts' log-sum-exps and partial rows are read kStreamBatch parts at a
// time, all loads of a batch in flight together, and folded into a running
// maximum, sum and weighted sum (the online form of the merge above).  No
// LDS, no barriers.
constexpr int kStreamBatch = 4;
constexpr int kStreamCols = 4;
constexpr int kStreamWaves = 4;
constexpr int kStreamMaxParts = 12;  // average parts per sequence up to which it is used
constexpr int kSplitMinParts = 48;   // ... and beyond which combine_split_kernel is

__global__ __launch_bounds__(64 * kStreamWaves) void combine_stream_kernel(DecodeArgs a) {
  const int b = blockIdx.x, w = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 4, li = lane & 15;
  const int kdb = a.dc / 16;
  // A last row block with at most four rows has data in lane group 0 only;
  // there the four lane groups take four different sets of column blocks of
  // those rows, so every lane of the wave loads.
  const bool thin = a.R - 16 * w <= 4;
  const int cell = blockIdx.z * kStreamWaves + wave;
  const int d0 = (thin ? 4 * cell + g : cell) * kStreamCols;  // first column block
  const int r0 = thin ? 16 * w : 16 * w + 4 * g;              // this lane's first row
  if (d0 >= kdb || r0 >= a.R) return;                         // no barriers below
  const int nrow = min(4, a.R - r0);
  const bool lse4 = (a.R & 3) == 0;  // then nrow = 4 and every lane's four log-sum-exps are one aligned float4

  int64_t g0 = 0, n = 0;
  int64_t N = 0, G = a.workers;
  if (a.num_splits > 0) {
    n = a.num_splits;
  } else {
    const int64_t te = a.tile_start[b + 1];
    const int64_t ts = a.tile_start[b] + plan_lead(a.tile_start[b], te, a.tile_start[a.B + 1]);  // first real tile
    N = a.tile_start[a.B];
    if (ts < te) {
      g0 = worker_of(ts, N, G);
      n = worker_of(te - 1, N, G) - g0 + 1;
    }
  }
  const int row_blocks = (a.R + 15) / 16;
  const int64_t slot_stride = (int64_t)row_blocks * kdb * 256;
  const float* po = a.part_o + ((int64_t)w * kdb + d0) * 256 + (thin ? li : lane) * 4;

  float m[4], z[4], acc[kStreamCols][4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    m[k] = -INFINITY;
    z[k] = 0.f;
#pragma unroll
    for (int c = 0; c < kStreamCols; ++c) acc[c][k] = 0.f;
  }
  for (int64_t i0 = 0; i0 < n; i0 += kStreamBatch) {
    float4 p[kStreamBatch][kStreamCols];
    float l[kStreamBatch][4];
#pragma unroll
    for (int j = 0; j < kStreamBatch; ++j) {
      const int64_t i = i0 + j;
      int64_t slot = -1;
      if (i < n) {
        if (a.num_splits > 0) {
          slot = (int64_t)b * a.num_splits + i;
        } else {
          const int64_t gg = g0 + i;
          if (tiles_begin(gg, N, G) < tiles_begin(gg + 1, N, G)) slot = gg + b;  // workers without tiles wrote nothing
        }
      }
#pragma unroll
      for (int c = 0; c < kStreamCols; ++c)
        p[j][c] = slot >= 0 && d0 + c < kdb ? *reinterpret_cast<const float4*>(po + slot * slot_stride + 256 * c)
                                            : make_float4(0.f, 0.f, 0.f, 0.f);
      if (lse4) {  // four rows of a part, 16-byte aligned
        const float4 v = slot >= 0 ? *reinterpret_cast<const float4*>(a.part_lse + slot * a.R + r0)
                                   : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
        l[j][0] = v.x, l[j][1] = v.y, l[j][2] = v.z, l[j][3] = v.w;
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) l[j][k] = slot >= 0 && k < nrow ? a.part_lse[slot * a.R + r0 + k] : -INFINITY;
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float mb = m[k];
#pragma unroll
      for (int j = 0; j < kStreamBatch; ++j) mb = fmaxf(mb, l[j][k]);
      if (mb == -INFINITY) continue;  // nothing visible so far in this row
      const float f = m[k] == -INFINITY ? 0.f : __expf(m[k] - mb);
      z[k] *= f;
#pragma unroll
      for (int c = 0; c < kStreamCols; ++c) acc[c][k] *= f;
#pragma unroll
      for (int j = 0; j < kStreamBatch; ++j) {
        const float wj = l[j][k] == -INFINITY ? 0.f : __expf(l[j][k] - mb);
        z[k] += wj;
#pragma unroll
        for (int c = 0; c < kStreamCols; ++c) {
          const float pv[4] = {p[j][c].x, p[j][c].y, p[j][c].z, p[j][c].w};
          acc[c][k] += wj != 0.f ? wj * pv[k] : 0.f;  // zero-weight parts may hold stale data: never multiplied
        }
      }
      m[k] = mb;
    }
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (k >= nrow) break;
    const int64_t out_row = (int64_t)b * a.R + r0 + k;
    const float inv = z[k] > 0.f ? 1.f / z[k] : 0.f;
#pragma unroll
    for (int c = 0; c < kStreamCols; ++c)
      if (d0 + c < kdb) a.o[out_row * a.dc + 16 * (d0 + c) + li] = acc[c][k] * inv;
    if (a.lse && d0 == 0 && li == 0) a.lse[out_row] = z[k] > 0.f ? m[k] + logf(z[k]) : -INFINITY;
  }
}

// Merge for the tiled partial layout when sequences have many parts: one
// workgroup of SPLIT waves per (sequence, 16-row block, 16-column block).
// Wave k folds parts k, k + SPLIT, ... (BATCH at a time, loads in
// flight together) into per-lane running maxima, sums and weighted sums as
// the streaming merge does; the SPLIT states are then merged through LDS.
template <int SPLIT, int BATCH>
__global__ __launch_bounds__(64 * SPLIT) void combine_split_kernel(DecodeArgs a) {
  __shared__ float4 s_state[3][SPLIT][64];  // per wave and lane: maxima, sums, weighted sums of 4 rows
  const int b = blockIdx.x, w = blockIdx.y, d = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 4, li = lane & 15;
  const int kdb = a.dc / 16;
  const int r0 = 16 * w + 4 * g;  // this lane's first row
  const bool active = r0 < a.R;
  const int nrow = active ? min(4, a.R - r0) : 0;

  int64_t g0 = 0, n = 0;
  int64_t N = 0, G = a.workers;
  if (a.num_splits > 0) {
    n = a.num_splits;
  } else {
    const int64_t te = a.tile_start[b + 1];
    const int64_t ts = a.tile_start[b] + plan_lead(a.tile_start[b], te, a.tile_start[a.B + 1]);  // first real tile
    N = a.tile_start[a.B];
    if (ts < te) {
      g0 = worker_of(ts, N, G);
      n = worker_of(te - 1, N, G) - g0 + 1;
    }
  }
  const int row_blocks = (a.R + 15) / 16;
  const int64_t slot_stride = (int64_t)row_blocks * kdb * 256;
  const float* po = a.part_o + ((int64_t)w * kdb + d) * 256 + lane * 4;

  float m[4], z[4], acc[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) m[k] = -INFINITY, z[k] = 0.f, acc[k] = 0.f;
  const bool lse4 = (a.R & 3) == 0;  // then nrow = 4 and every lane's four log-sum-exps are one aligned float4
  if (active) {
    for (int64_t i0 = wave; i0 < n; i0 += (int64_t)SPLIT * BATCH) {
      float4 p[BATCH];
      float l[BATCH][4];
#pragma unroll
      for (int j = 0; j < BATCH; ++j) {
        const int64_t i = i0 + (int64_t)SPLIT * j;
        int64_t slot = -1;
        if (i < n) {
          if (a.num_splits > 0) {
            slot = (int64_t)b * a.num_splits + i;
          } else {
            // every worker has tiles when there are at least as many tiles as workers
            const int64_t gg = g0 + i;
            if (N >= G || tiles_begin(gg, N, G) < tiles_begin(gg + 1, N, G)) slot = gg + b;
          }
        }
        p[j] = slot >= 0 ? *reinterpret_cast<const float4*>(po + slot * slot_stride) : make_float4(0.f, 0.f, 0.f, 0.f);
        if (lse4) {
          const float4 v = slot >= 0 ? *reinterpret_cast<const float4*>(a.part_lse + slot * a.R + r0)
                                     : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
          l[j][0] = v.x, l[j][1] = v.y, l[j][2] = v.z, l[j][3] = v.w;
        } else {
#pragma unroll
          for (int k = 0; k < 4; ++k) l[j][k] = slot >= 0 && k < nrow ? a.part_lse[slot * a.R + r0 + k] : -INFINITY;
        }
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float mb = m[k];
#pragma unroll
        for (int j = 0; j < BATCH; ++j) mb = fmaxf(mb, l[j][k]);
        if (mb == -INFINITY) continue;
        const float f = m[k] == -INFINITY ? 0.f : __expf(m[k] - mb);
        z[k] *= f;
        acc[k] *= f;
#pragma unroll
        for (int j = 0; j < BATCH; ++j) {
          const float pv[4] = {p[j].x, p[j].y, p[j].z, p[j].w};
          const float wj = l[j][k] == -INFINITY ? 0.f : __expf(l[j][k] - mb);
          z[k] += wj;
          acc[k] += wj != 0.f ? wj * pv[k] : 0.f;  // zero-weight parts may hold stale data: never multiplied
        }
        m[k] = mb;
      }
    }
  }
  s_state[0][wave][lane] = make_float4(m[0], m[1], m[2], m[3]);
  s_state[1][wave][lane] = make_float4(z[0], z[1], z[2], z[3]);
  s_state[2][wave][lane] = make_float4(acc[0], acc[1], acc[2], acc[3]);
  __syncthreads();
  if (wave != 0 || !active) return;
  float M[4], Z[4], A[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) M[k] = -INFINITY, Z[k] = 0.f, A[k] = 0.f;
#pragma unroll
  for (int v = 0; v < SPLIT; ++v) {
    const float4 mv = s_state[0][v][lane];
    M[0] = fmaxf(M[0], mv.x), M[1] = fmaxf(M[1], mv.y), M[2] = fmaxf(M[2], mv.z), M[3] = fmaxf(M[3], mv.w);
  }
#pragma unroll 4
  for (int v = 0; v < SPLIT; ++v) {  // (4 at a time: 16 states in registers at once would spill)
    const float4 mv = s_state[0][v][lane], zv = s_state[1][v][lane], av = s_state[2][v][lane];
    const float mm[4] = {mv.x, mv.y, mv.z, mv.w}, zz[4] = {zv.x, zv.y, zv.z, zv.w}, aa[4] = {av.x, av.y, av.z, av.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float f = mm[k] == -INFINITY ? 0.f : __expf(mm[k] - M[k]);
      Z[k] += f * zz[k];
      A[k] += f * aa[k];
    }
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (k >= nrow) break;
    const int64_t out_row = (int64_t)b * a.R + r0 + k;
    a.o[out_row * a.dc + 16 * d + li] = Z[k] > 0.f ? A[k] / Z[k] : 0.f;
    if (a.lse && d == 0 && li == 0) a.lse[out_row] = Z[k] > 0.f ? M[k] + logf(Z[k]) : -INFINITY;
  }
}
}  // namespace

hipError_t launch_plan(const DecodeArgs& a, hipStream_t s) {
  plan_kernel<<<1, kPlanThreads, 0, s>>>(a.seq_lens, a.B, a.workers, a.tile_start);
  return hipGetLastError();
}

hipError_t launch_combine(const DecodeArgs& a, hipStream_t s) {
  if ((int64_t)a.B * a.R == 0) return hipSuccess;
  if (a.part_tiled) {
    const int kdb = a.dc / 16;
    const int64_t cells = (int64_t)a.B * ((a.R + 15) / 16) * kdb;
    const int64_t parts = a.num_splits > 0 ? a.num_splits : (a.workers + a.B - 1) / a.B + 1;
    // Few parts per sequence (on average): the streaming merge, one wave per
    // 16 x 16 output cell.
    if (parts <= kStreamMaxParts) {
      const int per_block = kStreamWaves * kStreamCols;
      const dim3 grid((unsigned)a.B, (unsigned)((a.R + 15) / 16), (unsigned)((kdb + per_block - 1) / per_block));
      combine_stream_kernel<<<grid, 64 * kStreamWaves, 0, s>>>(a);
      return hipGetLastError();
    }
    // Many parts (long sequences over few workers each): the parts of each
    // 16 x 16 output cell split over the 16 waves of a workgroup.
    // Four parts per wave at a time: larger batches spill at the 128
    // registers a 16-wave workgroup leaves each wave (129 parts: 8 per wave
    // 14.3-17.2 us, 12 per wave 28.4-31 us, 4 per wave 13.2-16.3 us).
    if (parts > kSplitMinParts) {
      const dim3 grid((unsigned)a.B, (unsigned)((a.R + 15) / 16), (unsigned)kdb);
      combine_split_kernel<16, 4><<<grid, 64 * 16, 0, s>>>(a);
      return hipGetLastError();
    }
    // Otherwise about 1024 workgroups: DPW column blocks per workgroup, a
    // power of two dividing dc/16; many parts per sequence favour DPW < 4
    // (waves share a column block and split its parts).
    int dpw = 1;
    while (dpw < 16 && cells / (2 * dpw) >= 1024 && kdb % (2 * dpw) == 0) dpw *= 2;
    if (parts > 32 && dpw > 1) dpw = 1;
    const dim3 grid((unsigned)a.B, (unsigned)((a.R + 15) / 16), (unsigned)(kdb / dpw));
    switch (dpw) {
      case 1: combine_tiled_kernel<1><<<grid, kTiledThreads, 0, s>>>(a); break;
      case 2: combine_tiled_kernel<2><<<grid, kTiledThreads, 0, s>>>(a); break;
      case 4: combine_tiled_kernel<4><<<grid, kTiledThreads, 0, s>>>(a); break;
      case 8: combine_tiled_kernel<8><<<grid, kTiledThreads, 0, s>>>(a); break;
      default: combine_tiled_kernel<16><<<grid, kTiledThreads, 0, s>>>(a); break;
    }
  } else {
    combine_kernel<<<dim3((unsigned)((int64_t)a.B * a.R)), kCombineThreads, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace mla
