// The log-sum-exp merge done inside the attention kernel (balanced plan).
//
// Every workgroup that writes a partial of a sequence with several parts
// counts its arrival on that sequence's counter once it has finished all of
// its work; the workgroup whose arrival completes the count merges the
// sequence's partials into o and lse (o = sum_s exp(lse_s - lse) o_s,
// lse = log sum_s exp(lse_s), as the merge kernels compute it) and resets
// the counter.  Nothing waits for another workgroup,
// so the scheme cannot stall whatever order workgroups run in.
//
// Visibility across XCDs (each has its own L2): every wave of an arriving
// workgroup makes its stores visible at agent scope (release fence) before
// the workgroup's arrival is counted, and every wave of the merging
// workgroup acquires at agent scope before it reads the partials.
//
// The counter is word 1 of the sequence's 16-byte record in the workspace's
// counter region; it is zero on entry and left zero on exit.
#pragma once

#include "decode_common.h"
#include "schedule.h"

namespace mla {
namespace mfma {

// Workers g0..g1 own real tiles of sequence b; n of them (those whose range
// is not empty) wrote a partial, to slot g + b.
struct PartRange {
  int g0, g1, n;
};

__device__ __forceinline__ PartRange part_range(const int32_t* ts, int B, int G, int b) {
  const int64_t te = ts[b + 1];
  const int64_t t0 = ts[b] + plan_lead(ts[b], te, ts[B + 1]);  // first real tile
  const int64_t N = ts[B];
  PartRange r{0, -1, 0};
  if (t0 >= te) return r;
  r.g0 = (int)worker_of_tile(t0, N, G);
  r.g1 = (int)worker_of_tile(te - 1, N, G);
  // With fewer positions than workers every non-empty range holds exactly
  // one position, so the count is the number of positions g0..g1 cover.
  r.n = N >= G ? r.g1 - r.g0 + 1 : (int)(worker_tile_begin(r.g1 + 1, N, G) - worker_tile_begin(r.g0, N, G));
  return r;
}

__device__ __forceinline__ uint32_t* arrival_counter(const DecodeArgs& a, int b) { return a.ctr + 4 + 4 * b + 1; }

// The four log-sum-exps of rows r0..r0+3 of one part (-inf past R).
__device__ __forceinline__ void load_lse4(const DecodeArgs& a, int64_t slot, int r0, float (&l)[4]) {
  const float* p = a.part_lse + slot * a.R + r0;
  if ((a.R & 3) == 0) {  // r0 is a multiple of 4: the four rows are all in or all out
    const float4 v = r0 < a.R ? *reinterpret_cast<const float4*>(p) : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
    l[0] = v.x, l[1] = v.y, l[2] = v.z, l[3] = v.w;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) l[i] = r0 + i < a.R ? p[i] : -INFINITY;
  }
}

// Merges the partials of sequence b (tiled layout, normalised, natural-log
// lse) into o[b] and lse[b].  Every wave of the workgroup calls it; nw waves.
// Jobs are (row block, group of kMergeCols column blocks); wave w takes the
// row block w % RB and every (nw / RB)-th column group from w / RB.
template <int KDB>
__device__ __forceinline__ void merge_sequence(const DecodeArgs& a, const int32_t* ts, int b, int nw, int wave,
                                               int lane) {
  constexpr int kCols = 8;   // column blocks per pass
  constexpr int kBatch = 4;  // parts per batch of loads
  static_assert(KDB % kCols == 0, "column groups");
  const int g = lane >> 4, li = lane & 15;
  const int RB = (a.R + 15) / 16;
  const int cs = nw / RB;  // waves per row block (the kernel has at least RB waves)
  if (wave >= RB * cs) return;
  const int rb = wave % RB;
  const int r0 = 16 * rb + 4 * g;  // this lane's first row
  const PartRange pr = part_range(ts, a.B, a.workers, b);
  const int64_t N = ts[a.B], G = a.workers;
  auto has_part = [&](int gg) { return N >= G || worker_tile_begin(gg, N, G) < worker_tile_begin(gg + 1, N, G); };

  // Row maxima and sums of exp(lse - max), online over the parts.
  float M[4], Z[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) M[i] = -INFINITY, Z[i] = 0.f;
  for (int g0 = pr.g0; g0 <= pr.g1; g0 += kBatch) {
    float l[kBatch][4];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int gg = g0 + j;
      if (gg <= pr.g1 && has_part(gg)) load_lse4(a, (int64_t)gg + b, r0, l[j]);
      else l[j][0] = l[j][1] = l[j][2] = l[j][3] = -INFINITY;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float mb = M[i];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) mb = fmaxf(mb, l[j][i]);
      if (mb == -INFINITY) continue;
      float z = M[i] == -INFINITY ? 0.f : Z[i] * __expf(M[i] - mb);
#pragma unroll
      for (int j = 0; j < kBatch; ++j) z += l[j][i] == -INFINITY ? 0.f : __expf(l[j][i] - mb);
      M[i] = mb, Z[i] = z;
    }
  }
  float invZ[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) invZ[i] = Z[i] > 0.f ? 1.f / Z[i] : 0.f;
  if (a.lse && wave < RB && li == 0)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (r0 + i < a.R) a.lse[(int64_t)b * a.R + r0 + i] = Z[i] > 0.f ? M[i] + logf(Z[i]) : -INFINITY;

  const int64_t slot_stride = (int64_t)RB * KDB * 256;
  for (int cg = wave / RB; cg < KDB / kCols; cg += cs) {
    const int d0 = cg * kCols;
    float4 acc[kCols];
#pragma unroll
    for (int c = 0; c < kCols; ++c) acc[c] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int g0 = pr.g0; g0 <= pr.g1; g0 += kBatch) {
      float l[kBatch][4];
      float4 p[kBatch][kCols];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int gg = g0 + j;
        const bool ok = gg <= pr.g1 && has_part(gg);
        const float* src = a.part_o + (((int64_t)gg + b) * slot_stride + ((int64_t)rb * KDB + d0) * 256 + lane * 4);
        if (ok) load_lse4(a, (int64_t)gg + b, r0, l[j]);
        else l[j][0] = l[j][1] = l[j][2] = l[j][3] = -INFINITY;
#pragma unroll
        for (int c = 0; c < kCols; ++c)
          p[j][c] = ok ? *reinterpret_cast<const float4*>(src + 256 * c) : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        float w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = l[j][i] == -INFINITY ? 0.f : __expf(l[j][i] - M[i]) * invZ[i];
        // Zero-weight parts (no visible token in these rows) may hold any
        // bytes: they are selected away, never multiplied.
#pragma unroll
        for (int c = 0; c < kCols; ++c) {
          acc[c].x += w[0] != 0.f ? w[0] * p[j][c].x : 0.f;
          acc[c].y += w[1] != 0.f ? w[1] * p[j][c].y : 0.f;
          acc[c].z += w[2] != 0.f ? w[2] * p[j][c].z : 0.f;
          acc[c].w += w[3] != 0.f ? w[3] * p[j][c].w : 0.f;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (r0 + i >= a.R) break;
      float* dst = a.o + ((int64_t)b * a.R + r0 + i) * a.dc + 16 * d0 + li;
#pragma unroll
      for (int c = 0; c < kCols; ++c) dst[16 * c] = i == 0 ? acc[c].x : i == 1 ? acc[c].y : i == 2 ? acc[c].z : acc[c].w;
    }
  }
}

// Zero result (o = 0, lse = -inf) for sequences with no tokens: they have no
// parts, so no workgroup would otherwise write them.  Workgroup x of `grid`
// takes sequences x, x + grid, ...; lens are the clamped lengths.
__device__ __forceinline__ void zero_empty_sequences(const DecodeArgs& a, const int32_t* lens, int grid) {
  for (int b = blockIdx.x; b < a.B; b += grid) {
    if (lens[b] > 0) continue;
    const int64_t n = (int64_t)a.R * a.dc;
    float* o = a.o + (int64_t)b * n;
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x) o[i] = 0.f;
    if (a.lse)
      for (int r = threadIdx.x; r < a.R; r += blockDim.x) a.lse[(int64_t)b * a.R + r] = -INFINITY;
  }
}

}  // namespace mfma
}  // namespace mla
