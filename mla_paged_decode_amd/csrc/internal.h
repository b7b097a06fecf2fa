// Internal launch interface between the C-ABI host layer (api.cpp) and the
// HIP kernels.  Everything here is validated by the host layer first.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace mla {

// Tokens per planning tile: balanced split-KV cuts every sequence into tiles
// of this many tokens and hands each worker a contiguous run of tiles.
constexpr int kPlanTile = 32;
// Virtual tiles charged to a worker for each sequence it starts (balanced
// mode): about what loading that sequence's queries and restarting the tile
// stream cost, measured in tile times on MI355X.
constexpr int kUnitCostTiles = 4;
// Worker count of balanced mode: two workgroups per compute unit on a
// 256-CU MI355X, which fills the chip in one pass.
constexpr int kBalancedWorkers = 512;
// LDS ring depth (tile buffers) of the bf16 matrix-core decode kernel and the
// balanced worker count it runs with (at most kBalancedWorkers).
constexpr int kRingBf16 = 2;
constexpr int kMfmaWorkersBf16 = 512;
// Balanced worker count of the fp8 / fp4 kernels for R query rows: one
// workgroup per CU, two for fp4 rows with at most two row blocks.
int fp8_rows_workers(int fmt, int R);
// Batches up to this size are planned inside the matrix-core decode kernel
// (each workgroup scans seq_lens itself); larger ones use the plan kernel.
constexpr int kMaxInKernelPlan = 512;

enum KvFormat : int { kF32 = 0, kBF16 = 1, kFP8 = 2, kFP4 = 3 };

struct DecodeArgs {
  int B, Sq, H, R;        // R = Sq * H query rows per sequence
  int dc, dr;             // latent and RoPE widths
  const void* q_abs;      // [B][R][dc + dr]
  int q_f32;              // 1: fp32 queries, 0: bf16
  const uint8_t* pool;    // [pages][P][row_bytes]
  int64_t row_bytes;
  int P;
  int P_log2;             // page_block = 1 << P_log2
  const int32_t* block_table;
  int max_blocks;
  const int32_t* seq_lens;
  float scale_log2;       // softmax_scale * log2(e): scores kept in base 2
  int num_splits;         // >= 1 uniform, 0 balanced
  int workers;            // balanced: worker count G
  float* part_o;          // part_tiled ? see below : [slots][R][dc]
  int part_tiled;         // 1: matrix-core layout [slots][ceil(R/16)][dc/16][64 lanes][4]:
                          //    row 16w + 4(l/16) + i, column 16d + l%16 at [slot][w][d][l][i]
  float* part_lse;        // [slots][R], natural log
  int32_t* tile_start;    // balanced: [B + 2] plan (schedule.h)
  int plan_in_kernel;     // balanced: the decode kernel computes tile_start
  float* o;               // [B][R][dc]
  float* lse;             // [B][R] or null
  // Sparse top-k mode (vector-ALU kernel, uniform splits): B counts
  // (sequence, query token) pairs, R = H, and pair b attends to the cached
  // tokens listed in topk[b][0 .. topk_width) of sequence b / sparse_sq
  // (query token b % sparse_sq).  sparse_sq = 0: dense.
  const int32_t* topk;
  int topk_width;
  int sparse_sq;
  // Dynamically scheduled mode (decode_dyn.hip) and the fused merge: the
  // counter region at the start of the workspace (zero between calls).
  uint32_t* ctr;
  // 1: the bf16 matrix-core kernel merges the partials itself (merge_fused.h)
  // and no merge kernel runs.
  int fuse_merge;
};

// Dynamically scheduled bf16 decode (decode_dyn.hip).  Workers take tiles
// of a sequence in claims of kDynClaimTiles from a per-sequence counter; a
// sequence accepts kDynStealParts visits beyond the workers the balanced plan
// assigns to it.  Batches up to kDynMaxB sequences.
constexpr int kDynClaimTiles = 4;
constexpr int kDynStealParts = 2;
constexpr int kDynMaxB = kMaxInKernelPlan;
// Every decode workspace starts with this counter region (a 16-byte header
// holding the exit counter, then 16 bytes per sequence).  Only the
// dynamically scheduled kernel uses it; it must be zero before a workspace's
// first use, and every call of that kernel leaves it zero again (the last
// workgroup to finish resets it), so no clearing is needed between calls.
constexpr size_t kDynCounterBytes = 256 + 16 * (size_t)kDynMaxB;
bool decode_dyn_supported(int fmt, int dc, int dr, int R, int q_f32, int num_splits, int B);
// Attention and merge: the decode kernel, then the merge kernel.
hipError_t launch_decode_dyn(const DecodeArgs& a, hipStream_t s);
hipError_t launch_combine_dyn(const DecodeArgs& a, hipStream_t s);

// Workspace layout shared by the size query and the launch.
struct WorkspaceLayout {
  size_t ctr_off, tile_start_off, part_lse_off, part_o_off, total;
  int64_t slots;
};
// Partial rows are padded to a multiple of 16 (the tiled layout's row blocks).
// dyn: the dynamically scheduled kernel's slot count (workers + B * (1 +
// kDynStealParts)) instead of the static modes'.
WorkspaceLayout workspace_layout(int B, int R, int dc, int num_splits, bool dyn = false);

hipError_t launch_plan(const DecodeArgs& a, hipStream_t s);
hipError_t launch_decode_simt(const DecodeArgs& a, int fmt, hipStream_t s);
hipError_t launch_decode_mfma(const DecodeArgs& a, int fmt, hipStream_t s);
bool decode_mfma_supported(int fmt, int dc, int dr, int R, int q_f32);
// Whether the bf16 matrix-core kernel merges in-kernel for this call shape
// (balanced mode, plan in the kernel, one workgroup shape, few parts).
bool decode_fused_merge_supported(int fmt, int dc, int dr, int R, int num_splits, int B, int workers);
// fp8 or fp4 cache with bf16 queries: one 16-row block per wave
// (decode_fp8.hip); launch_decode_mfma dispatches to it when it applies.
bool decode_fp8_rows_supported(int fmt, int dc, int dr, int R, int q_f32);
hipError_t launch_decode_fp8_rows(const DecodeArgs& a, int fmt, hipStream_t s);
// The same kernel in sparse top-k mode: uniform splits, index lists a
// multiple of 32 wide.
bool decode_fp8_rows_sparse_supported(int fmt, int dc, int dr, int R, int q_f32, int topk_width);
hipError_t launch_decode_fp8_rows_sparse(const DecodeArgs& a, int fmt, hipStream_t s);
hipError_t launch_combine(const DecodeArgs& a, hipStream_t s);
// Sparse top-k mode on the matrix cores: bf16 cache, R <= 64, uniform splits,
// index lists a multiple of 32 wide (tiles never pass the end of a list).
bool decode_mfma_sparse_supported(int fmt, int dc, int dr, int R, int topk_width);
hipError_t launch_decode_mfma_sparse(const DecodeArgs& a, hipStream_t s);

struct ProjArgs {
  int N, H, dn, dr, dv, dc;
  const void* in;  // absorb: q [N][H][dn+dr]; out_proj: o [N][H][dc] (f32)
  int in_f32;
  const void* w;   // [H][dn+dv][dc]
  int w_f32;
  void* out;       // absorb: q_abs [N][H][dc+dr]; out_proj: [N][H][dv] (f32)
  int out_f32;
  int tok_blocks;  // matrix-core kernels: 16-token blocks per workgroup (set at launch)
  int tok_groups;  // matrix-core kernels: workgroups per (head, column group) (set at launch)
};
// Dispatchers: matrix-core kernels where the dtypes and shapes allow,
// vector-ALU kernels otherwise.
hipError_t launch_absorb_q(const ProjArgs& a, hipStream_t s);
hipError_t launch_out_proj(const ProjArgs& a, hipStream_t s);
bool absorb_mfma_supported(const ProjArgs& a);
bool out_proj_mfma_supported(const ProjArgs& a);
hipError_t launch_absorb_mfma(const ProjArgs& a, hipStream_t s);
hipError_t launch_out_proj_mfma(const ProjArgs& a, hipStream_t s);

struct CacheWriteArgs {
  int64_t n_rows;
  int n_vals;              // d_latent + d_rope values per row
  const void* rows;        // [n_rows][n_vals], f32 or bf16
  int rows_f32;
  const int64_t* slots;    // [n_rows] physical token slot (page * P + offset), < 0 skips
  int64_t n_slots;         // num_pages * P; slots at or beyond it are skipped too
  uint8_t* pool;           // [n_slots][row_bytes]
  int64_t row_bytes;
  int fmt;                 // KvFormat
};
hipError_t launch_cache_write(const CacheWriteArgs& a, hipStream_t s);

// Unabsorbed prefill (prefill_simt.hip).
struct PrefillArgs {
  int B, Sq, H, dn, dr, dv, dc;
  int P, max_blocks;
  int64_t Lcap;               // token capacity per sequence: max_blocks * P
  const void* q;              // [B*Sq][H][dn + dr]
  int q_f32;
  const void* w;              // [H][dn + dv][dc]
  int w_f32;
  const uint8_t* pool;
  int64_t row_bytes;
  const int32_t* block_table;
  const int32_t* seq_lens;
  float scale_log2;
  float* kn;                  // workspace: [B][Lcap][H][dn]
  float* kr;                  // workspace: [B][Lcap][dr]
  float* v;                   // workspace: [B][Lcap][H][dv]
  float* out;                 // [B*Sq][H][dv]
  float* lse;                 // [B*Sq][H] or null
  int splits;                 // matrix-core attention: key ranges per query block (1: none)
  float* part_o;              // workspace, splits > 1: [B*Sq][H][splits][dv], normalised
  float* part_lse;            // workspace, splits > 1: [B*Sq][H][splits]
};
bool prefill_supported(int dc, int dr, int dn, int dv);
hipError_t launch_prefill(const PrefillArgs& a, int fmt, hipStream_t s);
// The K/V rebuild on the matrix cores (prefill_mfma.hip): bf16 weights.
bool prefill_expand_mfma_supported(const PrefillArgs& a);
hipError_t launch_prefill_expand_mfma(const PrefillArgs& a, int fmt, hipStream_t s);
// The causal attention on the matrix cores: keys and values 256 wide.
bool prefill_attn_mfma_supported(const PrefillArgs& a);
// Key ranges per query block of the matrix-core attention (host only; 1 if
// that kernel does not apply): enough workgroups to fill the chip.
int prefill_attn_splits(int B, int Sq, int H, int64_t Lcap, int dn, int dr, int dv);
hipError_t launch_prefill_attn_mfma(const PrefillArgs& a, hipStream_t s);

}  // namespace mla
