/*
 * libmla: multi-head latent attention (MLA) decode over a paged latent KV
 * cache, for AMD Instinct MI355X (gfx950).
 *
 * The method.  GLM-4.7-Flash uses DeepSeek-V2 style MLA with the weights
 * kv_a_proj_with_mqa and kv_b_proj (model record "GLM-4.7-Flash", config
 * facts; vLLM pull request "fix: Add glm4_moe_lite to MLA detection",
 * Summary).  Its cache holds, per token and layer, one shared low-rank latent
 * c_t (kv_lora_rank = 512 values) followed by a decoupled RoPE key k^R_t (64
 * values): 576 values, 1,152 bytes in bf16 (model record, "SERVICEABILITY
 * JOIN" and the kv_cache_bytes_per_token formula).  An fp8 variant stores 512
 * e4m3 values, RoPE dims included, plus one e8m0 scale byte per 32 values,
 * 528 bytes per token (model record, ENGINE KERNEL CONSTRAINTS item (2));
 * with 64 RoPE dims that leaves a 448-wide latent.  Decode kernels are built
 * per page-block size (same list, item (1)); this library takes the page
 * block as an argument.
 *
 * kv_b_proj is stored per head as [d_nope + d_v][d_latent]: rows 0..d_nope-1
 * are W_UK^h (key half), rows d_nope..d_nope+d_v-1 are W_UV^h (value half).
 * The query head is d_nope + d_rope = 192 + 64 and the value head d_v = 256
 * (model record, "head_dim FILLED = 256").
 *
 * A decode step is three calls, in the absorbed form:
 *   mla_absorb_q      q_abs^h = [ (W_UK^h)^T q^{N,h} , q^{R,h} ]
 *   mla_decode_paged  o_lat^h = sum_t softmax_t(scale <q_abs^h,[c_t,k^R_t]>) c_t
 *                     (split-KV over the token range + log-sum-exp merge)
 *   mla_out_proj      o^h     = W_UV^h o_lat^h
 * which equals softmax attention with K^h_t = [W_UK^h c_t, k^R_t] and
 * V^h_t = W_UV^h c_t.
 *
 * Conventions for every call:
 *  - Pointers are device pointers owned by the caller.  The library
 *    allocates nothing, frees nothing and keeps no state between calls.
 *  - Inputs are read only; outputs are overwritten in full.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Calls are
 *    asynchronous on it and never synchronise with the host.
 *  - Everything checkable on the host is checked before any launch.  A
 *    failed check returns a non-zero status and sets a thread-local message
 *    of the form "<argument>: expected <X>, got <Y>"; nothing is launched.
 *  - Values that live on the device (seq_lens, block_table) are trusted:
 *    block_table entries for logical pages [0, ceil(seq_len/page_block))
 *    must lie in [0, num_pages) and seq_lens must be in
 *    [0, max_blocks_per_seq * page_block].  Entries past a sequence's last
 *    page are never read.  mla_validate_tables checks host copies of both
 *    tables against these ranges.
 */
#ifndef LIBMLA_MLA_H
#define LIBMLA_MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_ABI_VERSION 3

typedef enum { MLA_F32 = 0, MLA_BF16 = 1 } mla_dtype_t;

/* Cache row formats.  Row = [latent (d_latent) | RoPE key (d_rope)].
 *  MLA_KV_F32            4 bytes per value   (2,304 B at 512 + 64)
 *  MLA_KV_BF16           2 bytes per value   (1,152 B at 512 + 64)
 *  MLA_KV_FP8_E4M3_E8M0  d_latent + d_rope e4m3fn bytes, then one e8m0 byte
 *                        per 32 values; value = e4m3fn * 2^(E - 127)
 *                        (528 B at 448 + 64).
 *  MLA_KV_FP4_E2M1_E4M3  (d_latent + d_rope) / 2 bytes of e2m1 codes (value
 *                        2i in the low nibble of byte i), then one e4m3fn
 *                        scale byte per 16 values; value = e2m1 * e4m3
 *                        (288 B at 448 + 64: the model record's fp4 variant;
 *                        its scale format is this library's reading).  With
 *                        bf16 q_abs it decodes on the matrix cores (the row is
 *                        expanded to bf16 in LDS, exactly); with f32 q_abs on
 *                        the fp32 vector-ALU kernel. */
typedef enum {
  MLA_KV_F32 = 0,
  MLA_KV_BF16 = 1,
  MLA_KV_FP8_E4M3_E8M0 = 2,
  MLA_KV_FP4_E2M1_E4M3 = 3
} mla_kv_format_t;

typedef enum {
  MLA_OK = 0,
  MLA_ERR_NULL_POINTER = 1,
  MLA_ERR_INVALID_SHAPE = 2,
  MLA_ERR_UNSUPPORTED = 3,
  MLA_ERR_ALIGNMENT = 4,
  MLA_ERR_WORKSPACE_TOO_SMALL = 5,
  MLA_ERR_HIP = 6
} mla_status_t;

/* Per-layer attention dimensions.  Supported: 1 <= num_heads <= 128,
 * d_rope = 64, d_nope and d_v multiples of 32 in [32, 512], d_latent = 512
 * (f32 / bf16 cache) or 448 (fp8 cache). */
typedef struct {
  int32_t num_heads;
  int32_t d_latent; /* kv_lora_rank, the shared latent width d_c */
  int32_t d_rope;   /* qk_rope_head_dim */
  int32_t d_nope;   /* qk_nope_head_dim */
  int32_t d_v;      /* v_head_dim */
} mla_dims_t;

/* Bytes of one cached row in `format`, or 0 if dims/format are invalid. */
size_t mla_kv_row_bytes(const mla_dims_t* dims, mla_kv_format_t format);

/* Fold the no-RoPE part of the query into latent space.
 *   q       [n_tokens][H][d_nope + d_rope]      q_dtype (F32 or BF16)
 *   w_kv_b  [H][d_nope + d_v][d_latent]         w_dtype (F32 or BF16)
 *   q_abs   [n_tokens][H][d_latent + d_rope]    q_abs_dtype (F32 or BF16)
 * q_abs[n][h][c] = sum_k w_kv_b[h][k][c] * q[n][h][k] for k < d_nope
 * (accumulated in fp32), and q_abs[n][h][d_latent + i] = q[n][h][d_nope + i].
 * Source of the step: the key half of kv_b_proj (model record, SERVICEABILITY
 * JOIN: kv_b_proj) applied to the query instead of to every cached token.
 * All pointers 16-byte aligned.  n_tokens = 0 is a no-op. */
mla_status_t mla_absorb_q(const mla_dims_t* dims, int32_t n_tokens,
                          const void* q, mla_dtype_t q_dtype,
                          const void* w_kv_b, mla_dtype_t w_dtype,
                          void* q_abs, mla_dtype_t q_abs_dtype, void* stream);

/* Kernel choice for mla_decode_paged. */
typedef enum {
  MLA_KERNEL_AUTO = 0, /* MFMA kernel where supported, else SIMT */
  MLA_KERNEL_SIMT = 1, /* fp32 vector-ALU kernel, every format */
  MLA_KERNEL_MFMA = 2  /* matrix-core kernel; MLA_ERR_UNSUPPORTED if not */
} mla_kernel_t;

typedef struct {
  mla_dims_t dims;
  int32_t batch;     /* B >= 0 sequences */
  int32_t q_per_seq; /* Sq in [1, 8]; the Sq new tokens are the last Sq
                        cached ones and attend causally among themselves */
  const void* q_abs; /* [B][Sq][H][d_latent + d_rope]; F32 = full precision,
                        BF16 = single-rounded queries */
  mla_dtype_t q_abs_dtype;
  const void* kv_pool; /* [num_pages][page_block][row_bytes], 16-B aligned */
  mla_kv_format_t kv_format;
  int64_t num_pages;
  int32_t page_block;           /* tokens per page: 16, 32, 64 or 128 */
  const int32_t* block_table;   /* [B][max_blocks_per_seq] physical page ids */
  int32_t max_blocks_per_seq;
  const int32_t* seq_lens;      /* [B] cached tokens per sequence, incl. Sq */
  float softmax_scale;
  int32_t num_splits;  /* >= 1: each sequence cut into num_splits equal
                          contiguous chunks; 0: balanced, chunks of whole
                          tiles spread evenly over a fixed worker count */
  mla_kernel_t kernel;
  void* workspace;     /* scratch of mla_decode_workspace_size() bytes,
                          16-B aligned.  With MLA_DECODE_DYNAMIC_SPLIT or
                          MLA_DECODE_FUSED_MERGE, zero-fill it once before
                          its first use (e.g. hipMemset at allocation): its
                          first bytes hold per-sequence counters, which
                          every call leaves zero again.  One call at a time
                          per workspace (calls that overlap on two streams
                          race). */
  size_t workspace_bytes;
  void* o_latent;      /* out: [B][Sq][H][d_latent], F32 */
  mla_dtype_t o_dtype;
  float* lse;          /* out (optional, may be NULL): [B][Sq][H], natural
                          log of the softmax denominator */
  void* kernel_start_event; /* optional hipEvent_t (NULL = none): recorded on
                               the stream right before the split-KV attention
                               kernel is launched */
  void* kernel_stop_event;  /* optional hipEvent_t (NULL = none): recorded right
                               after it, before the merge kernel (if the merge
                               runs inside the attention kernel, after both).
                               Both are caller-owned; they time the dominant
                               kernel alone. */
  uint32_t flags;           /* MLA_DECODE_* bits below; 0 by default */
} mla_decode_params_t;

/* Accept bf16 q_abs with a bf16 or f32 cache.  Without this bit such calls
 * return MLA_ERR_UNSUPPORTED: absorbed queries rounded once to bf16 (and the
 * softmax weights with them) measure up to 1.3e-2 of the output RMS on the
 * 256-sequence ragged batch, beyond the 1e-2 match criterion for bf16
 * caches; f32 q_abs (split into bf16 hi + lo products) measures ~2e-5.  The
 * fp8 and fp4 caches take bf16 q_abs without it (their criterion is 5e-2). */
#define MLA_DECODE_ALLOW_BF16_QUERIES 0x1u
/* Balanced mode (num_splits = 0) on the bf16 matrix-core kernel gives every
 * worker one fixed, contiguous share of the tiles (the static split).  This
 * bit hands each sequence's tiles out at run time instead, four at a time,
 * from per-sequence counters in the workspace, to whichever worker asks
 * next.  Both give the same result up to rounding.  (On MI355X the run-time
 * split measures slower on the benchmark workloads: the many workers of a
 * long sequence queue on its counter.) */
#define MLA_DECODE_DYNAMIC_SPLIT 0x2u
/* The caller keeps the workspace's counter region zero (zero-filled once at
 * allocation; every call leaves it zero), which lets balanced mode merge the
 * partial results inside the attention kernel instead of in a second kernel:
 * the last workgroup to finish a part of a sequence merges that sequence,
 * and a sequence held by one worker is written out directly.  Applies to the
 * bf16 matrix-core kernel with up to 32 query rows (q_per_seq * num_heads)
 * and batches with few parts per sequence (at least a fifth as many
 * sequences as workers); otherwise the bit changes nothing.  Same result up
 * to rounding.  Ignored by mla_decode_paged_noalloc.  (On MI355X it measures
 * slower than the separate merge kernel on the 256-sequence ragged batch:
 * making every partial visible across the XCDs' L2 caches before its
 * arrival is counted, and the merges left to the last workgroups, each cost
 * more than the merge kernel saves.) */
#define MLA_DECODE_FUSED_MERGE 0x4u

/* Workspace bytes mla_decode_paged needs for these parameters.  Reads only
 * host scalars (no pointers are dereferenced, no device is touched). */
mla_status_t mla_decode_workspace_size(const mla_decode_params_t* p, size_t* bytes);

/* Which kernel mla_decode_paged would run for these parameters
 * (MLA_KERNEL_SIMT or MLA_KERNEL_MFMA); host scalars only. */
mla_status_t mla_decode_select_kernel(const mla_decode_params_t* p, mla_kernel_t* chosen);

/* Paged MLA decode.  For sequence b (length L = seq_lens[b]) and query j in
 * [0, Sq), row r = j*H + h attends to cached tokens t in [0, L - Sq + j]:
 *   s_t   = softmax_scale * < q_abs[b][j][h], row_t >   (all d_latent + d_rope)
 *   o_lat = sum_t softmax(s)_t * latent_t ,  lse = log sum_t exp(s_t)
 * where token t is read from page block_table[b][t / page_block], slot
 * t % page_block.  A row with no visible token gets o_lat = 0, lse = -inf.
 * The token range is split into chunks (num_splits), each chunk's partial
 * result is written to the workspace, and a log-sum-exp merge produces the
 * outputs.  Source of the operation: model record "GLM-4.7-Flash",
 * SERVICEABILITY JOIN (the required MLA decode kernel class over the latent
 * plus RoPE-key cache) and ENGINE KERNEL CONSTRAINTS (1)-(2) (page-block
 * size and fp8 row format).  Errors: see the conventions above. */
mla_status_t mla_decode_paged(const mla_decode_params_t* p, void* stream);

/* mla_decode_paged without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  It runs the same kernels with the split
 * partials in a scratch array inside the library, MLA_NOALLOC_SCRATCH_BYTES
 * (128 MiB) per GPU, which each GPU holds from the library's first use on it
 * until the process ends.  The first call on a GPU looks the array's address
 * up (make that call outside graph capture).  p->workspace and
 * p->workspace_bytes are ignored; every other field means what it means for
 * mla_decode_paged.  Errors: MLA_ERR_WORKSPACE_TOO_SMALL when the call's
 * workspace (mla_decode_workspace_size) exceeds the scratch,
 * MLA_ERR_UNSUPPORTED with MLA_DECODE_DYNAMIC_SPLIT; otherwise as
 * mla_decode_paged.  All calls on one GPU share its scratch, which keeps the
 * last call's partials: calls in one stream are ordered, calls of one
 * process that overlap on one GPU (two streams, two threads) race.  Each
 * process has its own copy.  Allocates nothing. */
#define MLA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
mla_status_t mla_decode_paged_noalloc(const mla_decode_params_t* p, void* stream);

/* Sparse top-k decode: each query attends only to the cached tokens its
 * index list names, as the sparse MLA path of the vLLM API page for
 * vllm.models.glm5next.common.model prepares it (a per-token buffer of top-k
 * token indices, padded to whole tiles, padded slots masked).
 *   topk_indices  [batch][q_per_seq][topk_width] int32, device: logical
 *                 token positions in the sequence.  Entries < 0 or beyond the
 *                 query's causal limit (L - Sq + j, as in mla_decode_paged)
 *                 are padding and masked.  Each listed entry is one score, so
 *                 a position listed twice counts twice; lists are expected to
 *                 hold distinct positions.
 * For query j of sequence b and head h:
 *   o_lat = sum_{t listed} softmax(s)_t latent_t over the listed tokens,
 *   lse   = log sum exp(s_t); no listed token: o_lat = 0, lse = -inf.
 * Every other parameter means what it means for mla_decode_paged, except:
 * num_splits >= 1 cuts each index list into that many uniform chunks (0 is
 * rejected), and the workspace size comes from
 * mla_decode_sparse_workspace_size.  Kernel: a matrix-core one (rows
 * gathered through the index list) when topk_width is a multiple of 32 (the
 * pages pad the list to 128) and either the cache is bf16 with num_heads <=
 * 64, or it is fp8 / fp4 (448 + 64 row) with bf16 q_abs and num_heads <= 128;
 * unless MLA_KERNEL_SIMT is asked for.  On every kernel a padding slot
 * contributes exactly nothing, whatever any cache row it could point at
 * holds (NaN bytes included): its score is masked and its value operand is
 * zeroed, not multiplied by a zero weight.  The fp32
 * vector-ALU one otherwise (MLA_KERNEL_MFMA where none applies is
 * rejected).  Errors: see the conventions above. */
mla_status_t mla_decode_sparse_workspace_size(const mla_decode_params_t* p, int32_t topk_width, size_t* bytes);
mla_status_t mla_decode_sparse_paged(const mla_decode_params_t* p, const int32_t* topk_indices,
                                     int32_t topk_width, void* stream);

/* Value up-projection.
 *   o_latent [n_tokens][H][d_latent]    F32
 *   w_kv_b   [H][d_nope + d_v][d_latent] w_dtype (F32 or BF16)
 *   out      [n_tokens][H][d_v]         out_dtype (F32)
 * out[n][h][v] = sum_c w_kv_b[h][d_nope + v][c] * o_latent[n][h][c], with
 * fp32 accumulation.  Source: the value half of kv_b_proj (model record,
 * SERVICEABILITY JOIN), applied once per query instead of per token. */
mla_status_t mla_out_proj(const mla_dims_t* dims, int32_t n_tokens,
                          const void* o_latent, mla_dtype_t o_dtype,
                          const void* w_kv_b, mla_dtype_t w_dtype,
                          void* out, mla_dtype_t out_dtype, void* stream);

/* Cache append: store new tokens' rows into the paged cache.
 *   rows        [n_rows][d_latent + d_rope]  rows_dtype (F32 or BF16): the
 *               latent c_t, then the RoPE key k^R_t (already rotated)
 *   slots       [n_rows] int64, device: physical token slot of row i,
 *               page * page_block + position in the page; slots[i] < 0, or
 *               >= num_pages * page_block, leaves the cache untouched for row i
 *   kv_pool     [num_pages][page_block][row bytes of kv_format], written in
 *               place; only the rows named by slots change
 * Formats: MLA_KV_F32 stores the values; MLA_KV_BF16 rounds them to nearest,
 * ties to even; MLA_KV_FP8_E4M3_E8M0 (d_latent 448 + d_rope 64 = 512 values)
 * quantises each block of 32 values with the scale 2^(E - 127), E the
 * smallest exponent in [0, 254] with max|value| <= 448 * 2^(E - 127) (127 for
 * an all-zero block), and stores each value / scale as the nearest e4m3fn
 * value, ties to the even code, sign taken from the value (-0 -> 0x80).
 * MLA_KV_FP4_E2M1_E4M3 (448 + 64 values) quantises each block of 16 values
 * with the smallest positive e4m3fn scale s for which max|value| <= 6 s (448
 * if none; 1.0 for an all-zero block) and stores each value as the e2m1 code
 * nearest to the float32 quotient value / s, ties to the even code, clamped
 * to +-6, sign taken from the value.
 * Inputs must be finite.  Two rows with the same slot race.  Source: the
 * cache row layouts of the model record "GLM-4.7-Flash" (SERVICEABILITY
 * JOIN: latent plus RoPE key per token; ENGINE KERNEL CONSTRAINTS (2): the
 * 528-byte e4m3 row with per-token e8m0 scales).  Errors: see the
 * conventions above (pool and rows 16-byte aligned, slots 8-byte aligned). */
mla_status_t mla_cache_write(const mla_dims_t* dims, int32_t n_rows,
                             const void* rows, mla_dtype_t rows_dtype,
                             const int64_t* slots,
                             void* kv_pool, mla_kv_format_t kv_format,
                             int64_t num_pages, int32_t page_block, void* stream);

/* Unabsorbed prefill (chunked prefill): a chunk of Sq new tokens per
 * sequence, already appended as the last Sq of its L cached tokens, attends
 * causally to the whole cache with per-head keys and values rebuilt through
 * kv_b_proj (DeepSeek-V2 multi-head latent attention in its unabsorbed
 * form, as the GLM-4.7-Flash model record uses it; the pages name chunked
 * prefill for MLA beside the decode kernel).  For sequence b, query i in
 * [0, Sq) (position L - Sq + i) and head h, over tokens t <= L - Sq + i:
 *   k_t = [W_UK[h] c_t ; k^R_t],  v_t = W_UV[h] c_t   (W_UK = rows [0, d_nope)
 *                                  and W_UV = rows [d_nope, d_nope + d_v) of
 *                                  w_kv_b[h])
 *   s_t = softmax_scale * q[b][i][h] . k_t,   out = sum_t softmax(s)_t v_t,
 *   lse = log sum_t exp(s_t); no visible token: out = 0, lse = -inf.
 * The keys and values of every token slot a sequence can hold
 * (max_blocks_per_seq * page_block) are rebuilt into the workspace in fp32
 * (bf16 weights: on the matrix cores, fp32 accumulation; f32 weights: fp32
 * vector ALUs), then each (query, head) runs online softmax over them: on
 * the matrix cores for 256-wide keys and values, with every operand split
 * into bf16 hi + lo (fp32-level accuracy), else on the fp32 vector ALUs. */
typedef struct {
  mla_dims_t dims;      /* d_nope + d_rope <= 256, d_v <= 256 */
  int32_t batch;        /* B >= 0 */
  int32_t q_per_seq;    /* Sq >= 1 new tokens per sequence */
  const void* q;        /* [B][Sq][H][d_nope + d_rope], q_dtype, 16-B aligned */
  mla_dtype_t q_dtype;  /* F32 or BF16 */
  const void* w_kv_b;   /* [H][d_nope + d_v][d_latent], w_dtype, 16-B aligned */
  mla_dtype_t w_dtype;  /* F32 or BF16 */
  const void* kv_pool;  /* [num_pages][page_block][row_bytes], any kv_format */
  mla_kv_format_t kv_format;
  int64_t num_pages;
  int32_t page_block;          /* 16, 32, 64 or 128 */
  const int32_t* block_table;  /* [B][max_blocks_per_seq] */
  int32_t max_blocks_per_seq;  /* max_blocks_per_seq * page_block <= 2^24 */
  const int32_t* seq_lens;     /* [B] cached tokens, the chunk included */
  float softmax_scale;
  void* workspace;             /* mla_prefill_workspace_size() bytes, 16-B aligned,
                                  no initialisation needed */
  size_t workspace_bytes;
  float* out;                  /* out: [B][Sq][H][d_v], F32 */
  float* lse;                  /* out (optional, may be NULL): [B][Sq][H] */
} mla_prefill_params_t;

/* Workspace bytes of mla_prefill_paged: 4 * B * max_blocks_per_seq *
 * page_block * (H * (d_nope + d_v) + d_rope) for the rebuilt keys and
 * values, plus, when the matrix-core attention splits each query block's
 * keys into S ranges (S chosen from B, Sq, H and the capacity), 4 * B * Sq *
 * H * S * (d_v + 1) for the partial results; each part rounded up to 256.
 * Host scalars only. */
mla_status_t mla_prefill_workspace_size(const mla_prefill_params_t* p, size_t* bytes);
/* Errors: see the conventions above; every check runs before any launch. */
mla_status_t mla_prefill_paged(const mla_prefill_params_t* p, void* stream);

/* Host-side check of the device-trusted tables, for callers that hold (or
 * copy back) host copies of them: seq_lens [batch] and block_table
 * [batch][max_blocks_per_seq] are HOST pointers here.  Checks that every
 * seq_lens[b] lies in [0, max_blocks_per_seq * page_block] and that every
 * block_table entry a decode reads (logical pages [0, ceil(seq_lens[b] /
 * page_block)) of each sequence) lies in [0, num_pages).  Returns MLA_OK,
 * or MLA_ERR_INVALID_SHAPE with a message naming the first offending entry
 * ("block_table[3][17]: expected 0..8191, got -1").  Touches no device and
 * launches nothing; the decode calls do not run it themselves (they take
 * the tables as device pointers and trust them, as stated at the top). */
mla_status_t mla_validate_tables(int32_t batch, const int32_t* seq_lens, const int32_t* block_table,
                                 int32_t max_blocks_per_seq, int64_t num_pages, int32_t page_block);

const char* mla_status_string(mla_status_t status);
/* Message of the last failed call on this thread ("" if none). */
const char* mla_last_error_message(void);
int32_t mla_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBMLA_MLA_H */
