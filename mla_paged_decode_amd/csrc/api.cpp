// C-ABI host layer of libmla: argument validation, workspace layout, kernel
// selection and launches.  No allocation, no host synchronisation.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "internal.h"
#include "mla.h"

namespace {

thread_local std::string g_last_error;

mla_status_t fail(mla_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

mla_status_t ok() {
  g_last_error.clear();
  return MLA_OK;
}

bool aligned(const void* p, size_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Shape checks common to all calls.  `d_latent_required` = 0 accepts any
// multiple of 32 in [32, 512].
mla_status_t check_dims(const mla_dims_t* d, int d_latent_required) {
  if (!d) return fail(MLA_ERR_NULL_POINTER, "dims: expected non-null, got NULL");
  if (d->num_heads < 1 || d->num_heads > 128)
    return fail(MLA_ERR_INVALID_SHAPE, "num_heads: expected 1..128, got %d", d->num_heads);
  if (d->d_rope != 64)
    return fail(MLA_ERR_UNSUPPORTED, "d_rope: expected 64, got %d", d->d_rope);
  if (d->d_nope < 32 || d->d_nope > 512 || d->d_nope % 32)
    return fail(MLA_ERR_UNSUPPORTED, "d_nope: expected a multiple of 32 in [32, 512], got %d", d->d_nope);
  if (d->d_v < 32 || d->d_v > 512 || d->d_v % 32)
    return fail(MLA_ERR_UNSUPPORTED, "d_v: expected a multiple of 32 in [32, 512], got %d", d->d_v);
  if (d_latent_required) {
    if (d->d_latent != d_latent_required)
      return fail(MLA_ERR_UNSUPPORTED, "d_latent: expected %d for this kv_format, got %d",
                  d_latent_required, d->d_latent);
  } else if (d->d_latent < 32 || d->d_latent > 512 || d->d_latent % 32) {
    return fail(MLA_ERR_UNSUPPORTED, "d_latent: expected a multiple of 32 in [32, 512], got %d",
                d->d_latent);
  }
  return MLA_OK;
}

bool valid_dtype(int t) { return t == MLA_F32 || t == MLA_BF16; }

int latent_for_format(int fmt) { return fmt == MLA_KV_FP8_E4M3_E8M0 || fmt == MLA_KV_FP4_E2M1_E4M3 ? 448 : 512; }

bool valid_format(int f) { return f >= MLA_KV_F32 && f <= MLA_KV_FP4_E2M1_E4M3; }

mla_status_t check_decode_scalars(const mla_decode_params_t* p) {
  if (!p) return fail(MLA_ERR_NULL_POINTER, "params: expected non-null, got NULL");
  if (!valid_format(p->kv_format))
    return fail(MLA_ERR_UNSUPPORTED, "kv_format: expected 0 (f32), 1 (bf16), 2 (fp8 e4m3+e8m0) or 3 (fp4 e2m1+e4m3), got %d",
                (int)p->kv_format);
  mla_status_t st = check_dims(&p->dims, latent_for_format(p->kv_format));
  if (st) return st;
  if (p->batch < 0) return fail(MLA_ERR_INVALID_SHAPE, "batch: expected >= 0, got %d", p->batch);
  if (p->q_per_seq < 1 || p->q_per_seq > 8)
    return fail(MLA_ERR_UNSUPPORTED, "q_per_seq: expected 1..8, got %d", p->q_per_seq);
  const int P = p->page_block;
  if (P != 16 && P != 32 && P != 64 && P != 128)
    return fail(MLA_ERR_UNSUPPORTED, "page_block: expected one of {16,32,64,128}, got %d", P);
  if (p->num_pages < 1) return fail(MLA_ERR_INVALID_SHAPE, "num_pages: expected >= 1, got %lld",
                                    (long long)p->num_pages);
  if (p->max_blocks_per_seq < 1)
    return fail(MLA_ERR_INVALID_SHAPE, "max_blocks_per_seq: expected >= 1, got %d", p->max_blocks_per_seq);
  if (p->num_splits < 0 || p->num_splits > 4096)
    return fail(MLA_ERR_INVALID_SHAPE, "num_splits: expected 0 (balanced) or 1..4096, got %d", p->num_splits);
  if ((int64_t)p->batch * (p->num_splits ? p->num_splits : 1) > 0x7fffffffLL)
    return fail(MLA_ERR_INVALID_SHAPE, "batch * num_splits: expected < 2^31, got %lld",
                (long long)p->batch * p->num_splits);
  if (!valid_dtype(p->q_abs_dtype))
    return fail(MLA_ERR_UNSUPPORTED, "q_abs_dtype: expected 0 (f32) or 1 (bf16), got %d", (int)p->q_abs_dtype);
  if (p->o_dtype != MLA_F32)
    return fail(MLA_ERR_UNSUPPORTED, "o_dtype: expected 0 (f32), got %d", (int)p->o_dtype);
  if (p->kernel != MLA_KERNEL_AUTO && p->kernel != MLA_KERNEL_SIMT && p->kernel != MLA_KERNEL_MFMA)
    return fail(MLA_ERR_UNSUPPORTED, "kernel: expected 0 (auto), 1 (simt) or 2 (mfma), got %d", (int)p->kernel);
  if (!std::isfinite(p->softmax_scale))
    return fail(MLA_ERR_INVALID_SHAPE, "softmax_scale: expected a finite value, got %g", (double)p->softmax_scale);
  const uint32_t known = MLA_DECODE_ALLOW_BF16_QUERIES | MLA_DECODE_DYNAMIC_SPLIT | MLA_DECODE_FUSED_MERGE;
  if (p->flags & ~known)
    return fail(MLA_ERR_UNSUPPORTED, "flags: expected a subset of 0x%x, got 0x%x", known, p->flags);
  if (p->q_abs_dtype == MLA_BF16 && (p->kv_format == MLA_KV_BF16 || p->kv_format == MLA_KV_F32) &&
      !(p->flags & MLA_DECODE_ALLOW_BF16_QUERIES))
    return fail(MLA_ERR_UNSUPPORTED,
                "q_abs_dtype: expected 0 (f32) with a bf16 or f32 cache, got 1 (bf16): single-rounded queries "
                "exceed the 1e-2 match bound there; set MLA_DECODE_ALLOW_BF16_QUERIES in flags to accept them");
  return MLA_OK;
}

// Kernel choice for validated scalars.
mla_status_t select_kernel(const mla_decode_params_t* p, mla_kernel_t* chosen) {
  const int R = p->q_per_seq * p->dims.num_heads;
  const bool mfma_ok = mla::decode_mfma_supported(p->kv_format, p->dims.d_latent, p->dims.d_rope, R,
                                                  p->q_abs_dtype == MLA_F32);
  if (p->kernel == MLA_KERNEL_MFMA && !mfma_ok)
    return fail(MLA_ERR_UNSUPPORTED, "kernel: MFMA path does not support kv_format %d with %d query rows",
                (int)p->kv_format, R);
  *chosen = (p->kernel == MLA_KERNEL_SIMT || !mfma_ok) ? MLA_KERNEL_SIMT : MLA_KERNEL_MFMA;
  return MLA_OK;
}

// The run-time scheduled bf16 kernel (dense decode, balanced mode).
bool use_dyn(const mla_decode_params_t* p, mla_kernel_t chosen) {
  return chosen == MLA_KERNEL_MFMA && (p->flags & MLA_DECODE_DYNAMIC_SPLIT) &&
         mla::decode_dyn_supported(p->kv_format, p->dims.d_latent, p->dims.d_rope,
                                   p->q_per_seq * p->dims.num_heads, p->q_abs_dtype == MLA_F32, p->num_splits,
                                   p->batch);
}

mla_status_t hip_fail(const char* what, hipError_t e) {
  return fail(MLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

namespace mla {

WorkspaceLayout workspace_layout(int B, int R, int dc, int num_splits, bool dyn) {
  WorkspaceLayout w{};
  w.slots = num_splits > 0 ? (int64_t)B * num_splits
            : dyn          ? (int64_t)kMfmaWorkersBf16 + (int64_t)B * (1 + kDynStealParts)
                           : (int64_t)kBalancedWorkers + B;
  w.ctr_off = 0;
  w.tile_start_off = kDynCounterBytes;
  size_t off = round_up(w.tile_start_off + sizeof(int32_t) * ((size_t)B + 2), 256);
  w.part_lse_off = off;
  off = round_up(off + sizeof(float) * (size_t)w.slots * R, 256);
  w.part_o_off = off;
  const size_t R16 = ((size_t)R + 15) / 16 * 16;
  off = round_up(off + sizeof(float) * (size_t)w.slots * R16 * dc, 256);
  w.total = off;
  return w;
}

}  // namespace mla

namespace {

// Sparse matrix-core kernels: the bf16 one (rows straight to LDS) and the
// quantised-row one (fp8 / fp4 rows decoded to bf16 in LDS).
bool sparse_bf16_mfma(const mla_decode_params_t* p, int32_t topk_width) {
  return mla::decode_mfma_sparse_supported(p->kv_format, p->dims.d_latent, p->dims.d_rope, p->dims.num_heads,
                                           topk_width);
}
bool sparse_rows_mfma(const mla_decode_params_t* p, int32_t topk_width) {
  return mla::decode_fp8_rows_sparse_supported(p->kv_format, p->dims.d_latent, p->dims.d_rope, p->dims.num_heads,
                                               p->q_abs_dtype == MLA_F32, topk_width);
}
bool sparse_mfma_ok(const mla_decode_params_t* p, int32_t topk_width) {
  return sparse_bf16_mfma(p, topk_width) || sparse_rows_mfma(p, topk_width);
}

mla_status_t check_sparse(const mla_decode_params_t* p, int32_t topk_width) {
  mla_status_t st = check_decode_scalars(p);
  if (st) return st;
  if (topk_width < 1 || topk_width > (1 << 24))
    return fail(MLA_ERR_INVALID_SHAPE, "topk_width: expected 1..16777216, got %d", topk_width);
  if (p->num_splits < 1)
    return fail(MLA_ERR_UNSUPPORTED,
                "num_splits: expected >= 1 (uniform chunks of each index list) for the sparse call, got %d",
                p->num_splits);
  if (p->kernel == MLA_KERNEL_MFMA && !sparse_mfma_ok(p, topk_width))
    return fail(MLA_ERR_UNSUPPORTED,
                "kernel: the sparse matrix-core kernels need topk_width a multiple of 32 and either a bf16 cache "
                "with num_heads <= 64, or an fp8 / fp4 cache with bf16 q_abs and num_heads <= 128 (got kv_format "
                "%d, q_abs_dtype %d, num_heads %d, topk_width %d)",
                (int)p->kv_format, (int)p->q_abs_dtype, p->dims.num_heads, topk_width);
  if ((int64_t)p->batch * p->q_per_seq * p->num_splits > 0x7fffffffLL)
    return fail(MLA_ERR_INVALID_SHAPE, "batch * q_per_seq * num_splits: expected < 2^31, got %lld",
                (long long)p->batch * p->q_per_seq * p->num_splits);
  return MLA_OK;
}

mla_status_t check_prefill(const mla_prefill_params_t* p) {
  if (!p) return fail(MLA_ERR_NULL_POINTER, "params: expected non-null, got NULL");
  if (!valid_format(p->kv_format))
    return fail(MLA_ERR_UNSUPPORTED, "kv_format: expected 0 (f32), 1 (bf16), 2 (fp8 e4m3+e8m0) or 3 (fp4 e2m1+e4m3), got %d",
                (int)p->kv_format);
  mla_status_t st = check_dims(&p->dims, latent_for_format(p->kv_format));
  if (st) return st;
  if (!mla::prefill_supported(p->dims.d_latent, p->dims.d_rope, p->dims.d_nope, p->dims.d_v))
    return fail(MLA_ERR_UNSUPPORTED, "dims: the prefill needs d_nope + d_rope <= 256 and d_v <= 256, got %d + %d and %d",
                p->dims.d_nope, p->dims.d_rope, p->dims.d_v);
  if (p->batch < 0) return fail(MLA_ERR_INVALID_SHAPE, "batch: expected >= 0, got %d", p->batch);
  if (p->q_per_seq < 1) return fail(MLA_ERR_INVALID_SHAPE, "q_per_seq: expected >= 1, got %d", p->q_per_seq);
  if ((int64_t)p->batch * p->q_per_seq > 0x7fffffffLL)
    return fail(MLA_ERR_INVALID_SHAPE, "batch * q_per_seq: expected < 2^31, got %lld",
                (long long)p->batch * p->q_per_seq);
  const int P = p->page_block;
  if (P != 16 && P != 32 && P != 64 && P != 128)
    return fail(MLA_ERR_UNSUPPORTED, "page_block: expected one of {16,32,64,128}, got %d", P);
  if (p->num_pages < 1)
    return fail(MLA_ERR_INVALID_SHAPE, "num_pages: expected >= 1, got %lld", (long long)p->num_pages);
  if (p->max_blocks_per_seq < 1 || (int64_t)p->max_blocks_per_seq * P > (1 << 24))
    return fail(MLA_ERR_INVALID_SHAPE, "max_blocks_per_seq: expected 1..%d for page_block %d, got %d", (1 << 24) / P, P,
                p->max_blocks_per_seq);
  if (!valid_dtype(p->q_dtype))
    return fail(MLA_ERR_UNSUPPORTED, "q_dtype: expected 0 (f32) or 1 (bf16), got %d", (int)p->q_dtype);
  if (!valid_dtype(p->w_dtype))
    return fail(MLA_ERR_UNSUPPORTED, "w_dtype: expected 0 (f32) or 1 (bf16), got %d", (int)p->w_dtype);
  if (!std::isfinite(p->softmax_scale))
    return fail(MLA_ERR_INVALID_SHAPE, "softmax_scale: expected a finite value, got %g", (double)p->softmax_scale);
  return MLA_OK;
}

struct PrefillLayout {
  int splits;
  int64_t kn_off, kr_off, v_off, part_o_off, part_lse_off;
  size_t total;
};

// Workspace of the prefill: rebuilt no-RoPE keys, RoPE keys and values of
// every token slot a sequence can hold (fp32), then, when the attention
// splits each query block's keys, the per-split partial outputs and
// log-sum-exps.
PrefillLayout prefill_workspace(const mla_prefill_params_t* p) {
  PrefillLayout w{};
  const int64_t Lcap = (int64_t)p->max_blocks_per_seq * p->page_block;
  const int64_t slots = (int64_t)p->batch * Lcap;
  const int64_t H = p->dims.num_heads, N = (int64_t)p->batch * p->q_per_seq;
  w.splits = mla::prefill_attn_splits(p->batch, p->q_per_seq, p->dims.num_heads, Lcap, p->dims.d_nope,
                                      p->dims.d_rope, p->dims.d_v);
  const int64_t kn = slots * H * p->dims.d_nope * 4, kr = slots * p->dims.d_rope * 4;
  const int64_t v = slots * H * p->dims.d_v * 4;
  const int64_t po = w.splits > 1 ? N * H * w.splits * p->dims.d_v * 4 : 0;
  const int64_t pl = w.splits > 1 ? N * H * w.splits * 4 : 0;
  auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
  w.kn_off = 0;
  w.kr_off = up(kn);
  w.v_off = w.kr_off + up(kr);
  w.part_o_off = w.v_off + up(v);
  w.part_lse_off = w.part_o_off + up(po);
  w.total = (size_t)(w.part_lse_off + up(pl));
  return w;
}

}  // namespace

namespace {

// Scratch of the allocation-free decode entry point: one copy per GPU, made
// when the library's code is loaded on that GPU and held until the process
// ends.  Host code never uses the array's name as an address: the device
// address of each GPU's copy is looked up once (hipGetSymbolAddress, with
// that GPU current) and kept per device.
constexpr size_t kNoAllocScratchBytes = MLA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

mla_status_t scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail("hipGetDevice", e);
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MLA_ERR_UNSUPPORTED, "device: expected an ordinal in 0..%d, got %d", kMaxDevices - 1, dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if ((e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch))) != hipSuccess)
      return hip_fail("hipGetSymbolAddress(scratch)", e);
    if (!ptr) return fail(MLA_ERR_HIP, "hipGetSymbolAddress(scratch): returned NULL");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MLA_OK;
}

// Dense decode.  The split partials go to p->workspace, or with `noalloc` to
// the current device's scratch array (p->workspace is then ignored).
mla_status_t decode_paged(const mla_decode_params_t* p, bool noalloc, void* stream) {
  mla_status_t st = check_decode_scalars(p);
  if (st) return st;
  const int B = p->batch, H = p->dims.num_heads, R = p->q_per_seq * H;
  const int dc = p->dims.d_latent, dr = p->dims.d_rope;
  const int fmt = p->kv_format;
  const int q_f32 = p->q_abs_dtype == MLA_F32;
  mla_kernel_t chosen;
  if ((st = select_kernel(p, &chosen)) != MLA_OK) return st;
  const bool use_mfma = chosen == MLA_KERNEL_MFMA;
  if (B == 0) return ok();
  const struct {
    const void* ptr;
    const char* name;
    size_t align;
  } ptrs[] = {{p->q_abs, "q_abs", 16},           {p->kv_pool, "kv_pool", 16},
              {p->block_table, "block_table", 4}, {p->seq_lens, "seq_lens", 4},
              {p->o_latent, "o_latent", 16},      {p->workspace, "workspace", 16}};
  for (const auto& x : ptrs) {
    if (noalloc && &x == &ptrs[5]) break;  // no workspace argument
    if (!x.ptr) return fail(MLA_ERR_NULL_POINTER, "%s: expected non-null, got NULL", x.name);
    if (!aligned(x.ptr, x.align))
      return fail(MLA_ERR_ALIGNMENT, "%s: expected %zu-byte alignment, got %p", x.name, x.align, x.ptr);
  }
  if (p->lse && !aligned(p->lse, 4)) return fail(MLA_ERR_ALIGNMENT, "lse: expected 4-byte alignment, got %p", p->lse);
  const bool dyn = use_dyn(p, chosen);
  if (noalloc && (p->flags & MLA_DECODE_DYNAMIC_SPLIT))
    return fail(MLA_ERR_UNSUPPORTED, "flags: MLA_DECODE_DYNAMIC_SPLIT is not offered without a workspace");
  const mla::WorkspaceLayout w = mla::workspace_layout(B, R, dc, p->num_splits, dyn);
  char* ws = static_cast<char*>(p->workspace);
  if (noalloc) {
    if (w.total > kNoAllocScratchBytes)
      return fail(MLA_ERR_WORKSPACE_TOO_SMALL,
                  "workspace: this call needs %zu bytes, beyond the %zu-byte scratch of the allocation-free entry "
                  "point; use mla_decode_paged with a workspace",
                  w.total, kNoAllocScratchBytes);
    void* sp = nullptr;
    if ((st = scratch_for_current_device(&sp)) != MLA_OK) return st;
    ws = static_cast<char*>(sp);
  } else if (p->workspace_bytes < w.total) {
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "workspace_bytes: expected >= %zu, got %zu", w.total,
                p->workspace_bytes);
  }

  mla::DecodeArgs a{};
  a.B = B;
  a.Sq = p->q_per_seq;
  a.H = H;
  a.R = R;
  a.dc = dc;
  a.dr = dr;
  a.q_abs = p->q_abs;
  a.q_f32 = q_f32;
  a.pool = static_cast<const uint8_t*>(p->kv_pool);
  a.row_bytes = (int64_t)mla_kv_row_bytes(&p->dims, p->kv_format);
  a.P = p->page_block;
  a.P_log2 = __builtin_ctz((unsigned)p->page_block);
  a.block_table = p->block_table;
  a.max_blocks = p->max_blocks_per_seq;
  a.seq_lens = p->seq_lens;
  a.scale_log2 = p->softmax_scale * 1.4426950408889634f;
  a.num_splits = p->num_splits;
  a.workers = mla::kBalancedWorkers;
  a.ctr = reinterpret_cast<uint32_t*>(ws + w.ctr_off);
  a.tile_start = reinterpret_cast<int32_t*>(ws + w.tile_start_off);
  a.part_lse = reinterpret_cast<float*>(ws + w.part_lse_off);
  a.part_o = reinterpret_cast<float*>(ws + w.part_o_off);
  a.o = static_cast<float*>(p->o_latent);
  a.lse = p->lse;

  a.plan_in_kernel = use_mfma && B <= mla::kMaxInKernelPlan;
  a.part_tiled = use_mfma ? 1 : 0;
  if (use_mfma && fmt == MLA_KV_BF16) a.workers = mla::kMfmaWorkersBf16;
  if (use_mfma && mla::decode_fp8_rows_supported(fmt, dc, dr, R, q_f32)) a.workers = mla::fp8_rows_workers(fmt, R);
  a.fuse_merge = !noalloc && !dyn && use_mfma && (p->flags & MLA_DECODE_FUSED_MERGE) && a.plan_in_kernel &&
                 mla::decode_fused_merge_supported(fmt, dc, dr, R, a.num_splits, B, a.workers);

  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (a.num_splits == 0 && !a.plan_in_kernel && (e = mla::launch_plan(a, s)) != hipSuccess)
    return hip_fail("plan launch", e);
  if (p->kernel_start_event && (e = hipEventRecord(static_cast<hipEvent_t>(p->kernel_start_event), s)) != hipSuccess)
    return hip_fail("kernel_start_event record", e);
  e = dyn ? mla::launch_decode_dyn(a, s) : use_mfma ? mla::launch_decode_mfma(a, fmt, s) : mla::launch_decode_simt(a, fmt, s);
  if (e != hipSuccess) return hip_fail("decode launch", e);
  if (p->kernel_stop_event && (e = hipEventRecord(static_cast<hipEvent_t>(p->kernel_stop_event), s)) != hipSuccess)
    return hip_fail("kernel_stop_event record", e);
  if (!a.fuse_merge) {
    e = dyn ? mla::launch_combine_dyn(a, s) : mla::launch_combine(a, s);
    if (e != hipSuccess) return hip_fail("combine launch", e);
  }
  return ok();
}

}  // namespace

extern "C" {

int32_t mla_abi_version(void) { return MLA_ABI_VERSION; }

mla_status_t mla_validate_tables(int32_t batch, const int32_t* seq_lens, const int32_t* block_table,
                                 int32_t max_blocks_per_seq, int64_t num_pages, int32_t page_block) {
  if (batch < 0) return fail(MLA_ERR_INVALID_SHAPE, "batch: expected >= 0, got %d", batch);
  if (page_block < 1) return fail(MLA_ERR_INVALID_SHAPE, "page_block: expected >= 1, got %d", page_block);
  if (max_blocks_per_seq < 1)
    return fail(MLA_ERR_INVALID_SHAPE, "max_blocks_per_seq: expected >= 1, got %d", max_blocks_per_seq);
  if (batch == 0) return ok();
  if (!seq_lens) return fail(MLA_ERR_NULL_POINTER, "seq_lens: expected non-null, got NULL");
  if (!block_table) return fail(MLA_ERR_NULL_POINTER, "block_table: expected non-null, got NULL");
  const int64_t cap = (int64_t)max_blocks_per_seq * page_block;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t L = seq_lens[b];
    if (L < 0 || L > cap)
      return fail(MLA_ERR_INVALID_SHAPE, "seq_lens[%d]: expected 0..%lld, got %lld", b, (long long)cap, (long long)L);
    const int64_t pages = (L + page_block - 1) / page_block;
    for (int64_t i = 0; i < pages; ++i) {
      const int64_t pg = block_table[(int64_t)b * max_blocks_per_seq + i];
      if (pg < 0 || pg >= num_pages)
        return fail(MLA_ERR_INVALID_SHAPE, "block_table[%d][%lld]: expected 0..%lld, got %lld", b, (long long)i,
                    (long long)num_pages - 1, (long long)pg);
    }
  }
  return ok();
}

const char* mla_status_string(mla_status_t s) {
  switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_NULL_POINTER: return "MLA_ERR_NULL_POINTER";
    case MLA_ERR_INVALID_SHAPE: return "MLA_ERR_INVALID_SHAPE";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED";
    case MLA_ERR_ALIGNMENT: return "MLA_ERR_ALIGNMENT";
    case MLA_ERR_WORKSPACE_TOO_SMALL: return "MLA_ERR_WORKSPACE_TOO_SMALL";
    case MLA_ERR_HIP: return "MLA_ERR_HIP";
  }
  return "MLA_ERR_UNKNOWN";
}

const char* mla_last_error_message(void) { return g_last_error.c_str(); }

size_t mla_kv_row_bytes(const mla_dims_t* dims, mla_kv_format_t format) {
  if (!dims || dims->d_latent < 1 || dims->d_rope < 0) return 0;
  const size_t n = (size_t)dims->d_latent + dims->d_rope;
  switch (format) {
    case MLA_KV_F32: return 4 * n;
    case MLA_KV_BF16: return 2 * n;
    case MLA_KV_FP8_E4M3_E8M0: return n % 32 ? 0 : n + n / 32;
    case MLA_KV_FP4_E2M1_E4M3: return n % 16 ? 0 : n / 2 + n / 16;
  }
  return 0;
}

mla_status_t mla_absorb_q(const mla_dims_t* dims, int32_t n_tokens, const void* q, mla_dtype_t q_dtype,
                          const void* w_kv_b, mla_dtype_t w_dtype, void* q_abs, mla_dtype_t q_abs_dtype,
                          void* stream) {
  mla_status_t st = check_dims(dims, 0);
  if (st) return st;
  if (n_tokens < 0) return fail(MLA_ERR_INVALID_SHAPE, "n_tokens: expected >= 0, got %d", n_tokens);
  if (!valid_dtype(q_dtype)) return fail(MLA_ERR_UNSUPPORTED, "q_dtype: expected 0 or 1, got %d", (int)q_dtype);
  if (!valid_dtype(w_dtype)) return fail(MLA_ERR_UNSUPPORTED, "w_dtype: expected 0 or 1, got %d", (int)w_dtype);
  if (!valid_dtype(q_abs_dtype))
    return fail(MLA_ERR_UNSUPPORTED, "q_abs_dtype: expected 0 or 1, got %d", (int)q_abs_dtype);
  if (n_tokens == 0) return ok();
  if (!q) return fail(MLA_ERR_NULL_POINTER, "q: expected non-null, got NULL");
  if (!w_kv_b) return fail(MLA_ERR_NULL_POINTER, "w_kv_b: expected non-null, got NULL");
  if (!q_abs) return fail(MLA_ERR_NULL_POINTER, "q_abs: expected non-null, got NULL");
  if (!aligned(q, 16) || !aligned(w_kv_b, 16) || !aligned(q_abs, 16))
    return fail(MLA_ERR_ALIGNMENT, "q/w_kv_b/q_abs: expected 16-byte aligned pointers, got %p/%p/%p", q,
                w_kv_b, q_abs);
  mla::ProjArgs a{};
  a.N = n_tokens;
  a.H = dims->num_heads;
  a.dn = dims->d_nope;
  a.dr = dims->d_rope;
  a.dv = dims->d_v;
  a.dc = dims->d_latent;
  a.in = q;
  a.in_f32 = q_dtype == MLA_F32;
  a.w = w_kv_b;
  a.w_f32 = w_dtype == MLA_F32;
  a.out = q_abs;
  a.out_f32 = q_abs_dtype == MLA_F32;
  hipError_t e = mla::launch_absorb_q(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail("mla_absorb_q launch", e);
  return ok();
}

mla_status_t mla_out_proj(const mla_dims_t* dims, int32_t n_tokens, const void* o_latent, mla_dtype_t o_dtype,
                          const void* w_kv_b, mla_dtype_t w_dtype, void* out, mla_dtype_t out_dtype,
                          void* stream) {
  mla_status_t st = check_dims(dims, 0);
  if (st) return st;
  if (n_tokens < 0) return fail(MLA_ERR_INVALID_SHAPE, "n_tokens: expected >= 0, got %d", n_tokens);
  if (o_dtype != MLA_F32) return fail(MLA_ERR_UNSUPPORTED, "o_dtype: expected 0 (f32), got %d", (int)o_dtype);
  if (!valid_dtype(w_dtype)) return fail(MLA_ERR_UNSUPPORTED, "w_dtype: expected 0 or 1, got %d", (int)w_dtype);
  if (out_dtype != MLA_F32)
    return fail(MLA_ERR_UNSUPPORTED, "out_dtype: expected 0 (f32), got %d", (int)out_dtype);
  if (n_tokens == 0) return ok();
  if (!o_latent) return fail(MLA_ERR_NULL_POINTER, "o_latent: expected non-null, got NULL");
  if (!w_kv_b) return fail(MLA_ERR_NULL_POINTER, "w_kv_b: expected non-null, got NULL");
  if (!out) return fail(MLA_ERR_NULL_POINTER, "out: expected non-null, got NULL");
  if (!aligned(o_latent, 16) || !aligned(w_kv_b, 16) || !aligned(out, 16))
    return fail(MLA_ERR_ALIGNMENT, "o_latent/w_kv_b/out: expected 16-byte aligned pointers, got %p/%p/%p",
                o_latent, w_kv_b, out);
  mla::ProjArgs a{};
  a.N = n_tokens;
  a.H = dims->num_heads;
  a.dn = dims->d_nope;
  a.dr = dims->d_rope;
  a.dv = dims->d_v;
  a.dc = dims->d_latent;
  a.in = o_latent;
  a.in_f32 = 1;
  a.w = w_kv_b;
  a.w_f32 = w_dtype == MLA_F32;
  a.out = out;
  a.out_f32 = 1;
  hipError_t e = mla::launch_out_proj(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail("mla_out_proj launch", e);
  return ok();
}

mla_status_t mla_cache_write(const mla_dims_t* dims, int32_t n_rows, const void* rows, mla_dtype_t rows_dtype,
                             const int64_t* slots, void* kv_pool, mla_kv_format_t kv_format, int64_t num_pages,
                             int32_t page_block, void* stream) {
  if (!valid_format(kv_format))
    return fail(MLA_ERR_UNSUPPORTED, "kv_format: expected 0 (f32), 1 (bf16), 2 (fp8 e4m3+e8m0) or 3 (fp4 e2m1+e4m3), got %d",
                (int)kv_format);
  mla_status_t st = check_dims(dims, latent_for_format(kv_format));
  if (st) return st;
  if (n_rows < 0) return fail(MLA_ERR_INVALID_SHAPE, "n_rows: expected >= 0, got %d", n_rows);
  if (!valid_dtype(rows_dtype))
    return fail(MLA_ERR_UNSUPPORTED, "rows_dtype: expected 0 (f32) or 1 (bf16), got %d", (int)rows_dtype);
  if (page_block != 16 && page_block != 32 && page_block != 64 && page_block != 128)
    return fail(MLA_ERR_UNSUPPORTED, "page_block: expected one of {16,32,64,128}, got %d", page_block);
  if (num_pages < 0) return fail(MLA_ERR_INVALID_SHAPE, "num_pages: expected >= 0, got %lld", (long long)num_pages);
  if (n_rows == 0) return ok();
  if (!rows) return fail(MLA_ERR_NULL_POINTER, "rows: expected non-null, got NULL");
  if (!slots) return fail(MLA_ERR_NULL_POINTER, "slots: expected non-null, got NULL");
  if (!kv_pool && num_pages > 0) return fail(MLA_ERR_NULL_POINTER, "kv_pool: expected non-null, got NULL");
  if (!aligned(rows, 16) || !aligned(kv_pool, 16) || !aligned(slots, 8))
    return fail(MLA_ERR_ALIGNMENT, "rows/kv_pool/slots: expected 16/16/8-byte aligned pointers, got %p/%p/%p", rows,
                kv_pool, slots);
  mla::CacheWriteArgs a{};
  a.n_rows = n_rows;
  a.n_vals = dims->d_latent + dims->d_rope;
  a.rows = rows;
  a.rows_f32 = rows_dtype == MLA_F32;
  a.slots = slots;
  a.n_slots = num_pages * (int64_t)page_block;
  a.pool = static_cast<uint8_t*>(kv_pool);
  a.row_bytes = (int64_t)mla_kv_row_bytes(dims, kv_format);
  a.fmt = kv_format;
  if (a.n_slots == 0) return ok();
  hipError_t e = mla::launch_cache_write(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail("mla_cache_write launch", e);
  return ok();
}

mla_status_t mla_prefill_workspace_size(const mla_prefill_params_t* p, size_t* bytes) {
  if (!bytes) return fail(MLA_ERR_NULL_POINTER, "bytes: expected non-null, got NULL");
  mla_status_t st = check_prefill(p);
  if (st) return st;
  *bytes = prefill_workspace(p).total;
  return ok();
}

mla_status_t mla_prefill_paged(const mla_prefill_params_t* p, void* stream) {
  mla_status_t st = check_prefill(p);
  if (st) return st;
  if (p->batch == 0) return ok();
  const struct {
    const void* ptr;
    const char* name;
    size_t align;
  } ptrs[] = {{p->q, "q", 16},           {p->w_kv_b, "w_kv_b", 16},        {p->kv_pool, "kv_pool", 16},
              {p->block_table, "block_table", 4}, {p->seq_lens, "seq_lens", 4}, {p->workspace, "workspace", 16},
              {p->out, "out", 16}};
  for (const auto& x : ptrs) {
    if (!x.ptr) return fail(MLA_ERR_NULL_POINTER, "%s: expected non-null, got NULL", x.name);
    if (!aligned(x.ptr, x.align))
      return fail(MLA_ERR_ALIGNMENT, "%s: expected %zu-byte alignment, got %p", x.name, x.align, x.ptr);
  }
  if (p->lse && !aligned(p->lse, 4)) return fail(MLA_ERR_ALIGNMENT, "lse: expected 4-byte alignment, got %p", p->lse);
  const PrefillLayout w = prefill_workspace(p);
  if (p->workspace_bytes < w.total)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "workspace_bytes: expected >= %zu, got %zu", w.total,
                p->workspace_bytes);
  mla::PrefillArgs a{};
  a.B = p->batch;
  a.Sq = p->q_per_seq;
  a.H = p->dims.num_heads;
  a.dn = p->dims.d_nope;
  a.dr = p->dims.d_rope;
  a.dv = p->dims.d_v;
  a.dc = p->dims.d_latent;
  a.P = p->page_block;
  a.max_blocks = p->max_blocks_per_seq;
  a.Lcap = (int64_t)p->max_blocks_per_seq * p->page_block;
  a.q = p->q;
  a.q_f32 = p->q_dtype == MLA_F32;
  a.w = p->w_kv_b;
  a.w_f32 = p->w_dtype == MLA_F32;
  a.pool = static_cast<const uint8_t*>(p->kv_pool);
  a.row_bytes = (int64_t)mla_kv_row_bytes(&p->dims, p->kv_format);
  a.block_table = p->block_table;
  a.seq_lens = p->seq_lens;
  a.scale_log2 = p->softmax_scale * 1.4426950408889634f;
  char* ws = static_cast<char*>(p->workspace);
  a.kn = reinterpret_cast<float*>(ws + w.kn_off);
  a.kr = reinterpret_cast<float*>(ws + w.kr_off);
  a.v = reinterpret_cast<float*>(ws + w.v_off);
  a.splits = w.splits;
  a.part_o = w.splits > 1 ? reinterpret_cast<float*>(ws + w.part_o_off) : nullptr;
  a.part_lse = w.splits > 1 ? reinterpret_cast<float*>(ws + w.part_lse_off) : nullptr;
  a.out = p->out;
  a.lse = p->lse;
  const hipError_t e = mla::launch_prefill(a, p->kv_format, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail("prefill launch", e);
  return ok();
}

mla_status_t mla_decode_sparse_workspace_size(const mla_decode_params_t* p, int32_t topk_width, size_t* bytes) {
  if (!bytes) return fail(MLA_ERR_NULL_POINTER, "bytes: expected non-null, got NULL");
  mla_status_t st = check_sparse(p, topk_width);
  if (st) return st;
  *bytes = mla::workspace_layout(p->batch * p->q_per_seq, p->dims.num_heads, p->dims.d_latent, p->num_splits).total;
  return ok();
}

mla_status_t mla_decode_sparse_paged(const mla_decode_params_t* p, const int32_t* topk_indices, int32_t topk_width,
                                     void* stream) {
  mla_status_t st = check_sparse(p, topk_width);
  if (st) return st;
  const int B = p->batch, Sq = p->q_per_seq, H = p->dims.num_heads;
  const int dc = p->dims.d_latent, dr = p->dims.d_rope;
  if (B == 0) return ok();
  const struct {
    const void* ptr;
    const char* name;
    size_t align;
  } ptrs[] = {{p->q_abs, "q_abs", 16},           {p->kv_pool, "kv_pool", 16},
              {p->block_table, "block_table", 4}, {p->seq_lens, "seq_lens", 4},
              {p->workspace, "workspace", 16},    {p->o_latent, "o_latent", 16},
              {topk_indices, "topk_indices", 4}};
  for (const auto& x : ptrs) {
    if (!x.ptr) return fail(MLA_ERR_NULL_POINTER, "%s: expected non-null, got NULL", x.name);
    if (!aligned(x.ptr, x.align))
      return fail(MLA_ERR_ALIGNMENT, "%s: expected %zu-byte alignment, got %p", x.name, x.align, x.ptr);
  }
  if (p->lse && !aligned(p->lse, 4)) return fail(MLA_ERR_ALIGNMENT, "lse: expected 4-byte alignment, got %p", p->lse);
  const mla::WorkspaceLayout w = mla::workspace_layout(B * Sq, H, dc, p->num_splits);
  if (p->workspace_bytes < w.total)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "workspace_bytes: expected >= %zu, got %zu", w.total,
                p->workspace_bytes);

  // Every (sequence, query token) pair is one sequence of H query rows.
  mla::DecodeArgs a{};
  a.B = B * Sq;
  a.Sq = 1;
  a.H = H;
  a.R = H;
  a.dc = dc;
  a.dr = dr;
  a.q_abs = p->q_abs;
  a.q_f32 = p->q_abs_dtype == MLA_F32;
  a.pool = static_cast<const uint8_t*>(p->kv_pool);
  a.row_bytes = (int64_t)mla_kv_row_bytes(&p->dims, p->kv_format);
  a.P = p->page_block;
  a.P_log2 = __builtin_ctz((unsigned)p->page_block);
  a.block_table = p->block_table;
  a.max_blocks = p->max_blocks_per_seq;
  a.seq_lens = p->seq_lens;
  a.scale_log2 = p->softmax_scale * 1.4426950408889634f;
  a.num_splits = p->num_splits;
  a.workers = mla::kBalancedWorkers;
  char* ws = static_cast<char*>(p->workspace);
  a.tile_start = reinterpret_cast<int32_t*>(ws + w.tile_start_off);
  a.part_lse = reinterpret_cast<float*>(ws + w.part_lse_off);
  a.part_o = reinterpret_cast<float*>(ws + w.part_o_off);
  a.o = static_cast<float*>(p->o_latent);
  a.lse = p->lse;
  a.topk = topk_indices;
  a.topk_width = topk_width;
  a.sparse_sq = Sq;
  const bool use_rows = p->kernel != MLA_KERNEL_SIMT && sparse_rows_mfma(p, topk_width);
  const bool use_mfma = use_rows || (p->kernel != MLA_KERNEL_SIMT && sparse_bf16_mfma(p, topk_width));
  a.part_tiled = use_mfma ? 1 : 0;

  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (p->kernel_start_event && (e = hipEventRecord(static_cast<hipEvent_t>(p->kernel_start_event), s)) != hipSuccess)
    return hip_fail("kernel_start_event record", e);
  e = use_rows   ? mla::launch_decode_fp8_rows_sparse(a, p->kv_format, s)
      : use_mfma ? mla::launch_decode_mfma_sparse(a, s)
                 : mla::launch_decode_simt(a, p->kv_format, s);
  if (e != hipSuccess) return hip_fail("sparse decode launch", e);
  if (p->kernel_stop_event && (e = hipEventRecord(static_cast<hipEvent_t>(p->kernel_stop_event), s)) != hipSuccess)
    return hip_fail("kernel_stop_event record", e);
  if ((e = mla::launch_combine(a, s)) != hipSuccess) return hip_fail("combine launch", e);
  return ok();
}

mla_status_t mla_decode_workspace_size(const mla_decode_params_t* p, size_t* bytes) {
  if (!bytes) return fail(MLA_ERR_NULL_POINTER, "bytes: expected non-null, got NULL");
  mla_status_t st = check_decode_scalars(p);
  if (st) return st;
  mla_kernel_t chosen;
  if ((st = select_kernel(p, &chosen)) != MLA_OK) return st;
  const int R = p->q_per_seq * p->dims.num_heads;
  *bytes = mla::workspace_layout(p->batch, R, p->dims.d_latent, p->num_splits, use_dyn(p, chosen)).total;
  return ok();
}

mla_status_t mla_decode_select_kernel(const mla_decode_params_t* p, mla_kernel_t* chosen) {
  if (!chosen) return fail(MLA_ERR_NULL_POINTER, "chosen: expected non-null, got NULL");
  mla_status_t st = check_decode_scalars(p);
  if (st) return st;
  if ((st = select_kernel(p, chosen)) != MLA_OK) return st;
  return ok();
}

mla_status_t mla_decode_paged(const mla_decode_params_t* p, void* stream) {
  return decode_paged(p, false, stream);
}

mla_status_t mla_decode_paged_noalloc(const mla_decode_params_t* p, void* stream) {
  return decode_paged(p, true, stream);
}

}  // extern "C"
