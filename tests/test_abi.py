"""The C-ABI library on a machine without a GPU: it loads, exports every
declared entry point, reports row sizes, and rejects every invalid argument
with its status code and message before touching a device."""
import ctypes
import json
import os
import re

import pytest

import mla_paged_decode_amd as mla
from mla_paged_decode_amd import (MLA_BF16, MLA_F32, MLA_KERNEL_MFMA, MLA_KV_BF16, MLA_KV_F32,
                                  MLA_KV_FP8_E4M3_E8M0, Dims, MlaError, make_decode_params)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GLM = Dims(20, 512, 64, 192, 256)
FP8 = Dims(20, 448, 64, 192, 256)
FAKE = 0x10000  # a 16-byte aligned address that is never dereferenced


def declared_functions():
    src = open(os.path.join(ROOT, "include", "mla.h")).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\*?\s+\*?(mla_\w+)\(", src, re.M)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) == 16, names
    L = mla.lib()
    for n in names:
        assert hasattr(L, n), n
    assert mla.mla_abi_version() == 3


def test_row_bytes_match_page_figures(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "page_invariants.json")))
    assert mla.mla_kv_row_bytes(GLM, MLA_KV_BF16) * g["num_layers"] == g["bf16_bytes_per_token_all_layers"]
    assert mla.mla_kv_row_bytes(FP8, MLA_KV_FP8_E4M3_E8M0) == g["fp8_row_bytes"]
    # the model record's fp4 variant: 288 bytes per token
    assert mla.mla_kv_row_bytes(FP8, mla.MLA_KV_FP4_E2M1_E4M3) == 288
    assert mla.mla_kv_row_bytes(GLM, MLA_KV_F32) == 2304
    assert mla.mla_kv_row_bytes(GLM, 7) == 0


def params(**kw):
    base = dict(dims=GLM, batch=4, q_per_seq=1, q_abs=FAKE, kv_pool=FAKE, kv_format=MLA_KV_BF16,
                num_pages=100, page_block=64, block_table=FAKE, max_blocks_per_seq=32,
                seq_lens=FAKE, softmax_scale=0.0625, num_splits=0, workspace=FAKE,
                workspace_bytes=1 << 40, o_latent=FAKE, lse=None, q_abs_dtype=MLA_F32)
    base.update(kw)
    return make_decode_params(**base)


def expect_error(fn, status, fragment):
    with pytest.raises(MlaError) as ei:
        fn()
    assert ei.value.status == status, ei.value
    assert fragment in ei.value.message, ei.value.message


@pytest.mark.parametrize("kw,status,fragment", [
    (dict(page_block=96), 3, "page_block: expected one of {16,32,64,128}, got 96"),
    (dict(q_per_seq=9), 3, "q_per_seq: expected 1..8, got 9"),
    (dict(q_per_seq=0), 3, "q_per_seq: expected 1..8, got 0"),
    (dict(dims=Dims(20, 448, 64, 192, 256)), 3, "d_latent: expected 512 for this kv_format, got 448"),
    (dict(dims=GLM, kv_format=MLA_KV_FP8_E4M3_E8M0), 3, "d_latent: expected 448 for this kv_format, got 512"),
    (dict(dims=Dims(20, 512, 32, 192, 256)), 3, "d_rope: expected 64, got 32"),
    (dict(dims=Dims(129, 512, 64, 192, 256)), 2, "num_heads: expected 1..128, got 129"),
    (dict(dims=Dims(0, 512, 64, 192, 256)), 2, "num_heads: expected 1..128, got 0"),
    (dict(dims=Dims(20, 512, 64, 100, 256)), 3, "d_nope: expected a multiple of 32"),
    (dict(kv_format=5), 3, "kv_format: expected 0 (f32), 1 (bf16), 2 (fp8 e4m3+e8m0) or 3"),
    (dict(batch=-1), 2, "batch: expected >= 0, got -1"),
    (dict(num_pages=0), 2, "num_pages: expected >= 1, got 0"),
    (dict(max_blocks_per_seq=0), 2, "max_blocks_per_seq: expected >= 1, got 0"),
    (dict(num_splits=-2), 2, "num_splits: expected 0 (balanced) or 1..4096, got -2"),
    (dict(q_abs_dtype=3), 3, "q_abs_dtype: expected 0 (f32) or 1 (bf16), got 3"),
    (dict(kernel=9), 3, "kernel: expected 0 (auto), 1 (simt) or 2 (mfma), got 9"),
    (dict(softmax_scale=float("nan")), 2, "softmax_scale: expected a finite value"),
    (dict(q_abs=None), 1, "q_abs: expected non-null, got NULL"),
    (dict(kv_pool=None), 1, "kv_pool: expected non-null, got NULL"),
    (dict(block_table=None), 1, "block_table: expected non-null, got NULL"),
    (dict(seq_lens=None), 1, "seq_lens: expected non-null, got NULL"),
    (dict(workspace=None), 1, "workspace: expected non-null, got NULL"),
    (dict(o_latent=None), 1, "o_latent: expected non-null, got NULL"),
    (dict(kv_pool=FAKE + 8), 4, "kv_pool: expected 16-byte alignment"),
    (dict(q_abs=FAKE + 4), 4, "q_abs: expected 16-byte alignment"),
    (dict(seq_lens=FAKE + 2), 4, "seq_lens: expected 4-byte alignment"),
    (dict(lse=FAKE + 1), 4, "lse: expected 4-byte alignment"),
    (dict(workspace_bytes=100), 5, "workspace_bytes: expected >= "),
    (dict(q_abs_dtype=MLA_BF16), 3, "q_abs_dtype: expected 0 (f32) with a bf16 or f32 cache, got 1 (bf16)"),
    (dict(q_abs_dtype=MLA_BF16, kv_format=MLA_KV_F32), 3, "set MLA_DECODE_ALLOW_BF16_QUERIES"),
    (dict(flags=0x9), 3, "flags: expected a subset of 0x7, got 0x9"),
])
def test_decode_rejects_before_launch(kw, status, fragment):
    p = params(**kw)
    expect_error(lambda: mla.mla_decode_paged(p, stream=0), status, fragment)


def test_mfma_request_rejected_where_unsupported():
    p = params(kv_format=MLA_KV_F32, kernel=MLA_KERNEL_MFMA)
    expect_error(lambda: mla.mla_decode_paged(p, stream=0), 3, "MFMA path does not support")
    expect_error(lambda: mla.mla_decode_select_kernel(p), 3, "MFMA path does not support")
    assert mla.mla_decode_select_kernel(params(kv_format=MLA_KV_F32)) == mla.MLA_KERNEL_SIMT


def test_workspace_size_is_host_only_and_monotone():
    small = mla.mla_decode_workspace_size(params(batch=4, num_splits=32))
    big = mla.mla_decode_workspace_size(params(batch=4, num_splits=64))
    bal = mla.mla_decode_workspace_size(params(batch=4, num_splits=0))
    assert 0 < small < big
    # 4 * 32 partial slots of 20 rows x (512 + 1) floats, plus the plan
    assert small >= 4 * 32 * 20 * 513 * 4
    assert bal >= (512 + 4) * 20 * 513 * 4
    expect_error(lambda: mla.mla_decode_workspace_size(params(page_block=8)), 3, "page_block")


def test_empty_batch_and_zero_tokens_are_no_ops():
    mla.mla_decode_paged(params(batch=0, q_abs=None, kv_pool=None, block_table=None,
                                seq_lens=None, workspace=None, o_latent=None), stream=0)
    mla.mla_absorb_q(GLM, 0, 0, 0, 0, q_dtype=MLA_BF16, w_dtype=MLA_BF16, q_abs_dtype=MLA_F32, stream=0)
    mla.mla_out_proj(GLM, 0, 0, 0, 0, w_dtype=MLA_BF16, stream=0)


@pytest.mark.parametrize("call", ["absorb", "out_proj"])
def test_projection_argument_checks(call):
    if call == "absorb":
        f = lambda dims, n, a, b, c, dt=MLA_BF16: mla.mla_absorb_q(dims, n, a, b, c, q_dtype=dt, w_dtype=MLA_BF16,
                                                                 q_abs_dtype=MLA_F32, stream=0)
    else:
        f = lambda dims, n, a, b, c, dt=MLA_BF16: mla.mla_out_proj(dims, n, a, b, c, w_dtype=dt, stream=0)
    expect_error(lambda: f(GLM, -1, FAKE, FAKE, FAKE), 2, "n_tokens: expected >= 0, got -1")
    expect_error(lambda: f(GLM, 4, 0, FAKE, FAKE), 1, "expected non-null, got NULL")
    expect_error(lambda: f(GLM, 4, FAKE + 8, FAKE, FAKE), 4, "expected 16-byte aligned pointers")
    expect_error(lambda: f(GLM, 4, FAKE, FAKE, FAKE, 7), 3, "expected 0 or 1, got 7")
    expect_error(lambda: f(Dims(20, 500, 64, 192, 256), 4, FAKE, FAKE, FAKE), 3, "d_latent: expected a multiple of 32")


@pytest.mark.parametrize("kw,status,fragment", [
    (dict(page_block=96), 3, "page_block"),
    (dict(dims=GLM, kv_format=MLA_KV_FP8_E4M3_E8M0), 3, "d_latent"),
    (dict(kv_format=7), 3, "kv_format"),
    (dict(n_rows=-1), 2, "n_rows"),
    (dict(rows_dtype=5), 3, "rows_dtype"),
    (dict(rows=0), 1, "rows"),
    (dict(slots=0), 1, "slots"),
    (dict(pool=0), 1, "kv_pool"),
    (dict(rows=FAKE + 4), 4, "aligned"),
    (dict(slots=FAKE + 4), 4, "aligned"),
])
def test_cache_write_rejects_before_launch(kw, status, fragment):
    args = dict(dims=GLM, n_rows=8, rows=FAKE, rows_dtype=MLA_F32, slots=FAKE, pool=FAKE,
                kv_format=MLA_KV_BF16, num_pages=4, page_block=16)
    args.update(kw)
    with pytest.raises(MlaError) as e:
        mla.mla_cache_write(args["dims"], args["n_rows"], args["rows"], args["slots"], args["pool"],
                            args["kv_format"], args["num_pages"], args["page_block"],
                            rows_dtype=args["rows_dtype"], stream=0)
    assert e.value.status == status
    assert fragment in e.value.message


def test_cache_write_without_rows_or_pages_is_a_no_op():
    mla.mla_cache_write(GLM, 0, 0, 0, 0, MLA_KV_BF16, 4, 16, rows_dtype=MLA_F32, stream=0)
    mla.mla_cache_write(GLM, 8, FAKE, FAKE, FAKE, MLA_KV_BF16, 0, 16, rows_dtype=MLA_F32, stream=0)


def sparse_params(**kw):
    base = dict(dims=GLM, batch=2, q_per_seq=1, q_abs=FAKE, kv_pool=FAKE, kv_format=MLA_KV_BF16, num_pages=8,
                page_block=64, block_table=FAKE, max_blocks_per_seq=4, seq_lens=FAKE, softmax_scale=0.0625,
                num_splits=2, workspace=FAKE, workspace_bytes=1 << 30, o_latent=FAKE, lse=None,
                q_abs_dtype=MLA_F32)
    base.update(kw)
    return make_decode_params(**base)


@pytest.mark.parametrize("kw,width,status,fragment", [
    (dict(num_splits=0), 128, 3, "num_splits"),
    (dict(kernel=MLA_KERNEL_MFMA), 100, 3, "kernel"),
    (dict(kernel=MLA_KERNEL_MFMA, kv_format=MLA_KV_F32), 128, 3, "kernel"),
    (dict(), 0, 2, "topk_width"),
    (dict(page_block=96), 128, 3, "page_block"),
    (dict(workspace_bytes=16), 128, 5, "workspace_bytes"),
])
def test_sparse_decode_rejects_before_launch(kw, width, status, fragment):
    with pytest.raises(MlaError) as e:
        mla.mla_decode_sparse_paged(sparse_params(**kw), FAKE, width, stream=0)
    assert e.value.status == status
    assert fragment in e.value.message


def test_sparse_decode_null_index_list_and_workspace_size():
    with pytest.raises(MlaError) as e:
        mla.mla_decode_sparse_paged(sparse_params(), 0, 128, stream=0)
    assert e.value.status == 1 and "topk_indices" in e.value.message
    # every (sequence, query token) pair is a sequence of H rows, padded to 16
    n1 = mla.mla_decode_sparse_workspace_size(sparse_params(q_per_seq=1), 128)
    n4 = mla.mla_decode_sparse_workspace_size(sparse_params(q_per_seq=4), 128)
    assert n4 > 3 * n1 // 2
    assert n4 >= mla.mla_decode_workspace_size(sparse_params(q_per_seq=4))


def prefill_params(**kw):
    base = dict(dims=GLM, batch=2, q_per_seq=64, q=FAKE, w_kv_b=FAKE, kv_pool=FAKE, kv_format=MLA_KV_BF16,
                num_pages=8, page_block=64, block_table=FAKE, max_blocks_per_seq=4, seq_lens=FAKE,
                softmax_scale=0.0625, out=FAKE, lse=None, workspace=FAKE, workspace_bytes=1 << 30,
                q_dtype=MLA_F32, w_dtype=MLA_F32)
    base.update(kw)
    return mla.make_prefill_params(**base)


@pytest.mark.parametrize("kw,status,fragment", [
    (dict(q_per_seq=0), 2, "q_per_seq"),
    (dict(kv_format=7), 3, "kv_format"),
    (dict(dims=Dims(20, 512, 64, 256, 256)), 3, "d_nope + d_rope"),
    (dict(dims=FP8), 3, "d_latent"),
    (dict(page_block=48), 3, "page_block"),
    (dict(q_dtype=4), 3, "q_dtype"),
    (dict(w_dtype=4), 3, "w_dtype"),
    (dict(max_blocks_per_seq=0), 2, "max_blocks_per_seq"),
    (dict(softmax_scale=float("inf")), 2, "softmax_scale"),
    (dict(q=0), 1, "q"),
    (dict(out=0), 1, "out"),
    (dict(workspace=0), 1, "workspace"),
    (dict(w_kv_b=FAKE + 8), 4, "w_kv_b"),
    (dict(workspace_bytes=1024), 5, "workspace_bytes"),
])
def test_prefill_rejects_before_launch(kw, status, fragment):
    with pytest.raises(MlaError) as e:
        mla.mla_prefill_paged(prefill_params(**kw), stream=0)
    assert e.value.status == status
    assert fragment in e.value.message


def test_prefill_workspace_size_and_empty_batch():
    p = prefill_params()
    slots = 2 * 4 * 64
    kv = 4 * slots * 20 * 192 + 4 * slots * 64 + 4 * slots * 20 * 256  # every part a multiple of 256 here
    # 2 sequences x 1 block of 64 queries x 20 heads = 40 workgroups: two key
    # splits (capacity 256 tokens allows at most 2), with their partials
    splits, n = 2, 2 * 64
    assert mla.mla_prefill_workspace_size(p) == kv + 4 * n * 20 * splits * 256 + 4 * n * 20 * splits
    # narrow heads run the vector-ALU attention: no partials
    narrow = prefill_params(dims=Dims(20, 512, 64, 128, 128))
    assert mla.mla_prefill_workspace_size(narrow) == 4 * slots * 20 * 128 * 2 + 4 * slots * 64
    mla.mla_prefill_paged(prefill_params(batch=0, q=0, out=0, workspace=0), stream=0)  # no-op, no launch


def test_bf16_queries_on_a_bf16_cache_need_the_opt_in():
    """Single-rounded queries on a bf16 / f32 cache are refused unless the
    caller sets MLA_DECODE_ALLOW_BF16_QUERIES; the fp8 and fp4 caches take
    them as they are.  (The checks run before any launch, so a call that
    passes them reaches the launch and fails there without a GPU.)"""
    p = params(q_abs_dtype=MLA_BF16)
    expect_error(lambda: mla.mla_decode_workspace_size(p), 3, "MLA_DECODE_ALLOW_BF16_QUERIES")
    expect_error(lambda: mla.mla_decode_select_kernel(p), 3, "MLA_DECODE_ALLOW_BF16_QUERIES")
    for ok in (params(q_abs_dtype=MLA_BF16, flags=mla.MLA_DECODE_ALLOW_BF16_QUERIES),
               params(dims=FP8, kv_format=MLA_KV_FP8_E4M3_E8M0, q_abs_dtype=MLA_BF16),
               params(dims=FP8, kv_format=mla.MLA_KV_FP4_E2M1_E4M3, q_abs_dtype=MLA_BF16)):
        assert mla.mla_decode_workspace_size(ok) > 0
        assert mla.mla_decode_select_kernel(ok) == mla.MLA_KERNEL_MFMA


def test_validate_tables_accepts_valid_tables():
    import numpy as np
    lens = np.array([0, 1, 64, 65, 128], dtype=np.int32)
    bt = np.full((5, 2), -1, dtype=np.int32)
    bt[1, 0] = 0
    bt[2, 0] = 3
    bt[3, :] = [1, 2]
    bt[4, :] = [4, 0]
    mla.mla_validate_tables(lens, bt, num_pages=5, page_block=64)
    mla.mla_validate_tables(np.zeros(0, np.int32), np.zeros((0, 1), np.int32), num_pages=1, page_block=16)


@pytest.mark.parametrize("case,fragment", [
    ("len_negative", "seq_lens[1]: expected 0..128, got -1"),
    ("len_too_long", "seq_lens[2]: expected 0..128, got 129"),
    ("page_negative", "block_table[3][1]: expected 0..4, got -1"),
    ("page_too_big", "block_table[0][0]: expected 0..4, got 5"),
])
def test_validate_tables_names_the_bad_entry(case, fragment):
    import numpy as np
    lens = np.array([10, 5, 100, 70], dtype=np.int32)
    bt = np.array([[0, -1], [1, -1], [2, 3], [4, 0]], dtype=np.int32)
    if case == "len_negative":
        lens[1] = -1
    elif case == "len_too_long":
        lens[2] = 129
    elif case == "page_negative":
        bt[3, 1] = -1
    else:
        bt[0, 0] = 5
    expect_error(lambda: mla.mla_validate_tables(lens, bt, num_pages=5, page_block=64), 2, fragment)
    # entries past a sequence's last page are never read, so they may hold anything
    bt2 = np.array([[0, 99], [1, -7], [2, 3], [4, 0]], dtype=np.int32)
    mla.mla_validate_tables(np.array([10, 5, 100, 70], np.int32), bt2, num_pages=5, page_block=64)


def test_synthetic_workload_tables_are_valid():
    """Every workload's generated tables pass the validator (the inputs the
    GPU tests and the benchmark use)."""
    from synth import WORKLOADS, make_inputs
    for name, wl in WORKLOADS.items():
        small = wl.with_(batch=min(wl.batch, 4), lens=("fixed", tuple([37, 4096, 1, 0][:min(wl.batch, 4)])))
        inp = make_inputs(small)
        mla.mla_validate_tables(inp.seq_lens, inp.block_table, inp.kv_pool.shape[0], small.page_block)


def test_noalloc_entry_rejects_before_any_device_work():
    """The allocation-free decode refuses, before touching a GPU, a call
    whose partials would not fit its scratch and the run-time split; the
    workspace fields are not read."""
    assert mla.MLA_NOALLOC_SCRATCH_BYTES == 128 << 20
    big = params(batch=4000, workspace=None, workspace_bytes=0)
    assert mla.mla_decode_workspace_size(big) > mla.MLA_NOALLOC_SCRATCH_BYTES
    expect_error(lambda: mla.mla_decode_paged_noalloc(big, stream=0), 5, "beyond the 134217728-byte scratch")
    dyn = params(workspace=None, workspace_bytes=0, flags=mla.MLA_DECODE_DYNAMIC_SPLIT)
    expect_error(lambda: mla.mla_decode_paged_noalloc(dyn, stream=0), 3, "MLA_DECODE_DYNAMIC_SPLIT")
    # the other checks still apply
    expect_error(lambda: mla.mla_decode_paged_noalloc(params(o_latent=None, workspace=None), stream=0), 1,
                 "o_latent")
    # a call with no sequences returns before looking up the scratch
    mla.mla_decode_paged_noalloc(params(batch=0, workspace=None, workspace_bytes=0), stream=0)
