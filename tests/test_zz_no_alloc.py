"""The allocation-free decode entry point (mla_decode_paged_noalloc) on the GPU.

It runs the kernels of mla_decode_paged with the partials in the library's
per-GPU scratch array instead of a caller's workspace, so on the same inputs
and stream both entry points must give the same bits.  Calls follow one
another with shrinking inputs (the scratch keeps the previous call's
partials), and every output is also held to the oracle's bar on the cases
small enough for it.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from synth import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

TAU = 1e-2  # bf16 matrix-core path, f32 queries: fraction of the output RMS


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_paged_decode_amd as mla
    mla.lib()


def rel(a, b):
    b = np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(np.asarray(a, dtype=np.float64) - b))) / math.sqrt(float(np.mean(b ** 2)))


def both_entry_points(inp, num_splits=0, q_abs_dtype=None):
    """o_latent and lse from mla_decode_paged (own workspace) and from
    mla_decode_paged_noalloc, on the same absorbed queries."""
    import mla_paged_decode_amd as mla
    from mla_paged_decode_amd.step import DecodeStep, DeviceBatch
    q_abs_dtype = mla.MLA_F32 if q_abs_dtype is None else q_abs_dtype
    st = DecodeStep(DeviceBatch.upload(inp), q_abs_dtype=q_abs_dtype, num_splits=num_splits)
    st.absorb()
    st.o_latent.fill_(float("nan"))
    st.lse.fill_(float("nan"))
    mla.mla_decode_paged(st.params)
    torch.cuda.synchronize()
    want = st.o_latent.clone(), st.lse.clone()
    st.o_latent.fill_(float("nan"))
    st.lse.fill_(float("nan"))
    p = mla.make_decode_params(
        dims=st.dev.dims, batch=st.dev.batch, q_per_seq=st.dev.q_per_seq, q_abs=st.q_abs,
        kv_pool=st.dev.kv_pool, kv_format=st.dev.kv_format, num_pages=st.dev.kv_pool.shape[0],
        page_block=st.dev.page_block, block_table=st.dev.block_table,
        max_blocks_per_seq=st.dev.block_table.shape[1], seq_lens=st.dev.seq_lens,
        softmax_scale=st.dev.softmax_scale, num_splits=num_splits, o_latent=st.o_latent, lse=st.lse,
        q_abs_dtype=q_abs_dtype)  # no workspace
    assert mla.mla_decode_select_kernel(p) == mla.mla_decode_select_kernel(st.params)
    assert mla.mla_decode_workspace_size(p) <= mla.MLA_NOALLOC_SCRATCH_BYTES
    mla.mla_decode_paged_noalloc(p)
    torch.cuda.synchronize()
    got = st.o_latent.clone(), st.lse.clone()
    st.project()  # out = W_UV o_latent, from the noalloc call's o_latent
    torch.cuda.synchronize()
    return want, got, st.out.cpu().numpy()


def test_noalloc_matches_the_workspace_entry_point_on_shrinking_calls():
    """Three calls in a row: the 256-sequence ragged batch at full size,
    then 40 and 7 of its sequences (new seeds, split counts that differ), each
    bit-identical to mla_decode_paged, the small ones also within the bar of
    the oracle."""
    base = WORKLOADS["ragged_b256_h20_ctx512_8k_bf16"]
    cases = [(base, 0, False),
             (base.with_(batch=40, seed=11, lens=("uniform", 1, 3000)), 0, True),
             (base.with_(batch=7, seed=12, lens=("fixed", (1, 31, 32, 33, 100, 2049, 0))), 5, True)]
    for wl, splits, check_oracle in cases:
        say(f"[noalloc] {wl.name} B={wl.batch} num_splits={splits}")
        inp = make_inputs(wl, poison_tail=True)
        (o_w, l_w), (o_n, l_n), out = both_entry_points(inp, splits)
        assert torch.isfinite(o_n).all()
        assert torch.equal(o_w, o_n), "noalloc output differs from mla_decode_paged"
        assert torch.equal(torch.isneginf(l_w), torch.isneginf(l_n))
        fin = torch.isfinite(l_w)
        assert torch.equal(l_w[fin], l_n[fin])
        if check_oracle:
            ref, ref_lse = oracle.mla_decode(inp)
            assert rel(out, ref) <= TAU
            fin = np.isfinite(ref_lse)
            l_np = l_n.cpu().numpy()
            assert np.array_equal(np.isneginf(l_np), np.isneginf(ref_lse))
            assert np.max(np.abs(l_np[fin] - ref_lse[fin]), initial=0.0) <= 1e-3


def test_noalloc_fp8_rows_then_smaller_bf16_call():
    """The quantised-row matrix-core kernel's partials (bf16 queries, four
    per sequence, the full 64-sequence batch) in the scratch, then a much
    smaller bf16 call: both bit-identical to the workspace entry point."""
    import mla_paged_decode_amd as mla
    fp8 = WORKLOADS["fp8_mtp4_b64_h20_ctx16k"]  # full size: 64 sequences x 4 queries
    small = WORKLOADS["glm_b32_h20_ctx4096_bf16"].with_(batch=3, lens=("fixed", (700, 64, 1500)))
    for wl, qd in ((fp8, mla.MLA_BF16), (small, mla.MLA_F32)):
        say(f"[noalloc] {wl.name} B={wl.batch}")
        inp = make_inputs(wl)
        (o_w, l_w), (o_n, l_n), _ = both_entry_points(inp, q_abs_dtype=qd)
        assert torch.equal(o_w, o_n)
        fin = torch.isfinite(l_w)
        assert torch.equal(l_w[fin], l_n[fin])
