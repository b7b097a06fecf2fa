"""The run-time scheduled split (MLA_DECODE_DYNAMIC_SPLIT: bf16 cache,
balanced mode) on the GPU.

Tiles of a sequence are handed out from per-sequence counters in the
workspace, so which worker sums which tiles changes from run to run: results
are compared with the oracle at the bf16 bar (1e-2 of the output RMS) and
with each other within 1e-4 of the RMS, not bit for bit: each run measures
about 3e-5 of the RMS from the oracle (bf16 hi + lo products, fp32 sums), and
two orders of the same sums can differ by twice that.  The counters must come back to zero after every call, so these
tests reuse one workspace across calls, batch sizes, graph replays and the
sparse call.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from synth import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

TAU = 1e-2
RERUN = 1e-4


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


def counters(ws):
    """The counter region: exit counter, then (claimed, parts, permits,
    pcount) per sequence."""
    c = ws[:8448].view(torch.int32).cpu().numpy()
    return c[0], c[4:].reshape(-1, 4)


def step_for(inp, ws=None, flags=None):
    import mla_paged_decode_amd as mla
    from mla_paged_decode_amd.step import DecodeStep, DeviceBatch
    flags = mla.MLA_DECODE_DYNAMIC_SPLIT if flags is None else flags
    st = DecodeStep(DeviceBatch.upload(inp), q_abs_dtype=mla.MLA_F32, flags=flags)
    if ws is not None:
        assert ws.numel() >= st.params.workspace_bytes
        st.workspace = ws
        st.params.workspace = ws.data_ptr()
    return st


CASES = [
    ("ragged_b256_h20_ctx512_8k_bf16", dict(batch=40, lens=("uniform", 1, 3000))),
    ("glm_b32_h20_ctx4096_bf16", dict(batch=6, lens=("fixed", (1, 31, 32, 33, 100, 2049)))),
    ("glm_b32_h20_ctx4096_bf16", dict(batch=8, heads=5, q_per_seq=4, lens=("fixed", (0, 1, 3, 4, 5, 17, 64, 900)))),
    ("glm_b32_h20_ctx4096_bf16", dict(batch=3, heads=40, lens=("fixed", (700, 64, 1500)))),
    ("long_b4_h20_ctx65k_203k_bf16", dict(batch=2, lens=("fixed", (9000, 20000)))),
]


@pytest.mark.parametrize("name,over", CASES)
def test_dynamic_split_matches_oracle_and_static(name, over):
    import mla_paged_decode_amd as mla
    wl = WORKLOADS[name].with_(num_splits=0, **over)
    inp = make_inputs(wl, poison_tail=True)
    mla.mla_validate_tables(inp.seq_lens, inp.block_table, inp.kv_pool.shape[0], wl.page_block)
    say(f"[dyn] {name} {over}")
    ref, ref_lse = oracle.mla_decode(inp)
    outs = []
    for flags in (mla.MLA_DECODE_DYNAMIC_SPLIT, 0):
        st = step_for(inp, flags=flags)
        st.out.fill_(float("nan"))
        st.run()
        torch.cuda.synchronize()
        out, lse = st.out.cpu().numpy(), st.lse.cpu().numpy()
        e = rel(out, ref)
        say(f"  flags={flags} rel err {e:.3e}")
        assert e <= TAU
        fin = np.isfinite(ref_lse)
        assert np.array_equal(np.isneginf(lse), np.isneginf(ref_lse))
        assert np.max(np.abs(lse[fin] - ref_lse[fin]), initial=0.0) <= 1e-3
        outs.append(out)
        if flags:
            ex, c = counters(st.workspace)
            assert ex == 0 and (c[:wl.batch, :3] == 0).all(), "counters not reset"
            # every non-empty sequence was merged from at least one part
            L = inp.seq_lens
            assert ((c[:wl.batch, 3] > 0) == (L > 0)).all()
    assert rel(outs[0], outs[1]) <= RERUN


def test_repeated_calls_and_batch_changes_share_one_workspace():
    """One workspace through calls of 40, 7 and 40 sequences, three times
    each: every call matches its own oracle result, and the counters are zero
    after each call."""
    import mla_paged_decode_amd as mla
    wl = WORKLOADS["ragged_b256_h20_ctx512_8k_bf16"].with_(num_splits=0, lens=("uniform", 1, 2500))
    big, small = make_inputs(wl.with_(batch=40)), make_inputs(wl.with_(batch=7, seed=3))
    refs = {id(big): oracle.mla_decode(big)[0], id(small): oracle.mla_decode(small)[0]}
    st_big = step_for(big)
    ws = st_big.workspace
    for rnd in range(3):
        for inp in (big, small, big):
            st = step_for(inp, ws)
            st.out.fill_(float("nan"))
            st.run()
            torch.cuda.synchronize()
            e = rel(st.out.cpu().numpy(), refs[id(inp)])
            say(f"  round {rnd} B={inp.wl.batch}: rel err {e:.3e}")
            assert e <= TAU
            ex, c = counters(ws)
            assert ex == 0 and (c[:, :3] == 0).all()


def test_graph_replays_of_the_dynamic_split():
    """A captured step replayed several times, with eager calls on the same
    workspace between replays: every replay stays within re-association of
    the eager result and within the bar of the oracle."""
    import mla_paged_decode_amd as mla
    from mla_paged_decode_amd.step import DecodeStep, DeviceBatch
    wl = WORKLOADS["ragged_b256_h20_ctx512_8k_bf16"].with_(batch=24, lens=("uniform", 1, 3000), num_splits=0)
    inp = make_inputs(wl)
    ref = oracle.mla_decode(inp)[0]
    step = DecodeStep(DeviceBatch.upload(inp), q_abs_dtype=mla.MLA_F32, flags=mla.MLA_DECODE_DYNAMIC_SPLIT)
    eager = step.run().clone()
    torch.cuda.synchronize()
    assert rel(eager.cpu().numpy(), ref) <= TAU
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step.run()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step.run()
    for rep in range(4):
        step.out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        got = step.out.cpu().numpy()
        assert rel(got, eager.cpu().numpy()) <= RERUN, rep
        assert rel(got, ref) <= TAU, rep
        step.run()  # eager work on the same workspace between replays
        torch.cuda.synchronize()
    ex, c = counters(step.workspace)
    assert ex == 0 and (c[:, :3] == 0).all()


def test_sparse_call_between_dense_calls_on_one_workspace():
    """The sparse call's partials live after the counter region, so a
    workspace can serve both calls in turn."""
    import mla_paged_decode_amd as mla
    from mla_paged_decode_amd.step import DecodeStep, DeviceBatch
    wl = WORKLOADS["glm_b32_h20_ctx4096_bf16"].with_(batch=4, lens=("fixed", (300, 1029, 64, 517)), num_splits=0)
    inp = make_inputs(wl)
    ref = oracle.mla_decode(inp)[0]
    dev = DeviceBatch.upload(inp)
    step = DecodeStep(dev, q_abs_dtype=mla.MLA_F32, flags=mla.MLA_DECODE_DYNAMIC_SPLIT)
    step.run()
    torch.cuda.synchronize()
    assert rel(step.out.cpu().numpy(), ref) <= TAU
    width = 256
    topk = np.full((wl.batch, 1, width), -1, dtype=np.int32)
    rng = np.random.default_rng(4)
    for b in range(wl.batch):
        L = int(inp.seq_lens[b])
        k = min(width, L)
        topk[b, 0, :k] = rng.choice(L, size=k, replace=False)
    o_sp = torch.empty_like(step.o_latent)
    p = mla.make_decode_params(
        dims=dev.dims, batch=wl.batch, q_per_seq=1, q_abs=step.q_abs, kv_pool=dev.kv_pool,
        kv_format=dev.kv_format, num_pages=dev.kv_pool.shape[0], page_block=dev.page_block,
        block_table=dev.block_table, max_blocks_per_seq=dev.block_table.shape[1], seq_lens=dev.seq_lens,
        softmax_scale=dev.softmax_scale, num_splits=2, o_latent=o_sp, lse=None, q_abs_dtype=mla.MLA_F32)
    need = mla.mla_decode_sparse_workspace_size(p, width)
    ws = step.workspace if step.workspace.numel() >= need else torch.zeros(need, dtype=torch.uint8, device="cuda")
    ws[:8448].zero_()
    p.workspace, p.workspace_bytes = ws.data_ptr(), ws.numel()
    step.workspace, step.params.workspace, step.params.workspace_bytes = ws, ws.data_ptr(), ws.numel()
    mla.mla_decode_sparse_paged(p, torch.from_numpy(topk).cuda(), width)
    for _ in range(2):
        step.out.fill_(float("nan"))
        step.run()
        torch.cuda.synchronize()
        assert rel(step.out.cpu().numpy(), ref) <= TAU
