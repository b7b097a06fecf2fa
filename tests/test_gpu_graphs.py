"""The sparse decode, prefill and cache-append calls captured into HIP graphs.

Serving loops replay captured graphs; none of these calls allocates, and
none records a memset.  Each call is captured once and replayed several
times, with eager work and synchronisations between the replays, and every
replay must equal the eager result bit for bit.
"""
import numpy as np
import pytest
import torch

import mla_paged_decode_amd as mla
from synth import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu


def capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def test_sparse_decode_graph_replays():
    from mla_paged_decode_amd.step import DeviceBatch
    wl = WORKLOADS["fp8_mtp4_b64_h20_ctx16k"].with_(batch=3, lens=("fixed", (300, 90, 513)))
    inp = make_inputs(wl)
    dev = DeviceBatch.upload(inp)
    N, H = wl.n_tokens, wl.heads
    q_abs = torch.empty((N, H, wl.d_latent + wl.d_rope), dtype=torch.bfloat16, device="cuda")
    mla.mla_absorb_q(dev.dims, N, dev.q, dev.w_kv_b, q_abs)
    rng = np.random.default_rng(5)
    topk = np.full((wl.batch, wl.q_per_seq, 128), -1, dtype=np.int32)
    for b in range(wl.batch):
        for j in range(wl.q_per_seq):
            lim = int(inp.seq_lens[b]) - wl.q_per_seq + j
            k = min(100, lim + 1)
            topk[b, j, :k] = rng.choice(lim + 1, size=k, replace=False)
    topk_t = torch.from_numpy(topk).cuda()
    o = torch.empty((N, H, wl.d_latent), device="cuda")
    lse = torch.empty((N, H), device="cuda")
    params = mla.make_decode_params(
        dims=dev.dims, batch=wl.batch, q_per_seq=wl.q_per_seq, q_abs=q_abs, kv_pool=dev.kv_pool,
        kv_format=dev.kv_format, num_pages=dev.kv_pool.shape[0], page_block=dev.page_block,
        block_table=dev.block_table, max_blocks_per_seq=dev.block_table.shape[1], seq_lens=dev.seq_lens,
        softmax_scale=dev.softmax_scale, num_splits=2, o_latent=o, lse=lse, q_abs_dtype=mla.MLA_BF16)
    nbytes = mla.mla_decode_sparse_workspace_size(params, 128)
    ws = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device="cuda")
    params.workspace, params.workspace_bytes = ws.data_ptr(), nbytes
    print("sparse decode graph (fp8 rows, matrix cores)", flush=True)
    mla.mla_decode_sparse_paged(params, topk_t, 128)
    torch.cuda.synchronize()
    o_eager, lse_eager = o.clone(), lse.clone()
    g = capture(lambda: mla.mla_decode_sparse_paged(params, topk_t, 128))
    for rep in range(3):
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_eager), rep
        assert torch.equal(lse, lse_eager), rep
        mla.mla_decode_sparse_paged(params, topk_t, 128)  # eager work between replays
        torch.cuda.synchronize()


def test_prefill_graph_replays():
    from mla_paged_decode_amd.step import DeviceBatch
    wl = WORKLOADS["glm_b32_h20_ctx4096_bf16"].with_(batch=2, q_per_seq=48, lens=("fixed", (48, 300)))
    inp = make_inputs(wl)
    dev = DeviceBatch.upload(inp)
    N, H = wl.n_tokens, wl.heads
    out = torch.empty((N, H, wl.d_v), device="cuda")
    lse = torch.empty((N, H), device="cuda")
    params = mla.make_prefill_params(
        dims=dev.dims, batch=wl.batch, q_per_seq=wl.q_per_seq, q=dev.q, w_kv_b=dev.w_kv_b, kv_pool=dev.kv_pool,
        kv_format=dev.kv_format, num_pages=dev.kv_pool.shape[0], page_block=dev.page_block,
        block_table=dev.block_table, max_blocks_per_seq=dev.block_table.shape[1], seq_lens=dev.seq_lens,
        softmax_scale=dev.softmax_scale, out=out, lse=lse)
    nbytes = mla.mla_prefill_workspace_size(params)
    ws = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device="cuda")
    params.workspace, params.workspace_bytes = ws.data_ptr(), nbytes
    print("prefill graph (matrix cores)", flush=True)
    mla.mla_prefill_paged(params)
    torch.cuda.synchronize()
    out_eager, lse_eager = out.clone(), lse.clone()
    g = capture(lambda: mla.mla_prefill_paged(params))
    for rep in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        ws.fill_(0xFF)  # the workspace needs no initialisation: replays rebuild it
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, out_eager), rep
        assert torch.equal(lse, lse_eager), rep
        mla.mla_prefill_paged(params)
        torch.cuda.synchronize()


def test_cache_write_graph_replays():
    dims = mla.Dims(20, 448, 64, 192, 256)
    rng = np.random.default_rng(6)
    rows = torch.from_numpy(rng.standard_normal((64, 512)).astype(np.float32)).cuda()
    slots = torch.from_numpy(rng.permutation(8 * 64)[:64].astype(np.int64)).cuda()
    pool0 = torch.from_numpy(rng.integers(0, 256, (8, 64, 528), dtype=np.uint8)).cuda()
    pool = pool0.clone()
    print("cache write graph (fp8 rows)", flush=True)
    mla.mla_cache_write(dims, 64, rows, slots, pool, mla.MLA_KV_FP8_E4M3_E8M0, 8, 64)
    torch.cuda.synchronize()
    want = pool.clone()
    g = capture(lambda: mla.mla_cache_write(dims, 64, rows, slots, pool, mla.MLA_KV_FP8_E4M3_E8M0, 8, 64))
    for rep in range(3):
        pool.copy_(pool0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(pool, want), rep
