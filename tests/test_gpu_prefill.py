"""mla_prefill_paged on the GPU against the oracle's unabsorbed definition.

The oracle's mla_decode is the unabsorbed form itself: per head it rebuilds
K = [C W_UK^T, K^R] and V = C W_UV^T for every visible token and runs a
two-pass softmax for each of the Sq new tokens, causally.  A prefill chunk is
that computation with Sq in the tens to hundreds, so the oracle serves as is.
The prefill is fp32 throughout (products and sums in fp32 FMAs over at most a
few thousand terms), held to 1e-4 of the output RMS and 1e-4 on the lse, the
bar of the other fp32 path.  Rows past each sequence's end are NaN-poisoned,
so a read past L shows.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from synth import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu
TAU = 1e-4


def run_prefill(inp):
    import mla_paged_decode_amd as mla
    from mla_paged_decode_amd.step import DeviceBatch
    wl = inp.wl
    dev = DeviceBatch.upload(inp)
    N, H = wl.n_tokens, wl.heads
    out = torch.full((N, H, wl.d_v), float("nan"), device="cuda")
    lse = torch.full((N, H), float("nan"), device="cuda")
    params = mla.make_prefill_params(
        dims=dev.dims, batch=wl.batch, q_per_seq=wl.q_per_seq, q=dev.q, w_kv_b=dev.w_kv_b,
        kv_pool=dev.kv_pool, kv_format=dev.kv_format, num_pages=dev.kv_pool.shape[0],
        page_block=dev.page_block, block_table=dev.block_table, max_blocks_per_seq=dev.block_table.shape[1],
        seq_lens=dev.seq_lens, softmax_scale=dev.softmax_scale, out=out, lse=lse)
    nbytes = mla.mla_prefill_workspace_size(params)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
    params.workspace, params.workspace_bytes = ws.data_ptr(), nbytes
    print(f"prefill {wl.kv_format} B={wl.batch} Sq={wl.q_per_seq} H={H} lens={list(inp.seq_lens)}", flush=True)
    mla.mla_prefill_paged(params)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def check(got, glse, ref, rlse):
    rms = math.sqrt(float(np.mean(ref ** 2)))
    err = float(np.max(np.abs(got - ref))) / rms
    print(f"  max|d|/rms = {err:.3e}", flush=True)
    assert err <= TAU
    assert np.array_equal(np.isneginf(glse), np.isneginf(rlse))
    fin = np.isfinite(rlse)
    assert np.max(np.abs(glse[fin] - rlse[fin]), initial=0.0) <= 1e-4


@pytest.mark.parametrize("name,sq,lens,kv", [
    ("glm_b32_h20_ctx4096_bf16", 37, (37, 300, 129), None),
    ("glm_b32_h20_ctx4096_bf16", 64, (64, 1000), None),
    ("glm_b32_h20_ctx4096_bf16", 20, (20, 170), "f32"),
    ("tiny_b2_h4_f32", 16, (16, 77), None),
    ("fp8_mtp4_b64_h20_ctx16k", 24, (24, 200, 65), None),
])
def test_prefill_matches_oracle(name, sq, lens, kv):
    """Chunks that are the whole sequence (L = Sq) and chunks after a
    cached context, block boundaries and ragged tails.  bf16 weights rebuild
    K and V on the matrix cores (bf16, fp8 and fp4 latents exact in bf16, an
    f32 latent split into hi + lo); f32 weights (the tiny case) on the
    vector ALUs.  The attention (256-wide keys and values) runs on the matrix
    cores with every operand split into bf16 hi + lo."""
    wl = WORKLOADS[name].with_(batch=len(lens), q_per_seq=sq, lens=("fixed", lens))
    if kv is not None:
        wl = wl.with_(kv_format=kv)
    inp = make_inputs(wl, poison_tail=True)
    got, glse = run_prefill(inp)
    ref, rlse = oracle.mla_decode(inp)
    check(got, glse, ref, rlse)


def test_prefill_narrow_heads_on_the_vector_alus():
    """Keys and values narrower than 256 (d_nope 128, d_v 128): the
    attention runs on the vector-ALU kernel."""
    wl = WORKLOADS["glm_b32_h20_ctx4096_bf16"].with_(batch=2, heads=6, d_nope=128, d_v=128, q_per_seq=40,
                                                      lens=("fixed", (40, 333)))
    inp = make_inputs(wl, poison_tail=True)
    got, glse = run_prefill(inp)
    ref, rlse = oracle.mla_decode(inp)
    check(got, glse, ref, rlse)


def test_prefill_fp4_cache_and_short_sequence():
    """The fp4 row, and a sequence shorter than the chunk (its first queries
    see nothing: out = 0, lse = -inf)."""
    from synth.gen import Inputs
    base = make_inputs(WORKLOADS["fp8_mtp4_b64_h20_ctx16k"].with_(batch=2, q_per_seq=20, kv_format="f32",
                                                                  lens=("fixed", (150, 12))))
    vals = oracle.decode_rows(base.kv_pool, "f32", base.wl.d_latent, base.wl.d_rope)
    pool = np.stack([oracle.encode_row(v, "fp4_e2m1_e4m3") for v in vals.reshape(-1, vals.shape[-1])])
    pool = pool.reshape(base.kv_pool.shape[0], base.kv_pool.shape[1], 288)
    inp = Inputs(wl=base.wl.with_(kv_format="fp4_e2m1_e4m3"), q=base.q, w_kv_b=base.w_kv_b, kv_pool=pool,
                 block_table=base.block_table, seq_lens=base.seq_lens)
    got, glse = run_prefill(inp)
    ref, rlse = oracle.mla_decode(inp)
    assert np.all(np.isneginf(rlse[20:28])) and np.all(ref[20:28] == 0)
    check(got, glse, ref, rlse)
