"""The C++ oracle (oracle/mla_oracle.cpp) against the numpy oracle.

Both compute the unabsorbed definition in double precision, written
independently (C++ loops with OpenMP; numpy matmuls).  They must agree to
rounding: max |out_cpp - out_py| <= 1e-12 * RMS(out_py) and |lse| within
1e-12, with identical -inf rows.  A closed form pins the C++ side on its
own: a sequence of one token gives out = W_UV c_0 and lse = s_0.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import native
from synth import WORKLOADS, make_inputs
from synth.gen import Inputs


@pytest.fixture(scope="module", autouse=True)
def _built():
    native.build()


def compare(inp, seqs=None):
    ref, rlse = oracle.mla_decode(inp, seqs=seqs)
    got, glse = native.mla_decode(inp, seqs=seqs)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    sel = ~np.isnan(ref)
    rms = math.sqrt(float(np.mean(ref[sel] ** 2)))
    err = float(np.max(np.abs(got[sel] - ref[sel]))) / rms
    assert err <= 1e-12, err
    assert np.array_equal(np.isneginf(glse), np.isneginf(rlse))
    fin = np.isfinite(rlse)
    assert np.max(np.abs(glse[fin] - rlse[fin]), initial=0.0) <= 1e-12
    return err


def fp4_inputs(lens, q_per_seq=1):
    wl32 = WORKLOADS["fp8_mtp4_b64_h20_ctx16k"].with_(batch=len(lens), heads=3, q_per_seq=q_per_seq,
                                                       lens=("fixed", tuple(lens)), kv_format="f32")
    base = make_inputs(wl32)
    vals = oracle.decode_rows(base.kv_pool, "f32", wl32.d_latent, wl32.d_rope)
    pool = np.stack([oracle.encode_row(v, "fp4_e2m1_e4m3") for v in vals.reshape(-1, vals.shape[-1])])
    pool = pool.reshape(base.kv_pool.shape[0], base.kv_pool.shape[1], 288)
    return Inputs(wl=wl32.with_(kv_format="fp4_e2m1_e4m3"), q=base.q, w_kv_b=base.w_kv_b, kv_pool=pool,
                  block_table=base.block_table, seq_lens=base.seq_lens)


@pytest.mark.parametrize("name,over", [
    ("tiny_b2_h4_f32", {}),
    ("glm_b32_h20_ctx4096_bf16", dict(batch=4, heads=5, lens=("fixed", (1, 33, 200, 517)))),
    ("ragged_b256_h20_ctx512_8k_bf16", dict(batch=3, heads=4, lens=("fixed", (0, 129, 300)))),
    ("fp8_mtp4_b64_h20_ctx16k", dict(batch=5, heads=4, lens=("fixed", (0, 2, 4, 65, 300)))),
    ("glm_b32_h20_ctx4096_bf16", dict(batch=2, heads=3, q_dtype="f32", w_dtype="f32", page_block=16,
                                      lens=("fixed", (47, 90)))),
])
def test_native_matches_numpy_oracle(name, over):
    compare(make_inputs(WORKLOADS[name].with_(**over)))


def test_native_matches_numpy_oracle_fp4():
    compare(fp4_inputs((3, 70), q_per_seq=2))


def test_native_selected_sequences_only():
    inp = make_inputs(WORKLOADS["glm_b32_h20_ctx4096_bf16"].with_(batch=4, heads=2, lens=("fixed", (5, 6, 7, 8))))
    compare(inp, seqs=[1, 3])


def test_native_single_token_closed_form():
    """L = 1: the softmax has one term, so out = W_UV c_0 and lse = s_0."""
    wl = WORKLOADS["glm_b32_h20_ctx4096_bf16"].with_(batch=1, heads=3, lens=("fixed", (1,)))
    inp = make_inputs(wl)
    got, glse = native.mla_decode(inp)
    row = oracle.decode_rows(inp.kv_pool[inp.block_table[0, 0], 0], "bf16", wl.d_latent, wl.d_rope)
    c, kr = row[:wl.d_latent], row[wl.d_latent:]
    q = oracle.bf16_to_f64(inp.q)[0]
    w = oracle.bf16_to_f64(inp.w_kv_b)
    for h in range(wl.heads):
        v = w[h, wl.d_nope:] @ c
        s = wl.softmax_scale * (q[h, :wl.d_nope] @ (w[h, :wl.d_nope] @ c) + q[h, wl.d_nope:] @ kr)
        assert np.allclose(got[0, h], v, rtol=1e-13, atol=1e-13 * np.abs(v).max())
        assert abs(glse[0, h] - s) <= 1e-12 * max(1.0, abs(s))


def test_native_rejects_bad_tables():
    inp = make_inputs(WORKLOADS["glm_b32_h20_ctx4096_bf16"].with_(batch=2, heads=2, lens=("fixed", (70, 10))))
    inp.block_table[0, 1] = inp.kv_pool.shape[0]
    with pytest.raises(ValueError):
        native.mla_decode(inp)
