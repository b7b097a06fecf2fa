"""Pins of the CPU oracle against facts that do not come from the oracle.

Each test names what it pins: values the pages print (tests/golden), library
routines that implement the same mathematics independently (torch's fp8 and
bf16 casts, torch's scaled_dot_product_attention and logsumexp), closed forms
of softmax attention, invariances of paging and of the causal MTP mask, and
brute force on tiny inputs.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from synth import WORKLOADS, make_inputs, stored_row_bytes
from tests.helpers import inputs_from_rows


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ------------------------------------------------- layout and byte counts --

def test_row_bytes_match_page_figures(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "page_invariants.json")))
    dc, dr = g["kv_lora_rank"], g["qk_rope_head_dim"]
    assert dc + dr == g["values_per_token_per_layer"] == 576
    assert sum(g["kv_a_proj_rows_split"]) == g["kv_a_proj_rows"] == dc + dr
    bf16 = oracle.row_bytes("bf16", dc, dr)
    assert bf16 * g["num_layers"] == g["bf16_bytes_per_token_all_layers"]
    assert round(bf16 * g["num_layers"] / 1024, 1) == g["bf16_kib_per_token_all_layers_1dp"]
    # fp8: 512 e4m3 values over all dims (RoPE included) + one e8m0 per 32.
    n8 = g["fp8_e4m3_values"]
    assert n8 // g["fp8_values_per_scale"] == g["fp8_scale_bytes"]
    assert oracle.row_bytes("fp8_e4m3_e8m0", n8 - dr, dr) == g["fp8_row_bytes"]
    assert g["qk_nope_head_dim"] + dr == g["query_head_width"] == g["v_head_dim"]
    # The generator lays rows out with the same sizes.
    for fmt, dl in (("f32", 512), ("bf16", 512), ("fp8_e4m3_e8m0", 448)):
        assert stored_row_bytes(fmt, dl, dr) == oracle.row_bytes(fmt, dl, dr)


def test_e4m3fn_all_codes_match_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = np.array([oracle.e4m3fn_value(c) for c in range(256)])
    nan = np.isnan(ref)
    assert (np.isnan(ours) == nan).all() and nan.sum() == 2  # 0x7F and 0xFF
    assert (ours[~nan] == ref[~nan]).all()
    # spot values of the format: 1.0, max 448, min subnormal 2^-9
    assert ours[0x38] == 1.0 and ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9


def test_e8m0_all_codes_match_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    ours = np.array([oracle.e8m0_value(c) for c in range(256)])
    assert np.isnan(ours[255]) and np.isnan(ref[255])
    assert (ours[:255] == ref[:255]).all()
    assert ours[127] == 1.0


def test_bf16_decode_matches_torch():
    bits = np.arange(0, 65536, 7, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    ours = oracle.bf16_to_f64(bits)
    nan = np.isnan(ref)
    assert (np.isnan(ours) == nan).all()
    assert (ours[~nan] == ref[~nan]).all()


def test_fp8_row_scale_blocks():
    """Scale byte k applies to values [32k, 32k+32): a row of e4m3 1.0 codes
    with scale bytes 120+k decodes to 2^(k-7) in block k."""
    row = np.zeros(528, dtype=np.uint8)
    row[:512] = 0x38
    row[512:] = 120 + np.arange(16)
    vals = oracle.decode_rows(row[None], "fp8_e4m3_e8m0", 448, 64)[0]
    expect = np.repeat(2.0 ** (np.arange(16) - 7), 32)
    assert (vals == expect).all()


def test_fp8_generator_roundtrip_within_half_ulp():
    """Generated fp8 rows decode to within half an e4m3 step of the drawn
    normal values (the generator's quantiser against the oracle's decoder)."""
    wl = WORKLOADS["fp8_mtp4_b64_h20_ctx16k"].with_(batch=1, lens=("const", 64))
    inp = make_inputs(wl)
    vals = oracle.decode_rows(inp.kv_pool.reshape(-1, 528), "fp8_e4m3_e8m0", 448, 64)
    assert np.isfinite(vals).all()
    assert 0.9 < vals.std() < 1.1


# ---------------------------------------------------------- small helpers --

def _rand_case(seed, B=2, H=3, Sq=1, dc=32, dr=8, dn=12, dv=10, lens=(9, 20), P=4, scale=0.3):
    g = np.random.default_rng(seed)
    rows = [g.standard_normal((L, dc + dr)).astype(np.float32) for L in lens]
    q = g.standard_normal((B * Sq, H, dn + dr)).astype(np.float32)
    w = (g.standard_normal((H, dn + dv, dc)) / math.sqrt(dc)).astype(np.float32)
    return rows, q, w, dict(page_block=P, q_per_seq=Sq, scale=scale, d_latent=dc, d_rope=dr)


# --------------------------------------------------- absorbed = unabsorbed --

@pytest.mark.parametrize("Sq", [1, 3])
def test_absorbed_equals_unabsorbed(Sq):
    rows, q, w, kw = _rand_case(1, Sq=Sq, lens=(9, 20))
    inp = inputs_from_rows(rows, q, w, **kw)
    out, lse = oracle.mla_decode(inp)
    q_abs = oracle.absorb_q(q.astype(np.float64), w.astype(np.float64), 12)
    o_lat, lse2 = oracle.latent_attention(q_abs, inp)
    out2 = oracle.out_proj(o_lat, w.astype(np.float64), 12)
    assert _rel(out2, out) < 1e-12
    assert np.max(np.abs(lse2 - lse)) < 1e-12


def test_absorbed_equals_unabsorbed_fp8_rows():
    wl = WORKLOADS["fp8_mtp4_b64_h20_ctx16k"].with_(batch=2, heads=3, lens=("fixed", (70, 5)))
    inp = make_inputs(wl)
    out, lse = oracle.mla_decode(inp)
    q = oracle.to_f64(inp.q, "bf16")
    w = oracle.to_f64(inp.w_kv_b, "bf16")
    o_lat, lse2 = oracle.latent_attention(oracle.absorb_q(q, w, 192), inp)
    out2 = oracle.out_proj(o_lat, w, 192)
    fin = np.isfinite(lse)
    assert _rel(out2, out) < 1e-12
    assert np.max(np.abs(lse2[fin] - lse[fin])) < 1e-12


# ------------------------------------------------------------ brute force --

def test_brute_force_tiny():
    """Scalar loops with exactly rounded sums on a tiny case."""
    rows, q, w, kw = _rand_case(2, B=1, H=2, Sq=2, dc=4, dr=2, dn=3, dv=2, lens=(5,), P=2, scale=0.7)
    inp = inputs_from_rows(rows, q, w, **kw)
    out, lse = oracle.mla_decode(inp)
    r = rows[0].astype(float)
    Q = q.astype(float)
    W = w.astype(float)
    for j in range(2):
        T = 5 - 2 + 1 + j
        for h in range(2):
            s = []
            for t in range(T):
                k_n = [math.fsum(W[h, i, c] * r[t, c] for c in range(4)) for i in range(3)]
                s.append(0.7 * math.fsum([*(Q[j, h, i] * k_n[i] for i in range(3)),
                                          *(Q[j, h, 3 + i] * r[t, 4 + i] for i in range(2))]))
            m = max(s)
            z = math.fsum(math.exp(x - m) for x in s)
            for v in range(2):
                o = math.fsum(math.exp(s[t] - m) / z *
                              math.fsum(W[h, 3 + v, c] * r[t, c] for c in range(4)) for t in range(T))
                assert abs(o - out[j, h, v]) < 1e-13
            assert abs(m + math.log(z) - lse[j, h]) < 1e-13


# ------------------------------------------------------------ closed forms --

def test_single_token_returns_its_value_row():
    rows, q, w, kw = _rand_case(3, B=1, lens=(1,))
    inp = inputs_from_rows(rows, q, w, **kw)
    out, lse = oracle.mla_decode(inp)
    c = rows[0][0, :32].astype(float)
    W = w.astype(float)
    for h in range(3):
        np.testing.assert_allclose(out[0, h], W[h, 12:] @ c, rtol=0, atol=1e-14)
        k = torch.cat([torch.from_numpy(W[h, :12] @ c), torch.from_numpy(rows[0][0, 32:].astype(float))])
        s0 = 0.3 * torch.dot(torch.from_numpy(q[0, h].astype(float)), k).item()
        assert abs(lse[0, h] - s0) < 1e-13


def test_zero_query_gives_mean_value_and_log_count():
    rows, q, w, kw = _rand_case(4, lens=(9, 20))
    q[:] = 0
    inp = inputs_from_rows(rows, q, w, **kw)
    out, lse = oracle.mla_decode(inp)
    W = w.astype(float)
    for b, L in enumerate((9, 20)):
        mean_c = rows[b][:, :32].astype(float).mean(axis=0)
        for h in range(3):
            np.testing.assert_allclose(out[b, h], W[h, 12:] @ mean_c, rtol=0, atol=1e-13)
            assert abs(lse[b, h] - math.log(L)) < 1e-13


def test_identical_rows_ignore_the_query():
    rows, q, w, kw = _rand_case(5, B=1, lens=(13,))
    rows[0][:] = rows[0][0]
    inp = inputs_from_rows(rows, q, w, **kw)
    out, lse = oracle.mla_decode(inp)
    W = w.astype(float)
    c = rows[0][0, :32].astype(float)
    for h in range(3):
        np.testing.assert_allclose(out[0, h], W[h, 12:] @ c, rtol=0, atol=1e-13)


def test_dominant_score_selects_its_row():
    rows, q, w, kw = _rand_case(6, B=1, lens=(17,))
    q[..., 12:] = 0
    q[..., 12] = 1.0
    rows[0][:, 32:] = 0
    rows[0][11, 32] = 4000.0  # k^R of token 11 aligned with q^R, huge score
    inp = inputs_from_rows(rows, q, w, **kw)
    out, lse = oracle.mla_decode(inp)
    W = w.astype(float)
    for h in range(3):
        np.testing.assert_allclose(out[0, h], W[h, 12:] @ rows[0][11, :32].astype(float), atol=1e-12)


def test_nope_equals_no_rope_dims():
    """With q^R = 0 and k^R = 0 the result equals MLA with no RoPE dims."""
    rows, q, w, kw = _rand_case(7, lens=(9, 20))
    for r in rows:
        r[:, 32:] = 0
    q[..., 12:] = 0
    out, lse = oracle.mla_decode(inputs_from_rows(rows, q, w, **kw))
    kw0 = dict(kw, d_rope=0)
    out0, lse0 = oracle.mla_decode(inputs_from_rows([r[:, :32].copy() for r in rows],
                                                    q[..., :12].copy(), w, **kw0))
    assert _rel(out, out0) < 1e-14 and np.max(np.abs(lse - lse0)) < 1e-13


# -------------------------------------------------------------- invariances --

def test_page_permutation_and_page_size_invariance():
    rows, q, w, kw = _rand_case(8, lens=(37, 64))
    base, lse_b = oracle.mla_decode(inputs_from_rows(rows, q, w, **kw))
    for P in (1, 4, 16, 64, 128):
        for seed in (None, 11):
            out, lse = oracle.mla_decode(inputs_from_rows(rows, q, w, **dict(kw, page_block=P), perm_seed=seed))
            assert (out == base).all() and (lse == lse_b).all()


def test_mtp_query_equals_shorter_single_decode():
    """Query j of an Sq=4 decode of length L equals an Sq=1 decode of length
    L-3+j with the same cache and that query row."""
    Sq, L = 4, 23
    rows, q, w, kw = _rand_case(9, B=1, Sq=Sq, lens=(L,))
    out, lse = oracle.mla_decode(inputs_from_rows(rows, q, w, **kw))
    for j in range(Sq):
        Lj = L - Sq + 1 + j
        o1, l1 = oracle.mla_decode(inputs_from_rows([rows[0][:Lj].copy()], q[j:j + 1].copy(), w,
                                                    **dict(kw, q_per_seq=1)))
        np.testing.assert_allclose(o1[0], out[j], rtol=0, atol=1e-14)
        np.testing.assert_allclose(l1[0], lse[j], rtol=0, atol=1e-14)


def test_rows_without_visible_tokens():
    """L = 0 gives o = 0, lse = -inf; with Sq = 4 and L = 2 the first two
    queries see nothing, the third one token, the last two."""
    rows, q, w, kw = _rand_case(10, B=2, Sq=4, lens=(0, 2))
    out, lse = oracle.mla_decode(inputs_from_rows(rows, q, w, **kw))
    assert (out[:4] == 0).all() and np.isneginf(lse[:4]).all()
    assert (out[4:6] == 0).all() and np.isneginf(lse[4:6]).all()
    assert np.isfinite(lse[6:]).all()
    o1, _ = oracle.mla_decode(inputs_from_rows([rows[1][:1].copy()], q[6:7].copy(), w, **dict(kw, q_per_seq=1)))
    np.testing.assert_allclose(o1[0], out[6], rtol=0, atol=1e-14)


# ------------------------------------------- reduction to library attention --

@pytest.mark.parametrize("dr", [0, 8])
def test_identity_weights_reduce_to_sdpa(dr):
    """H = 1, d_c = d_nope = d_v, W_UK = W_UV = I: MLA is single-head softmax
    attention with K = [c, k^R] and V = c (torch SDPA, float64, CPU)."""
    d = 16
    g = np.random.default_rng(12)
    L = 45
    rows = [g.standard_normal((L, d + dr)).astype(np.float32)]
    q = g.standard_normal((1, 1, d + dr)).astype(np.float32)
    w = np.concatenate([np.eye(d), np.eye(d)])[None].astype(np.float32)
    scale = 0.21
    out, lse = oracle.mla_decode(inputs_from_rows(rows, q, w, page_block=8, scale=scale, d_rope=dr))
    K = torch.from_numpy(rows[0].astype(np.float64))
    V = K[:, :d]
    Q = torch.from_numpy(q[0].astype(np.float64))
    ref = torch.nn.functional.scaled_dot_product_attention(Q[None], K[None], V[None], scale=scale)[0, 0]
    np.testing.assert_allclose(out[0, 0], ref.numpy(), rtol=0, atol=1e-13)
    ref_lse = torch.logsumexp(scale * (K @ Q[0]), dim=0).item()
    assert abs(lse[0, 0] - ref_lse) < 1e-12


def test_combine_partials_matches_whole_softmax():
    """Attention over disjoint token sets merged by the log-sum-exp rule
    equals attention over their union (torch SDPA on each part and on all)."""
    g = np.random.default_rng(13)
    K = torch.from_numpy(g.standard_normal((50, 24)))
    V = torch.from_numpy(g.standard_normal((50, 16)))
    Q = torch.from_numpy(g.standard_normal((3, 24)))
    sdpa = torch.nn.functional.scaled_dot_product_attention

    def part(sl):
        o = sdpa(Q[None], K[None, sl], V[None, sl], scale=0.3)[0]
        lse = torch.logsumexp(0.3 * Q @ K[sl].T, dim=1)
        return o.numpy(), lse.numpy()

    whole_o, whole_lse = part(slice(0, 50))
    parts = [part(slice(0, 7)), part(slice(7, 31)), part(slice(31, 50))]
    empty = (np.full((3, 16), np.nan), np.full(3, -np.inf))
    o_parts = np.stack([p[0] for p in parts] + [empty[0]])
    l_parts = np.stack([p[1] for p in parts] + [empty[1]])
    o, lse = oracle.combine_partials(o_parts, l_parts)
    np.testing.assert_allclose(o, whole_o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, whole_lse, rtol=0, atol=1e-13)
    o0, l0 = oracle.combine_partials(np.zeros((2, 3, 16)), np.full((2, 3), -np.inf))
    assert (o0 == 0).all() and np.isneginf(l0).all()


# ---------------------------------------------------- generator structure --

def test_shared_prefix_pages_are_shared_and_private_tail():
    wl = WORKLOADS["ragged_b256_h20_ctx512_8k_bf16"].with_(batch=16)
    inp = make_inputs(wl)
    P = wl.page_block
    n = (inp.seq_lens + P - 1) // P
    s_b = np.minimum(np.floor(0.1 * n + 0.5).astype(int), n - 1)
    top = int(np.argmax(s_b))
    chain = inp.block_table[top, :s_b[top]]
    shared_frac = []
    for b in range(16):
        assert (inp.block_table[b, :s_b[b]] == chain[:s_b[b]]).all()
        # the pages after the prefix, the last one included, are private
        for page in inp.block_table[b, s_b[b]:n[b]]:
            assert (inp.block_table == page).sum() == 1
        shared_frac.append(s_b[b] / n[b])
    assert 0.05 < np.mean(shared_frac) < 0.15
    used = inp.block_table[inp.block_table >= 0]
    assert used.max() < inp.num_pages


def test_shared_prefix_equals_private_copy():
    """A sequence that reads shared prefix pages gives the same result as one
    whose prefix pages are private copies of the same data."""
    wl = WORKLOADS["ragged_b256_h20_ctx512_8k_bf16"].with_(batch=3, heads=2, lens=("fixed", (700, 900, 1300)))
    inp = make_inputs(wl)
    out, lse = oracle.mla_decode(inp)
    # copy every page referenced by sequence 2 into fresh pages
    pool = inp.kv_pool
    n2 = (1300 + 127) // 128
    fresh = np.arange(pool.shape[0], pool.shape[0] + n2)
    pool2 = np.concatenate([pool, pool[inp.block_table[2, :n2]]])
    table2 = inp.block_table.copy()
    table2[2, :n2] = fresh
    inp2 = type(inp)(wl=inp.wl, q=inp.q, w_kv_b=inp.w_kv_b, kv_pool=pool2,
                     block_table=table2, seq_lens=inp.seq_lens)
    out2, lse2 = oracle.mla_decode(inp2)
    assert (out2 == out).all() and (lse2 == lse).all()
