"""Pins of the oracle's unabsorbed definition at prefill-chunk sizes (CPU).

The prefill call reads a chunk of Sq new tokens as the last Sq of the L
cached ones, query i at position L - Sq + i (the chunked-prefill reading).
These pins tie that reading, at chunk sizes in the tens, to torch's
scaled_dot_product_attention (float64, CPU) with its own causal masks, and
to single-query decode over the truncated sequence.
"""
import math

import numpy as np
import torch

import oracle
from tests.helpers import inputs_from_rows


def _identity_case(seed, L, Sq, d=16, dr=8, scale=0.23):
    """H = 1, d_c = d_nope = d_v = d, W_UK = W_UV = I: the rebuilt key is
    [c_t, k^R_t] and the value c_t."""
    g = np.random.default_rng(seed)
    rows = [g.standard_normal((L, d + dr)).astype(np.float32)]
    q = g.standard_normal((Sq, 1, d + dr)).astype(np.float32)
    w = np.concatenate([np.eye(d), np.eye(d)])[None].astype(np.float32)
    inp = inputs_from_rows(rows, q, w, page_block=8, q_per_seq=Sq, scale=scale, d_rope=dr)
    K = torch.from_numpy(rows[0].astype(np.float64))
    Q = torch.from_numpy(q[:, 0].astype(np.float64))
    return inp, Q, K, K[:, :d], scale


def test_whole_sequence_chunk_is_causal_sdpa():
    """L = Sq: query i sees keys 0..i, torch's is_causal mask exactly."""
    inp, Q, K, V, scale = _identity_case(31, L=40, Sq=40)
    out, lse = oracle.mla_decode(inp)
    ref = torch.nn.functional.scaled_dot_product_attention(Q[None], K[None], V[None], is_causal=True,
                                                           scale=scale)[0]
    np.testing.assert_allclose(out[:, 0], ref.numpy(), rtol=0, atol=1e-13)
    for i in (0, 17, 39):
        want = torch.logsumexp(scale * (K[:i + 1] @ Q[i]), dim=0).item()
        assert abs(lse[i, 0] - want) < 1e-12


def test_chunk_after_context_uses_the_offset_causal_mask():
    """L = 70, Sq = 24: query i sees keys 0..46 + i (a boolean mask for
    SDPA, built from the positions, not from the oracle)."""
    L, Sq = 70, 24
    inp, Q, K, V, scale = _identity_case(32, L=L, Sq=Sq)
    out, _ = oracle.mla_decode(inp)
    pos = torch.arange(L)[None, :]
    qpos = (L - Sq + torch.arange(Sq))[:, None]
    ref = torch.nn.functional.scaled_dot_product_attention(Q[None], K[None], V[None], attn_mask=pos <= qpos,
                                                           scale=scale)[0]
    np.testing.assert_allclose(out[:, 0], ref.numpy(), rtol=0, atol=1e-13)


def test_chunk_query_equals_single_decode_of_the_prefix():
    """Query i of a 32-token chunk over L = 50 equals a one-query decode of
    the first 50 - 32 + i + 1 tokens (random kv_b_proj, 3 heads)."""
    g = np.random.default_rng(33)
    dc, dr, dn, dv, H, L, Sq = 32, 8, 12, 10, 3, 50, 32
    rows = [g.standard_normal((L, dc + dr)).astype(np.float32)]
    q = g.standard_normal((Sq, H, dn + dr)).astype(np.float32)
    w = (g.standard_normal((H, dn + dv, dc)) / math.sqrt(dc)).astype(np.float32)
    kw = dict(page_block=4, scale=0.3, d_latent=dc, d_rope=dr)
    out, lse = oracle.mla_decode(inputs_from_rows(rows, q, w, q_per_seq=Sq, **kw))
    for i in (0, 5, 31):
        Li = L - Sq + i + 1
        o1, l1 = oracle.mla_decode(inputs_from_rows([rows[0][:Li].copy()], q[i:i + 1].copy(), w, q_per_seq=1, **kw))
        np.testing.assert_allclose(o1[0], out[i], rtol=0, atol=1e-14)
        np.testing.assert_allclose(l1[0], lse[i], rtol=0, atol=1e-14)
