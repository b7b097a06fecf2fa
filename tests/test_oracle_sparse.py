"""Pins of the oracle's sparse top-k decode (CPU only).

The vLLM API page for vllm.models.glm5next.common.model describes the sparse
path as attention over a per-token buffer of top-k cached-token indices,
padded to whole tiles with the padded slots masked.  The oracle is pinned to
the dense definition (a full list), to re-paging the listed rows into a
sequence of their own, and to the invariances a list must have.
"""
import numpy as np

import oracle
from synth import WORKLOADS, make_inputs
from tests.helpers import inputs_from_rows


def small(kv="bf16", sq=1, lens=(37, 64, 5)):
    name = "fp8_mtp4_b64_h20_ctx16k" if kv == "fp8_e4m3_e8m0" else "glm_b32_h20_ctx4096_bf16"
    return make_inputs(WORKLOADS[name].with_(batch=len(lens), heads=3, q_per_seq=sq, lens=("fixed", lens)))


def padded(lists, width):
    out = np.full((len(lists), width), -1, dtype=np.int32)
    for i, l in enumerate(lists):
        out[i, :len(l)] = l
    return out


def test_full_list_equals_dense_decode():
    inp = small(sq=2)
    B, Sq = inp.wl.batch, inp.wl.q_per_seq
    lists = [list(range(int(inp.seq_lens[b]))) for b in range(B) for _ in range(Sq)]
    topk = padded(lists, 128).reshape(B, Sq, 128)
    got, glse = oracle.mla_decode_sparse(inp, topk)
    ref, rlse = oracle.mla_decode(inp)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(glse, rlse, rtol=0, atol=1e-12)


def test_listed_rows_equal_a_sequence_of_just_those_rows():
    """Attending to a subset equals dense attention over a new sequence whose
    cache holds only the listed rows (in list order)."""
    inp = small(kv="bf16", lens=(50, 64, 20))
    rng = np.random.default_rng(4)
    B = inp.wl.batch
    lists = [sorted(rng.choice(int(inp.seq_lens[b]), size=int(inp.seq_lens[b]) // 2, replace=False).tolist())
             for b in range(B)]
    got, glse = oracle.mla_decode_sparse(inp, padded(lists, 64).reshape(B, 1, 64))
    wl = inp.wl
    for b in range(B):
        rows = oracle.sequence_rows(inp, b, int(inp.seq_lens[b]))[lists[b]]
        q = oracle.to_f64(inp.q, wl.q_dtype)[b:b + 1]
        w = oracle.to_f64(inp.w_kv_b, wl.w_dtype)
        sub = inputs_from_rows([rows.astype(np.float32)], q.astype(np.float32), w.astype(np.float32),
                               d_rope=wl.d_rope, scale=wl.softmax_scale)
        # rows, q and w are exact in float32 (they came from bf16), so this is the same data
        ref, rlse = oracle.mla_decode(sub)
        np.testing.assert_allclose(got[b], ref[0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(glse[b], rlse[0], rtol=0, atol=1e-12)


def test_order_and_padding_do_not_matter():
    inp = small(lens=(40, 64, 9))
    rng = np.random.default_rng(5)
    B = inp.wl.batch
    lists = [rng.choice(int(inp.seq_lens[b]), size=7, replace=False).tolist() for b in range(B)]
    base, blse = oracle.mla_decode_sparse(inp, padded(lists, 16).reshape(B, 1, 16))
    shuffled = [list(rng.permutation(l)) + [-1, -7, 10**6] for l in lists]
    got, glse = oracle.mla_decode_sparse(inp, padded(shuffled, 16).reshape(B, 1, 16))
    np.testing.assert_allclose(got, base, rtol=0, atol=1e-12)
    np.testing.assert_allclose(glse, blse, rtol=0, atol=1e-12)


def test_mtp_queries_mask_entries_past_their_causal_limit():
    """Query j of Sq = 4 may see tokens up to L - 4 + j: listing the later ones
    changes nothing, and a query whose list is all padding gets 0 and -inf."""
    inp = small(sq=4, lens=(30, 12))
    B, Sq = inp.wl.batch, inp.wl.q_per_seq
    L = inp.seq_lens
    vis = [[list(range(0, int(L[b]) - Sq + j + 1, 2)) for j in range(Sq)] for b in range(B)]
    extra = [[v + list(range(int(L[b]) - Sq + j + 1, int(L[b]))) for j, v in enumerate(vb)] for b, vb in enumerate(vis)]
    a, alse = oracle.mla_decode_sparse(inp, padded(sum(vis, []), 32).reshape(B, Sq, 32))
    c, clse = oracle.mla_decode_sparse(inp, padded(sum(extra, []), 32).reshape(B, Sq, 32))
    np.testing.assert_allclose(c, a, rtol=0, atol=1e-12)
    empty = np.full((B, Sq, 32), -1, dtype=np.int32)
    z, zlse = oracle.mla_decode_sparse(inp, empty)
    assert np.all(z == 0) and np.all(np.isneginf(zlse))


def test_duplicate_entry_counts_twice():
    """Listing a token twice is a softmax with that score twice: for two
    tokens listed as [0, 0, 1] the weights are 2e^s0 : e^s1."""
    inp = small(lens=(10,))
    got, _ = oracle.mla_decode_sparse(inp, np.array([[[0, 0, 1, -1]]], dtype=np.int32))
    full, _ = oracle.mla_decode_sparse(inp, np.array([[[0, -1, -1, -1]]], dtype=np.int32))
    one, _ = oracle.mla_decode_sparse(inp, np.array([[[1, -1, -1, -1]]], dtype=np.int32))
    # recover the two scores' weights from the three results per head: got = w0 V0 + w1 V1
    wl = inp.wl
    q = oracle.to_f64(inp.q, wl.q_dtype)[0]
    W = oracle.to_f64(inp.w_kv_b, wl.w_dtype)
    rows = oracle.sequence_rows(inp, 0, 2)
    for h in range(wl.heads):
        K = np.concatenate([rows[:, :wl.d_latent] @ W[h, :wl.d_nope].T, rows[:, wl.d_latent:]], axis=1)
        s = wl.softmax_scale * (K @ q[h])
        w0 = 2 * np.exp(s[0]) / (2 * np.exp(s[0]) + np.exp(s[1]))
        np.testing.assert_allclose(got[0, h], w0 * full[0, h] + (1 - w0) * one[0, h], rtol=0, atol=1e-12)
