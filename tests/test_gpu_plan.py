"""The balanced split plan, index for index.

In balanced mode (num_splits = 0) the decode kernels compute the plan
themselves (the matrix-core kernels inside the kernel for up to 512
sequences, otherwise a one-workgroup plan kernel) and publish it in the
workspace for the merge: tile_start[0..B+1].  Its definition:

- sequence b of length L_b has n_b = ceil(L_b / 32) tiles, preceded by c
  virtual tiles when L_b > 0 (c is 0 or 4, below);
- tile_start[b] is the exclusive prefix sum of those counts,
  tile_start[B] = N (all positions) and tile_start[B + 1] = c;
- with N0 the number of real tiles and G workers, c = 4 exactly when some
  non-empty sequence starts, in the plan without virtual tiles, strictly
  inside a worker's range [g N0 / G, (g + 1) N0 / G).

The published values are compared with the host's, bit for bit (integer
work).  The host then checks what the kernels and the merge derive from the
plan: worker g owns positions [g N / G, (g + 1) N / G); its real tiles in
sequence b form one unit whose partial goes to slot g + b; every token of
every sequence lies in exactly one unit; slots are unique and below G + B;
and the merge's part range for b (first and last worker holding one of its
real tiles, workers with an empty range skipped) names exactly the workers
that wrote a unit of b.
"""
import sys

import numpy as np
import pytest
import torch

from synth import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

TILE, UNIT_COST = 32, 4
COUNTER_BYTES = 256 + 16 * 512  # counter region in front of tile_start


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_paged_decode_amd as mla
    mla.lib()


def host_plan(lens, G):
    L = np.maximum(np.asarray(lens, dtype=np.int64), 0)
    n = (L + TILE - 1) // TILE
    ne = (L > 0).astype(np.int64)
    p = np.concatenate([[0], np.cumsum(n)[:-1]]).astype(np.int64)   # real tiles before b
    q = np.concatenate([[0], np.cumsum(ne)[:-1]]).astype(np.int64)  # non-empty sequences before b
    N0 = int(n.sum())

    def starts_worker(pos):
        r = (pos * G) % N0
        return r == 0 or N0 - r < G

    crossing = any(L[b] > 0 and p[b] > 0 and not starts_worker(int(p[b])) for b in range(len(L)))
    c = UNIT_COST if crossing else 0
    ts = p + c * q
    return np.concatenate([ts, [N0 + c * int(ne.sum()), c]]).astype(np.int64)


def units_of(ts, lens, G):
    """(worker, b, t0, t1, slot) of every unit, as the kernels walk them."""
    B = len(lens)
    N, c = int(ts[B]), int(ts[B + 1])
    out = []
    for g in range(G):
        tb, te = g * N // G, (g + 1) * N // G
        for b in range(B):
            if ts[b] >= te:
                break
            first = ts[b] + (c if ts[b + 1] > ts[b] else 0)
            s0, s1 = max(tb, first), min(te, int(ts[b + 1]))
            if s0 >= s1:
                continue
            L = max(int(lens[b]), 0)
            out.append((g, b, (s0 - first) * TILE, min(L, (s1 - first) * TILE), g + b))
    return out


def check_host_invariants(ts, lens, G):
    B = len(lens)
    N = int(ts[B])
    units = units_of(ts, lens, G)
    slots = [u[4] for u in units]
    assert len(set(slots)) == len(slots) and (not slots or max(slots) < G + B)
    for b in range(B):
        L = max(int(lens[b]), 0)
        spans = sorted((t0, t1) for (_, bb, t0, t1, _) in units if bb == b)
        pos = 0
        for t0, t1 in spans:  # contiguous, no overlap, no gap
            assert t0 == pos and t1 > t0, (b, spans)
            pos = t1
        assert pos == L, (b, pos, L)
        # the merge's part range
        writers = sorted(g for (g, bb, *_rest) in units if bb == b)
        if L == 0:
            assert not writers
            continue
        first = int(ts[b]) + int(ts[B + 1])
        g0 = ((first + 1) * G - 1) // N
        g1 = (int(ts[b + 1]) * G - 1) // N
        named = [g for g in range(g0, g1 + 1) if g * N // G < (g + 1) * N // G]
        assert writers == named, (b, writers, named)


def published_plan(name, over, kernel, q_abs):
    import mla_paged_decode_amd as mla
    from mla_paged_decode_amd.step import DecodeStep, DeviceBatch
    wl = WORKLOADS[name].with_(num_splits=0, **over)
    inp = make_inputs(wl)
    st = DecodeStep(DeviceBatch.upload(inp), q_abs_dtype=q_abs, kernel=kernel)
    st.workspace.fill_(0xEE)  # no stale plan can pass
    st.workspace[:COUNTER_BYTES].zero_()
    st.run()
    torch.cuda.synchronize()
    B = wl.batch
    ts = st.workspace[COUNTER_BYTES:COUNTER_BYTES + 4 * (B + 2)].view(torch.int32).cpu().numpy()
    return ts.astype(np.int64), np.asarray(inp.seq_lens, dtype=np.int64)


RAGGED, GLM, FP8 = "ragged_b256_h20_ctx512_8k_bf16", "glm_b32_h20_ctx4096_bf16", "fp8_mtp4_b64_h20_ctx16k"
MIX = tuple([0, 1, 31, 32, 33, 64, 65, 0, 2047, 4096, 4097, 7, 0, 96, 3000] * 3)
CASES = [
    # (workload, overrides, kernel, workers, expected c or None)
    (RAGGED, dict(lens=("uniform", 1, 2000)), 2, 512, 4),               # in-kernel plan
    (GLM, {}, 2, 512, 0),                                               # sequences start on worker starts
    (RAGGED, dict(batch=len(MIX), lens=("fixed", MIX)), 2, 512, None),  # empty and one-token sequences
    (RAGGED, dict(batch=8, lens=("uniform", 1, 200)), 2, 512, None),    # fewer tiles than workers
    (RAGGED, dict(batch=600, lens=("uniform", 1, 600)), 2, 512, 4),     # B > 512: the plan kernel
    (RAGGED, dict(batch=len(MIX), lens=("fixed", MIX)), 1, 512, None),  # vector-ALU kernel: the plan kernel
    (FP8, dict(batch=24, lens=("uniform", 1, 5000)), 0, 256, 4),        # MX kernel, one workgroup per CU
]


@pytest.mark.parametrize("name,over,kernel,G,c", CASES)
def test_published_plan_matches_host_plan(name, over, kernel, G, c):
    import mla_paged_decode_amd as mla
    q_abs = mla.MLA_BF16 if name == FP8 else mla.MLA_F32
    say(f"[plan] {name} {over} kernel {kernel} G {G}")
    got, lens = published_plan(name, over, kernel, q_abs)
    want = host_plan(lens, G)
    say(f"  N {want[-2]} c {want[-1]}")
    assert np.array_equal(got, want), (got[:8], want[:8], got[-2:], want[-2:])
    if c is not None:
        assert want[-1] == c
    check_host_invariants(want, lens, G)
