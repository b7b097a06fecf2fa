"""Test helpers: build decode inputs from explicit logical rows."""
from __future__ import annotations

import numpy as np

from synth import Inputs, Workload


def inputs_from_rows(rows, q, w, *, page_block=16, q_per_seq=1, scale=1.0 / 16.0,
                     d_latent=None, d_rope=0, d_nope=None, d_v=None, perm_seed=None,
                     seq_lens=None):
    """rows: list of float arrays [L_b, d_latent + d_rope] (stored as f32);
    q float [B*Sq, H, d_nope + d_rope]; w float [H, d_nope + d_v, d_latent].
    Pages of each sequence are laid out one after another, then optionally
    permuted with a seeded permutation of the physical ids."""
    B = len(rows)
    H = q.shape[1]
    d_latent = w.shape[2] if d_latent is None else d_latent
    d_nope = q.shape[2] - d_rope if d_nope is None else d_nope
    d_v = w.shape[1] - d_nope if d_v is None else d_v
    lens = [r.shape[0] for r in rows] if seq_lens is None else list(seq_lens)
    P = page_block
    n_blk = [(r.shape[0] + P - 1) // P for r in rows]
    num_pages = max(1, sum(n_blk))
    phys = np.arange(num_pages)
    if perm_seed is not None:
        phys = np.random.default_rng(perm_seed).permutation(num_pages)
    width = max(1, max(n_blk))
    table = np.full((B, width), -1, dtype=np.int32)
    d_row = d_latent + d_rope
    pool = np.zeros((num_pages, P, d_row), dtype=np.float32)
    k = 0
    for b, r in enumerate(rows):
        for i in range(n_blk[b]):
            p = phys[k]
            k += 1
            table[b, i] = p
            chunk = r[i * P:(i + 1) * P]
            pool[p, :chunk.shape[0]] = chunk
    wl = Workload(name="explicit", batch=B, heads=H, q_per_seq=q_per_seq,
                  d_latent=d_latent, d_rope=d_rope, d_nope=d_nope, d_v=d_v,
                  page_block=P, kv_format="f32", q_dtype="f32", w_dtype="f32",
                  lens=("fixed", tuple(lens)), softmax_scale=scale)
    return Inputs(wl=wl, q=np.asarray(q, np.float32), w_kv_b=np.asarray(w, np.float32),
                  kv_pool=pool.view(np.uint8).reshape(num_pages, P, d_row * 4),
                  block_table=table, seq_lens=np.asarray(lens, dtype=np.int32))
