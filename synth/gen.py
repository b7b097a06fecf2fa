"""Seeded input generator: queries, kv_b_proj weights and a paged latent cache.

Shapes follow the GLM-4.7-Flash model record ("GLM-4.7-Flash", the config
facts at the top of the record): kv_lora_rank 512, qk_rope_head_dim 64,
qk_nope_head_dim 192, v_head_dim 256, context up to 202,752 tokens.  The
cache row is the shared latent followed by the decoupled RoPE key (same
record, "SERVICEABILITY JOIN"); the fp8 row is 512 e4m3 values (RoPE dims
included) plus one e8m0 scale byte per 32 values, 528 B per token (same
record, "ENGINE KERNEL CONSTRAINTS", item (2)).  Page-block sizes 16..128 come
from item (1) there and from the vLLM pull request "fix: Add glm4_moe_lite to
MLA detection" (Summary: CUTLASS_MLA enforces block_size 128).  Four query
tokens per sequence model the MTP verify step of the SGLang pull request
"[Fix] GLM 4.7 + NVFP4 + MTP" (Benchmarking and Profiling: accept length /
accept rate is about 4).

Random draws: every tensor has its own numpy Generator seeded from
SeedSequence(seed, spawn_key=(tag,)).  q, the latent and the RoPE key are
N(0, 1); kv_b_proj is N(0, 1/512).  Values are drawn in float32 and rounded to
the storage type with round-to-nearest-even.

Nothing here computes attention.  The fp8 encoder below only produces test
inputs in the stored format; decoding them is the consumer's job.
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

# Tags that separate the per-tensor random streams.
_TAG_Q, _TAG_W, _TAG_KV, _TAG_LENS, _TAG_PERM = 1, 2, 3, 4, 5

KV_FORMATS = ("f32", "bf16", "fp8_e4m3_e8m0")
FP8_BLOCK = 32  # values per e8m0 scale
_CHUNK_ROWS = 16384  # rows per independently seeded pool chunk


@dataclass(frozen=True)
class Workload:
    """One decode step's shape.  `lens` is ("fixed", (L0, L1, ...)),
    ("const", L) or ("uniform", lo, hi) with both ends inclusive."""

    name: str
    batch: int
    heads: int
    q_per_seq: int
    d_latent: int
    d_rope: int
    d_nope: int
    d_v: int
    page_block: int
    kv_format: str
    q_dtype: str
    w_dtype: str
    lens: tuple
    shared_prefix: float = 0.0
    num_splits: int = 0
    softmax_scale: float = 1.0 / 16.0
    permute_pages: bool = True
    seed: int = 0

    @property
    def n_tokens(self) -> int:
        return self.batch * self.q_per_seq

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    # Tiny fp32 case: batch 2, 4 heads, lengths 37 and 64, page block 16.
    "tiny_b2_h4_f32": Workload(
        name="tiny_b2_h4_f32", batch=2, heads=4, q_per_seq=1, d_latent=512,
        d_rope=64, d_nope=192, d_v=256, page_block=16, kv_format="f32",
        q_dtype="f32", w_dtype="f32", lens=("fixed", (37, 64))),
    # One GLM-4.7-Flash layer: batch 32, 20 heads, 4096 tokens each, bf16,
    # page block 64, randomly permuted block table.
    "glm_b32_h20_ctx4096_bf16": Workload(
        name="glm_b32_h20_ctx4096_bf16", batch=32, heads=20, q_per_seq=1,
        d_latent=512, d_rope=64, d_nope=192, d_v=256, page_block=64,
        kv_format="bf16", q_dtype="bf16", w_dtype="bf16", lens=("const", 4096)),
    # Long context: batch 4, lengths uniform in [65536, 202752], page block
    # 64, 32 uniform split-KV chunks per sequence.
    "long_b4_h20_ctx65k_203k_bf16": Workload(
        name="long_b4_h20_ctx65k_203k_bf16", batch=4, heads=20, q_per_seq=1,
        d_latent=512, d_rope=64, d_nope=192, d_v=256, page_block=64,
        kv_format="bf16", q_dtype="bf16", w_dtype="bf16",
        lens=("uniform", 65536, 202752), num_splits=32),
    # Large ragged batch: 256 sequences, lengths uniform in [512, 8192], page
    # block 128, about 10% of block-table entries on a shared prefix chain.
    "ragged_b256_h20_ctx512_8k_bf16": Workload(
        name="ragged_b256_h20_ctx512_8k_bf16", batch=256, heads=20,
        q_per_seq=1, d_latent=512, d_rope=64, d_nope=192, d_v=256,
        page_block=128, kv_format="bf16", q_dtype="bf16", w_dtype="bf16",
        lens=("uniform", 512, 8192), shared_prefix=0.10),
    # fp8 latent + 4 MTP query tokens: batch 64, 16384 tokens each; the 528-B
    # row holds 448 latent + 64 RoPE e4m3 values and 16 e8m0 scales.
    "fp8_mtp4_b64_h20_ctx16k": Workload(
        name="fp8_mtp4_b64_h20_ctx16k", batch=64, heads=20, q_per_seq=4,
        d_latent=448, d_rope=64, d_nope=192, d_v=256, page_block=64,
        kv_format="fp8_e4m3_e8m0", q_dtype="bf16", w_dtype="bf16",
        lens=("const", 16384)),
}


@dataclass
class Inputs:
    """Host buffers for one decode step, in their stored formats.

    q            [B*Sq, H, d_nope+d_rope]  uint16 (bf16 bits) or float32
    w_kv_b       [H, d_nope+d_v, d_latent] uint16 (bf16 bits) or float32
    kv_pool      [num_pages, page_block, row_bytes] uint8
    block_table  [B, max_blocks] int32, -1 for unused entries
    seq_lens     [B] int32, each including the Sq new tokens
    """

    wl: Workload
    q: np.ndarray
    w_kv_b: np.ndarray
    kv_pool: np.ndarray
    block_table: np.ndarray
    seq_lens: np.ndarray

    @property
    def num_pages(self) -> int:
        return int(self.kv_pool.shape[0])

    @property
    def row_bytes(self) -> int:
        return int(self.kv_pool.shape[2])


def _rng(seed: int, tag: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(entropy=seed, spawn_key=(tag,)))


def stored_row_bytes(kv_format: str, d_latent: int, d_rope: int) -> int:
    """Bytes of one stored cache row (latent then RoPE key)."""
    n = d_latent + d_rope
    if kv_format == "f32":
        return 4 * n
    if kv_format == "bf16":
        return 2 * n
    if kv_format == "fp8_e4m3_e8m0":
        return n + n // FP8_BLOCK
    if kv_format == "fp4_e2m1_e4m3":  # two 4-bit codes per byte, one scale byte per 16 values
        return n // 2 + n // 16
    raise ValueError(f"unknown kv format {kv_format!r}")


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return the bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    out = (rounded >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def _e4m3_encode(a: np.ndarray) -> np.ndarray:
    """Encode values already within [-448, 448] as e4m3fn codes, rounding to
    nearest with ties to even."""
    a = np.asarray(a, dtype=np.float64)
    sign = np.signbit(a).astype(np.uint8) << 7
    mag = np.minimum(np.abs(a), 448.0)
    # Binade exponent floor(log2(mag)), clamped at the normal minimum 2^-6;
    # below it the step is the subnormal quantum 2^-9.
    _, ex = np.frexp(mag)
    e = np.maximum(ex - 1, -6)
    r = np.rint(np.ldexp(mag, 3 - e))           # mantissa steps of 2^(e-3)
    r = np.minimum(np.ldexp(r, e - 3), 448.0)
    mr, exr = np.frexp(r)                       # r = mr * 2^exr, mr in [0.5, 1)
    normal = r >= 2.0 ** -6
    exp_field = np.where(normal, exr - 1 + 7, 0)
    mant = np.where(normal, mr * 16.0 - 8.0, np.ldexp(r, 9))
    code = (exp_field.astype(np.uint8) << 3) | np.rint(mant).astype(np.uint8)
    code = np.where(r == 0, 0, code).astype(np.uint8)
    return code | sign


def quantize_e4m3_e8m0(vals: np.ndarray):
    """Quantise rows of values (last axis a multiple of 32) to e4m3fn codes with
    one e8m0 scale byte per 32 values.  The scale is the smallest power of two
    that brings the block's largest magnitude to at most 448.  Returns
    (codes uint8 [..., n], scales uint8 [..., n/32])."""
    vals = np.asarray(vals, dtype=np.float32)
    n = vals.shape[-1]
    assert n % FP8_BLOCK == 0
    blocks = vals.reshape(vals.shape[:-1] + (n // FP8_BLOCK, FP8_BLOCK)).astype(np.float64)
    amax = np.abs(blocks).max(axis=-1)
    ratio = np.where(amax > 0, amax / 448.0, 1.0)
    m, ex = np.frexp(ratio)  # ratio = m * 2^ex, m in [0.5, 1)
    k = np.where(m > 0.5, ex, ex - 1)  # ceil(log2(ratio))
    k = np.clip(k, -127, 127)
    scales = (k + 127).astype(np.uint8)
    scaled = blocks / np.exp2(k)[..., None]
    codes = _e4m3_encode(scaled).reshape(vals.shape)
    return codes, scales


def _encode_rows(vals: np.ndarray, kv_format: str) -> np.ndarray:
    """vals float32 [..., d_latent + d_rope] -> stored bytes [..., row_bytes]."""
    if kv_format == "f32":
        return np.ascontiguousarray(vals, dtype=np.float32).view(np.uint8)
    if kv_format == "bf16":
        return bf16_bits_from_f32(vals).view(np.uint8)
    codes, scales = quantize_e4m3_e8m0(vals)
    return np.concatenate([codes, scales], axis=-1)


def _draw_lens(wl: Workload) -> np.ndarray:
    kind = wl.lens[0]
    if kind == "fixed":
        lens = np.asarray(wl.lens[1], dtype=np.int64)
        assert len(lens) == wl.batch
    elif kind == "const":
        lens = np.full(wl.batch, wl.lens[1], dtype=np.int64)
    elif kind == "uniform":
        lo, hi = wl.lens[1], wl.lens[2]
        lens = _rng(wl.seed, _TAG_LENS).integers(lo, hi + 1, size=wl.batch)
    else:
        raise ValueError(kind)
    return lens.astype(np.int32)


def _store(vals: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(vals, dtype=np.float32)
    if dtype == "bf16":
        return bf16_bits_from_f32(vals)
    raise ValueError(dtype)


def make_inputs(
    wl: Workload,
    *,
    seq_lens: Optional[Sequence[int]] = None,
    poison_tail: bool = False,
    max_blocks: Optional[int] = None,
) -> Inputs:
    """Draw one decode step's inputs for workload `wl`.

    seq_lens     overrides the drawn lengths (len must equal wl.batch).
    poison_tail  fills the unused slots of each sequence's last page with NaN
                 codes, so a consumer that reads past a sequence's end shows it.
    max_blocks   block-table width (default: the longest sequence's pages).
    """
    B, H, Sq, P = wl.batch, wl.heads, wl.q_per_seq, wl.page_block
    lens = _draw_lens(wl) if seq_lens is None else np.asarray(seq_lens, dtype=np.int32)
    assert lens.shape == (B,)

    q = _rng(wl.seed, _TAG_Q).standard_normal((B * Sq, H, wl.d_nope + wl.d_rope), dtype=np.float32)
    w = _rng(wl.seed, _TAG_W).standard_normal((H, wl.d_nope + wl.d_v, wl.d_latent), dtype=np.float32)
    w *= np.float32(1.0 / math.sqrt(512.0))

    # Block tables: logical pages are [shared prefix chain] + [each sequence's
    # private pages]; a seeded permutation maps them to physical page ids.
    n_blk = (lens.astype(np.int64) + P - 1) // P
    if wl.shared_prefix > 0:
        shared = np.floor(wl.shared_prefix * n_blk + 0.5).astype(np.int64)
        shared = np.minimum(shared, np.maximum(n_blk - 1, 0))
    else:
        shared = np.zeros(B, dtype=np.int64)
    chain = int(shared.max()) if B else 0
    private = n_blk - shared
    num_pages = chain + int(private.sum())
    num_pages = max(num_pages, 1)
    if wl.permute_pages:
        phys = _rng(wl.seed, _TAG_PERM).permutation(num_pages).astype(np.int32)
    else:
        phys = np.arange(num_pages, dtype=np.int32)
    width = int(n_blk.max()) if B else 1
    width = max(width, 1) if max_blocks is None else max_blocks
    assert width >= (int(n_blk.max()) if B else 0)
    table = np.full((B, width), -1, dtype=np.int32)
    off = chain
    for b in range(B):
        s, p = int(shared[b]), int(private[b])
        table[b, :s] = phys[:s]
        table[b, s:s + p] = phys[off:off + p]
        off += p

    # Pool contents: the flattened rows are drawn in fixed chunks, each chunk
    # from its own seeded stream, so the result does not depend on threading.
    d_row = wl.d_latent + wl.d_rope
    rb = stored_row_bytes(wl.kv_format, wl.d_latent, wl.d_rope)
    pool = np.empty((num_pages, P, rb), dtype=np.uint8)
    flat = pool.reshape(num_pages * P, rb)
    n_rows = num_pages * P

    def fill(i: int) -> None:
        r0, r1 = i * _CHUNK_ROWS, min(n_rows, (i + 1) * _CHUNK_ROWS)
        g = np.random.default_rng(np.random.SeedSequence(entropy=wl.seed, spawn_key=(_TAG_KV, i)))
        vals = g.standard_normal((r1 - r0, d_row), dtype=np.float32)
        flat[r0:r1] = _encode_rows(vals, wl.kv_format)

    n_chunks = (n_rows + _CHUNK_ROWS - 1) // _CHUNK_ROWS
    with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        list(ex.map(fill, range(n_chunks)))

    if poison_tail:
        for b in range(B):
            L = int(lens[b])
            if L % P and n_blk[b] > 0:
                page = table[b, n_blk[b] - 1]
                tail = pool[page, L % P:]
                if wl.kv_format == "f32":
                    tail.view(np.float32)[...] = np.nan
                elif wl.kv_format == "bf16":
                    tail.view(np.uint16)[...] = 0x7FC0
                else:
                    tail[...] = 0x7F  # e4m3fn NaN code
                    tail[:, d_row:] = 0xFF  # e8m0 NaN

    return Inputs(
        wl=wl,
        q=_store(q, wl.q_dtype),
        w_kv_b=_store(w, wl.w_dtype),
        kv_pool=pool,
        block_table=table,
        seq_lens=lens,
    )


def make_q_abs(wl: Workload, *, seed: Optional[int] = None) -> np.ndarray:
    """Absorbed queries [B*Sq, H, d_latent + d_rope] float32 for exercising
    the decode step on its own: the latent part is N(0, d_nope/512) (the
    spread of W_UK^T q for the weights above), the RoPE part N(0, 1)."""
    g = _rng(wl.seed if seed is None else seed, 6)
    N = wl.batch * wl.q_per_seq
    lat = g.standard_normal((N, wl.heads, wl.d_latent), dtype=np.float32)
    lat *= np.float32(math.sqrt(wl.d_nope / 512.0))
    rope = g.standard_normal((N, wl.heads, wl.d_rope), dtype=np.float32)
    return np.ascontiguousarray(np.concatenate([lat, rope], axis=-1))


def make_o_latent(wl: Workload, *, seed: Optional[int] = None) -> np.ndarray:
    """Latent attention outputs [B*Sq, H, d_latent] float32, N(0, 1/64), for
    exercising the value up-projection on its own."""
    g = _rng(wl.seed if seed is None else seed, 7)
    N = wl.batch * wl.q_per_seq
    return g.standard_normal((N, wl.heads, wl.d_latent), dtype=np.float32) * np.float32(0.125)
