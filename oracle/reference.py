"""CPU oracle for MLA decode over a paged latent cache (test infrastructure).

This module is test infrastructure.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import it; the GPU library never does, and
this module imports nothing from the GPU library.

It computes the plain definition in float64 with numpy.  The method is the
multi-head latent attention of DeepSeek-V2 as used by GLM-4.7-Flash (model
record "GLM-4.7-Flash": the attention is MLA with kv_a_proj_with_mqa and
kv_b_proj; "SERVICEABILITY JOIN": the cache holds a shared low-rank latent
plus a decoupled RoPE key, not per-head K/V).  For head h, with kv_b_proj
viewed per head as rows [W_UK^h (d_nope rows); W_UV^h (d_v rows)] over the
latent width d_c:

    K^h_t = [ W_UK^h c_t , k^R_t ]      (query head 192 + 64 = 256 wide)
    V^h_t =   W_UV^h c_t                (value head 256 wide)
    s_t   = scale * < q^h , K^h_t >
    o^h   = sum_t softmax(s)_t V^h_t ,  lse^h = log sum_t exp(s_t)

The record's "head_dim FILLED = 256" paragraph fixes the query head as
qk_nope 192 + qk_rope 64 and the value head as 256.  The row order (latent
first, then the RoPE key) follows kv_a_proj_with_mqa's output of
4*128 + 64 rows on the page "vllm.models.glm5next.common.model" (block-FP8
dequant helper), where the RoPE rows follow the kv_lora_rank rows.

Readings where the pages are silent (each listed in the design notes):
  * kv_b_proj is stored [H][d_nope + d_v][d_latent], key rows first.
  * RoPE is already applied to q^R and to the cached k^R.
  * seq_lens include the Sq new tokens; query j of a sequence of length L
    sees cached tokens 0 .. L - Sq + j (causal among the Sq new tokens).
  * a query row that sees no token returns o = 0 and lse = -inf.
  * lse is the natural log.

The fp8 row is 512 e4m3fn values (latent and RoPE dims alike) followed by one
e8m0 scale per 32 values (model record "GLM-4.7-Flash", ENGINE KERNEL
CONSTRAINTS item (2): 528 bytes per token).  Decoded value = e4m3fn(code) *
2^(E - 127), with both codes decoded below from their format definitions.

Parity pins live in tests/test_oracle_pins.py.  The pages print no numeric
MLA output for any input, so no stored value comes from them; the function is
pinned by closed forms, invariances, brute force on tiny inputs and a
reduction to a library attention routine.
"""
from __future__ import annotations

import math
from typing import Iterable, Optional

import numpy as np

FP8_BLOCK = 32
FP4_BLOCK = 16  # values per e4m3 scale of the 288-byte fp4 row


# ---------------------------------------------------------------- formats --

def row_bytes(kv_format: str, d_latent: int, d_rope: int) -> int:
    """Stored bytes per cached token: (d_latent + d_rope) values at 4 or 2
    bytes, or for fp8 one byte per value plus one scale byte per 32 values."""
    n = d_latent + d_rope
    if kv_format == "f32":
        return n * 4
    if kv_format == "bf16":
        return n * 2
    if kv_format == "fp8_e4m3_e8m0":
        assert n % FP8_BLOCK == 0
        return n + n // FP8_BLOCK
    if kv_format == "fp4_e2m1_e4m3":
        assert n % FP4_BLOCK == 0
        return n // 2 + n // FP4_BLOCK
    raise ValueError(kv_format)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 is the upper half of an IEEE binary32."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def e4m3fn_value(code: int) -> float:
    """OCP e4m3fn: 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent 0
    is subnormal (m/8 * 2^-6); S.1111.111 is NaN; there is no infinity."""
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return s * (m / 8.0) * 2.0 ** -6
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def e8m0_value(code: int) -> float:
    """OCP e8m0 scale: 2^(E - 127); E = 255 is NaN."""
    if code == 0xFF:
        return math.nan
    return 2.0 ** (code - 127)


def e2m1_value(code: int) -> float:
    """OCP e2m1 (fp4): 1 sign, 2 exponent (bias 1), 1 mantissa bit; exponent 0
    is subnormal (m/2); magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6."""
    s = -1.0 if code & 0x8 else 1.0
    e, m = (code >> 1) & 0x3, code & 0x1
    if e == 0:
        return s * m * 0.5
    return s * (1.0 + m / 2.0) * 2.0 ** (e - 1)


_E4M3 = np.array([e4m3fn_value(c) for c in range(256)], dtype=np.float64)
_E2M1 = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
_E8M0 = np.array([e8m0_value(c) for c in range(256)], dtype=np.float64)


def decode_rows(rows: np.ndarray, kv_format: str, d_latent: int, d_rope: int) -> np.ndarray:
    """Stored rows uint8 [..., row_bytes] -> float64 [..., d_latent + d_rope]."""
    n = d_latent + d_rope
    rows = np.ascontiguousarray(rows, dtype=np.uint8)
    assert rows.shape[-1] == row_bytes(kv_format, d_latent, d_rope)
    if kv_format == "f32":
        return rows.view(np.float32).astype(np.float64)
    if kv_format == "bf16":
        return bf16_to_f64(rows.view(np.uint16))
    if kv_format == "fp4_e2m1_e4m3":
        codes = rows[..., :n // 2]
        lo, hi = _E2M1[codes & 0xF], _E2M1[codes >> 4]  # value 2i in the low nibble of byte i
        vals = np.stack([lo, hi], axis=-1).reshape(rows.shape[:-1] + (n,))
        scales = _E4M3[rows[..., n // 2:]]
        return vals * np.repeat(scales, FP4_BLOCK, axis=-1)
    vals = _E4M3[rows[..., :n]]
    scales = _E8M0[rows[..., n:]]
    return vals * np.repeat(scales, FP8_BLOCK, axis=-1)


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """A stored q / weight tensor (bf16 bits or float32) as float64."""
    if dtype == "bf16":
        return bf16_to_f64(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(dtype)


# ----------------------------------------------------------------- paging --

def sequence_rows(inp, b: int, length: int) -> np.ndarray:
    """Decoded cache rows of logical tokens 0..length-1 of sequence b.

    Token t lives in page block_table[b][t // P] at slot t % P."""
    wl = inp.wl
    P = wl.page_block
    t = np.arange(length)
    pages = inp.block_table[b, t // P]
    assert (pages >= 0).all() and (pages < inp.kv_pool.shape[0]).all()
    raw = inp.kv_pool[pages, t % P]
    return decode_rows(raw, wl.kv_format, wl.d_latent, wl.d_rope)


# -------------------------------------------------------------- attention --

def _softmax_attend(s: np.ndarray, V: np.ndarray):
    """Textbook softmax over scores s [T] applied to values V [T, d]:
    returns (sum_t p_t V_t, log sum_t exp(s_t))."""
    m = s.max()
    e = np.exp(s - m)
    z = e.sum()
    return (e / z) @ V, m + math.log(z)


def _visible(L: int, Sq: int, j: int) -> int:
    """Number of cached tokens query j (0-based of Sq) may attend to."""
    return L - Sq + 1 + j


def mla_decode(inp, seqs: Optional[Iterable[int]] = None,
               heads: Optional[Iterable[int]] = None):
    """Unabsorbed MLA decode.  Rebuilds per-head K and V through kv_b_proj for
    every visible token and runs two-pass softmax attention.

    Returns out float64 [B*Sq, H, d_v] and lse float64 [B*Sq, H]; entries of
    sequences/heads not selected are NaN."""
    wl = inp.wl
    B, Sq, H = wl.batch, wl.q_per_seq, wl.heads
    dn, dr, dc, dv = wl.d_nope, wl.d_rope, wl.d_latent, wl.d_v
    q = to_f64(inp.q, wl.q_dtype)            # [B*Sq, H, dn + dr]
    W = to_f64(inp.w_kv_b, wl.w_dtype)       # [H, dn + dv, dc]
    out = np.full((B * Sq, H, dv), np.nan)
    lse = np.full((B * Sq, H), np.nan)
    seqs = range(B) if seqs is None else list(seqs)
    heads = range(H) if heads is None else list(heads)
    for b in seqs:
        L = int(inp.seq_lens[b])
        rows = sequence_rows(inp, b, max(L, 0))
        C, KR = rows[:, :dc], rows[:, dc:]
        for h in heads:
            W_UK, W_UV = W[h, :dn, :], W[h, dn:, :]
            K = np.concatenate([C @ W_UK.T, KR], axis=1)   # [L, dn + dr]
            V = C @ W_UV.T                                 # [L, dv]
            for j in range(Sq):
                n = b * Sq + j
                T = _visible(L, Sq, j)
                if T <= 0:
                    out[n, h], lse[n, h] = 0.0, -math.inf
                    continue
                s = wl.softmax_scale * (K[:T] @ q[n, h])
                out[n, h], lse[n, h] = _softmax_attend(s, V[:T])
    return out, lse


def mla_decode_sparse(inp, topk: np.ndarray, seqs: Optional[Iterable[int]] = None):
    """Unabsorbed MLA decode over listed tokens (the sparse top-k path of the
    vLLM API page for vllm.models.glm5next.common.model: a per-token buffer of
    top-k cached-token indices, padded, padded slots masked).  Query j of
    sequence b attends to the cached tokens topk[b, j, :] (logical positions);
    entries < 0 or past its causal limit L - Sq + j are padding.  Each listed
    entry is one score (a position listed twice counts twice).  A query with
    no listed token gets out = 0, lse = -inf.

    Returns out float64 [B*Sq, H, d_v] and lse float64 [B*Sq, H] (NaN for
    sequences not selected)."""
    wl = inp.wl
    B, Sq, H = wl.batch, wl.q_per_seq, wl.heads
    dn, dc, dv = wl.d_nope, wl.d_latent, wl.d_v
    topk = np.asarray(topk).reshape(B, Sq, -1)
    q = to_f64(inp.q, wl.q_dtype)
    W = to_f64(inp.w_kv_b, wl.w_dtype)
    out = np.full((B * Sq, H, dv), np.nan)
    lse = np.full((B * Sq, H), np.nan)
    for b in (range(B) if seqs is None else list(seqs)):
        L = int(inp.seq_lens[b])
        rows = sequence_rows(inp, b, max(L, 0))
        C, KR = rows[:, :dc], rows[:, dc:]
        for h in range(H):
            W_UK, W_UV = W[h, :dn, :], W[h, dn:, :]
            K = np.concatenate([C @ W_UK.T, KR], axis=1)
            V = C @ W_UV.T
            for j in range(Sq):
                n = b * Sq + j
                limit = L - Sq + j
                idx = [int(t) for t in topk[b, j] if 0 <= t <= limit]
                if not idx:
                    out[n, h], lse[n, h] = 0.0, -math.inf
                    continue
                s = wl.softmax_scale * (K[idx] @ q[n, h])
                out[n, h], lse[n, h] = _softmax_attend(s, V[idx])
    return out, lse


# ---- the three steps of the absorbed form, each by its own definition ----

def absorb_q(q: np.ndarray, w: np.ndarray, d_nope: int):
    """q [N, H, d_nope + d_rope], w [H, d_nope + d_v, d_c] (float64) ->
    q_abs [N, H, d_c + d_rope] = [ (W_UK^h)^T q^N , q^R ]."""
    W_UK = w[:, :d_nope, :]                                  # [H, dn, dc]
    q_lat = np.einsum("hkc,nhk->nhc", W_UK, q[..., :d_nope])
    return np.concatenate([q_lat, q[..., d_nope:]], axis=-1)


def latent_attention(q_abs: np.ndarray, inp, seqs: Optional[Iterable[int]] = None):
    """Softmax attention of q_abs [B*Sq, H, d_c + d_rope] over the cached rows
    [c_t, k^R_t] with values c_t.  Returns o_lat [B*Sq, H, d_c], lse."""
    wl = inp.wl
    B, Sq, H, dc = wl.batch, wl.q_per_seq, wl.heads, wl.d_latent
    o = np.full((B * Sq, H, dc), np.nan)
    lse = np.full((B * Sq, H), np.nan)
    seqs = range(B) if seqs is None else list(seqs)
    for b in seqs:
        L = int(inp.seq_lens[b])
        rows = sequence_rows(inp, b, max(L, 0))
        for j in range(Sq):
            n = b * Sq + j
            T = _visible(L, Sq, j)
            for h in range(H):
                if T <= 0:
                    o[n, h], lse[n, h] = 0.0, -math.inf
                    continue
                s = wl.softmax_scale * (rows[:T] @ q_abs[n, h])
                o[n, h], lse[n, h] = _softmax_attend(s, rows[:T, :dc])
    return o, lse


def out_proj(o_lat: np.ndarray, w: np.ndarray, d_nope: int):
    """o_lat [N, H, d_c], w [H, d_nope + d_v, d_c] -> out [N, H, d_v] = W_UV^h o."""
    W_UV = w[:, d_nope:, :]                                  # [H, dv, dc]
    return np.einsum("hvc,nhc->nhv", W_UV, o_lat)


def combine_partials(o_parts: np.ndarray, lse_parts: np.ndarray):
    """Merge attention results over disjoint token sets: with partials
    (o_s, lse_s), lse = log sum_s exp(lse_s) and o = sum_s exp(lse_s - lse) o_s.
    Parts with lse_s = -inf carry no weight; if all are -inf the result is
    o = 0, lse = -inf.  o_parts [S, ..., d], lse_parts [S, ...]."""
    m = np.max(lse_parts, axis=0)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    w = np.where(np.isfinite(lse_parts), np.exp(lse_parts - m_safe), 0.0)
    z = w.sum(axis=0)
    lse = np.where(finite, m_safe + np.log(np.where(finite, z, 1.0)), -np.inf)
    o = np.where(finite[..., None],
                 (w[..., None] * np.nan_to_num(o_parts)).sum(axis=0) / np.where(finite, z, 1.0)[..., None],
                 0.0)
    return o, lse


# ------------------------------------------------------------ cache write --
# Storing new tokens' rows in the cache's row formats: f32 as is, bf16 by
# rounding to the nearest bfloat16, and the fp8 row of the model record
# "GLM-4.7-Flash" (ENGINE KERNEL CONSTRAINTS (2): 512 e4m3 values, RoPE dims
# included, plus one e8m0 scale per 32 values, 528 B per token).  The
# record fixes the layout but not how a scale is chosen; the reading taken
# here is the smallest power of two that brings the block's largest
# magnitude within the largest e4m3fn value, 448, and round to nearest with
# ties to even for the codes.  Each step below is the definition searched
# out directly, with no bit tricks.

_E4M3_NONNEG = _E4M3[:127]  # codes 0..126: 0 and the positive finite values, increasing


def e8m0_for_block(amax: float) -> int:
    """Scale code of a block: the smallest E in [0, 254] with
    amax <= 448 * 2^(E - 127); 127 (scale 1) for an all-zero block."""
    if amax == 0.0:
        return 127
    for E in range(255):
        if amax <= 448.0 * 2.0 ** (E - 127):
            return E
    return 254


def e4m3fn_nearest(x: float) -> int:
    """Code of the e4m3fn value nearest to x (|x| <= 448), ties to the code
    whose last (mantissa) bit is 0; the sign bit is x's (so -0.0 -> 0x80)."""
    mag = abs(float(x))
    assert mag <= 448.0
    c = int(np.searchsorted(_E4M3_NONNEG, mag))  # first code with value >= mag
    if c == 0:
        best = 0
    else:
        lo, hi = c - 1, c
        d_lo, d_hi = mag - _E4M3_NONNEG[lo], _E4M3_NONNEG[hi] - mag
        if d_lo < d_hi:
            best = lo
        elif d_hi < d_lo:
            best = hi
        else:
            best = lo if lo % 2 == 0 else hi
    return best | (0x80 if math.copysign(1.0, float(x)) < 0 else 0)


def bf16_nearest(x) -> int:
    """Bits of the bfloat16 nearest to the float32 value x (finite), ties to
    the even bit pattern; the sign is x's."""
    u = int(np.asarray(x, dtype=np.float32).view(np.uint32))
    sign, t = (u >> 16) & 0x8000, (u & 0x7FFFFFFF) >> 16
    mag = abs(float(np.float32(x)))
    lo, hi = float(bf16_to_f64(np.uint16(t))), float(bf16_to_f64(np.uint16(t + 1)))
    if mag - lo < hi - mag:
        best = t
    elif hi - mag < mag - lo:
        best = t + 1
    else:
        best = t if t % 2 == 0 else t + 1
    return sign | best


_E4M3_POS_FINITE = _E4M3[1:127]  # codes 1..126, the positive finite values


def e4m3_scale_for_fp4(amax: float) -> int:
    """Scale code of a 16-value fp4 block: the smallest positive e4m3fn value s
    with amax <= 6 * s (6 is the largest e2m1 magnitude); 448 (0x7E) if none
    is large enough (the values then saturate at +-6), 1.0 (0x38) for an
    all-zero block."""
    if amax == 0.0:
        return 0x38
    for c in range(1, 127):
        if amax <= 6.0 * _E4M3[c]:
            return c
    return 0x7E


def e2m1_nearest(x: float) -> int:
    """fp4 code of the e2m1 value nearest to x, ties to the even code, |x|
    clamped to 6; the sign bit is x's."""
    mag = min(abs(float(x)), 6.0)
    best = min(range(8), key=lambda c: (abs(_E2M1[c] - mag), c % 2))
    return best | (0x8 if math.copysign(1.0, float(x)) < 0 else 0)


def encode_row_fp4(vals) -> np.ndarray:
    """One row (a multiple of 16 values) -> the fp4 row: two e2m1 codes per
    byte (value 2i in the low nibble), then one e4m3 scale per 16 values.  A
    value is stored as the nearest e2m1 to fl32(value / scale), the quotient
    rounded once to float32 as the kernel computes it."""
    vals = np.asarray(vals, dtype=np.float64)
    codes, scales = [], []
    for k in range(vals.size // FP4_BLOCK):
        block = vals[k * FP4_BLOCK:(k + 1) * FP4_BLOCK]
        sc = e4m3_scale_for_fp4(float(np.max(np.abs(block))))
        scales.append(sc)
        s32 = np.float32(_E4M3[sc])
        codes.extend(e2m1_nearest(float(np.float32(v) / s32)) for v in block)
    packed = [codes[2 * i] | (codes[2 * i + 1] << 4) for i in range(len(codes) // 2)]
    return np.array(packed + scales, dtype=np.uint8)


def encode_row(vals, kv_format: str) -> np.ndarray:
    """One row of values (float64, exactly the f32 / bf16 input) -> stored bytes."""
    vals = np.asarray(vals, dtype=np.float64)
    if kv_format == "f32":
        return vals.astype(np.float32).view(np.uint8)
    if kv_format == "bf16":
        return np.array([bf16_nearest(v) for v in vals], dtype=np.uint16).view(np.uint8)
    if kv_format == "fp4_e2m1_e4m3":
        return encode_row_fp4(vals)
    assert kv_format == "fp8_e4m3_e8m0" and vals.size % FP8_BLOCK == 0
    codes, scales = [], []
    for k in range(vals.size // FP8_BLOCK):
        block = vals[k * FP8_BLOCK:(k + 1) * FP8_BLOCK]
        E = e8m0_for_block(float(np.max(np.abs(block))))
        scales.append(E)
        codes.extend(e4m3fn_nearest(v / 2.0 ** (E - 127)) for v in block)
    return np.array(codes + scales, dtype=np.uint8)


def cache_write(pool: np.ndarray, rows: np.ndarray, rows_dtype: str, slots, kv_format: str) -> np.ndarray:
    """A copy of pool ([num_pages][page_block][row_bytes] uint8) with row i
    of rows ([n][d_latent + d_rope], stored as rows_dtype) encoded at token
    slot slots[i] = page * page_block + offset; slots outside
    [0, num_pages * page_block) leave the pool unchanged for that row."""
    out = np.array(pool, dtype=np.uint8, copy=True)
    flat = out.reshape(-1, out.shape[-1])
    vals = to_f64(rows, rows_dtype)
    for i, s in enumerate(np.asarray(slots, dtype=np.int64)):
        if 0 <= s < flat.shape[0]:
            flat[s] = encode_row(vals[i], kv_format)
    return out
