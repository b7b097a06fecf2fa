"""Pins of the oracle's cache-write encoders (CPU only).

The pages fix the fp8 row's layout (model record "GLM-4.7-Flash", ENGINE
KERNEL CONSTRAINTS (2): 512 e4m3 values plus one e8m0 scale per 32 values,
528 B) and the bf16 row; the encoders are pinned here to the format
definitions, to a library conversion and to an independently written
quantiser, so that a wrong rounding, tie rule, scale choice or slot mapping
fails one of them.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle.reference import _E4M3
from synth.gen import quantize_e4m3_e8m0


def test_every_finite_e4m3_code_encodes_to_itself():
    for c in range(256):
        v = oracle.e4m3fn_value(c)
        if math.isnan(v):
            continue
        assert oracle.e4m3fn_nearest(v if c != 0x80 else -0.0) == c, hex(c)


def test_e4m3_midpoints_round_to_the_even_code():
    pos = _E4M3[:127]
    for c in range(126):
        mid = (pos[c] + pos[c + 1]) / 2.0
        even = c if c % 2 == 0 else c + 1
        assert oracle.e4m3fn_nearest(mid) == even, c
        assert oracle.e4m3fn_nearest(-mid) == even | 0x80, c
        # just off the midpoint: the nearer code
        eps = (pos[c + 1] - pos[c]) * 1e-6
        assert oracle.e4m3fn_nearest(mid - eps) == c
        assert oracle.e4m3fn_nearest(mid + eps) == c + 1
    # the subnormal / normal boundary: 15/16 * 2^-6 lies between 7/8 * 2^-6
    # (code 7) and 2^-6 (code 8)
    assert oracle.e4m3fn_nearest(15.0 / 16.0 * 2.0 ** -6) == 8
    # below half the smallest subnormal 2^-9 everything is zero
    assert oracle.e4m3fn_nearest(2.0 ** -11) == 0
    assert oracle.e4m3fn_nearest(-(2.0 ** -11)) == 0x80


def test_e8m0_scale_is_the_smallest_power_that_fits():
    assert oracle.e8m0_for_block(0.0) == 127
    for k in (-100, -7, -1, 0, 1, 5, 80):
        a = 448.0 * 2.0 ** k
        assert oracle.e8m0_for_block(a) == 127 + k
        assert oracle.e8m0_for_block(a * (1 + 2.0 ** -20)) == 128 + k
        assert oracle.e8m0_for_block(a * (1 - 2.0 ** -20)) == 127 + k
    # extremes clamp into the code range
    assert oracle.e8m0_for_block(1e-45) == 0
    assert oracle.e8m0_for_block(3.0e38) == 127 + 120


def test_bf16_nearest_matches_torch_conversion():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(2000).astype(np.float32),
                        (rng.standard_normal(200) * 1e30).astype(np.float32),
                        (rng.standard_normal(200) * 1e-30).astype(np.float32)])
    # exact ties: bf16 value plus half its last place, both parities
    base = torch.from_numpy(rng.standard_normal(200).astype(np.float32)).to(torch.bfloat16)
    bits = base.view(torch.int16).numpy().astype(np.uint16).astype(np.uint32) << 16
    ties = (bits | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, np.float32([0.0, -0.0, 1.0, -3.5])])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    got = np.array([oracle.bf16_nearest(v) for v in x], dtype=np.uint16)
    np.testing.assert_array_equal(got, ref)


def test_fp8_row_encoding_matches_an_independent_quantiser():
    """The generator's quantiser (frexp arithmetic, written separately) and
    the oracle's search give the same bytes."""
    rng = np.random.default_rng(11)
    rows = rng.standard_normal((24, 512)).astype(np.float32)
    rows[1] *= 1e-3
    rows[2] *= 3e4
    rows[3, :32] = 0.0
    rows[4, 32:64] = 448.0 * 2.0 ** 3
    codes, scales = quantize_e4m3_e8m0(rows)
    want = np.concatenate([codes, scales], axis=-1)
    got = np.stack([oracle.encode_row(r.astype(np.float64), "fp8_e4m3_e8m0") for r in rows])
    np.testing.assert_array_equal(got, want)


def test_fp8_round_trip_error_is_at_most_half_a_step():
    rng = np.random.default_rng(12)
    rows = (rng.standard_normal((16, 512)) * np.exp(rng.uniform(-8, 8, (16, 1)))).astype(np.float32)
    for r in rows:
        enc = oracle.encode_row(r.astype(np.float64), "fp8_e4m3_e8m0")
        dec = oracle.decode_rows(enc[None], "fp8_e4m3_e8m0", 448, 64)[0]
        for k in range(16):
            scale = 2.0 ** (int(enc[512 + k]) - 127)
            blk = r[32 * k:32 * (k + 1)].astype(np.float64)
            assert np.max(np.abs(blk)) <= 448 * scale
            # e4m3 spacing at |v|: 2^(floor(log2 |v|) - 3), at least 2^-9
            mag = np.abs(blk) / scale
            step = np.exp2(np.maximum(np.floor(np.log2(np.maximum(mag, 2.0 ** -9))), -6) - 3)
            assert np.all(np.abs(dec[32 * k:32 * (k + 1)] - blk) <= 0.5 * step * scale + 1e-300)


@pytest.mark.parametrize("fmt", ["f32", "bf16", "fp8_e4m3_e8m0", "fp4_e2m1_e4m3"])
def test_cache_write_places_rows_at_their_slots(fmt):
    d_lat = 448 if fmt.startswith("fp") else 512
    rb = oracle.row_bytes(fmt, d_lat, 64)
    P, pages = 16, 5
    pool = np.full((pages, P, rb), 0x5A, dtype=np.uint8)
    rng = np.random.default_rng(3)
    rows = rng.standard_normal((6, d_lat + 64)).astype(np.float32)
    slots = [17, -1, 0, P * pages, 79, 33]  # -1 and one past the end are skipped
    out = oracle.cache_write(pool, rows, "f32", slots, fmt)
    flat = out.reshape(-1, rb)
    written = {17: 0, 0: 2, 79: 4, 33: 5}
    for s in range(P * pages):
        if s in written:
            np.testing.assert_array_equal(flat[s], oracle.encode_row(rows[written[s]].astype(np.float64), fmt))
        else:
            assert np.all(flat[s] == 0x5A)
    dec = oracle.decode_rows(flat[[17, 0, 79, 33]], fmt, d_lat, 64)
    tol = {"f32": 0.0, "bf16": 2.0 ** -8, "fp8_e4m3_e8m0": 2.0 ** -3, "fp4_e2m1_e4m3": 0.5}[fmt]
    ref = rows[[0, 2, 4, 5]].astype(np.float64)
    slack = {"f32": 0, "bf16": 0, "fp8_e4m3_e8m0": 2.0 ** -6, "fp4_e2m1_e4m3": 0.5}[fmt]
    assert np.all(np.abs(dec - ref) <= tol * np.abs(ref) + slack)


# ----------------------------------------------------------- the fp4 row --
# The model record gives an fp4 variant of the cache at 288 bytes per token.
# With 512 values that is 256 bytes of 4-bit codes plus 32 scale bytes, one
# per 16 values; the codes are read as OCP e2m1 and the scales as e4m3fn.

def test_fp4_row_is_288_bytes():
    assert oracle.row_bytes("fp4_e2m1_e4m3", 448, 64) == 288


def test_every_e2m1_code_encodes_to_itself():
    for c in range(16):
        v = oracle.e2m1_value(c)
        assert oracle.e2m1_nearest(v) == c, c


def test_e2m1_midpoints_round_to_the_even_code():
    mags = [oracle.e2m1_value(c) for c in range(8)]
    for c in range(7):
        mid = (mags[c] + mags[c + 1]) / 2
        even = c if c % 2 == 0 else c + 1
        assert oracle.e2m1_nearest(mid) == even
        assert oracle.e2m1_nearest(-mid) == even | 0x8
    assert oracle.e2m1_nearest(100.0) == 7  # saturates at 6


def test_fp4_scale_is_the_smallest_e4m3_that_fits():
    for c in (1, 8, 40, 56, 100, 126):
        s = oracle.e4m3fn_value(c)
        assert oracle.e4m3_scale_for_fp4(6 * s) == c
        if c < 126:
            assert oracle.e4m3_scale_for_fp4(6 * s * (1 + 1e-6)) == c + 1
    assert oracle.e4m3_scale_for_fp4(0.0) == 0x38
    assert oracle.e4m3_scale_for_fp4(1e9) == 0x7E


def test_fp4_round_trip_error_is_at_most_half_a_step():
    rng = np.random.default_rng(21)
    for _ in range(8):
        r = (rng.standard_normal(512) * np.exp(rng.uniform(-6, 6))).astype(np.float32)
        enc = oracle.encode_row(r.astype(np.float64), "fp4_e2m1_e4m3")
        dec = oracle.decode_rows(enc[None], "fp4_e2m1_e4m3", 448, 64)[0]
        for k in range(32):
            s = oracle.e4m3fn_value(int(enc[256 + k]))
            blk = r[16 * k:16 * (k + 1)].astype(np.float64)
            assert np.max(np.abs(blk)) <= 6 * s
            mag = np.abs(blk) / s
            step = np.where(mag < 2, 0.5, np.where(mag < 4, 1.0, 2.0))
            # half a step, plus the float32 rounding of value / scale
            assert np.all(np.abs(dec[16 * k:16 * (k + 1)] - blk) <= (0.5 * step + 1e-6 * mag) * s)


def test_e2m1_codes_are_the_ocp_values():
    """All 16 e2m1 codes against the OCP table written out: magnitudes 0,
    0.5, 1, 1.5, 2, 3, 4, 6 for codes 0..7, the same negated for 8..15 (the
    fp4 row of the model record "GLM-4.7-Flash", SERVICEABILITY JOIN)."""
    import math as _m
    table = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for c in range(16):
        want = table[c & 7] * (-1.0 if c & 8 else 1.0)
        got = oracle.e2m1_value(c)
        assert got == want and _m.copysign(1.0, got) == _m.copysign(1.0, want), (c, got, want)
