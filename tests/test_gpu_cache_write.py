"""mla_cache_write on the GPU against the oracle, byte for byte.

Storing a row is integer and exactly rounded work (bf16 rounding, the e8m0
scale choice and the e4m3 codes), so the pool the kernel writes must equal
the oracle's bit for bit, including ties, zero and -0 blocks, and the slots
it must leave alone.
"""
import numpy as np
import pytest
import torch

import mla_paged_decode_amd as mla
import oracle
from oracle.reference import _E4M3

pytestmark = pytest.mark.gpu

FORMATS = {"f32": mla.MLA_KV_F32, "bf16": mla.MLA_KV_BF16, "fp8_e4m3_e8m0": mla.MLA_KV_FP8_E4M3_E8M0,
           "fp4_e2m1_e4m3": mla.MLA_KV_FP4_E2M1_E4M3}


def special_rows(n_vals: int, rng) -> np.ndarray:
    """Rows that exercise the rounding rules: e4m3 midpoints at scale 1
    (block maximum 448), bf16 ties, zero / -0 / tiny-negative blocks, and
    blocks of very large and very small magnitude."""
    rows = []
    pos = _E4M3[:127]
    mids = ((pos[:-1] + pos[1:]) / 2.0).astype(np.float32)
    r = rng.standard_normal(n_vals).astype(np.float32)
    for k in range(n_vals // 32):
        blk = mids[(np.arange(32) + 31 * k) % len(mids)] * np.where(np.arange(32) % 3 == 0, -1, 1)
        blk[0] = 448.0
        r[32 * k:32 * (k + 1)] = blk
    rows.append(r)
    base = torch.from_numpy(rng.standard_normal(n_vals).astype(np.float32)).to(torch.bfloat16)
    bits = base.view(torch.int16).numpy().astype(np.uint16).astype(np.uint32) << 16
    rows.append((bits | 0x8000).view(np.float32))  # exact bf16 ties
    r = rng.standard_normal(n_vals).astype(np.float32)
    r[:32] = 0.0
    r[32:64] = -0.0
    r[64:96] = np.float32(-1e-3) * np.abs(r[64:96])
    r[64] = 1000.0  # the rest of that block rounds to zero, keeping the sign
    rows.append(r)
    rows.append((rng.standard_normal(n_vals) * 1e30).astype(np.float32))
    rows.append((rng.standard_normal(n_vals) * 1e-30).astype(np.float32))
    rows.append((rng.standard_normal(n_vals) * np.exp(rng.uniform(-20, 20, n_vals))).astype(np.float32))
    return np.stack(rows)


def run_case(fmt: str, rows_dtype: str, n_rows: int, page_block: int, num_pages: int, seed: int):
    d_lat = 448 if fmt.startswith("fp") else 512
    n_vals = d_lat + 64
    rb = oracle.row_bytes(fmt, d_lat, 64)
    rng = np.random.default_rng(seed)
    rows = rng.standard_normal((n_rows, n_vals)).astype(np.float32)
    sp = special_rows(n_vals, rng)
    rows[:len(sp)] = sp[:n_rows]
    n_slots = num_pages * page_block
    slots = rng.permutation(n_slots)[:n_rows].astype(np.int64)
    slots[1::7] = -1
    slots[3::11] = n_slots + 5  # past the end: skipped
    pool0 = np.full((num_pages, page_block, rb), 0x5A, dtype=np.uint8)

    if rows_dtype == "bf16":
        rows_t = torch.from_numpy(rows).to(torch.bfloat16)
        stored = rows_t.view(torch.int16).numpy().astype(np.uint16)
    else:
        rows_t = torch.from_numpy(rows)
        stored = rows
    dims = mla.Dims(20, d_lat, 64, 192, 256)
    pool = torch.from_numpy(pool0.copy()).cuda()
    print(f"cache_write {fmt} rows={rows_dtype} n={n_rows} P={page_block} pages={num_pages}", flush=True)
    mla.mla_cache_write(dims, n_rows, rows_t.cuda(), torch.from_numpy(slots).cuda(), pool, FORMATS[fmt],
                        num_pages, page_block)
    torch.cuda.synchronize()
    want = oracle.cache_write(pool0, stored, rows_dtype, slots, fmt)
    got = pool.cpu().numpy()
    bad = np.argwhere(got.reshape(-1, rb) != want.reshape(-1, rb))
    assert bad.size == 0, f"{len(bad)} bytes differ, first at (slot, byte) {bad[:5].tolist()}"


@pytest.mark.parametrize("fmt", list(FORMATS))
@pytest.mark.parametrize("rows_dtype", ["f32", "bf16"])
def test_cache_write_bit_exact(fmt, rows_dtype):
    run_case(fmt, rows_dtype, n_rows=40, page_block=16, num_pages=6, seed=1)


@pytest.mark.parametrize("fmt", ["bf16", "fp8_e4m3_e8m0", "fp4_e2m1_e4m3"])
def test_cache_write_batch_of_new_tokens(fmt):
    """One new token per sequence of a 256-sequence batch into 128-token pages."""
    run_case(fmt, "f32", n_rows=256, page_block=128, num_pages=40, seed=2)


def test_cache_write_rejects_bad_arguments():
    dims = mla.Dims(20, 512, 64, 192, 256)
    rows = torch.zeros((4, 576), device="cuda")
    slots = torch.zeros(4, dtype=torch.int64, device="cuda")
    pool = torch.zeros((2, 16, 1152), dtype=torch.uint8, device="cuda")
    with pytest.raises(mla.MlaError, match="page_block"):
        mla.mla_cache_write(dims, 4, rows, slots, pool, mla.MLA_KV_BF16, 2, 96)
    with pytest.raises(mla.MlaError, match="d_latent"):
        mla.mla_cache_write(dims, 4, rows, slots, pool, mla.MLA_KV_FP8_E4M3_E8M0, 2, 16)
    mla.mla_cache_write(dims, 0, rows, slots, pool, mla.MLA_KV_BF16, 2, 16)  # empty: no-op
    torch.cuda.synchronize()
    assert int(pool.sum()) == 0
