"""Decode over the 288-byte fp4 cache row (e2m1 codes, one e4m3 scale per 16
values) on the GPU against the oracle on the same decoded values.

The fp4 pool is written by the oracle's encoder from seeded values, so the
inputs do not come from the GPU path; decode runs on the fp32 vector-ALU
kernel and is held to 1e-4 of the output RMS.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from synth import WORKLOADS, make_inputs
from synth.gen import Inputs

pytestmark = pytest.mark.gpu


def fp4_inputs(lens, q_per_seq=1, seed_batch=None):
    wl32 = WORKLOADS["fp8_mtp4_b64_h20_ctx16k"].with_(batch=len(lens), q_per_seq=q_per_seq,
                                                       lens=("fixed", tuple(lens)), kv_format="f32")
    base = make_inputs(wl32)
    vals = oracle.decode_rows(base.kv_pool, "f32", wl32.d_latent, wl32.d_rope)
    pool = np.stack([oracle.encode_row(v, "fp4_e2m1_e4m3") for v in vals.reshape(-1, vals.shape[-1])])
    pool = pool.reshape(base.kv_pool.shape[0], base.kv_pool.shape[1], 288)
    wl = wl32.with_(kv_format="fp4_e2m1_e4m3")
    return Inputs(wl=wl, q=base.q, w_kv_b=base.w_kv_b, kv_pool=pool, block_table=base.block_table,
                  seq_lens=base.seq_lens)


@pytest.mark.parametrize("lens,sq", [((37, 300, 5), 1), ((130, 64), 4)])
def test_fp4_decode_matches_oracle(lens, sq):
    import mla_paged_decode_amd as mla
    from mla_paged_decode_amd.step import DecodeStep, DeviceBatch
    inp = fp4_inputs(lens, sq)
    print(f"fp4 decode lens={lens} Sq={sq}", flush=True)
    step = DecodeStep(DeviceBatch.upload(inp), q_abs_dtype=mla.MLA_F32)
    assert mla.mla_decode_select_kernel(step.params) == mla.MLA_KERNEL_SIMT
    out = step.run()
    torch.cuda.synchronize()
    ref, rlse = oracle.mla_decode(inp)
    got = out.cpu().numpy()
    err = float(np.max(np.abs(got - ref))) / math.sqrt(float(np.mean(ref ** 2)))
    print(f"  max|d|/rms = {err:.3e}", flush=True)
    assert err <= 1e-4
