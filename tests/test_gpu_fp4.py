"""Decode over the 288-byte fp4 cache row (e2m1 codes, one e4m3 scale per 16
values) on the GPU against the oracle on the same decoded values.

The fp4 pool is written by the oracle's encoder from seeded values, so the
inputs do not come from the GPU path.  With fp32 queries decode runs on the
fp32 vector-ALU kernel and is held to 1e-4 of the output RMS; with bf16
queries it runs on the matrix cores (each value decoded exactly to bf16, P
rounded to bf16) and is held to 5e-2 of the RMS, the fp8 cache's bar, against
the oracle on the same bf16 queries.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from synth import WORKLOADS, make_inputs
from synth.gen import Inputs

pytestmark = pytest.mark.gpu


def fp4_inputs(lens, q_per_seq=1, heads=None):
    wl32 = WORKLOADS["fp8_mtp4_b64_h20_ctx16k"].with_(batch=len(lens), q_per_seq=q_per_seq,
                                                       lens=("fixed", tuple(lens)), kv_format="f32")
    if heads is not None:
        wl32 = wl32.with_(heads=heads)
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


@pytest.mark.parametrize("lens,sq,heads", [((37, 300, 5), 1, 20), ((130, 64, 1000), 4, 20), ((77, 512), 1, 4),
                                           ((200, 33), 4, 32)])
def test_fp4_decode_matrix_cores(lens, sq, heads):
    """bf16 queries over the fp4 cache: 1 to 8 row blocks, ragged tails,
    tiles across pages."""
    import mla_paged_decode_amd as mla
    from mla_paged_decode_amd.step import DecodeStep, DeviceBatch
    from synth import bf16_bits_from_f32, make_q_abs
    inp = fp4_inputs(lens, sq, heads)
    print(f"fp4 mfma decode lens={lens} Sq={sq} H={heads}", flush=True)
    q_abs = bf16_bits_from_f32(make_q_abs(inp.wl))
    step = DecodeStep(DeviceBatch.upload(inp), q_abs_dtype=mla.MLA_BF16)
    assert mla.mla_decode_select_kernel(step.params) == mla.MLA_KERNEL_MFMA
    step.o_latent.fill_(float("nan"))
    step.q_abs.copy_(torch.from_numpy(q_abs.view(np.int16)).view(torch.bfloat16))
    step.decode()
    torch.cuda.synchronize()
    ref_o, ref_lse = oracle.latent_attention(oracle.bf16_to_f64(q_abs), inp)
    o, lse = step.o_latent.cpu().numpy(), step.lse.cpu().numpy()
    err = float(np.max(np.abs(o - ref_o))) / math.sqrt(float(np.mean(ref_o ** 2)))
    print(f"  max|d|/rms = {err:.3e}", flush=True)
    assert err <= 5e-2
    assert np.max(np.abs(lse - ref_lse)) <= 1e-3
