"""Seeded synthetic inputs for MLA decode over a paged latent cache.

This package is shared by the oracle-side tests and the GPU path's tests and
benchmark.  It only draws random numbers and lays them out in the storage
formats the decode consumes (fp32, bf16, fp8 e4m3 with e8m0 block scales); it
contains none of the attention arithmetic.
"""
from .gen import (  # noqa: F401
    WORKLOADS,
    Inputs,
    Workload,
    bf16_bits_from_f32,
    make_inputs,
    make_o_latent,
    make_q_abs,
    quantize_e4m3_e8m0,
    stored_row_bytes,
)
