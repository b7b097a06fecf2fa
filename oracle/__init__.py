"""CPU oracle for MLA paged decode.  Test infrastructure: only the tests, the
smoke check and the benchmark's CPU-baseline leg use it."""
from .reference import (  # noqa: F401
    absorb_q,
    bf16_nearest,
    bf16_to_f64,
    cache_write,
    combine_partials,
    decode_rows,
    encode_row,
    e4m3fn_nearest,
    e4m3fn_value,
    e8m0_for_block,
    e8m0_value,
    latent_attention,
    mla_decode,
    mla_decode_sparse,
    out_proj,
    row_bytes,
    sequence_rows,
    to_f64,
)
