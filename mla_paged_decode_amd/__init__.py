"""Python binding of libmla (MLA decode over a paged latent KV cache, gfx950).

Argument marshalling only: every step runs in the HIP kernels of
libmla.so.  Tensors are passed by device pointer (``data_ptr()``); integers
are taken as raw device addresses.  The stream defaults to torch's current
stream.  A non-zero status raises :class:`MlaError` carrying the library's
"<argument>: expected X, got Y" message.

There is no fallback: if libmla.so is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

__all__ = [
    "MlaError", "Dims", "DecodeParams", "lib", "library_path",
    "mla_kv_row_bytes", "mla_absorb_q", "mla_decode_workspace_size",
    "mla_decode_paged", "mla_decode_paged_noalloc", "MLA_NOALLOC_SCRATCH_BYTES", "mla_decode_select_kernel", "mla_out_proj", "mla_cache_write", "mla_abi_version",
    "mla_decode_sparse_paged", "mla_decode_sparse_workspace_size",
    "MLA_F32", "MLA_BF16", "MLA_KV_F32", "MLA_KV_BF16", "MLA_KV_FP8_E4M3_E8M0", "MLA_KV_FP4_E2M1_E4M3",
    "MLA_KERNEL_AUTO", "MLA_KERNEL_SIMT", "MLA_KERNEL_MFMA", "KV_FORMAT",
    "MLA_DECODE_ALLOW_BF16_QUERIES", "MLA_DECODE_DYNAMIC_SPLIT", "MLA_DECODE_FUSED_MERGE", "mla_validate_tables",
]

MLA_F32, MLA_BF16 = 0, 1
MLA_KV_F32, MLA_KV_BF16, MLA_KV_FP8_E4M3_E8M0, MLA_KV_FP4_E2M1_E4M3 = 0, 1, 2, 3
MLA_KERNEL_AUTO, MLA_KERNEL_SIMT, MLA_KERNEL_MFMA = 0, 1, 2
MLA_DECODE_ALLOW_BF16_QUERIES = 0x1
MLA_DECODE_DYNAMIC_SPLIT = 0x2
MLA_DECODE_FUSED_MERGE = 0x4
MLA_NOALLOC_SCRATCH_BYTES = 128 << 20
KV_FORMAT = {"f32": MLA_KV_F32, "bf16": MLA_KV_BF16, "fp8_e4m3_e8m0": MLA_KV_FP8_E4M3_E8M0,
             "fp4_e2m1_e4m3": MLA_KV_FP4_E2M1_E4M3}

STATUS = {
    0: "MLA_OK", 1: "MLA_ERR_NULL_POINTER", 2: "MLA_ERR_INVALID_SHAPE",
    3: "MLA_ERR_UNSUPPORTED", 4: "MLA_ERR_ALIGNMENT",
    5: "MLA_ERR_WORKSPACE_TOO_SMALL", 6: "MLA_ERR_HIP",
}

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libmla.so")


class MlaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status
        self.message = message


class Dims(ctypes.Structure):
    _fields_ = [("num_heads", ctypes.c_int32), ("d_latent", ctypes.c_int32),
                ("d_rope", ctypes.c_int32), ("d_nope", ctypes.c_int32),
                ("d_v", ctypes.c_int32)]


class DecodeParams(ctypes.Structure):
    _fields_ = [
        ("dims", Dims),
        ("batch", ctypes.c_int32),
        ("q_per_seq", ctypes.c_int32),
        ("q_abs", ctypes.c_void_p),
        ("q_abs_dtype", ctypes.c_int),
        ("kv_pool", ctypes.c_void_p),
        ("kv_format", ctypes.c_int),
        ("num_pages", ctypes.c_int64),
        ("page_block", ctypes.c_int32),
        ("block_table", ctypes.c_void_p),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("seq_lens", ctypes.c_void_p),
        ("softmax_scale", ctypes.c_float),
        ("num_splits", ctypes.c_int32),
        ("kernel", ctypes.c_int),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("o_latent", ctypes.c_void_p),
        ("o_dtype", ctypes.c_int),
        ("lse", ctypes.c_void_p),
        ("kernel_start_event", ctypes.c_void_p),
        ("kernel_stop_event", ctypes.c_void_p),
        ("flags", ctypes.c_uint32),
    ]


class PrefillParams(ctypes.Structure):
    _fields_ = [
        ("dims", Dims),
        ("batch", ctypes.c_int32),
        ("q_per_seq", ctypes.c_int32),
        ("q", ctypes.c_void_p),
        ("q_dtype", ctypes.c_int),
        ("w_kv_b", ctypes.c_void_p),
        ("w_dtype", ctypes.c_int),
        ("kv_pool", ctypes.c_void_p),
        ("kv_format", ctypes.c_int),
        ("num_pages", ctypes.c_int64),
        ("page_block", ctypes.c_int32),
        ("block_table", ctypes.c_void_p),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("seq_lens", ctypes.c_void_p),
        ("softmax_scale", ctypes.c_float),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("out", ctypes.c_void_p),
        ("lse", ctypes.c_void_p),
    ]


# Must equal MLA_ABI_VERSION of include/mla.h (the parameter struct layout).
ABI_VERSION = 3

_lib = None


def lib() -> ctypes.CDLL:
    """Load libmla.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise RuntimeError(f"{library_path} is not built; run `python -m mla_paged_decode_amd.build`")
        L = ctypes.CDLL(library_path)
        vp, i32, st = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int
        L.mla_kv_row_bytes.argtypes = [ctypes.POINTER(Dims), st]
        L.mla_kv_row_bytes.restype = ctypes.c_size_t
        L.mla_absorb_q.argtypes = [ctypes.POINTER(Dims), i32, vp, st, vp, st, vp, st, vp]
        L.mla_absorb_q.restype = st
        L.mla_out_proj.argtypes = [ctypes.POINTER(Dims), i32, vp, st, vp, st, vp, st, vp]
        L.mla_out_proj.restype = st
        L.mla_cache_write.argtypes = [ctypes.POINTER(Dims), i32, vp, st, vp, vp, st, ctypes.c_int64, i32, vp]
        L.mla_cache_write.restype = st
        L.mla_decode_workspace_size.argtypes = [ctypes.POINTER(DecodeParams), ctypes.POINTER(ctypes.c_size_t)]
        L.mla_decode_workspace_size.restype = st
        L.mla_decode_select_kernel.argtypes = [ctypes.POINTER(DecodeParams), ctypes.POINTER(ctypes.c_int)]
        L.mla_decode_select_kernel.restype = st
        L.mla_decode_sparse_workspace_size.argtypes = [ctypes.POINTER(DecodeParams), i32,
                                                       ctypes.POINTER(ctypes.c_size_t)]
        L.mla_decode_sparse_workspace_size.restype = st
        L.mla_decode_sparse_paged.argtypes = [ctypes.POINTER(DecodeParams), vp, i32, vp]
        L.mla_decode_sparse_paged.restype = st
        L.mla_decode_paged.argtypes = [ctypes.POINTER(DecodeParams), vp]
        L.mla_decode_paged.restype = st
        L.mla_decode_paged_noalloc.argtypes = [ctypes.POINTER(DecodeParams), vp]
        L.mla_decode_paged_noalloc.restype = st
        L.mla_prefill_workspace_size.argtypes = [ctypes.POINTER(PrefillParams), ctypes.POINTER(ctypes.c_size_t)]
        L.mla_prefill_workspace_size.restype = st
        L.mla_prefill_paged.argtypes = [ctypes.POINTER(PrefillParams), vp]
        L.mla_prefill_paged.restype = st
        L.mla_status_string.argtypes = [st]
        L.mla_status_string.restype = ctypes.c_char_p
        L.mla_last_error_message.argtypes = []
        L.mla_last_error_message.restype = ctypes.c_char_p
        L.mla_validate_tables.argtypes = [i32, vp, vp, i32, ctypes.c_int64, i32]
        L.mla_validate_tables.restype = st
        L.mla_abi_version.argtypes = []
        L.mla_abi_version.restype = i32
        if L.mla_abi_version() != ABI_VERSION:
            raise RuntimeError(f"{library_path} has ABI version {L.mla_abi_version()}, this binding expects "
                               f"{ABI_VERSION}; rebuild with `python -m mla_paged_decode_amd.build`")
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != 0:
        raise MlaError(status, lib().mla_last_error_message().decode())


def _ptr(x) -> int:
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _dtype_code(x, explicit: Optional[int] = None) -> int:
    if explicit is not None:
        return explicit
    import torch
    if x.dtype == torch.float32:
        return MLA_F32
    if x.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return MLA_BF16
    raise TypeError(f"unsupported tensor dtype {x.dtype}")


def _stream(stream) -> int:
    if stream is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


def _dims(dims) -> Dims:
    if isinstance(dims, Dims):
        return dims
    return Dims(*dims)


def mla_abi_version() -> int:
    return int(lib().mla_abi_version())


def mla_kv_row_bytes(dims, kv_format: int) -> int:
    return int(lib().mla_kv_row_bytes(ctypes.byref(_dims(dims)), kv_format))


def mla_absorb_q(dims, n_tokens: int, q, w_kv_b, q_abs, *, q_dtype=None, w_dtype=None,
                 q_abs_dtype=None, stream=None) -> None:
    _check(lib().mla_absorb_q(ctypes.byref(_dims(dims)), n_tokens,
                              _ptr(q), _dtype_code(q, q_dtype),
                              _ptr(w_kv_b), _dtype_code(w_kv_b, w_dtype),
                              _ptr(q_abs), _dtype_code(q_abs, q_abs_dtype), _stream(stream)))


def mla_out_proj(dims, n_tokens: int, o_latent, w_kv_b, out, *, w_dtype=None, stream=None) -> None:
    _check(lib().mla_out_proj(ctypes.byref(_dims(dims)), n_tokens,
                              _ptr(o_latent), MLA_F32, _ptr(w_kv_b), _dtype_code(w_kv_b, w_dtype),
                              _ptr(out), MLA_F32, _stream(stream)))


def mla_cache_write(dims, n_rows: int, rows, slots, kv_pool, kv_format: int, num_pages: int,
                    page_block: int, *, rows_dtype=None, stream=None) -> None:
    """Store rows [n_rows][d_latent + d_rope] at the int64 token slots
    (page * page_block + offset) of kv_pool, in kv_format."""
    _check(lib().mla_cache_write(ctypes.byref(_dims(dims)), n_rows, _ptr(rows), _dtype_code(rows, rows_dtype),
                                 _ptr(slots), _ptr(kv_pool), kv_format, num_pages, page_block,
                                 _stream(stream)))


def make_decode_params(*, dims, batch, q_per_seq, q_abs, kv_pool, kv_format, num_pages,
                       page_block, block_table, max_blocks_per_seq, seq_lens, softmax_scale,
                       num_splits=0, kernel=MLA_KERNEL_AUTO, workspace=None, workspace_bytes=0,
                       o_latent=None, lse=None, q_abs_dtype=None, flags=0) -> DecodeParams:
    """Fill the C parameter struct (pointers from tensors or raw ints)."""
    qd = q_abs_dtype if q_abs_dtype is not None else (
        _dtype_code(q_abs) if not isinstance(q_abs, int) and q_abs is not None else MLA_F32)
    return DecodeParams(
        dims=_dims(dims), batch=batch, q_per_seq=q_per_seq,
        q_abs=_ptr(q_abs), q_abs_dtype=qd,
        kv_pool=_ptr(kv_pool), kv_format=kv_format, num_pages=num_pages,
        page_block=page_block, block_table=_ptr(block_table),
        max_blocks_per_seq=max_blocks_per_seq, seq_lens=_ptr(seq_lens),
        softmax_scale=softmax_scale, num_splits=num_splits, kernel=kernel,
        workspace=_ptr(workspace), workspace_bytes=workspace_bytes,
        o_latent=_ptr(o_latent), o_dtype=MLA_F32, lse=_ptr(lse), flags=flags)


def mla_validate_tables(seq_lens, block_table, num_pages: int, page_block: int) -> None:
    """Host-side range check of the tables (numpy arrays or CPU tensors):
    seq_lens [B] int32 and block_table [B][max_blocks] int32.  Raises
    MlaError naming the first entry out of range."""
    import numpy as np
    sl = np.ascontiguousarray(np.asarray(seq_lens), dtype=np.int32)
    bt = np.ascontiguousarray(np.asarray(block_table), dtype=np.int32)
    if bt.ndim != 2 or bt.shape[0] != sl.shape[0]:
        raise ValueError(f"block_table: expected shape [{sl.shape[0]}, max_blocks], got {bt.shape}")
    _check(lib().mla_validate_tables(sl.shape[0], sl.ctypes.data, bt.ctypes.data, bt.shape[1],
                                     num_pages, page_block))


def mla_decode_workspace_size(params: DecodeParams) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().mla_decode_workspace_size(ctypes.byref(params), ctypes.byref(n)))
    return int(n.value)


def mla_decode_select_kernel(params: DecodeParams) -> int:
    k = ctypes.c_int(0)
    _check(lib().mla_decode_select_kernel(ctypes.byref(params), ctypes.byref(k)))
    return int(k.value)


def mla_decode_paged(params: DecodeParams, stream=None) -> None:
    _check(lib().mla_decode_paged(ctypes.byref(params), _stream(stream)))


def mla_decode_paged_noalloc(params: DecodeParams, stream=None) -> None:
    """mla_decode_paged with the library's own per-GPU scratch in place of
    the workspace (params.workspace is ignored); allocates nothing."""
    _check(lib().mla_decode_paged_noalloc(ctypes.byref(params), _stream(stream)))


def mla_decode_sparse_workspace_size(params: DecodeParams, topk_width: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().mla_decode_sparse_workspace_size(ctypes.byref(params), topk_width, ctypes.byref(n)))
    return int(n.value)


def mla_decode_sparse_paged(params: DecodeParams, topk_indices, topk_width: int, stream=None) -> None:
    """Decode over the cached tokens named by topk_indices [B][Sq][topk_width] int32."""
    _check(lib().mla_decode_sparse_paged(ctypes.byref(params), _ptr(topk_indices), topk_width, _stream(stream)))


def make_prefill_params(*, dims, batch, q_per_seq, q, w_kv_b, kv_pool, kv_format, num_pages, page_block,
                        block_table, max_blocks_per_seq, seq_lens, softmax_scale, out, lse=None,
                        workspace=None, workspace_bytes=0, q_dtype=None, w_dtype=None) -> PrefillParams:
    """Fill the C prefill parameter struct (pointers from tensors or raw ints)."""
    return PrefillParams(
        dims=_dims(dims), batch=batch, q_per_seq=q_per_seq,
        q=_ptr(q), q_dtype=_dtype_code(q, q_dtype), w_kv_b=_ptr(w_kv_b), w_dtype=_dtype_code(w_kv_b, w_dtype),
        kv_pool=_ptr(kv_pool), kv_format=kv_format, num_pages=num_pages, page_block=page_block,
        block_table=_ptr(block_table), max_blocks_per_seq=max_blocks_per_seq, seq_lens=_ptr(seq_lens),
        softmax_scale=softmax_scale, workspace=_ptr(workspace), workspace_bytes=workspace_bytes,
        out=_ptr(out), lse=_ptr(lse))


def mla_prefill_workspace_size(params: PrefillParams) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().mla_prefill_workspace_size(ctypes.byref(params), ctypes.byref(n)))
    return int(n.value)


def mla_prefill_paged(params: PrefillParams, stream=None) -> None:
    """Unabsorbed causal prefill of the last q_per_seq cached tokens of every sequence."""
    _check(lib().mla_prefill_paged(ctypes.byref(params), _stream(stream)))
