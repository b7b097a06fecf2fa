"""The C++ oracle (oracle/mla_oracle.cpp): build and call.

Test infrastructure, like the rest of oracle/: only the tests, the smoke
check and the benchmark's CPU-baseline leg use it.  It is the same
unabsorbed definition as `reference.mla_decode`, written independently in
C++ with OpenMP over (sequence, head) pairs, and pinned against it in
tests/test_oracle_native.py.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "mla_oracle.cpp")
LIBRARY = os.path.join(_HERE, "libmla_oracle.so")
# x86-64-v3 (AVX2 + FMA): every host this runs on has it; no -march=native,
# so a library built here also runs on another host.
FLAGS = ["-O3", "-march=x86-64-v3", "-fopenmp", "-shared", "-fPIC", "-std=c++17", "-Wall"]

_FMT = {"f32": 0, "bf16": 1, "fp8_e4m3_e8m0": 2, "fp4_e2m1_e4m3": 3}
_lib = None


def build(verbose: bool = False) -> str:
    """Compile libmla_oracle.so with g++ (every call)."""
    tmp = f"{LIBRARY}.{os.getpid()}.tmp"  # one per process: concurrent builds each rename a whole file
    r = subprocess.run(["g++", *FLAGS, SOURCE, "-o", tmp], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"g++ failed on {SOURCE}:\n{r.stderr}")
    os.replace(tmp, LIBRARY)
    if verbose:
        print(f"built {LIBRARY}")
    return LIBRARY


def lib() -> ctypes.CDLL:
    """Load the oracle library, building it if it is not there."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY):
            build()
        L = ctypes.CDLL(LIBRARY)
        vp, i32, i64, f64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        L.mla_oracle_decode.argtypes = [i32, i32, i32, i32, i32, i32, i32, vp, i32, vp, i32, vp, i32, i64, i32,
                                        vp, i32, vp, f64, vp, i32, vp, vp, i32]
        L.mla_oracle_decode.restype = i32
        L.mla_oracle_max_threads.argtypes = []
        L.mla_oracle_max_threads.restype = i32
        _lib = L
    return _lib


def max_threads() -> int:
    return int(lib().mla_oracle_max_threads())


def mla_decode(inp, seqs=None, threads: int = 0):
    """Unabsorbed MLA decode of `inp` (synth.Inputs layout) in C++.

    Returns out float64 [B*Sq, H, d_v] and lse float64 [B*Sq, H]; entries
    of sequences not selected are NaN (as reference.mla_decode)."""
    wl = inp.wl
    B, Sq, H = wl.batch, wl.q_per_seq, wl.heads
    q = np.ascontiguousarray(inp.q)
    w = np.ascontiguousarray(inp.w_kv_b)
    pool = np.ascontiguousarray(inp.kv_pool, dtype=np.uint8)
    bt = np.ascontiguousarray(inp.block_table, dtype=np.int32)
    sl = np.ascontiguousarray(inp.seq_lens, dtype=np.int32)
    sel = np.arange(B, dtype=np.int32) if seqs is None else np.ascontiguousarray(list(seqs), dtype=np.int32)
    out = np.full((B * Sq, H, wl.d_v), np.nan)
    lse = np.full((B * Sq, H), np.nan)
    qf = 0 if wl.q_dtype == "f32" else 1
    wf = 0 if wl.w_dtype == "f32" else 1
    st = lib().mla_oracle_decode(
        B, Sq, H, wl.d_nope, wl.d_rope, wl.d_v, wl.d_latent, q.ctypes.data, qf, w.ctypes.data, wf,
        pool.ctypes.data, _FMT[wl.kv_format], pool.shape[0], wl.page_block, bt.ctypes.data, bt.shape[1],
        sl.ctypes.data, float(wl.softmax_scale), sel.ctypes.data, len(sel), out.ctypes.data, lse.ctypes.data,
        threads)
    if st != 0:
        raise ValueError("mla_oracle_decode: a block-table entry or length is out of range")
    return out, lse
