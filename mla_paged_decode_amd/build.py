"""Build libmla.so in-tree with hipcc for gfx950.

    python -m mla_paged_decode_amd.build

Every source under csrc/ is compiled for gfx950 only, with packed fp32 ALU
instructions disabled, and linked into mla_paged_decode_amd/libmla.so.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmla.so")
ARCH = "gfx950"

SOURCES = [
    "api.cpp",
    "combine.hip",
    "decode_simt.hip",
    "decode_mfma.hip",
    "decode_dyn.hip",
    "decode_fp8.hip",
    "proj_simt.hip",
    "proj_mfma.hip",
    "cache_write.hip",
    "prefill_simt.hip",
    "prefill_mfma.hip",
]

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # LDS is laid out by hand in every kernel; do not move private arrays there
    "-mllvm", "-disable-promote-alloca-to-lds",
    # Single-lane counter atomics stay plain atomics: the atomic optimiser
    # would turn them into a wave reduction that waits for the result at once,
    # where the run-time scheduler wants it a tile later.
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP toolchain is required to build libmla")
    return path


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = f"{LIB}.{os.getpid()}.tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
