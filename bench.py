"""Benchmark: MLA decode over a paged latent cache on one MI355X.

One step = one decode step of one attention layer for the whole batch:
mla_absorb_q -> mla_decode_paged (split-KV attention and LSE merge) ->
mla_out_proj, on synthetic seeded inputs already resident in HBM.  The
timed steps are replayed from HIP graphs (as a serving loop would run
them); the per-kernel roofline comes from a second, eager pass.

The default workload is the largest one that the metric's target names:
256 sequences of one GLM-4.7-Flash layer (20 heads, bf16 latent cache of
512 + 64 values per token, page block 128), context lengths uniform in
[512, 8192], about 10% of block-table entries on a shared prefix.  The same
JSON line carries sub-records for the long-context workload (4 sequences,
65,536 to 202,752 tokens; balanced split and its literal 32 chunks) and the
fp8 cache with 4 MTP query tokens, each with its attention-kernel and
decode-call (merge included) fractions of the 8 TB/s HBM peak.  A cache
smaller than 4x the 256 MB Infinity Cache is cycled through several copies,
each at its own address, so that no step is served from it.

Output: one JSON line with query-tokens/s for the whole step, the achieved
HBM bandwidth of the decode call (latent bytes read / its average
duration), the roofline of its dominant kernel (the split-KV attention
kernel: latent bytes read / its average duration, HIP events the library
records on the launch stream around that launch alone), MFMA utilisation
from the committed counter summaries, and the C++ CPU oracle timed on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MLA decode query-tokens/s and achieved HBM GB/s (% of 8 TB/s) at 1 GPU"
HBM_PEAK_GBS = 8000.0
INFINITY_CACHE_BYTES = 256 << 20


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, target_s: float):
    """The C++ oracle (unabsorbed definition, double precision, OpenMP over
    (sequence, head) pairs on every host core) on whole sequences of the same
    workload, one sequence per call, until about target_s seconds of work
    have run."""
    import numpy as np

    from oracle import native
    from synth import make_inputs

    inp = make_inputs(wl)
    native.lib()
    threads = native.max_threads()
    t0 = time.perf_counter()
    done = 0
    for b in range(wl.batch):
        native.mla_decode(inp, seqs=[b], threads=threads)
        done += 1
        if time.perf_counter() - t0 >= target_s:
            break
    dt = time.perf_counter() - t0
    qtok = done * wl.q_per_seq
    tokens = int(np.sum(inp.seq_lens[:done].astype(np.int64)))
    return {
        "value": qtok / dt,
        "unit": "query-tokens/s",
        "cores": int(threads),
        "kind": "oracle",
        "nproc": os.cpu_count(),
        "cpu_model": cpu_model(),
        "latent_gbs": tokens * inp.row_bytes / dt / 1e9,
        "sample": f"{done} of {wl.batch} sequences of {wl.name} ({tokens} cached tokens), unabsorbed "
                  f"double-precision C++ oracle (oracle/mla_oracle.cpp), {threads} OpenMP threads, {dt:.1f} s",
    }


COUNTER_SOURCES = ["decode_mfma.hip", "decode_fp8.hip", "decode_common.h", "staging_bf16.h", "merge_fused.h",
                   "schedule.h", "internal.h", "device_common.h"]


def code_without_comments(text: str) -> str:
    """C++ source with its comments, trailing blanks and blank lines removed
    (string literals in these sources hold no comment markers)."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*$", "", ln).rstrip() for ln in text.splitlines())
    return "\n".join(ln for ln in lines if ln)


def kernel_source_digest(read=None) -> str:
    """sha256 over the attention kernel's sources, comments left out (counters
    go stale when the code changes, not when a comment does).  `read(name)`
    returns a source's text; by default the file in csrc/."""
    import hashlib
    if read is None:
        def read(f):
            with open(os.path.join(ROOT, "mla_paged_decode_amd", "csrc", f), encoding="utf-8") as fh:
                return fh.read()
    h = hashlib.sha256()
    for f in COUNTER_SOURCES:
        h.update(code_without_comments(read(f)).encode())
        h.update(b"\0")
    return h.hexdigest()


def counter_file(workload: str, splits: int) -> str:
    """Name of the committed counter summary of a workload (and split mode)."""
    tag = "" if splits == 0 else f"_splits{splits}"
    return os.path.join(ROOT, "profiles", f"decode_mfma_{workload}{tag}_counters.txt")


def counter_summary(workload: str, splits: int = 0):
    """The committed counter summary of this workload's attention kernel as
    a dict of its "key: value" lines, or None if there is none or the kernel
    has changed since the counters were taken."""
    path = counter_file(workload, splits)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith(" "):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != kernel_source_digest():
        return None
    return kv


def counter_traffic(workload: str, splits: int = 0):
    """HBM bytes per attention-kernel launch (FETCH_SIZE + WRITE_SIZE, each
    scaled by the same counter's reading for a plain copy of known size), or
    None if the counters are missing or stale."""
    kv = counter_summary(workload, splits)
    try:
        return float(kv["hbm_bytes_per_launch"]) if kv else None
    except (KeyError, ValueError):
        return None


# MI355X: 8 XCDs, each with its own GRBM (so GRBM_GUI_ACTIVE sums 8 clocks
# per GPU cycle), and 256 CUs x 4 SIMDs, each with one matrix core.
N_XCD, N_SIMD = 8, 1024
BF16_MFMA_PEAK_TFLOPS = 2500.0


def mfma_utilisation(workload: str, splits: int = 0):
    """Matrix-core utilisation of the attention kernel from the committed
    counters: SQ_VALU_MFMA_BUSY_CYCLES / (GPU cycles x SIMDs), GPU cycles =
    GRBM_GUI_ACTIVE / XCDs; also the executed bf16 MFMA flops
    (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512) per dispatch.  None if the counters
    are missing or stale."""
    kv = counter_summary(workload, splits)
    if not kv:
        return None
    try:
        busy = float(kv["mfma_busy_cycles_per_dispatch"])
        gui = float(kv["grbm_gui_active_per_dispatch"])
        flops = float(kv["mfma_flops_executed_per_dispatch"])
    except (KeyError, ValueError):
        return None
    return {"busy_frac": busy / (gui / N_XCD * N_SIMD), "flops_executed": flops,
            "source": os.path.relpath(counter_file(workload, splits), ROOT)}


def cache_write_timing(inp, dev, reps: int):
    """mla_cache_write of the step's new tokens: B * Sq rows (synthetic,
    seeded N(0, 1) f32) stored at the slots of the last Sq positions of each
    sequence, into a copy of the cache; average over reps calls (HIP events
    on the launch stream)."""
    import torch

    import mla_paged_decode_amd as mla

    wl = inp.wl
    P = wl.page_block
    slots = []
    for b in range(wl.batch):
        L = int(inp.seq_lens[b])
        for j in range(wl.q_per_seq):
            t = L - wl.q_per_seq + j
            slots.append(int(inp.block_table[b, t // P]) * P + t % P if t >= 0 else -1)
    n = len(slots)
    n_vals = wl.d_latent + wl.d_rope
    rows = torch.randn((n, n_vals), generator=torch.Generator().manual_seed(7)).cuda()
    slots_t = torch.tensor(slots, dtype=torch.int64).cuda()
    pool = dev.kv_pool.clone()
    fmt = dev.kv_format
    args = (dev.dims, n, rows, slots_t, pool, fmt, pool.shape[0], P)
    for _ in range(3):
        mla.mla_cache_write(*args)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(reps):
        mla.mla_cache_write(*args)
    ev1.record()
    torch.cuda.synchronize()
    us = ev0.elapsed_time(ev1) * 1e3 / reps
    nbytes = n * n_vals * 4 + n * inp.row_bytes + n * 8
    return {"rows": n, "us": us, "bytes": nbytes, "gbs": nbytes / (us * 1e-6) / 1e9}


def sparse_on_matrix_cores(wl, q_abs_dtype, topk_width: int) -> bool:
    """The library's sparse kernel choice: matrix cores for whole 32-slot
    tiles with a bf16 cache (up to 64 heads), or an fp8 / fp4 cache of the
    448 + 64 row with bf16 queries (up to 128 heads)."""
    import mla_paged_decode_amd as mla
    if topk_width % 32:
        return False
    if wl.kv_format == "bf16":
        return wl.d_latent == 512 and wl.heads <= 64
    return (wl.kv_format in ("fp8_e4m3_e8m0", "fp4_e2m1_e4m3") and wl.d_latent == 448
            and q_abs_dtype == mla.MLA_BF16 and wl.heads <= 128)


def sparse_timing(inp, dev, q_abs, q_abs_dtype, topk_width: int, num_splits: int, reps: int):
    """mla_decode_sparse_paged over topk_width listed tokens per query (a
    seeded random half of the visible positions, -1 padded): the attention
    kernel's average duration (HIP events the library records on the launch
    stream) and the listed rows' bytes per launch."""
    import numpy as np
    import torch

    import mla_paged_decode_amd as mla

    wl = inp.wl
    rng = np.random.default_rng(11)
    topk = np.full((wl.batch, wl.q_per_seq, topk_width), -1, dtype=np.int32)
    listed = 0
    for b in range(wl.batch):
        for j in range(wl.q_per_seq):
            limit = int(inp.seq_lens[b]) - wl.q_per_seq + j
            k = min(topk_width, max(0, limit + 1))
            if k:
                topk[b, j, :k] = rng.choice(limit + 1, size=k, replace=False)
            listed += k
    N, H = wl.n_tokens, wl.heads
    o_lat = torch.empty((N, H, wl.d_latent), device="cuda")
    params = mla.make_decode_params(
        dims=dev.dims, batch=wl.batch, q_per_seq=wl.q_per_seq, q_abs=q_abs, kv_pool=dev.kv_pool,
        kv_format=dev.kv_format, num_pages=dev.kv_pool.shape[0], page_block=dev.page_block,
        block_table=dev.block_table, max_blocks_per_seq=dev.block_table.shape[1], seq_lens=dev.seq_lens,
        softmax_scale=dev.softmax_scale, num_splits=num_splits, o_latent=o_lat, lse=None,
        q_abs_dtype=q_abs_dtype)
    nbytes = mla.mla_decode_sparse_workspace_size(params, topk_width)
    ws = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device="cuda")
    params.workspace, params.workspace_bytes = ws.data_ptr(), nbytes
    topk_t = torch.from_numpy(topk).cuda()
    for _ in range(2):
        mla.mla_decode_sparse_paged(params, topk_t, topk_width)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e in evs:
        for x in e:
            x.record()
    torch.cuda.synchronize()
    for e in evs:
        params.kernel_start_event, params.kernel_stop_event = e[0].cuda_event, e[1].cuda_event
        mla.mla_decode_sparse_paged(params, topk_t, topk_width)
    torch.cuda.synchronize()
    us = sum(a.elapsed_time(b) for a, b in evs) / reps * 1e3
    row_bytes = inp.row_bytes
    return {"topk_width": topk_width, "listed_tokens": listed, "num_splits": num_splits,
            "kernel": "mfma" if sparse_on_matrix_cores(wl, q_abs_dtype, topk_width) else "simt",
            "attention_kernel_us": us, "bytes": listed * row_bytes,
            "gbs": listed * row_bytes / (us * 1e-6) / 1e9}


def fp4_timing(inp, dev, reps: int):
    """mla_decode_paged over an fp4 copy of the cache (288-byte rows, same
    pages and lengths): seeded N(0, 1) rows written for every slot by
    mla_cache_write, bf16 absorbed queries, then the attention kernel timed
    with HIP events the library records on the launch stream.  Only for the
    448 + 64 row shape."""
    import numpy as np
    import torch

    import mla_paged_decode_amd as mla

    wl = inp.wl
    if wl.d_latent != 448:
        return None
    pages, P = dev.kv_pool.shape[0], dev.kv_pool.shape[1]
    n = pages * P
    pool = torch.empty((pages, P, 288), dtype=torch.uint8, device="cuda")
    rows = torch.randn((n, wl.d_latent + wl.d_rope), generator=torch.Generator().manual_seed(5)).cuda()
    slots = torch.arange(n, dtype=torch.int64, device="cuda")
    mla.mla_cache_write(dev.dims, n, rows, slots, pool, mla.MLA_KV_FP4_E2M1_E4M3, pages, P)
    del rows, slots
    N, H = wl.n_tokens, wl.heads
    q_abs = torch.empty((N, H, wl.d_latent + wl.d_rope), dtype=torch.bfloat16, device="cuda")
    mla.mla_absorb_q(dev.dims, N, dev.q, dev.w_kv_b, q_abs)
    o_lat = torch.empty((N, H, wl.d_latent), device="cuda")
    params = mla.make_decode_params(
        dims=dev.dims, batch=wl.batch, q_per_seq=wl.q_per_seq, q_abs=q_abs, kv_pool=pool,
        kv_format=mla.MLA_KV_FP4_E2M1_E4M3, num_pages=pages, page_block=P, block_table=dev.block_table,
        max_blocks_per_seq=dev.block_table.shape[1], seq_lens=dev.seq_lens, softmax_scale=dev.softmax_scale,
        num_splits=0, o_latent=o_lat, lse=None, q_abs_dtype=mla.MLA_BF16)
    nbytes = mla.mla_decode_workspace_size(params)
    ws = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device="cuda")
    params.workspace, params.workspace_bytes = ws.data_ptr(), nbytes
    mla.mla_decode_paged(params)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e in evs:
        for x in e:
            x.record()
    torch.cuda.synchronize()
    for e in evs:
        params.kernel_start_event, params.kernel_stop_event = e[0].cuda_event, e[1].cuda_event
        mla.mla_decode_paged(params)
    torch.cuda.synchronize()
    us = sum(a.elapsed_time(b) for a, b in evs) / reps * 1e3
    nbytes = int(np.sum(inp.seq_lens.astype(np.int64))) * 288
    used = mla.mla_decode_select_kernel(params)
    return {"row_bytes": 288, "kernel": {1: "simt", 2: "mfma"}[used], "attention_kernel_us": us,
            "bytes": nbytes, "gbs": nbytes / (us * 1e-6) / 1e9}


def prefill_timing(inp, dev, chunk: int, n_seqs: int, reps: int):
    """mla_prefill_paged over the first n_seqs sequences of the batch, each
    treating its last `chunk` cached tokens as the new chunk (seeded N(0, 1)
    queries): time per call (both kernels, torch events on the stream) and
    the algorithmic fp32 flops, K/V rebuild 2 L H (d_nope + d_v) d_latent per
    sequence plus attention 2 H (d_nope + d_rope + d_v) per visible
    (query, token) pair.  Only for d_nope + d_rope <= 256 and d_v <= 256."""
    import numpy as np
    import torch

    import mla_paged_decode_amd as mla

    wl = inp.wl
    if chunk <= 0 or wl.d_nope + wl.d_rope > 256 or wl.d_v > 256:
        return None
    B = min(n_seqs, wl.batch)
    lens = inp.seq_lens[:B].astype(np.int64)
    if int(lens.min()) < chunk or int(lens.sum()) > 65536:  # keep the leg to a fraction of a second
        return None
    H = wl.heads
    g = torch.Generator().manual_seed(9)
    q = torch.randn((B * chunk, H, wl.d_nope + wl.d_rope), generator=g).cuda()
    out = torch.empty((B * chunk, H, wl.d_v), device="cuda")
    bt = dev.block_table[:B].contiguous()  # kept alive: the struct holds raw pointers
    sl = dev.seq_lens[:B].contiguous()
    params = mla.make_prefill_params(
        dims=dev.dims, batch=B, q_per_seq=chunk, q=q, w_kv_b=dev.w_kv_b, kv_pool=dev.kv_pool,
        kv_format=dev.kv_format, num_pages=dev.kv_pool.shape[0], page_block=dev.page_block,
        block_table=bt, max_blocks_per_seq=dev.block_table.shape[1], seq_lens=sl,
        softmax_scale=dev.softmax_scale, out=out)
    nbytes = mla.mla_prefill_workspace_size(params)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
    params.workspace, params.workspace_bytes = ws.data_ptr(), nbytes
    mla.mla_prefill_paged(params)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        mla.mla_prefill_paged(params)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / reps * 1e3
    expand = 2.0 * float(lens.sum()) * H * (wl.d_nope + wl.d_v) * wl.d_latent
    pairs = float(sum(int(L - chunk + i + 1) for L in lens for i in range(chunk)))
    attn = 2.0 * pairs * H * (wl.d_nope + wl.d_rope + wl.d_v)
    tflops = (expand + attn) / (us * 1e-6) / 1e12
    # Both contractions run on the bf16 matrix cores: the rebuild as one bf16
    # product per term (bf16 weights and latent), the attention as three per
    # term (hi * hi + hi * lo + lo * hi, for fp32-level accuracy).  The
    # fraction counts the matrix-core flops so executed against the bf16 peak.
    mfma_flops = expand + 3.0 * attn
    return {"sequences": B, "chunk": chunk, "context": [int(x) for x in lens], "us": us,
            "flops": expand + attn, "flops_rebuild": expand, "flops_attention": attn, "tflops": tflops,
            "mfma_flops_executed": mfma_flops, "peak_bf16_mfma_tflops": BF16_MFMA_PEAK_TFLOPS,
            "frac": mfma_flops / (us * 1e-6) / 1e12 / BF16_MFMA_PEAK_TFLOPS, "kernel": "mfma"}


def decode_timing(wl, splits: int, qd: int, kernel: int, reps: int, cache_bytes: float, warmup: int = 3,
                  extra_flags: int = 0):
    """Eager decode calls on one workload: per call, the decode call
    (mla_decode_paged: attention and merge; torch events around it) and the
    attention kernel alone (HIP events the library records on the launch
    stream).  Calls cycle through copies of the cache, each at its own
    address, so that together they exceed the Infinity Cache."""
    import numpy as np
    import torch

    import mla_paged_decode_amd as mla
    from mla_paged_decode_amd.step import DecodeStep, DeviceBatch
    from synth import make_inputs

    inp = make_inputs(wl)
    mla.mla_validate_tables(inp.seq_lens, inp.block_table, inp.kv_pool.shape[0], wl.page_block)
    dev = DeviceBatch.upload(inp)
    step = DecodeStep(dev, q_abs_dtype=qd, num_splits=splits, kernel=kernel, flags=extra_flags)
    pool_bytes = dev.kv_pool.numel()
    copies = max(1, math.ceil(cache_bytes / pool_bytes))
    pools = [dev.kv_pool] + [dev.kv_pool.clone() for _ in range(copies - 1)]
    step.absorb()
    # untimed calls: at least `warmup`, and at least 30 ms of them, so that
    # the clocks have settled after the host-side input generation
    t_end = time.perf_counter() + 0.03
    i = 0
    while i < warmup or time.perf_counter() < t_end:
        step.params.kv_pool = pools[i % copies].data_ptr()
        step.decode()
        i += 1
        if i % 4 == 0:
            torch.cuda.synchronize()
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(4)) for _ in range(reps)]
    for e in evs:
        for x in e:
            x.record()
    torch.cuda.synchronize()
    # the decode calls, then the attention kernels (events between the
    # attention and merge kernels would delay the merge)
    for i, e in enumerate(evs):
        step.params.kv_pool = pools[i % copies].data_ptr()
        e[0].record()
        step.decode()
        e[1].record()
    for i, e in enumerate(evs):
        step.params.kv_pool = pools[i % copies].data_ptr()
        step.params.kernel_start_event, step.params.kernel_stop_event = e[2].cuda_event, e[3].cuda_event
        step.decode()
    step.params.kernel_start_event = step.params.kernel_stop_event = None
    torch.cuda.synchronize()
    call_us = sum(e[0].elapsed_time(e[1]) for e in evs) / reps * 1e3
    kern_us = sum(e[2].elapsed_time(e[3]) for e in evs) / reps * 1e3
    latent = int(np.sum(inp.seq_lens.astype(np.int64))) * inp.row_bytes
    used = mla.mla_decode_select_kernel(step.params)
    rec = {
        "workload": wl.name, "num_splits": splits, "batch": wl.batch, "q_per_seq": wl.q_per_seq,
        "kv_format": wl.kv_format, "kernel": {1: "simt", 2: "mfma"}[used],
        "q_abs": "f32" if qd == mla.MLA_F32 else "bf16", "cache_copies": copies,
        "latent_bytes": latent, "unique_bytes": pool_bytes,
        "attention_kernel_us": kern_us, "decode_call_us": call_us,
        "attention_frac": latent / (kern_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
        "decode_frac": latent / (call_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
        "decode_query_tokens_per_s": wl.n_tokens / (call_us * 1e-6),
        "traffic": counter_traffic(wl.name, splits),
        "mfma": mfma_utilisation(wl.name, splits),
    }
    del step, pools, dev
    torch.cuda.empty_cache()
    return rec


def parse_extra(spec: str):
    out = []
    for item in filter(None, (x.strip() for x in spec.split(","))):
        name, _, sp = item.partition(":")
        out.append((name, int(sp) if sp else None))
    return out


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # The GPU raises its clocks only after some tens of ms of sustained work:
    # with 5 warm-up steps the first blocks of 20 replayed steps ran at 293,
    # 282 and 275 us per step before settling at 272.  100 untimed steps of
    # each kind (eager, then replayed) reach the settled rate a serving loop
    # runs at.
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="ragged_b256_h20_ctx512_8k_bf16")
    ap.add_argument("--num-splits", type=int, default=0,
                    help="split-KV chunks per sequence (0 = balanced, the default; -1: the workload's own)")
    ap.add_argument("--extra", default="long_b4_h20_ctx65k_203k_bf16:0,long_b4_h20_ctx65k_203k_bf16:32,"
                                       "fp8_mtp4_b64_h20_ctx16k:0",
                    help="comma-separated workload[:num_splits] sub-records (decode call and attention "
                         "kernel, eager); empty: none")
    ap.add_argument("--extra-reps", type=int, default=10)
    ap.add_argument("--kernel", choices=["auto", "simt", "mfma"], default="auto")
    ap.add_argument("--fused-merge", action="store_true",
                    help="set MLA_DECODE_FUSED_MERGE (merge inside the attention kernel where it applies; "
                         "measured slower on MI355X)")
    ap.add_argument("--q-abs", choices=["auto", "bf16", "f32"], default="auto",
                    help="absorbed-query dtype fed to the attention kernel; auto: f32 (hi + lo bf16 "
                         "products) for bf16 and f32 caches, bf16 for the fp8 cache")
    ap.add_argument("--cache-bytes", type=float, default=1.0e9,
                    help="total bytes of rotated cache copies (>= 4x the Infinity Cache)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prefill-chunk", type=int, default=256,
                    help="also time mla_prefill_paged with this many new tokens on 4 sequences (0: skip)")
    ap.add_argument("--sparse-topk", type=int, default=2048,
                    help="also time mla_decode_sparse_paged over this many listed tokens per query (0: skip)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="run one plain device-to-device copy of this many MiB before the timed "
                         "region, as the reference kernel for scaling byte counters")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the library has no "
              f"multi-GPU path; sequences would shard across GPUs with no exchange.",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import mla_paged_decode_amd as mla
    from mla_paged_decode_amd.step import DecodeStep, DeviceBatch
    from synth import WORKLOADS, make_inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    mla.lib()
    wl = WORKLOADS[args.workload]
    splits = wl.num_splits if args.num_splits < 0 else args.num_splits
    kernel = {"auto": mla.MLA_KERNEL_AUTO, "simt": mla.MLA_KERNEL_SIMT, "mfma": mla.MLA_KERNEL_MFMA}[args.kernel]

    def q_dtype(w):
        q = args.q_abs if args.q_abs != "auto" else ("bf16" if w.kv_format == "fp8_e4m3_e8m0" else "f32")
        return mla.MLA_BF16 if q == "bf16" and kernel != mla.MLA_KERNEL_SIMT else mla.MLA_F32

    qd = q_dtype(wl)
    log(f"[bench] generating {wl.name}")
    inp = make_inputs(wl)
    mla.mla_validate_tables(inp.seq_lens, inp.block_table, inp.kv_pool.shape[0], wl.page_block)
    dev = DeviceBatch.upload(inp)
    flags = mla.MLA_DECODE_ALLOW_BF16_QUERIES if qd == mla.MLA_BF16 and wl.kv_format in ("bf16", "f32") else 0
    # --fused-merge: the merge inside the attention kernel (the step's
    # workspace is zero-filled once at allocation, as that mode asks).
    fused = mla.MLA_DECODE_FUSED_MERGE if args.fused_merge else 0
    step = DecodeStep(dev, q_abs_dtype=qd, num_splits=splits, kernel=kernel, flags=flags | fused)
    pool_bytes = dev.kv_pool.numel()
    copies = max(1, math.ceil(args.cache_bytes / pool_bytes))
    pools = [dev.kv_pool] + [dev.kv_pool.clone() for _ in range(copies - 1)]
    log(f"[bench] {copies} cache copies of {pool_bytes / 1e6:.1f} MB")

    if args.calibrate_copy_mib > 0:
        src = torch.empty(args.calibrate_copy_mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"[bench] calibration copy of {args.calibrate_copy_mib} MiB done")

    latent_bytes = int(np.sum(inp.seq_lens.astype(np.int64))) * inp.row_bytes
    unique_bytes = pool_bytes  # every page of the pool is referenced once or more
    q_tokens = wl.n_tokens

    def one_step(i, ev=None, kernel_ev=None):
        """One step; ev = (start, stop) events around the decode call, or
        kernel_ev = (start, stop) events the library records around the
        attention kernel (never both: events between the attention and merge
        kernels delay the merge and would inflate the call's time)."""
        step.params.kv_pool = pools[i % copies].data_ptr()
        step.absorb()
        if ev is not None:
            ev[0].record()
        if kernel_ev is not None:
            step.params.kernel_start_event = kernel_ev[0].cuda_event
            step.params.kernel_stop_event = kernel_ev[1].cuda_event
        step.decode()
        if ev is not None:
            ev[1].record()
        step.params.kernel_start_event = None
        step.params.kernel_stop_event = None
        step.project()

    for i in range(args.warmup):
        one_step(i)
    torch.cuda.synchronize()
    log(f"[bench] eager warmup {args.warmup} done")

    # Timed region 1 (the metric): whole steps replayed from HIP graphs, one
    # graph per cache copy, so the measurement is the GPU's work and not the
    # host's launch rate.
    graphs = []
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(copies):
            one_step(i)
    torch.cuda.current_stream().wait_stream(side)
    for i in range(copies):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            one_step(i)
        graphs.append(g)
    for i in range(args.warmup):
        graphs[i % copies].replay()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        graphs[i % copies].replay()
    stop.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    ms_per_step = total_ms / args.steps

    # Timed region 2 (the roofline): eager steps, twice: first with events
    # around each decode call (attention + merge), then with the events the
    # library records on the launch stream around the attention kernel alone.
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(4)) for _ in range(args.steps)]
    for e in evs:
        for x in e:
            x.record()  # creates the underlying HIP event
    torch.cuda.synchronize()
    for i in range(args.steps):
        one_step(i, ev=evs[i][:2])
    torch.cuda.synchronize()
    for i in range(args.steps):
        one_step(i, kernel_ev=evs[i][2:])
    torch.cuda.synchronize()
    decode_ms = [e[0].elapsed_time(e[1]) for e in evs]
    kernel_ms = [e[2].elapsed_time(e[3]) for e in evs]
    decode_avg_s = sum(decode_ms) / len(decode_ms) / 1e3
    kernel_avg_s = sum(kernel_ms) / len(kernel_ms) / 1e3
    achieved_call = latent_bytes / decode_avg_s / 1e9
    achieved = latent_bytes / kernel_avg_s / 1e9
    log(f"[bench] {args.steps} graph-replayed steps: {ms_per_step * 1e3:.1f} us/step; eager: decode call "
        f"{decode_avg_s * 1e6:.1f} us ({achieved_call:.0f} GB/s), attention kernel "
        f"{kernel_avg_s * 1e6:.1f} us ({achieved:.0f} GB/s)")

    cache_write = cache_write_timing(inp, dev, args.steps)
    log(f"[bench] mla_cache_write of {cache_write['rows']} new rows: {cache_write['us']:.1f} us")
    sparse = None
    if args.sparse_topk > 0:
        # about 512 workgroups (measured: GLM batch best at 16 chunks, 256 sequences at 2-4)
        pairs = wl.batch * wl.q_per_seq
        chunks = max(1, min((args.sparse_topk + 31) // 32, round(512 / pairs)))
        sparse = sparse_timing(inp, dev, step.q_abs, qd, args.sparse_topk, chunks, min(args.steps, 10))
        log(f"[bench] sparse decode over {args.sparse_topk} listed tokens per query: "
            f"{sparse['attention_kernel_us']:.1f} us ({sparse['gbs']:.0f} GB/s)")
    fp4 = fp4_timing(inp, dev, min(args.steps, 5))
    if fp4 is not None:
        log(f"[bench] fp4 cache copy: attention kernel {fp4['attention_kernel_us']:.1f} us ({fp4['gbs']:.0f} GB/s)")
    prefill = prefill_timing(inp, dev, args.prefill_chunk, 4, 3)
    if prefill is not None:
        log(f"[bench] prefill of {prefill['chunk']} new tokens on {prefill['sequences']} sequences: "
            f"{prefill['us'] / 1e3:.2f} ms ({prefill['tflops']:.1f} TFLOP/s algorithmic, "
            f"{prefill['frac']:.3f} of the bf16 matrix-core peak)")
    used = mla.mla_decode_select_kernel(step.params)
    main_cfg = {
        "workload": wl.name, "batch": wl.batch, "heads": wl.heads, "q_per_seq": wl.q_per_seq,
        "context": list(wl.lens), "page_block": wl.page_block, "kv_format": wl.kv_format,
        "d_latent": wl.d_latent, "d_rope": wl.d_rope, "num_splits": splits,
        "kernel": {1: "simt", 2: "mfma"}[used], "q_abs": "f32" if qd == mla.MLA_F32 else "bf16",
        "cache_copies": copies, "fused_merge_flag": args.fused_merge,
    }
    del graphs, step, pools, dev
    torch.cuda.empty_cache()

    extras = []
    for name, sp in parse_extra(args.extra):
        w = WORKLOADS[name]
        sp = w.num_splits if sp is None else sp
        log(f"[bench] sub-record {name} num_splits={sp}")
        rec = decode_timing(w, sp, q_dtype(w), kernel, args.extra_reps, args.cache_bytes,
                            extra_flags=mla.MLA_DECODE_FUSED_MERGE if args.fused_merge else 0)
        log(f"[bench]   attention kernel {rec['attention_kernel_us']:.1f} us ({rec['attention_frac']:.3f} of 8 TB/s), "
            f"decode call {rec['decode_call_us']:.1f} us ({rec['decode_frac']:.3f})")
        extras.append(rec)

    base = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle")
        base = cpu_baseline(wl, args.cpu_seconds)

    qtok_s = q_tokens / (ms_per_step / 1e3)
    compute = "f32" if used == mla.MLA_KERNEL_SIMT else "bf16"
    line = {
        "metric": METRIC,
        "value": qtok_s,
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": compute,
        "data": "synthetic",
        "config": main_cfg,
        "hbm_gbs": achieved_call,
        "pct_of_8tbs": 100.0 * achieved_call / HBM_PEAK_GBS,
        "decode_call_us": decode_avg_s * 1e6,
        "attention_kernel_us": kernel_avg_s * 1e6,
        "decode_frac": achieved_call / HBM_PEAK_GBS,
        "latent_bytes": latent_bytes,
        "unique_bytes": unique_bytes,
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": counter_traffic(wl.name, splits),
        },
        "mfma": mfma_utilisation(wl.name, splits),
        "cpu_baseline": base,
        "configs": extras,
        "cache_write": cache_write,
        "sparse_decode": sparse,
        "fp4_decode": fp4,
        "prefill": prefill,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
