"""One MLA decode step on the GPU: device buffers plus the three library calls.

torch provides the device memory and the stream; the arithmetic is
libmla's (mla_absorb_q -> mla_decode_paged -> mla_out_proj).
"""
from __future__ import annotations

from dataclasses import dataclass
import numpy as np
import torch

from . import (KV_FORMAT, MLA_F32, MLA_KERNEL_AUTO, Dims, make_decode_params,
               mla_absorb_q, mla_decode_paged, mla_decode_workspace_size, mla_out_proj)


def _as_device(a: np.ndarray, device) -> torch.Tensor:
    """Host array -> device tensor; uint16 arrays are bf16 bit patterns."""
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


@dataclass
class DeviceBatch:
    """Inputs of one decode step resident in device memory."""

    dims: Dims
    batch: int
    q_per_seq: int
    kv_format: int
    page_block: int
    softmax_scale: float
    q: torch.Tensor            # [N, H, d_nope + d_rope]
    w_kv_b: torch.Tensor       # [H, d_nope + d_v, d_latent]
    kv_pool: torch.Tensor      # [num_pages, P, row_bytes] uint8
    block_table: torch.Tensor  # [B, max_blocks] int32
    seq_lens: torch.Tensor     # [B] int32

    @property
    def n_tokens(self) -> int:
        return self.batch * self.q_per_seq

    @classmethod
    def upload(cls, inp, device="cuda") -> "DeviceBatch":
        """From host buffers with the layout of synth.Inputs."""
        wl = inp.wl
        return cls(
            dims=Dims(wl.heads, wl.d_latent, wl.d_rope, wl.d_nope, wl.d_v),
            batch=wl.batch, q_per_seq=wl.q_per_seq, kv_format=KV_FORMAT[wl.kv_format],
            page_block=wl.page_block, softmax_scale=wl.softmax_scale,
            q=_as_device(inp.q, device), w_kv_b=_as_device(inp.w_kv_b, device),
            kv_pool=_as_device(inp.kv_pool, device),
            block_table=_as_device(inp.block_table, device),
            seq_lens=_as_device(inp.seq_lens, device))


class DecodeStep:
    """Allocates the step's outputs and workspace once; run() launches the
    three calls on the stream."""

    def __init__(self, dev: DeviceBatch, *, q_abs_dtype: int = MLA_F32, num_splits: int = 0,
                 kernel: int = MLA_KERNEL_AUTO, with_lse: bool = True, flags: int = 0):
        d = dev.dims
        N, H = dev.n_tokens, d.num_heads
        device = dev.q.device
        self.dev = dev
        qt = torch.float32 if q_abs_dtype == MLA_F32 else torch.bfloat16
        self.q_abs = torch.empty((N, H, d.d_latent + d.d_rope), dtype=qt, device=device)
        self.o_latent = torch.empty((N, H, d.d_latent), dtype=torch.float32, device=device)
        self.lse = torch.empty((N, H), dtype=torch.float32, device=device) if with_lse else None
        self.out = torch.empty((N, H, d.d_v), dtype=torch.float32, device=device)
        self.params = make_decode_params(
            dims=d, batch=dev.batch, q_per_seq=dev.q_per_seq, q_abs=self.q_abs,
            kv_pool=dev.kv_pool, kv_format=dev.kv_format, num_pages=dev.kv_pool.shape[0],
            page_block=dev.page_block, block_table=dev.block_table,
            max_blocks_per_seq=dev.block_table.shape[1], seq_lens=dev.seq_lens,
            softmax_scale=dev.softmax_scale, num_splits=num_splits, kernel=kernel,
            o_latent=self.o_latent, lse=self.lse, q_abs_dtype=q_abs_dtype, flags=flags)
        nbytes = mla_decode_workspace_size(self.params)
        # zero-filled once: its counter region must start at zero (calls keep it so)
        self.workspace = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=device)
        self.params.workspace = self.workspace.data_ptr()
        self.params.workspace_bytes = nbytes

    def absorb(self, stream=None) -> None:
        dv = self.dev
        mla_absorb_q(dv.dims, dv.n_tokens, dv.q, dv.w_kv_b, self.q_abs, stream=stream)

    def decode(self, stream=None) -> None:
        mla_decode_paged(self.params, stream=stream)

    def project(self, stream=None) -> None:
        dv = self.dev
        mla_out_proj(dv.dims, dv.n_tokens, self.o_latent, dv.w_kv_b, self.out, stream=stream)

    def run(self, stream=None) -> torch.Tensor:
        self.absorb(stream)
        self.decode(stream)
        self.project(stream)
        return self.out

