"""Upload seeded host inputs (sparse_attention_14_amd.inputs.Problem) to the GPU.

Plumbing only: copies numpy storage into torch device tensors and builds the
dsa_cache descriptors the library takes.  Every host->device copy completes
before this returns (torch.cuda.synchronize), so no kernel can read a buffer
whose upload is still in flight.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from .binding import DeviceCache


def _t(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def upload_cache(cache, device="cuda") -> DeviceCache:
    rows = _t(cache.storage.reshape(-1), device)
    scale = None if cache.scale is None else _t(cache.scale.astype(np.float32).reshape(-1), device)
    table = None if cache.block_table is None else _t(cache.block_table.astype(np.int32), device)
    return DeviceCache(rows, cache.dtype, cache.width, cache.block_size, cache.row_stride, cache.block_stride,
                       scale=scale, scale_block_stride=cache.scale_block_stride, block_table=table)


def _q(a: np.ndarray, dtype: str, device) -> torch.Tensor:
    if dtype == "f32":
        return _t(a.astype(np.float32), device)
    return _t(a.view(np.int16), device)   # bf16 raw bits


@dataclass
class DeviceProblem:
    q_idx: torch.Tensor
    w_idx: torch.Tensor
    keys: DeviceCache
    q_mla: torch.Tensor
    latent: DeviceCache
    q_seq: torch.Tensor
    q_len: torch.Tensor
    host: object


def upload(p, device="cuda") -> DeviceProblem:
    dp = DeviceProblem(q_idx=_q(p.q_idx, p.q_idx_dtype, device), w_idx=_t(p.w_idx, device),
                       keys=upload_cache(p.keys, device), q_mla=_q(p.q_mla, p.q_mla_dtype, device),
                       latent=upload_cache(p.latent, device), q_seq=_t(p.q_seq.astype(np.int32), device),
                       q_len=_t(p.q_len.astype(np.int32), device), host=p)
    torch.cuda.synchronize()
    return dp
