"""Test-side marshalling: problems from gbsa_inputs to oracle inputs (numpy bit patterns)."""
from __future__ import annotations

import numpy as np
import torch

from oracle.attention import Inputs


def storage_numpy(t: torch.Tensor, dtype: str) -> np.ndarray:
    t = t.detach().cpu()
    if dtype == "f16":
        return t.numpy()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    if dtype == "fp8":
        return t.view(torch.uint8).numpy()
    raise ValueError(dtype)


def oracle_inputs(p, q=None, k=None, v=None) -> Inputs:
    """Oracle view of a problem; q/k/v may be given as already-host numpy bit patterns."""
    q = storage_numpy(p.q, p.dtype) if q is None else q
    k = storage_numpy(p.k, p.dtype) if k is None else k
    v = storage_numpy(p.v, p.dtype) if v is None else v
    return Inputs(q, k, v, p.sparse_block_idx, p.sparse_block_count, p.cu_seqlens_q,
                  p.seqused_q, p.seqused_kv, p.block_table, dtype=p.dtype, block_x=p.block_x,
                  scale=p.scale, mask_mode=p.mask_mode, win_left=p.win_left,
                  win_right=p.win_right, q_scale=p.q_scale, k_scale=p.k_scale,
                  v_scale=p.v_scale)


def dequant(t: torch.Tensor, dtype: str, scale=None, head_axis=None) -> torch.Tensor:
    """float64 copy of a storage tensor via torch's own dtype conversion."""
    x = t.detach().cpu().to(torch.float64)
    if scale is not None:
        shape = [1] * x.dim()
        shape[head_axis] = -1
        x = x * torch.as_tensor(scale, dtype=torch.float64).view(shape)
    return x
