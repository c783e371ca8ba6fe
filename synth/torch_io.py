"""Moves generated numpy inputs onto the GPU as torch tensors (bit for bit)."""
from __future__ import annotations

import numpy as np
import torch


def to_device(a: np.ndarray, kind: str, device="cuda") -> torch.Tensor:
    """kind: 'bf16' (uint16 bit patterns), 'f32', 'u8' or 'i32'."""
    if kind == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    elif kind == "f32":
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    elif kind == "u8":
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8))
    elif kind == "i32":
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32))
    else:
        raise ValueError(kind)
    return t.to(device)


def act(a: np.ndarray, wl, device="cuda") -> torch.Tensor:
    """An activation / cache tensor in the workload's storage dtype."""
    return to_device(a, "bf16" if wl.dtype == "bf16" else "f32", device)
