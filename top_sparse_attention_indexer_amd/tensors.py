"""Moves synthetic host arrays into device tensors of the workload's dtypes.

Plumbing for tests and the bench: float32 host values that are bf16-exact
become torch.bfloat16 device tensors (an exact conversion), the rest keep
their types.  No arithmetic of the method happens here.
"""
from __future__ import annotations

from typing import Dict

import numpy as np
import torch


def to_device(w, x: Dict[str, np.ndarray], device="cuda") -> Dict[str, torch.Tensor]:
    qkv = torch.bfloat16 if w.qkv_dtype == "bf16" else torch.float32
    idx = torch.bfloat16 if w.idx_dtype == "bf16" else torch.float32
    kinds = {"q_idx": idx, "k_idx": idx, "q": qkv, "k": qkv, "v": qkv,
             "gate": torch.float32, "y2": torch.float32}
    out = {}
    for name, arr in x.items():
        if name == "route":
            out[name] = torch.from_numpy(np.ascontiguousarray(arr)).to(device)
        elif name in kinds:
            t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)
            out[name] = t.to(kinds[name]).contiguous()
    return out
