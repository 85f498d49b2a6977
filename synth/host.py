"""Host copies of the seeded storage tensors as float64 NumPy arrays (dtype plumbing only).

bf16 / fp32 tensors widen exactly to float64; uint8 tensors (fp8 or MXFP4 codes and e8m0 scales)
are returned as their raw bytes.  Nothing here computes any part of the method.
"""
from __future__ import annotations

import numpy as np
import torch


def np64(t):
    """A storage tensor (any device) as a float64 array, or its raw bytes for uint8 codes."""
    if t is None:
        return None
    if t.dtype == torch.uint8:
        return t.cpu().numpy()
    return t.float().cpu().numpy().astype(np.float64)


def layer_np(L: dict) -> dict:
    """Every tensor of one layer's storage dict through np64."""
    return {k: np64(v) for k, v in L.items()}
