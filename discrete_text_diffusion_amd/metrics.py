"""Inference-efficiency accounting of block-AR generation [TR §추론 효율 지표] from the per-canvas
outputs of dg_generate (host arithmetic on [K][B] arrays).

With K_b canvases up to and including sequence b's first EOS (all K if none), s_k denoising steps
and n_k valid tokens of canvas k: tokens = sum n_k, steps = sum s_k, effective denoising steps =
sum n_k s_k / tokens, TPF = tokens / (steps + K_b - 1) (the K_b - 1 forward passes that append a
finished canvas to the cache), TPS = TPF / t_fwd for a measured time t_fwd of one forward pass.
"""
from __future__ import annotations

import numpy as np


def block_ar_metrics(steps, valid, eos_seen, t_fwd_s=None):
    """steps, valid, eos_seen: [K][B] (torch tensors or arrays).  Returns one dict per sequence."""
    s = np.asarray(steps.cpu() if hasattr(steps, "cpu") else steps, dtype=np.float64)
    n = np.asarray(valid.cpu() if hasattr(valid, "cpu") else valid, dtype=np.float64)
    e = np.asarray(eos_seen.cpu() if hasattr(eos_seen, "cpu") else eos_seen).astype(bool)
    K, B = s.shape
    res = []
    for b in range(B):
        first = np.argmax(e[:, b]) if e[:, b].any() else K - 1
        kb = int(first) + 1
        tok, stp = n[:kb, b].sum(), s[:kb, b].sum()
        d = {"canvases": kb, "tokens": float(tok), "steps": float(stp),
             "effective_steps": float((n[:kb, b] * s[:kb, b]).sum() / tok) if tok > 0 else 0.0,
             "tpf": float(tok / (stp + kb - 1)) if stp + kb - 1 > 0 else 0.0}
        if t_fwd_s:
            d["tps"] = d["tpf"] / t_fwd_s
        res.append(d)
    return res
