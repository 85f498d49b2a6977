"""Degenerate and extreme shapes of the denoising pass against the oracle.

- no prefix at all (attention over the canvas alone: zero prefix key tiles);
- a sliding-window layer whose prefix is shorter than its window (a partly filled ring);
- the shortest canvas the boundary accepts (16 positions, one partial key tile) and the longest
  (1024 positions, 16 canvas key tiles and 16 query blocks per KV head).

bf16 on a small model with head_dim 256 (the bf16 attention kernels) and top-k = all experts, so
that no near-tie reroute separates the two sides: the fp32 residual before the final norm within
2e-2.  fp32 on the tiny model: the hidden states within 1e-4."""
import numpy as np
import pytest
import torch

from oracle import model as M
from synth import configs
from tests.gpu_util import build, log
from tests.helpers import np64, oracle_kv_dev, oracle_weights
from tests.test_gpu_mixed import SMALL_BF16, _tokens

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _denoise(cfg, plen, L, seed):
    model, W, kv = build(cfg)
    model.set_kv(kv, plen)
    B = len(plen)
    toks = _tokens(cfg, B, L, seed)
    ws = model.workspace(B, L, cfg.prefix)
    dt = torch.float32 if cfg.act_dtype == "f32" else torch.bfloat16
    H = torch.empty(B * L, cfg.d_model, dtype=dt, device=DEV)
    R = torch.empty(B * L, cfg.d_model, dtype=torch.float32, device=DEV)
    log(f"  {cfg.name}: canvas {L}, prefixes {plen}")
    model.denoise_step(toks, L, ws, hidden_out=H, resid_out=R)
    torch.cuda.synchronize()
    oH, oR = M.denoise_forward(cfg, oracle_weights(W, cfg), oracle_kv_dev(kv), plen, canvas=toks.cpu().numpy())
    return np64(H), oH, R.cpu().numpy(), oR


@pytest.mark.parametrize("plen,L", [([0, 40, 100], 16), ([0], 1024), ([30], 1024)])
def test_small_bf16_denoise_edge_shapes(plen, L):
    """Layer 0 is a 64-slot ring, layer 1 global; prefix 40 < window 64 leaves the ring partly
    filled, 100 wraps it."""
    cfg = SMALL_BF16.replace(batch=len(plen))
    got, want, r, oR = _denoise(cfg, plen, L, 61)
    er = float(np.abs(r - oR).max())
    log(f"  max |resid - oracle| {er:.2e} (bf16 H: {np.abs(got - want).max():.2e}, reported)")
    assert er <= 2e-2


@pytest.mark.parametrize("plen,L", [([0, 5], 16), ([0], 1024)])
def test_tiny_fp32_denoise_edge_shapes(plen, L):
    """The tiny model with a 16-slot ring layer and a global layer."""
    cfg = configs.C0.replace(batch=len(plen), window=16, global_every=2, prefix=64, kv_source="random")
    got, want, r, oR = _denoise(cfg, plen, L, 71)
    err = max(float(np.abs(got - want).max()), float(np.abs(r - oR).max()))
    log(f"  max |H - oracle| {err:.2e}")
    assert err <= 1e-4
