"""dg_step_sample_noalloc (the Step for callers that cannot allocate: scratch in a static device array)
against dg_step_sample with a caller workspace: the same kernels, so canvas, locks and locked counts
must agree bit for bit.  Two calls in a row on the same GPU, the second with a smaller input, so the
second runs over the first one's leftovers in the shared array."""
import numpy as np
import pytest
import torch

from discrete_text_diffusion_amd import dg
from synth import configs, gen
from tests.gpu_util import build, log

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _pair(model, cfg, B, L, seed, t, theta):
    H = gen.hidden_input(cfg.replace(batch=B, canvas=L), DEV)
    cv0 = torch.empty(B, L, dtype=torch.int32, device=DEV)
    dg.dg_init_canvas(cv0, None, B, L, cfg.vocab, seed)
    lk0 = torch.zeros(B, L, dtype=torch.uint8, device=DEV)
    lk0[:, ::5] = 1
    p = dg.StepParams(schedule=cfg.schedule, t=t, h=0.25, tau=cfg.tau, lock_threshold=theta, seed=seed, step=1)
    ws = model.workspace(B, L, 0)
    out = {}
    for name in ("workspace", "noalloc"):
        cv, lk = cv0.clone(), lk0.clone()
        nl = torch.full((B,), -7, dtype=torch.int32, device=DEV)
        if name == "workspace":
            dg.dg_step_sample(model.ctx, H, cv, lk, nl, None, B, L, p, ws)
        else:
            dg.dg_step_sample_noalloc(model.ctx, H, cv, lk, nl, None, B, L, p)
        torch.cuda.synchronize()
        out[name] = (cv.cpu().numpy(), lk.cpu().numpy(), nl.cpu().numpy())
    changed = int((out["noalloc"][0] != cv0.cpu().numpy()).sum())
    log(f"  B={B} L={L}: tokens changed by the Step {changed}, locked {out['noalloc'][2].tolist()}")
    for a, b in zip(out["workspace"], out["noalloc"]):
        assert np.array_equal(a, b)
    assert changed > 0


@pytest.mark.parametrize("case", ["vocab262k-bf16", "tiny-fp32"])
def test_noalloc_step_equals_workspace_step_twice(case):
    if case == "tiny-fp32":
        cfg = configs.C0
        first, second = (3, 64), (1, 32)
        theta = 0.002            # some positions lock at this vocabulary's confidences
    else:
        cfg = configs.C2.replace(n_layers=1)
        first, second = (2, 256), (1, 64)
        theta = 2.0
    log(f"[noalloc] {case}: calls with {first} then {second} canvases x positions")
    model, _, _ = build(cfg)
    _pair(model, cfg, *first, seed=3, t=0.75, theta=theta)
    _pair(model, cfg, *second, seed=4, t=0.5, theta=theta)
