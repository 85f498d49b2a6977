"""Shared plumbing for the GPU parity tests: device inputs from `synth`, the library model
wrapper, and host copies for the oracle."""
import sys

import numpy as np
import torch

from discrete_text_diffusion_amd import dg
from discrete_text_diffusion_amd.model import Model, values_dmajor
from synth import gen


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def build(cfg, kv_mode=None):
    """Seeded weights and caches for `cfg` on cuda:0 and a library Model around them; the caches
    are returned in the library's layout (values d-major)."""
    dev = torch.device("cuda:0")
    W = gen.make_weights(cfg, dev)
    mode = kv_mode or cfg.kv_source
    if mode == "random":
        kv = gen.make_random_kv(cfg, dev)
        plen = [cfg.prefix] * cfg.batch
    else:
        kv = gen.empty_kv(cfg, dev)
        plen = [0] * cfg.batch
    kv = values_dmajor(kv)
    return Model(cfg, W, kv, plen), W, kv


def step_params(schedule, t, h, tau, theta, seed, step):
    return dg.StepParams(schedule=schedule, t=t, h=h, tau=tau, lock_threshold=theta, seed=seed, step=step)


def read_stats(model, ws, rows):
    dev = torch.device("cuda:0")
    m = torch.empty(rows, dtype=torch.float32, device=dev)
    a = torch.empty(rows, dtype=torch.int32, device=dev)
    c = torch.empty(rows, dtype=torch.float32, device=dev)
    y = torch.empty(rows, dtype=torch.int32, device=dev)
    best = torch.empty(rows, dtype=torch.float32, device=dev)
    H = torch.empty(rows, dtype=torch.float32, device=dev)
    dg.dg_test_read_stats(model.ctx, ws, rows, m, a, c, y, best, H)
    torch.cuda.synchronize()
    return {"m": m.cpu().numpy(), "a": a.cpu().numpy(), "c": c.cpu().numpy(), "y": y.cpu().numpy(),
            "best": best.cpu().numpy(), "H": H.cpu().numpy()}


def check_routing(cfg, gidx, g_r, info):
    """Routing parity of one layer.  The GPU's selection gidx must be exactly the top-k of its own fp32
    router scores g_r (bit-exact given equal scores).  It may differ from the oracle's own selection
    (info["idx"] from scores info["r32"]) only on a row whose k-th/(k+1)-th oracle score gap is within
    twice that row's own measured score error, and on at most max(2, 2.5%) of the rows: a systematic
    score error could otherwise excuse many rows.  Returns (selection for the oracle to take,
    rerouted rows, max score error)."""
    from oracle import model as M
    sel_from_gpu_scores, _ = M.router_topk(g_r, cfg.top_k)
    assert np.array_equal(gidx, sel_from_gpu_scores), "GPU top-k is not the top-k of its own scores"
    row_err = np.abs(g_r - info["r32"]).max(axis=1)
    lg_err = float(row_err.max())
    assert lg_err <= (1e-4 if cfg.act_dtype == "f32" else 2e-2), f"router logits differ by {lg_err}"
    r = info["r32"].astype(np.float64)
    srt = -np.sort(-r, axis=1)
    gap = srt[:, cfg.top_k - 1] - srt[:, cfg.top_k] if cfg.top_k < cfg.n_experts else np.full(len(r), np.inf)
    near = gap <= 2 * row_err + 1e-6
    mism = np.any(np.sort(gidx, 1) != np.sort(info["idx"], 1), axis=1)
    n = int(mism.sum())
    print(f"  routing: score error max {lg_err:.2e} (row median {np.median(row_err):.2e}); rows within their "
          f"own error of a tie {int(near.sum())}; rerouted {n} of {len(r)}", flush=True)
    assert not (mism & ~near).any(), f"routing differs beyond the row's score error at rows {np.nonzero(mism & ~near)[0][:8]}"
    assert n <= max(2, len(r) * 25 // 1000), f"{n} of {len(r)} rows rerouted"
    return np.where(mism[:, None], gidx, info["idx"]), n, lg_err


def top2_gap(z):
    p = np.partition(z, -2, axis=-1)
    return p[..., -1] - p[..., -2]


def compare_step(gpu_canvas, gpu_lock, gpu_stats, orc_canvas, orc_lock, orc_stats, z_gap, theta,
                 y_gap_tol=1e-3, a_gap_tol=1e-5, c_tol=1e-5):
    """Selection parity: token ids, argmaxes and locks equal except where the oracle's own margin
    says floating-point order may decide (Gumbel top-2 gap < y_gap_tol, logit top-2 gap <
    a_gap_tol, |c - theta| < c_tol).  Returns the number of rows whose token or lock actually
    differs under such an excuse (rows that agree are not counted)."""
    ga, gy, gc = gpu_stats["a"], gpu_stats["y"], gpu_stats["c"]
    oa, oy, oc = orc_stats["a"], orc_stats["y"], orc_stats["c"]
    excuse_a = z_gap < a_gap_tol
    excuse_y = orc_stats["gap"] < y_gap_tol
    excuse_c = np.abs(oc - theta) < c_tol
    bad_a = (ga != oa) & ~excuse_a
    bad_y = (gy != oy) & ~excuse_y
    assert not bad_a.any(), f"argmax differs at rows {np.nonzero(bad_a)[0][:10]}"
    assert not bad_y.any(), f"Gumbel argmax differs at rows {np.nonzero(bad_y)[0][:10]}"
    excused = ((ga != oa) | (gy != oy) | excuse_c).reshape(gpu_canvas.shape)
    differ = (gpu_canvas != orc_canvas) | (gpu_lock.astype(bool) != orc_lock)
    diff = differ & ~excused
    assert not diff.any(), f"canvas or lock differs at {np.argwhere(diff)[:10]}"
    return int((differ & excused).sum())


def max_excused(rows):
    """Disagreements the 99.9% agreement rule allows among `rows` checked rows."""
    return rows // 1000
