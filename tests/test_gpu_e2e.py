"""End-to-end parity on the tiny fp32 denoiser: causal prefill of 64 random tokens, then the
4-step linear-schedule canvas run.  Each step is teacher-forced (the oracle recomputes the
decoder pass and the Step from the GPU's canvas) so a single excused near-tie cannot cascade;
dg_canvas_run must then reproduce the step-by-step loop bit for bit, and the oracle's own
free-running loop must reach the same canvas.  The adaptive loop (stop once all positions are
locked) is checked with a low temperature that makes positions lock."""
import numpy as np
import pytest
import torch

from discrete_text_diffusion_amd import dg
from oracle import model as M
from oracle import step as S
from synth import configs, gen
from tests.gpu_util import build, compare_step, log, max_excused, read_stats, step_params, top2_gap
from tests.helpers import np64, oracle_kv, oracle_kv_dev, oracle_weights

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _prefilled(cfg):
    model, W, kv = build(cfg, kv_mode="empty")
    ws = model.workspace(cfg.batch, max(cfg.canvas, cfg.prefix), cfg.prefix)
    toks = gen.prefix_tokens(cfg).to(DEV)
    model.prefill_kv(toks, ws)
    torch.cuda.synchronize()
    OW = oracle_weights(W, cfg)
    okv, plen = M.prefill(cfg, OW, oracle_kv(gen.empty_kv(cfg)), [0] * cfg.batch, toks.cpu().numpy())
    return model, W, kv, ws, OW, okv, plen


def test_prefill_matches_oracle():
    cfg = configs.C0
    model, W, kv, ws, OW, okv, plen = _prefilled(cfg)
    assert model.prefix_len == plen == [64]
    for l in range(cfg.n_layers):
        for j in range(2):
            got = np64(kv[l][0]) if j == 0 else np64(kv[l][1].transpose(-1, -2))
            err = np.abs(got - okv[l][j]).max()
            log(f"  layer {l} {'KV'[j]} cache max err {err:.2e}")
            assert err <= 1e-4


def test_tiny_fp32_canvas_run_teacher_forced_and_free_running():
    cfg = configs.C0
    B, L, V = cfg.batch, cfg.canvas, cfg.vocab
    model, W, kv, ws, OW, okv, plen = _prefilled(cfg)
    ws = model.workspace(B, L, cfg.prefix)
    cv = torch.empty(B, L, dtype=torch.int32, device=DEV)
    dg.dg_init_canvas(cv, None, B, L, V, cfg.seed)
    lk = torch.zeros(B, L, dtype=torch.uint8, device=DEV)
    nl = torch.empty(B, dtype=torch.int32, device=DEV)
    H = torch.empty(B * L, cfg.d_model, dtype=torch.float32, device=DEV)
    R = torch.empty(B * L, cfg.d_model, dtype=torch.float32, device=DEV)
    ts, h = S.time_grid(cfg.steps)
    excused_total = 0
    for s, t in enumerate(ts):
        before = cv.cpu().numpy().copy()
        lock_before = lk.cpu().numpy().astype(bool)
        model.denoise_step(cv, L, ws, hidden_out=H, resid_out=R)
        model.step_sample(H, cv, lk, nl, step_params(cfg.schedule, t, h, cfg.tau, cfg.lock_threshold, cfg.seed, s), ws)
        torch.cuda.synchronize()
        oH, oR = M.denoise_forward(cfg, OW, okv, plen, canvas=before)
        eh = np.abs(H.cpu().numpy() - oH).max()
        er = np.abs(R.cpu().numpy() - oR).max()
        log(f"  step {s}: |H - oracle| {eh:.2e}, |resid - oracle| {er:.2e}")
        assert eh <= 1e-4 and er <= 1e-4
        Hg = H.cpu().numpy().astype(np.float64)
        z = S.logits(Hg, OW["embed"], cfg.tau)
        ocv, olk, onl, ost, lam = S.step(Hg, OW["embed"], before, lock_before, float(np.float32(t)),
                                         float(np.float32(h)), cfg.schedule, cfg.tau, cfg.lock_threshold, cfg.seed, s)
        st = read_stats(model, ws, B * L)
        excused_total += compare_step(cv.cpu().numpy(), lk.cpu().numpy(), st, ocv, olk, ost, top2_gap(z),
                                      cfg.lock_threshold)
    loop_canvas = cv.cpu().numpy()
    # the library's own loop reproduces the step-by-step calls bit for bit
    cv2 = torch.empty(B, L, dtype=torch.int32, device=DEV)
    lk2 = torch.empty(B, L, dtype=torch.uint8, device=DEV)
    taken = torch.empty(B, dtype=torch.int32, device=DEV)
    rp = dg.RunParams(schedule=cfg.schedule, max_steps=cfg.steps, tau=cfg.tau, lock_threshold=cfg.lock_threshold,
                      seed=cfg.seed, adaptive=0, init_canvas=1)
    model.canvas_run(cv2, lk2, taken, rp, ws)
    torch.cuda.synchronize()
    assert np.array_equal(cv2.cpu().numpy(), loop_canvas)
    assert taken.tolist() == [cfg.steps] * B
    # the oracle's own loop from its own prefill
    fwd = lambda c: M.denoise_forward(cfg, OW, okv, plen, canvas=c)[0]
    ocv, olk, otaken = S.canvas_run(cfg, OW, okv, plen, fwd)
    log(f"  excused rows over the run: {excused_total}; free-running mismatches: {int((ocv != loop_canvas).sum())}")
    assert excused_total <= max_excused(B * L * cfg.steps)
    if excused_total == 0:
        assert np.array_equal(ocv, loop_canvas)


def test_adaptive_run_locks_and_stops_like_the_oracle():
    cfg = configs.C0.replace(batch=3, steps=8, adaptive=True, lock_threshold=0.95, tau=0.02, kv_source="random")
    B, L = cfg.batch, cfg.canvas
    model, W, kv = build(cfg)
    ws = model.workspace(B, L, cfg.prefix)
    cv = torch.empty(B, L, dtype=torch.int32, device=DEV)
    lk = torch.empty(B, L, dtype=torch.uint8, device=DEV)
    taken = torch.empty(B, dtype=torch.int32, device=DEV)
    rp = dg.RunParams(schedule=cfg.schedule, max_steps=cfg.steps, tau=cfg.tau, lock_threshold=cfg.lock_threshold,
                      seed=3, adaptive=1, init_canvas=1)
    model.canvas_run(cv, lk, taken, rp, ws)
    torch.cuda.synchronize()
    OW = oracle_weights(W, cfg)
    okv = oracle_kv_dev(kv)
    plen = [cfg.prefix] * B
    fwd = lambda c: M.denoise_forward(cfg, OW, okv, plen, canvas=c)[0]
    ocv, olk, otaken = S.canvas_run(cfg, OW, okv, plen, fwd, seed=3)
    log(f"  steps taken gpu {taken.tolist()} oracle {otaken.tolist()}; locked gpu "
        f"{lk.sum(dim=1).tolist()} oracle {olk.sum(axis=1).tolist()}")
    assert lk.sum().item() > 0
    assert taken.tolist() == otaken.tolist()
    assert np.array_equal(lk.cpu().numpy().astype(bool), olk)
    assert np.array_equal(cv.cpu().numpy(), ocv)
