"""Self-conditioning on the GPU against the oracle [TR §디노이징 반복과 self-conditioning].

  * one Step's signal s = FFW(p_hat_0 . E) from given hidden states: fp32 on the tiny model (all
    rows), bf16 at the 262,144-token vocabulary with the Gemma-like widths and an 896-wide block, at
    temperature 1 (a flat p_hat_0) and 0.05 (a peaked one), for one canvas (all 256 rows) and for
    eight (2048 rows, 64 sampled: a row's signal depends on that row alone); the Step's own outputs
    are unchanged by asking for the signal
  * the canvas loop with self-conditioning, Euler and entropy-bounded samplers, tiny fp32 model
    with the block's weights scaled up so the signal moves tokens: canvas, locks and steps equal to
    the oracle's free-running loop
  * block-AR generation with self-conditioning, lockstep and continuous: equal to each other and to
    the oracle's generation

bf16 bounds: p_hat_0 is rounded to bf16 before its product with E (fp32 accumulation) and the
block's input and hidden product are stored in bf16, so the signal carries a few bf16 roundings:
relative RMS error <= 1e-2 and no element off by more than 5e-2 of the largest |s|.  fp32: 1e-5.
"""
import numpy as np
import pytest
import torch

from discrete_text_diffusion_amd import dg
from oracle import blockar as BA
from oracle import eb as EB
from oracle import model as M
from oracle import selfcond as SC
from oracle import step as S
from oracle.numerics import rounder
from synth import configs, gen
from tests.gpu_util import build, log
from tests.helpers import np64, oracle_kv, oracle_kv_dev, oracle_weights

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _sc_weights(W):
    return np64(W["sc_gate"]), np64(W["sc_up"]), np64(W["sc_down"])


@pytest.mark.parametrize("case", ["tiny-fp32", "vocab262k-bf16", "vocab262k-bf16-peaked", "vocab262k-bf16-b8"])
def test_step_signal_matches_oracle(case):
    rows_checked = None
    if case == "tiny-fp32":
        cfg = configs.C0.replace(sc_hidden=64)
    elif case == "vocab262k-bf16":
        cfg = configs.C2.replace(n_layers=1, sc_hidden=896)
    elif case == "vocab262k-bf16-peaked":
        cfg = configs.C2.replace(n_layers=1, sc_hidden=896, tau=0.05)
    else:
        cfg = configs.C2.replace(n_layers=1, sc_hidden=896, batch=8)
        rows_checked = np.arange(3, 2048, 32)
    B, L = cfg.batch, cfg.canvas
    log(f"[self-cond step] {case}: rows {B * L}, V {cfg.vocab}, d {cfg.d_model}, block {cfg.sc_hidden}, tau {cfg.tau}")
    model, W, _ = build(cfg)
    ws = model.workspace(B, L, cfg.prefix)
    H = gen.hidden_input(cfg, DEV)
    cv0 = torch.empty(B, L, dtype=torch.int32, device=DEV)
    dg.dg_init_canvas(cv0, None, B, L, cfg.vocab, 1)
    p = dg.StepParams(schedule=cfg.schedule, t=0.75, h=0.25, tau=cfg.tau, lock_threshold=cfg.lock_threshold,
                      seed=2, step=1)
    outs = []
    for want_sc in (False, True):
        cv, lk = cv0.clone(), torch.zeros(B, L, dtype=torch.uint8, device=DEV)
        nl = torch.empty(B, dtype=torch.int32, device=DEV)
        sc = torch.full((B * L, cfg.d_model), float("nan"), dtype=torch.float32, device=DEV) if want_sc else None
        model.step_sample(H, cv, lk, nl, p, ws, sc_out=sc)
        torch.cuda.synchronize()
        outs.append((cv.cpu().numpy(), lk.cpu().numpy(), nl.cpu().numpy(), sc))
    for a, b in zip(outs[0][:3], outs[1][:3]):
        assert np.array_equal(a, b), "asking for the signal changed the Step"
    s = outs[1][3].cpu().numpy()
    assert np.isfinite(s).all()
    rows = np.arange(B * L) if rows_checked is None else rows_checked
    H64 = np64(H)[rows]
    so = SC.self_condition(H64, np64(W["embed"]), float(np.float32(cfg.tau)), _sc_weights(W), rounder(cfg.act_dtype))
    d = s[rows] - so
    rel = float(np.sqrt(np.mean(d * d) / np.mean(so * so)))
    mx = float(np.abs(d).max() / np.abs(so).max())
    log(f"  signal: |s| max {np.abs(so).max():.3e}; relative RMS error {rel:.2e}, max error / max |s| {mx:.2e}")
    if cfg.act_dtype == "f32":
        assert rel <= 1e-5 and mx <= 1e-5
    else:
        assert rel <= 1e-2 and mx <= 5e-2


def _tiny_sc_cfg(**kw):
    kw.setdefault("kv_source", "random")
    return configs.C0.replace(sc_hidden=64, **kw)


def _strong_block(W):
    """At N(0, 0.02) the block's output is ~1e-8 and moves no token; weights 25x larger (std 0.5)
    give a signal at the embedding's own scale, so the loops below depend on it."""
    for k in ("sc_gate", "sc_up", "sc_down"):
        W[k].mul_(25.0)


@pytest.mark.parametrize("sampler", ["euler", "eb"])
def test_canvas_loop_with_self_conditioning_matches_oracle(sampler):
    cfg = _tiny_sc_cfg(batch=3, steps=8, adaptive=True, lock_threshold=0.9, tau=0.02)
    B, L = cfg.batch, cfg.canvas
    model, W, kv = build(cfg)
    _strong_block(W)
    ws = model.workspace(B, L, cfg.prefix)
    eb_kw = dict(tau_start=0.05, tau_end=0.02)
    rp = dg.RunParams(schedule=cfg.schedule, max_steps=cfg.steps, tau=cfg.tau, lock_threshold=cfg.lock_threshold,
                      seed=3, adaptive=1, init_canvas=1, self_condition=1,
                      sampler=dg.DG_SAMPLER_ENTROPY_BOUNDED if sampler == "eb" else dg.DG_SAMPLER_EULER,
                      gamma=0.1, stop_entropy=0.005, tau_end=eb_kw["tau_end"])
    if sampler == "eb":
        rp.tau = eb_kw["tau_start"]
    cv = torch.empty(B, L, dtype=torch.int32, device=DEV)
    lk = torch.zeros(B, L, dtype=torch.uint8, device=DEV)
    taken = torch.empty(B, dtype=torch.int32, device=DEV)
    model.canvas_run(cv, lk, taken, rp, ws)
    torch.cuda.synchronize()
    OW = oracle_weights(W, cfg)
    okv = oracle_kv_dev(kv)
    plen = [cfg.prefix] * B
    Wsc = _sc_weights(W)
    sc_fn = lambda H, tau: SC.self_condition(H, OW["embed"], float(np.float32(tau)), Wsc, rounder(cfg.act_dtype))
    fwd = lambda c, sc=None: M.denoise_forward(cfg, OW, okv, plen, canvas=c, sc=sc)[0]
    if sampler == "euler":
        ocv, olk, otaken = S.canvas_run(cfg, OW, okv, plen, fwd, seed=3, self_cond=sc_fn)
    else:
        ocv, otaken = EB.run(cfg, OW, fwd, steps=cfg.steps, seed=3, self_cond=sc_fn, **eb_kw)
    # the same loop without self-conditioning, for contrast
    rp.self_condition = 0
    cv0 = torch.empty_like(cv)
    lk0 = torch.zeros_like(lk)
    model.canvas_run(cv0, lk0, taken.clone(), rp, ws)
    torch.cuda.synchronize()
    g = cv.cpu().numpy()
    log(f"  {sampler}: steps gpu {taken.tolist()} oracle {otaken.tolist()}; tokens that self-conditioning changed "
        f"{int((g != cv0.cpu().numpy()).sum())}; mismatches with the oracle {int((g != ocv).sum())}")
    assert int((g != cv0.cpu().numpy()).sum()) > 0, "the signal should change the run"
    assert taken.tolist() == otaken.tolist()
    assert np.array_equal(g, ocv)
    if sampler == "euler":
        assert np.array_equal(lk.cpu().numpy().astype(bool), olk)


def test_generation_with_self_conditioning_lockstep_and_continuous():
    K, P0 = 3, 48
    cfg = _tiny_sc_cfg(batch=3, prefix=P0 + (K - 1) * 32, steps=8, tau=0.03, lock_threshold=0.9, kv_source="prefill")
    B, L, V = cfg.batch, cfg.canvas, cfg.vocab
    prompt = torch.from_numpy(np.random.default_rng(5).integers(0, V, (B, P0)).astype(np.int32)).to(DEV)
    rp = dg.RunParams(schedule=cfg.schedule, max_steps=cfg.steps, tau=cfg.tau, lock_threshold=cfg.lock_threshold,
                      seed=11, adaptive=1, init_canvas=1, sampler=dg.DG_SAMPLER_EULER, self_condition=1)
    res = {}
    for mode in ("continuous", "lockstep"):
        model, W, kv = build(cfg, kv_mode="empty")
        _strong_block(W)
        model.set_kv(kv, [0] * B)
        ws = model.workspace(B, max(L, P0), cfg.prefix)
        model.prefill_kv(prompt, ws)
        out = torch.empty(K, B, L, dtype=torch.int32, device=DEV)
        steps = torch.empty(K, B, dtype=torch.int32, device=DEV)
        passes = torch.zeros(1, dtype=torch.int32, device=DEV)
        if mode == "continuous":
            model.generate_continuous(out, steps, None, None, passes, 17, rp, ws)
        else:
            model.generate(out, steps, None, None, 17, rp, ws)
        torch.cuda.synchronize()
        res[mode] = (out.cpu().numpy(), steps.cpu().numpy(), int(passes.item()))
    OW = oracle_weights(W, cfg)
    okv, plen = M.prefill(cfg, OW, oracle_kv(gen.empty_kv(cfg)), [0] * B, prompt.cpu().numpy())
    Wsc = _sc_weights(W)
    sc_fn = lambda H, tau: SC.self_condition(H, OW["embed"], float(np.float32(tau)), Wsc, rounder(cfg.act_dtype))
    oout, osteps, _, _ = BA.generate(cfg.replace(adaptive=True), OW, okv, plen, K, 17, seed=11, self_cond=sc_fn)
    g, gs, npass = res["continuous"]
    log(f"  steps gpu {gs.T.tolist()} oracle {osteps.T.tolist()}; passes {npass} "
        f"(oracle {BA.continuous_passes(osteps)[0]})")
    assert np.array_equal(g, oout) and np.array_equal(gs, osteps)
    assert np.array_equal(res["lockstep"][0], g) and np.array_equal(res["lockstep"][1], gs)
    assert npass == BA.continuous_passes(osteps)[0]
