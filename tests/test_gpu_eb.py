"""Parity of the entropy-bounded step (the pages' default sampler, [TR §DiffusionGemma 샘플러]) on
the GPU against the oracle:
  * the selection from given float32 entropies, argmax and draws: bit-exact (canvas, accepted
    counts, mean entropy, done flags, the stored argmax), including ties, stops, final steps and
    finished canvases;
  * the step from given logits: entropies within float32 error, argmax / draws exact except at
    near-ties, decisions exact unless the oracle's own margins say float order may decide;
  * the tiny fp32 model's loop with the entropy-bounded sampler, teacher-forced step by step,
    then as one dg_canvas_run call (bit-identical to the step-by-step calls) and against the
    oracle's free-running loop."""
import numpy as np
import pytest
import torch

from discrete_text_diffusion_amd import dg
from oracle import eb
from oracle import model as M
from oracle import step as S
from synth import configs, gen
from tests.gpu_util import build, log, read_stats, top2_gap
from tests.helpers import oracle_kv_dev, oracle_weights

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _params(t, step, has_prev, final=False, adaptive=True, tau_start=0.8, tau_end=0.4, gamma=0.1, stop=0.005,
            seed=9):
    return dg.EbParams(t=t, tau_start=tau_start, tau_end=tau_end, gamma=gamma, stop_entropy=stop, seed=seed,
                       step=step, has_prev=int(has_prev), final_step=int(final), adaptive=int(adaptive))


def _tau(p):
    """tau_t as the library forms it: in double from the float32 parameters, rounded to float32."""
    return float(np.float32(float(p.tau_end) + (float(p.tau_start) - float(p.tau_end)) * float(p.t)))


def _t(x, dtype=torch.int32):
    return torch.from_numpy(np.ascontiguousarray(x)).to(dtype).to(DEV)


@pytest.mark.parametrize("B,L", [(3, 256), (2, 1024), (4, 48)])
@pytest.mark.parametrize("mode", ["adaptive", "final", "first", "fixed-steps"])
def test_eb_select_bit_exact(B, L, mode):
    V = 1024
    rng = np.random.default_rng(B * 1000 + L)
    H = np.exp(rng.uniform(np.log(1e-7), np.log(0.05), (B, L))).astype(np.float32)
    H[:, ::9] = rng.uniform(0.5, 7.0, H[:, ::9].shape).astype(np.float32)
    H[:, 3::17] = H[:, 3:4]                              # exact ties
    H[0] = np.float32(1e-6)                              # canvas 0: confident everywhere (mean < 0.005)
    H[0, 7] = np.float32(0.0)
    a = rng.integers(0, V, (B, L)); y = rng.integers(0, V, (B, L))
    prev = a.copy()
    prev[1, 5] = (prev[1, 5] + 1) % V                    # canvas 1: prediction changed
    done = np.zeros(B, np.int32)
    if B > 2:
        done[-1] = 1                                     # a finished canvas is left alone
    cv_in = rng.integers(0, V, (B, L))
    has_prev = mode != "first"
    p = _params(0.5, 3, has_prev, final=(mode == "final"), adaptive=(mode != "fixed-steps"))
    model, _, _ = build(configs.C0.replace(vocab=V, batch=B, canvas=L))
    ws = model.workspace(B, L, 0)
    cv, pv, dn = _t(cv_in), _t(prev), _t(done)
    nacc = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    mean = torch.full((B,), -1.0, dtype=torch.float32, device=DEV)
    dg.dg_test_eb_select(model.ctx, _t(H, torch.float32), _t(a), _t(y), cv, pv, dn, nacc, mean, B, L, p, ws)
    torch.cuda.synchronize()
    ocv, odone, onacc, omean, ostop = eb.update(a, y, H, prev if has_prev else None, done.astype(bool), p.seed,
                                                p.step, V, p.gamma, p.stop_entropy, final=(mode == "final"),
                                                canvas=cv_in, adaptive=(mode != "fixed-steps"))
    log(f"  B={B} L={L} {mode}: accepted {onacc.tolist()} mean {omean.tolist()} stopped {ostop.tolist()}")
    live = done == 0
    assert np.array_equal(cv.cpu().numpy(), ocv)
    assert np.array_equal(dn.cpu().numpy().astype(bool), odone)
    assert np.array_equal(nacc.cpu().numpy()[live], onacc[live])
    assert np.array_equal(mean.cpu().numpy()[live].view(np.uint32), omean[live].view(np.uint32))
    assert np.array_equal(pv.cpu().numpy()[live], a[live])
    assert np.array_equal(pv.cpu().numpy()[~live], prev[~live])
    if mode == "adaptive":
        assert ostop[0] and not ostop[1]                 # the planted stop and the planted change


def _fragile(H64, a_gap, y_gap, L, gamma, stop, tol):
    """Canvases whose decisions the oracle itself cannot take robustly in float32: an entropy
    within `tol` of another across the acceptance cut, a running sum within `tol` of gamma near
    the cut, the mean within `tol` of the stop threshold, or a near-tie in an argmax / draw."""
    B = H64.shape[0] // L
    out = np.zeros(B, bool)
    for b in range(B):
        h = np.sort(H64[b * L:(b + 1) * L])
        run = np.cumsum(h)
        k = int(np.count_nonzero(run <= gamma))
        near_cut = np.abs(run - gamma) < tol * (1 + np.arange(L))
        lo, hi = max(0, k - 1), min(L, k + 1)
        swap = k > 0 and k < L and (h[k] - h[k - 1]) < tol
        out[b] = near_cut[lo:hi].any() or swap or abs(run[-1] / L - stop) < tol
        out[b] |= (a_gap[b * L:(b + 1) * L] < 1e-5).any() or (y_gap[b * L:(b + 1) * L] < 1e-3).any()
    return out


@pytest.mark.parametrize("t,has_prev", [(1.0, False), (0.5, True), (0.125, True)])
def test_eb_from_logits_parity(t, has_prev):
    B, L, V = 3, 64, 4096
    g = torch.Generator(device="cpu").manual_seed(int(t * 1000))
    z = torch.randn(B * L, V, generator=g)
    spike = 6.0 + 16.0 * torch.rand(B * L, generator=g)    # entropies from ~1 nat down to ~1e-6
    z[torch.arange(B * L), (torch.arange(B * L) * 37) % V] += spike
    z[2 * L:] *= 0.05                                        # canvas 2: near-uniform, nothing accepted
    model, _, _ = build(configs.C0.replace(vocab=V, batch=B, canvas=L))
    ws = model.workspace(B, L, 0)
    p = _params(t, 5, has_prev)
    tau = _tau(p)
    zz = z.double().numpy() / tau
    st = eb.stats_from_logits(zz, p.seed, p.step, B, L)
    a_o, y_o = st["a"].reshape(B, L), st["y"].reshape(B, L)
    prev = a_o.copy()
    prev[1, 0] = (prev[1, 0] + 1) % V
    cv, pv = torch.zeros(B, L, dtype=torch.int32, device=DEV), _t(prev)
    dn = torch.zeros(B, dtype=torch.int32, device=DEV)
    nacc = torch.empty(B, dtype=torch.int32, device=DEV)
    mean = torch.empty(B, dtype=torch.float32, device=DEV)
    dg.dg_test_eb_from_logits(model.ctx, z.to(DEV), cv, pv, dn, nacc, mean, B, L, p, ws)
    torch.cuda.synchronize()
    gs = read_stats(model, ws, B * L)
    eH = np.abs(gs["H"] - st["H"])
    tolH = 2e-5 + 1e-5 * st["H"]
    log(f"  t={t}: entropy max err {eH.max():.2e}; oracle entropies {st['H'].min():.2e} .. {st['H'].max():.2f}")
    assert np.all(eH <= tolH)
    agap = top2_gap(zz)
    bad_a = (gs["a"] != st["a"]) & (agap >= 1e-5)
    bad_y = (gs["y"] != st["y"]) & (st["gap"] >= 1e-3)
    assert not bad_a.any() and not bad_y.any()
    ocv, odone, onacc, omean, _ = eb.update(a_o, y_o, st["H"].astype(np.float32).reshape(B, L),
                                            prev if has_prev else None, np.zeros(B, bool), p.seed, p.step, V,
                                            p.gamma, p.stop_entropy)
    frag = _fragile(st["H"], agap, st["gap"], L, p.gamma, p.stop_entropy, 1e-4)
    log(f"  accepted gpu {nacc.tolist()} oracle {onacc.tolist()}; fragile canvases {frag.tolist()}")
    assert frag.sum() <= 1
    for b in np.flatnonzero(~frag):
        assert nacc[b].item() == onacc[b]
        assert np.array_equal(cv[b].cpu().numpy(), ocv[b])
        assert bool(dn[b].item()) == odone[b]
    assert onacc[2] == 0 and onacc[0] > 0


def test_tiny_model_eb_loop_teacher_forced_and_canvas_run():
    cfg = configs.C0.replace(batch=2, kv_source="random")
    B, L, V = cfg.batch, cfg.canvas, cfg.vocab
    T, tau_start, tau_end = 8, 0.03, 0.01                   # sharp predictions: positions get accepted
    model, W, kv = build(cfg)
    ws = model.workspace(B, L, cfg.prefix)
    OW = oracle_weights(W, cfg)
    okv = oracle_kv_dev(kv)
    plen = [cfg.prefix] * B
    cv = torch.empty(B, L, dtype=torch.int32, device=DEV)
    dg.dg_init_canvas(cv, None, B, L, V, 4)
    pv = torch.zeros(B, L, dtype=torch.int32, device=DEV)
    dn = torch.zeros(B, dtype=torch.int32, device=DEV)
    nacc = torch.empty(B, dtype=torch.int32, device=DEV)
    mean = torch.empty(B, dtype=torch.float32, device=DEV)
    Hd = torch.empty(B * L, cfg.d_model, dtype=torch.float32, device=DEV)
    ts, h = S.time_grid(T)
    steps_gpu = np.zeros(B, np.int64)
    excused = 0
    o_prev = None
    for s, t in enumerate(ts):
        before = cv.cpu().numpy().copy()
        done_before = dn.cpu().numpy().astype(bool)
        if done_before.all():
            break
        p = _params(float(np.float32(t)), s, s > 0, final=(s == T - 1), tau_start=tau_start, tau_end=tau_end, seed=4)
        model.denoise_step(cv, L, ws, hidden_out=Hd)
        dg.dg_step_entropy_bounded(model.ctx, Hd, cv, pv, dn, nacc, mean, B, L, p, ws)
        torch.cuda.synchronize()
        steps_gpu += ~done_before
        oH = M.denoise_forward(cfg, OW, okv, plen, canvas=before)[0]
        assert np.abs(Hd.cpu().numpy() - oH).max() <= 1e-4
        zz = S.logits(Hd.cpu().numpy().astype(np.float64), OW["embed"], _tau(p))
        st = eb.stats_from_logits(zz, 4, s, B, L)
        a_o = st["a"].reshape(B, L)
        ocv, odone, onacc, omean, ostop = eb.update(a_o, st["y"].reshape(B, L),
                                                    st["H"].astype(np.float32).reshape(B, L), o_prev, done_before,
                                                    4, s, V, final=(s == T - 1), canvas=before)
        frag = _fragile(st["H"], top2_gap(zz), st["gap"], L, 0.1, 0.005, 1e-4) & ~done_before
        excused += int(frag.sum())
        log(f"  step {s}: accepted gpu {nacc.tolist()} oracle {onacc.tolist()}, mean {mean.tolist()}, "
            f"done {dn.tolist()}, fragile {frag.tolist()}")
        for b in np.flatnonzero(~frag):
            assert np.array_equal(cv[b].cpu().numpy(), ocv[b])
            assert bool(dn[b].item()) == odone[b]
        o_prev = a_o
    loop_canvas = cv.cpu().numpy()
    assert dn.cpu().numpy().all()
    # the library's loop reproduces the step-by-step calls bit for bit
    cv2 = torch.empty(B, L, dtype=torch.int32, device=DEV)
    taken = torch.empty(B, dtype=torch.int32, device=DEV)
    rp = dg.RunParams(schedule=0, max_steps=T, tau=tau_start, lock_threshold=1.0, seed=4, adaptive=1,
                      init_canvas=1, sampler=dg.DG_SAMPLER_ENTROPY_BOUNDED, gamma=0.1, stop_entropy=0.005,
                      tau_end=tau_end)
    model.canvas_run(cv2, None, taken, rp, ws)
    torch.cuda.synchronize()
    log(f"  dg_canvas_run steps {taken.tolist()} (step by step {steps_gpu.tolist()}); excused {excused}")
    assert np.array_equal(cv2.cpu().numpy(), loop_canvas)
    assert taken.tolist() == steps_gpu.tolist()
    # the oracle's free-running loop
    fwd = lambda c: M.denoise_forward(cfg, OW, okv, plen, canvas=c)[0]
    ocv, otaken = eb.run(cfg, OW, fwd, steps=T, tau_start=tau_start, tau_end=tau_end, seed=4)
    if excused == 0:
        assert np.array_equal(ocv, loop_canvas) and otaken.tolist() == steps_gpu.tolist()
