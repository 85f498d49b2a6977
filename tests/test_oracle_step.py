"""Pins of the oracle's Step, noising and canvas loop against closed forms and invariants (CPU).

  * forward marginal kappa_t delta(x0) + (1 - kappa_t)/V  [TR §Forward Process]
  * Euler move with the planted perfect denoiser: the fraction of positions equal to x0 after a
    step from t is kappa(t-h) + (1-kappa(t-h))/V (exact for linear kappa); the last step of the
    linear grid has lambda = 1 and lands exactly on x0
  * Gumbel-max sampling frequencies equal softmax(z); tau -> 0 reduces to the argmax
  * lock-in: a fully locked canvas is a fixed point, locks are monotone, confident positions
    lock at the argmax [PBD glossary]
"""
import math

import numpy as np
import pytest
import scipy.special
import scipy.stats as st

from oracle import philox
from oracle import step as S


V = 1024


def _embed(V=V, d=64, seed=0):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((V, d)) * 0.02


def _planted_H(E, x0):
    """H_i = 50 E[x0_i] / |E[x0_i]|^2 gives z_{x0} = 50, far above every other logit."""
    e = E[x0.reshape(-1)]
    return 50.0 * e / (e * e).sum(axis=1, keepdims=True)


def test_jump_prob_closed_forms():
    for t, h in ((1.0, 0.25), (0.5, 0.25), (0.25, 0.25)):
        assert S.jump_prob(S.LINEAR, t, h) == np.float32(min(1.0, h / t))
    for t, h in ((1.0, 1 / 12), (0.5, 1 / 12), (2 / 12, 1 / 12), (1 / 12, 1 / 12)):
        assert S.jump_prob(S.QUADRATIC, t, h) == np.float32(min(1.0, 2 * h / t))
    t, h = 0.7, 1 / 48
    want = h * (math.pi / 2) * math.sin(math.pi * t / 2) / (1 - math.cos(math.pi * t / 2))
    assert S.jump_prob(S.COSINE, t, h) == np.float32(want)
    # kappa runs from 1 at t = 0 to 0 at t = 1 and decreases
    for sch in (S.LINEAR, S.QUADRATIC, S.COSINE):
        ts = np.linspace(0, 1, 101)
        k = S.kappa(sch, ts)
        assert abs(k[0] - 1) < 1e-15 and abs(k[-1]) < 1e-15 and np.all(np.diff(k) < 0)
        # |kappa'| is the derivative's magnitude
        num = -(S.kappa(sch, ts[1:-1] + 1e-6) - S.kappa(sch, ts[1:-1] - 1e-6)) / 2e-6
        assert np.allclose(num, S.kappa_rate(sch, ts[1:-1]), atol=1e-6)


@pytest.mark.parametrize("t", [0.25, 0.5, 0.9, 1.0])
def test_forward_marginal_closed_form(t):
    B, L = 1024, 1024                       # 2^20 draws
    rng = np.random.default_rng(1)
    x0 = rng.integers(0, V, size=(B, L))
    xt = S.noise(x0, t, S.LINEAR, seed=42, step=int(t * 100), vocab=V)
    kap = 1 - t
    p_same = kap + (1 - kap) / V
    n = B * L
    frac = np.mean(xt == x0)
    assert abs(frac - p_same) < 5 * math.sqrt(p_same * (1 - p_same) / n)
    # the changed positions are uniform over the vocab: offset (x_t - x0) mod V is uniform
    off = (xt - x0) % V
    counts = np.bincount(off[xt != x0], minlength=V)[1:]
    chi2 = ((counts - counts.mean()) ** 2 / counts.mean()).sum()
    assert st.chi2.sf(chi2, V - 2) > 1e-4


def test_forward_marginal_endpoints():
    x0 = np.random.default_rng(2).integers(0, V, size=(4, 256))
    assert np.array_equal(S.noise(x0, 0.0, S.QUADRATIC, 0, 0, V), x0)
    init = S.init_canvas(0, 256, 1024, V)
    counts = np.bincount(init.reshape(-1), minlength=V)
    chi2 = ((counts - counts.mean()) ** 2 / counts.mean()).sum()
    assert st.chi2.sf(chi2, V - 1) > 1e-4


def test_gumbel_max_frequencies_are_softmax():
    Vs = 16
    z = np.linspace(-2, 1.5, Vs)
    rows = 200000
    G = philox.gumbel_noise(7, 3, 0, np.arange(rows)[:, None], np.arange(Vs)[None, :])
    y = np.argmax(z[None, :] + G, axis=1)
    counts = np.bincount(y, minlength=Vs)
    p = scipy.special.softmax(z)
    chi2 = ((counts - rows * p) ** 2 / (rows * p)).sum()
    assert st.chi2.sf(chi2, Vs - 1) > 1e-4


def test_tau_to_zero_is_argmax_and_confidence_is_softmax_max():
    E = _embed()
    rng = np.random.default_rng(3)
    H = rng.standard_normal((64, 64))
    z = S.logits(H, E, 1e-4)
    st_ = S.sample_stats(z, 0, 0, np.zeros(64, int), np.arange(64))
    assert np.array_equal(st_["y"], np.argmax(H @ E.T, axis=1))
    z1 = S.logits(H, E, 1.0)
    st1 = S.sample_stats(z1, 0, 0, np.zeros(64, int), np.arange(64))
    assert np.allclose(st1["c"], scipy.special.softmax(H @ E.T, axis=1).max(axis=1), rtol=1e-12)


@pytest.mark.parametrize("t_idx", [0, 1, 2])
def test_planted_denoiser_euler_fraction(t_idx):
    """Lock-in off (theta > 1); linear kappa; 2^16 positions."""
    T = 4
    ts, h = S.time_grid(T)
    t = ts[t_idx]
    E = _embed()
    B, L = 64, 1024
    rng = np.random.default_rng(4 + t_idx)
    x0 = rng.integers(0, V, size=(B, L))
    xt = S.noise(x0, t, S.LINEAR, seed=5, step=17, vocab=V)
    lock = np.zeros((B, L), bool)
    new, _, _, _, lam = S.step(_planted_H(E, x0), E, xt, lock, t, h, S.LINEAR, 1.0, 2.0, 9, t_idx)
    k_next = 1 - (t - h)
    want = k_next + (1 - k_next) / V
    n = B * L
    frac = np.mean(new == x0)
    assert abs(frac - want) < 4 * math.sqrt(want * (1 - want) / n)


def test_planted_denoiser_last_linear_step_is_exact():
    ts, h = S.time_grid(4)
    E = _embed()
    x0 = np.random.default_rng(6).integers(0, V, size=(8, 256))
    xt = S.noise(x0, ts[-1], S.LINEAR, seed=1, step=0, vocab=V)
    assert S.jump_prob(S.LINEAR, ts[-1], h) == 1.0
    new, _, _, _, _ = S.step(_planted_H(E, x0), E, xt, np.zeros_like(x0, bool), ts[-1], h,
                             S.LINEAR, 1.0, 2.0, 3, 3)
    assert np.array_equal(new, x0)


def test_change_probability_at_random_init():
    """P(position changes) = lambda * (1 - p(x_old)) when nothing locks."""
    E = _embed(d=64)
    rng = np.random.default_rng(8)
    B, L = 16, 1024
    H = rng.standard_normal((B * L, 64)) * 3.0
    x = S.init_canvas(0, B, L, V)
    t, h = 0.5, 0.25
    new, _, _, st_, lam = S.step(H, E, x, np.zeros((B, L), bool), t, h, S.LINEAR, 1.0, 2.0, 11, 2)
    p = scipy.special.softmax(H @ E.T, axis=1)
    p_old = p[np.arange(B * L), x.reshape(-1)]
    want = (lam * (1 - p_old)).sum()
    var = (lam * (1 - p_old) * (1 - lam * (1 - p_old))).sum()
    got = np.sum(new != x)
    assert abs(got - want) < 4 * math.sqrt(var)


def test_locked_canvas_is_fixed_point():
    E = _embed()
    rng = np.random.default_rng(9)
    B, L = 4, 64
    H = rng.standard_normal((B * L, 64))
    x = rng.integers(0, V, size=(B, L))
    lock = np.ones((B, L), bool)
    for s in range(4):
        new, lk, nl, _, _ = S.step(H, E, x, lock, 1 - s / 4, 0.25, S.LINEAR, 1.0, 0.0, 1, s)
        assert np.array_equal(new, x) and lk.all() and np.all(nl == L)


def test_confident_positions_lock_at_argmax_and_locks_are_monotone():
    E = _embed()
    rng = np.random.default_rng(10)
    B, L = 2, 128
    x0 = rng.integers(0, V, size=(B, L))
    H = rng.standard_normal((B * L, 64)) * 0.1
    planted = rng.random(B * L) < 0.3
    H[planted] = _planted_H(E, x0)[planted]
    x = S.init_canvas(1, B, L, V)
    lock = np.zeros((B, L), bool)
    new, lk, nl, st_, _ = S.step(H, E, x, lock, 1.0, 0.25, S.LINEAR, 1.0, 0.9, 2, 0)
    assert np.array_equal(lk.reshape(-1), planted)
    assert np.array_equal(new.reshape(-1)[planted], x0.reshape(-1)[planted])
    assert np.array_equal(nl, planted.reshape(B, L).sum(axis=1))
    # later steps keep every lock and every locked token
    prev_lock, prev = lk, new
    for s in range(1, 4):
        H2 = rng.standard_normal((B * L, 64))
        cur, lk2, _, _, _ = S.step(H2, E, prev, prev_lock, 1 - s / 4, 0.25, S.LINEAR, 1.0, 0.9, 2, s)
        assert np.all(lk2 >= prev_lock)
        assert np.array_equal(cur[prev_lock], prev[prev_lock])
        prev_lock, prev = lk2, cur


def test_adaptive_run_stops_when_all_locked():
    """Planted denoiser with a tiny tau: every position locks at the first step."""
    from synth.configs import C0
    cfg = C0.replace(batch=3, canvas=32, steps=8, adaptive=True, lock_threshold=0.95)
    E = _embed(d=64)
    x0 = np.random.default_rng(12).integers(0, V, size=(3, 32))
    W = {"embed": E}
    calls = []

    def fwd(canvas):
        calls.append(canvas.copy())
        H = _planted_H(E, x0)
        H[32:64] *= 0.0               # canvas 1 never becomes confident (uniform p)
        return H

    cv, lk, taken = S.canvas_run(cfg, W, None, None, fwd)
    assert taken[0] == 1 and taken[2] == 1 and taken[1] == 8
    assert np.array_equal(cv[0], x0[0]) and np.array_equal(cv[2], x0[2])
    assert lk[0].all() and lk[2].all() and not lk[1].any()
