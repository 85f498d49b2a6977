"""Pins of the oracle's entropy-bounded sampler (the pages' default sampler, [TR §DiffusionGemma
샘플러]) against closed forms, brute force and planted cases (CPU).

  * entropy of softmax: ln V for uniform logits, the two-point closed form, the one-large-logit
    closed form, scipy's entropy on random rows, shift / permutation invariance, monotone in tau
  * selection: the accepted count is the largest k within the budget gamma (brute force over
    every subset of tiny canvases), accepted positions are the lowest-entropy ones, ties to the
    lower position, k = 0 and k = L edge cases
  * adaptive stop: needs both the entropy condition and two equal consecutive argmax sequences;
    a stopped (or final) canvas is the argmax sequence
  * the loop: a planted confident model is accepted in full at the first step and stops at the
    second; an uncertain model accepts nothing and runs every step
"""
import itertools
import math
import types

import numpy as np
import pytest
import scipy.special
import scipy.stats as st

from oracle import eb
from oracle import philox
from oracle import step as S


def test_entropy_uniform_is_log_v():
    for V in (2, 17, 1024):
        z = np.full((3, V), 1.7)
        assert np.allclose(eb.entropy(z), math.log(V), atol=1e-12, rtol=0)


def test_entropy_two_point_closed_form():
    for p in (0.5, 0.1, 1e-3, 0.999):
        z = np.full((1, 8), -1e4)
        z[0, 3], z[0, 5] = math.log(p), math.log(1 - p)
        want = -p * math.log(p) - (1 - p) * math.log(1 - p)
        assert abs(eb.entropy(z)[0] - want) < 1e-12


def test_entropy_one_large_logit_closed_form():
    V, c = 16, 3.0
    z = np.zeros((1, V)); z[0, 7] = c
    Z = math.exp(c) + (V - 1)
    p1, pr = math.exp(c) / Z, 1.0 / Z
    want = -p1 * math.log(p1) - (V - 1) * pr * math.log(pr)
    assert abs(eb.entropy(z)[0] - want) < 1e-12


def test_entropy_matches_scipy_and_invariances():
    rng = np.random.default_rng(3)
    z = rng.standard_normal((40, 300)) * 3
    H = eb.entropy(z)
    ref = st.entropy(scipy.special.softmax(z, axis=1), axis=1)
    assert np.allclose(H, ref, atol=1e-10, rtol=0)
    assert np.allclose(eb.entropy(z + 123.0), H, atol=1e-10, rtol=0)
    perm = rng.permutation(300)
    assert np.allclose(eb.entropy(z[:, perm]), H, atol=1e-10, rtol=0)
    # sharper (lower tau) predictions have lower entropy
    Hs = [eb.entropy(z / tau) for tau in (0.4, 0.6, 0.8, 1.0)]
    for lo, hi in zip(Hs, Hs[1:]):
        assert np.all(lo < hi)


def test_temperature_schedule_linear_08_to_04():
    assert eb.temperature(1.0) == pytest.approx(0.8)
    assert eb.temperature(0.0) == pytest.approx(0.4)
    assert eb.temperature(0.5) == pytest.approx(0.6)
    ts, _ = S.time_grid(48)
    taus = [eb.temperature(t) for t in ts]
    assert taus[0] == pytest.approx(0.8) and np.all(np.diff(taus) < 0)
    assert np.allclose(np.diff(taus), -0.4 / 48)


def test_select_planted_example():
    H = np.array([0.01, 0.5, 0.02, 0.03, 0.2], np.float32)
    acc, k, mean = eb.select(H, 0.1)
    assert k == 3 and set(np.flatnonzero(acc)) == {0, 2, 3}
    assert mean == np.float32(np.cumsum(np.sort(H), dtype=np.float32)[-1]) / np.float32(5)


def test_select_edges_and_ties():
    acc, k, _ = eb.select(np.array([0.2, 0.5, 0.11], np.float32), 0.1)
    assert k == 0 and not acc.any()
    acc, k, _ = eb.select(np.full(64, 1e-4, np.float32), 0.1)
    assert k == 64 and acc.all()
    acc, k, _ = eb.select(np.array([0.05, 0.05, 0.05, 0.05], np.float32), 0.1)
    assert k == 2 and list(np.flatnonzero(acc)) == [0, 1]
    # rounding noise below zero counts as zero entropy
    acc, k, _ = eb.select(np.array([-1e-9, 0.2], np.float32), 0.1)
    assert k == 1 and acc[0]


def test_select_is_the_largest_subset_within_budget_brute_force():
    rng = np.random.default_rng(11)
    gamma = 0.1
    checked = 0
    for _ in range(300):
        L = int(rng.integers(1, 9))
        H = np.exp(rng.uniform(np.log(1e-4), np.log(0.3), L)).astype(np.float32)
        sums = {}
        for r in range(L + 1):
            for sub in itertools.combinations(range(L), r):
                sums[sub] = float(np.sum(H[list(sub)], dtype=np.float64))
        if any(abs(v - gamma) < 1e-5 for v in sums.values()):
            continue                          # too close to the budget for a float32 decision
        best = max(len(sub) for sub, v in sums.items() if v <= gamma)
        acc, k, _ = eb.select(H, gamma)
        assert k == best
        # the accepted set is a largest feasible subset of minimal total entropy
        chosen = tuple(np.flatnonzero(acc))
        assert sums[chosen] <= gamma
        assert sums[chosen] == pytest.approx(min(v for sub, v in sums.items() if len(sub) == best), abs=1e-7)
        checked += 1
    assert checked > 200


def _planted_stats(B=2, L=6, V=64, seed=5):
    rng = np.random.default_rng(seed)
    a = rng.integers(0, V, (B, L)); y = rng.integers(0, V, (B, L))
    return a, y


def test_update_stop_requires_entropy_and_stability():
    V = 64
    a, y = _planted_stats(V=V)
    B, L = a.shape
    low = np.full((B, L), 1e-4, np.float32)           # mean 1e-4 < 0.005; all accepted
    high = np.full((B, L), 0.01, np.float32)          # mean 0.01 >= 0.005; 10 accepted at most
    done0 = np.zeros(B, bool)
    # first step: no previous prediction, no stop; accepted positions take y
    x, done, n_acc, mean, stopped = eb.update(a, y, low, None, done0, 7, 0, V)
    assert not done.any() and not stopped.any() and (n_acc == L).all() and np.array_equal(x, y)
    # stable and confident: stop with the argmax sequence
    x, done, n_acc, mean, stopped = eb.update(a, y, low, a.copy(), done0, 7, 1, V)
    assert done.all() and stopped.all() and np.array_equal(x, a)
    # stable but not confident enough: keep going
    x, done, _, mean, stopped = eb.update(a, y, high, a.copy(), done0, 7, 1, V)
    assert not done.any() and (mean >= np.float32(0.005)).all()
    # confident but not stable
    prev = a.copy(); prev[0, 0] = (prev[0, 0] + 1) % V
    x, done, _, _, stopped = eb.update(a, y, low, prev, done0, 7, 1, V)
    assert list(done) == [False, True]
    # without adaptive stopping only the final step finishes, with the argmax sequence
    x, done, _, _, stopped = eb.update(a, y, low, a.copy(), done0, 7, 1, V, adaptive=False)
    assert not done.any()
    x, done, _, _, stopped = eb.update(a, y, high, None, done0, 7, 2, V, final=True)
    assert done.all() and not stopped.any() and np.array_equal(x, a)
    # a finished canvas keeps its tokens
    keep = np.full((B, L), 9)
    x, done, n_acc, _, _ = eb.update(a, y, high, None, np.array([True, False]), 7, 2, V, canvas=keep)
    assert (x[0] == 9).all() and n_acc[0] == 0


def test_unaccepted_positions_are_renoised_uniformly():
    V, B, L = 64, 4, 4096
    toks = philox.renoise_tokens(13, 3, B, L, V)
    counts = np.bincount(toks.reshape(-1), minlength=V)
    assert st.chisquare(counts).pvalue > 1e-4
    # its own stream: not the forward-noise token stream of the same step
    _, wt = philox.noise_words(13, 3, B, L)
    assert (philox.token(wt, V) != toks).mean() > 0.9
    a = np.zeros((1, 8), np.int64); y = np.ones((1, 8), np.int64)
    H = np.array([[0.0, 0.0, 0.0, 0.0, 5.0, 5.0, 5.0, 5.0]], np.float32)
    x, _, n_acc, _, _ = eb.update(a, y, H, None, np.zeros(1, bool), 13, 3, V)
    ren = philox.renoise_tokens(13, 3, 1, 8, V)
    assert n_acc[0] == 4 and (x[0, :4] == 1).all() and np.array_equal(x[0, 4:], ren[0, 4:])


def _cfg(B=2, L=16, V=256):
    return types.SimpleNamespace(batch=B, canvas=L, vocab=V, seed=21)


def test_run_planted_confident_model_stops_at_second_step():
    cfg = _cfg()
    rng = np.random.default_rng(0)
    E = rng.standard_normal((cfg.vocab, 32)) * 0.02
    target = rng.integers(0, cfg.vocab, (cfg.batch, cfg.canvas))

    def forward(x):
        e = E[target.reshape(-1)]
        return 50.0 * e / (e * e).sum(axis=1, keepdims=True)     # z_target = 50 / tau

    x, taken = eb.run(cfg, {"embed": E}, forward, steps=48)
    assert np.array_equal(x, target) and list(taken) == [2, 2]


def test_run_uncertain_model_accepts_nothing_and_runs_every_step():
    cfg = _cfg(B=1, L=8, V=64)
    rng = np.random.default_rng(1)
    E = rng.standard_normal((cfg.vocab, 16)) * 0.02
    trace = []

    def forward(x):
        return rng.standard_normal((x.size, 16))

    x, taken = eb.run(cfg, {"embed": E}, forward, steps=5, trace=trace)
    assert list(taken) == [5]
    assert all((t["n_acc"] == 0).all() for t in trace)
    last = trace[-1]["stats"]["a"].reshape(1, 8)
    assert np.array_equal(x, last)
    for t in trace[:-1]:
        ren = philox.renoise_tokens(cfg.seed, t["s"], 1, 8, cfg.vocab)
        assert np.array_equal(t["canvas"], ren)
