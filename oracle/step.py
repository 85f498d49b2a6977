"""The discrete flow-matching Step with confidence lock-in, and the canvas loop (test
infrastructure only).

Pages: the forward process corrupts each canvas position independently,
    p_t(x_t | x_0) = prod_i [ kappa_t * delta(x_t^i, x_0^i) + (1 - kappa_t) / |V| ],
with kappa decreasing from kappa_0 = 1 to kappa_1 = 0, so at t = 1 the canvas is i.i.d. uniform
[TR §Forward Process].  Generation moves back by h with x_{t-h} ~ Step(x_t, p_theta(. | x_t)),
a discrete Euler update (Gat et al. 2024), factorised per position [TR §Backward Denoising
Process]; p_hat_0 = softmax(logits / tau) and each canvas is refined for at most T steps with
h = 1/T [TR §디노이징 반복과 self-conditioning].  Each pass locks in the high-confidence tokens
and re-evaluates the rest [PBD glossary, "Iterative denoising"].

Readings where the pages are silent:
  * Euler move: an unlocked position jumps with probability lambda = min(1, h*|kappa'(t)|/(1-kappa(t)))
    to a token drawn from p_theta (the draw may repeat the current token), else it stays; the
    rate is taken at the start t of the interval.  lambda is rounded to float32 once per step.
  * Lock-in: an unlocked position whose argmax probability c = max_v p_theta(v) is >= theta is
    set to the argmax and locked; locked positions never change.
  * Ties: argmax and the Gumbel argmax go to the lowest token id.
  * Time grid: t_s = 1 - s*h for s = 0..T-1.
"""
from __future__ import annotations

import math

import numpy as np

from . import philox

LINEAR, QUADRATIC, COSINE = 0, 1, 2


def kappa(schedule, t):
    t = np.asarray(t, dtype=np.float64)
    if schedule == LINEAR:
        return 1.0 - t
    if schedule == QUADRATIC:
        return 1.0 - t * t
    if schedule == COSINE:
        return np.cos(np.pi * t / 2.0)
    raise ValueError(schedule)


def kappa_rate(schedule, t):
    """|d kappa / dt|."""
    t = np.asarray(t, dtype=np.float64)
    if schedule == LINEAR:
        return np.ones_like(t)
    if schedule == QUADRATIC:
        return 2.0 * t
    if schedule == COSINE:
        return (np.pi / 2.0) * np.sin(np.pi * t / 2.0)
    raise ValueError(schedule)


def jump_prob(schedule, t, h):
    """lambda = min(1, h |kappa'(t)| / (1 - kappa(t))), as a float32 value."""
    den = 1.0 - float(kappa(schedule, t))
    lam = 1.0 if den <= 0.0 else min(1.0, h * float(kappa_rate(schedule, t)) / den)
    return float(np.float32(lam))


def time_grid(steps):
    h = 1.0 / steps
    return [1.0 - s * h for s in range(steps)], h


def init_canvas(seed, batch, length, vocab):
    """Canvas at t = 1: every position an independent uniform token."""
    return philox.init_tokens(seed, batch, length, vocab)


def noise(x0, t, schedule, seed, step, vocab):
    """Draw x_t ~ p_t(. | x0): keep x0_i with probability kappa_t, else a uniform token."""
    x0 = np.asarray(x0)
    B, L = x0.shape
    wk, wt = philox.noise_words(seed, step, B, L)
    # the keep decision is taken against kappa rounded to float32, the precision in which the
    # kernel holds it (the 24-bit uniform is exact in both)
    keep = philox.unit_open_closed(wk) < float(np.float32(kappa(schedule, t)))
    return np.where(keep, x0, philox.token(wt, vocab))


def logits(H, E, tau):
    """z = (H E^T) / tau in float64."""
    return (np.asarray(H, np.float64) @ np.asarray(E, np.float64).T) / tau


def sample_stats(z, seed, step, b_of_row, i_of_row, rows_chunk=64):
    """Per row: max m, argmax a (lowest id), confidence c = 1 / sum exp(z - m), Gumbel argmax
    y = argmax(z + G) (lowest id), and the gap between the best and second-best z + G."""
    T, V = z.shape
    m = np.empty(T); a = np.empty(T, np.int64); c = np.empty(T)
    y = np.empty(T, np.int64); gap = np.empty(T); best = np.empty(T)
    v = np.arange(V)
    for r0 in range(0, T, rows_chunk):
        rs = slice(r0, min(T, r0 + rows_chunk))
        zz = z[rs]
        m[rs] = zz.max(axis=1)
        a[rs] = np.argmax(zz, axis=1)                         # first occurrence: lowest id
        c[rs] = 1.0 / np.exp(zz - m[rs, None]).sum(axis=1)
        G = philox.gumbel_noise(seed, step, b_of_row[rs, None], i_of_row[rs, None], v[None, :])
        key = zz + G
        y[rs] = np.argmax(key, axis=1)
        best[rs] = key[np.arange(key.shape[0]), y[rs]]
        top2 = np.partition(key, -2, axis=1)[:, -2:]
        gap[rs] = top2[:, 1] - top2[:, 0]
    return {"m": m, "a": a, "c": c, "y": y, "gap": gap, "best": best}


def apply_step(canvas, lock, stats, lam, theta, seed, step, done=None):
    """The per-position update, given the sampler statistics of every row (b-major)."""
    canvas = np.array(canvas, copy=True)
    lock = np.array(lock, dtype=bool, copy=True)
    B, L = canvas.shape
    b, i = np.meshgrid(np.arange(B), np.arange(L), indexing="ij")
    u = philox.jump_uniform(seed, step, b, i)
    a = stats["a"].reshape(B, L); c = stats["c"].reshape(B, L); y = stats["y"].reshape(B, L)
    active = ~lock
    if done is not None:
        active &= ~np.asarray(done, dtype=bool)[:, None]
    confident = active & (c >= theta)
    jump = active & ~confident & (u < lam)
    canvas = np.where(confident, a, np.where(jump, y, canvas))
    lock = lock | confident
    n_locked = lock.sum(axis=1)
    return canvas, lock, n_locked


def step(H, E, canvas, lock, t, h, schedule, tau, theta, seed, s, done=None):
    """One Step from hidden states H [B*L][d] with the tied embedding E [V][d]."""
    canvas = np.asarray(canvas)
    B, L = canvas.shape
    z = logits(H, E, tau)
    rows = np.arange(B * L)
    st = sample_stats(z, seed, s, rows // L, rows % L)
    lam = jump_prob(schedule, t, h)
    cv, lk, nl = apply_step(canvas, lock, st, lam, theta, seed, s, done)
    return cv, lk, nl, st, lam


def step_from_logits(z32, canvas, lock, t, h, schedule, theta, seed, s, done=None):
    """The same Step from given logits (already divided by tau), float64 arithmetic."""
    canvas = np.asarray(canvas)
    B, L = canvas.shape
    rows = np.arange(B * L)
    st = sample_stats(np.asarray(z32, np.float64), seed, s, rows // L, rows % L)
    lam = jump_prob(schedule, t, h)
    cv, lk, nl = apply_step(canvas, lock, st, lam, theta, seed, s, done)
    return cv, lk, nl, st, lam


def canvas_run(cfg, W, kv, prefix_len, forward, canvas=None, lock=None, steps=None,
               tau=None, theta=None, schedule=None, adaptive=None, seed=None, self_cond=None):
    """The denoising loop for one block of canvases.

    `forward(canvas) -> H` is the decoder pass; with `self_cond` (a function (H, tau) -> s) it is
    called as forward(canvas, s) with s = None at the first step and s = self_cond(H, tau) of the
    previous step afterwards [TR §디노이징 반복과 self-conditioning].  At t = 1 the canvas is drawn uniform
    (unless given).  For s = 0..T-1: canvases that are done are skipped, the rest take one Step at
    t_s; with adaptive stopping a canvas is done once all its positions are locked.
    Returns canvas, lock, steps_taken[B]."""
    B, L = cfg.batch, cfg.canvas
    T = cfg.steps if steps is None else steps
    tau = cfg.tau if tau is None else tau
    theta = cfg.lock_threshold if theta is None else theta
    schedule = cfg.schedule if schedule is None else schedule
    adaptive = cfg.adaptive if adaptive is None else adaptive
    seed = cfg.seed if seed is None else seed
    if canvas is None:
        canvas = init_canvas(seed, B, L, cfg.vocab)
        lock = np.zeros((B, L), dtype=bool)
    canvas = np.asarray(canvas).copy()
    lock = np.zeros((B, L), bool) if lock is None else np.asarray(lock, bool).copy()
    done = np.zeros(B, dtype=bool)
    taken = np.zeros(B, dtype=np.int64)
    ts, h = time_grid(T)
    sc = None
    for s, t in enumerate(ts):
        if adaptive and done.all():
            break
        H = forward(canvas) if self_cond is None else forward(canvas, sc)
        if self_cond is not None:
            sc = self_cond(H, tau)
        canvas, lock, nl, _, _ = step(H, W["embed"], canvas, lock, t, h, schedule, tau, theta, seed, s,
                                      done if adaptive else None)
        taken += ~done if adaptive else 1
        if adaptive:
            done = nl == L
    return canvas, lock, taken
