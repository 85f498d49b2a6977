"""The pages' default sampler: entropy-bounded refinement with temperature annealing and adaptive
stopping (test infrastructure only).

Pages [TR §DiffusionGemma 샘플러]: the recommended sampler computes the predictive entropy of every
canvas position and accepts positions in ascending order of entropy (MaskGIT-like), as many as
keep the running sum of the accepted entropies (a bound on their mutual information) within the
budget gamma = 0.1; every position that is not accepted is re-noised to a uniform random token so
the next forward pass explores it.  The temperature falls linearly from 0.8 to 0.4 along the
denoising time axis.  Denoising stops early once the mean predictive entropy over the canvas is
below 0.005 and the deterministic prediction (the most likely token sequence) is the same in two
consecutive steps; at most T = 48 steps.  The model's prediction is p_hat_0 = softmax(logits / tau)
[TR §디노이징 반복과 self-conditioning]; the noise is uniform over the vocabulary (multinomial
diffusion), so tokens settled at one step may change at a later one [TR §아키텍처와 블록 자기회귀 생성].

Readings where the pages leave a step open:
  * entropy in nats, of softmax(z / tau_t) over the whole vocabulary;
  * an accepted position takes a draw from p_hat_0 (Gumbel-max, the same draw as the Euler Step),
    which is what the temperature acts on; every step re-evaluates every position (no locks);
  * the accepted count is the largest k whose sum of the k smallest entropies is <= gamma (it may
    be 0); ties in entropy go to the lower position;
  * decisions are taken on float32 entropies: the ascending order, the running sum (sequential,
    float32) and the mean (float32 total over all positions, in the same order, divided by L);
  * tau_t = tau_end + (tau_start - tau_end) * t with t_s = 1 - s/T;
  * the first step has no previous prediction, so it never stops; when a canvas stops, and at
    the last step, it takes the deterministic prediction (argmax of every position);
  * re-noise tokens come from their own Philox stream (tag 5).
"""
from __future__ import annotations

import numpy as np

from . import philox
from . import step as S

GAMMA = 0.1
STOP_ENTROPY = 0.005
TAU_START, TAU_END = 0.8, 0.4


def temperature(t, tau_start=TAU_START, tau_end=TAU_END):
    """Linear in the denoising time: tau(1) = tau_start, tau(0) = tau_end."""
    return tau_end + (tau_start - tau_end) * t


def entropy(z, rows_chunk=64):
    """H = -sum_v p_v ln p_v of p = softmax(z) per row, float64 (z already divided by tau)."""
    z = np.asarray(z, np.float64)
    out = np.empty(z.shape[0])
    for r0 in range(0, z.shape[0], rows_chunk):
        zz = z[r0:r0 + rows_chunk]
        m = zz.max(axis=1, keepdims=True)
        e = np.exp(zz - m)
        s = e.sum(axis=1, keepdims=True)
        p = e / s
        # ln Z - E_p[z], with ln Z = m + ln s
        out[r0:r0 + rows_chunk] = (m + np.log(s))[:, 0] - (p * zz).sum(axis=1)
    return out


def select(H32, gamma=GAMMA):
    """Accepted positions of one canvas from float32 entropies [L].

    Returns (accepted mask [L], k, mean entropy as float32)."""
    H32 = np.maximum(np.asarray(H32, np.float32), np.float32(0.0))
    L = H32.shape[0]
    order = np.lexsort((np.arange(L), H32))          # ascending entropy, then position
    run = np.cumsum(H32[order], dtype=np.float32)     # sequential float32 running sum
    k = int(np.count_nonzero(run <= np.float32(gamma)))
    acc = np.zeros(L, dtype=bool)
    acc[order[:k]] = True
    mean = np.float32(run[-1]) / np.float32(L)
    return acc, k, np.float32(mean)


def update(a, y, H32, prev_a, done, seed, s, vocab, gamma=GAMMA, stop_entropy=STOP_ENTROPY, final=False,
           canvas=None, adaptive=True):
    """One entropy-bounded step for a block of canvases, from the per-position argmax a, the
    Gumbel-max draw y and float32 entropies (all [B][L]).  `prev_a` is the previous step's
    argmax (None at the first step); canvases with done[b] keep `canvas[b]`.  Without `adaptive`
    a canvas only finishes at the final step.

    Returns canvas, done, n_accepted [B], mean entropy [B] (float32), stopped [B]."""
    a = np.asarray(a); y = np.asarray(y); H32 = np.asarray(H32, np.float32)
    B, L = a.shape
    renoise = philox.renoise_tokens(seed, s, B, L, vocab)
    out = np.array(canvas, copy=True) if canvas is not None else np.zeros((B, L), np.int64)
    done = np.array(done, dtype=bool, copy=True)
    n_acc = np.zeros(B, np.int64)
    mean = np.zeros(B, np.float32)
    stopped = np.zeros(B, dtype=bool)
    for b in range(B):
        if done[b]:
            continue
        acc, k, mb = select(H32[b], gamma)
        n_acc[b], mean[b] = k, mb
        stable = prev_a is not None and np.array_equal(np.asarray(prev_a)[b], a[b])
        stop = adaptive and stable and mb < np.float32(stop_entropy)
        if stop or final:
            out[b] = a[b]
            done[b] = True
            stopped[b] = stop
        else:
            out[b] = np.where(acc, y[b], renoise[b])
    return out, done, n_acc, mean, stopped


def stats_from_logits(z, seed, s, B, L):
    """argmax, Gumbel-max draw and float64 entropy per row of z (already divided by tau)."""
    rows = np.arange(B * L)
    st = S.sample_stats(np.asarray(z, np.float64), seed, s, rows // L, rows % L)
    st["H"] = entropy(z)
    return st


def run(cfg, W, forward, steps=48, tau_start=TAU_START, tau_end=TAU_END, gamma=GAMMA,
        stop_entropy=STOP_ENTROPY, adaptive=True, seed=None, canvas=None, trace=None, self_cond=None):
    """The sampler's loop over one block of canvases: uniform canvas at t = 1, then at most `steps`
    forward passes.  With `self_cond` ((H, tau_t) -> s) the decoder is called as forward(x, s) with
    s = None at the first step and the previous step's signal afterwards.  Returns canvas,
    steps_taken [B]."""
    B, L = cfg.batch, cfg.canvas
    seed = cfg.seed if seed is None else seed
    x = S.init_canvas(seed, B, L, cfg.vocab) if canvas is None else np.asarray(canvas).copy()
    done = np.zeros(B, dtype=bool)
    taken = np.zeros(B, dtype=np.int64)
    prev = None
    sc = None
    ts, h = S.time_grid(steps)
    for s, t in enumerate(ts):
        if done.all():
            break
        tau = temperature(t, tau_start, tau_end)
        Hh = forward(x) if self_cond is None else forward(x, sc)
        if self_cond is not None:
            sc = self_cond(Hh, tau)
        z = S.logits(Hh, W["embed"], tau)
        st = stats_from_logits(z, seed, s, B, L)
        a, y = st["a"].reshape(B, L), st["y"].reshape(B, L)
        H32 = st["H"].astype(np.float32).reshape(B, L)
        was_done = done.copy()
        x, done, n_acc, mean, stopped = update(a, y, H32, prev, done, seed, s, cfg.vocab, gamma, stop_entropy,
                                               final=(s == steps - 1), canvas=x, adaptive=adaptive)
        taken += ~was_done
        prev = a
        if trace is not None:
            trace.append({"s": s, "tau": tau, "stats": st, "n_acc": n_acc, "mean": mean, "canvas": x.copy()})
    return x, taken
