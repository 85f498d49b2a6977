"""Block-autoregressive generation and its efficiency accounting (test infrastructure only).

Pages [TR §아키텍처와 블록 자기회귀 생성]: flow matching works on fixed-length sequences, so long
outputs are generated block by block: (1) the system and user prompt pass through the causal
encoder into a KV cache; (2) a 256-token canvas of uniform random tokens is refined by the
bidirectional decoder, which attends to the cache; (3) the finished canvas passes through the
causal encoder again, is appended to the cache, and the next canvas starts.  This repeats until
the end-of-turn token appears; the canvases concatenated are the response.

[TR §추론 효율 지표]: with K canvases, s_k denoising steps and n_k valid tokens (up to the first
EOS) of canvas k: total tokens = sum n_k, total steps = sum s_k, effective denoising steps =
sum n_k s_k / total tokens, TPF = total tokens / (total steps + K - 1) (the K - 1 passes that
append each finished canvas), TPS = TPF / t_fwd.

Readings where the pages leave a step open:
  * canvas k draws its random numbers from seed + k (the same streams as a single canvas run);
  * every canvas but the last is appended, whatever it holds; the generation runs a fixed number
    of canvases and the EOS only decides which tokens count (no host-side early exit);
  * n_k counts the tokens before the first EOS of the sequence (the EOS itself is not counted); a
    canvas with no EOS counts L; canvases after the one holding the first EOS count 0;
  * K in the accounting is the number of canvases up to and including the one with the first EOS
    (all canvases if none), and only their steps count.
"""
from __future__ import annotations

import numpy as np

from . import eb
from . import model as M
from . import step as S


def valid_counts(out, eos):
    """n[k][b] for canvases out [K][B][L]."""
    out = np.asarray(out)
    K, B, L = out.shape
    n = np.zeros((K, B), np.int64)
    for b in range(B):
        ended = False
        for k in range(K):
            if ended:
                continue
            hits = np.flatnonzero(out[k, b] == eos)
            if hits.size:
                n[k, b] = hits[0]
                ended = True
            else:
                n[k, b] = L
    return n


def metrics(steps, valid, eos_seen):
    """Per sequence b: total tokens, total steps, effective steps, TPF (over the K_b canvases up to
    and including the first EOS, all of them if none).  steps, valid [K][B]; eos_seen [K][B] bool."""
    steps = np.asarray(steps); valid = np.asarray(valid); eos_seen = np.asarray(eos_seen, bool)
    K, B = steps.shape
    out = []
    for b in range(B):
        hit = np.flatnonzero(eos_seen[:, b])
        Kb = int(hit[0]) + 1 if hit.size else K
        n = valid[:Kb, b].astype(np.float64)
        s = steps[:Kb, b].astype(np.float64)
        tokens, total_steps = n.sum(), s.sum()
        out.append({"canvases": Kb, "tokens": tokens, "steps": total_steps,
                    "effective_steps": float((n * s).sum() / tokens) if tokens > 0 else 0.0,
                    "tpf": float(tokens / (total_steps + Kb - 1))})
    return out


def continuous_passes(steps):
    """Forward passes of the continuous schedule [TR §CPU-GPU 동기화 제거: denoising canvases and
    cache updates share a batch; TR §추론 효율 지표: K - 1 append passes]: every sequence proceeds on
    its own, s_k,b denoising passes for canvas k and one append pass after every canvas but the
    last, and a batch runs until its longest sequence is done: max_b (sum_k s_k,b + K - 1).
    The lockstep schedule (every canvas k waits for the slowest sequence, then all append together)
    takes sum_k max_b s_k,b + K - 1.  steps [K][B]; returns (continuous, lockstep)."""
    steps = np.asarray(steps, dtype=np.int64)
    K = steps.shape[0]
    return int(steps.sum(axis=0).max() + K - 1), int(steps.max(axis=1).sum() + K - 1)


def eos_mask(out, eos):
    out = np.asarray(out)
    return (out == eos).any(axis=2)


def generate(cfg, W, kv, prefix_len, K, eos, sampler="euler", steps=None, seed=None, eb_kw=None, trace=None,
             self_cond=None):
    """K canvases after an encoded prompt (kv, prefix_len).  Returns out [K][B][L], steps [K][B],
    the caches and prefix lengths after the appends.  With `self_cond` ((H, tau) -> s) every canvas
    starts from s = 0 and feeds each step's signal into its next decoder pass; the appending
    encoder pass takes none."""
    B, L = cfg.batch, cfg.canvas
    seed = cfg.seed if seed is None else seed
    T = cfg.steps if steps is None else steps
    out = np.zeros((K, B, L), np.int64)
    taken = np.zeros((K, B), np.int64)
    plen = list(prefix_len)
    for k in range(K):
        fwd = lambda c, sc=None, kv=kv, plen=plen: M.denoise_forward(cfg, W, kv, plen, canvas=c, sc=sc)[0]
        if sampler == "euler":
            x, _, tk = S.canvas_run(cfg, W, kv, plen, fwd, steps=T, seed=seed + k, self_cond=self_cond)
        else:
            x, tk = eb.run(cfg, W, fwd, steps=T, seed=seed + k, self_cond=self_cond, **(eb_kw or {}))
        out[k], taken[k] = x, tk
        if trace is not None:
            trace.append({"k": k, "prefix": list(plen)})
        if k + 1 < K:
            kv, plen = M.prefill(cfg, W, kv, plen, x)
    return out, taken, kv, plen
