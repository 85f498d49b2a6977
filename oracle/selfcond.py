"""Self-conditioning, plainly (test infrastructure only).

Pages [TR §디노이징 반복과 self-conditioning]: the decoder takes the noisy canvas x_t, the context
KV cache and a continuous self-conditioning signal s_t that feeds the previous prediction back in:
    logits = Decoder(x_t, KV, s_t);  p_hat_0 = softmax(logits / tau_t);
    s_(t-h) = FFW(p_hat_0 . E)   (E: the token embedding matrix);  x_(t-h) ~ Step(x_t, p_hat_0).
The parameter table lists a 7.8M-parameter self-conditioning block [TR parameter table], trained
with half of each batch conditioned on the previous pass's signal and half on zero [TR §Downstream
finetuning]; [TR §GPU 시간 분석] counts the embedding product over the whole 262k vocabulary and the
canvas-wide softmax, in full precision, in the sampling time.

Readings where the pages are silent:
  * p_hat_0 . E is the expected embedding under p_hat_0: e_i = sum_v p_hat_0(v | i) E_v, with the
    same temperature as the Step's softmax; float64 here;
  * FFW is a gated feed-forward block like the model's experts: A = silu(x W_g^T) * (x W_u^T),
    s = A W_d^T, with x = e stored in the activation dtype and A stored in it too; at the assumed
    widths (d 2816) a hidden width of 896 gives 3 * 2816 * 896 = 7.57M parameters, the multiple of
    64 nearest the pages' 7.8M; no normalisation in front of it (the pages write FFW(p_hat_0 . E));
  * s enters the decoder added to the embedded canvas, h_0 = E[x_t] + s_t (the signal injects a
    continuous vector into the sequence); s = 0 at a canvas's first step (no previous prediction).
"""
from __future__ import annotations

import numpy as np


def expected_embedding(H, E, tau):
    """e = softmax(H E^T / tau) E, row by row, float64.  H [T][d], E [V][d] -> [T][d]."""
    H = np.asarray(H, np.float64)
    E = np.asarray(E, np.float64)
    out = np.empty((H.shape[0], E.shape[1]))
    for r0 in range(0, H.shape[0], 64):
        z = (H[r0:r0 + 64] @ E.T) / tau
        p = np.exp(z - z.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        out[r0:r0 + 64] = p @ E
    return out


def ffw(x, Wg, Wu, Wd, rnd):
    """The gated feed-forward block: x stored (rnd), A = silu(x Wg^T) * (x Wu^T) stored, s = A Wd^T."""
    x = rnd(x)
    g = x @ Wg.T
    A = rnd(g / (1.0 + np.exp(-g)) * (x @ Wu.T))
    return A @ Wd.T


def self_condition(H, E, tau, W_sc, rnd):
    """s_(t-h) from the final hidden states H of a decoder pass; W_sc = (Wg [f][d], Wu [f][d], Wd [d][f])."""
    Wg, Wu, Wd = W_sc
    return ffw(expected_embedding(H, E, tau), Wg, Wu, Wd, rnd)
