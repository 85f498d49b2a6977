"""Pins of the oracle's layer composition and of its Philox bits (CPU).

The decoder layer is a pre-norm residual block [TR §아키텍처와 블록 자기회귀 생성; reading: pre-norm
RMSNorm blocks, a final norm before the LM head].  Its parts (attention, RoPE, RMSNorm, MoE) are
pinned one by one in test_oracle_model.py; here zero-weight reductions tie their composition to
expectations written out independently in this file:

  * W_o = 0 and every routed and shared down matrix = 0: each layer adds nothing, so the residual
    is the embedding and H = stored(RMSNorm(E[x]) * g_final) exactly;
  * W_o = 0: layer(h) = h + MoE(RMSNorm(h) * g_ffn), the MoE written as the dense softmax mixture
    (top-k = all experts) plus the shared expert, with explicit loops;
  * every down matrix = 0: layer(h) = h + Attn(RMSNorm(h) * g_attn) W_o^T, the attention written
    as explicit per-query loops with the rotation of each (j, j + dh/2) pair spelled out, on a
    global layer and on a local (ring) layer.

Planted mistakes (a post-norm layer, a dropped residual, swapped norm gains, swapped Philox
multipliers) are applied to the oracle on the CPU and must fail these checks.

The Philox4x32-10 known-answer vectors in golden/philox4x32_10_kat.txt are those published with
the Random123 library of Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2,
3" (SC'11).
"""
import math
import os

import numpy as np
import pytest

from oracle import model as M
from oracle import philox as PX
from oracle.numerics import identity, round_bf16
from synth.configs import C0

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.txt")


# ---------------------------------------------------------------- Philox known answers ---------

def _kat():
    rows = []
    for line in open(GOLDEN):
        if line.strip() and not line.startswith("#"):
            w = [int(x, 16) for x in line.split()]
            rows.append((w[:4], w[4:6], w[6:]))
    assert len(rows) == 3
    return rows


def _matches_kat():
    return all([int(x) for x in PX.philox4x32_10(np.array(c), k)] == o for c, k, o in _kat())


def test_philox_known_answer_vectors():
    for c, k, o in _kat():
        got = [int(x) for x in PX.philox4x32_10(np.array(c), k)]
        assert got == o, (c, k, [hex(x) for x in got])
    # the same vectors through a batched call (broadcast over leading axes)
    ctr = np.array([c for c, _, _ in _kat()])
    for j, (c, k, o) in enumerate(_kat()):
        assert [int(x) for x in PX.philox4x32_10(ctr, k)[j]] == o


@pytest.mark.parametrize("mutation", ["swap_mul", "weyl", "one_round_less"])
def test_planted_philox_mistakes_fail_the_vectors(monkeypatch, mutation):
    if mutation == "swap_mul":
        monkeypatch.setattr(PX, "MUL0", PX.MUL1)
        monkeypatch.setattr(PX, "MUL1", 0xD2511F53)
    elif mutation == "weyl":
        monkeypatch.setattr(PX, "WEYL0", PX.WEYL0 ^ 1)
    else:
        real = PX.philox4x32_10

        def nine_rounds(ctr, key):
            # ten rounds from the key bumped once = rounds 2..11, not rounds 1..10
            k = ((int(key[0]) + 0x9E3779B9) & 0xFFFFFFFF, (int(key[1]) + 0xBB67AE85) & 0xFFFFFFFF)
            return real(ctr, k)
        monkeypatch.setattr(PX, "philox4x32_10", nine_rounds)
    assert not _matches_kat()


# ---------------------------------------------------------------- layer composition ------------

def tiny(**kw):
    base = dict(n_layers=2, d_model=32, n_q_heads=4, n_kv_heads=2, head_dim=8, n_experts=4,
                top_k=4, expert_hidden=16, shared_hidden=24, vocab=64, window=0, global_every=0,
                act_dtype="f32", expert_dtype="f32", batch=2, canvas=6, prefix=10)
    base.update(kw)
    return C0.replace(**base)


def rand_layer(cfg, rng, std=0.3):
    d, E, f, fs = cfg.d_model, cfg.n_experts, cfg.expert_hidden, cfg.shared_hidden
    n = lambda *s: rng.standard_normal(s) * std
    return {"attn_norm": 0.5 + rng.random(d), "ffn_norm": 0.5 + rng.random(d),
            "w_qkv": n(cfg.qkv_rows, d), "w_o": n(d, cfg.n_q_heads * cfg.head_dim), "w_router": n(E, d),
            "router_bias": None, "w_gate": n(E, f, d), "w_up": n(E, f, d), "w_down": n(E, d, f),
            "sh_gate": n(fs, d), "sh_up": n(fs, d), "sh_down": n(d, fs)}


def zero_down(lw):
    lw = dict(lw)
    lw["w_down"] = np.zeros_like(lw["w_down"])
    lw["sh_down"] = np.zeros_like(lw["sh_down"])
    return lw


def zero_wo(lw):
    lw = dict(lw)
    lw["w_o"] = np.zeros_like(lw["w_o"])
    return lw


def caches(cfg, rng, layer, P):
    cap = P if M.is_global(cfg, layer) else cfg.window
    sh = (cfg.batch, cfg.n_kv_heads, cap, cfg.head_dim)
    return rng.standard_normal(sh), rng.standard_normal(sh)


def norm_rows(h, g, eps):
    out = np.empty_like(h)
    for t in range(h.shape[0]):
        ms = sum(float(v) * float(v) for v in h[t]) / h.shape[1]
        out[t] = h[t] / math.sqrt(ms + eps) * g
    return out


def expect_moe(x, lw):
    """Dense mixture over all experts (softmax of the float32 router logits) plus the shared
    expert, with explicit loops."""
    T, d = x.shape
    E = lw["w_router"].shape[0]
    out = np.zeros((T, d))
    for t in range(T):
        r = [float(np.float32(sum(x[t, c] * lw["w_router"][e, c] for c in range(d)))) for e in range(E)]
        mx = max(r)
        w = [math.exp(v - mx) for v in r]
        tot = sum(w)
        for e in range(E):
            g = lw["w_gate"][e] @ x[t]
            u = lw["w_up"][e] @ x[t]
            a = np.array([gi / (1.0 + math.exp(-gi)) * ui for gi, ui in zip(g, u)])
            out[t] += (w[e] / tot) * (lw["w_down"][e] @ a)
        g = lw["sh_gate"] @ x[t]
        u = lw["sh_up"] @ x[t]
        a = np.array([gi / (1.0 + math.exp(-gi)) * ui for gi, ui in zip(g, u)])
        out[t] += lw["sh_down"] @ a
    return out


def rotate(vec, p, theta):
    """Rotary embedding of one head vector at position p: element j pairs with j + dh/2."""
    dh = len(vec)
    h2 = dh // 2
    out = np.array(vec, dtype=np.float64)
    for j in range(h2):
        a = p * theta ** (-2.0 * j / dh)
        x1, x2 = vec[j], vec[j + h2]
        out[j] = x1 * math.cos(a) - x2 * math.sin(a)
        out[j + h2] = x2 * math.cos(a) + x1 * math.sin(a)
    return out


def expect_attention_out(cfg, layer, x, lw, K, V, plen):
    """Bidirectional canvas attention of the normalised rows x [B*L][d], projected by W_o.
    Visible prefix slots: all P on a global layer, the first min(P, W) ring slots on a local one
    (block-anchored window); plus every canvas key."""
    B, L = len(plen), x.shape[0] // len(plen)
    Hq, Hkv, dh = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    Wq = lw["w_qkv"][:Hq * dh]
    Wk = lw["w_qkv"][Hq * dh:(Hq + Hkv) * dh]
    Wv = lw["w_qkv"][(Hq + Hkv) * dh:]
    o = np.zeros((B * L, Hq * dh))
    for b in range(B):
        P = plen[b]
        nvis = P if M.is_global(cfg, layer) else min(P, cfg.window)
        rows = range(b * L, (b + 1) * L)
        kc = {g: [rotate(Wk[g * dh:(g + 1) * dh] @ x[t], P + i, cfg.rope_theta) for i, t in enumerate(rows)]
              for g in range(Hkv)}
        vc = {g: [Wv[g * dh:(g + 1) * dh] @ x[t] for t in rows] for g in range(Hkv)}
        for i, t in enumerate(rows):
            for j in range(Hq):
                g = j // (Hq // Hkv)
                q = rotate(Wq[j * dh:(j + 1) * dh] @ x[t], P + i, cfg.rope_theta)
                keys = [K[b, g, s] for s in range(nvis)] + kc[g]
                vals = [V[b, g, s] for s in range(nvis)] + vc[g]
                sc = [float(q @ k) / math.sqrt(dh) for k in keys]
                mx = max(sc)
                w = [math.exp(s - mx) for s in sc]
                tot = sum(w)
                o[t, j * dh:(j + 1) * dh] = sum(wi * v for wi, v in zip(w, vals)) / tot
    return o @ lw["w_o"].T


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_all_outputs_zero_gives_normed_embedding(act):
    """W_o = 0 and every down matrix = 0: the residual is E[x] exactly and H = stored(RMSNorm(E[x]) *
    g_final)."""
    cfg = tiny(act_dtype=act, n_layers=3, window=4, global_every=3)
    rng = np.random.default_rng(20)
    rnd = round_bf16 if act == "bf16" else identity
    emb = rnd(rng.standard_normal((cfg.vocab, cfg.d_model)))
    gfin = rnd(0.5 + rng.random(cfg.d_model))
    W = {"embed": emb, "final_norm": gfin,
         "layers": [zero_wo(zero_down(rand_layer(cfg, rng))) for _ in range(cfg.n_layers)]}
    kv = [caches(cfg, rng, l, 10) for l in range(cfg.n_layers)]
    canvas = rng.integers(0, cfg.vocab, size=(cfg.batch, cfg.canvas))
    H, h = M.denoise_forward(cfg, W, kv, [10, 10], canvas=canvas)
    h0 = emb[canvas.reshape(-1)]
    assert np.array_equal(h, h0)
    # equal up to the float64 summation order of the mean square
    assert np.allclose(H, rnd(norm_rows(h0, gfin, cfg.norm_eps)), rtol=1e-12, atol=0)


def test_zero_attention_output_gives_residual_plus_moe():
    """W_o = 0: layer(h) = h + MoE(RMSNorm(h) * g_ffn)."""
    cfg = tiny()
    rng = np.random.default_rng(21)
    lw = zero_wo(rand_layer(cfg, rng))
    K, V = caches(cfg, rng, 0, 10)
    h = rng.standard_normal((cfg.batch * cfg.canvas, cfg.d_model)) * 2.0
    got, _ = M.denoise_layer(cfg, 0, h, lw, K, V, [10, 10], identity)
    want = h + expect_moe(norm_rows(h, lw["ffn_norm"], cfg.norm_eps), lw)
    assert np.allclose(got, want, rtol=1e-10, atol=1e-10)


@pytest.mark.parametrize("local", [False, True])
def test_zero_ffn_output_gives_residual_plus_attention(local):
    """Every routed and shared down matrix = 0: layer(h) = h + Attn(RMSNorm(h) * g_attn) W_o^T."""
    cfg = tiny(window=4, global_every=6) if local else tiny()
    rng = np.random.default_rng(22)
    lw = zero_down(rand_layer(cfg, rng))
    plen = [10, 3]
    K, V = caches(cfg, rng, 0, 10)
    h = rng.standard_normal((cfg.batch * cfg.canvas, cfg.d_model)) * 2.0
    got, _ = M.denoise_layer(cfg, 0, h, lw, K, V, plen, identity)
    want = h + expect_attention_out(cfg, 0, norm_rows(h, lw["attn_norm"], cfg.norm_eps), lw, K, V, plen)
    assert np.allclose(got, want, rtol=1e-10, atol=1e-10)


def test_full_layer_is_the_two_residual_blocks_in_order():
    """With every weight live: layer(h) = h1 + MoE(RMSNorm(h1) g_ffn), h1 = h + Attn(RMSNorm(h) g_attn) W_o^T."""
    cfg = tiny(window=4, global_every=6)
    rng = np.random.default_rng(23)
    lw = rand_layer(cfg, rng)
    plen = [10, 7]
    K, V = caches(cfg, rng, 0, 10)
    h = rng.standard_normal((cfg.batch * cfg.canvas, cfg.d_model)) * 2.0
    got, _ = M.denoise_layer(cfg, 0, h, lw, K, V, plen, identity)
    h1 = h + expect_attention_out(cfg, 0, norm_rows(h, lw["attn_norm"], cfg.norm_eps), lw, K, V, plen)
    want = h1 + expect_moe(norm_rows(h1, lw["ffn_norm"], cfg.norm_eps), lw)
    assert np.allclose(got, want, rtol=1e-10, atol=1e-10)


# ---------------------------------------------------------------- planted layer mistakes -------

_REAL_LAYER = M.denoise_layer


def _post_norm_layer(cfg, layer, h, lw, K, V, prefix_len, rnd, forced_idx=None):
    """A post-norm variant: h1 = RMSNorm(h + Attn(h)), out = RMSNorm(h1 + MoE(h1))."""
    o = np.zeros((h.shape[0], cfg.n_q_heads * cfg.head_dim))
    B, L = len(prefix_len), h.shape[0] // len(prefix_len)
    for b in range(B):
        rows = slice(b * L, (b + 1) * L)
        q, k, v = M.qkv(cfg, h[rows], lw, prefix_len[b] + np.arange(L), rnd)
        o[rows] = M.canvas_attention(cfg, layer, q, k.transpose(1, 0, 2), v.transpose(1, 0, 2), K[b], V[b],
                                     prefix_len[b]).reshape(L, -1)
    h1 = M.rmsnorm(h + o @ lw["w_o"].T, lw["attn_norm"], cfg.norm_eps)
    f, info = M.moe(cfg, h1, lw, rnd)
    return M.rmsnorm(h1 + f, lw["ffn_norm"], cfg.norm_eps), info


def _dropped_residual_layer(cfg, layer, h, lw, K, V, prefix_len, rnd, forced_idx=None):
    out, info = _REAL_LAYER(cfg, layer, h, lw, K, V, prefix_len, rnd, forced_idx)
    return out - h, info


def _swapped_gains_layer(cfg, layer, h, lw, K, V, prefix_len, rnd, forced_idx=None):
    lw2 = dict(lw)
    lw2["attn_norm"], lw2["ffn_norm"] = lw["ffn_norm"], lw["attn_norm"]
    return _REAL_LAYER(cfg, layer, h, lw2, K, V, prefix_len, rnd, forced_idx)


def _reductions():
    return (lambda: test_all_outputs_zero_gives_normed_embedding("f32"),
            test_zero_attention_output_gives_residual_plus_moe,
            lambda: test_zero_ffn_output_gives_residual_plus_attention(False),
            test_full_layer_is_the_two_residual_blocks_in_order)


@pytest.mark.parametrize("mutant", [_post_norm_layer, _dropped_residual_layer, _swapped_gains_layer])
def test_planted_layer_mistakes_fail_a_reduction(monkeypatch, mutant):
    monkeypatch.setattr(M, "denoise_layer", mutant)
    failures = 0
    for check in _reductions():
        try:
            check()
        except AssertionError:
            failures += 1
    assert failures >= 1
