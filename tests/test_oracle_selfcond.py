"""Pins of the self-conditioning oracle (CPU) [TR §디노이징 반복과 self-conditioning; parameter table].

  * the expected embedding p_hat_0 . E: a near-zero temperature with a clear winner gives the
    winner's embedding row; all-equal logits give the mean of E; an explicit softmax-weighted
    loop on a tiny case; relabelling the vocabulary (rows of E and the logit columns together)
    changes nothing
  * the feed-forward block against explicit loops, with bf16 storage at its input and hidden product
  * the decoder input: with W_o and every down matrix zero the residual is E[x] + s exactly
  * the loop: a self-conditioning function that returns zeros leaves the run unchanged, and the
    first step of a canvas always sees s = 0
  * the assumed block width: 3 * 2816 * 896 is within 3% of the pages' 7.8M parameters
"""
import math

import numpy as np

from oracle import model as M
from oracle import selfcond as SC
from oracle import step as S
from oracle.numerics import identity, round_bf16
from synth.configs import C0, C2


def test_low_temperature_gives_the_argmax_row():
    rng = np.random.default_rng(30)
    E = rng.standard_normal((50, 8))
    H = rng.standard_normal((6, 8))
    z = H @ E.T
    a = np.argmax(z, axis=1)
    srt = np.sort(z, axis=1)
    gap = srt[:, -1] - srt[:, -2]
    tau = float(gap.min()) / 60.0          # exp(-60) below double precision relative to 1
    e = SC.expected_embedding(H, E, tau)
    assert np.allclose(e, E[a], rtol=0, atol=1e-12)


def test_equal_logits_give_the_mean_embedding():
    rng = np.random.default_rng(31)
    E = rng.standard_normal((37, 5))
    e = SC.expected_embedding(np.zeros((3, 5)), E, 0.7)
    mean = [sum(E[v, c] for v in range(37)) / 37 for c in range(5)]
    for r in range(3):
        assert np.allclose(e[r], mean, rtol=1e-13, atol=1e-15)


def test_expected_embedding_explicit_loop_and_relabelling():
    rng = np.random.default_rng(32)
    V, d = 23, 6
    E = rng.standard_normal((V, d))
    H = rng.standard_normal((4, d)) * 2
    tau = 0.8
    e = SC.expected_embedding(H, E, tau)
    for r in range(4):
        z = [sum(H[r, c] * E[v, c] for c in range(d)) / tau for v in range(V)]
        mx = max(z)
        w = [math.exp(x - mx) for x in z]
        tot = sum(w)
        want = [sum(w[v] * E[v, c] for v in range(V)) / tot for c in range(d)]
        assert np.allclose(e[r], want, rtol=1e-12, atol=1e-14)
    perm = rng.permutation(V)
    assert np.allclose(SC.expected_embedding(H, E[perm], tau), e, rtol=1e-12, atol=1e-14)


def test_ffw_explicit_loops_and_storage_rounding():
    rng = np.random.default_rng(33)
    d, f = 8, 5
    x = rng.standard_normal((3, d))
    Wg, Wu, Wd = rng.standard_normal((f, d)), rng.standard_normal((f, d)), rng.standard_normal((d, f))
    for rnd in (identity, round_bf16):
        got = SC.ffw(x, Wg, Wu, Wd, rnd)
        xs = rnd(x)
        for t in range(3):
            A = []
            for j in range(f):
                g = sum(xs[t, c] * Wg[j, c] for c in range(d))
                u = sum(xs[t, c] * Wu[j, c] for c in range(d))
                A.append(g / (1.0 + math.exp(-g)) * u)
            A = rnd(np.array(A))
            want = [sum(A[j] * Wd[c, j] for j in range(f)) for c in range(d)]
            assert np.allclose(got[t], want, rtol=1e-11, atol=1e-12)


def _tiny_model(rng, cfg, zero_out=False):
    d, E_, f, fs = cfg.d_model, cfg.n_experts, cfg.expert_hidden, cfg.shared_hidden
    n = lambda *s: rng.standard_normal(s) * 0.3
    layers = []
    for _ in range(cfg.n_layers):
        lw = {"attn_norm": np.ones(d), "ffn_norm": np.ones(d), "w_qkv": n(cfg.qkv_rows, d),
              "w_o": n(d, cfg.n_q_heads * cfg.head_dim), "w_router": n(E_, d), "router_bias": None,
              "w_gate": n(E_, f, d), "w_up": n(E_, f, d), "w_down": n(E_, d, f),
              "sh_gate": n(fs, d), "sh_up": n(fs, d), "sh_down": n(d, fs)}
        if zero_out:
            lw["w_o"] = np.zeros_like(lw["w_o"])
            lw["w_down"] = np.zeros_like(lw["w_down"])
            lw["sh_down"] = np.zeros_like(lw["sh_down"])
        layers.append(lw)
    return {"embed": rng.standard_normal((cfg.vocab, d)), "final_norm": np.ones(d), "layers": layers}


def _tiny_cfg():
    return C0.replace(n_layers=2, d_model=16, n_q_heads=2, n_kv_heads=2, head_dim=8, n_experts=4, top_k=2,
                      expert_hidden=8, shared_hidden=8, vocab=40, batch=2, canvas=6, prefix=5, steps=3,
                      tau=0.5, lock_threshold=0.99)


def test_signal_enters_as_an_addition_to_the_embedded_canvas():
    cfg = _tiny_cfg()
    rng = np.random.default_rng(34)
    W = _tiny_model(rng, cfg, zero_out=True)
    kv = [(rng.standard_normal((2, 2, 5, 8)), rng.standard_normal((2, 2, 5, 8))) for _ in range(2)]
    canvas = rng.integers(0, cfg.vocab, size=(2, 6))
    s = rng.standard_normal((12, 16)) * 0.1
    _, h = M.denoise_forward(cfg, W, kv, [5, 5], canvas=canvas, sc=s)
    assert np.array_equal(h, W["embed"][canvas.reshape(-1)] + s)


def test_zero_signal_leaves_the_loop_unchanged_and_first_step_sees_zero():
    cfg = _tiny_cfg()
    rng = np.random.default_rng(35)
    W = _tiny_model(rng, cfg)
    kv = [(rng.standard_normal((2, 2, 5, 8)), rng.standard_normal((2, 2, 5, 8))) for _ in range(2)]
    seen = []

    def fwd(c, s=None):
        seen.append(s)
        return M.denoise_forward(cfg, W, kv, [5, 5], canvas=c, sc=s)[0]
    base = S.canvas_run(cfg, W, kv, [5, 5], lambda c: fwd(c))
    seen.clear()
    zero = S.canvas_run(cfg, W, kv, [5, 5], fwd, self_cond=lambda H, tau: np.zeros_like(H))
    assert seen[0] is None and all(x is not None for x in seen[1:])
    for a, b in zip(base, zero):
        assert np.array_equal(a, b)
    # a non-zero signal changes the run only from the second step on
    seen.clear()
    sc_w = (rng.standard_normal((8, 16)), rng.standard_normal((8, 16)), rng.standard_normal((16, 8)))
    cond = S.canvas_run(cfg, W, kv, [5, 5], fwd, steps=1,
                        self_cond=lambda H, tau: SC.self_condition(H, W["embed"], tau, sc_w, identity))
    first = S.canvas_run(cfg, W, kv, [5, 5], lambda c: fwd(c), steps=1)
    for a, b in zip(cond, first):
        assert np.array_equal(a, b)


def test_block_width_matches_the_parameter_table():
    assert abs(3 * C2.d_model * 896 / 7.8e6 - 1.0) < 0.03
