"""Pins of the oracle's forward pass (CPU): brute force, invariants and special cases.

  * attention equals an explicit per-query softmax loop; canvas attention without positional
    encoding is permutation-equivariant over the canvas and invariant to prefix-slot order; a
    single key returns its value; equal scores give the mean of V; a window at least as long as
    the prefix makes a local layer equal a global one; an empty prefix is plain bidirectional
    self-attention
  * RoPE preserves norms, is the identity at position 0 and q(m).k(n) depends on m - n only
  * MoE with top-k = E equals the dense softmax-weighted sum of all experts plus the shared
    expert; top-1 is the argmax expert plus the shared expert; relabelling experts together with
    router rows changes nothing; routing tables are a consistent grouping
  * causal prefill in two chunks equals one call (append-after-encode)
  * the assumed layer widths reproduce the pages' parameter table
"""
import math

import numpy as np
import pytest

from oracle import model as M
from oracle.numerics import identity, round_bf16
from synth.configs import C0, C2


def tiny(**kw):
    base = dict(n_layers=2, d_model=32, n_q_heads=4, n_kv_heads=2, head_dim=8, n_experts=6,
                top_k=2, expert_hidden=16, shared_hidden=24, vocab=64, window=0, global_every=0,
                act_dtype="f32", expert_dtype="f32", batch=2, canvas=8, prefix=12)
    base.update(kw)
    return C0.replace(**base)


def rand_layer(cfg, rng, std=0.3):
    d, E, f, fs = cfg.d_model, cfg.n_experts, cfg.expert_hidden, cfg.shared_hidden
    n = lambda *s: rng.standard_normal(s) * std
    return {"attn_norm": np.ones(d), "ffn_norm": np.ones(d), "w_qkv": n(cfg.qkv_rows, d),
            "w_o": n(d, cfg.n_q_heads * cfg.head_dim), "w_router": n(E, d), "router_bias": None,
            "w_gate": n(E, f, d), "w_up": n(E, f, d), "w_down": n(E, d, f),
            "sh_gate": n(fs, d), "sh_up": n(fs, d), "sh_down": n(d, fs)}


def rand_weights(cfg, rng):
    return {"embed": rng.standard_normal((cfg.vocab, cfg.d_model)),
            "final_norm": np.ones(cfg.d_model),
            "layers": [rand_layer(cfg, rng) for _ in range(cfg.n_layers)]}


# ---------------------------------------------------------------- attention -------------------

def test_attend_matches_explicit_loop():
    rng = np.random.default_rng(0)
    q, K, V = rng.standard_normal((5, 8)), rng.standard_normal((7, 8)), rng.standard_normal((7, 3))
    vis = rng.random((5, 7)) < 0.6
    vis[:, 0] = True
    got = M.attend(q, K, V, vis)
    for i in range(5):
        sc = [sum(q[i, c] * K[j, c] for c in range(8)) / math.sqrt(8) if vis[i, j] else None
              for j in range(7)]
        mx = max(s for s in sc if s is not None)
        w = [math.exp(s - mx) if s is not None else 0.0 for s in sc]
        tot = sum(w)
        want = [sum(w[j] * V[j, c] for j in range(7)) / tot for c in range(3)]
        assert np.allclose(got[i], want, rtol=1e-12, atol=1e-14)


def _canvas_inputs(rng, L=8, Hq=4, Hkv=2, dh=8, cap=12):
    return (rng.standard_normal((L, Hq, dh)), rng.standard_normal((Hkv, L, dh)),
            rng.standard_normal((Hkv, L, dh)), rng.standard_normal((Hkv, cap, dh)),
            rng.standard_normal((Hkv, cap, dh)))


@pytest.mark.parametrize("layer_global", [True, False])
def test_canvas_attention_permutation_equivariance(layer_global):
    cfg = tiny(window=0 if layer_global else 5, global_every=0 if layer_global else 6)
    rng = np.random.default_rng(1)
    q, kc, vc, Kp, Vp = _canvas_inputs(rng)
    P = 12 if layer_global else 5
    o = M.canvas_attention(cfg, 0, q, kc, vc, Kp, Vp, P)
    perm = rng.permutation(8)
    o2 = M.canvas_attention(cfg, 0, q[perm], kc[:, perm], vc[:, perm], Kp, Vp, P)
    assert np.allclose(o2, o[perm], rtol=1e-12, atol=1e-13)
    # order of the visible prefix slots does not matter
    n = M.prefix_slots(cfg, 0, P)
    sp = np.concatenate([rng.permutation(n), np.arange(n, 12)])
    o3 = M.canvas_attention(cfg, 0, q, kc, vc, Kp[:, sp], Vp[:, sp], P)
    assert np.allclose(o3, o, rtol=1e-12, atol=1e-13)


def test_attention_special_cases():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((3, 8))
    K1, V1 = rng.standard_normal((1, 8)), rng.standard_normal((1, 8))
    assert np.allclose(M.attend(q, K1, V1), np.repeat(V1, 3, axis=0))
    K = np.zeros((5, 8)); V = rng.standard_normal((5, 8))
    assert np.allclose(M.attend(q, K, V), np.repeat(V.mean(axis=0, keepdims=True), 3, axis=0))


def test_local_with_long_window_equals_global_and_empty_prefix_is_self_attention():
    rng = np.random.default_rng(3)
    q, kc, vc, Kp, Vp = _canvas_inputs(rng, cap=12)
    g = tiny()
    loc = tiny(window=64, global_every=6)
    assert not M.is_global(loc, 0)
    assert np.allclose(M.canvas_attention(g, 0, q, kc, vc, Kp, Vp, 12),
                       M.canvas_attention(loc, 0, q, kc, vc, Kp, Vp, 12), atol=1e-14)
    o = M.canvas_attention(g, 0, q, kc, vc, Kp, Vp, 0)
    for j in range(4):
        assert np.allclose(o[:, j], M.attend(q[:, j], kc[j // 2], vc[j // 2]), atol=1e-14)


def test_local_window_sees_only_last_w_positions():
    """Prefix keys older than the window do not change a local layer's output."""
    cfg = tiny(window=4, global_every=6)
    rng = np.random.default_rng(4)
    q, kc, vc, Kp, Vp = _canvas_inputs(rng, cap=4)
    o = M.canvas_attention(cfg, 0, q, kc, vc, Kp, Vp, 100)   # ring of 4 slots, prefix 100
    g = tiny()
    assert np.allclose(o, M.canvas_attention(g, 0, q, kc, vc, Kp, Vp, 4), atol=1e-14)


# ---------------------------------------------------------------- RoPE / norm -----------------

def test_rope_properties():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((6, 3, 16))
    pos = np.array([0, 1, 5, 100, 8191, 131071])
    r = M.rope(x, pos, 10000.0)
    assert np.allclose(np.linalg.norm(r, axis=-1), np.linalg.norm(x, axis=-1))
    assert np.allclose(r[0], x[0])
    q, k = rng.standard_normal((1, 1, 16)), rng.standard_normal((1, 1, 16))
    d1 = (M.rope(q, [7], 1e4) * M.rope(k, [3], 1e4)).sum()
    d2 = (M.rope(q, [1004], 1e4) * M.rope(k, [1000], 1e4)).sum()
    d3 = (M.rope(q, [3], 1e4) * M.rope(k, [7], 1e4)).sum()
    assert abs(d1 - d2) < 1e-9 and abs(d1 - d3) > 1e-6
    # pair (j, j + dh/2) rotates by pos * theta^(-2j/dh): check one element by hand
    e = np.zeros((1, 1, 16)); e[0, 0, 3] = 1.0
    ang = 5 * 10000.0 ** (-2 * 3 / 16)
    rr = M.rope(e, [5], 10000.0)
    assert np.isclose(rr[0, 0, 3], math.cos(ang)) and np.isclose(rr[0, 0, 11], math.sin(ang))


def test_rmsnorm_unit_rms():
    x = np.random.default_rng(6).standard_normal((4, 64)) * 7
    y = M.rmsnorm(x, np.ones(64), 1e-12)
    assert np.allclose(np.sqrt((y * y).mean(axis=1)), 1.0)


# ---------------------------------------------------------------- MoE -------------------------

def test_moe_topk_all_equals_dense_mixture():
    cfg = tiny(top_k=6)
    rng = np.random.default_rng(7)
    lw = rand_layer(cfg, rng)
    x = rng.standard_normal((10, cfg.d_model))
    out, info = M.moe(cfg, x, lw, identity)
    r = (x @ lw["w_router"].T).astype(np.float32).astype(np.float64)
    p = np.exp(r - r.max(axis=1, keepdims=True)); p /= p.sum(axis=1, keepdims=True)
    dense = np.zeros_like(x)
    for t in range(10):
        for e in range(cfg.n_experts):
            g = x[t] @ lw["w_gate"][e].T
            u = x[t] @ lw["w_up"][e].T
            dense[t] += p[t, e] * ((g / (1 + np.exp(-g)) * u) @ lw["w_down"][e].T)
        g = x[t] @ lw["sh_gate"].T
        u = x[t] @ lw["sh_up"].T
        dense[t] += (g / (1 + np.exp(-g)) * u) @ lw["sh_down"].T
    assert np.allclose(out, dense, rtol=1e-10, atol=1e-10)


def test_moe_top1_and_relabel_invariance():
    cfg = tiny(top_k=1)
    rng = np.random.default_rng(8)
    lw = rand_layer(cfg, rng)
    x = rng.standard_normal((10, cfg.d_model))
    out, info = M.moe(cfg, x, lw, identity)
    e = np.argmax((x @ lw["w_router"].T).astype(np.float32), axis=1)
    sh = M.swiglu(x, lw["sh_gate"], lw["sh_up"], lw["sh_down"], identity)
    for t in range(10):
        ex = M.swiglu(x[t:t + 1], lw["w_gate"][e[t]], lw["w_up"][e[t]], lw["w_down"][e[t]], identity)
        assert np.allclose(out[t], ex[0] + sh[t])
    cfg2 = tiny(top_k=2)
    out2, _ = M.moe(cfg2, x, lw, identity)
    perm = rng.permutation(cfg.n_experts)
    lw2 = dict(lw)
    for k in ("w_router", "w_gate", "w_up", "w_down"):
        lw2[k] = lw[k][perm]
    out3, _ = M.moe(cfg2, x, lw2, identity)
    assert np.allclose(out2, out3, rtol=1e-12, atol=1e-12)


def test_router_ties_and_tables():
    r = np.array([[1.0, 2.0, 2.0, 0.5, 2.0], [0.0, 0.0, 0.0, 0.0, 0.0]], dtype=np.float32)
    idx, gates = M.router_topk(r, 2)
    assert idx.tolist() == [[1, 2], [0, 1]]
    assert np.allclose(gates, 0.5)
    rng = np.random.default_rng(9)
    idx = np.stack([rng.choice(16, 4, replace=False) for _ in range(50)])
    counts, offsets, perm = M.route_tables(idx, 16)
    assert counts.sum() == 200 and offsets[0] == 0 and np.all(np.diff(offsets) == counts[:-1])
    assert sorted(perm.tolist()) == list(range(200))
    flat = idx.reshape(-1)
    for e in range(16):
        seg = perm[offsets[e]:offsets[e] + counts[e]]
        assert np.all(flat[seg] == e) and np.all(np.diff(seg) > 0)


# ---------------------------------------------------------------- prefill / forward -----------

@pytest.mark.parametrize("windowed", [False, True])
def test_prefill_in_chunks_equals_one_call(windowed):
    cfg = tiny(n_layers=3, window=5 if windowed else 0, global_every=3 if windowed else 0, batch=2)
    rng = np.random.default_rng(10)
    W = rand_weights(cfg, rng)
    cap = lambda l: 16 if M.is_global(cfg, l) else cfg.window
    kv0 = [(np.zeros((2, 2, cap(l), 8)), np.zeros((2, 2, cap(l), 8))) for l in range(3)]
    toks = rng.integers(0, cfg.vocab, size=(2, 11))
    kv_a, pa = M.prefill(cfg, W, kv0, [0, 0], toks)
    kv_b, pb = M.prefill(cfg, W, kv0, [0, 0], toks[:, :4])
    kv_b, pb = M.prefill(cfg, W, kv_b, pb, toks[:, 4:])
    assert pa == pb == [11, 11]
    for l in range(3):
        assert np.allclose(kv_a[l][0], kv_b[l][0], atol=1e-12)
        assert np.allclose(kv_a[l][1], kv_b[l][1], atol=1e-12)


def test_prefill_first_token_attends_to_itself_only():
    cfg = tiny(n_layers=1, batch=1)
    rng = np.random.default_rng(11)
    q = rng.standard_normal((3, 4, 8)); kn = rng.standard_normal((2, 3, 8)); vn = rng.standard_normal((2, 3, 8))
    o = M.causal_attention(cfg, 0, q, kn, vn, np.zeros((2, 8, 8)), np.zeros((2, 8, 8)), 0)
    for j in range(4):
        assert np.allclose(o[0, j], vn[j // 2, 0])


def test_denoise_forward_runs_and_bf16_rounds_at_storage_points():
    cfg = tiny(act_dtype="bf16")
    rng = np.random.default_rng(12)
    W = rand_weights(cfg, rng)
    kv = [(rng.standard_normal((2, 2, 12, 8)), rng.standard_normal((2, 2, 12, 8))) for _ in range(2)]
    canvas = rng.integers(0, cfg.vocab, size=(2, 8))
    H, h = M.denoise_forward(cfg, W, kv, [12, 12], canvas=canvas)
    assert np.array_equal(H, round_bf16(H))
    H2, _ = M.denoise_forward(cfg, W, kv, [12, 12], canvas=canvas)
    assert np.array_equal(H, H2)


# ---------------------------------------------------------------- shapes vs the pages ----------

def test_assumed_widths_reproduce_parameter_table():
    """25.2B total, 3.85B active (incl. 7.8M self-conditioning), 740M embedder
    [TR parameter table; CA §스펙 정리]."""
    c = C2
    d, dh = c.d_model, c.head_dim
    attn = d * c.qkv_rows + c.n_q_heads * dh * d
    expert = 3 * d * c.expert_hidden
    shared = 3 * d * c.shared_hidden
    router = d * c.n_experts
    emb = c.vocab * d
    total = c.n_layers * (attn + c.n_experts * expert + shared + router) + emb
    active = c.n_layers * (attn + c.top_k * expert + shared + router) + emb
    assert abs(emb / 1e6 - 740) / 740 < 0.01
    assert abs(total / 1e9 - 25.2) / 25.2 < 0.01
    assert abs((active + 7.8e6) / 1e9 - 3.85) / 3.85 < 0.03


def test_tiny_fp32_workload_end_to_end_oracle():
    """The tiny fp32 workload through the oracle: causal prefill of 64 random tokens, uniform
    canvas at t = 1, four linear-schedule Euler steps; deterministic, tokens in range."""
    from synth import gen
    from synth.configs import C0 as cfg
    from oracle import step as S
    from tests.helpers import oracle_weights, oracle_kv
    W = oracle_weights(gen.make_weights(cfg), cfg)
    kv0 = oracle_kv(gen.empty_kv(cfg))
    toks = gen.prefix_tokens(cfg).numpy()
    kv, plen = M.prefill(cfg, W, kv0, [0] * cfg.batch, toks)
    assert plen == [64]
    fwd = lambda cv: M.denoise_forward(cfg, W, kv, plen, canvas=cv)[0]
    cv1, lk1, n1 = S.canvas_run(cfg, W, kv, plen, fwd)
    cv2, lk2, n2 = S.canvas_run(cfg, W, kv, plen, fwd)
    assert np.array_equal(cv1, cv2) and np.array_equal(n1, [4])
    assert cv1.min() >= 0 and cv1.max() < cfg.vocab
    # random init: nothing is confident enough to lock at theta = 0.9
    assert not lk1.any()
