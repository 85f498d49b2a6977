"""The denoiser forward pass, plainly (test infrastructure only).

What the pages fix: the decoder is a transformer whose canvas attention is bidirectional (no
causal mask) and which also attends to the prefix KV cache built by a causal encoder that shares
its weights [TR §아키텍처와 블록 자기회귀 생성, block-AR steps]; 30 layers, sliding window 1024,
MoE with 8 of 128 experts active plus one always-on shared expert, tied 262k embedding
[CA §스펙 정리; TR parameter table].  Everything the pages leave open (normalisation, RoPE
variant, window semantics for a bidirectional canvas, gate normalisation, where values are
stored in bf16) follows the readings listed at the top of each function.

All arithmetic is float64; `rnd` applies the storage rounding (bf16 in bf16 mode, none in fp32
mode) at exactly the points where the activations are stored:
    x_hat after each RMSNorm, q/k/v after RoPE, the attention output o, the SwiGLU product A
    and the final normed hidden state H.
Residual stream, router logits (rounded to float32), gates and expert outputs stay wide.
"""
from __future__ import annotations

import numpy as np

from .numerics import dequant_rows, mxfp4_dequant, quant_rows_e4m3, rounder


# ---------------------------------------------------------------- weights in float64 -----------

def layer_arrays(L: dict, expert_dtype: str) -> dict:
    """Storage arrays of one layer (float64 values, or uint8 codes + scales for fp8 / mxfp4) ->
    float64 weight matrices.  fp8 weights are q * s with the per-output-row scale; mxfp4 weights
    are e2m1(q) * 2^(s - 127) with one scale per 32 consecutive input elements."""
    out = {}
    for k in ("attn_norm", "ffn_norm", "w_qkv", "w_o", "w_router"):
        out[k] = np.asarray(L[k], dtype=np.float64)
    out["router_bias"] = None if L.get("router_bias") is None else np.asarray(L["router_bias"], np.float64)
    for k, s in (("w_gate", "s_gate"), ("w_up", "s_up"), ("w_down", "s_down"),
                 ("sh_gate", "sh_s_gate"), ("sh_up", "sh_s_up"), ("sh_down", "sh_s_down")):
        if expert_dtype == "fp8":
            out[k] = dequant_rows(L[k], L[s])
        elif expert_dtype == "mxfp4":
            out[k] = mxfp4_dequant(L[k], L[s])
        else:
            out[k] = np.asarray(L[k], dtype=np.float64)
    return out


# ---------------------------------------------------------------- building blocks --------------

def rmsnorm(x, g, eps):
    """Reading: y = x / sqrt(mean(x^2) + eps) * g over the model dimension."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * g


def rope(x, pos, theta):
    """Rotary embedding, rotate-half pairing: element j pairs with j + dh/2 and the pair at
    position p turns by p * theta^(-2j/dh).  x: [n][H][dh], pos: [n]."""
    x = np.asarray(x, dtype=np.float64)
    dh = x.shape[-1]
    half = dh // 2
    inv = theta ** (-2.0 * np.arange(half, dtype=np.float64) / dh)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]          # [n][half]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def attend(q, K, V, visible=None):
    """softmax(q K^T / sqrt(dh)) V for one head.  q: [n][dh], K, V: [m][dh]; visible: [n][m]
    bool or None (all keys visible).  A row with no visible key returns zeros."""
    dh = q.shape[-1]
    s = (q @ K.T) / np.sqrt(dh)
    if visible is not None:
        s = np.where(visible, s, -np.inf)
    mx = np.max(s, axis=-1, keepdims=True)
    mx = np.where(np.isfinite(mx), mx, 0.0)
    p = np.exp(s - mx)
    den = p.sum(axis=-1, keepdims=True)
    den = np.where(den > 0, den, 1.0)
    return (p / den) @ V


def is_global(cfg, layer):
    return cfg.window <= 0 or cfg.global_every <= 0 or (layer + 1) % cfg.global_every == 0


def prefix_slots(cfg, layer, prefix_len):
    """Valid cache slots for a canvas whose prefix has `prefix_len` tokens.

    Reading (window semantics with a bidirectional canvas): on local layers every canvas query
    sees the last `window` prefix positions [max(0, P - W), P) plus the whole canvas; global
    layers see the whole prefix.  A local layer's cache is a ring of W slots, position p in slot
    p mod W, so the visible set is the first min(P, W) slots; key order does not matter."""
    if is_global(cfg, layer):
        return prefix_len
    return min(prefix_len, cfg.window)


def slot_positions(cfg, layer, pos0, cap):
    """Position held by each slot of a cache that has received positions [0, pos0)."""
    s = np.arange(cap)
    if is_global(cfg, layer):
        return np.where(s < pos0, s, -1)
    W = cfg.window
    lo = max(0, pos0 - W)
    # the p in [lo, pos0) with p = s (mod W)
    p = lo + ((s - lo) % W)
    return np.where(p < pos0, p, -1)


def canvas_attention(cfg, layer, q, kc, vc, Kp, Vp, prefix_len):
    """Bidirectional canvas attention for one canvas.

    q: [L][Hq][dh]; kc, vc: [Hkv][L][dh] (this canvas's keys/values); Kp, Vp: [Hkv][cap][dh]
    prefix cache.  Query head j reads KV head j // (Hq / Hkv).  No mask inside the canvas."""
    L, Hq, dh = q.shape
    Hkv = kc.shape[0]
    n = prefix_slots(cfg, layer, prefix_len)
    o = np.zeros_like(q)
    for j in range(Hq):
        g = j // (Hq // Hkv)
        K = np.concatenate([Kp[g, :n], kc[g]], axis=0)
        V = np.concatenate([Vp[g, :n], vc[g]], axis=0)
        o[:, j, :] = attend(q[:, j, :], K, V)
    return o


def causal_attention(cfg, layer, q, kn, vn, Kp, Vp, pos0):
    """Causal attention of n new tokens at positions pos0.. over the cache and themselves.

    Key at position p is visible to the query at position t iff p <= t and, on local layers,
    t - p < window.  kn, vn: [Hkv][n][dh]; Kp, Vp: [Hkv][cap][dh]."""
    n, Hq, dh = q.shape
    Hkv = kn.shape[0]
    cap = Kp.shape[1]
    spos = slot_positions(cfg, layer, pos0, cap)
    valid = spos >= 0
    kpos = np.concatenate([spos[valid], pos0 + np.arange(n)])
    qpos = pos0 + np.arange(n)
    vis = kpos[None, :] <= qpos[:, None]
    if not is_global(cfg, layer):
        vis &= (qpos[:, None] - kpos[None, :]) < cfg.window
    o = np.zeros_like(q)
    for j in range(Hq):
        g = j // (Hq // Hkv)
        K = np.concatenate([Kp[g][valid], kn[g]], axis=0)
        V = np.concatenate([Vp[g][valid], vn[g]], axis=0)
        o[:, j, :] = attend(q[:, j, :], K, V, vis)
    return o


def router_topk(r32, k):
    """Top-k experts per row by (logit descending, expert id ascending); gates are the softmax
    over the k selected logits.  r32: float32-valued router logits [T][E].

    Reading: ties go to the lower expert id; the gate is normalised over the selected experts
    (all conventions agree when k = E)."""
    r = np.asarray(r32, dtype=np.float64)
    T, E = r.shape
    # stable sort of -r keeps equal logits in ascending expert order
    order = np.argsort(-r, axis=1, kind="stable")
    idx = order[:, :k]
    sel = np.take_along_axis(r, idx, axis=1)
    w = np.exp(sel - sel.max(axis=1, keepdims=True))
    return idx.astype(np.int64), w / w.sum(axis=1, keepdims=True)


def route_tables(idx, n_experts):
    """Per-expert row lists in (token, slot) order: counts[E], offsets[E] (exclusive scan) and
    perm[T*k] holding the flat assignment id t*k + s at each grouped position."""
    flat = np.asarray(idx).reshape(-1)
    counts = np.bincount(flat, minlength=n_experts)
    offsets = np.concatenate([[0], np.cumsum(counts)[:-1]])
    perm = np.argsort(flat, kind="stable")            # ascending expert, then assignment order
    return counts.astype(np.int64), offsets.astype(np.int64), perm.astype(np.int64)


def silu(x):
    return x / (1.0 + np.exp(-x))


def swiglu(x, Wg, Wu, Wd, rnd, act_q=None):
    """SwiGLU FFN: A = silu(x Wg^T) * (x Wu^T), stored (rnd); y = A Wd^T, stored (rnd): an expert's
    output rows are activations like the others (reading 13).  With act_q (W8A8 experts) both GEMM
    inputs, x and A, pass through it (per-row e4m3 quantisation) first."""
    if act_q is not None:
        x = act_q(x)
    A = rnd(silu(x @ Wg.T) * (x @ Wu.T))
    if act_q is not None:
        A = act_q(A)
    return rnd(A @ Wd.T)


def act_quantiser(cfg):
    """The expert GEMMs' activation quantisation: per-row dynamic e4m3 (W8A8 experts), or None.

    Reading (the pages measure FP8 builds but fix no scheme): each row of the expert input (the
    normalised rows, and the SwiGLU product before the down matrix) is scaled by its own
    max|x| / 448 and rounded to e4m3; the weights keep their per-output-row scales, so a product is
    (codes . codes) * s_row * s_col."""
    if getattr(cfg, "act_quant", "") != "fp8":
        return None
    return lambda x: quant_rows_e4m3(x)[0]


def moe(cfg, a2, lw, rnd, forced_idx=None, forced_q=None):
    """Routed experts plus the always-on shared expert.

    out[t] = sum over slots s in order of gate[t,s] * FFN_{idx[t,s]}(a2[t]) + FFN_shared(a2[t]).
    The shared expert enters with weight 1.  `forced_idx` replaces the top-k choice (used only
    when comparing against another implementation that saw a near-tie).  `forced_q(e, x)`, for
    W8A8 experts only, replaces the activation quantiser of expert e ("shared" for the shared
    expert; its rows in ascending token-then-slot order, first with the expert's input, then with
    its SwiGLU product): it lets a comparison hand in another implementation's code decisions,
    which tiny input differences can move, the way forced_idx hands in its expert choice."""
    r = a2 @ lw["w_router"].T
    if lw["router_bias"] is not None:
        r = r + lw["router_bias"]
    r32 = r.astype(np.float32)
    idx, gates = router_topk(r32, cfg.top_k)
    if forced_idx is not None:
        idx = np.asarray(forced_idx, dtype=np.int64)
        sel = np.take_along_axis(r32.astype(np.float64), idx, axis=1)
        w = np.exp(sel - sel.max(axis=1, keepdims=True))
        gates = w / w.sum(axis=1, keepdims=True)
    T = a2.shape[0]
    aq = act_quantiser(cfg)
    if forced_q is not None:
        assert aq is not None, "forced_q needs W8A8 experts"
        q_of = lambda e: (lambda x: forced_q(e, x))
    else:
        q_of = lambda e: aq
    y = np.zeros((T, cfg.top_k, a2.shape[1]))
    for e in np.unique(idx):
        rows, slots = np.nonzero(idx == e)
        y[rows, slots] = swiglu(a2[rows], lw["w_gate"][e], lw["w_up"][e], lw["w_down"][e], rnd, q_of(int(e)))
    out = np.zeros_like(a2)
    for s in range(cfg.top_k):
        out = out + gates[:, s:s + 1] * y[:, s]
    out = out + swiglu(a2, lw["sh_gate"], lw["sh_up"], lw["sh_down"], rnd, q_of("shared"))
    return out, {"r32": r32, "idx": idx, "gates": gates}


# ---------------------------------------------------------------- one layer --------------------

def qkv(cfg, x_hat, lw, pos, rnd):
    """q, k, v of rows x_hat at positions pos; RoPE on q and k; stored (rnd)."""
    Hq, Hkv, dh = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    y = x_hat @ lw["w_qkv"].T
    n = y.shape[0]
    q = y[:, :Hq * dh].reshape(n, Hq, dh)
    k = y[:, Hq * dh:(Hq + Hkv) * dh].reshape(n, Hkv, dh)
    v = y[:, (Hq + Hkv) * dh:].reshape(n, Hkv, dh)
    return rnd(rope(q, pos, cfg.rope_theta)), rnd(rope(k, pos, cfg.rope_theta)), rnd(v)


def denoise_layer(cfg, layer, h, lw, K, V, prefix_len, rnd, forced_idx=None, forced_q=None):
    """One pre-norm decoder layer over all canvases.  h: [B*L][d] residual (float64).
    K, V: this layer's caches [B][Hkv][cap][dh].  Returns (h_new, info); forced_idx and
    forced_q as in moe."""
    B, L = len(prefix_len), h.shape[0] // len(prefix_len)
    Hq, dh = cfg.n_q_heads, cfg.head_dim
    x = rnd(rmsnorm(h, lw["attn_norm"], cfg.norm_eps))
    o = np.zeros((B * L, Hq * dh))
    for b in range(B):
        rows = slice(b * L, (b + 1) * L)
        pos = prefix_len[b] + np.arange(L)
        q, k, v = qkv(cfg, x[rows], lw, pos, rnd)
        ob = canvas_attention(cfg, layer, q, k.transpose(1, 0, 2), v.transpose(1, 0, 2),
                              K[b], V[b], prefix_len[b])
        o[rows] = ob.reshape(L, Hq * dh)
    o = rnd(o)
    h = h + o @ lw["w_o"].T
    a2 = rnd(rmsnorm(h, lw["ffn_norm"], cfg.norm_eps))
    f, info = moe(cfg, a2, lw, rnd, forced_idx, forced_q)
    info["o"] = o
    info["a2"] = a2
    return h + f, info


def denoise_forward(cfg, W, kv, prefix_len, canvas=None, resid_in=None, n_layers=None, sc=None):
    """Decoder pass over the canvases.

    W: {"embed": [V][d] | None, "final_norm": [d], "layers": [layer_arrays ...]};
    kv: per layer (K, V) float64 [B][Hkv][cap][dh]; canvas: int [B][L] or resid_in [B*L][d];
    sc: the self-conditioning signal s_t [B*L][d], added to the embedded canvas (None: s = 0).
    Returns (H, resid): H = stored(RMSNorm(resid) * g_final), resid = pre-norm residual.
    Reading: the embedding is a plain row lookup of the tied matrix (no sqrt(d) scale)."""
    rnd = rounder(cfg.act_dtype)
    if resid_in is not None:
        h = np.asarray(resid_in, dtype=np.float64).copy()
    else:
        h = W["embed"][np.asarray(canvas).reshape(-1)].astype(np.float64)
        if sc is not None:
            h = h + np.asarray(sc, np.float64)
    nl = cfg.n_layers if n_layers is None else n_layers
    for l in range(nl):
        h, _ = denoise_layer(cfg, l, h, W["layers"][l], kv[l][0], kv[l][1], prefix_len, rnd)
    H = rnd(rmsnorm(h, W["final_norm"], cfg.norm_eps))
    return H, h


def write_cache(cfg, layer, Kb, Vb, pos, kn, vn):
    """Store new keys / values kn, vn [Hkv][n][dh] at positions pos in one canvas's caches
    Kb, Vb [Hkv][cap][dh]: slot p on global layers; on local layers a ring of `window` slots
    (slot p mod window) that keeps only the last `window` positions."""
    if is_global(cfg, layer):
        Kb[:, pos] = kn
        Vb[:, pos] = vn
    else:
        keep = pos >= pos[-1] + 1 - cfg.window
        Kb[:, pos[keep] % cfg.window] = kn[:, keep]
        Vb[:, pos[keep] % cfg.window] = vn[:, keep]


def prefill(cfg, W, kv, prefix_len, tokens):
    """Causal encoder pass over tokens [B][n] at positions prefix_len[b].. that appends their
    post-RoPE keys and values to the caches [TR §아키텍처와 블록 자기회귀 생성: context encoding
    and append-after-encode].  Same weights as the decoder.  Returns new caches (copies) and
    the new prefix lengths.  Slot of position p: p on global layers, p mod window on local."""
    rnd = rounder(cfg.act_dtype)
    tokens = np.asarray(tokens)
    B, n = tokens.shape
    Hq, Hkv, dh = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    kv = [(K.copy(), V.copy()) for K, V in kv]
    h = W["embed"][tokens.reshape(-1)].astype(np.float64)
    for l in range(cfg.n_layers):
        lw = W["layers"][l]
        K, V = kv[l]
        x = rnd(rmsnorm(h, lw["attn_norm"], cfg.norm_eps))
        o = np.zeros((B * n, Hq * dh))
        news = []
        for b in range(B):
            rows = slice(b * n, (b + 1) * n)
            pos = prefix_len[b] + np.arange(n)
            q, k, v = qkv(cfg, x[rows], lw, pos, rnd)
            kn, vn = k.transpose(1, 0, 2), v.transpose(1, 0, 2)
            ob = causal_attention(cfg, l, q, kn, vn, K[b], V[b], prefix_len[b])
            o[rows] = ob.reshape(n, Hq * dh)
            news.append((pos, kn, vn))
        for b, (pos, kn, vn) in enumerate(news):
            write_cache(cfg, l, K[b], V[b], pos, kn, vn)
        o = rnd(o)
        h = h + o @ lw["w_o"].T
        a2 = rnd(rmsnorm(h, lw["ffn_norm"], cfg.norm_eps))
        f, _ = moe(cfg, a2, lw, rnd)
        h = h + f
    return kv, [p + n for p in prefix_len]


def mixed_forward(cfg, W, kv, prefix_len, tokens, append, with_resid=False):
    """One pass over a batch whose canvases take different passes [TR §CPU-GPU 동기화 제거: denoising
    steps and KV-cache updates share a batch, told apart by a per-sequence causal flag].

    tokens [B][n]; append[b] true: canvas b takes the causal encoder pass of `prefill` (causal
    attention to its cache and itself; its keys and values written to its caches); false: the
    bidirectional decoder pass of `denoise_forward` (its cache untouched).  Every row runs every
    layer's FFN.  Canvases share nothing but the weights, so each canvas's result is that of its
    own pass run alone.  Returns (H [B*n][d] = stored(RMSNorm(resid) * g_final), new caches); with
    `with_resid` also the residual before the final norm."""
    rnd = rounder(cfg.act_dtype)
    tokens = np.asarray(tokens)
    B, n = tokens.shape
    Hq, dh = cfg.n_q_heads, cfg.head_dim
    kv = [(K.copy(), V.copy()) for K, V in kv]
    h = W["embed"][tokens.reshape(-1)].astype(np.float64)
    for l in range(cfg.n_layers):
        lw = W["layers"][l]
        K, V = kv[l]
        x = rnd(rmsnorm(h, lw["attn_norm"], cfg.norm_eps))
        o = np.zeros((B * n, Hq * dh))
        news = []
        for b in range(B):
            rows = slice(b * n, (b + 1) * n)
            pos = prefix_len[b] + np.arange(n)
            q, k, v = qkv(cfg, x[rows], lw, pos, rnd)
            kn, vn = k.transpose(1, 0, 2), v.transpose(1, 0, 2)
            if append[b]:
                ob = causal_attention(cfg, l, q, kn, vn, K[b], V[b], prefix_len[b])
                news.append((b, pos, kn, vn))
            else:
                ob = canvas_attention(cfg, l, q, kn, vn, K[b], V[b], prefix_len[b])
            o[rows] = ob.reshape(n, Hq * dh)
        for b, pos, kn, vn in news:
            write_cache(cfg, l, K[b], V[b], pos, kn, vn)
        o = rnd(o)
        h = h + o @ lw["w_o"].T
        a2 = rnd(rmsnorm(h, lw["ffn_norm"], cfg.norm_eps))
        f, _ = moe(cfg, a2, lw, rnd)
        h = h + f
    H = rnd(rmsnorm(h, W["final_norm"], cfg.norm_eps))
    return (H, kv, h) if with_resid else (H, kv)
