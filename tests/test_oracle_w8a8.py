"""Pins of the W8A8 activation quantisation in the oracle (CPU).

The experts' inputs are quantised per row to OCP e4m3 (reading: scale max|x| / 448, nearest code,
ties to even, saturating) while the weights keep their per-output-row scales.

  * round_e4m3 equals torch's float8_e4m3fn cast on in-range values, ties included; every e4m3
    value round-trips; hand-checked ties go to the even code; values beyond 448 saturate
  * quant_rows_e4m3: the largest element of a row codes to exactly 448 (so it dequantises to
    itself); a zero row stays zero; every element is within half a code step of its input; a row
    scaled by a power of two keeps its codes
  * the MoE with W8A8 equals the MoE without it when every row's inputs are already exactly
    representable (codes times the row's own scale), and differs otherwise
"""
import numpy as np
import torch

from oracle import model as M
from oracle.numerics import E4M3_MAX, e4m3_decode_table, identity, quant_rows_e4m3, round_e4m3
from synth.configs import C0


def test_round_e4m3_matches_torch_cast():
    rng = np.random.default_rng(40)
    x = np.concatenate([rng.standard_normal(20000) * 3, rng.standard_normal(20000) * 100,
                        rng.standard_normal(5000) * 1e-3]).astype(np.float32)
    x = np.clip(x, -E4M3_MAX, E4M3_MAX)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    assert np.array_equal(round_e4m3(x.astype(np.float64)), want)


def test_codes_round_trip_ties_and_saturation():
    tab = e4m3_decode_table()
    vals = tab[np.isfinite(tab)]
    assert np.array_equal(round_e4m3(vals), vals)
    # midpoints: 1 + 1/16 lies between 1 and 1.125 (mantissas 0 and 1) -> 1; 1 + 3/16 between 1.125
    # and 1.25 (mantissas 1 and 2) -> 1.25
    assert round_e4m3(1.0 + 1 / 16) == 1.0 and round_e4m3(1.0 + 3 / 16) == 1.25
    assert round_e4m3(-(1.0 + 3 / 16)) == -1.25
    assert round_e4m3(500.0) == 448.0 and round_e4m3(-1e6) == -448.0
    # the subnormal spacing 2^-9 below 2^-6
    assert round_e4m3(3 * 2.0 ** -10) == 2 * 2.0 ** -9      # tie between 1 and 2 steps -> even (2)


def test_row_quantisation_properties():
    rng = np.random.default_rng(41)
    x = rng.standard_normal((6, 64)) * np.array([1e-3, 0.1, 1, 10, 300, 5])[:, None]
    x[2] = 0.0
    deq, s = quant_rows_e4m3(x)
    assert np.all(deq[2] == 0) and s[2] == 1.0
    for r in (0, 1, 3, 4, 5):
        j = np.argmax(np.abs(x[r]))
        xr = np.float32(x[r, j])
        assert abs(deq[r, j]) == abs(float(xr)) or np.isclose(deq[r, j], float(xr), rtol=2 ** -23)
        # within half a code step: the e4m3 spacing at |x| / s is at most 2^-3 relative (2^-9 absolute
        # below 2^-6), so |x - deq| <= s * max(|x| / s * 2^-4, 2^-10)
        bound = s[r] * np.maximum(np.abs(x[r]) / s[r] * 2.0 ** -4, 2.0 ** -10) * (1 + 1e-6)
        assert np.all(np.abs(x[r] - deq[r]) <= bound)
    deq2, s2 = quant_rows_e4m3(x * 8.0)
    assert np.allclose(deq2, deq * 8.0, rtol=0, atol=0) and np.allclose(s2[[0, 1, 3, 4, 5]], s[[0, 1, 3, 4, 5]] * 8.0)


def _tiny():
    return C0.replace(d_model=32, n_experts=4, top_k=2, expert_hidden=16, shared_hidden=16, expert_dtype="fp8")


def _layer(cfg, rng):
    d, E, f, fs = cfg.d_model, cfg.n_experts, cfg.expert_hidden, cfg.shared_hidden
    n = lambda *s: rng.standard_normal(s) * 0.3
    return {"w_router": n(E, d), "router_bias": None, "w_gate": n(E, f, d), "w_up": n(E, f, d), "w_down": n(E, d, f),
            "sh_gate": n(fs, d), "sh_up": n(fs, d), "sh_down": n(d, fs)}


def test_w8a8_moe_is_exact_on_representable_inputs_and_differs_otherwise():
    rng = np.random.default_rng(42)
    base = _tiny()
    q8 = base.replace(act_quant="fp8")
    lw = _layer(base, rng)
    # rows made of e4m3 codes times a per-row scale with one element at 448: quantisation is the
    # identity on them (the SwiGLU products are quantised too, so compare the gate/up input alone)
    tab = e4m3_decode_table()
    vals = tab[np.isfinite(tab) & (np.abs(tab) <= 448)]
    x = rng.choice(vals, size=(5, base.d_model))
    x[:, 0] = 448.0
    x = x * (2.0 ** rng.integers(-12, -6, size=(5, 1)))
    deq, _ = quant_rows_e4m3(x)
    assert np.array_equal(deq, x)
    # the whole MoE: on generic inputs W8A8 differs from the unquantised experts, but stays close
    xg = rng.standard_normal((5, base.d_model))
    out8, _ = M.moe(q8, xg, lw, identity)
    out, _ = M.moe(base, xg, lw, identity)
    assert not np.allclose(out8, out, rtol=0, atol=1e-12)
    assert np.allclose(out8, out, rtol=0.1, atol=0.1 * np.abs(out).max())
    # and with act_q applied by hand to both GEMM inputs of every expert, it is the same function
    aq = M.act_quantiser(q8)
    want = M.swiglu(xg, lw["sh_gate"], lw["sh_up"], lw["sh_down"], identity, aq)
    xs = quant_rows_e4m3(xg)[0]
    g = xs @ lw["sh_gate"].T
    A = (g / (1 + np.exp(-g))) * (xs @ lw["sh_up"].T)
    assert np.allclose(want, quant_rows_e4m3(A)[0] @ lw["sh_down"].T, rtol=1e-12, atol=1e-12)


def test_forced_quantiser_hook():
    """forced_q hands each expert's quantiser calls to the caller: input rows first, then the SwiGLU
    product, in token-then-slot order; handing back the quantiser's own output reproduces the layer,
    and handing back anything else changes it."""
    rng = np.random.default_rng(43)
    cfg = _tiny().replace(act_quant="fp8")
    lw = _layer(cfg, rng)
    x = rng.standard_normal((7, cfg.d_model))
    want, info = M.moe(cfg, x, lw, identity)
    calls = []

    def same(e, v):
        calls.append((e, v.shape))
        return quant_rows_e4m3(v)[0]
    got, _ = M.moe(cfg, x, lw, identity, forced_q=same)
    assert np.array_equal(got, want)
    idx = info["idx"]
    routed = [c for c in calls if c[0] != "shared"]
    assert [c[0] for c in routed] == [e for e in np.unique(idx) for _ in (0, 1)]
    for j in range(0, len(routed), 2):
        e = routed[j][0]
        n = int((idx == e).sum())
        assert routed[j][1] == (n, cfg.d_model) and routed[j + 1][1] == (n, cfg.expert_hidden)
    assert [c for c in calls if c[0] == "shared"] == [("shared", (7, cfg.d_model)), ("shared", (7, cfg.shared_hidden))]
    other, _ = M.moe(cfg, x, lw, identity, forced_q=lambda e, v: v)
    assert not np.allclose(other, want, rtol=0, atol=1e-12)
