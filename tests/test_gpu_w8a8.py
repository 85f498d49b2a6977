"""W8A8 experts on the GPU against the oracle (fp8 e4m3 weights and activations, fp8 MFMA).

  * the activation coding alone: per-row float32 scale and e4m3 code of every element, bit-exact
    with the oracle's quantiser (which is pinned to torch's e4m3 cast, ties and saturation) on bf16
    rows of many magnitudes, a zero row, rows whose quotients fall exactly on midpoints between
    codes (ties to even), and ragged row counts
  * teacher-forced layer parity with W8A8 experts: a tiny model (64-row expert tiles), one canvas
    at the Gemma-like widths (64-row tiles, about 16 rows per expert) and eight canvases over
    4096-token prefixes with Zipf routing (the full 2048-row shape: 128 x 256 tiles), local and
    global layers.  The codes are integer decisions taken from floats, and at these widths they
    amplify: a 1e-6 relative change of a layer's input moves the oracle's own W8A8 output by up to
    0.1 (a row's scale follows its largest element, so one bf16 step there recodes much of the
    row).  So the decisions are checked where they are taken and then handed on, like the expert
    choice on a near-tie:
      - the GPU's codes and scales equal the oracle quantiser applied to the GPU's own bf16 rows,
        bit for bit (the FFN-normalised rows, the routed SwiGLU products in grouped order, the
        shared expert's);
      - the GPU's normalised rows match the oracle's within one bf16 step plus 5e-3;
      - the oracle takes the GPU's codes as its quantiser's output (forced_q) and its SwiGLU
        products, computed from those codes, match the GPU's within one bf16 step;
      - the fp32 residual after the layer matches the forced oracle within 2e-2, as for every bf16
        layer.  The free-running difference is reported.
  * W8A8 is a different function from W8A16: the same layer with weight-only fp8 differs
"""
import numpy as np
import pytest
import torch

from discrete_text_diffusion_amd import dg
from oracle import model as M
from oracle.numerics import e4m3_decode_table, quant_rows_e4m3, rounder
from synth import configs, gen
from tests.gpu_util import build, check_routing, log
from tests.helpers import np64, oracle_layer

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
_TAB = e4m3_decode_table()


def _bf16_rows(rng, rows, K):
    mags = 10.0 ** rng.uniform(-6, 6, size=(rows, 1))
    x = rng.standard_normal((rows, K)) * mags
    x[rows // 3] = 0.0                                                 # a zero row
    # a row whose max is 448 exactly (scale 1): midpoints between codes land on ties
    t = rows // 2
    x[t] = rng.choice([0.5, -1.0, 3.0, 100.0], size=K)
    x[t, :6] = [448.0, 1.0 + 1 / 16, 1.0 + 3 / 16, -(1.0 + 3 / 16), 432.0, 3 * 2.0 ** -10]
    # the same pattern scaled by 2^-20 (the scale then is 2^-20 exactly)
    x[t + 1] = x[t] * 2.0 ** -20
    xb = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)
    return xb


@pytest.mark.parametrize("rows,K", [(1, 8), (37, 704), (256, 2816), (2051, 2112)])
def test_activation_codes_bit_exact(rows, K):
    rng = np.random.default_rng(rows * 31 + K)
    n = max(rows, 4)
    xb = _bf16_rows(rng, n, K)[:rows].contiguous()
    log(f"[w8a8 codes] rows {rows} K {K}")
    xd = xb.to(DEV)
    q = torch.full((rows, K), 0x7F, dtype=torch.uint8, device=DEV)        # NaN codes: every one must be written
    s = torch.full((rows,), float("nan"), dtype=torch.float32, device=DEV)
    dg.dg_test_quant_rows(xd, rows, K, q, s)
    torch.cuda.synchronize()
    x64 = xb.float().numpy().astype(np.float64)
    deq, os_ = quant_rows_e4m3(x64)
    gs = s.cpu().numpy().astype(np.float64)
    assert np.array_equal(gs, os_)
    codes = q.cpu().numpy()
    assert not np.any((codes & 0x7F) == 0x7F), "NaN code written"
    got = _TAB[codes] * gs[:, None]
    assert np.array_equal(got, deq)
    for t in (n // 2, n // 2 + 1):
        if t < rows:       # the tie rows: codes of 448, 1 + 1/16, 1 + 3/16, -(1 + 3/16), 432, 3 * 2^-10
            assert list(_TAB[codes[t, :6]]) == [448.0, 1.0, 1.25, -1.25, 448.0, 2 * 2.0 ** -9]


def _deq(codes, scales):
    return _TAB[codes] * scales.astype(np.float64)[:, None]


def _w8a8_layer_parity(cfg, layer, tol=2e-2):
    log(f"W8A8 layer parity: {cfg.name} layer {layer} ({'global' if cfg.is_global(layer) else 'local'}), "
        f"rows={cfg.rows} prefix={cfg.prefix}")
    model, W, kv = build(cfg)
    B, L = cfg.batch, cfg.canvas
    R, E, k, d, f, fs = B * L, cfg.n_experts, cfg.top_k, cfg.d_model, cfg.expert_hidden, cfg.shared_hidden
    ws = model.workspace(B, L, cfg.prefix)
    rin = gen.resid_input(cfg, DEV)
    rout = torch.empty_like(rin)
    model.denoise_step(None, L, ws, resid_out=rout, resid_in=rin, layer_begin=layer, layer_end=layer + 1)
    r_logits = torch.empty(R, E, dtype=torch.float32, device=DEV)
    r_idx = torch.empty(R, k, dtype=torch.int32, device=DEV)
    dg.dg_test_read_routing(model.ctx, ws, R, r_logits, r_idx, None)
    bf = dict(dtype=torch.bfloat16, device=DEV)
    u8 = dict(dtype=torch.uint8, device=DEV)
    f32 = dict(dtype=torch.float32, device=DEV)
    t = {"xhat": torch.empty(R, d, **bf), "xq": torch.empty(R, d, **u8), "xs": torch.empty(R, **f32),
         "a_grp": torch.empty(R * k, f, **bf), "aq": torch.empty(R * k, f, **u8), "as_": torch.empty(R * k, **f32),
         "sh_a": torch.empty(R, fs, **bf), "shq": torch.empty(R, fs, **u8), "shs": torch.empty(R, **f32)}
    dg.dg_test_read_expert_inputs(model.ctx, ws, B, L, **t)
    torch.cuda.synchronize()
    assert dg.dg_query_status(model.ctx, ws) == dg.DG_OK
    g = {n: (v.float() if v.dtype == torch.bfloat16 else v).cpu().numpy() for n, v in t.items()}
    # 1. the GPU's code decisions equal the quantiser on its own rows, bit for bit
    for rows, codes, sc in (("xhat", "xq", "xs"), ("a_grp", "aq", "as_"), ("sh_a", "shq", "shs")):
        deq, s_ = quant_rows_e4m3(g[rows].astype(np.float64))
        assert np.array_equal(g[sc].astype(np.float64), s_), f"{sc}: scales differ"
        assert np.array_equal(_deq(g[codes], g[sc]), deq), f"{codes}: codes differ"
    # 2. routing as for every layer; the oracle then takes the GPU's selection, slot order included
    lw = oracle_layer(W["layers"][layer], cfg)
    K, V = np64(kv[layer][0]), np64(kv[layer][1].transpose(-1, -2))
    h0 = rin.cpu().numpy().astype(np.float64)
    rnd = rounder(cfg.act_dtype)
    hfree, info = M.denoise_layer(cfg, layer, h0, lw, K, V, [cfg.prefix] * B, rnd)
    gidx = r_idx.cpu().numpy()
    _, n_rer, lg_err = check_routing(cfg, gidx, r_logits.cpu().numpy(), info)
    counts, offsets, perm = M.route_tables(gidx, E)
    xdeq, adeq, shdeq = _deq(g["xq"], g["xs"]), _deq(g["aq"], g["as_"]), _deq(g["shq"], g["shs"])
    seen = {}

    def forced_q(e, x):
        # first call: the expert's input rows; second: its SwiGLU products (recorded for step 3)
        n = seen.get(e, 0)
        seen[e] = n + 1
        if e == "shared":
            if n == 0:
                return xdeq
            seen["A_shared"] = x
            return shdeq
        o, c = int(offsets[e]), int(counts[e])
        if n == 0:
            return xdeq[perm[o:o + c] // k]
        seen[("A", e)] = x
        return adeq[o:o + c]
    h1, info1 = M.denoise_layer(cfg, layer, h0, lw, K, V, [cfg.prefix] * B, rnd, forced_idx=gidx, forced_q=forced_q)
    # 3. normalised rows, and the SwiGLU products from the GPU's input codes
    # normalised rows: one bf16 step at |x| (a rounding flip) plus the attention block's residual
    # difference, a few 1e-3 at most
    x_step = np.ldexp(1.0, np.frexp(np.maximum(np.abs(info1["a2"]), 1e-30))[1] - 8)
    e_x = float((np.abs(g["xhat"] - info1["a2"]) - x_step).max())
    A_or = np.zeros((R * k, f))
    for e in range(E):
        if counts[e]:
            A_or[offsets[e]:offsets[e] + counts[e]] = seen[("A", e)]
    # one bf16 step at |A|, plus a floor for products that cancel toward zero: there the float32
    # sums of the gate and up products (and the exponential in silu) carry an absolute error that
    # is small beside the row's largest product, not beside the small product itself
    def excess(gpu, orc):
        ulp = np.ldexp(1.0, np.frexp(np.maximum(np.abs(orc), 1e-30))[1] - 8)
        floor = 1e-4 * np.abs(orc).max(axis=1, keepdims=True)
        return np.abs(gpu - orc) - ulp - floor, int((gpu != orc).sum())
    x_a, n_a = excess(g["a_grp"], A_or)
    x_sh, n_sh = excess(g["sh_a"], seen["A_shared"])
    log(f"  SwiGLU products unequal: routed {n_a} of {A_or.size}, shared {n_sh} of {x_sh.size}; largest excess over "
        f"the bound {max(x_a.max(), x_sh.max()):.2e}")
    err = float(np.abs(rout.cpu().numpy() - h1).max())
    free = float(np.abs(rout.cpu().numpy() - hfree).max())
    log(f"  normalised rows: largest difference beyond one bf16 step {e_x:.2e}; router logits err {lg_err:.2e}, reroutes {n_rer}")
    log(f"  max |resid - oracle| with the GPU's codes {err:.3e} (tol {tol}); free-running {free:.3e} (reported)")
    assert x_a.max() <= 0 and x_sh.max() <= 0, "SwiGLU products beyond one bf16 step"
    assert e_x <= 5e-3
    assert err <= tol


def _w8a8(cfg, **kw):
    return cfg.replace(expert_dtype="fp8", act_quant="fp8", **kw)


def test_tiny_w8a8_layer_parity():
    cfg = _w8a8(configs.C0, act_dtype="bf16", kv_source="random", resid_input=True, name="tiny-w8a8")
    _w8a8_layer_parity(cfg, 0)
    _w8a8_layer_parity(cfg, 1)


def test_single_canvas_w8a8_layer_parity():
    """One global layer at the Gemma-like widths over a 2048-token prefix: 256 rows, about 16 per
    expert, on 64-row W8A8 tiles."""
    _w8a8_layer_parity(_w8a8(configs.C1, name="layer-w8a8-p2048"), 0)


def test_batch8_w8a8_layers_parity_full_shape():
    """Eight canvases over 4096-token prefixes with a Zipf(1.1) router prior, W8A8 experts: one local
    and one global layer at the full 2048-row shape (128 x 256 tiles)."""
    cfg = _w8a8(configs.C4, n_layers=6, resid_input=True, name="c4-w8a8")
    _w8a8_layer_parity(cfg, 0)
    _w8a8_layer_parity(cfg, 5)


def test_w8a8_differs_from_weight_only():
    cfg16 = configs.C4.replace(n_layers=1, batch=2, prefix=1024, resid_input=True, window=0, global_every=0)
    outs = []
    for c in (cfg16, cfg16.replace(act_quant="fp8")):
        model, W, kv = build(c)
        ws = model.workspace(c.batch, c.canvas, c.prefix)
        rin = gen.resid_input(c, DEV)
        r = torch.empty_like(rin)
        model.denoise_step(None, c.canvas, ws, resid_out=r, resid_in=rin, layer_begin=0, layer_end=1)
        torch.cuda.synchronize()
        assert dg.dg_query_status(model.ctx, ws) == dg.DG_OK
        outs.append((r - rin).cpu())
        del model, W, kv, ws
    d = float((outs[0] - outs[1]).abs().max())
    ref = float(outs[0].abs().max())
    log(f"  layer update: max |W8A16 - W8A8| {d:.3e} of max |update| {ref:.3e}")
    assert 0 < d < 0.2 * ref
