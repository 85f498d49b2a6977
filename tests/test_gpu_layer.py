"""Parity of the decoder layer on the GPU against the oracle.

Routing is checked bit-exactly from identical fp32 scores.  Layers are teacher-forced: the GPU
runs one layer from a given fp32 residual and the oracle recomputes that layer from the same
residual and the same weights/caches; the fp32 residual after the layer must agree within the
float tolerance (2e-2 max-abs in bf16 mode, 1e-4 in fp32 mode).  The GPU's expert selection must
be exactly the top-k of its own fp32 router scores; it may differ from the oracle's selection only
where the oracle's k-th/(k+1)-th score gap is within the measured score difference, and there the
oracle takes the GPU's selection ("equal scores") before the residuals are compared."""
import numpy as np
import pytest
import torch

from discrete_text_diffusion_amd import dg
from oracle import model as M
from oracle.numerics import rounder
from synth import configs, gen
from tests.gpu_util import build, check_routing, log
from tests.helpers import np64, oracle_layer

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.mark.parametrize("T,E,k,shift", [(256, 128, 8, 0), (2048, 128, 8, 0), (2048, 128, 8, 1), (37, 8, 2, 0),
                                         (37, 8, 2, 3), (64, 256, 16, 0), (4096, 128, 8, 0), (4096, 128, 8, 1)])
@pytest.mark.parametrize("seed", [0, 1])
def test_router_topk_and_grouping_bit_exact(T, E, k, shift, seed):
    """shift > 0 places the caller's pick buffer `shift` int32 past a 16-byte boundary: the routing
    tables then stage the picks element by element instead of in 16-byte loads.  4096 rows take the
    tables' unstaged path (more picks than the LDS stage holds).  Two seeds per shape."""
    g = torch.Generator(device="cpu").manual_seed(T * 7 + E + 1000 * seed)
    s = torch.randn(T, E, generator=g)
    s[::9, 5] = s[::9, 6] = s[::9, 7] = 3.5           # exact ties at the top
    s[1::13] = 0.0                                      # all-equal rows
    s[5::29] = 0.0
    s[5::29, ::3] = -0.0                                # signed zeros compare equal
    s[6::31, 3:] = -float("inf")                        # fewer finite scores than k
    sd = s.to(DEV)
    idx = torch.empty(T * k + shift, dtype=torch.int32, device=DEV)[shift:].view(T, k)
    assert (idx.data_ptr() % 16 != 0) == (shift != 0)
    gates = torch.empty(T, k, dtype=torch.float32, device=DEV)
    counts = torch.empty(E, dtype=torch.int32, device=DEV)
    offs = torch.empty(E, dtype=torch.int32, device=DEV)
    perm = torch.empty(T * k, dtype=torch.int32, device=DEV)
    ws = torch.empty(1 << 22, dtype=torch.uint8, device=DEV)
    dg.dg_test_router_topk(sd, T, E, k, idx, gates, counts, offs, perm, ws)
    torch.cuda.synchronize()
    oidx, ogates = M.router_topk(s.numpy(), k)
    oc, oo, op = M.route_tables(oidx, E)
    assert np.array_equal(idx.cpu().numpy(), oidx)
    assert np.allclose(gates.cpu().numpy(), ogates, rtol=1e-5, atol=1e-7)
    assert np.array_equal(counts.cpu().numpy(), oc)
    assert np.array_equal(offs.cpu().numpy(), oo)
    assert np.array_equal(perm.cpu().numpy(), op)


def _layer_parity(cfg, layer, tol, resid=None, scale_v=None):
    log(f"layer parity: {cfg.name} layer {layer} ({'global' if cfg.is_global(layer) else 'local'}), "
        f"rows={cfg.rows} prefix={cfg.prefix} experts={cfg.expert_dtype}"
        + (f", prefix values x{scale_v:g}, W_o x{1 / scale_v:g}" if scale_v else ""))
    model, W, kv = build(cfg)
    if scale_v:
        # powers of two: exact in bf16 on both sides (the model holds these very tensors)
        kv[layer][1].mul_(scale_v)
        W["layers"][layer]["w_o"].mul_(1.0 / scale_v)
    B, L = cfg.batch, cfg.canvas
    ws = model.workspace(B, L, cfg.prefix)
    rin = gen.resid_input(cfg, DEV) if resid is None else resid
    rout = torch.empty_like(rin)
    model.denoise_step(None, L, ws, resid_out=rout, resid_in=rin, layer_begin=layer, layer_end=layer + 1)
    r_logits = torch.empty(B * L, cfg.n_experts, dtype=torch.float32, device=DEV)
    r_idx = torch.empty(B * L, cfg.top_k, dtype=torch.int32, device=DEV)
    dg.dg_test_read_routing(model.ctx, ws, B * L, r_logits, r_idx, None)
    torch.cuda.synchronize()
    st = dg.dg_query_status(model.ctx, ws)
    assert st == dg.DG_OK
    lw = oracle_layer(W["layers"][layer], cfg)
    K, V = np64(kv[layer][0]), np64(kv[layer][1].transpose(-1, -2))
    h0 = rin.cpu().numpy().astype(np.float64)
    rnd = rounder(cfg.act_dtype)
    # routing: the GPU's own top-k, reroutes only where the score error explains them (bounded)
    _, info = M.denoise_layer(cfg, layer, h0, lw, K, V, [cfg.prefix] * B, rnd)
    forced, n_rer, lg_err = check_routing(cfg, r_idx.cpu().numpy(), r_logits.cpu().numpy(), info)
    h1, _ = M.denoise_layer(cfg, layer, h0, lw, K, V, [cfg.prefix] * B, rnd, forced_idx=forced)
    got = rout.cpu().numpy()
    err = np.abs(got - h1).max()
    log(f"  max |resid - oracle| = {err:.3e} (tol {tol}); router logits max err {lg_err:.2e}; "
        f"near-tie reroutes {n_rer}")
    assert err <= tol
    return err


def test_tiny_fp32_layer_parity():
    cfg = configs.C0.replace(kv_source="random", resid_input=True)
    _layer_parity(cfg, 0, 1e-4)
    _layer_parity(cfg, 1, 1e-4)


def test_gemma_like_layer_parity_bf16():
    """One global layer of the assumed Gemma-4-like widths over a 2048-token prefix."""
    _layer_parity(configs.C1, 0, 2e-2)


def test_local_and_global_layers_parity_bf16():
    """Sliding-window (ring cache, window 1024) and global layers over an 8192-token prefix."""
    cfg = configs.C2.replace(n_layers=6, resid_input=True)
    _layer_parity(cfg, 0, 2e-2)
    _layer_parity(cfg, 5, 2e-2)


def test_large_prefix_values_through_split_attention():
    """Prefix values x 2^12 (split partials O_s / l_s up to ~2^14.5, inside the half-precision range
    the split partials are stored in) and W_o x 2^-12, so the residual keeps its scale: the split
    partials and their merge at large magnitude, on a local and a global layer of C2 shapes."""
    cfg = configs.C2.replace(n_layers=6, resid_input=True)
    for layer in (0, 5):
        _layer_parity(cfg, layer, 2e-2, scale_v=4096.0)


def test_fp8_experts_batched_layer_parity():
    """fp8 e4m3 expert weights with bf16 scales (weights-only), Zipf-skewed routing, 2 canvases."""
    cfg = configs.C4.replace(n_layers=1, batch=2, prefix=1024, resid_input=True, window=0, global_every=0)
    _layer_parity(cfg, 0, 2e-2)


def test_mxfp4_experts_layer_parity():
    """MXFP4 expert weights (e2m1 codes, one e8m0 scale per 32 inputs; weights-only, bf16 math):
    one global layer over a 2048-token prefix, and two Zipf-routed canvases."""
    _layer_parity(configs.C1.replace(expert_dtype="mxfp4"), 0, 2e-2)
    cfg = configs.C4.replace(expert_dtype="mxfp4", n_layers=1, batch=2, prefix=1024, resid_input=True,
                             window=0, global_every=0)
    _layer_parity(cfg, 0, 2e-2)


def test_layer_is_deterministic():
    cfg = configs.C1
    model, W, kv = build(cfg)
    ws = model.workspace(1, 256, cfg.prefix)
    rin = gen.resid_input(cfg, DEV)
    outs = []
    for _ in range(2):
        r = torch.empty_like(rin)
        model.denoise_step(None, 256, ws, resid_out=r, resid_in=rin, layer_begin=0, layer_end=1)
        outs.append(r)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])


def test_fp8_batch8_layers_parity_full_shape():
    """Eight canvases over a 4096-token prefix each, fp8 e4m3 experts with a Zipf(1.1) router
    prior: one local and one global layer at the full 2048-row shape."""
    cfg = configs.C4.replace(n_layers=6, resid_input=True)
    _layer_parity(cfg, 0, 2e-2)
    _layer_parity(cfg, 5, 2e-2)


@pytest.mark.parametrize("experts", ["bf16", "mxfp4"])
def test_batch8_wide_expert_tiles_layer_parity(experts):
    """Eight canvases (2048 rows, Zipf-routed experts averaging 128 rows): the grouped GEMMs take
    128-row expert tiles; bf16 and MXFP4 expert weights (fp8 runs in the full-shape test above)."""
    cfg = configs.C4.replace(expert_dtype=experts, n_layers=1, prefix=1024, resid_input=True, window=0,
                             global_every=0)
    _layer_parity(cfg, 0, 2e-2)


def test_long_prefix_global_layer_sampled_rows():
    """A global layer over a 131072-token prefix (131328 keys per query).  The GPU runs the whole
    layer; the oracle recomputes q/k/v for every canvas row (the canvas keys need all of them) and
    the attention, output projection and MoE for 12 sampled rows, which depend on no other row."""
    cfg = configs.C3.replace(n_layers=6, resid_input=True)
    layer = 5
    log(f"sampled-row parity: {cfg.name} layer {layer}, prefix {cfg.prefix}")
    model, W, kv = build(cfg)
    B, L = cfg.batch, cfg.canvas
    ws = model.workspace(B, L, cfg.prefix)
    rin = gen.resid_input(cfg, DEV)
    rout = torch.empty_like(rin)
    model.denoise_step(None, L, ws, resid_out=rout, resid_in=rin, layer_begin=layer, layer_end=layer + 1)
    r_logits = torch.empty(B * L, cfg.n_experts, dtype=torch.float32, device=DEV)
    r_idx = torch.empty(B * L, cfg.top_k, dtype=torch.int32, device=DEV)
    dg.dg_test_read_routing(model.ctx, ws, B * L, r_logits, r_idx, None)
    torch.cuda.synchronize()
    assert dg.dg_query_status(model.ctx, ws) == dg.DG_OK
    rows = np.array([0, 1, 17, 63, 64, 100, 127, 128, 191, 200, 254, 255])
    lw = oracle_layer(W["layers"][layer], cfg)
    K = np64(kv[layer][0])[0]
    V = np64(kv[layer][1].transpose(-1, -2))[0]
    rnd = rounder(cfg.act_dtype)
    h0 = rin.cpu().numpy().astype(np.float64)
    x = rnd(M.rmsnorm(h0, lw["attn_norm"], cfg.norm_eps))
    pos = cfg.prefix + np.arange(L)
    q, k, v = M.qkv(cfg, x, lw, pos, rnd)
    o = M.canvas_attention(cfg, layer, q[rows], k.transpose(1, 0, 2), v.transpose(1, 0, 2), K, V, cfg.prefix)
    o = rnd(o.reshape(len(rows), -1))
    h1 = h0[rows] + o @ lw["w_o"].T
    a2 = rnd(M.rmsnorm(h1, lw["ffn_norm"], cfg.norm_eps))
    f, info = M.moe(cfg, a2, lw, rnd)
    gidx = r_idx.cpu().numpy()[rows]
    g_r = r_logits.cpu().numpy()[rows]
    assert np.array_equal(gidx, M.router_topk(g_r, cfg.top_k)[0])
    lg_err = float(np.abs(g_r - info["r32"]).max())
    srt = -np.sort(-info["r32"].astype(np.float64), axis=1)
    near = srt[:, cfg.top_k - 1] - srt[:, cfg.top_k] <= 2 * lg_err + 1e-6
    mism = np.any(np.sort(gidx, 1) != np.sort(info["idx"], 1), axis=1)
    assert lg_err <= 2e-2 and not (mism & ~near).any()
    if mism.any():
        f, _ = M.moe(cfg, a2, lw, rnd, forced_idx=np.where(mism[:, None], gidx, info["idx"]))
    err = np.abs(rout.cpu().numpy()[rows] - (h1 + f)).max()
    log(f"  max |resid - oracle| over {len(rows)} rows = {err:.3e}; router logits max err {lg_err:.2e}")
    assert err <= 2e-2
