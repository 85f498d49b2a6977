"""Mixed batches (dg_mixed_forward, [TR §CPU-GPU 동기화 제거]): denoising canvases and cache-update
canvases in one pass, told apart by a per-canvas causal flag that only the kernels read.

- tiny fp32 model with a sliding-window layer and a global layer: hidden states and caches equal
  the oracle's mixed pass; the Step with the flags as `done` moves only the denoising canvas;
- a small bf16 model (head_dim 256, the bf16 attention kernels) with top-k = all experts, so that
  no near-tie reroute can move a row between the two sides: the causal encoder pass
  (dg_prefill_kv) and the mixed pass equal the oracle within 2e-2 plus one bf16 storage step of
  the value (the outputs compared here are stored in bf16);
- the assumed Gemma-like widths: every canvas of a mixed batch equals, bit for bit, the same canvas
  in a batch where all canvases take its kind of pass (rows never interact, and both batches
  launch the same tiles and splits)."""
import numpy as np
import pytest
import torch

from oracle import model as M
from oracle import step as S
from synth import configs
from tests.gpu_util import build, compare_step, log, read_stats, step_params, top2_gap
from tests.helpers import np64, oracle_kv_dev, oracle_weights

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _tokens(cfg, B, n, seed):
    rng = np.random.default_rng(seed)
    return torch.from_numpy(rng.integers(0, cfg.vocab, (B, n)).astype(np.int32)).to(DEV)


def _caches(kv):
    return [(k.clone(), v.clone()) for k, v in kv]


def _restore(kv, saved):
    for (k, v), (k0, v0) in zip(kv, saved):
        k.copy_(k0)
        v.copy_(v0)


def _cache_err(kv, okv, canvases):
    """Largest |cache - oracle| over the given canvases (keys and values are stored in bf16 on both
    sides, at magnitudes below 4 here, so one rounding flip stays below 2^-6)."""
    err = 0.0
    for (k, v), (K, V) in zip(kv, okv):
        for b in canvases:
            err = max(err, float(np.abs(np64(k[b]) - K[b]).max()), float(np.abs(np64(v[b].transpose(-1, -2)) - V[b]).max()))
    return err


def test_mixed_forward_tiny_fp32_matches_oracle():
    cfg = configs.C0.replace(batch=3, window=16, global_every=2, prefix=80, kv_source="random")
    B, n = cfg.batch, 16
    plen = [40, 25, 48]
    flags = [1, 0, 1]
    model, W, kv = build(cfg)
    model.set_kv(kv, plen)
    saved = _caches(kv)
    okv = oracle_kv_dev(kv)
    OW = oracle_weights(W, cfg)
    toks = _tokens(cfg, B, n, 31)
    append = torch.tensor(flags, dtype=torch.int32, device=DEV)
    ws = model.workspace(B, n, cfg.prefix)
    H = torch.empty(B * n, cfg.d_model, dtype=torch.float32, device=DEV)
    log(f"  mixed pass: tiny fp32, flags {flags}, prefixes {plen}")
    model.mixed_forward(toks, append, H, ws)
    torch.cuda.synchronize()
    oH, okv2 = M.mixed_forward(cfg, OW, okv, plen, toks.cpu().numpy(), flags)
    eh = float(np.abs(H.cpu().numpy() - oH).max())
    ek = max(float(np.abs(np64(k) - K).max()) for (k, _), (K, _) in zip(kv, okv2))
    ev = max(float(np.abs(np64(v.transpose(-1, -2)) - V).max()) for (_, v), (_, V) in zip(kv, okv2))
    log(f"  |H - oracle| {eh:.2e}; |K caches - oracle| {ek:.2e}; |V caches - oracle| {ev:.2e}")
    assert eh <= 1e-4 and ek <= 1e-4 and ev <= 1e-4
    for (k, v), (k0, v0) in zip(kv, saved):
        assert torch.equal(k[1], k0[1]) and torch.equal(v[1], v0[1]), "a denoising canvas's cache changed"
    # the Step with the flags as `done`: only the denoising canvas moves
    canvas = toks.clone()
    lock = torch.zeros(B, n, dtype=torch.uint8, device=DEV)
    nl = torch.empty(B, dtype=torch.int32, device=DEV)
    t, h = 1.0, 1.0      # jump probability 1 at t = 1: every unlocked position of the canvas draws
    model.step_sample(H, canvas, lock, nl, step_params(cfg.schedule, t, h, cfg.tau, cfg.lock_threshold, 5, 0), ws,
                      done=append)
    torch.cuda.synchronize()
    g = canvas.cpu().numpy()
    before = toks.cpu().numpy()
    assert np.array_equal(g[[0, 2]], before[[0, 2]]) and not lock.cpu().numpy()[[0, 2]].any()
    Hg = H.cpu().numpy().astype(np.float64)
    z = S.logits(Hg, OW["embed"], cfg.tau)
    ocv, olk, _, ost, _ = S.step(Hg, OW["embed"], before, np.zeros((B, n), bool), t, h, cfg.schedule, cfg.tau,
                                 cfg.lock_threshold, 5, 0, done=np.array(flags))
    st = read_stats(model, ws, B * n)
    compare_step(g, lock.cpu().numpy(), st, ocv, olk, ost, top2_gap(z), cfg.lock_threshold)
    assert (g[1] != before[1]).any()


SMALL_BF16 = configs.Workload(
    name="small-bf16-topall", n_layers=2, d_model=512, n_q_heads=4, n_kv_heads=2, head_dim=256, n_experts=8,
    top_k=8, expert_hidden=256, shared_hidden=512, vocab=1024, window=64, global_every=2, act_dtype="bf16",
    expert_dtype="bf16", batch=3, canvas=48, prefix=200, kv_source="random", resid_input=False, zipf=0.0,
    steps=1, schedule=configs.KAPPA_LINEAR, lock_threshold=0.9, tau=1.0, adaptive=False)


def test_small_bf16_prefill_and_mixed_pass_match_oracle():
    """Layer 0 keeps a 64-slot ring (canvas 0's prefix of 120 wraps it), layer 1 is global; 48 new
    tokens per canvas (a partial 64-key tile)."""
    cfg = SMALL_BF16
    B, n = cfg.batch, 48
    plen = [120, 70, 90]
    model, W, kv = build(cfg)
    model.set_kv(kv, plen)
    saved = _caches(kv)
    okv = oracle_kv_dev(kv)
    OW = oracle_weights(W, cfg)
    toks = _tokens(cfg, B, n, 41)
    ws = model.workspace(B, n, cfg.prefix)
    # the causal encoder pass on every canvas
    log(f"  bf16 prefill: prefixes {plen}, {n} tokens")
    model.prefill_kv(toks, ws)
    torch.cuda.synchronize()
    okv_p, _ = M.prefill(cfg, OW, okv, plen, toks.cpu().numpy())
    ek = _cache_err(kv, okv_p, range(B))
    log(f"  prefill: max |cache - oracle| {ek:.2e}")
    assert ek <= 2e-2
    # the mixed pass from the same caches
    _restore(kv, saved)
    model.set_kv(kv, plen)
    flags = [0, 1, 0]
    append = torch.tensor(flags, dtype=torch.int32, device=DEV)
    H = torch.empty(B * n, cfg.d_model, dtype=torch.bfloat16, device=DEV)
    R = torch.empty(B * n, cfg.d_model, dtype=torch.float32, device=DEV)
    log(f"  bf16 mixed pass: flags {flags}")
    model.mixed_forward(toks, append, H, ws, resid_out=R)
    torch.cuda.synchronize()
    oH, okv_m, oR = M.mixed_forward(cfg, OW, okv, plen, toks.cpu().numpy(), flags, with_resid=True)
    er = float(np.abs(R.cpu().numpy() - oR).max())
    ek = _cache_err(kv, okv_m, range(B))
    log(f"  mixed: max |resid - oracle| {er:.2e}, max |cache - oracle| {ek:.2e} "
        f"(bf16 H: {float(np.abs(np64(H) - oH).max()):.2e}, reported)")
    assert er <= 2e-2 and ek <= 2e-2
    for (k, v), (k0, v0) in zip(kv, saved):
        for b in (0, 2):
            assert torch.equal(k[b], k0[b]) and torch.equal(v[b], v0[b]), "a denoising canvas's cache changed"


def test_long_causal_chunk_prefill_matches_oracle():
    """A 400-token chunk per canvas through the causal encoder: key tiles past a query block's last
    position, and on the 64-slot sliding-window layer tiles wholly older than its first query's
    window, are skipped; blocks of 128 query rows straddle the two heads' row ranges at 400."""
    cfg = SMALL_BF16.replace(batch=2, prefix=448)
    B, n = cfg.batch, 400
    plen = [0, 37]
    model, W, kv = build(cfg)
    model.set_kv(kv, plen)
    okv = oracle_kv_dev(kv)
    OW = oracle_weights(W, cfg)
    toks = _tokens(cfg, B, n, 43)
    ws = model.workspace(B, n, cfg.prefix)
    log(f"  long causal chunk: prefixes {plen}, {n} tokens")
    model.prefill_kv(toks, ws)
    torch.cuda.synchronize()
    okv_p, oplen = M.prefill(cfg, OW, okv, plen, toks.cpu().numpy())
    ek = _cache_err(kv, okv_p, range(B))
    log(f"  prefill: max |cache - oracle| {ek:.2e}; prefix lengths {model.prefix_len} (oracle {list(oplen)})")
    assert ek <= 2e-2
    assert list(model.prefix_len) == [int(x) for x in oplen]


@pytest.mark.parametrize("flags", [[1, 0, 0], [0, 1, 1]])
def test_mixed_pass_equals_uniform_passes_bit_exact(flags):
    """Two layers at the assumed Gemma-like widths (a 1024-slot ring layer, then a global layer),
    three 256-token canvases over prefixes 1500 / 700 / 1100."""
    cfg = configs.C2.replace(n_layers=2, global_every=2, batch=3, prefix=1792, vocab=4096)
    B, n = cfg.batch, cfg.canvas
    plen = [1500, 700, 1100]
    model, W, kv = build(cfg)
    saved = _caches(kv)
    toks = _tokens(cfg, B, n, 51)
    ws = model.workspace(B, n, cfg.prefix)
    append = torch.tensor(flags, dtype=torch.int32, device=DEV)
    Hm = torch.empty(B * n, cfg.d_model, dtype=torch.bfloat16, device=DEV)
    log(f"  Gemma-like mixed pass: flags {flags}, prefixes {plen}")
    model.set_kv(kv, plen)
    model.mixed_forward(toks, append, Hm, ws)
    torch.cuda.synchronize()
    mixed = _caches(kv)
    # all canvases appended by the causal encoder
    _restore(kv, saved)
    model.set_kv(kv, plen)
    model.prefill_kv(toks, ws)
    torch.cuda.synchronize()
    enc = _caches(kv)
    # all canvases denoised
    _restore(kv, saved)
    model.set_kv(kv, plen)
    Hd = torch.empty_like(Hm)
    model.denoise_step(toks, n, ws, hidden_out=Hd)
    torch.cuda.synchronize()
    for b, f in enumerate(flags):
        want = enc if f else saved
        for l, ((k, v), (kw, vw)) in enumerate(zip(mixed, want)):
            assert torch.equal(k[b], kw[b]) and torch.equal(v[b], vw[b]), f"canvas {b} layer {l} cache"
        if not f:
            rows = slice(b * n, (b + 1) * n)
            assert torch.equal(Hm[rows], Hd[rows]), f"canvas {b} hidden states"
