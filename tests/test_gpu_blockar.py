"""Parity of block-AR generation (dg_generate, [TR §아키텍처와 블록 자기회귀 생성]) on the tiny fp32
model: prompt encoded by the causal encoder, three canvases each denoised by the canvas loop
(Euler with lock-in, and the entropy-bounded sampler) and appended to the cache; canvases, step
counts and the appended caches equal the oracle's, and the valid-token counts / EOS flags of
planted canvases are exact."""
import numpy as np
import pytest
import torch

from discrete_text_diffusion_amd import dg
from oracle import blockar as BA
from oracle import model as M
from synth import configs, gen
from tests.gpu_util import build, log
from tests.helpers import np64, oracle_kv, oracle_weights

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.mark.parametrize("sampler", ["euler", "eb"])
def test_generate_three_canvases_matches_oracle(sampler):
    K, P0 = 3, 48
    cfg = configs.C0.replace(batch=2, prefix=P0 + (K - 1) * 32, steps=4, tau=0.05, lock_threshold=0.9)
    B, L, V = cfg.batch, cfg.canvas, cfg.vocab
    model, W, kv = build(cfg, kv_mode="empty")
    ws = model.workspace(B, max(L, P0), cfg.prefix)
    model.set_kv(kv, [0] * B)
    prompt = torch.from_numpy(np.random.default_rng(5).integers(0, V, (B, P0)).astype(np.int32)).to(DEV)
    model.prefill_kv(prompt, ws)
    out = torch.empty(K, B, L, dtype=torch.int32, device=DEV)
    steps = torch.empty(K, B, dtype=torch.int32, device=DEV)
    valid = torch.empty(K, B, dtype=torch.int32, device=DEV)
    seen = torch.empty(K, B, dtype=torch.int32, device=DEV)
    eb_kw = dict(tau_start=0.05, tau_end=0.02)
    rp = dg.RunParams(schedule=cfg.schedule, max_steps=cfg.steps, tau=cfg.tau, lock_threshold=cfg.lock_threshold,
                      seed=11, adaptive=1, init_canvas=1,
                      sampler=dg.DG_SAMPLER_ENTROPY_BOUNDED if sampler == "eb" else dg.DG_SAMPLER_EULER,
                      gamma=0.1, stop_entropy=0.005, tau_end=eb_kw["tau_end"])
    if sampler == "eb":
        rp.tau = eb_kw["tau_start"]
    eos = 17
    model.generate(out, steps, valid, seen, eos, rp, ws)
    torch.cuda.synchronize()
    assert model.prefix_len == [P0 + (K - 1) * L] * B
    OW = oracle_weights(W, cfg)
    okv, plen = M.prefill(cfg, OW, oracle_kv(gen.empty_kv(cfg)), [0] * B, prompt.cpu().numpy())
    cfg_run = cfg.replace(adaptive=True)
    oout, osteps, okv2, oplen = BA.generate(cfg_run, OW, okv, plen, K, eos, sampler=sampler, seed=11,
                                            eb_kw=eb_kw if sampler == "eb" else None)
    g = out.cpu().numpy()
    log(f"  {sampler}: steps gpu {steps.cpu().numpy().T.tolist()} oracle {osteps.T.tolist()}; "
        f"mismatched tokens {int((g != oout).sum())}")
    assert np.array_equal(g, oout)
    assert np.array_equal(steps.cpu().numpy(), osteps)
    assert oplen == model.prefix_len
    # the appended canvases in the caches (global layers: slot = position)
    for l in range(cfg.n_layers):
        got = np64(kv[l][0])[:, :, :oplen[0]]
        assert np.abs(got - okv2[l][0][:, :, :oplen[0]]).max() <= 1e-4
    want_n = BA.valid_counts(g, eos)
    assert np.array_equal(valid.cpu().numpy(), want_n)
    assert np.array_equal(seen.cpu().numpy().astype(bool), BA.eos_mask(g, eos))


def test_valid_token_counts_planted():
    """The counting kernel through dg_generate (K = 1): with an eos that never occurs every
    canvas counts L; with an eos taken from canvas 0's tokens (and absent from canvas 2) the counts
    and flags equal the oracle's on the same tokens."""
    cfg = configs.C0.replace(batch=3, prefix=64, steps=1)
    B, L = cfg.batch, cfg.canvas
    model, W, kv = build(cfg, kv_mode="empty")
    ws = model.workspace(B, max(L, 64), cfg.prefix)
    model.set_kv(kv, [0] * B)
    out = torch.empty(1, B, L, dtype=torch.int32, device=DEV)
    valid = torch.empty(1, B, dtype=torch.int32, device=DEV)
    seen = torch.empty(1, B, dtype=torch.int32, device=DEV)
    rp = dg.RunParams(schedule=cfg.schedule, max_steps=1, tau=1.0, lock_threshold=0.9, seed=2, adaptive=0,
                      init_canvas=1)
    # first pass: find a token that occurs in canvas 0 but not canvas 2
    model.generate(out, None, valid, seen, -1, rp, ws)
    torch.cuda.synchronize()
    g = out.cpu().numpy()
    assert (valid.cpu().numpy() == L).all() and not seen.cpu().numpy().any()
    cand = [t for t in np.unique(g[0, 0]) if t not in g[0, 2]]
    eos = int(cand[0])
    model.set_kv(kv, [0] * B)
    model.generate(out, None, valid, seen, eos, rp, ws)
    torch.cuda.synchronize()
    g = out.cpu().numpy()
    assert np.array_equal(valid.cpu().numpy(), BA.valid_counts(g, eos))
    assert seen.cpu().numpy()[0, 0] == 1 and seen.cpu().numpy()[0, 2] == 0


def test_continuous_generation_matches_oracle_and_saves_passes():
    """dg_generate_continuous: every sequence on its own schedule, a stopped canvas appended in the
    next mixed pass while the other sequences keep denoising.  Per sequence the canvases, step counts
    and appended caches equal the oracle's block-AR generation (and the lockstep dg_generate's); the
    passes that ran equal max_b (sum_k s_k,b + K - 1)."""
    K, P0 = 3, 48
    cfg = configs.C0.replace(batch=3, prefix=P0 + (K - 1) * 32, steps=8, tau=0.03, lock_threshold=0.9)
    B, L, V = cfg.batch, cfg.canvas, cfg.vocab
    prompt = torch.from_numpy(np.random.default_rng(5).integers(0, V, (B, P0)).astype(np.int32)).to(DEV)
    rp = dg.RunParams(schedule=cfg.schedule, max_steps=cfg.steps, tau=cfg.tau, lock_threshold=cfg.lock_threshold,
                      seed=11, adaptive=1, init_canvas=1, sampler=dg.DG_SAMPLER_EULER)
    eos = 17

    def encoded():
        model, W, kv = build(cfg, kv_mode="empty")
        model.set_kv(kv, [0] * B)
        ws = model.workspace(B, max(L, P0), cfg.prefix)
        model.prefill_kv(prompt, ws)
        return model, W, kv, ws

    outs = {}
    for mode in ("continuous", "lockstep"):
        model, W, kv, ws = encoded()
        out = torch.empty(K, B, L, dtype=torch.int32, device=DEV)
        steps = torch.empty(K, B, dtype=torch.int32, device=DEV)
        valid = torch.empty(K, B, dtype=torch.int32, device=DEV)
        seen = torch.empty(K, B, dtype=torch.int32, device=DEV)
        passes = torch.full((1,), -1, dtype=torch.int32, device=DEV)
        if mode == "continuous":
            model.generate_continuous(out, steps, valid, seen, passes, eos, rp, ws)
        else:
            model.generate(out, steps, valid, seen, eos, rp, ws)
        torch.cuda.synchronize()
        assert dg.dg_query_status(model.ctx, ws) == dg.DG_OK
        outs[mode] = (out.cpu().numpy(), steps.cpu().numpy(), valid.cpu().numpy(), seen.cpu().numpy(),
                      int(passes.item()), model.prefix_len, [np64(kv[l][0]) for l in range(cfg.n_layers)])
    g, gs, gv, gseen, npass, gplen, gk = outs["continuous"]
    OW = oracle_weights(W, cfg)
    okv, plen = M.prefill(cfg, OW, oracle_kv(gen.empty_kv(cfg)), [0] * B, prompt.cpu().numpy())
    oout, osteps, okv2, oplen = BA.generate(cfg.replace(adaptive=True), OW, okv, plen, K, eos, seed=11)
    want_cont, want_lock = BA.continuous_passes(osteps)
    log(f"  steps gpu {gs.T.tolist()} oracle {osteps.T.tolist()}; passes {npass} (oracle {want_cont}, "
        f"lockstep schedule {want_lock})")
    assert np.array_equal(g, oout) and np.array_equal(gs, osteps)
    assert np.array_equal(g, outs["lockstep"][0]) and np.array_equal(gs, outs["lockstep"][1])
    assert npass == want_cont
    assert gplen == oplen == [P0 + (K - 1) * L] * B
    for l in range(cfg.n_layers):
        assert np.abs(gk[l][:, :, :oplen[0]] - okv2[l][0][:, :, :oplen[0]]).max() <= 1e-4
    assert np.array_equal(gv, BA.valid_counts(g, eos))
    assert np.array_equal(gseen.astype(bool), BA.eos_mask(g, eos))
