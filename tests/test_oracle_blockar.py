"""Pins of the oracle's block-AR accounting [TR §추론 효율 지표] and loop [TR §아키텍처와 블록
자기회귀 생성] (CPU): valid-token counts by hand, the TPF / effective-step formulas on a worked
example and their single-canvas special case, and the append-after-encode loop against chunked
prefill (appending canvas k equals encoding prompt + canvases 0..k in one causal pass)."""
import numpy as np
import pytest

from oracle import blockar as BA
from oracle import model as M
from synth import configs, gen
from tests.helpers import oracle_kv, oracle_weights


def test_valid_counts_by_hand():
    eos = 7
    out = np.array([[[1, 2, 3, 4], [7, 1, 1, 1]],
                    [[5, 7, 7, 2], [1, 2, 3, 4]],
                    [[7, 1, 2, 3], [1, 1, 7, 1]]])            # [K=3][B=2][L=4]
    n = BA.valid_counts(out, eos)
    assert n.tolist() == [[4, 0], [1, 0], [0, 0]]
    assert BA.eos_mask(out, eos).tolist() == [[False, True], [True, False], [True, True]]


def test_metrics_worked_example_and_single_canvas():
    # three canvases of 256: 256 + 256 + 40 tokens in 10, 14, 6 steps; EOS in the third
    steps = np.array([[10], [14], [6]]); valid = np.array([[256], [256], [40]])
    seen = np.array([[False], [False], [True]])
    m = BA.metrics(steps, valid, seen)[0]
    assert m["canvases"] == 3 and m["tokens"] == 552 and m["steps"] == 30
    assert m["tpf"] == pytest.approx(552 / 32)
    assert m["effective_steps"] == pytest.approx((256 * 10 + 256 * 14 + 40 * 6) / 552)
    # canvases after the EOS canvas do not count
    m2 = BA.metrics(np.vstack([steps, [[9]]]), np.vstack([valid, [[0]]]), np.vstack([seen, [[True]]]))[0]
    assert m2 == m
    # one canvas: TPF = n / s, effective steps = s
    m1 = BA.metrics(np.array([[12]]), np.array([[200]]), np.array([[True]]))[0]
    assert m1["tpf"] == pytest.approx(200 / 12) and m1["effective_steps"] == pytest.approx(12)


def test_append_after_encode_equals_one_causal_pass():
    cfg = configs.C0.replace(batch=2)
    W = gen.make_weights(cfg, "cpu")
    OW = oracle_weights(W, cfg)
    rng = np.random.default_rng(3)
    prompt = rng.integers(0, cfg.vocab, (cfg.batch, 24))
    canv = [rng.integers(0, cfg.vocab, (cfg.batch, 16)) for _ in range(2)]
    kv0 = oracle_kv(gen.empty_kv(cfg))
    kv, plen = M.prefill(cfg, OW, kv0, [0, 0], prompt)
    for c in canv:
        kv, plen = M.prefill(cfg, OW, kv, plen, c)
    kv1, plen1 = M.prefill(cfg, OW, kv0, [0, 0], np.concatenate([prompt] + canv, axis=1))
    assert plen == plen1 == [56, 56]
    for (K, V), (K1, V1) in zip(kv, kv1):
        assert np.allclose(K[:, :, :56], K1[:, :, :56], atol=1e-10)
        assert np.allclose(V[:, :, :56], V1[:, :, :56], atol=1e-10)


def test_package_metrics_match_the_oracle():
    from discrete_text_diffusion_amd.metrics import block_ar_metrics
    rng = np.random.default_rng(9)
    for _ in range(20):
        K, B = int(rng.integers(1, 5)), int(rng.integers(1, 4))
        steps = rng.integers(1, 49, (K, B))
        seen = rng.random((K, B)) < 0.3
        valid = np.where(seen, rng.integers(0, 256, (K, B)), 256)
        want = BA.metrics(steps, valid, seen)
        got = block_ar_metrics(steps, valid, seen, t_fwd_s=0.0125)
        for g, w in zip(got, want):
            for key in ("canvases", "tokens", "steps", "effective_steps", "tpf"):
                assert g[key] == pytest.approx(w[key])
            assert g["tps"] == pytest.approx(w["tpf"] / 0.0125)


def _mixed_case():
    """Tiny fp32 model with a sliding-window layer (ring of 16 slots) and a global layer; random
    caches; three canvases at different prefix lengths (the first wraps its ring)."""
    cfg = configs.C0.replace(batch=3, window=16, global_every=2, prefix=80, kv_source="random")
    W = gen.make_weights(cfg, "cpu")
    OW = oracle_weights(W, cfg)
    kv = oracle_kv(gen.make_random_kv(cfg, "cpu"))
    rng = np.random.default_rng(21)
    toks = rng.integers(0, cfg.vocab, (cfg.batch, 16))
    return cfg, OW, kv, [40, 25, 48], toks


def _one(kv, b):
    return [(K[b:b + 1], V[b:b + 1]) for K, V in kv]


def test_mixed_pass_single_kind_batches_are_the_plain_passes():
    """[TR §CPU-GPU 동기화 제거] all-denoise: the decoder pass's hidden states and untouched caches;
    all-append: the causal encoder pass's caches."""
    cfg, OW, kv, plen, toks = _mixed_case()
    H, kv2 = M.mixed_forward(cfg, OW, kv, plen, toks, [0, 0, 0])
    H0, _ = M.denoise_forward(cfg, OW, kv, plen, canvas=toks)
    assert np.allclose(H, H0, rtol=0, atol=1e-12)
    for (K, V), (K2, V2) in zip(kv, kv2):
        assert np.array_equal(K, K2) and np.array_equal(V, V2)
    _, kv3 = M.mixed_forward(cfg, OW, kv, plen, toks, [1, 1, 1])
    kv4, plen4 = M.prefill(cfg, OW, kv, plen, toks)
    assert plen4 == [p + 16 for p in plen]
    for (K, V), (K4, V4) in zip(kv3, kv4):
        assert np.allclose(K, K4, rtol=0, atol=1e-12) and np.allclose(V, V4, rtol=0, atol=1e-12)


def test_mixed_pass_equals_each_canvas_alone():
    """A batch of [append, denoise, append]: each canvas's hidden states and caches equal those of
    its own kind of pass run on that canvas alone; the denoising canvas's caches are untouched and
    the appended ones differ from the input exactly at the new positions' slots."""
    cfg, OW, kv, plen, toks = _mixed_case()
    flags = [1, 0, 1]
    H, kv2 = M.mixed_forward(cfg, OW, kv, plen, toks, flags)
    n = toks.shape[1]
    for b, f in enumerate(flags):
        kvb = _one(kv, b)
        rows = slice(b * n, (b + 1) * n)
        if f:
            want, _ = M.prefill(cfg, OW, kvb, [plen[b]], toks[b:b + 1])
            for l, ((K2, V2), (Kw, Vw), (K0, _)) in enumerate(zip(kv2, want, kv)):
                assert np.allclose(K2[b:b + 1], Kw, rtol=0, atol=1e-12)
                assert np.allclose(V2[b:b + 1], Vw, rtol=0, atol=1e-12)
                changed = np.nonzero(np.any(K2[b] != K0[b], axis=(0, 2)))[0]
                pos = plen[b] + np.arange(n)
                slots = pos if cfg.is_global(l) else np.unique(pos[pos >= pos[-1] + 1 - cfg.window] % cfg.window)
                assert np.array_equal(changed, np.sort(slots))
            Hb, _ = M.mixed_forward(cfg, OW, kvb, [plen[b]], toks[b:b + 1], [1])
        else:
            for (K2, V2), (K0, V0) in zip(kv2, kv):
                assert np.array_equal(K2[b], K0[b]) and np.array_equal(V2[b], V0[b])
            Hb, _ = M.denoise_forward(cfg, OW, kvb, [plen[b]], canvas=toks[b:b + 1])
        assert np.allclose(H[rows], Hb, rtol=0, atol=1e-12)


def test_continuous_pass_count_by_hand():
    """Two sequences, three canvases: sequence 0 takes 2, 5, 1 steps, sequence 1 takes 4, 1, 3.
    Continuous: 8 + 2 and 8 + 2 passes -> 10; lockstep: 4 + 5 + 3 + 2 = 14.  One canvas: the
    continuous count is the slowest sequence's steps."""
    steps = np.array([[2, 4], [5, 1], [1, 3]])
    assert BA.continuous_passes(steps) == (10, 14)
    assert BA.continuous_passes(np.array([[3, 7, 5]])) == (7, 7)
    # equal step counts everywhere: the two schedules coincide
    assert BA.continuous_passes(np.full((4, 3), 6)) == (27, 27)
