"""The C-ABI library without a GPU: it loads, exports every function include/dg.h declares, and
its host-side pieces (validation, workspace sizing, the Euler jump probability) behave as
documented.  No call here reaches a kernel."""
import ctypes as C
import os
import re

import numpy as np
import pytest

from discrete_text_diffusion_amd import dg
from discrete_text_diffusion_amd.model import model_desc
from oracle import step as S
from synth import configs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "dg.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dg_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = dg.load()
    names = header_functions()
    assert len(names) >= 17
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(dg.EXPORTS), set(names) ^ set(dg.EXPORTS)


@pytest.mark.parametrize("name", ["C0", "C2", "C4"])
def test_jump_prob_matches_oracle_on_every_grid_point(name):
    cfg = configs.get(name)
    ts, h = S.time_grid(cfg.steps)
    # the library's Euler rate at the grid points (float t, h as passed through the ABI)
    for t in ts:
        want = S.jump_prob(cfg.schedule, float(np.float32(t)), float(np.float32(h)))
        got = dg.dg_jump_prob(cfg.schedule, float(t), float(h))
        assert got == want, (t, got, want)


def _weights_null():
    lw = (dg.LayerWeights * 2)()
    return dg.Weights(embed=None, final_norm=None, layers=C.cast(lw, C.POINTER(dg.LayerWeights))), lw


def test_create_rejects_unsupported_shapes_and_null_weights():
    w, keep = _weights_null()
    bad = model_desc(configs.C0.replace(head_dim=48))
    with pytest.raises(dg.DGError) as e:
        dg.dg_create(bad, w)
    assert e.value.status == dg.DG_EUNSUPPORTED and "head_dim" in dg.dg_last_error()
    for q in ("fp8", "mxfp4"):                  # quantised experts need bf16 activations
        bad = model_desc(configs.C0.replace(act_dtype="f32", expert_dtype=q))
        with pytest.raises(dg.DGError) as e:
            dg.dg_create(bad, w)
        assert e.value.status == dg.DG_EUNSUPPORTED
    # W8A8 needs fp8 weights and bf16 activations
    for kw in (dict(act_dtype="bf16", expert_dtype="bf16"), dict(act_dtype="bf16", expert_dtype="mxfp4"),
               dict(act_dtype="f32", expert_dtype="f32")):
        bad = model_desc(configs.C0.replace(act_quant="fp8", **kw))
        with pytest.raises(dg.DGError) as e:
            dg.dg_create(bad, w)
        assert e.value.status == dg.DG_EUNSUPPORTED and "expert_act_fp8" in dg.dg_last_error()
    ok = model_desc(configs.C0)
    with pytest.raises(dg.DGError) as e:
        dg.dg_create(ok, w)                     # NULL matrices
    assert e.value.status == dg.DG_EINVAL


class _FakeTensor:
    """Stands in for a device tensor: a non-null address that no call ever dereferences."""
    def __init__(self, addr, nbytes):
        self.addr, self.nbytes = addr, nbytes

    def data_ptr(self):
        return self.addr

    def numel(self):
        return self.nbytes

    def element_size(self):
        return 1


def _ctx_with_fake_pointers(cfg):
    lw = (dg.LayerWeights * cfg.n_layers)()
    for l in range(cfg.n_layers):
        for i, f in enumerate(dg.LAYER_FIELDS):
            if f.startswith("s_") or f.startswith("sh_s_") or f == "router_bias":
                continue
            setattr(lw[l], f, 0x1000 + 0x100 * i)
    w = dg.Weights(embed=0x2000, final_norm=0x3000, layers=C.cast(lw, C.POINTER(dg.LayerWeights)))
    return dg.dg_create(model_desc(cfg), w), lw


def test_validation_enqueues_nothing_on_bad_calls():
    cfg = configs.C0
    ctx, keep = _ctx_with_fake_pointers(cfg)
    try:
        need = dg.dg_workspace_bytes(ctx, 1, 32, 64)
        assert need > 0
        assert dg.dg_workspace_bytes(ctx, 2, 32, 64) > need
        n = cfg.n_layers
        kp = (C.c_void_p * n)(0x5000, 0x6000)
        cap = (C.c_int32 * n)(128, 128)
        kv = dg.KV(k=kp, v=kp, cap=cap, prefix_len=0x8000, max_prefix=64, batch=1)
        ws = _FakeTensor(0x10000000, need)
        canvas = _FakeTensor(0x7000, 128)
        # workspace too small
        with pytest.raises(dg.DGError) as e:
            dg.dg_denoise_step(ctx, kv, canvas, None, 32, 0, n, None, None, _FakeTensor(0x10000000, need - 1), 0)
        assert e.value.status == dg.DG_EWORKSPACE
        # misaligned workspace
        with pytest.raises(dg.DGError) as e:
            dg.dg_denoise_step(ctx, kv, canvas, None, 32, 0, n, None, None, _FakeTensor(0x10000010, need), 0)
        assert e.value.status == dg.DG_EWORKSPACE
        # canvas length not a multiple of 16
        with pytest.raises(dg.DGError) as e:
            dg.dg_denoise_step(ctx, kv, canvas, None, 30, 0, n, None, None, ws, 0)
        assert e.value.status == dg.DG_EUNSUPPORTED
        # bad layer range
        with pytest.raises(dg.DGError) as e:
            dg.dg_denoise_step(ctx, kv, canvas, None, 32, 1, 3, None, None, ws, 0)
        assert e.value.status == dg.DG_EINVAL
        # cache too small for the prefix
        cap[0] = 32
        with pytest.raises(dg.DGError) as e:
            dg.dg_denoise_step(ctx, kv, canvas, None, 32, 0, n, None, None, ws, 0)
        assert e.value.status == dg.DG_EINVAL and "cap" in dg.dg_last_error()
        cap[0] = 128
        # Step parameters
        p = dg.StepParams(schedule=0, t=1.0, h=0.25, tau=0.0, lock_threshold=0.9, seed=0, step=0)
        with pytest.raises(dg.DGError) as e:
            dg.dg_step_sample(ctx, canvas, canvas, canvas, None, None, 1, 32, p, ws, 0)
        assert e.value.status == dg.DG_EINVAL and "tau" in dg.dg_last_error()
        p = dg.StepParams(schedule=7, t=1.0, h=0.25, tau=1.0, lock_threshold=0.9, seed=0, step=0)
        with pytest.raises(dg.DGError):
            dg.dg_step_sample(ctx, canvas, canvas, canvas, None, None, 1, 32, p, ws, 0)
        # prefill: cache must hold prefix + new tokens
        tok = _FakeTensor(0x8000, 4 * 200)
        with pytest.raises(dg.DGError) as e:
            dg.dg_prefill_kv(ctx, kv, tok, 100, _FakeTensor(ws.addr, 1 << 40), 0)
        assert e.value.status == dg.DG_EINVAL and "cap" in dg.dg_last_error()
        del tok
        # mixed pass: flags and output required, room for L more positions on every canvas, the
        # canvas-length rule of the decoder pass
        flags = _FakeTensor(0x9000, 4)
        hid = _FakeTensor(0xa000, 4 * 32 * cfg.d_model)
        with pytest.raises(dg.DGError) as e:
            dg.dg_mixed_forward(ctx, kv, canvas, None, 32, hid, ws, 0)
        assert e.value.status == dg.DG_EINVAL
        with pytest.raises(dg.DGError) as e:
            dg.dg_mixed_forward(ctx, kv, canvas, flags, 32, None, ws, 0)
        assert e.value.status == dg.DG_EINVAL
        cap[0] = cap[1] = 64 + 16
        with pytest.raises(dg.DGError) as e:
            dg.dg_mixed_forward(ctx, kv, canvas, flags, 32, hid, ws, 0)
        assert e.value.status == dg.DG_EINVAL and "cap" in dg.dg_last_error()
        cap[0] = cap[1] = 128
        with pytest.raises(dg.DGError) as e:
            dg.dg_mixed_forward(ctx, kv, canvas, flags, 24, hid, ws, 0)
        assert e.value.status == dg.DG_EUNSUPPORTED
        with pytest.raises(dg.DGError) as e:
            dg.dg_mixed_forward(ctx, kv, canvas, flags, 32, hid, _FakeTensor(0x10000000, need - 1), 0)
        assert e.value.status == dg.DG_EWORKSPACE
    finally:
        dg.dg_destroy(ctx)


def test_noalloc_step_rejects_shapes_beyond_its_static_scratch():
    """dg_step_sample_noalloc keeps its scratch in a 2 MiB static array: 64 canvases of 1024 rows
    need more (statistics and partials of 65,536 rows), so the call fails on the host with
    DG_EUNSUPPORTED before any HIP call (no GPU needed to see it)."""
    cfg = configs.C0
    ctx, keep = _ctx_with_fake_pointers(cfg)
    try:
        p = dg.StepParams(schedule=0, t=1.0, h=0.25, tau=1.0, lock_threshold=0.9, seed=0, step=0)
        t = _FakeTensor(0x7000, 16)
        with pytest.raises(dg.DGError) as e:
            dg.dg_step_sample_noalloc(ctx, t, t, t, t, None, 64, 1024, p, 0)
        assert e.value.status == dg.DG_EUNSUPPORTED
        assert "static scratch" in str(e.value)
        # bad arguments are caught first, as for dg_step_sample
        with pytest.raises(dg.DGError) as e:
            dg.dg_step_sample_noalloc(ctx, t, t, None, t, None, 1, 32, p, 0)
        assert e.value.status == dg.DG_EINVAL
    finally:
        dg.dg_destroy(ctx)
