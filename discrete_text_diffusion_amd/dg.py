"""ctypes binding of libdg.so: the C ABI of include/dg.h under the same names.

Argument marshalling only — every step of the denoise path runs in the library's HIP kernels.
torch tensors provide device memory and the stream; pointers are taken with .data_ptr().
Loading fails loudly when libdg.so has not been built: there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdg.so")

DG_OK, DG_EINVAL, DG_EUNSUPPORTED, DG_EWORKSPACE, DG_EHIP, DG_ENONFINITE = 0, -1, -2, -3, -4, -5
DG_F32, DG_BF16, DG_FP8E4M3, DG_MXFP4 = 0, 1, 2, 3
DG_KAPPA_LINEAR, DG_KAPPA_QUADRATIC, DG_KAPPA_COSINE = 0, 1, 2


class DGError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"dg status {status}: {msg}")
        self.status = status


class ModelDesc(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("n_layers", "d_model", "n_q_heads", "n_kv_heads", "head_dim",
                                          "n_experts", "top_k", "expert_hidden", "shared_hidden", "vocab",
                                          "window", "global_every")] + \
               [("rope_theta", C.c_float), ("norm_eps", C.c_float), ("act_dtype", C.c_int), ("expert_dtype", C.c_int),
                ("sc_hidden", C.c_int32), ("expert_act_fp8", C.c_int32)]


LAYER_FIELDS = ("attn_norm", "w_qkv", "w_o", "ffn_norm", "w_router", "router_bias", "w_gate", "w_up", "w_down",
                "s_gate", "s_up", "s_down", "sh_gate", "sh_up", "sh_down", "sh_s_gate", "sh_s_up", "sh_s_down")


class LayerWeights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in LAYER_FIELDS]


class Weights(C.Structure):
    _fields_ = [("embed", C.c_void_p), ("final_norm", C.c_void_p), ("layers", C.POINTER(LayerWeights)),
                ("embed_t", C.c_void_p), ("sc_gate", C.c_void_p), ("sc_up", C.c_void_p), ("sc_down", C.c_void_p)]


class KV(C.Structure):
    _fields_ = [("k", C.POINTER(C.c_void_p)), ("v", C.POINTER(C.c_void_p)), ("cap", C.POINTER(C.c_int32)),
                ("prefix_len", C.c_void_p), ("max_prefix", C.c_int32), ("batch", C.c_int32)]


class StepParams(C.Structure):
    _fields_ = [("schedule", C.c_int), ("t", C.c_float), ("h", C.c_float), ("tau", C.c_float),
                ("lock_threshold", C.c_float), ("seed", C.c_uint64), ("step", C.c_uint32)]


class RunParams(C.Structure):
    _fields_ = [("schedule", C.c_int), ("max_steps", C.c_int32), ("tau", C.c_float), ("lock_threshold", C.c_float),
                ("seed", C.c_uint64), ("adaptive", C.c_int32), ("init_canvas", C.c_int32), ("sampler", C.c_int),
                ("gamma", C.c_float), ("stop_entropy", C.c_float), ("tau_end", C.c_float),
                ("self_condition", C.c_int32)]


DG_SAMPLER_EULER, DG_SAMPLER_ENTROPY_BOUNDED = 0, 1


class EbParams(C.Structure):
    _fields_ = [("t", C.c_float), ("tau_start", C.c_float), ("tau_end", C.c_float), ("gamma", C.c_float),
                ("stop_entropy", C.c_float), ("seed", C.c_uint64), ("step", C.c_uint32), ("has_prev", C.c_int32),
                ("final_step", C.c_int32), ("adaptive", C.c_int32)]


EXPORTS = {
    "dg_create": (C.c_int, [C.POINTER(ModelDesc), C.POINTER(Weights), C.POINTER(C.c_void_p)]),
    "dg_destroy": (None, [C.c_void_p]),
    "dg_workspace_bytes": (C.c_size_t, [C.c_void_p, C.c_int32, C.c_int32, C.c_int32]),
    "dg_last_error": (C.c_char_p, []),
    "dg_query_status": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p]),
    "dg_clear_status": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p]),
    "dg_prefill_kv": (C.c_int, [C.c_void_p, C.POINTER(KV), C.c_void_p, C.c_int32, C.c_void_p, C.c_size_t,
                                C.c_void_p]),
    "dg_denoise_step": (C.c_int, [C.c_void_p, C.POINTER(KV), C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32,
                                  C.c_int32, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t,
                                  C.c_void_p]),
    "dg_mixed_forward": (C.c_int, [C.c_void_p, C.POINTER(KV), C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p,
                                   C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]),
    "dg_step_sample": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                 C.c_void_p, C.c_int32, C.c_int32, C.POINTER(StepParams), C.c_void_p, C.c_size_t,
                                 C.c_void_p]),
    "dg_step_sample_noalloc": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                         C.c_int32, C.c_int32, C.POINTER(StepParams), C.c_void_p]),
    "dg_canvas_run": (C.c_int, [C.c_void_p, C.POINTER(KV), C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32,
                                C.POINTER(RunParams), C.c_void_p, C.c_size_t, C.c_void_p]),
    "dg_jump_prob": (C.c_float, [C.c_int, C.c_float, C.c_float]),
    "dg_generate": (C.c_int, [C.c_void_p, C.POINTER(KV), C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32,
                              C.c_int32, C.c_int32, C.POINTER(RunParams), C.c_void_p, C.c_size_t, C.c_void_p]),
    "dg_generate_continuous": (C.c_int, [C.c_void_p, C.POINTER(KV), C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                         C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.POINTER(RunParams),
                                         C.c_void_p, C.c_size_t, C.c_void_p]),
    "dg_test_step_from_logits": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32,
                                           C.c_int32, C.POINTER(StepParams), C.c_void_p, C.c_size_t, C.c_void_p]),
    "dg_test_read_stats": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p,
                                     C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p]),
    "dg_step_entropy_bounded": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                          C.c_void_p, C.c_int32, C.c_int32, C.POINTER(EbParams), C.c_void_p,
                                          C.c_size_t, C.c_void_p]),
    "dg_test_eb_from_logits": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                         C.c_void_p, C.c_int32, C.c_int32, C.POINTER(EbParams), C.c_void_p,
                                         C.c_size_t, C.c_void_p]),
    "dg_test_eb_select": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                    C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_int32, C.POINTER(EbParams),
                                    C.c_void_p, C.c_size_t, C.c_void_p]),
    "dg_test_router_topk": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p,
                                      C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]),
    "dg_test_read_routing": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p,
                                       C.c_void_p]),
    "dg_test_read_expert_inputs": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int32, C.c_int32] + [C.c_void_p] * 10),
    "dg_test_quant_rows": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p]),
    "dg_test_noise": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_int, C.c_float,
                                C.c_uint64, C.c_uint32, C.c_void_p]),
    "dg_init_canvas": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_uint64, C.c_void_p]),
    "dg_profile_enable": (C.c_int, [C.c_void_p, C.c_uint32]),
    "dg_profile_read": (C.c_int, [C.c_void_p, C.c_int32, C.POINTER(C.c_double), C.POINTER(C.c_int32)]),
}

_lib = None


def load(path: str = LIB_PATH) -> C.CDLL:
    """Load libdg.so and declare its exports.  Raises if the library is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run discrete_text_diffusion_amd.build.build() first")
    lib = C.CDLL(path)
    for name, (res, args) in EXPORTS.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _check(status):
    if status != DG_OK:
        msg = load().dg_last_error()
        raise DGError(status, msg.decode() if msg else "")
    return status


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream):
    """A torch stream, a raw hipStream_t handle (int; 0 = the null stream), or None for torch's
    current stream."""
    if isinstance(stream, int):
        return C.c_void_p(stream or None)
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


# ---------------------------------------------------------------- same-named calls ------------

def dg_create(desc: ModelDesc, weights: Weights):
    ctx = C.c_void_p()
    _check(load().dg_create(C.byref(desc), C.byref(weights), C.byref(ctx)))
    return ctx


def dg_destroy(ctx):
    load().dg_destroy(ctx)


def dg_workspace_bytes(ctx, batch, rows_per_canvas, max_prefix):
    return load().dg_workspace_bytes(ctx, batch, rows_per_canvas, max_prefix)


def dg_last_error():
    m = load().dg_last_error()
    return m.decode() if m else ""


def dg_query_status(ctx, ws, stream=None):
    return load().dg_query_status(ctx, _ptr(ws), _stream(stream))


def dg_clear_status(ctx, ws, stream=None):
    _check(load().dg_clear_status(ctx, _ptr(ws), _stream(stream)))


def dg_prefill_kv(ctx, kv: KV, tokens, n, ws, stream=None):
    _check(load().dg_prefill_kv(ctx, C.byref(kv), _ptr(tokens), n, _ptr(ws), ws.numel() * ws.element_size(),
                                _stream(stream)))


def dg_denoise_step(ctx, kv: KV, canvas, resid_in, L, layer_begin, layer_end, hidden_out, resid_out, ws,
                    stream=None, sc_in=None):
    _check(load().dg_denoise_step(ctx, C.byref(kv), _ptr(canvas), _ptr(resid_in), _ptr(sc_in), L, layer_begin,
                                  layer_end, _ptr(hidden_out), _ptr(resid_out), _ptr(ws),
                                  ws.numel() * ws.element_size(), _stream(stream)))


def dg_mixed_forward(ctx, kv: KV, tokens, append, L, hidden_out, ws, stream=None, resid_out=None):
    _check(load().dg_mixed_forward(ctx, C.byref(kv), _ptr(tokens), _ptr(append), L, _ptr(hidden_out),
                                   _ptr(resid_out), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def dg_step_sample(ctx, hidden, canvas, lock, n_locked, done, batch, L, params: StepParams, ws, stream=None,
                   sc_out=None):
    _check(load().dg_step_sample(ctx, _ptr(hidden), _ptr(canvas), _ptr(lock), _ptr(n_locked), _ptr(done),
                                 _ptr(sc_out), batch, L, C.byref(params), _ptr(ws), ws.numel() * ws.element_size(),
                                 _stream(stream)))


def dg_step_sample_noalloc(ctx, hidden, canvas, lock, n_locked, done, B, L, params: StepParams, stream=None):
    _check(load().dg_step_sample_noalloc(ctx, _ptr(hidden), _ptr(canvas), _ptr(lock), _ptr(n_locked), _ptr(done),
                                         B, L, C.byref(params), _stream(stream)))


def dg_canvas_run(ctx, kv: KV, canvas, lock, steps_taken, L, params: RunParams, ws, stream=None):
    _check(load().dg_canvas_run(ctx, C.byref(kv), _ptr(canvas), _ptr(lock), _ptr(steps_taken), L, C.byref(params),
                                _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def dg_generate(ctx, kv: KV, out, steps, valid, eos_seen, K, L, eos_id, params: RunParams, ws, stream=None):
    _check(load().dg_generate(ctx, C.byref(kv), _ptr(out), _ptr(steps), _ptr(valid), _ptr(eos_seen), K, L, eos_id,
                              C.byref(params), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def dg_generate_continuous(ctx, kv: KV, out, steps, valid, eos_seen, passes, K, L, eos_id, params: RunParams, ws,
                           stream=None):
    _check(load().dg_generate_continuous(ctx, C.byref(kv), _ptr(out), _ptr(steps), _ptr(valid), _ptr(eos_seen),
                                         _ptr(passes), K, L, eos_id, C.byref(params), _ptr(ws),
                                         ws.numel() * ws.element_size(), _stream(stream)))


def dg_jump_prob(schedule, t, h):
    return load().dg_jump_prob(schedule, t, h)


def dg_test_step_from_logits(ctx, logits, canvas, lock, n_locked, batch, L, params: StepParams, ws, stream=None):
    _check(load().dg_test_step_from_logits(ctx, _ptr(logits), _ptr(canvas), _ptr(lock), _ptr(n_locked), batch, L,
                                           C.byref(params), _ptr(ws), ws.numel() * ws.element_size(),
                                           _stream(stream)))


def dg_test_read_stats(ctx, ws, rows, m=None, a=None, c=None, y=None, best=None, entropy=None, stream=None):
    _check(load().dg_test_read_stats(ctx, _ptr(ws), rows, _ptr(m), _ptr(a), _ptr(c), _ptr(y), _ptr(best),
                                     _ptr(entropy), _stream(stream)))


def dg_step_entropy_bounded(ctx, hidden, canvas, prev_argmax, done, n_accepted, mean_entropy, batch, L,
                            params: EbParams, ws, stream=None):
    _check(load().dg_step_entropy_bounded(ctx, _ptr(hidden), _ptr(canvas), _ptr(prev_argmax), _ptr(done),
                                          _ptr(n_accepted), _ptr(mean_entropy), batch, L, C.byref(params), _ptr(ws),
                                          ws.numel() * ws.element_size(), _stream(stream)))


def dg_test_eb_from_logits(ctx, logits, canvas, prev_argmax, done, n_accepted, mean_entropy, batch, L,
                           params: EbParams, ws, stream=None):
    _check(load().dg_test_eb_from_logits(ctx, _ptr(logits), _ptr(canvas), _ptr(prev_argmax), _ptr(done),
                                         _ptr(n_accepted), _ptr(mean_entropy), batch, L, C.byref(params), _ptr(ws),
                                         ws.numel() * ws.element_size(), _stream(stream)))


def dg_test_eb_select(ctx, entropy, argmax, draw, canvas, prev_argmax, done, n_accepted, mean_entropy, batch, L,
                      params: EbParams, ws, stream=None):
    _check(load().dg_test_eb_select(ctx, _ptr(entropy), _ptr(argmax), _ptr(draw), _ptr(canvas), _ptr(prev_argmax),
                                    _ptr(done), _ptr(n_accepted), _ptr(mean_entropy), batch, L, C.byref(params),
                                    _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def dg_test_router_topk(scores, T, E, k, idx, gates, counts, offsets, perm, ws, stream=None):
    _check(load().dg_test_router_topk(_ptr(scores), T, E, k, _ptr(idx), _ptr(gates), _ptr(counts), _ptr(offsets),
                                      _ptr(perm), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def dg_test_read_routing(ctx, ws, rows, logits=None, idx=None, gates=None, stream=None):
    _check(load().dg_test_read_routing(ctx, _ptr(ws), rows, _ptr(logits), _ptr(idx), _ptr(gates), _stream(stream)))


def dg_test_read_expert_inputs(ctx, ws, batch, L, xhat=None, xq=None, xs=None, a_grp=None, aq=None, as_=None,
                               sh_a=None, shq=None, shs=None, stream=None):
    _check(load().dg_test_read_expert_inputs(ctx, _ptr(ws), batch, L, _ptr(xhat), _ptr(xq), _ptr(xs), _ptr(a_grp),
                                             _ptr(aq), _ptr(as_), _ptr(sh_a), _ptr(shq), _ptr(shs),
                                             _stream(stream)))


def dg_test_quant_rows(x, rows, K, q, s, stream=None):
    _check(load().dg_test_quant_rows(_ptr(x), rows, K, _ptr(q), _ptr(s), _stream(stream)))


def dg_test_noise(x0, xt, batch, L, vocab, schedule, t, seed, step, stream=None):
    _check(load().dg_test_noise(_ptr(x0), _ptr(xt), batch, L, vocab, schedule, t, seed, step, _stream(stream)))


def dg_init_canvas(canvas, lock, batch, L, vocab, seed, stream=None):
    _check(load().dg_init_canvas(_ptr(canvas), _ptr(lock), batch, L, vocab, seed, _stream(stream)))


PROF_MOE_GATE_UP, PROF_MOE_DOWN, PROF_ATTENTION, PROF_SAMPLER, PROF_QKV, PROF_O_PROJ, PROF_SHARED, \
    PROF_ROUTING, PROF_SELF_COND, PROF_NORM_COMBINE, PROF_STEP, PROF_EMBED = range(12)
PROF_NAMES = ("moe_gate_up", "moe_down", "attention", "sampler", "qkv_rope", "o_proj", "shared_expert", "routing",
              "self_condition", "norm_combine", "step_merge", "embed_rope")


def dg_profile_enable(ctx, mask):
    _check(load().dg_profile_enable(ctx, mask))


def dg_profile_read(ctx, cls):
    ms, n = C.c_double(), C.c_int32()
    _check(load().dg_profile_read(ctx, cls, C.byref(ms), C.byref(n)))
    return ms.value, n.value
