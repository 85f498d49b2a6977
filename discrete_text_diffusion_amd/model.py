"""Marshalling helpers: build the C structs of dg.h from torch tensors and keep them alive.

`Model` wraps one dg_ctx plus the prefix KV cache description; its methods call the
same-named C entry points.  Any object with the model-shape attributes (n_layers, d_model, ...,
act_dtype "f32"/"bf16", expert_dtype "f32"/"bf16"/"fp8"/"mxfp4") describes the model.
"""
from __future__ import annotations

import ctypes as C

import torch

from . import dg

_DT = {"f32": dg.DG_F32, "bf16": dg.DG_BF16, "fp8": dg.DG_FP8E4M3, "mxfp4": dg.DG_MXFP4}


def model_desc(cfg) -> dg.ModelDesc:
    return dg.ModelDesc(n_layers=cfg.n_layers, d_model=cfg.d_model, n_q_heads=cfg.n_q_heads,
                        n_kv_heads=cfg.n_kv_heads, head_dim=cfg.head_dim, n_experts=cfg.n_experts,
                        top_k=cfg.top_k, expert_hidden=cfg.expert_hidden, shared_hidden=cfg.shared_hidden,
                        vocab=cfg.vocab, window=cfg.window, global_every=cfg.global_every,
                        rope_theta=cfg.rope_theta, norm_eps=cfg.norm_eps, act_dtype=_DT[cfg.act_dtype],
                        expert_dtype=_DT[cfg.expert_dtype], sc_hidden=getattr(cfg, "sc_hidden", 0),
                        expert_act_fp8=int(getattr(cfg, "act_quant", "") == "fp8"))


def _p(t):
    return None if t is None else t.data_ptr()


def values_dmajor(kv: list) -> list:
    """Per layer (K, V) with V [B][Hkv][cap][dh] -> (K, V) with V d-major [B][Hkv][dh][cap],
    the value layout that dg_kv takes."""
    return [(k, v.transpose(-1, -2).contiguous()) for k, v in kv]


def values_rowmajor(kv: list) -> list:
    """Inverse of values_dmajor (views, no copy)."""
    return [(k, v.transpose(-1, -2)) for k, v in kv]


class Model:
    def __init__(self, cfg, weights: dict, kv: list | None = None, prefix_len=None):
        self.cfg = cfg
        self._keep = [weights]
        self.desc = model_desc(cfg)
        n = cfg.n_layers
        self._layers = (dg.LayerWeights * n)()
        for l, L in enumerate(weights["layers"]):
            for f in dg.LAYER_FIELDS:
                setattr(self._layers[l], f, _p(L.get(f)))
        self.weights = dg.Weights(embed=_p(weights.get("embed")), final_norm=_p(weights["final_norm"]),
                                  layers=C.cast(self._layers, C.POINTER(dg.LayerWeights)),
                                  embed_t=_p(weights.get("embed_t")), sc_gate=_p(weights.get("sc_gate")),
                                  sc_up=_p(weights.get("sc_up")), sc_down=_p(weights.get("sc_down")))
        self.ctx = dg.dg_create(self.desc, self.weights)
        self.kv_struct = None
        if kv is not None:
            self.set_kv(kv, prefix_len)

    def set_kv(self, kv: list, prefix_len, max_prefix=None):
        """kv: per layer (K [B][Hkv][cap][dh], V [B][Hkv][dh][cap]) tensors (see values_dmajor);
        prefix_len: ints [B] (copied to a device int32 tensor, `plen_dev`, which the library reads
        and advances); max_prefix: the host bound passed with every call (default max(prefix_len))."""
        self._kv = kv
        n = self.cfg.n_layers
        self._kp = (C.c_void_p * n)(*[k.data_ptr() for k, _ in kv])
        self._vp = (C.c_void_p * n)(*[v.data_ptr() for _, v in kv])
        self._cap = (C.c_int32 * n)(*[k.shape[2] for k, _ in kv])
        self.batch = kv[0][0].shape[0]
        plen = [int(p) for p in prefix_len]
        self.plen_dev = torch.tensor(plen, dtype=torch.int32, device=kv[0][0].device)
        self._plen_host = plen
        bound = max(plen) if max_prefix is None else int(max_prefix)
        self.kv_struct = dg.KV(k=self._kp, v=self._vp, cap=self._cap, prefix_len=self.plen_dev.data_ptr(),
                               max_prefix=bound, batch=self.batch)

    @property
    def max_prefix(self):
        return self.kv_struct.max_prefix

    @property
    def prefix_len(self):
        """Host copy of the prefix lengths; read back from the device (a synchronisation) after a
        pass whose appends were decided there."""
        if self._plen_host is None:
            self._plen_host = [int(x) for x in self.plen_dev.cpu().tolist()]
        return list(self._plen_host)

    def _grew(self, n, known=True):
        self.kv_struct.max_prefix += n
        if known and self._plen_host is not None:
            self._plen_host = [p + n for p in self._plen_host]
        else:
            self._plen_host = None

    def workspace(self, batch, rows_per_canvas, max_prefix=0, device="cuda"):
        nbytes = dg.dg_workspace_bytes(self.ctx, batch, rows_per_canvas, max_prefix)
        ws = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
        off = (-ws.data_ptr()) % 256
        ws = ws[off:off + nbytes]
        dg.dg_clear_status(self.ctx, ws)
        return ws

    # ---- calls -----------------------------------------------------------------------------
    def prefill_kv(self, tokens, ws, stream=None):
        dg.dg_prefill_kv(self.ctx, self.kv_struct, tokens, tokens.shape[1], ws, stream)
        self._grew(tokens.shape[1])

    def denoise_step(self, canvas, L, ws, hidden_out=None, resid_out=None, resid_in=None, layer_begin=0,
                     layer_end=None, stream=None, sc_in=None):
        le = self.cfg.n_layers if layer_end is None else layer_end
        dg.dg_denoise_step(self.ctx, self.kv_struct, canvas, resid_in, L, layer_begin, le, hidden_out, resid_out,
                           ws, stream, sc_in)

    def mixed_forward(self, tokens, append, hidden_out, ws, stream=None, resid_out=None):
        """One pass over canvases of two kinds: append[b] != 0 (device int32 [B]) encodes canvas b
        causally into the cache (its device prefix length grows by L), the others take the
        bidirectional denoising pass."""
        dg.dg_mixed_forward(self.ctx, self.kv_struct, tokens, append, tokens.shape[1], hidden_out, ws, stream,
                            resid_out)
        self._grew(tokens.shape[1], known=False)

    def step_sample(self, hidden, canvas, lock, n_locked, params: dg.StepParams, ws, done=None, stream=None,
                    sc_out=None):
        B, L = canvas.shape
        dg.dg_step_sample(self.ctx, hidden, canvas, lock, n_locked, done, B, L, params, ws, stream, sc_out)

    def canvas_run(self, canvas, lock, steps_taken, params: dg.RunParams, ws, stream=None):
        dg.dg_canvas_run(self.ctx, self.kv_struct, canvas, lock, steps_taken, canvas.shape[1], params, ws, stream)

    def generate(self, out, steps, valid, eos_seen, eos_id, params: dg.RunParams, ws, stream=None):
        """Block-AR generation into out [K][B][L] after the encoded prompt; the prefix then
        covers the K - 1 appended canvases."""
        K, _, L = out.shape
        dg.dg_generate(self.ctx, self.kv_struct, out, steps, valid, eos_seen, K, L, eos_id, params, ws, stream)
        self._grew((K - 1) * L)

    def generate_continuous(self, out, steps, valid, eos_seen, passes, eos_id, params: dg.RunParams, ws,
                            stream=None):
        """Block-AR generation with every sequence on its own schedule (stopped canvases appended in
        the next mixed pass while others keep denoising); `passes` receives the passes that ran."""
        K, _, L = out.shape
        dg.dg_generate_continuous(self.ctx, self.kv_struct, out, steps, valid, eos_seen, passes, K, L, eos_id,
                                  params, ws, stream)
        self._grew((K - 1) * L)

    def close(self):
        if self.ctx:
            dg.dg_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
