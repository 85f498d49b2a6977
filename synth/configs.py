"""Workload registry: the five synthetic denoise-step workloads (shapes and run parameters only).

Nothing here computes any part of the method; it only names sizes, dtypes and schedule ids that
both the HIP path and the oracle read.  The architecture facts (30 layers, sliding window 1024,
128 experts top-8 plus one shared expert, 262k vocabulary, 256-token canvas) come from the spec
section of "DiffusionGemma 완전분석" (cell-devlog) and the parameter table in the technical-report
summary ("DiffusionGemma Technical Report 정리", section 아키텍처와 블록 자기회귀 생성).  The
per-layer widths (d_model 2816, 16/8 heads x 256, expert hidden 704, shared hidden 2112) are
assumed shapes: with them the parameter table's totals come out right (checked by a test).
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

# schedule ids, same numbering as dg_schedule in include/dg.h
KAPPA_LINEAR = 0      # kappa_t = 1 - t
KAPPA_QUADRATIC = 1   # kappa_t = 1 - t^2
KAPPA_COSINE = 2      # kappa_t = cos(pi t / 2)

F32, BF16, FP8, MXFP4 = "f32", "bf16", "fp8", "mxfp4"


@dataclass(frozen=True)
class Workload:
    name: str
    # model shape
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_experts: int
    top_k: int
    expert_hidden: int
    shared_hidden: int
    vocab: int
    window: int            # <= 0: every layer global
    global_every: int      # layer l (0-based) is global iff (l+1) % global_every == 0; 0: all global
    act_dtype: str         # "f32" | "bf16": activations, attention and embedding storage
    expert_dtype: str      # "f32" | "bf16" | "fp8" | "mxfp4": routed and shared expert weights
    # inputs
    batch: int
    canvas: int
    prefix: int
    kv_source: str         # "prefill": encode random prefix tokens; "random": N(0,1) caches
    resid_input: bool      # True: the layer stack starts from an N(0,1) residual (no embedding, no LM head)
    zipf: float            # >0: router bias ln p_e with p_e ~ rank^-zipf over a seeded permutation
    # run
    steps: int             # Euler steps (cap when adaptive)
    schedule: int
    lock_threshold: float
    tau: float
    adaptive: bool
    seed: int = 0
    rope_theta: float = 10000.0
    norm_eps: float = 1e-6
    weight_std: float = 0.02
    sc_hidden: int = 0     # >0: a self-conditioning block of this hidden width (896 at the Gemma-like widths)
    act_quant: str = ""    # "fp8": the expert GEMMs take per-row e4m3 activations (W8A8, with fp8 experts)

    def is_global(self, layer: int) -> bool:
        if self.window <= 0 or self.global_every <= 0:
            return True
        return (layer + 1) % self.global_every == 0

    def kv_cap(self, layer: int) -> int:
        """Slots of the layer's prefix cache: the whole prefix on global layers, a ring of
        `window` slots on local layers."""
        if self.is_global(layer):
            return self.prefix
        return min(self.window, self.prefix) if self.prefix > 0 else 0

    @property
    def qkv_rows(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    @property
    def rows(self) -> int:
        return self.batch * self.canvas

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _gemma_like(**kw):
    base = dict(n_layers=30, d_model=2816, n_q_heads=16, n_kv_heads=8, head_dim=256,
                n_experts=128, top_k=8, expert_hidden=704, shared_hidden=2112, vocab=262144,
                window=1024, global_every=6, act_dtype=BF16, expert_dtype=BF16,
                batch=1, canvas=256, prefix=8192, kv_source="random", resid_input=False, zipf=0.0,
                steps=12, schedule=KAPPA_QUADRATIC, lock_threshold=0.9, tau=1.0, adaptive=False)
    base.update(kw)
    return Workload(**base)


C0 = Workload(name="tiny-fp32", n_layers=2, d_model=256, n_q_heads=4, n_kv_heads=4, head_dim=64,
              n_experts=8, top_k=2, expert_hidden=512, shared_hidden=512, vocab=1024,
              window=0, global_every=0, act_dtype=F32, expert_dtype=F32,
              batch=1, canvas=32, prefix=64, kv_source="prefill", resid_input=False, zipf=0.0,
              steps=4, schedule=KAPPA_LINEAR, lock_threshold=0.9, tau=1.0, adaptive=False)

C1 = _gemma_like(name="layer-bf16-p2048", n_layers=1, window=0, global_every=0, prefix=2048,
                 resid_input=True, steps=1)

C2 = _gemma_like(name="30L-bf16-p8192-canvas256")

C3 = _gemma_like(name="30L-bf16-p131072-canvas256", prefix=131072, steps=1)

C4 = _gemma_like(name="30L-fp8experts-b8-p4096-adaptive", expert_dtype=FP8, batch=8, prefix=4096,
                 zipf=1.1, steps=48, schedule=KAPPA_COSINE, lock_threshold=0.95, adaptive=True)

WORKLOADS = {"C0": C0, "C1": C1, "C2": C2, "C3": C3, "C4": C4}


def get(name: str) -> Workload:
    return WORKLOADS[name]
