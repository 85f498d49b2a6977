"""Seeded synthetic inputs shared by the HIP path's tests/bench and by the oracle.

This module holds no step of the method: it draws random weights, caches, tokens and residuals
of the workloads' shapes and stores them in the storage formats the library reads (fp32, bf16,
fp8 e4m3 with per-output-row bf16 scales, or OCP MXFP4: e2m1 codes with one e8m0 power-of-two
scale per 32 consecutive K-elements).  torch is used as a random-number and dtype plumbing
library only; the same call on the same device returns the same tensors.

Layouts (row-major; every weight matrix is [out][in] so both GEMM operands are K-contiguous):
  embed      [V][d]                 tied input embedding and LM head
  attn_norm, ffn_norm, final_norm   [d]  RMSNorm gains (ones at init)
  w_qkv      [(Hq+2Hkv)*dh][d]      rows: q heads, then k heads, then v heads; dh rows per head
  w_o        [d][Hq*dh]
  w_router   [E][d], router_bias [E] fp32 (None unless the workload sets a Zipf prior)
  w_gate, w_up [E][f][d]; w_down [E][d][f]; sh_gate, sh_up [fs][d]; sh_down [d][fs]
  fp8 only:  s_gate, s_up [E][f]; s_down [E][d]; sh_s_gate, sh_s_up [fs]; sh_s_down [d]  (bf16)
  mxfp4:     expert matrices as codes uint8 [..][N][K/2] (element 2j in the low nibble of byte j)
             with scales uint8 [..][N][K/32] (e8m0: 2^(s - 127)) under the same s_* names
  kv         per layer K and V [B][Hkv][cap][dh]
  self-conditioning (sc_hidden > 0): embed_t [d][V] (embed transposed), sc_gate, sc_up [f][d],
             sc_down [d][f] in the activation dtype
"""
from __future__ import annotations

import hashlib
import math

import numpy as np
import torch

from .configs import Workload, F32, BF16, FP8, MXFP4

FP8_MAX = 448.0
MX_BLOCK = 32          # elements sharing one scale (OCP MX)
E2M1_EMAX = 2          # exponent of the largest e2m1 magnitude, 6 = 1.5 * 2^2


def tensor_seed(seed: int, name: str) -> int:
    h = hashlib.sha256(f"{seed}:{name}".encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(device, seed, name):
    g = torch.Generator(device=device)
    g.manual_seed(tensor_seed(seed, name))
    return g


def normal(shape, std, seed, name, device="cpu") -> torch.Tensor:
    """fp32 N(0, std^2) draw, reproducible per (seed, name, device type)."""
    t = torch.randn(*shape, generator=_gen(device, seed, name), device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t


def uniform_tokens(shape, vocab, seed, name, device="cpu") -> torch.Tensor:
    return torch.randint(0, vocab, tuple(shape), generator=_gen(device, seed, name),
                         device=device, dtype=torch.int32)


def store_act(t: torch.Tensor, dtype: str) -> torch.Tensor:
    """fp32 draw -> storage dtype (torch's round-to-nearest-even cast for bf16)."""
    if dtype == F32:
        return t.contiguous()
    if dtype == BF16:
        return t.to(torch.bfloat16).contiguous()
    raise ValueError(dtype)


def fp8_rows(w: torch.Tensor):
    """Per-output-row e4m3 storage of an fp32 [..., N, K] matrix.

    scale[n] = bf16(max_k |w[n,k]| / 448); code = e4m3(w / scale), saturated at +-448, round to
    nearest even (torch's float8_e4m3fn cast).  Returns (codes as uint8, scales as bf16)."""
    amax = w.abs().amax(dim=-1)
    scale = (amax / FP8_MAX).clamp_min(2.0 ** -126).to(torch.bfloat16)
    q = (w / scale.float().unsqueeze(-1)).clamp(-FP8_MAX, FP8_MAX)
    codes = q.to(torch.float8_e4m3fn).view(torch.uint8).contiguous()
    return codes, scale.contiguous()


def mxfp4_rows(w: torch.Tensor):
    """OCP MX "MXFP4" storage of an fp32 [..., N, K] matrix, K a multiple of 32.

    Per block of 32 consecutive K-elements: X = floor(log2(max |w|)) - 2 (the largest e2m1
    exponent), clamped to [-127, 127] (-127 for an all-zero block), stored as the e8m0 byte X + 127;
    each element is the e2m1 code of w / 2^X rounded to nearest, ties to even, magnitudes above 6
    saturated to 6 (the format's conversion rule).  Codes pack two per byte, element 2j in the low
    nibble.  Returns (codes uint8 [..., N, K/2], scales uint8 [..., N, K/32])."""
    *lead, K = w.shape
    assert K % MX_BLOCK == 0
    blk = w.reshape(*lead, K // MX_BLOCK, MX_BLOCK)
    amax = blk.abs().amax(dim=-1)
    _, ex = torch.frexp(amax)                         # amax = m 2^ex, m in [0.5, 1): floor(log2) = ex - 1
    X = (ex.to(torch.int32) - 1 - E2M1_EMAX).clamp(-127, 127)
    X = torch.where(amax > 0, X, torch.full_like(X, -127))
    y = blk * torch.exp2(-X.to(torch.float32)).unsqueeze(-1)   # power-of-two scaling: exact
    a = y.abs().clamp(max=6.0)
    # e2m1 magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6 (codes 0..7); a tie goes to the even code
    mag = ((a > 0.25).int() + (a >= 0.75).int() + (a > 1.25).int() + (a >= 1.75).int()
           + (a > 2.5).int() + (a >= 3.5).int() + (a > 5.0).int())
    code = (mag | torch.where(y < 0, 8, 0)).to(torch.uint8).reshape(*lead, K)
    pairs = code.reshape(*lead, K // 2, 2)
    packed = (pairs[..., 0] | (pairs[..., 1] << 4)).to(torch.uint8).contiguous()
    return packed, (X + 127).to(torch.uint8).contiguous()


def zipf_bias(n_experts: int, exponent: float, seed: int) -> torch.Tensor:
    """ln p_e with p_e proportional to rank^-exponent, ranks assigned by a seeded permutation."""
    rng = np.random.default_rng(tensor_seed(seed, "zipf-perm") & 0xFFFFFFFF)
    rank = rng.permutation(n_experts) + 1
    p = rank.astype(np.float64) ** (-exponent)
    p /= p.sum()
    return torch.from_numpy(np.log(p).astype(np.float32))


def _expert_store(w32: torch.Tensor, cfg: Workload, out: dict, key: str, skey: str):
    if cfg.expert_dtype == FP8:
        codes, scale = fp8_rows(w32)
        out[key] = codes
        out[skey] = scale
    elif cfg.expert_dtype == MXFP4:
        codes, scale = mxfp4_rows(w32)
        out[key] = codes
        out[skey] = scale
    else:
        out[key] = store_act(w32, cfg.expert_dtype)
        out[skey] = None


def make_layer(cfg: Workload, layer: int, device="cpu") -> dict:
    s, std, d = cfg.seed, cfg.weight_std, cfg.d_model
    E, f, fs = cfg.n_experts, cfg.expert_hidden, cfg.shared_hidden
    act = cfg.act_dtype
    nm = lambda k: f"layer{layer}.{k}"
    L = {}
    L["attn_norm"] = store_act(torch.ones(d, device=device), act)
    L["ffn_norm"] = store_act(torch.ones(d, device=device), act)
    L["w_qkv"] = store_act(normal((cfg.qkv_rows, d), std, s, nm("w_qkv"), device), act)
    L["w_o"] = store_act(normal((d, cfg.n_q_heads * cfg.head_dim), std, s, nm("w_o"), device), act)
    L["w_router"] = store_act(normal((E, d), std, s, nm("w_router"), device), act)
    L["router_bias"] = zipf_bias(E, cfg.zipf, s).to(device) if cfg.zipf > 0 else None
    _expert_store(normal((E, f, d), std, s, nm("w_gate"), device), cfg, L, "w_gate", "s_gate")
    _expert_store(normal((E, f, d), std, s, nm("w_up"), device), cfg, L, "w_up", "s_up")
    _expert_store(normal((E, d, f), std, s, nm("w_down"), device), cfg, L, "w_down", "s_down")
    _expert_store(normal((fs, d), std, s, nm("sh_gate"), device), cfg, L, "sh_gate", "sh_s_gate")
    _expert_store(normal((fs, d), std, s, nm("sh_up"), device), cfg, L, "sh_up", "sh_s_up")
    _expert_store(normal((d, fs), std, s, nm("sh_down"), device), cfg, L, "sh_down", "sh_s_down")
    return L


def make_weights(cfg: Workload, device="cpu") -> dict:
    W = {"layers": [make_layer(cfg, l, device) for l in range(cfg.n_layers)]}
    W["final_norm"] = store_act(torch.ones(cfg.d_model, device=device), cfg.act_dtype)
    if cfg.resid_input:
        W["embed"] = None
    else:
        W["embed"] = store_act(normal((cfg.vocab, cfg.d_model), cfg.weight_std, cfg.seed, "embed",
                                      device), cfg.act_dtype)
    if cfg.sc_hidden > 0:
        # the self-conditioning block: the embedding transposed ([d][V], the same values) and a
        # gated feed-forward block d -> sc_hidden -> d in the activation dtype
        W["embed_t"] = W["embed"].t().contiguous()
        f, d = cfg.sc_hidden, cfg.d_model
        W["sc_gate"] = store_act(normal((f, d), cfg.weight_std, cfg.seed, "sc.gate", device), cfg.act_dtype)
        W["sc_up"] = store_act(normal((f, d), cfg.weight_std, cfg.seed, "sc.up", device), cfg.act_dtype)
        W["sc_down"] = store_act(normal((d, f), cfg.weight_std, cfg.seed, "sc.down", device), cfg.act_dtype)
    return W


def make_random_kv(cfg: Workload, device="cpu") -> list:
    """N(0,1) caches: per layer (K, V), each [B][Hkv][cap][dh] in the activation dtype.
    Random keys count as already rotated (post-RoPE)."""
    out = []
    for l in range(cfg.n_layers):
        cap = cfg.kv_cap(l)
        shp = (cfg.batch, cfg.n_kv_heads, cap, cfg.head_dim)
        k = store_act(normal(shp, 1.0, cfg.seed, f"layer{l}.K", device), cfg.act_dtype)
        v = store_act(normal(shp, 1.0, cfg.seed, f"layer{l}.V", device), cfg.act_dtype)
        out.append((k, v))
    return out


def empty_kv(cfg: Workload, device="cpu") -> list:
    """Zero caches of the workload's capacities (to be filled by prefill)."""
    dt = torch.float32 if cfg.act_dtype == F32 else torch.bfloat16
    out = []
    for l in range(cfg.n_layers):
        shp = (cfg.batch, cfg.n_kv_heads, cfg.kv_cap(l), cfg.head_dim)
        out.append((torch.zeros(shp, dtype=dt, device=device), torch.zeros(shp, dtype=dt, device=device)))
    return out


def prefix_tokens(cfg: Workload, device="cpu") -> torch.Tensor:
    return uniform_tokens((cfg.batch, cfg.prefix), cfg.vocab, cfg.seed, "prefix-tokens", device)


def resid_input(cfg: Workload, device="cpu") -> torch.Tensor:
    """N(0,1) residual stream input [B*L][d] fp32, holding bf16-representable values in bf16 mode."""
    r = normal((cfg.rows, cfg.d_model), 1.0, cfg.seed, "resid-in", device)
    if cfg.act_dtype == BF16:
        r = r.to(torch.bfloat16).float()
    return r.contiguous()


def hidden_input(cfg: Workload, device="cpu", scale: float = 1.0) -> torch.Tensor:
    """Final-normed hidden states [B*L][d] for sampler-only tests: rows of N(0,1)*scale."""
    return store_act(normal((cfg.rows, cfg.d_model), scale, cfg.seed, "hidden", device), cfg.act_dtype)


def bf16_bits_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def to_numpy_f64(t: torch.Tensor) -> np.ndarray:
    """Storage tensor -> float64 numpy (bf16/fp32 exactly; fp8 / mxfp4 codes and scales stay uint8)."""
    if t.dtype == torch.uint8:
        return t.cpu().numpy()
    return t.float().cpu().numpy().astype(np.float64)
