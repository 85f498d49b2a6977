"""Test plumbing: turn the seeded storage tensors of `synth` into the oracle's float64 arrays."""
import numpy as np
import torch

from oracle.model import layer_arrays


def np64(t):
    if t is None:
        return None
    if t.dtype == torch.uint8:
        return t.cpu().numpy()
    return t.float().cpu().numpy().astype(np.float64)


def oracle_layer(L: dict, cfg) -> dict:
    raw = {k: np64(v) for k, v in L.items()}
    return layer_arrays(raw, cfg.expert_dtype)


def oracle_weights(W: dict, cfg, layers=None) -> dict:
    ls = range(cfg.n_layers) if layers is None else layers
    return {"embed": np64(W["embed"]), "final_norm": np64(W["final_norm"]),
            "layers": [oracle_layer(W["layers"][l], cfg) for l in ls]}


def oracle_kv(kv) -> list:
    """(K, V) tensors with V [B][Hkv][cap][dh] -> float64 arrays."""
    return [(np64(k), np64(v)) for k, v in kv]


def oracle_kv_dev(kv) -> list:
    """The library's cache layout (V d-major [B][Hkv][dh][cap]) -> float64 arrays of the oracle's."""
    return [(np64(k), np64(v.transpose(-1, -2))) for k, v in kv]
