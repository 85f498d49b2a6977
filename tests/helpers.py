"""Test plumbing: turn the seeded storage tensors of `synth` into the oracle's float64 arrays."""
from oracle.model import layer_arrays
from synth.host import layer_np, np64  # noqa: F401  (re-exported for the tests)


def oracle_layer(L: dict, cfg) -> dict:
    return layer_arrays(layer_np(L), cfg.expert_dtype)


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
