"""Storage-format arithmetic for the oracle (test infrastructure only).

bf16 is IEEE binary32 truncated to 8 significant bits (1 sign, 8 exponent, 7 stored mantissa
bits); rounding to it is round-to-nearest, ties to even.  e4m3 is the OCP 8-bit float format
"E4M3FN": 1 sign, 4 exponent (bias 7) and 3 mantissa bits, no infinities, the all-ones
exponent-and-mantissa pattern is NaN, largest finite value 448.
"""
from __future__ import annotations

import numpy as np

BF16_MIN_NORMAL_EXP = -126
BF16_MANT_BITS = 7


def round_bf16(x):
    """Nearest bf16 value (ties to even) of float64 x, returned as float64.

    For finite x with |x| in [2^e, 2^(e+1)) the bf16 spacing is 2^(e-7), and never below the
    subnormal spacing 2^-133."""
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    fin = np.isfinite(x) & (x != 0)
    if not np.any(fin):
        return out
    _, ex = np.frexp(x[fin])              # x = m * 2^ex, |m| in [0.5, 1)  ->  e = ex - 1
    e = np.maximum(ex - 1, BF16_MIN_NORMAL_EXP)
    ulp = np.ldexp(1.0, e - BF16_MANT_BITS)
    out[fin] = np.round(x[fin] / ulp) * ulp   # np.round: half to even; scaling by 2^k is exact
    big = np.abs(out) > 3.3895313892515355e38
    out[big] = np.sign(out[big]) * np.inf
    return out


def identity(x):
    return np.asarray(x, dtype=np.float64)


def rounder(act_dtype: str):
    """Storage rounding of activations: bf16 mode rounds at the storage points, fp32 mode is exact
    to within the oracle's float64 (the HIP path computes fp32 there)."""
    return round_bf16 if act_dtype == "bf16" else identity


def e4m3_decode_table():
    """Value of each of the 256 e4m3 codes, from the format definition."""
    tab = np.zeros(256, dtype=np.float64)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            tab[code] = np.nan
        elif e == 0:
            tab[code] = s * (m / 8.0) * 2.0 ** (1 - 7)
        else:
            tab[code] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return tab


_E4M3 = e4m3_decode_table()


def dequant_rows(codes, scales):
    """fp8 weight [..., N, K] codes + per-row scale [..., N] -> float64 values q * s."""
    return _E4M3[np.asarray(codes, dtype=np.uint8)] * np.asarray(scales, dtype=np.float64)[..., None]
