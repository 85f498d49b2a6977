"""Storage-format arithmetic for the oracle (test infrastructure only).

bf16 is IEEE binary32 truncated to 8 significant bits (1 sign, 8 exponent, 7 stored mantissa
bits); rounding to it is round-to-nearest, ties to even.  e4m3 is the OCP 8-bit float format
"E4M3FN": 1 sign, 4 exponent (bias 7) and 3 mantissa bits, no infinities, the all-ones
exponent-and-mantissa pattern is NaN, largest finite value 448.  MXFP4 is the OCP microscaling
format: e2m1 elements (1 sign, 2 exponent bits with bias 1, 1 mantissa bit; largest magnitude 6)
in blocks of 32 sharing one e8m0 scale (an 8-bit biased exponent, value 2^(s - 127)).
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


E4M3_MAX = 448.0


def round_e4m3(x):
    """Nearest e4m3 value (ties to even) of float64 x, saturating at +-448.

    For |x| in [2^e, 2^(e+1)) with e >= -6 the spacing is 2^(e-3); below 2^-6 (subnormals) it is
    2^-9.  Ties to even: np.round halves to even, and scaling by a power of two is exact."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    out = np.zeros_like(a)
    nz = a > 0
    _, ex = np.frexp(a[nz])                  # a = m * 2^ex, m in [0.5, 1)  ->  e = ex - 1
    e = np.maximum(ex - 1, -6)
    ulp = np.ldexp(1.0, e - 3)
    out[nz] = np.minimum(np.round(a[nz] / ulp) * ulp, E4M3_MAX)
    return np.sign(x) * out


def quant_rows_e4m3(x):
    """Per-row dynamic e4m3 quantisation of activations x [..., K] (bf16-valued float64): the row's
    scale s = fp32(max|x|) / 448 in float32, and its reciprocal r = 448 / fp32(max|x|) (one IEEE
    float32 division per row); each element is coded as the nearest e4m3 value of the float32
    product fp32(x) * r (the decision the kernels take in float32); an all-zero row has s = r = 1.
    Returns (dequantised values q * s as float64, s as float64)."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    amax = np.max(np.abs(x32), axis=-1, keepdims=True)
    pos = amax > 0
    safe = np.where(pos, amax, np.float32(1.0)).astype(np.float32)
    s = np.where(pos, safe / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    r = np.where(pos, np.float32(E4M3_MAX) / safe, np.float32(1.0)).astype(np.float32)
    q = round_e4m3((x32 * r).astype(np.float64))
    return q * s.astype(np.float64), s[..., 0].astype(np.float64)


def e2m1_decode_table():
    """Value of each of the 16 e2m1 codes, from the format definition: exponent field 0 is
    subnormal (m / 2), otherwise (1 + m / 2) * 2^(e - 1)."""
    tab = np.zeros(16, dtype=np.float64)
    for code in range(16):
        s = -1.0 if code & 0x8 else 1.0
        e = (code >> 1) & 0x3
        m = code & 0x1
        tab[code] = s * (m / 2.0 if e == 0 else (1.0 + m / 2.0) * 2.0 ** (e - 1))
    return tab


_E2M1 = e2m1_decode_table()
MX_BLOCK = 32


def mxfp4_dequant(codes, scales):
    """MXFP4 weight -> float64 [..., N, K]: codes uint8 [..., N, K/2] with element 2j in the low
    nibble of byte j, scales uint8 [..., N, K/32] (e8m0, 2^(s - 127); 255 would be NaN)."""
    c = np.asarray(codes, dtype=np.uint8)
    s = np.asarray(scales, dtype=np.uint8)
    el = np.stack([c & 0xF, c >> 4], axis=-1).reshape(*c.shape[:-1], c.shape[-1] * 2)
    val = _E2M1[el]
    sc = np.where(s == 255, np.nan, np.ldexp(1.0, s.astype(np.int64) - 127))
    return val * np.repeat(sc, MX_BLOCK, axis=-1)
