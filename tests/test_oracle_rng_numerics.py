"""Pins of the oracle's random draws and storage formats (CPU).

Philox has no known-answer vectors available here, so its words are pinned by what any correct
implementation must show: uniform words, balanced bits, avalanche on a one-bit counter change,
and the exact distributions of the converters built on top of it.  bf16 rounding and the e4m3
table are pinned against independent library conversions (torch) and the format's definition;
the MXFP4 decode against the values the OCP microscaling specification lists for e2m1 and
hand-packed blocks, and the MXFP4 storage conversion by exact round trips and its tie rule.
"""
import math

import numpy as np
import pytest
import scipy.stats as st
import torch

from oracle import philox
from oracle.numerics import round_bf16, e4m3_decode_table, dequant_rows, e2m1_decode_table, mxfp4_dequant
from synth.gen import mxfp4_rows


def _words(n, seed=123, tag=0):
    c = np.arange(n)
    return philox.word(seed, c >> 2, 7, 3, tag, c & 3)


def test_philox_uniform_words():
    w = _words(1 << 18)
    counts = np.bincount((w >> np.uint64(24)).astype(np.int64), minlength=256)
    chi2 = ((counts - counts.mean()) ** 2 / counts.mean()).sum()
    assert st.chi2.sf(chi2, 255) > 1e-4


def test_philox_bit_balance_and_avalanche():
    w = _words(1 << 16)
    bits = ((w[:, None] >> np.arange(32, dtype=np.uint64)[None, :]) & np.uint64(1)).astype(np.float64)
    p = bits.mean(axis=0)
    sigma = math.sqrt(0.25 / len(w))
    assert np.all(np.abs(p - 0.5) < 5 * sigma)
    # flip each of the 128 counter bits in turn: about half the output bits change
    rng = np.random.default_rng(5)
    ctr = rng.integers(0, 1 << 32, size=(256, 4), dtype=np.uint64)
    base = philox.philox4x32_10(ctr, (11, 22))
    flips = []
    for bit in range(128):
        c2 = ctr.copy()
        c2[:, bit // 32] ^= np.uint64(1 << (bit % 32))
        d = philox.philox4x32_10(c2, (11, 22)) ^ base
        flips.append(np.mean([bin(int(x)).count("1") for x in d.reshape(-1)]))
    assert 15.0 < np.mean(flips) < 17.0
    assert min(flips) > 13.0


def test_philox_key_changes_stream():
    c = np.arange(4096)
    a = philox.word(1, c, 0, 0, 0, 0)
    b = philox.word(2, c, 0, 0, 0, 0)
    assert np.mean(a == b) < 1e-3
    # the 64-bit seed uses both key words
    a2 = philox.word(1 + (1 << 32), c, 0, 0, 0, 0)
    assert np.mean(a == a2) < 1e-3


def test_converters_exact_ranges():
    w = np.array([0, 0xFF, 0x100, 0xFFFFFFFF], dtype=np.uint64)
    u = philox.unit_open_closed(w)
    assert u[0] == 0.0 and u[1] == 0.0 and u[2] == 2.0 ** -24 and u[3] == 1.0 - 2.0 ** -24
    uo = philox.unit_open(w)
    assert uo[0] == 2.0 ** -24 and uo[3] == 1.0 - 2.0 ** -24
    assert np.all(np.float32(uo) == uo)          # exact in float32
    assert philox.token(np.array([0xFFFFFFFF], np.uint64), 1024)[0] == 1023
    assert philox.token(np.array([0x003FFFFF], np.uint64), 1024)[0] == 0
    assert philox.token(np.array([0x80000000], np.uint64), 1000)[0] == 500


def test_gumbel_moments_and_cdf():
    g = philox.gumbel(_words(1 << 18, seed=9))
    assert abs(g.mean() - 0.5772156649) < 5 * math.sqrt(math.pi ** 2 / 6 / len(g))
    assert abs(g.var() - math.pi ** 2 / 6) < 0.03
    ks = st.kstest(g, st.gumbel_r.cdf)
    assert ks.pvalue > 1e-4


def test_token_uniform_chi2():
    for V in (1024, 1000):
        t = philox.token(_words(1 << 18, seed=3), V)
        counts = np.bincount(t, minlength=V)
        chi2 = ((counts - counts.mean()) ** 2 / counts.mean()).sum()
        assert st.chi2.sf(chi2, V - 1) > 1e-4


def test_streams_are_distinct():
    B, L = 2, 64
    b, i = np.meshgrid(np.arange(B), np.arange(L), indexing="ij")
    ju = philox.jump_uniform(0, 0, b, i)
    init = philox.init_tokens(0, B, L, 1 << 20)
    assert len(np.unique(ju)) == B * L
    assert len(np.unique(init)) > B * L - 5


# ---- bf16 ------------------------------------------------------------------------------------

def test_round_bf16_matches_torch_on_float32_values():
    rng = np.random.default_rng(0)
    x32 = np.concatenate([rng.standard_normal(100000) * 10.0 ** rng.integers(-30, 30, 100000),
                          rng.standard_normal(1000) * 1e-39]).astype(np.float32)
    # exact ties: bf16 value + half an ulp
    base = torch.randn(1000).to(torch.bfloat16).float().numpy()
    ulp = np.ldexp(np.float32(1), (np.frexp(base)[1] - 1 - 7).astype(np.int32)).astype(np.float32)
    ties = (base + ulp / 2).astype(np.float32)
    x32 = np.concatenate([x32, ties])
    ref = torch.from_numpy(x32).to(torch.bfloat16).float().numpy().astype(np.float64)
    got = round_bf16(x32.astype(np.float64))
    assert np.array_equal(got, ref)


def test_round_bf16_is_nearest():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(2000) * 3
    r = round_bf16(x)
    for xi, ri in zip(x[:200], r[:200]):
        e = math.floor(math.log2(abs(xi)))
        ulp = 2.0 ** (e - 7)
        assert abs(ri - xi) <= ulp / 2 + 1e-300
        assert ri / ulp == round(ri / ulp)


# ---- e4m3 ------------------------------------------------------------------------------------

def test_e4m3_table_definition_points():
    t = e4m3_decode_table()
    assert t[0x38] == 1.0
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert math.isnan(t[0x7F]) and math.isnan(t[0xFF])
    assert t[0x08] == 2.0 ** -6                     # smallest normal
    assert t[0x01] == 2.0 ** -9                     # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9
    assert t[0x00] == 0.0 and t[0x80] == 0.0
    fin = t[np.isfinite(t)]
    assert fin.max() == 448.0 and len(fin) == 254


def test_e4m3_table_matches_torch_float8():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    t = e4m3_decode_table()
    nan = np.isnan(t)
    assert np.array_equal(nan, np.isnan(ref))
    assert np.array_equal(t[~nan], ref[~nan])


def test_dequant_rows():
    codes = np.array([[0x38, 0x40], [0xB8, 0x00]], dtype=np.uint8)   # 1, 2 / -1, 0
    s = np.array([0.5, 4.0])
    assert np.array_equal(dequant_rows(codes, s), np.array([[0.5, 1.0], [-4.0, 0.0]]))


# ---- MXFP4 (OCP microscaling: e2m1 elements, e8m0 scale per 32) --------------------------------

def test_e2m1_table_lists_the_format_values():
    # the eight magnitudes of FP4 E2M1 as listed by the OCP MX specification; codes 8..15 negate
    t = e2m1_decode_table()
    assert list(t[:8]) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert list(t[8:]) == [-0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]


def test_mxfp4_dequant_hand_packed():
    # one row of 64 elements = 2 blocks; byte j holds element 2j (low nibble) and 2j + 1 (high)
    codes = np.zeros((1, 32), dtype=np.uint8)
    codes[0, 0] = 0x72          # element 0 = code 2 (1.0), element 1 = code 7 (6.0)
    codes[0, 15] = 0x9F         # element 30 = code 15 (-6), element 31 = code 9 (-0.5)
    codes[0, 16] = 0x01         # element 32 = code 1 (0.5), first element of block 1
    scales = np.array([[126, 130]], dtype=np.uint8)   # 2^-1, 2^3
    w = mxfp4_dequant(codes, scales)
    assert w.shape == (1, 64)
    expect = np.zeros(64)
    expect[0], expect[1], expect[30], expect[31], expect[32] = 0.5, 3.0, -3.0, -0.25, 4.0
    assert np.array_equal(w[0], expect)
    assert math.isnan(mxfp4_dequant(np.zeros((1, 16), np.uint8) + 0x22, np.array([[255]], np.uint8))[0, 0])


def test_mxfp4_storage_exact_blocks_round_trip():
    rng = np.random.default_rng(5)
    grid = e2m1_decode_table()
    for X in (-9, -1, 0, 4):
        idx = rng.integers(0, 16, size=(3, 64))
        idx[:, 0] = 7                                   # each block holds its maximum 6
        idx[:, 32] = 15
        w = np.ldexp(grid[idx], X).astype(np.float32)
        codes, scales = mxfp4_rows(torch.from_numpy(w))
        assert np.array_equal(scales.numpy(), np.full((3, 2), X + 127, np.uint8))
        assert np.array_equal(mxfp4_dequant(codes.numpy(), scales.numpy()), w.astype(np.float64))


def test_mxfp4_storage_ties_saturation_and_zero():
    # block maximum 4 gives X = floor(log2 4) - 2 = 0, so elements are rounded in units of 1
    row = np.zeros(32, np.float32)
    row[:10] = [4.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, -5.0, -0.1, 0.3]
    codes, scales = mxfp4_rows(torch.from_numpy(row[None]))
    assert scales.numpy()[0, 0] == 127
    got = mxfp4_dequant(codes.numpy(), scales.numpy())[0]
    # ties go to the even code: 0.25 -> 0, 0.75 -> 1, 1.25 -> 1, 1.75 -> 2, 2.5 -> 2, 3.5 -> 4, 5 -> 4
    assert list(got[:10]) == [4.0, 0.0, 1.0, 1.0, 2.0, 2.0, 4.0, -4.0, -0.0, 0.5]
    sat = np.zeros(32, np.float32)
    sat[0], sat[1] = 7.9, -7.0                             # X = 0; magnitudes above 6 saturate
    g = mxfp4_dequant(*[t.numpy() for t in mxfp4_rows(torch.from_numpy(sat[None]))])[0]
    assert g[0] == 6.0 and g[1] == -6.0
    zc, zs = mxfp4_rows(torch.zeros(1, 32))
    assert zs.numpy()[0, 0] == 0 and not zc.numpy().any()


def test_mxfp4_storage_error_bound():
    # within a block: half a step of the e2m1 grid below 6 * 2^X, at most 2 * 2^X at saturation
    w = torch.randn(8, 4, 128) * 0.02
    codes, scales = mxfp4_rows(w)
    q = mxfp4_dequant(codes.numpy(), scales.numpy())
    unit = np.repeat(np.ldexp(1.0, scales.numpy().astype(np.int64) - 127), 32, axis=-1)
    err = np.abs(q - w.numpy().astype(np.float64)) / unit
    y = np.abs(w.numpy().astype(np.float64)) / unit
    step = np.where(y < 2, 0.5, np.where(y < 4, 1.0, 2.0))
    assert np.all(err <= np.where(y > 6, y - 6, step / 2) + 1e-12)
    assert np.all(y < 8)
