"""Counter-based random draws of the step — oracle side (test infrastructure only).

Philox4x32-10 as defined by Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as
1, 2, 3" (SC'11): a 128-bit counter (c0, c1, c2, c3) and a 64-bit key (k0, k1); each of the ten
rounds multiplies c0 and c2 by two fixed 32-bit constants, mixes the high halves with the other
two counter words and the round key, and the key is bumped by two Weyl constants between rounds.

Every random number the method draws is one 32-bit word of one Philox block.  Stream layout
(counter words; `tag` goes in the low byte of c3, the canvas index b above it):
    Gumbel noise for logit (b, i, v) at step s   ctr = (v, i >> 2, s, b << 8 | 0), word i & 3
    jump uniform for position (b, i) at step s   ctr = (i >> 2, 0, s, b << 8 | 1), word i & 3
    uniform canvas token at t = 1 for (b, i)     ctr = (i >> 2, 0, 0, b << 8 | 2), word i & 3
    forward-noise keep test (b, i) at step s     ctr = (i >> 2, 0, s, b << 8 | 3), word i & 3
    forward-noise token (b, i) at step s         ctr = (i >> 2, 0, s, b << 8 | 4), word i & 3
    re-noise token of the entropy-bounded step   ctr = (i >> 2, 0, s, b << 8 | 5), word i & 3
key = (seed mod 2^32, seed >> 32).
"""
from __future__ import annotations

import numpy as np

MUL0 = 0xD2511F53
MUL1 = 0xCD9E8D57
WEYL0 = 0x9E3779B9
WEYL1 = 0xBB67AE85
MASK32 = 0xFFFFFFFF

TAG_GUMBEL, TAG_JUMP, TAG_INIT, TAG_NOISE_KEEP, TAG_NOISE_TOKEN, TAG_RENOISE = 0, 1, 2, 3, 4, 5


def philox4x32_10(ctr, key):
    """ctr: integer array [..., 4] (values < 2^32); key: (k0, k1). Returns uint64 array [..., 4]
    holding the four 32-bit output words."""
    c = np.asarray(ctr, dtype=np.uint64) & np.uint64(MASK32)
    c0, c1, c2, c3 = (c[..., j].copy() for j in range(4))
    k0 = np.uint64(int(key[0]) & MASK32)
    k1 = np.uint64(int(key[1]) & MASK32)
    m = np.uint64(MASK32)
    for rnd in range(10):
        if rnd:
            k0 = np.uint64((int(k0) + WEYL0) & MASK32)
            k1 = np.uint64((int(k1) + WEYL1) & MASK32)
        p0 = c0 * np.uint64(MUL0)          # < 2^64: exact in uint64
        p1 = c2 * np.uint64(MUL1)
        hi0, lo0 = p0 >> np.uint64(32), p0 & m
        hi1, lo1 = p1 >> np.uint64(32), p1 & m
        c0, c1, c2, c3 = (hi1 ^ c1 ^ k0), lo1, (hi0 ^ c3 ^ k1), lo0
    return np.stack([c0, c1, c2, c3], axis=-1)


def seed_key(seed: int):
    seed = int(seed)
    return (seed & MASK32, (seed >> 32) & MASK32)


def word(seed, c0, c1, c2, c3, w):
    """Word `w` (0..3) of Philox(key(seed), (c0, c1, c2, c3)); arguments broadcast."""
    c0, c1, c2, c3, w = np.broadcast_arrays(*(np.asarray(x, dtype=np.int64) for x in (c0, c1, c2, c3, w)))
    out = philox4x32_10(np.stack([c0, c1, c2, c3], axis=-1), seed_key(seed))
    return np.take_along_axis(out, w[..., None].astype(np.int64), axis=-1)[..., 0]


# ---- converters from a 32-bit word -------------------------------------------------------------

def unit_open_closed(w):
    """U = (w >> 8) * 2^-24, in [0, 1); used for the jump test u < lambda."""
    return (np.asarray(w, dtype=np.uint64) >> np.uint64(8)).astype(np.float64) * 2.0 ** -24


def unit_open(w):
    """U = ((w >> 9) + 1/2) * 2^-23, strictly inside (0, 1) and exact in float32."""
    return ((np.asarray(w, dtype=np.uint64) >> np.uint64(9)).astype(np.float64) + 0.5) * 2.0 ** -23


def gumbel(w):
    """Standard Gumbel variate -log(-log U) from one word (float64)."""
    return -np.log(-np.log(unit_open(w)))


def token(w, vocab: int):
    """Uniform token id in [0, vocab): the top log2(vocab) bits when vocab is a power of two,
    else floor(w * vocab / 2^32)."""
    w = np.asarray(w, dtype=np.uint64)
    if vocab & (vocab - 1) == 0:
        bits = vocab.bit_length() - 1
        if bits == 0:
            return np.zeros(w.shape, dtype=np.int64)
        return (w >> np.uint64(32 - bits)).astype(np.int64)
    return ((w * np.uint64(vocab)) >> np.uint64(32)).astype(np.int64)


# ---- the streams -------------------------------------------------------------------------------

def gumbel_noise(seed, step, b, i, v):
    """G(b, i, v) at step s; b, i, v broadcast against each other."""
    b, i, v = np.broadcast_arrays(*(np.asarray(x, dtype=np.int64) for x in (b, i, v)))
    return gumbel(word(seed, v, i >> 2, step, (b << 8) | TAG_GUMBEL, i & 3))


def jump_uniform(seed, step, b, i):
    b, i = np.broadcast_arrays(np.asarray(b, dtype=np.int64), np.asarray(i, dtype=np.int64))
    return unit_open_closed(word(seed, i >> 2, 0, step, (b << 8) | TAG_JUMP, i & 3))


def init_tokens(seed, batch, length, vocab):
    b, i = np.meshgrid(np.arange(batch), np.arange(length), indexing="ij")
    return token(word(seed, i >> 2, 0, 0, (b << 8) | TAG_INIT, i & 3), vocab)


def noise_words(seed, step, batch, length):
    b, i = np.meshgrid(np.arange(batch), np.arange(length), indexing="ij")
    keep = word(seed, i >> 2, 0, step, (b << 8) | TAG_NOISE_KEEP, i & 3)
    tok = word(seed, i >> 2, 0, step, (b << 8) | TAG_NOISE_TOKEN, i & 3)
    return keep, tok


def renoise_tokens(seed, step, batch, length, vocab):
    """Uniform replacement tokens of the entropy-bounded step s for every (b, i)."""
    b, i = np.meshgrid(np.arange(batch), np.arange(length), indexing="ij")
    return token(word(seed, i >> 2, 0, step, (b << 8) | TAG_RENOISE, i & 3), vocab)
