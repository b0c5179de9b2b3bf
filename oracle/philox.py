"""Philox4x32-10 counter-based generator (oracle side; test infrastructure only).

The pages never name a random number generator. The generator used here is the
Philox4x32 family with ten rounds from Salmon, Moraes, Dror and Shaw, "Parallel
Random Numbers: As Easy as 1, 2, 3" (SC'11). One round multiplies counter words
0 and 2 by two fixed 32-bit multipliers, takes the high and low halves of the
64-bit products, and mixes them with the other two counter words and the key;
between rounds the two key words are advanced by two Weyl constants (the golden
ratio and sqrt(3) fractional parts scaled by 2^32). This module is an
independent restatement of that definition in plain Python integers, with a
numpy twin for bulk use.

Layout of a draw (a reading; the pages fix none of it):
  counter = (request, position, draw >> 2, domain)
  key     = (seed mod 2^32, seed >> 32)
  word    = output[draw & 3]
Domains: SAMPLE = 0, ACCEPT = 1, RESIDUAL = 2, GUMBEL = 3.

Transforms:
  u24(w)    = (w >> 8) * 2^-24, a uniform on [0, 1) exact in binary32 and binary64.
  gumbel(w) = -ln(-ln U), U = 1 - (w + 0.5) * 2^-32, evaluated as
              -ln(-log1p(-(w + 0.5) * 2^-32)) so it stays accurate as U -> 1.
"""
from __future__ import annotations

import math

import numpy as np

MASK32 = 0xFFFFFFFF
M0 = 0xD2511F53
M1 = 0xCD9E8D57
W0 = 0x9E3779B9  # floor(2^32 * (golden ratio - 1))
W1 = 0xBB67AE85  # floor(2^32 * (sqrt(3) - 1))

SAMPLE = 0
ACCEPT = 1
RESIDUAL = 2
GUMBEL = 3


def philox4x32_10(ctr, key):
    """Ten Philox rounds on a 4-word counter under a 2-word key (plain ints)."""
    x0, x1, x2, x3 = (int(c) & MASK32 for c in ctr)
    k0, k1 = (int(k) & MASK32 for k in key)
    for rnd in range(10):
        if rnd > 0:
            k0 = (k0 + W0) & MASK32
            k1 = (k1 + W1) & MASK32
        p0 = M0 * x0
        p1 = M1 * x2
        hi0, lo0 = p0 >> 32, p0 & MASK32
        hi1, lo1 = p1 >> 32, p1 & MASK32
        x0, x1, x2, x3 = (hi1 ^ x1 ^ k0) & MASK32, lo1, (hi0 ^ x3 ^ k1) & MASK32, lo0
    return x0, x1, x2, x3


def philox4x32_10_np(c0, c1, c2, c3, k0, k1):
    """Vectorised twin of philox4x32_10 over numpy arrays (broadcasting).

    Arithmetic runs in uint64 so that the 32x32->64 products are exact.
    Returns four uint32 arrays.
    """
    x0 = np.asarray(c0, dtype=np.uint64) & MASK32
    x1 = np.asarray(c1, dtype=np.uint64) & MASK32
    x2 = np.asarray(c2, dtype=np.uint64) & MASK32
    x3 = np.asarray(c3, dtype=np.uint64) & MASK32
    x0, x1, x2, x3 = np.broadcast_arrays(x0, x1, x2, x3)
    x0, x1, x2, x3 = (a.copy() for a in (x0, x1, x2, x3))
    ka = np.uint64(int(k0) & MASK32)
    kb = np.uint64(int(k1) & MASK32)
    m0 = np.uint64(M0)
    m1 = np.uint64(M1)
    msk = np.uint64(MASK32)
    s32 = np.uint64(32)
    for rnd in range(10):
        if rnd > 0:
            ka = np.uint64((int(ka) + W0) & MASK32)
            kb = np.uint64((int(kb) + W1) & MASK32)
        p0 = x0 * m0
        p1 = x2 * m1
        hi0, lo0 = p0 >> s32, p0 & msk
        hi1, lo1 = p1 >> s32, p1 & msk
        x0, x1, x2, x3 = hi1 ^ x1 ^ ka, lo1, hi0 ^ x3 ^ kb, lo0
    return (x0.astype(np.uint32), x1.astype(np.uint32),
            x2.astype(np.uint32), x3.astype(np.uint32))


def key_of(seed):
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    return seed & MASK32, seed >> 32


def word(seed, request, position, draw, domain):
    """The 32-bit word for one (seed, request, position, draw, domain) draw."""
    out = philox4x32_10((request, position, int(draw) >> 2, domain), key_of(seed))
    return out[int(draw) & 3]


def words_np(seed, request, position, draws, domain):
    """Words for a vector of draw indices at one (seed, request, position, domain)."""
    draws = np.asarray(draws, dtype=np.int64)
    k0, k1 = key_of(seed)
    blocks = draws >> 2
    o = philox4x32_10_np(np.uint64(int(request) & MASK32), np.uint64(int(position) & MASK32),
                         blocks.astype(np.uint64), np.uint64(domain), k0, k1)
    stacked = np.stack(o, axis=-1)
    return np.take_along_axis(stacked, (draws & 3)[..., None], axis=-1)[..., 0]


def u24(w):
    """Uniform on [0, 1): the top 24 bits of a word scaled by 2^-24 (exact in f32)."""
    return (int(w) >> 8) * (2.0 ** -24)


def u24_np(w):
    return (np.asarray(w, dtype=np.uint32) >> np.uint32(8)).astype(np.float64) * (2.0 ** -24)


def gumbel(w):
    """Standard Gumbel variate from all 32 bits of a word, in binary64."""
    x = (int(w) + 0.5) * (2.0 ** -32)
    e = -math.log1p(-x)
    return -math.log(e)


def gumbel_np(w):
    x = (np.asarray(w, dtype=np.uint32).astype(np.float64) + 0.5) * (2.0 ** -32)
    e = -np.log1p(-x)
    return -np.log(e)


def uniform(seed, request, position, draw, domain):
    return u24(word(seed, request, position, draw, domain))
