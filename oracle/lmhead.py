"""LM-head projection with Gumbel-max sampling (oracle; test infrastructure only).

What it follows
---------------
FlashSampling news item (meineki.news, bullet list and body): exact sampling is
folded into the LM-head matrix multiplication; logits are formed in small
on-chip tiles, Gumbel noise is added, only the per-row maximum of each
vocabulary tile is kept, and a small final reduction over tiles gives the
result; it stays exact because argmax decomposes over partitions. The kept item
is a (max, argmax) pair, since a token needs an index.

Definition computed here:
  z[b, v] = sum_k h[b, k] * W[v, k] in binary64 from the bfloat16 inputs (the
            products of two bf16 values are exact in binary64).
  s[b, v] = z[b, v] / T_b + g(Philox GUMBEL word at (seed, request_b,
            position_b, draw v)) for T_b > 0; token = lowest v attaining max s.
  T_b == 0: token = lowest v attaining max z (no noise).
A draw is flagged when the two largest scores of its row differ by < 1e-5:
binary32 accumulation over K = 8192 carries errors of that order, and a
Gumbel-max draw has no single uniform to apply a 1e-6 rule to.
"""
from __future__ import annotations

import numpy as np

from . import philox
from .pipeline import bf16_bits_to_f32

GAP_EPS = 1e-5
TILE = 256


def logits_fp64(hidden_bits, weight_bits, chunk=8192):
    """z = H W^T in binary64 from bf16 bit patterns ([B,K] and [V,K] uint16)."""
    H = bf16_bits_to_f32(hidden_bits).astype(np.float64)
    V = weight_bits.shape[0]
    z = np.empty((H.shape[0], V), dtype=np.float64)
    for v0 in range(0, V, chunk):
        Wc = bf16_bits_to_f32(weight_bits[v0:v0 + chunk]).astype(np.float64)
        z[:, v0:v0 + chunk] = H @ Wc.T
    return z


def gumbel_row(seed, request, position, V):
    w = philox.words_np(seed, request, position, np.arange(V), philox.GUMBEL)
    return philox.gumbel_np(w)


def scores_row(z_row, temperature, seed, request, position):
    T = float(np.float32(temperature))
    if T == 0.0:
        return np.asarray(z_row, dtype=np.float64)
    return np.asarray(z_row, dtype=np.float64) / T + gumbel_row(seed, request, position,
                                                               len(z_row))


def argmax_and_gap(s):
    i = int(np.argmax(s))  # first maximum = lowest id
    if len(s) < 2:
        return i, np.inf
    top2 = np.partition(s, -2)[-2:]
    return i, float(top2[1] - top2[0])


def tile_partials(s, tile=TILE):
    """Per-tile (max, lowest argmax) pairs over consecutive vocabulary tiles."""
    V = len(s)
    n = (V + tile - 1) // tile
    vals = np.empty(n)
    idx = np.empty(n, dtype=np.int64)
    for t in range(n):
        seg = s[t * tile:(t + 1) * tile]
        j = int(np.argmax(seg))
        vals[t] = seg[j]
        idx[t] = t * tile + j
    return vals, idx


def reduce_partials(vals, idx):
    """Cross-tile reduction: the largest value, ties toward the lower token id."""
    best = 0
    for t in range(1, len(vals)):
        if vals[t] > vals[best] or (vals[t] == vals[best] and idx[t] < idx[best]):
            best = t
    return int(idx[best])


def sample(z, temperature, request_ids, positions, seed):
    """Tokens and boundary flags for every row of z ([B, V] binary64)."""
    B = z.shape[0]
    toks = np.empty(B, dtype=np.int32)
    flags = np.zeros(B, dtype=bool)
    for b in range(B):
        s = scores_row(z[b], temperature[b], seed, int(request_ids[b]), int(positions[b]))
        toks[b], gap = argmax_and_gap(s)
        flags[b] = gap < GAP_EPS
    return toks, flags
