"""Pins for the oracle's LM-head + Gumbel-max sampler (CPU only).

Gumbel-max theorem (textbook): argmax(z / T + Gumbel noise) is distributed as
softmax(z / T); checked by chi-square. Partition invariance (argmax decomposes
over any tiling of the vocabulary, the property the FlashSampling page relies
on). The binary64 GEMM against exactly rounded sums of exact products.
"""
import math

import numpy as np
from scipy import stats

from oracle import lmhead as L
from oracle import pipeline as P


def bf16(rng, shape, scale):
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def test_bf16_widening_known_values():
    vals = P.bf16_bits_to_f32(np.array([0x3F80, 0xBF80, 0x4049, 0x0000, 0x8000, 0x7F80], np.uint16))
    assert vals[:4].tolist() == [1.0, -1.0, 3.140625, 0.0]
    assert math.copysign(1.0, vals[4]) == -1.0 and vals[5] == np.inf


def test_fp64_gemm_is_exact_sum():
    rng = np.random.default_rng(1)
    H = bf16(rng, (3, 96), 1.0)
    W = bf16(rng, (40, 96), 0.02)
    z = L.logits_fp64(H, W, chunk=16)
    Hf = P.bf16_bits_to_f32(H).astype(np.float64)
    Wf = P.bf16_bits_to_f32(W).astype(np.float64)
    for b in range(3):
        for v in range(0, 40, 7):
            exact = math.fsum(float(Hf[b, k]) * float(Wf[v, k]) for k in range(96))
            assert abs(z[b, v] - exact) <= 1e-13 * max(1.0, abs(exact))


def test_gumbel_max_follows_softmax():
    rng = np.random.default_rng(2)
    V = 12
    z = rng.standard_normal(V) * 1.5
    for T in (1.0, 0.5):
        n = 30000
        toks = np.empty(n, dtype=np.int64)
        for s in range(n):
            toks[s] = L.argmax_and_gap(L.scores_row(z, T, s, 0, 0))[0]
        p = np.exp(z / np.float32(T) - (z / np.float32(T)).max())
        p /= p.sum()
        obs = np.bincount(toks, minlength=V)
        assert stats.chisquare(obs, p * n).pvalue > 1e-4


def test_partition_invariance():
    rng = np.random.default_rng(3)
    for _ in range(50):
        V = int(rng.integers(1, 2000))
        s = np.round(rng.standard_normal(V) * 3) / 3  # ties
        want = int(np.argmax(s))
        for tile in (1, 7, 256, V):
            assert L.reduce_partials(*L.tile_partials(s, tile)) == want
        # an arbitrary uneven partition
        cuts = np.sort(rng.choice(np.arange(1, V), min(V - 1, 9), replace=False)) if V > 1 else []
        bounds = [0] + list(cuts) + [V]
        vals = [s[a:b].max() for a, b in zip(bounds[:-1], bounds[1:])]
        idxs = [a + int(np.argmax(s[a:b])) for a, b in zip(bounds[:-1], bounds[1:])]
        assert L.reduce_partials(np.array(vals), np.array(idxs)) == want


def test_greedy_and_tiled_sample_agree():
    rng = np.random.default_rng(4)
    z = rng.standard_normal((5, 700))
    T = np.array([0.0, 1.0, 1.0, 0.5, 2.0], np.float32)
    req = np.arange(5, dtype=np.int32)
    pos = np.array([0, 0, 3, 1, 2], np.int32)
    toks, _ = L.sample(z, T, req, pos, 11)
    assert toks[0] == int(np.argmax(z[0]))
    for b in range(1, 5):
        s = L.scores_row(z[b], T[b], 11, req[b], pos[b])
        assert toks[b] == L.reduce_partials(*L.tile_partials(s))
