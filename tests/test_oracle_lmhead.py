"""Pins for the oracle's LM-head + Gumbel-max sampler (CPU only).

Gumbel-max theorem (textbook): argmax(z / T + Gumbel noise) is distributed as
softmax(z / T); checked by chi-square. Partition invariance (argmax decomposes
over any tiling of the vocabulary, the property the FlashSampling page relies
on). The binary64 GEMM against exactly rounded sums of exact products.

The per-request pipeline before the Gumbel step: it reduces to the plain
draw without processing, top_k = 1 gives the argmax of the processed logits,
the draws follow the filtered distribution (chi-square), and the cut flags
fire on either side of their distance.
"""
import math

import numpy as np
import pytest
from scipy import stats

from oracle import lmhead as L
from oracle import lmhead as OL
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


# --- the per-request pipeline before the Gumbel step ---------------------------

def _params(B, T, **kw):
    from oracle import pipeline as P
    n = lambda v, dt: np.full(B, v, dt)
    return P.Params(temperature=np.asarray(T, np.float32) if np.ndim(T) else n(T, np.float32),
                    top_k=kw.get("top_k", n(0, np.int32)), top_p=kw.get("top_p", n(1.0, np.float32)),
                    min_p=kw.get("min_p", n(0.0, np.float32)), rep=kw.get("rep"),
                    freq=kw.get("freq"), pres=kw.get("pres"), hist=kw.get("hist"),
                    bias_ids=kw.get("bias_ids"), bias_vals=kw.get("bias_vals"),
                    mask=kw.get("mask"), request_ids=np.arange(B, dtype=np.int32) * 5 + 1,
                    positions=np.arange(B, dtype=np.int32) % 3, seed=kw.get("seed", 9))


def test_processed_reduces_to_plain_gumbel_max():
    # no processing and no filter: the plain Gumbel-max draw (the two differ
    # only by binary32 rounding of z / T, far inside the flag gap)
    rng = np.random.default_rng(41)
    B, V = 24, 500
    z = rng.standard_normal((B, V)) * 2.0
    T = rng.choice(np.array([0.0, 0.5, 1.0, 2.0], np.float32), B)
    prm = _params(B, T)
    got, gflags = OL.sample_processed(z, prm)
    want, wflags = OL.sample(z, T, prm.request_ids, prm.positions, prm.seed)
    ok = gflags | wflags | (got == want)
    assert ok.all(), np.nonzero(~ok)


def test_processed_top_k_one_is_the_argmax_of_processed_logits():
    rng = np.random.default_rng(42)
    B, V = 16, 300
    z = rng.standard_normal((B, V)) * 3.0
    hist = [rng.integers(0, V, 8) for _ in range(B)]
    for b in range(B):
        hist[b][0] = int(np.argmax(z[b]))  # penalise the raw argmax
    prm = _params(B, 1.0, top_k=np.ones(B, np.int32), rep=np.full(B, 3.0, np.float32),
                  freq=np.full(B, 1.0, np.float32), pres=np.full(B, 0.5, np.float32), hist=hist)
    toks, _ = OL.sample_processed(z, prm)
    for b in range(B):
        xp = P.process_row(z[b].astype(np.float32), hist[b], 3.0, 1.0, 0.5, (), (), None)
        assert toks[b] == int(np.argmax(xp))
        assert toks[b] != int(np.argmax(z[b]))


def test_processed_draws_follow_the_filtered_distribution():
    from scipy import stats
    V, n = 8, 6000
    z = np.random.default_rng(43).standard_normal((1, V)) * 1.5
    counts = np.zeros(V)
    for sd in range(n):
        prm = _params(1, 1.0, top_k=np.array([5], np.int32), top_p=np.array([0.95], np.float32),
                      seed=sd)
        t, _ = OL.sample_processed(z, prm)
        counts[t[0]] += 1
    pi = P.filter_row(z[0].astype(np.float32), 1.0, 5, 0.95, 0.0).probs
    assert counts[pi == 0].sum() == 0
    assert stats.chisquare(counts[pi > 0], pi[pi > 0] * n).pvalue > 1e-4


@pytest.mark.parametrize("delta,flag", [(1.9e-5, True), (2.1e-5, False)])
def test_processed_top_k_cut_flag(delta, flag):
    # top-1 between two logits delta apart: both lie within 1e-5 of the cut's
    # midpoint when delta < 2e-5, and the winner (the only kept entry) is one
    # of them, so the draw could change
    z = np.array([[1.0, 1.0 - delta, -1.0]])  # |x'| <= 1: the bands are unscaled
    prm = _params(1, 1.0, top_k=np.array([1], np.int32))
    toks, flags = OL.sample_processed(z, prm)
    assert toks[0] == 0
    assert bool(flags[0]) is flag


@pytest.mark.parametrize("delta,flag", [(1.9e-4, True), (2.1e-4, False)])
def test_processed_flag_bands_scale_with_the_logits(delta, flag):
    # the same top-1 cut with logits of magnitude 10: the band is ten times wider
    z = np.array([[10.0, 10.0 - delta, -10.0]])
    prm = _params(1, 1.0, top_k=np.array([1], np.int32))
    assert bool(OL.sample_processed(z, prm)[1][0]) is flag


def test_processed_top_p_cut_flag():
    # equal logits: exclusive masses 0, 1/4, 1/2, 3/4 in id order. top_p =
    # 1/2 + 0.9e-5 keeps tokens 0..2 with token 2's membership within the band:
    # the row is flagged exactly when token 2 wins. At 1/2 + 1.1e-5 nothing is
    # ambiguous and no seed is flagged.
    z = np.zeros((1, 4))
    won_by_2 = 0
    for sd in range(40):
        prm = _params(1, 1.0, top_p=np.array([0.5 + 0.9e-5], np.float32), seed=sd)
        toks, flags = OL.sample_processed(z, prm)
        assert toks[0] in (0, 1, 2)
        assert bool(flags[0]) == bool(toks[0] == 2)
        won_by_2 += toks[0] == 2
        prm = _params(1, 1.0, top_p=np.array([0.5 + 1.1e-5], np.float32), seed=sd)
        assert not OL.sample_processed(z, prm)[1][0]
    assert 0 < won_by_2 < 40
