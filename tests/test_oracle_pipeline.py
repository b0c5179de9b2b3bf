"""Pins for the oracle's per-request pipeline (CPU only).

Each check ties the oracle to something other than itself: exact rational
arithmetic rounded to binary32 (for the bit-exact steps), brute-force ordering by
Python's own sort (top-k and ties), the mass invariants that define top-p and
min-p, numpy's argmax (greedy), a full enumeration of all 2^24 uniforms (the
inverse-CDF map), and chi-square tests of the draws against the softmax.
"""
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st
from scipy import stats

from oracle import philox
from oracle import pipeline as P
from tests import exact_f32 as X


def f32(v):
    return float(np.float32(v))


# --------------------------------------------------------------------------
# exact-arithmetic helper sanity (textbook binary32 values)

def test_exact_helper_known_values():
    assert X.float_to_bits(X.round_f32(Fraction(1, 3))) == 0x3EAAAAAB
    assert X.float_to_bits(X.round_f32(Fraction(1, 10))) == 0x3DCCCCCD
    assert X.round_f32(Fraction(2) ** -149) == 2.0 ** -149          # smallest subnormal
    assert X.round_f32(Fraction(2) ** -150) == 0.0                  # tie to even -> 0
    assert X.round_f32(Fraction(3) * Fraction(2) ** -151) == 2.0 ** -149
    assert X.round_f32(Fraction(2) ** 128) == float("inf")
    # 1 + 2^-24 is a tie between 1 and 1 + 2^-23: even mantissa wins
    assert X.round_f32(1 + Fraction(1, 2 ** 24)) == 1.0


# --------------------------------------------------------------------------
# penalties, bias, mask: bit-exact against exact rational arithmetic

def expected_penalised(x, r, f, p, c):
    x = f32(x)
    r, f, p = f32(r), f32(f), f32(p)
    if x > 0:
        y = X.f32_div(x, r)
    else:
        y = X.f32_mul(x, r)
    y = X.f32_sub(y, X.f32_mul(f, float(c)))
    return X.f32_sub(y, p)


def test_penalties_match_exact_rounding():
    rng = np.random.default_rng(11)
    V = 64
    for trial in range(40):
        x = (rng.standard_normal(V) * 5).astype(np.float32)
        x[0] = 0.0
        x[1] = -0.0
        r = f32(rng.choice([1.1, 1.3, 0.7, 1.0]))
        f = f32(rng.uniform(0, 0.5))
        p = f32(rng.uniform(0, 0.5))
        hist = list(rng.integers(0, V, 40)) + [0, 1, 1, -5, V, V + 3]  # out-of-range ignored
        out = P.process_row(x, hist, r, f, p)
        counts = {}
        for h in hist:
            if 0 <= h < V:
                counts[int(h)] = counts.get(int(h), 0) + 1
        for v in range(V):
            want = expected_penalised(x[v], r, f, p, counts[v]) if v in counts else float(x[v])
            assert X.float_to_bits(float(out[v])) == X.float_to_bits(want), (trial, v)


def test_penalty_sign_rule_hand_cases():
    # positive logits are divided by r, non-positive ones multiplied (CTRL form)
    out = P.process_row(np.array([2.0, -2.0, 0.5, 7.0], np.float32), [0, 1, 2, 2, 2], 2.0, 0.25, 0.5)
    # token 0: 2/2 - 0.25*1 - 0.5 = 0.25 ; token 1: -2*2 - 0.25 - 0.5 = -4.75
    # token 2: 0.5/2 - 0.25*3 - 0.5 = -1.0 ; token 3 untouched
    assert out.tolist() == [0.25, -4.75, -1.0, 7.0]


def test_bias_accumulates_in_array_order():
    x = np.array([1.0, 2.0, 3.0], np.float32)
    big, tiny = f32(3e7), f32(1.0)
    out = P.process_row(x, bias_ids=[0, 0, 2, 7, -1], bias_vals=[big, tiny, -3.0, 100.0, 5.0])
    want0 = X.f32_add(X.f32_add(1.0, big), tiny)
    assert float(out[0]) == want0
    assert float(out[1]) == 2.0
    assert float(out[2]) == 0.0


def test_mask_lsb_first():
    V = 70
    words = np.zeros(3, np.uint32)
    words[0] = 0b101          # tokens 0 and 2
    words[1] = 1 << 31        # token 63
    words[2] = 1 << 5         # token 69
    out = P.process_row(np.zeros(V, np.float32), mask_words=words)
    allowed = [v for v in range(V) if np.isfinite(out[v])]
    assert allowed == [0, 2, 63, 69]
    assert np.all(out[[v for v in range(V) if v not in allowed]] == -np.inf)


def test_mask_commutes_with_penalties_and_bias():
    rng = np.random.default_rng(5)
    V = 100
    x = rng.standard_normal(V).astype(np.float32)
    words = rng.integers(0, 2 ** 32, 4, dtype=np.uint64).astype(np.uint32)
    hist = rng.integers(0, V, 30)
    a = P.process_row(x, hist, 1.2, 0.3, 0.1, [3, 4], [1.0, -2.0], words)
    allowed = P.mask_allowed(words, V)
    b = P.process_row(x, hist, 1.2, 0.3, 0.1, [3, 4], [1.0, -2.0])
    b[~allowed] = -np.inf
    assert np.array_equal(a, b)


# --------------------------------------------------------------------------
# temperature + top-k ordering: brute force with Python's sort

def brute_order(xp, T):
    zs = {}
    for v, xv in enumerate(xp):
        if np.isfinite(xv):
            zs[v] = X.f32_div(float(xv), f32(T))
    return sorted(zs, key=lambda v: (-zs[v], v))


@pytest.mark.parametrize("quant", [False, True])
def test_topk_matches_bruteforce(quant):
    rng = np.random.default_rng(21 if quant else 22)
    for trial in range(30):
        V = int(rng.integers(1, 300))
        x = rng.standard_normal(V).astype(np.float32)
        if quant:  # bf16-like quantisation gives tie storms, plus signed zeros
            x = np.round(x * 4) / 4
            x = x.astype(np.float32)
            x[rng.random(V) < 0.1] = 0.0
            x[rng.random(V) < 0.1] = -0.0
        x[rng.random(V) < 0.1] = -np.inf
        T = f32(rng.choice([0.3, 0.7, 1.0, 1.7]))
        k = int(rng.integers(1, V + 2))
        filt = P.filter_row(x, T, k, 1.0, 0.0)
        order = brute_order(x, T)
        n = min(k, len(order)) if k < V else len(order)
        assert filt.order[:filt.n_topk].tolist() == order[:n]


def test_temperature_division_is_correctly_rounded():
    rng = np.random.default_rng(9)
    x = (rng.standard_normal(2000) * 30).astype(np.float32)
    for T in (0.7, 0.3, 1.9):
        want = [X.f32_div(float(v), f32(T)) for v in x]
        got = (x / np.float32(T)).astype(np.float32)
        assert [X.float_to_bits(float(g)) for g in got] == [X.float_to_bits(w) for w in want]


# --------------------------------------------------------------------------
# greedy, top-p and min-p invariants

def test_greedy_is_numpy_argmax():
    rng = np.random.default_rng(4)
    for _ in range(50):
        V = int(rng.integers(1, 200))
        x = np.round(rng.standard_normal(V) * 2).astype(np.float32)  # many ties
        x[rng.random(V) < 0.2] = -np.inf
        res = P.draw(P.filter_row(x, 0.0, 5, 0.5, 0.1), 0.3)
        if np.isfinite(x).any():
            assert res.token == int(np.argmax(x))
        else:
            assert res.token == -1


def test_topp_mass_invariants():
    rng = np.random.default_rng(8)
    for _ in range(200):
        V = int(rng.integers(2, 400))
        x = (rng.standard_normal(V) * rng.uniform(0.1, 5)).astype(np.float32)
        T = rng.uniform(0.2, 2.0)
        k = int(rng.choice([0, 1, 5, 50, V + 1]))
        tp = f32(rng.uniform(0.01, 0.999))
        filt = P.filter_row(x, T, k, tp, 0.0)
        wk = filt.w[:filt.n_topk]
        Pn = wk / wk.sum()
        kept = Pn[:filt.n_topp].sum()
        assert filt.n_topp >= 1
        assert kept >= tp - 1e-12 or filt.n_topp == filt.n_topk
        assert kept - Pn[filt.n_topp - 1] < tp + 1e-12
        # kept set is a prefix of the top-k set in key order
        assert set(np.nonzero(filt.probs)[0]) == set(filt.order[:filt.n_kept].tolist())


def test_minp_invariants_and_order():
    rng = np.random.default_rng(12)
    for _ in range(200):
        V = int(rng.integers(2, 300))
        x = (rng.standard_normal(V) * 3).astype(np.float32)
        mp = f32(rng.uniform(0.0, 1.0))
        tp = f32(rng.choice([1.0, 0.95, 0.6]))
        filt = P.filter_row(x, 1.0, 0, tp, mp)
        kept = filt.order[:filt.n_kept]
        pmax = filt.probs.max()
        assert np.all(filt.probs[kept] >= mp * pmax * (1 - 1e-12))
        dropped = filt.order[filt.n_kept:filt.n_topp]
        wd = filt.w[filt.n_kept:filt.n_topp]
        assert np.all(wd < mp)
        assert len(dropped) == len(wd)
        assert abs(filt.probs.sum() - 1.0) < 1e-12


def test_edge_cases():
    V = 40
    x = np.linspace(-3, 3, V).astype(np.float32)
    # all masked -> -1
    none = np.zeros(2, np.uint32)
    xp = P.process_row(x, mask_words=none)
    assert P.draw(P.filter_row(xp, 0.7, 0, 1.0, 0.0), 0.5).token == -1
    assert P.draw(P.filter_row(xp, 0.0, 0, 1.0, 0.0), 0.5).token == -1
    # single allowed token wins at any temperature and any u
    one = np.zeros(2, np.uint32)
    one[0] = 1 << 7
    xp = P.process_row(x, mask_words=one)
    for T in (0.0, 0.5, 3.0):
        for u in (0.0, 0.999):
            assert P.draw(P.filter_row(xp, T, 0, 1.0, 0.0), u).token == 7
    # top_k = 1 is the argmax of z; top_p -> 0+ keeps exactly one token
    y = np.zeros(V, np.float32)
    y[[3, 9, 20]] = 5.0
    for u in (0.0, 0.5, 0.99):
        assert P.draw(P.filter_row(y, 1.0, 1, 1.0, 0.0), u).token == 3
        assert P.draw(P.filter_row(y, 1.0, 0, f32(1e-7), 0.0), u).token == 3
    # min_p = 1 keeps exactly the tied maxima
    filt = P.filter_row(y, 1.0, 0, 1.0, 1.0)
    assert filt.kept_ids.tolist() == [3, 9, 20]


# --------------------------------------------------------------------------
# the inverse-CDF map: enumerate every one of the 2^24 uniforms

def test_enumerate_all_uniforms_tiny_vocab():
    x = np.array([0.3, -1.2, 2.0, 0.3, -0.5], np.float32)
    filt = P.filter_row(x, 0.9, 0, 1.0, 0.0)
    u = np.arange(1 << 24, dtype=np.float64) * 2.0 ** -24
    idx = P.inverse_cdf(filt.cdf, u)
    counts = np.bincount(idx, minlength=filt.n_kept)
    pi_key = filt.probs[filt.order]
    assert np.all(np.abs(counts - pi_key * 2 ** 24) <= 1.0)
    # the lowest uniforms go to the largest key (descending order), the highest to the smallest
    assert filt.order[idx[0]] == 2
    assert filt.order[idx[-1]] == 1
    # equal logits (tokens 0 and 3): the lower id comes first in the CDF
    assert filt.order.tolist().index(0) < filt.order.tolist().index(3)


def test_chi_square_draws_follow_filtered_softmax():
    rng = np.random.default_rng(31)
    V = 24
    x = rng.standard_normal(V).astype(np.float32)
    for (T, k, tp, mp) in [(1.0, 0, 1.0, 0.0), (0.6, 10, 0.9, 0.0), (1.4, 0, 1.0, 0.05)]:
        filt = P.filter_row(x, T, k, tp, mp)
        n = 20000
        toks = np.array([P.draw(filt, philox.uniform(s, 3, 11, 0, philox.SAMPLE)).token
                         for s in range(n)])
        kept = filt.order[:filt.n_kept]
        obs = np.array([np.count_nonzero(toks == v) for v in kept])
        exp = filt.probs[kept] * n
        assert obs.sum() == n
        assert stats.chisquare(obs, exp).pvalue > 1e-4


def test_sample_batch_uses_request_and_position_keys():
    x = np.zeros((3, 16), np.float32)
    prm = P.Params(temperature=np.ones(3, np.float32), top_k=np.zeros(3, np.int32),
                   top_p=np.ones(3, np.float32), min_p=np.zeros(3, np.float32),
                   request_ids=np.array([5, 5, 6], np.int32),
                   positions=np.array([0, 0, 9], np.int32), seed=77)
    res = P.sample_batch(x, prm)
    # uniform logits: token index = floor(u * 16) exactly
    for b, r in enumerate(res):
        u = philox.uniform(77, prm.request_ids[b], prm.positions[b], 0, philox.SAMPLE)
        assert r.token == int(u * 16)
    assert res[0].token == res[1].token


@settings(max_examples=60, deadline=None)
@given(st.lists(st.sampled_from([-2.0, -0.0, 0.0, 0.5, 1.0, 1.0, 3.0, float("-inf")]),
                min_size=1, max_size=24),
       st.sampled_from([0.0, 0.5, 1.0, 2.0]), st.integers(0, 30),
       st.sampled_from([1.0, 0.5, 1e-6]), st.sampled_from([0.0, 0.3, 1.0]),
       st.floats(0.0, 1.0 - 2 ** -24))
def test_hypothesis_edge_rows(vals, T, k, tp, mp, u):
    x = np.array(vals, np.float32)
    filt = P.filter_row(x, T, k, tp, mp)
    res = P.draw(filt, u)
    finite = np.isfinite(x)
    if not finite.any():
        assert res.token == -1
        return
    assert finite[res.token]
    if T == 0:
        assert res.token == int(np.argmax(np.where(finite, x, -np.inf)))
    else:
        order = brute_order(x, T)
        assert filt.order.tolist() == order
        assert res.token in filt.kept_ids.tolist()
        assert filt.kept_ids[0] == order[0]
        assert abs(filt.probs.sum() - 1.0) < 1e-12
