"""Pins of the oracle's boundary flags (CPU only).

The parity rule excuses a GPU/oracle mismatch only on draws whose uniform lies
within 1e-6 of a CDF or acceptance boundary (and, by the same reasoning, on
top-p / min-p cuts decided within 1e-6, and on LM-head draws whose two best
perturbed scores lie within 1e-5). These flags decide which mismatches are
excused, so each is pinned here on both sides of its threshold, with cases whose
distances are exact by construction:

  * equal logits over n = 4 tokens give weights exactly 1 and probabilities
    exactly 1/4, so every CDF breakpoint and exclusive mass is a multiple of
    1/4 in binary64;
  * thresholds are placed k * 2^-24 (or k * 2^-25 below 1/2) away from those
    values: exact in binary32 and binary64, 16 steps = 9.5e-7 (inside the
    1e-6 band) or 18 steps = 1.07e-6 (outside), 32 steps below 1/2 = 9.5e-7,
    36 steps = 1.07e-6;
  * acceptance ratios pi / q use pi = 1/4 and binary32 q chosen so the ratio
    is 1/2, exactly 1, or 1 / (1 - 2^-23) (just above 1);
  * LM-head scores are given directly at temperature 0 (no noise), with gaps
    of 0.9e-5 and 1.1e-5 between the two best.

A slip in any flag -- a wrong breakpoint index, an epsilon off by a factor,
an inclusive comparison, the last breakpoint counted as interior, a side of 1
ignored -- fails one of these cases.
"""
import numpy as np
import pytest

from oracle import lmhead as OL
from oracle import pipeline as P
from oracle import spec as S

UP16 = 16 * 2.0 ** -24   # 9.54e-7 above a value in [1/2, 1)
UP18 = 18 * 2.0 ** -24   # 1.07e-6
DN32 = 32 * 2.0 ** -25   # 9.54e-7 below 1/2 (binary32 spacing there is 2^-25)
DN36 = 36 * 2.0 ** -25   # 1.07e-6


def test_step_sizes_straddle_the_band():
    assert UP16 < 1e-6 < UP18
    assert DN32 < 1e-6 < DN36
    for v in (0.5 + UP16, 0.5 + UP18, 0.5 - DN32, 0.5 - DN36, 1 - UP16 / 2, 1 - UP18 / 2):
        assert float(np.float32(v)) == v  # the thresholds themselves are exact


# --- the draw's breakpoints -------------------------------------------------

CDF4 = np.array([0.25, 0.5, 0.75, 1.0])


@pytest.mark.parametrize("u,flag", [
    (0.5 + UP16, True), (0.5 - DN32, True),        # within 1e-6 of breakpoint 1/2
    (0.5 + UP18, False), (0.5 - DN36, False),      # just outside
    (0.25 + UP16 / 2, True), (0.25 + UP18, False),  # the first breakpoint counts
    (1.0 - UP16 / 2, False),                       # the last breakpoint is not interior
    (0.375, False)])
def test_boundary_draw(u, flag):
    assert P.boundary_draw(CDF4, u) is flag


def test_draw_breaks_ties_at_a_breakpoint_upward():
    # token = first i with u < C_i: u exactly at C_1 = 1/2 draws token 2
    assert int(P.inverse_cdf(CDF4, 0.5)) == 2
    assert int(P.inverse_cdf(CDF4, 0.5 - 2.0 ** -25)) == 1
    assert int(P.inverse_cdf(CDF4, 1.0)) == 3  # rounding past the end: the last token


def _equal_row():
    return np.zeros(4, np.float32)  # x' = 0: z = 0, w = 1, probabilities 1/4


def test_equal_row_is_exact():
    f = P.filter_row(_equal_row(), 1.0, 0, 1.0, 0.0)
    assert f.cdf.tolist() == [0.25, 0.5, 0.75, 1.0]
    assert f.order.tolist() == [0, 1, 2, 3]


# --- top-p -------------------------------------------------------------------

@pytest.mark.parametrize("top_p,n_topp,flag", [
    # exclusive masses are 0, 1/4, 1/2, 3/4; keep i iff excl_i < top_p
    (0.5 + UP16, 3, True),    # the crossing token (excl 1/2) kept, 9.5e-7 away
    (0.5 + UP18, 3, False),
    (0.5 - DN32, 2, True),    # the first dropped token (excl 1/2) is 9.5e-7 away
    (0.5 - DN36, 2, False),
    (0.25 + UP16 / 2, 2, True),
    (0.625, 3, False)])
def test_topp_cut_flag(top_p, n_topp, flag):
    f = P.filter_row(_equal_row(), 1.0, 0, top_p, 0.0)
    assert f.n_topp == n_topp
    assert f.flag_topp is flag


def test_topp_flag_ignores_the_first_token():
    # the first token's exclusive mass is 0 on any implementation: a top_p
    # within 1e-6 of 0 keeps exactly one token and raises no flag
    f = P.filter_row(_equal_row(), 1.0, 0, 5e-7, 0.0)
    assert f.n_topp == 1 and not f.flag_topp


def test_topp_flag_inside_topk():
    # renormalised over the top-2 set the exclusive masses are 0 and 1/2
    f = P.filter_row(_equal_row(), 1.0, 2, 0.5 + UP16, 0.0)
    assert f.n_topk == 2 and f.n_topp == 2 and f.flag_topp
    f = P.filter_row(_equal_row(), 1.0, 2, 0.5 - DN32, 0.0)
    assert f.n_topp == 1 and f.flag_topp
    f = P.filter_row(_equal_row(), 1.0, 2, 0.5 - DN36, 0.0)
    assert f.n_topp == 1 and not f.flag_topp


# --- min-p -------------------------------------------------------------------

@pytest.mark.parametrize("min_p,flag", [
    (1.0 - UP16 / 2, True),    # weight 1 of tokens 1..3 within 4.8e-7 of min_p
    (1.0 - UP18, False),       # 1.07e-6 away
])
def test_minp_flag_on_later_tokens(min_p, flag):
    f = P.filter_row(_equal_row(), 1.0, 0, 1.0, min_p)
    assert f.n_kept == 4  # w = 1 >= min_p for every token
    assert f.flag_minp is flag


def test_minp_flag_ignores_the_first_token():
    # only the first token (weight exactly 1 everywhere) is near min_p; the
    # others weigh e^-4 and are dropped far from the cut
    x = np.array([0.0, -4.0, -4.0, -4.0], np.float32)
    f = P.filter_row(x, 1.0, 0, 1.0, 1.0 - UP16 / 2)
    assert f.n_kept == 1 and not f.flag_minp


def test_minp_flag_below_the_cut():
    # a dropped token whose weight is just below min_p is a boundary case:
    # w = exp(-1) for x' = -1, T = 1 (binary64 exp of an exact binary32 -1)
    x = np.array([0.0, -1.0], np.float32)
    w1 = float(np.exp(np.float64(-1.0)))
    near = float(np.float32(w1 + 5e-7))   # min_p 5e-7 above w1 (up to binary32 rounding, <3e-8)
    far = float(np.float32(w1 + 2e-6))
    f = P.filter_row(x, 1.0, 0, 1.0, near)
    assert f.n_kept == 1 and f.flag_minp
    f = P.filter_row(x, 1.0, 0, 1.0, far)
    assert f.n_kept == 1 and not f.flag_minp


# --- acceptance --------------------------------------------------------------

def _verify(q_d, u_accept):
    """One draft position over the equal 4-token row: pi(d) = 1/4 exactly."""
    target = np.zeros((2, 4), np.float32)
    q = np.full((1, 4), 0.25, np.float32)
    q[0, 1] = q_d

    def uniform(domain, pos):
        return u_accept if domain == 1 else 0.1  # ACCEPT: the chosen u; others away from any boundary

    return S.verify_request(target, q, np.array([1], np.int32), temperature=1.0, uniform=uniform)


@pytest.mark.parametrize("q_d,u,accept,flag", [
    (0.5, 0.5 - DN32, True, True),       # ratio 1/2, u 9.5e-7 below: accepted, flagged
    (0.5, 0.5 + UP16, False, True),      # u 9.5e-7 above: rejected, flagged
    (0.5, 0.5 - DN36, True, False),
    (0.5, 0.5 + UP18, False, False),
    (0.25, 1.0 - UP16 / 2, True, True),  # ratio exactly 1, u within 1e-6 below it
    (0.25, 1.0 - UP18, True, False),
    # ratio 1 / (1 - 2^-23) = 1 + 1.19e-7 (q = 1/4 - 2^-25, exact in binary32):
    # a binary32 device may see a ratio below 1, so u within 1e-6 is flagged
    (0.25 - 2.0 ** -25, 1.0 - UP16 / 2, True, True),
    (0.25 - 2.0 ** -25, 1.0 - 2 * UP16, True, False),
])
def test_accept_flag_both_sides_of_one(q_d, u, accept, flag):
    assert float(np.float32(q_d)) == q_d
    r = _verify(q_d, u)
    assert (r.n_acc == 1) is accept
    assert r.flagged is flag


# --- the residual draw -------------------------------------------------------

def test_residual_draw_breakpoints():
    # pi = 1/4 everywhere, q = (1/2, 0, 0, 1/2): residual r = (0, 1/4, 1/4, 0),
    # normalised (0, 1/2, 1/2, 0) in token-id order: one interior breakpoint 1/2
    pi = np.full(4, 0.25)
    q = np.array([0.5, 0.0, 0.0, 0.5])
    assert S.residual_draw(pi, q, 0.5 - DN32) == (1, True)
    assert S.residual_draw(pi, q, 0.5 + UP16) == (2, True)
    assert S.residual_draw(pi, q, 0.5 - DN36) == (1, False)
    assert S.residual_draw(pi, q, 0.5 + UP18) == (2, False)
    # the residual's last breakpoint (1) is not interior
    assert S.residual_draw(pi, q, 1.0 - UP16 / 2) == (2, False)


# --- LM-head gap -------------------------------------------------------------

@pytest.mark.parametrize("gap,flag", [(0.9e-5, True), (1.1e-5, False), (0.0, True)])
def test_lmhead_gap_flag(gap, flag):
    # temperature 0: the scores are the logits themselves, no noise
    z = np.array([[0.5, 1.0, 1.0 - gap, -3.0]])
    toks, flags = OL.sample(z, np.zeros(1, np.float32), np.zeros(1, np.int32),
                            np.zeros(1, np.int32), seed=0)
    assert int(toks[0]) == 1  # ties go to the lower id
    assert bool(flags[0]) is flag
