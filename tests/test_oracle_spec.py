"""Pins for the oracle's speculative verification (CPU only).

The rejection rule's defining property (the textbook speculative-sampling
theorem) is checked by integrating the oracle's output over grids of uniforms:
every emitted token must follow the target's filtered distribution at its
position. The expected number of accepted drafts is checked against its closed
form, and greedy verification against exact-match acceptance.
"""
import numpy as np
from scipy import stats

from oracle import philox
from oracle import pipeline as P
from oracle import spec as S

N_GRID = 1024
GRID = (np.arange(N_GRID) + 0.5) / N_GRID


def call(target, q, d, T=1.0, uni=None, **kw):
    return S.verify_request(target, q, d, temperature=T, uniform=uni, **kw)


def pi_of(row, T=1.0, **kw):
    return P.filter_row(row, T, kw.get("top_k", 0), kw.get("top_p", 1.0), kw.get("min_p", 0.0)).probs


def law_at_position(target, q, fixed_prefix, j, kw):
    """Law of out[j] given that positions < j were accepted (integrated over u's)."""
    V = target.shape[1]
    G = q.shape[0]
    law = np.zeros(V)
    for d in range(V):
        drafts = list(fixed_prefix) + [d] + [0] * (G - j - 1)
        acc = 0
        for ua in GRID:
            def uni(dom, pos, ua=ua):
                if dom == philox.ACCEPT:
                    return 0.0 if pos < j else ua
                return 0.5
            r = call(target, q, drafts, uni=uni, **kw)
            assert r.n_acc >= j
            acc += r.n_acc > j
        a = acc / N_GRID
        law[d] += q[j, d] * a
        if a < 1.0:
            rho = np.zeros(V)
            for ur in GRID:
                def uni(dom, pos, ur=ur):
                    if dom == philox.ACCEPT:
                        return 0.0 if pos < j else 1.0 - 2.0 ** -24
                    return ur
                r = call(target, q, drafts, uni=uni, **kw)
                if r.n_acc == j:
                    rho[r.tokens[j]] += 1
            if rho.sum() > 0:
                law += q[j, d] * (1 - a) * rho / rho.sum()
    return law


def make_case(rng, V, G, scale=1.5):
    target = (rng.standard_normal((G + 1, V)) * scale).astype(np.float32)
    dl = target[:G].astype(np.float64) + rng.normal(0, 1.0, (G, V))
    q = np.exp(dl - dl.max(axis=1, keepdims=True))
    q /= q.sum(axis=1, keepdims=True)
    return target, q.astype(np.float32)


def test_first_token_follows_target():
    rng = np.random.default_rng(1)
    target, q = make_case(rng, 5, 1)
    qn = q.astype(np.float64) / q.astype(np.float64).sum(axis=1, keepdims=True)
    law = law_at_position(target, qn.astype(np.float32), [], 0, {})
    want = pi_of(target[0])
    # grid integration error: at most one grid cell per breakpoint per token
    assert np.abs(law - want).max() < 6.0 / N_GRID


def test_second_token_follows_target_given_acceptance():
    rng = np.random.default_rng(2)
    target, q = make_case(rng, 4, 2)
    law = law_at_position(target, q, [int(np.argmax(target[0]))], 1, {"top_p": 0.95})
    want = pi_of(target[1], top_p=0.95)
    assert np.abs(law - want * law.sum()).max() < 6.0 / N_GRID
    assert abs(law.sum() - 1.0) < 6.0 / N_GRID


def test_bonus_token_after_full_acceptance():
    rng = np.random.default_rng(3)
    target, q = make_case(rng, 6, 2)
    drafts = [int(np.argmax(target[0])), int(np.argmax(target[1]))]
    counts = np.zeros(6)
    for us in (np.arange(1 << 16) + 0.5) / (1 << 16):
        def uni(dom, pos, us=us):
            return 0.0 if dom == philox.ACCEPT else us
        r = call(target, q, drafts, uni=uni)
        assert r.n_acc == 2
        counts[r.tokens[2]] += 1
    assert np.abs(counts / counts.sum() - pi_of(target[2])).max() < 2.0 / (1 << 16)


def test_expected_accepted_closed_form():
    rng = np.random.default_rng(4)
    V, G, n = 8, 3, 6000
    target, q = make_case(rng, V, G, scale=1.0)
    pis = [pi_of(target[j]) for j in range(G)]
    qd = q.astype(np.float64)
    beta = [np.minimum(pis[j], qd[j] / qd[j].sum()).sum() for j in range(G)]
    want = sum(np.prod(beta[:k]) for k in range(1, G + 1))
    drng = np.random.default_rng(99)
    acc = []
    firsts = []
    for t in range(n):
        d = [int(drng.choice(V, p=qd[j] / qd[j].sum())) for j in range(G)]
        r = call(target, q, d, seed=1234, request=t, position=0)
        acc.append(r.n_acc)
        firsts.append(r.tokens[0])
        assert 1 <= np.count_nonzero(r.tokens >= 0) == r.n_acc + 1 <= G + 1
        assert list(r.tokens[:r.n_acc]) == d[:r.n_acc]
    acc = np.array(acc, dtype=np.float64)
    assert abs(acc.mean() - want) < 4.5 * acc.std() / np.sqrt(n)
    obs = np.bincount(firsts, minlength=V)
    assert stats.chisquare(obs, pis[0] * n).pvalue > 1e-4


def test_greedy_exact_match_acceptance():
    rng = np.random.default_rng(5)
    V, G = 30, 4
    target = rng.standard_normal((G + 1, V)).astype(np.float32)
    g = [int(np.argmax(target[j])) for j in range(G + 1)]
    q = np.full((G, V), 1.0 / V, np.float32)
    for m in range(G + 1):
        d = g[:m] + [(g[j] + 1) % V for j in range(m, G)]
        r = call(target, q, d, T=0.0)
        assert r.n_acc == m
        assert list(r.tokens[:m + 1]) == g[:m + 1]
        assert np.all(r.tokens[m + 1:] == -1)


def test_draft_prefix_enters_penalty_history():
    # with a huge frequency penalty a token already drafted cannot be accepted again
    V = 10
    target = np.zeros((3, V), np.float32)
    target[:, 4] = 5.0
    q = np.full((2, V), 0.1, np.float32)
    r = call(target, q, [4, 4], T=1.0, freq=100.0, uni=lambda dom, pos: 0.5)
    assert r.n_acc == 1 and r.tokens[0] == 4 and r.tokens[1] != 4


# --- greedy drafts (q one-hot at the draft token) -----------------------------

def test_greedy_draft_closed_form():
    # equal 4-token row: pi = 1/4 each. Draft d = 1 with one-hot q: accept iff
    # u < pi(1) = 1/4; on rejection the residual is pi without token 1, i.e.
    # 1/3 on each of tokens 0, 2, 3 in id order (breakpoints 1/3, 2/3)
    target = np.zeros((2, 4), np.float32)

    def run(ua, ur):
        def uni(dom, pos):
            return {philox.ACCEPT: ua, philox.RESIDUAL: ur}.get(dom, 0.1)
        return call(target, None, [1], uni=uni)

    r = run(0.24, 0.5)
    assert r.n_acc == 1 and r.tokens[0] == 1
    assert r.accept_ratios == [0.25]
    for ur, tok in ((0.2, 0), (0.34, 2), (0.5, 2), (0.67, 3), (0.99, 3)):
        r = run(0.26, ur)
        assert r.n_acc == 0 and r.tokens[0] == tok, (ur, r.tokens)
        assert r.tokens[1] == -1


def test_greedy_draft_first_token_follows_target():
    # the rejection rule's law holds for any q, one-hot included: integrate the
    # first emitted token over the uniforms for each possible draft token
    rng = np.random.default_rng(6)
    V = 5
    target = (rng.standard_normal((2, V)) * 1.5).astype(np.float32)
    pi = pi_of(target[0])
    for d in range(V):
        # acceptance share over the accept uniform, then the law of the
        # residual token over the residual uniform given a rejection
        acc = sum(call(target, None, [d], uni=lambda dom, pos, ua=ua:
                       ua if dom == philox.ACCEPT else 0.5).n_acc for ua in GRID) / N_GRID
        rho = np.zeros(V)
        for ur in GRID:
            r = call(target, None, [d], uni=lambda dom, pos, ur=ur:
                     1.0 - 2.0 ** -24 if dom == philox.ACCEPT else ur)
            if r.n_acc == 0:
                rho[r.tokens[0]] += 1
        law = acc * np.eye(V)[d]
        if rho.sum() > 0:
            law += (1.0 - acc) * rho / rho.sum()
        assert np.abs(law - pi).max() < 6.0 / N_GRID, (d, law, pi)


def test_greedy_draft_probs_shape_and_out_of_range_ids():
    q = S.greedy_draft_probs([2, -1, 7], 5)
    assert q.dtype == np.float32 and q.shape == (3, 5)
    assert q[0].tolist() == [0, 0, 1, 0, 0]
    assert not q[1].any() and not q[2].any()


def test_append_to_sequences():
    seq = np.full((3, 6), -9, np.int32)
    ln = np.array([1, 4, 6], np.int32)
    res = [S.SpecResult(np.array([5, 6, 7], np.int32), 2, False, []),
           S.SpecResult(np.array([8, 9, -1], np.int32), 1, False, []),
           S.SpecResult(np.array([3, -1, -1], np.int32), 0, False, [])]
    S.append_to_sequences(seq, ln, 6, res)
    assert seq[0].tolist() == [-9, 5, 6, 7, -9, -9] and ln[0] == 4
    assert seq[1].tolist() == [-9, -9, -9, -9, 8, 9] and ln[1] == 6
    assert seq[2].tolist() == [-9] * 6 and ln[2] == 6  # full: nothing written
    ln2 = np.array([5], np.int32)
    seq2 = np.zeros((1, 6), np.int32)
    S.append_to_sequences(seq2, ln2, 6, res[:1])  # only one slot left
    assert seq2[0].tolist() == [0, 0, 0, 0, 0, 5] and ln2[0] == 6
