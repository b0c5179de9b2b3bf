"""Pins for the oracle's tree verification (CPU only).

* Tree bookkeeping: depths, paths and unreachable nodes of hand-made trees.
* A chain (one child per node) is linear verification with a greedy draft: the
  outputs equal verify_request's with draft_probs=None, token for token, over
  seeds, positions, temperatures, filters and penalties.
* Closed form on an equal 4-token row with two root children: the first is
  accepted iff u_0 < 1/4, the second iff u_1 < (1/4) / (3/4) = 1/3, otherwise
  the residual puts 1/2 on each of the two remaining tokens in id order.
* Greedy trees accept the branch whose token is the target's greedy token.
* The law of the first emitted token with three root children is the target's
  filtered distribution (the rejection rule's defining property), checked by a
  chi-square test over Philox draws.
"""
import numpy as np
from scipy import stats

from oracle import philox
from oracle import pipeline as P
from oracle import spec as S


def test_tree_nodes_depths_paths_and_unreachable():
    parents = [-1, 0, 0, 1, 3, 7, 2, 9, 4]
    depth, path = S.tree_nodes(parents)
    assert depth == [0, 1, 1, 2, 3, -1, 2, -1, 4]
    assert path[4] == [1, 3, 4] and path[6] == [2, 6] and path[8] == [1, 3, 4, 8]
    assert path[5] is None and path[7] is None  # parent after the node / out of range
    assert S.tree_children(parents, depth, 0) == [1, 2]
    assert S.tree_children(parents, depth, 3) == [4]
    assert S.tree_children(parents, depth, 8) == []


def _rows(rng, N, V, scale=2.0):
    return (rng.standard_normal((N, V)) * scale).astype(np.float32)


def test_chain_is_linear_greedy_draft_verification():
    rng = np.random.default_rng(21)
    V, G = 40, 4
    for trial in range(60):
        target = _rows(rng, G + 1, V)
        T = float(rng.choice([0.0, 0.7, 1.0, 1.6]))
        kw = dict(temperature=T, top_k=int(rng.choice([0, 5])), top_p=float(rng.choice([1.0, 0.9])),
                  min_p=float(rng.choice([0.0, 0.05])), rep=1.2, freq=0.3, pres=0.1,
                  hist=rng.integers(0, V, 6).tolist())
        # drafts near the target's greedy tokens so that acceptance is common
        d = [int(np.argmax(target[j])) if rng.random() < 0.7 else int(rng.integers(0, V))
             for j in range(G)]
        parents = [-1] + list(range(G))
        tokens = [0] + d
        pos = int(rng.integers(0, 1 << 20))
        lin = S.verify_request(target, None, d, seed=trial, request=3, position=pos, **kw)
        tree = S.verify_tree(target, parents, tokens, seed=trial, request=3, position=pos, **kw)
        assert tree.n_acc == lin.n_acc, trial
        assert tree.tokens.tolist() == lin.tokens.tolist(), trial
        assert tree.nodes[:tree.n_acc].tolist() == list(range(1, tree.n_acc + 1))
        assert tree.flagged == lin.flagged


def test_two_children_closed_form():
    target = np.zeros((3, 4), np.float32)  # pi = 1/4 on each token at every node
    parents, tokens = [-1, 0, 0], [0, 1, 2]

    def run(u0, u1, ur):
        def uni(dom, pos, draw=0):
            if dom == philox.ACCEPT:
                return (u0, u1)[draw]
            return ur if dom == philox.RESIDUAL else 0.3
        return S.verify_tree(target, parents, tokens, temperature=1.0, uniform=uni)

    r = run(0.24, 0.9, 0.5)
    assert r.n_acc == 1 and r.nodes[0] == 1 and r.tokens[0] == 1
    assert r.tokens[1] == 1  # leaf: the bonus draw at u = 0.3 is token 1 of (1/4)-steps
    r = run(0.26, 0.33, 0.5)
    assert r.n_acc == 1 and r.nodes[0] == 2 and r.tokens[0] == 2
    for ur, tok in ((0.1, 0), (0.49, 0), (0.51, 3), (0.99, 3)):
        r = run(0.26, 0.34, ur)  # both rejected: residual 1/2 on tokens 0 and 3
        assert r.n_acc == 0 and r.tokens[0] == tok and r.tokens[1] == -1, (ur, r.tokens)


def test_greedy_tree_takes_the_matching_branch():
    V = 10
    target = np.zeros((6, V), np.float32)
    target[0, 7] = 5.0   # root's greedy token: 7
    target[2, 3] = 5.0   # after node 2 (token 7): 3
    target[4, 9] = 5.0   # after node 4 (token 3): 9
    target[5, 1] = 5.0
    parents = [-1, 0, 0, 1, 2, 2]
    tokens = [0, 4, 7, 7, 3, 8]
    r = S.verify_tree(target, parents, tokens, temperature=0.0)
    assert r.n_acc == 2 and r.nodes[:2].tolist() == [2, 4]
    assert r.tokens[:3].tolist() == [7, 3, 9] and r.tokens[3] == -1


def test_first_token_law_with_three_children():
    rng = np.random.default_rng(8)
    V = 6
    target = _rows(rng, 4, V, 1.0)
    pi = P.filter_row(target[0], 1.0, 0, 1.0, 0.0).probs
    order = np.argsort(-pi)
    parents, tokens = [-1, 0, 0, 0], [0, int(order[0]), int(order[2]), int(order[1])]
    n = 20000
    first = np.zeros(V)
    for t in range(n):
        r = S.verify_tree(target, parents, tokens, temperature=1.0, seed=5, request=t, position=11)
        first[r.tokens[0]] += 1
    assert stats.chisquare(first, pi * n).pvalue > 1e-4
