"""Speculative verification by rejection sampling (oracle; test infrastructure only).

What it follows
---------------
"Accelerating Sonar through speculation" (Perplexity blog): a draft proposes n
tokens and the target verifies them, so one step emits up to n + 1 tokens
(section on speculative decoding); acceptance compares the full draft and target
distributions and the target's logits after the accepted prefix are sampled for
one extra token (section on target-draft decoding). Its reference list names
"Fast inference from transformers via speculative decoding", the source of the
rejection rule. SonicSampler's abstract puts verification inside the same
batched sampler as the logit processing. The rule itself (a reading consistent
with all of these):

For request b, position j = 0 .. G-1 in order, with target row j processed by
the full per-request pipeline (the penalty history of row j is the request's
history followed by the draft tokens d_0 .. d_{j-1}, since row j is only reached
if those were accepted; a per-position grammar mask is used when given):
  * greedy (T == 0): accept iff d_j equals the greedy token of row j; otherwise
    emit that greedy token and stop.
  * T > 0: with pi_j the filtered target distribution and q_j the draft
    probabilities, draw u = u24(Philox ACCEPT word at (seed, request, pos + j, 0))
    and accept iff u < pi_j(d_j) / q_j(d_j) (if q_j(d_j) == 0: accept iff
    pi_j(d_j) > 0); the decision is flagged when |u - pi/q| < 1e-6, whichever
    side of 1 the ratio lies. On the first rejection draw u' = u24(Philox RESIDUAL word at
    (seed, request, pos + j, 0)) and emit the token of the normalised residual
    r = max(0, pi_j - q_j) by inverse CDF in ascending token-id order (pi_j if
    the residual sums to zero); then stop.
  * If all G drafts are accepted, the bonus token is sampled from row G exactly
    as the plain sampler would (SAMPLE word at (seed, request, pos + G, 0)).
Output: tokens d_0 .. d_{n-1}, the final token, then -1 padding to G + 1;
n_acc = n in [0, G].

The residual CDF runs in token-id order (not by residual size) because the
residual's values are binary64 here and binary32 on a GPU: an ordering by them
could differ between the two sides by whole tokens, while an id-ordered CDF can
only move its breakpoints by rounding.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import philox
from .pipeline import BOUNDARY_EPS, boundary_draw, draw, filter_row, process_row


@dataclass
class SpecResult:
    tokens: np.ndarray      # [G+1] int32, -1 padded
    n_acc: int
    flagged: bool           # a decision of this request lies on a boundary
    accept_ratios: list     # per examined position: pi/q (sampling) or None


def residual_draw(pi, q, u):
    """Inverse CDF in token-id order over max(0, pi - q); returns (token, flagged)."""
    r = np.maximum(0.0, np.asarray(pi, dtype=np.float64) - np.asarray(q, dtype=np.float64))
    R = r.sum()
    if not R > 0.0:
        r = np.asarray(pi, dtype=np.float64).copy()
        R = r.sum()
    if not R > 0.0:
        return -1, False
    pos = np.nonzero(r > 0.0)[0]
    cdf = np.cumsum(r[pos]) / R
    i = int(np.searchsorted(cdf, u, side="right"))
    i = min(i, pos.size - 1)
    return int(pos[i]), boundary_draw(cdf, u)


def greedy_draft_probs(draft_tokens, V):
    """The draft distributions of a draft model that takes its top token at every
    step ("Accelerating Sonar through speculation", Perplexity blog, section on
    target-draft decoding: the draft samples its top token): one-hot at each
    draft token, [G, V] binary32. An id outside [0, V) gives an all-zero row.

    With this q the general rule specialises to: accept d_j iff u < pi_j(d_j);
    on rejection the residual max(0, pi_j - q_j) is pi_j with d_j removed."""
    G = len(draft_tokens)
    q = np.zeros((G, V), dtype=np.float32)
    for j, d in enumerate(draft_tokens):
        if 0 <= int(d) < V:
            q[j, int(d)] = 1.0
    return q


def append_to_sequences(seq_tokens, seq_len, capacity, results):
    """Device-side bookkeeping after verification (Perplexity blog, section on
    single-token MTP scheduling: after acceptance a kernel places the next
    target tokens into their slots, so no GPU-to-CPU synchronisation is needed).

    Reading: each request's emitted tokens -- its accepted drafts, then its final
    token -- are appended to its token sequence at its current length, and the
    length advances by their number; slots at or beyond `capacity` are not
    written and the length stops at `capacity`. seq_tokens [B, >= capacity] and
    seq_len [B] are updated in place (numpy int32 arrays)."""
    for b, r in enumerate(results):
        n = r.n_acc + 1
        L = int(seq_len[b])
        for k in range(n):
            if 0 <= L + k < capacity:
                seq_tokens[b, L + k] = r.tokens[k]
        seq_len[b] = min(L + n, capacity)


def filtered_rows(target_rows, draft_tokens, *, temperature, top_k=0, top_p=1.0, min_p=0.0,
                  rep=1.0, freq=0.0, pres=0.0, hist=(), bias_ids=(), bias_vals=(), masks=None):
    """rows(j): target row j's filtered distribution, formed on first use.

    Row j is processed with the request's history followed by the draft tokens
    d_0 .. d_{j-1} (it is only reached if those were accepted) and, when given,
    its own position's grammar mask. It depends on neither the seed nor the
    position, so one rows() serves every draw over the same request.
    """
    hist = [int(h) for h in hist]
    cache = {}

    def rows(j):
        if j not in cache:
            hj = hist + [int(d) for d in draft_tokens[:j]]
            mj = None if masks is None else masks[j]
            xp = process_row(target_rows[j], hj, rep, freq, pres, bias_ids, bias_vals, mj)
            cache[j] = filter_row(xp, temperature, top_k, top_p, min_p)
        return cache[j]

    return rows


def verify_request(target_rows, draft_probs, draft_tokens, *, temperature, top_k=0,
                   top_p=1.0, min_p=0.0, rep=1.0, freq=0.0, pres=0.0, hist=(),
                   bias_ids=(), bias_vals=(), masks=None, seed=0, request=0, position=0,
                   uniform=None, rows=None):
    """Verify one request's linear draft. target_rows: [G+1, V] float32;
    draft_probs: [G, V] float32, or None for a greedy draft (greedy_draft_probs).

    uniform(domain, pos) -> u overrides the Philox uniforms (used by tests that
    integrate over the uniforms); by default u = u24 of the Philox word at
    (seed, request, pos, draw 0, domain).
    rows: the request's filtered_rows() (tests that sweep seeds and positions
    over fixed rows form it once); by default it is formed here.
    """
    if uniform is None:
        def uniform(domain, pos):
            return philox.uniform(seed, request, pos, 0, domain)
    G = len(draft_tokens)
    if draft_probs is None:
        draft_probs = greedy_draft_probs(draft_tokens, target_rows.shape[1])
    out = np.full(G + 1, -1, dtype=np.int32)
    flagged = False
    ratios = []
    if rows is None:
        rows = filtered_rows(target_rows, draft_tokens, temperature=temperature, top_k=top_k,
                             top_p=top_p, min_p=min_p, rep=rep, freq=freq, pres=pres, hist=hist,
                             bias_ids=bias_ids, bias_vals=bias_vals, masks=masks)
    for j in range(G + 1):
        filt = rows(j)
        flagged = flagged or filt.flag_topp or filt.flag_minp
        if j == G:
            u = uniform(philox.SAMPLE, position + G)
            res = draw(filt, u)
            out[G] = res.token
            return SpecResult(out, G, flagged or res.flag_draw, ratios)
        d = int(draft_tokens[j])
        if filt.greedy or filt.n_kept == 0:
            g = filt.argmax if filt.n_kept else -1
            ratios.append(None)
            if g >= 0 and d == g:
                out[j] = d
                continue
            out[j] = g
            return SpecResult(out, j, flagged, ratios)
        p = float(filt.probs[d]) if 0 <= d < len(filt.probs) else 0.0
        q = float(draft_probs[j][d]) if 0 <= d < len(filt.probs) else 0.0
        u = uniform(philox.ACCEPT, position + j)
        if q > 0.0:
            ratio = p / q
            accept = u < ratio
            # the decision u < ratio is a boundary case whenever u lies within
            # 1e-6 of the ratio, on either side of 1: a ratio just above 1 in
            # binary64 can round below u on a binary32 device
            if abs(u - ratio) < BOUNDARY_EPS:
                flagged = True
        else:
            ratio = np.inf if p > 0.0 else 0.0
            accept = p > 0.0
        ratios.append(ratio)
        if accept:
            out[j] = d
            continue
        u2 = uniform(philox.RESIDUAL, position + j)
        tok, fl = residual_draw(filt.probs, draft_probs[j], u2)
        out[j] = tok
        return SpecResult(out, j, flagged or fl, ratios)
    raise AssertionError("unreachable")


def _filter_args(params, b):
    pr = params.row(b)
    return dict(temperature=float(params.temperature[b]), top_k=int(params.top_k[b]),
                top_p=float(params.top_p[b]), min_p=float(params.min_p[b]),
                rep=pr["rep"], freq=pr["freq"], pres=pr["pres"], hist=pr["hist"],
                bias_ids=pr["bias_ids"], bias_vals=pr["bias_vals"],
                masks=None if params.mask is None else params.mask[b])


def batch_rows(target, draft_tokens, params):
    """filtered_rows() of every request of a batch (seed and position independent)."""
    return [filtered_rows(target[b], draft_tokens[b], **_filter_args(params, b))
            for b in range(target.shape[0])]


def verify_batch(target, draft_probs, draft_tokens, params, rows=None):
    """target [B, G+1, V] f32, draft_probs [B, G, V] f32 (None: greedy drafts),
    draft_tokens [B, G] int. rows: batch_rows() of the same target, drafts and
    parameters, or None."""
    res = []
    for b in range(target.shape[0]):
        pr = params.row(b)
        res.append(verify_request(
            target[b], None if draft_probs is None else draft_probs[b], draft_tokens[b],
            **_filter_args(params, b),
            seed=params.seed, request=pr["request"], position=pr["position"],
            rows=None if rows is None else rows[b]))
    return res


# --- tree verification ---------------------------------------------------------

@dataclass
class TreeResult:
    tokens: np.ndarray      # [N] int32: accepted path tokens, the final token, -1 padding
    nodes: np.ndarray       # [N] int32: tree node of each accepted token, -1 padding
    n_acc: int              # accepted path length (nodes below the root)
    flagged: bool           # a decision lies on a boundary


def tree_nodes(parents):
    """(depth, path) per node of a draft tree given as parent indices.

    Node 0 is the root (the last committed token): depth 0, empty path. Node
    n >= 1 hangs below parents[n], which must precede it (0 <= parents[n] < n);
    a node that breaks this, or hangs below such a node, is unreachable (depth
    -1). path[n] lists the nodes from the root's child down to n."""
    N = len(parents)
    depth = [-1] * N
    path = [None] * N
    depth[0], path[0] = 0, []
    for n in range(1, N):
        p = int(parents[n])
        if 0 <= p < n and depth[p] >= 0:
            depth[n] = depth[p] + 1
            path[n] = path[p] + [n]
    return depth, path


def tree_children(parents, depth, x):
    """Children of reachable node x in index order."""
    return [n for n in range(1, len(parents)) if depth[n] >= 0 and int(parents[n]) == x]


def tree_rows(target_rows, parents, tokens, *, temperature, top_k=0, top_p=1.0, min_p=0.0,
              rep=1.0, freq=0.0, pres=0.0, hist=(), bias_ids=(), bias_vals=(), masks=None):
    """rows(n): node n's filtered distribution, formed on first use. Node n is
    processed with the request history followed by the tokens on its root path
    and masks[n] when given; it depends on neither the seed nor the position."""
    depth, path = tree_nodes(parents)
    hist = [int(h) for h in hist]
    cache = {}

    def rows(n):
        if n not in cache:
            hx = hist + [int(tokens[m]) for m in (path[n] or [])]
            mx = None if masks is None else masks[n]
            xp = process_row(target_rows[n], hx, rep, freq, pres, bias_ids, bias_vals, mx)
            cache[n] = filter_row(xp, temperature, top_k, top_p, min_p)
        return cache[n]

    return rows


def verify_tree(target_rows, parents, tokens, *, temperature, top_k=0, top_p=1.0, min_p=0.0,
                rep=1.0, freq=0.0, pres=0.0, hist=(), bias_ids=(), bias_vals=(), masks=None,
                seed=0, request=0, position=0, uniform=None, rows=None):
    """Verify one request's draft tree ("Accelerating Sonar through speculation",
    Perplexity blog, EAGLE section: draft sequences explored as a tree in which
    each node considers its draft's top-K candidates; the longest acceptable
    path is kept and the target adds one token).

    target_rows [N, V] float32: row n holds the target's logits after the path
    root -> n (node 0 = the root). parents [N], tokens [N]: the tree (tokens[0]
    unused). Row n is processed with the request history followed by its path's
    tokens as penalty history, masks[n] when given, and the request's filters.

    Reading: the children of a node are deterministic candidates, so each is a
    one-hot proposal. Walking down from the root, the children of the current
    node are tested in index order against the residual target: child i with
    token d is accepted iff u_i < p(d) / (1 - sum of p over the tokens of the
    siblings already rejected), u_i = u24 of the ACCEPT word at (request,
    position + depth, draw i) (a token equal to a rejected sibling's has
    residual probability 0). An accepted child becomes the current node. If
    every child is rejected, the final token is drawn from p with the rejected
    tokens removed, by inverse CDF in token-id order (RESIDUAL word at position
    + depth, draw 0); at a leaf it is drawn from p as the plain sampler would
    (SAMPLE word at position + depth). Greedy rows (T = 0) accept the child
    whose token is the greedy token and end with the greedy token. With one
    child per node this is verify_request with a greedy draft.
    rows: the request's tree_rows() (tests sweeping seeds and positions form it
    once); by default it is formed here.
    """
    if uniform is None:
        def uniform(domain, pos, draw=0):
            return philox.uniform(seed, request, pos, draw, domain)
    N, V = target_rows.shape
    depth, path = tree_nodes(parents)
    if rows is None:
        rows = tree_rows(target_rows, parents, tokens, temperature=temperature, top_k=top_k,
                         top_p=top_p, min_p=min_p, rep=rep, freq=freq, pres=pres, hist=hist,
                         bias_ids=bias_ids, bias_vals=bias_vals, masks=masks)
    out_t = np.full(N, -1, dtype=np.int32)
    out_n = np.full(N, -1, dtype=np.int32)
    flagged = False
    cur, k = 0, 0
    while True:
        filt = rows(cur)
        flagged = flagged or filt.flag_topp or filt.flag_minp
        dpt = depth[cur]
        ch = tree_children(parents, depth, cur)
        if filt.greedy or filt.n_kept == 0:
            g = filt.argmax if filt.n_kept else -1
            nxt = next((c for c in ch if g >= 0 and int(tokens[c]) == g), None)
            if nxt is None:
                out_t[k] = g
                return TreeResult(out_t, out_n, k, flagged)
        else:
            nxt = None
            rejected = []
            remaining = 1.0
            for i, c in enumerate(ch):
                d = int(tokens[c])
                p = float(filt.probs[d]) if 0 <= d < V and d not in rejected else 0.0
                u = uniform(philox.ACCEPT, position + dpt, i)
                ratio = p / remaining if remaining > 0.0 else 0.0
                if abs(u - ratio) < BOUNDARY_EPS:
                    flagged = True
                if u < ratio:
                    nxt = c
                    break
                if 0 <= d < V and d not in rejected:
                    rejected.append(d)
                    remaining -= p
            if nxt is None:
                if ch:
                    q = np.zeros(V)
                    for d in rejected:
                        q[d] = 1.0
                    tok, fl = residual_draw(filt.probs, q, uniform(philox.RESIDUAL, position + dpt))
                else:
                    res = draw(filt, uniform(philox.SAMPLE, position + dpt))
                    tok, fl = res.token, res.flag_draw
                out_t[k] = tok
                return TreeResult(out_t, out_n, k, flagged or fl)
        out_t[k] = int(tokens[nxt])
        out_n[k] = nxt
        k += 1
        cur = nxt


def verify_tree_batch(target, parents, tokens, params, rows=None):
    """target [B, N, V] f32, parents / tokens [B, N] int. rows: per request
    tree_rows() of the same inputs, or None."""
    res = []
    for b in range(target.shape[0]):
        pr = params.row(b)
        res.append(verify_tree(target[b], parents[b], tokens[b], **_filter_args(params, b),
                               seed=params.seed, request=pr["request"], position=pr["position"],
                               rows=None if rows is None else rows[b]))
    return res


def batch_tree_rows(target, parents, tokens, params):
    """tree_rows() of every request of a batch."""
    return [tree_rows(target[b], parents[b], tokens[b], **_filter_args(params, b))
            for b in range(target.shape[0])]
