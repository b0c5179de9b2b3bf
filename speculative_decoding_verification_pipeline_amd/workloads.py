"""Seeded synthetic workloads for the five sampling configurations.

This module only builds inputs. It holds none of the sampling method's
arithmetic, so both the GPU path and the CPU oracle can be fed from it. Every
array is a host numpy array; callers move them to the device themselves.

Recipes (all numpy PCG64 generators; data seeds 101..105 are fixed here):
  low_entropy     B=4, V=32000 float32. N(0,1) logits with 5 distinct ids per
                  row raised by +8. T=0.8, top_k=50, top_p=0.9, no penalties,
                  bias or mask. Sampler seed 0, one draw per row.
  heterogeneous   B=64, V=128256 float32 Zipf rows: logit of rank r is
                  -4.4 ln r + N(0, 0.3), placed at a fresh permutation per row.
                  Per row: T in {0, 0.7, 1.0}; top_k in {off, 20, 50, 1000};
                  top_p in {1, 0.9, 0.95}; min_p in {0, 0.05}; repetition 1.1;
                  frequency and presence U(0, 0.5); 512 history ids drawn with
                  replacement; 16 distinct logit-bias ids with values U(-5, 5).
  grammar         B=256, V=152064 Zipf rows cast to bfloat16 (round to nearest
                  even). T, top_k, top_p mixed as above, no min_p, penalties or
                  bias. Packed LSB-first uint32 allow-mask per row with density
                  U[0.01, 0.5], at least one allowed token.
  speculative     B=32, G=4, V=128256. Target [32, 5, V] Zipf float32; draft
                  logits = target[:, :4] + N(0, 0.5); draft probabilities =
                  softmax of the draft logits (binary64, stored float32); draft
                  tokens drawn from them with numpy's generator (or, for a
                  greedy draft, each draft row's argmax); 16 requests greedy
                  (T=0), the others T=1 with no filters.
  lmhead          hidden [64, 8192] bf16 from N(0,1); weight [128256, 8192] bf16
                  from N(0, 0.02^2); T=1.0.
  tree            B=32 requests, N=16-node static draft trees (4 children at the
                  root, 2 below each, then chains), V=128256 f32 Zipf target
                  rows per node; children carry the top tokens of draft logits
                  = target row + N(0, 0.5); 16 requests greedy, the others T=1
                  with no filters.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

ZIPF_SLOPE = -1.1 * 4.0
ZIPF_NOISE = 0.3


def f32_to_bf16_bits(x):
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return b.astype(np.uint16)


def pack_mask(allowed):
    """Pack a boolean [.., V] allow-array into LSB-first uint32 words [.., ceil(V/32)]."""
    allowed = np.asarray(allowed, dtype=bool)
    V = allowed.shape[-1]
    nw = (V + 31) // 32
    pad = np.zeros(allowed.shape[:-1] + (nw * 32,), dtype=bool)
    pad[..., :V] = allowed
    bits = pad.reshape(allowed.shape[:-1] + (nw, 32)).astype(np.uint64)
    weights = (np.uint64(1) << np.arange(32, dtype=np.uint64))
    return (bits * weights).sum(axis=-1).astype(np.uint32)


def zipf_rows(rng, B, V):
    """B rows of permuted Zipf-shaped float32 logits."""
    base = ZIPF_SLOPE * np.log(np.arange(1, V + 1, dtype=np.float64))
    out = np.empty((B, V), dtype=np.float32)
    for b in range(B):
        vals = base + rng.normal(0.0, ZIPF_NOISE, V)
        out[b, rng.permutation(V)] = vals.astype(np.float32)
    return out


@dataclass
class SampleWorkload:
    name: str
    logits: np.ndarray                 # [B, V] float32, or uint16 bf16 bits
    dtype: str                         # "f32" or "bf16"
    temperature: np.ndarray
    top_k: np.ndarray
    top_p: np.ndarray
    min_p: np.ndarray
    rep: np.ndarray | None = None
    freq: np.ndarray | None = None
    pres: np.ndarray | None = None
    hist: np.ndarray | None = None     # [B, H] int32
    bias_ids: np.ndarray | None = None  # [B, NB] int32
    bias_vals: np.ndarray | None = None  # [B, NB] float32
    mask: np.ndarray | None = None     # [B, words] uint32
    request_ids: np.ndarray | None = None
    positions: np.ndarray | None = None
    seed: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def B(self):
        return self.logits.shape[0]

    @property
    def V(self):
        return self.logits.shape[1]


def _mixed_params(rng, B, with_minp=True):
    T = rng.choice(np.array([0.0, 0.7, 1.0], dtype=np.float32), B)
    top_k = rng.choice(np.array([0, 20, 50, 1000], dtype=np.int32), B)
    top_p = rng.choice(np.array([1.0, 0.9, 0.95], dtype=np.float32), B)
    if with_minp:
        min_p = rng.choice(np.array([0.0, 0.05], dtype=np.float32), B)
    else:
        min_p = np.zeros(B, dtype=np.float32)
    return T.astype(np.float32), top_k, top_p.astype(np.float32), min_p.astype(np.float32)


def low_entropy(B=4, V=32000, seed=101):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, V)).astype(np.float32)
    for b in range(B):
        ids = rng.choice(V, 5, replace=False)
        x[b, ids] += np.float32(8.0)
    return SampleWorkload(
        "low_entropy", x, "f32",
        temperature=np.full(B, 0.8, np.float32), top_k=np.full(B, 50, np.int32),
        top_p=np.full(B, 0.9, np.float32), min_p=np.zeros(B, np.float32),
        request_ids=np.arange(B, dtype=np.int32), positions=np.zeros(B, np.int32), seed=0)


def heterogeneous(B=64, V=128256, H=512, NB=16, seed=102):
    rng = np.random.default_rng(seed)
    x = zipf_rows(rng, B, V)
    T, top_k, top_p, min_p = _mixed_params(rng, B)
    hist = rng.integers(0, V, (B, H), dtype=np.int64).astype(np.int32)
    bias_ids = np.stack([rng.choice(V, NB, replace=False) for _ in range(B)]).astype(np.int32)
    bias_vals = rng.uniform(-5.0, 5.0, (B, NB)).astype(np.float32)
    return SampleWorkload(
        "heterogeneous", x, "f32", T, top_k, top_p, min_p,
        rep=np.full(B, 1.1, np.float32),
        freq=rng.uniform(0.0, 0.5, B).astype(np.float32),
        pres=rng.uniform(0.0, 0.5, B).astype(np.float32),
        hist=hist, bias_ids=bias_ids, bias_vals=bias_vals,
        request_ids=np.arange(B, dtype=np.int32), positions=np.zeros(B, np.int32), seed=0)


def grammar(B=256, V=152064, seed=103):
    rng = np.random.default_rng(seed)
    x = zipf_rows(rng, B, V)
    bits = f32_to_bf16_bits(x)
    T, top_k, top_p, min_p = _mixed_params(rng, B, with_minp=False)
    dens = rng.uniform(0.01, 0.5, B)
    allowed = rng.random((B, V)) < dens[:, None]
    for b in range(B):
        if not allowed[b].any():
            allowed[b, rng.integers(0, V)] = True
    return SampleWorkload(
        "grammar", bits, "bf16", T, top_k, top_p, min_p, mask=pack_mask(allowed),
        request_ids=np.arange(B, dtype=np.int32), positions=np.zeros(B, np.int32), seed=0)


@dataclass
class SpecWorkload:
    target: np.ndarray        # [B, G+1, V] float32
    draft_probs: np.ndarray   # [B, G, V] float32
    draft_tokens: np.ndarray  # [B, G] int32
    temperature: np.ndarray
    top_k: np.ndarray
    top_p: np.ndarray
    min_p: np.ndarray
    request_ids: np.ndarray
    positions: np.ndarray
    seed: int = 0

    @property
    def B(self):
        return self.target.shape[0]

    @property
    def G(self):
        return self.draft_tokens.shape[1]

    @property
    def V(self):
        return self.target.shape[2]


def speculative(B=32, G=4, V=128256, seed=104, draft_seed=1, n_greedy=None,
                greedy_draft=False):
    rng = np.random.default_rng(seed)
    target = zipf_rows(rng, B * (G + 1), V).reshape(B, G + 1, V)
    draft = target[:, :G].astype(np.float64) + rng.normal(0.0, 0.5, (B, G, V))
    draft -= draft.max(axis=-1, keepdims=True)
    q = np.exp(draft)
    q /= q.sum(axis=-1, keepdims=True)
    qf = q.astype(np.float32)
    drng = np.random.default_rng(draft_seed)
    toks = np.empty((B, G), dtype=np.int32)
    for b in range(B):
        for j in range(G):
            if greedy_draft:  # the draft takes its top token
                toks[b, j] = int(np.argmax(draft[b, j]))
                continue
            c = np.cumsum(q[b, j])
            toks[b, j] = min(int(np.searchsorted(c, drng.random() * c[-1], side="right")), V - 1)
    n_greedy = B // 2 if n_greedy is None else n_greedy
    T = np.ones(B, dtype=np.float32)
    T[rng.permutation(B)[:n_greedy]] = 0.0
    return SpecWorkload(target, qf, toks, T, np.zeros(B, np.int32), np.ones(B, np.float32),
                        np.zeros(B, np.float32), np.arange(B, dtype=np.int32),
                        np.zeros(B, np.int32), seed=0)


@dataclass
class LMHeadWorkload:
    hidden: np.ndarray   # [B, K] uint16 bf16 bits
    weight: np.ndarray   # [V, K] uint16 bf16 bits
    temperature: np.ndarray
    request_ids: np.ndarray
    positions: np.ndarray
    seed: int = 0


def lmhead(B=64, K=8192, V=128256, seed=105, chunk=4096):
    rng = np.random.default_rng(seed)
    hidden = f32_to_bf16_bits(rng.standard_normal((B, K), dtype=np.float32))
    weight = np.empty((V, K), dtype=np.uint16)
    for v0 in range(0, V, chunk):
        n = min(chunk, V - v0)
        w = rng.standard_normal((n, K), dtype=np.float32) * np.float32(0.02)
        weight[v0:v0 + n] = f32_to_bf16_bits(w)
    return LMHeadWorkload(hidden, weight, np.ones(B, np.float32),
                          np.arange(B, dtype=np.int32), np.zeros(B, np.int32), seed=0)


@dataclass
class TreeWorkload:
    target: np.ndarray       # [B, N, V] float32
    parents: np.ndarray      # [B, N] int32
    tokens: np.ndarray       # [B, N] int32
    temperature: np.ndarray
    top_k: np.ndarray
    top_p: np.ndarray
    min_p: np.ndarray
    request_ids: np.ndarray
    positions: np.ndarray
    seed: int = 0

    @property
    def B(self):
        return self.target.shape[0]

    @property
    def N(self):
        return self.target.shape[1]

    @property
    def V(self):
        return self.target.shape[2]


def tree_shape(N, branching=(4, 2, 1)):
    """Parent indices of a static draft tree of N nodes built breadth-first:
    each node at depth k gets branching[k] children (the last entry repeats)
    until N nodes exist."""
    parents = [-1]
    frontier = [0]
    k = 0
    while len(parents) < N and frontier:
        nxt = []
        for p in frontier:
            for _ in range(branching[min(k, len(branching) - 1)]):
                if len(parents) == N:
                    break
                parents.append(p)
                nxt.append(len(parents) - 1)
        frontier = nxt
        k += 1
    return np.array(parents, dtype=np.int32)


def tree(B=32, N=16, V=128256, seed=107, n_greedy=None, branching=(4, 2, 1)):
    """Draft trees: the same static shape for every request; each node's
    children carry its draft's top-K tokens, the draft logits being the target
    row plus N(0, 0.5) noise. Target rows are Zipf rows; half the requests are
    greedy (T = 0), the others T = 1 with no filters."""
    rng = np.random.default_rng(seed)
    target = zipf_rows(rng, B * N, V).reshape(B, N, V)
    parents = np.tile(tree_shape(N, branching), (B, 1))
    tokens = np.zeros((B, N), dtype=np.int32)
    for b in range(B):
        for x in range(N):
            kids = np.nonzero(parents[b] == x)[0]
            kids = kids[kids > 0]
            if kids.size == 0:
                continue
            draft = target[b, x].astype(np.float64) + rng.normal(0.0, 0.5, V)
            top = np.argsort(-draft, kind="stable")[:kids.size]
            tokens[b, kids] = top.astype(np.int32)
    n_greedy = B // 2 if n_greedy is None else n_greedy
    T = np.ones(B, dtype=np.float32)
    T[rng.permutation(B)[:n_greedy]] = 0.0
    return TreeWorkload(target, parents, tokens, T, np.zeros(B, np.int32), np.ones(B, np.float32),
                        np.zeros(B, np.float32), np.arange(B, dtype=np.int32),
                        np.zeros(B, np.int32), seed=0)
