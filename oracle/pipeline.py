"""Per-request logit processing and sampling (oracle; test infrastructure only).

What it follows
---------------
SonicSampler abstract (arxivdaily page, English abstract): one batched kernel
applies, per request, grammar-constrained decoding, repetition / frequency /
presence penalties, logit bias, temperature scaling and top-k / top-p / min-p
filtering, then selects a token. The pages name these steps but give no
formulas, constants, tie rules or precision. Everything below that they leave
open is a stated reading:

  * Penalties (reading: the common CTRL / OpenAI forms). For every token v that
    occurs c_v > 0 times in the request's token history (ids outside [0, V) are
    ignored), in this order and each rounded to binary32:
        repetition  x = x / r   if x > 0   else  x * r   (once per distinct id)
        frequency   x = x - f32(f * f32(c_v))
        presence    x = x - p
  * Logit bias: x[id] = f32(x[id] + b) for every entry in array order, so
    duplicate ids accumulate in order; ids outside [0, V) are ignored.
  * Grammar mask: packed uint32 words, least-significant bit first, bit set =
    allowed. A disallowed token becomes -inf. -inf is fixed under every earlier
    step, so the mask commutes with them.
  * Temperature: T == 0 means greedy (lowest id among the maxima of the
    processed logits; no uniform is consumed). T > 0: z = f32(x / T).
  * Key order: z descending, then token id ascending (ties toward the lower id);
    -0.0 and +0.0 compare equal. Only finite z take part.
  * Weights w = exp(z - max z) in binary64.
  * top-k: k <= 0 or k >= V is off; otherwise the first k tokens in key order.
  * top-p: off when top_p >= 1. Otherwise with P the weights renormalised over
    the top-k set, token i (key order) is kept iff the sum of P over the tokens
    before it is < top_p, so the token that crosses top_p is kept.
  * min-p: off when min_p <= 0. Otherwise a token survives iff w >= min_p
    (w of the maximum is 1), applied after top-p.
  * Draw: pi = w / sum(w) over the kept prefix, C_i the inclusive cumulative sum
    in key order, token = first kept token with u < C_i (the last one if
    rounding leaves u >= every C_i), u = u24 of the Philox SAMPLE word at
    (seed, request, position, draw 0).

Flags (counted, not compared): a draw is a boundary draw if u lies within 1e-6
of any interior C_i; a top-p cut is flagged if a decisive exclusive cumulative
sum after the first token lies within 1e-6 of top_p; a min-p cut is flagged if
a surviving token after the first has a weight within 1e-6 of min_p (the first
token's exclusive sum 0 and weight 1 are exact everywhere). These are the cases a binary32 GPU cannot be
asked to decide the same way as this binary64 oracle.

Binary32 steps use numpy float32 scalars: one rounding per operation, no fused
multiply-add, correctly rounded division.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import philox

BOUNDARY_EPS = 1e-6


def bf16_bits_to_f32(bits):
    """Widen bfloat16 bit patterns (uint16) to float32 exactly."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def mask_allowed(mask_words, V):
    """Boolean allow-vector from packed LSB-first uint32 words."""
    words = np.asarray(mask_words, dtype=np.uint32)
    v = np.arange(V, dtype=np.int64)
    return ((words[v >> 5] >> (v & 31).astype(np.uint32)) & np.uint32(1)).astype(bool)


def process_row(x, hist_ids=(), rep=1.0, freq=0.0, pres=0.0,
                bias_ids=(), bias_vals=(), mask_words=None):
    """Penalties, then logit bias, then the grammar mask, all in binary32.

    x is one row of logits (float32, already widened if it was bf16).
    Returns the processed row x' (float32), compared bit for bit.
    """
    x = np.array(x, dtype=np.float32, copy=True)
    V = x.shape[0]
    r = np.float32(rep)
    f = np.float32(freq)
    p = np.float32(pres)
    counts = {}
    for t in hist_ids:
        t = int(t)
        if 0 <= t < V:
            counts[t] = counts.get(t, 0) + 1
    for v, c in counts.items():
        xv = x[v]
        if xv > np.float32(0.0):
            xv = np.float32(xv / r)
        else:
            xv = np.float32(xv * r)
        xv = np.float32(xv - np.float32(f * np.float32(c)))
        xv = np.float32(xv - p)
        x[v] = xv
    for t, b in zip(bias_ids, bias_vals):
        t = int(t)
        if 0 <= t < V:
            x[t] = np.float32(x[t] + np.float32(b))
    if mask_words is not None:
        x[~mask_allowed(mask_words, V)] = np.float32(-np.inf)
    return x


@dataclass
class Filtered:
    """The outcome of temperature + top-k + top-p + min-p on one row."""
    greedy: bool
    order: np.ndarray          # finite token ids in key order (z desc, id asc)
    w: np.ndarray              # binary64 weights exp(z - max z) in key order
    n_topk: int                # size of the top-k set (prefix length)
    n_topp: int                # size after top-p
    n_kept: int                # size after min-p (the sampling support)
    probs: np.ndarray          # dense binary64 probabilities over V
    topk_active: bool
    flag_topp: bool = False
    flag_minp: bool = False
    argmax: int = -1
    cdf: np.ndarray = field(default_factory=lambda: np.zeros(0))

    @property
    def kept_ids(self):
        return self.order[:self.n_kept]


def filter_row(xp, temperature, top_k, top_p, min_p):
    """Temperature, ordering, top-k, top-p and min-p on a processed row."""
    xp = np.asarray(xp, dtype=np.float32)
    V = xp.shape[0]
    T = np.float32(temperature)
    assert np.isfinite(T) and T >= 0, "temperature must be finite and >= 0"
    assert 0.0 < float(top_p) <= 1.0, "top_p must lie in (0, 1]"
    assert 0.0 <= float(min_p) <= 1.0, "min_p must lie in [0, 1]"
    finite = np.isfinite(xp)
    ids = np.nonzero(finite)[0]
    probs = np.zeros(V, dtype=np.float64)
    topk_active = 0 < int(top_k) < V
    if ids.size == 0:
        return Filtered(T == 0, ids, np.zeros(0), 0, 0, 0, probs, topk_active)
    if T == 0:
        am = int(np.argmax(np.where(finite, xp, -np.inf)))
        probs[am] = 1.0
        return Filtered(True, np.array([am]), np.ones(1), 1, 1, 1, probs, topk_active,
                        argmax=am, cdf=np.ones(1))
    z = (xp[ids] / T).astype(np.float32)  # elementwise binary32 division, correctly rounded
    z = z + np.float32(0.0)  # -0.0 -> +0.0 so both zeros share one key
    zs = z.astype(np.float64)
    perm = np.lexsort((ids, -zs))
    order = ids[perm]
    zo = zs[perm]
    w = np.exp(zo - zo[0])
    n = order.size
    n_topk = min(int(top_k), n) if topk_active else n
    flag_topp = False
    if float(top_p) < 1.0:
        P = w[:n_topk] / w[:n_topk].sum()
        excl = np.concatenate(([0.0], np.cumsum(P)[:-1]))
        tp = float(np.float32(top_p))
        n_topp = int(np.count_nonzero(excl < tp))
        # the exclusive sum before the first token is exactly 0 on any
        # implementation, so only later comparisons can be boundary cases
        near = [excl[n_topp - 1]] if n_topp > 1 else []
        if n_topp < n_topk:
            near.append(excl[n_topp])
        flag_topp = any(abs(e - tp) < BOUNDARY_EPS for e in near)
    else:
        n_topp = n_topk
    flag_minp = False
    if float(min_p) > 0.0:
        mp = float(np.float32(min_p))
        n_kept = int(np.count_nonzero(w[:n_topp] >= mp))
        # w of the first token is exactly 1 on any implementation
        flag_minp = bool(np.any(np.abs(w[1:n_topp] - mp) < BOUNDARY_EPS))
    else:
        n_kept = n_topp
    pk = w[:n_kept] / w[:n_kept].sum()
    probs[order[:n_kept]] = pk
    return Filtered(False, order, w, n_topk, n_topp, n_kept, probs, topk_active,
                    flag_topp, flag_minp, argmax=int(order[0]), cdf=np.cumsum(pk))


def inverse_cdf(cdf, u):
    """Index of the first breakpoint with u < C_i (vectorised over u), clamped."""
    idx = np.searchsorted(np.asarray(cdf), u, side="right")
    return np.minimum(idx, len(cdf) - 1)


def boundary_draw(cdf, u):
    """True if u is within 1e-6 of an interior breakpoint of the CDF."""
    if len(cdf) <= 1:
        return False
    return bool(np.min(np.abs(np.asarray(cdf[:-1]) - u)) < BOUNDARY_EPS)


@dataclass
class RowResult:
    token: int
    filt: Filtered
    u: float
    flag_draw: bool

    @property
    def flagged(self):
        return self.flag_draw or self.filt.flag_topp or self.filt.flag_minp


def draw(filt: Filtered, u):
    """Inverse-CDF draw in key order over the kept prefix."""
    if filt.n_kept == 0:
        return RowResult(-1, filt, u, False)
    if filt.greedy:
        return RowResult(filt.argmax, filt, u, False)
    i = int(inverse_cdf(filt.cdf, u))
    return RowResult(int(filt.order[i]), filt, u, boundary_draw(filt.cdf, u))


def sample_row(xp, temperature, top_k, top_p, min_p, seed, request, position):
    filt = filter_row(xp, temperature, top_k, top_p, min_p)
    u = philox.uniform(seed, request, position, 0, philox.SAMPLE)
    return draw(filt, u)


@dataclass
class Params:
    """Per-request parameters for a batch (host numpy arrays, one entry per row)."""
    temperature: np.ndarray
    top_k: np.ndarray
    top_p: np.ndarray
    min_p: np.ndarray
    rep: np.ndarray | None = None
    freq: np.ndarray | None = None
    pres: np.ndarray | None = None
    hist: list | None = None          # per row: array of history ids
    bias_ids: list | None = None      # per row: array of ids
    bias_vals: list | None = None     # per row: array of values
    mask: np.ndarray | None = None    # [B, words] uint32 (or [B, G+1, words] for spec)
    request_ids: np.ndarray | None = None
    positions: np.ndarray | None = None
    seed: int = 0

    def row(self, b):
        def get(a, default):
            return default if a is None else a[b]
        return dict(
            rep=float(get(self.rep, 1.0)), freq=float(get(self.freq, 0.0)),
            pres=float(get(self.pres, 0.0)),
            hist=() if self.hist is None else self.hist[b],
            bias_ids=() if self.bias_ids is None else self.bias_ids[b],
            bias_vals=() if self.bias_vals is None else self.bias_vals[b],
            mask=None if self.mask is None else self.mask[b],
            request=int(get(self.request_ids, b)), position=int(get(self.positions, 0)),
        )


def sample_batch(logits_f32, params: Params):
    """Run the whole per-request pipeline on every row; returns per-row results."""
    out = []
    for b in range(logits_f32.shape[0]):
        pr = params.row(b)
        xp = process_row(logits_f32[b], pr["hist"], pr["rep"], pr["freq"], pr["pres"],
                         pr["bias_ids"], pr["bias_vals"], pr["mask"])
        res = sample_row(xp, params.temperature[b], params.top_k[b], params.top_p[b],
                         params.min_p[b], params.seed, pr["request"], pr["position"])
        res.xp = xp
        out.append(res)
    return out
