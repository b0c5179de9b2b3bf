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
from . import pipeline as P
from .pipeline import bf16_bits_to_f32

GAP_EPS = 1e-5
# A processed row's scores and filter cuts move with the GEMM's rounding:
# binary32 accumulation over K = 8192 stays below 1e-5 of the logits'
# magnitude (about 7e-6 measured on the full-size LM-head). In
# sample_processed both distances are scaled by Z = max(1, largest |x'| / T of
# the row): the top-two score gap GAP_EPS Z and the cut distance CUT_EPS Z.
CUT_EPS = 1e-5
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


def processed_rows(z, params: P.Params):
    """(x', filtered row) of every row of z: the seed-independent part of
    sample_processed, for tests that sweep seeds over fixed logits."""
    out = []
    for b in range(z.shape[0]):
        pr = params.row(b)
        x = np.asarray(z[b], dtype=np.float64).astype(np.float32)
        xp = P.process_row(x, pr["hist"], pr["rep"], pr["freq"], pr["pres"], pr["bias_ids"],
                           pr["bias_vals"], pr["mask"])
        filt = P.filter_row(xp, float(np.float32(params.temperature[b])), int(params.top_k[b]),
                            float(params.top_p[b]), float(params.min_p[b]))
        out.append((xp, filt))
    return out


def sample_processed(z, params: P.Params, rows=None):
    """The per-request sampling pipeline applied to LM-head logits before the
    Gumbel step (SonicSampler abstract: penalties, bias, grammar mask,
    temperature, top-k / top-p / min-p per request in one batched pass;
    FlashSampling news item: Gumbel-max sampling folded into the LM-head GEMM).

    Reading, row b: x = binary32(z[b]) (z is the binary64 GEMM); x' =
    pipeline.process_row(x, ...) with the request's history, bias and mask;
    the filtered support K = pipeline.filter_row(x', T, top_k, top_p, min_p);
    T > 0: the token is the lowest id attaining the largest s_v = z'_v + g_v
    over v in K, with z'_v = binary32(x'_v / T) (the sampler's z) and g_v the
    Gumbel variate of the GUMBEL word at (seed, request, position, draw v) --
    Gumbel-max over K samples exactly from the filtered distribution. T = 0:
    the greedy token. Returns (tokens, flags); a row is flagged when its two
    largest scores (largest x' for T = 0) lie within GAP_EPS Z, or when an
    entry whose membership of the support a change of z' by CUT_EPS Z could
    flip (z' near a cutting top-k's boundary, an exclusive mass near top_p, a
    weight near min_p) is the winner or scores within GAP_EPS Z of it, Z =
    max(1, largest |x'| / T of the row). rows:
    processed_rows() of the same z and parameters, or None."""
    B, V = z.shape
    toks = np.full(B, -1, dtype=np.int32)
    flags = np.zeros(B, dtype=bool)
    if rows is None:
        rows = processed_rows(z, params)
    for b in range(B):
        pr = params.row(b)
        T = float(np.float32(params.temperature[b]))
        xp, filt = rows[b]
        if filt.n_kept == 0:
            continue
        fin = np.sort(xp[np.isfinite(xp)].astype(np.float64))
        Z = max(1.0, float(np.max(np.abs(fin))) / (T if T > 0.0 else 1.0))
        if filt.greedy:
            toks[b] = filt.argmax
            flags[b] = fin.size > 1 and fin[-1] - fin[-2] < GAP_EPS * Z
            continue
        kept = filt.order[:filt.n_kept]
        req, pos = pr["request"], pr["position"]
        sc = _scores(xp, kept, T, params.seed, req, pos)
        best = np.max(sc)
        win = int(np.min(kept[sc == best]))
        toks[b] = win
        top2 = np.sort(sc)[-2:] if sc.size > 1 else None
        flag = top2 is not None and top2[1] - top2[0] < GAP_EPS * Z
        if not flag:
            # entries a GEMM-sized change of z' could move across a cut: the
            # draw changes only if the winner is one of them or one of them
            # outscores it
            amb = _ambiguous(filt, params, b, CUT_EPS * Z)
            if amb.size:
                flag = win in set(amb.tolist()) or bool(
                    np.any(_scores(xp, amb, T, params.seed, req, pos) > best - GAP_EPS * Z))
        flags[b] = flag
    return toks, flags


def _scores(xp, ids, T, seed, request, position):
    """s_v = binary32(x'_v / T) + g_v for the given ids (binary64)."""
    ids = np.asarray(ids, dtype=np.int64)
    zk = (xp[ids] / np.float32(T)).astype(np.float32) + np.float32(0.0)
    g = philox.gumbel_np(philox.words_np(seed, request, position, ids, philox.GUMBEL))
    return zk.astype(np.float64) + g


def _ambiguous(filt, params, b, eps):
    """Ids whose membership of the kept support a change of z' by eps could
    flip: z' within eps of a cutting top-k's boundary value, an exclusive mass
    within eps of top_p, or a weight within a factor 1 +- eps of min_p."""
    zo = np.log(filt.w)  # z' - max z' in key order
    n = filt.order.size
    near = np.zeros(n, dtype=bool)
    if filt.topk_active and filt.n_topk < n:
        zc = 0.5 * (zo[filt.n_topk - 1] + zo[filt.n_topk])
        near |= np.abs(zo - zc) < eps
    tp = float(np.float32(params.top_p[b]))
    if tp < 1.0:
        pk = filt.w[:filt.n_topk] / filt.w[:filt.n_topk].sum()
        excl = np.concatenate(([0.0], np.cumsum(pk)[:-1]))
        near[1:filt.n_topk] |= np.abs(excl[1:] - tp) < eps
    mp = float(np.float32(params.min_p[b]))
    if mp > 0.0:
        near[1:] |= np.abs(filt.w[1:] - mp) < eps * mp
    return filt.order[near]
