"""Benchmark of the fused batched sampler on one MI355X.

Headline (one JSON line on stdout): the heterogeneous workload -- B=64 rows,
V=128256 float32 Zipf-shaped logits, per-request temperature / top-k / top-p /
min-p, repetition + frequency + presence penalties over 512 history ids and 16
logit-bias entries -- sampled by ss_sample. A step is one ss_sample call over
one batch. Inputs are resident in HBM and rotate over enough copies (>= 512 MB,
twice the 256 MB Infinity Cache) that every call reads its logits from HBM.
The K timed steps are one HIP-graph replay; the kernel's own duration is taken
with HIP events around each launch on the launch stream.

The JSON line also carries:
  roofline      the algorithmic bytes of one call (logits, history, bias,
                parameters, tokens) / ms_per_step -- the whole ss_sample call,
                both launches and the gap between them -- vs the 8 TB/s peak;
                `kernel` holds the same figure for the tile kernel alone (its
                duration from HIP events recorded by its own dispatch), and
                `traffic` the HBM bytes per call from committed rocprofv3
                counter runs (null when the kernel sources changed since);
  cpu_baseline  the CPU oracle on the host over a bounded sample, rows split
                across worker processes (taken before the GPU is touched);
  secondary     the other configurations (us per call, tokens/s, the same
                whole-call and tile-kernel fractions), and unfiltered N(0, 1)
                rows at T = 1, which exercise the exact whole-row path.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import multiprocessing
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MALL_BYTES = 256 << 20
ROTATE_MIN = 2 * MALL_BYTES
ROWS_SRC = os.path.join(ROOT, "speculative_decoding_verification_pipeline_amd", "csrc", "ss_rows.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_sample_heterogeneous_counters.md")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_sha():
    h = hashlib.sha256()
    for f in ("ss_rows.hip", "ss_device.h", "ss_internal.h"):
        with open(os.path.join(os.path.dirname(ROWS_SRC), f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def committed_traffic(key):
    """HBM bytes (`key` = TRAFFIC_BYTES_PER_LAUNCH for the tile kernel,
    TRAFFIC_BYTES_PER_CALL for both launches) from the committed counter
    summary, if it was taken on the current kernel sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    m = re.search(key + r"\s*=\s*([0-9.eE+]+)", text)
    s = re.search(r"SOURCE_SHA\s*=\s*([0-9a-f]+)", text)
    if not m or not s or s.group(1) != source_sha():
        return None
    return float(m.group(1))


def fraction(nbytes, seconds):
    gbs = nbytes / seconds / 1e9
    return {"achieved": gbs, "frac": gbs / HBM_PEAK_GBS}


def to_dev(a, dt, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(device=dev, dtype=dt)


def sampling_params(w, dev, positions=None):
    import torch
    from speculative_decoding_verification_pipeline_amd.sampler import SamplingParams
    B = w.B
    kw = {}
    if w.hist is not None:
        kw["history_ids"] = to_dev(w.hist, torch.int32, dev)
        kw["history_len"] = to_dev(np.full(B, w.hist.shape[1], np.int32), torch.int32, dev)
    if w.bias_ids is not None:
        kw["bias_ids"] = to_dev(w.bias_ids, torch.int32, dev)
        kw["bias_values"] = to_dev(w.bias_vals, torch.float32, dev)
        kw["bias_len"] = to_dev(np.full(B, w.bias_ids.shape[1], np.int32), torch.int32, dev)
    for name, a in (("repetition_penalty", w.rep), ("frequency_penalty", w.freq),
                    ("presence_penalty", w.pres)):
        if a is not None:
            kw[name] = to_dev(a, torch.float32, dev)
    if w.mask is not None:
        kw["grammar_mask"] = to_dev(w.mask.view(np.int32), torch.int32, dev)
    pos = w.positions if positions is None else positions
    return SamplingParams(temperature=to_dev(w.temperature, torch.float32, dev),
                          top_k=to_dev(w.top_k, torch.int32, dev),
                          top_p=to_dev(w.top_p, torch.float32, dev),
                          min_p=to_dev(w.min_p, torch.float32, dev),
                          request_ids=to_dev(w.request_ids, torch.int32, dev),
                          positions=to_dev(pos, torch.int32, dev), seed=w.seed, **kw)


def time_graph(step_fns, steps, warmup):
    """Warm up eagerly, capture `steps` calls in one graph, time one replay (ms)."""
    import torch
    n = len(step_fns)
    for i in range(warmup):
        step_fns[i % n]()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            step_fns[i % n]()
    g.replay()  # first replay uploads the graph
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    g.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end), g


def time_launches(step_fns, n):
    """Average duration (ms) of single calls, HIP events around each one."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    torch.cuda.synchronize()
    for i in range(n):
        ev[i][0].record()
        step_fns[i % len(step_fns)]()
        ev[i][1].record()
    torch.cuda.synchronize()
    d = np.array([a.elapsed_time(b) for a, b in ev])
    return float(d.mean()), float(np.median(d)), float(np.percentile(d, 10)), float(np.percentile(d, 90))


def time_stages(sampler, step_fns, n, n_launches):
    """Per-kernel durations (ms) of n calls: the library launches each kernel
    with a start and a stop HIP event that the dispatch itself records."""
    import torch
    evs = []
    for _ in range(n):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n_launches)]
        for x in e:
            x.record()  # creates the HIP event
        evs.append(e)
    torch.cuda.synchronize()
    for i in range(n):
        sampler.set_launch_events(evs[i])
        step_fns[i % len(step_fns)]()
    sampler.set_launch_events(None)
    torch.cuda.synchronize()
    d = np.array([[evs[i][2 * k].elapsed_time(evs[i][2 * k + 1]) for k in range(n_launches)]
                  for i in range(n)])
    return d  # [n, n_launches] ms


def stage_summary(d, names):
    out = {}
    for k, nm in enumerate(names):
        col = d[:, k] * 1e3
        out[nm] = {"us_mean": float(col.mean()), "us_median": float(np.median(col)),
                   "us_p10": float(np.percentile(col, 10)), "us_p90": float(np.percentile(col, 90))}
    return out


_CPU_W = None  # the workload, inherited by the forked baseline workers


def _cpu_worker(args):
    """Rows first, first + stride, ... of the workload through the oracle until
    the budget runs out; returns (rows, seconds)."""
    from oracle import philox
    from oracle import pipeline as OP
    first, stride, budget_s = args
    w = _CPU_W
    t0 = time.perf_counter()
    rows = 0
    while time.perf_counter() - t0 < budget_s:
        b = (first + rows * stride) % w.B
        xp = OP.process_row(w.logits[b], w.hist[b], w.rep[b], w.freq[b], w.pres[b],
                            w.bias_ids[b], w.bias_vals[b], None)
        f = OP.filter_row(xp, w.temperature[b], w.top_k[b], w.top_p[b], w.min_p[b])
        OP.draw(f, philox.uniform(w.seed, int(w.request_ids[b]), int(w.positions[b]), 0,
                                  philox.SAMPLE))
        rows += 1
    return rows, time.perf_counter() - t0


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, budget_s, max_workers=16):
    """The oracle as it stands on this host's cores, on a bounded sample: the
    rows are dealt round-robin to one worker process per available core (at
    most max_workers), each running for budget_s. Call it before the GPU is
    initialised: the workers are forked from this process."""
    global _CPU_W
    _CPU_W = w
    n = max(1, min(len(os.sched_getaffinity(0)), max_workers))
    t0 = time.perf_counter()
    with multiprocessing.get_context("fork").Pool(n) as pool:
        res = pool.map(_cpu_worker, [(i, n, budget_s) for i in range(n)])
    wall = time.perf_counter() - t0
    rows = sum(r for r, _ in res)
    per_proc = [r / t for r, t in res]
    return {"value": float(sum(per_proc)), "unit": "tokens/s", "cores": n, "kind": "oracle",
            "cpu_model": cpu_model(),
            "single_process_value": float(np.mean(per_proc)),
            "sample": f"{rows} rows of the heterogeneous workload (V=128256 f32, penalties, bias, "
                      f"mixed filters) through the oracle's process/filter/draw, rows dealt "
                      f"round-robin to {n} worker processes for {budget_s:.0f} s each "
                      f"({wall:.1f} s wall); value = sum of the per-process rates"}


def headline(args, dev, w):
    import torch
    from speculative_decoding_verification_pipeline_amd.sampler import Sampler
    B, V = w.B, w.V
    logits_bytes = B * V * 4
    R = max(2, -(-ROTATE_MIN // logits_bytes))
    base = torch.from_numpy(w.logits).to(dev)
    bufs = [base] + [base.clone() for _ in range(R - 1)]
    prms = [sampling_params(w, dev, positions=np.full(B, r, np.int32)) for r in range(R)]
    s = Sampler(B, V, device=0)
    out = torch.empty(B, dtype=torch.int32, device=dev)
    fns = [(lambda x=bufs[r], p=prms[r]: s.sample(x, p, out=out)) for r in range(R)]
    ms, g = time_graph(fns, args.steps, args.warmup)
    c_mean, c_med, c_p10, c_p90 = time_launches(fns, max(args.steps, 50))
    st = time_stages(s, fns, max(args.steps, 50), 2)
    stages = stage_summary(st, ["k_sample_tiles<f32>", "k_sample_rows<f32>"])
    t_mean = stages["k_sample_tiles<f32>"]["us_mean"]
    alg = {"logits": logits_bytes, "history": B * 512 * 4, "bias": B * 16 * 8,
           "params": B * 7 * 4, "tokens": B * 4}
    alg_total = sum(alg.values())
    call = fraction(alg_total, ms / args.steps * 1e-3)
    tile = fraction(alg_total, t_mean * 1e-6)
    res = {
        "metric": "sampled tokens/s and HBM GB/s (% of peak) at B=64, V=128256 fp32",
        "value": B * args.steps / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "heterogeneous sampling: B=64, V=128256 f32 Zipf logits, mixed "
                               "T/top-k/top-p/min-p, penalties over 512 history ids, 16 bias ids",
                   "global_batch": B, "vocab": V, "parallelism": "none (1 GPU)",
                   "rotated_buffers": R},
        "roofline": {"bound": "hbm", "achieved": call["achieved"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": call["frac"],
                     "traffic": committed_traffic("TRAFFIC_BYTES_PER_CALL"),
                     "scope": "whole ss_sample call: algorithmic bytes per call / ms_per_step",
                     "bytes": alg_total,
                     "kernel": {"name": "k_sample_tiles<f32>", "us_mean": t_mean,
                                "achieved": tile["achieved"], "frac": tile["frac"],
                                "traffic": committed_traffic("TRAFFIC_BYTES_PER_LAUNCH")}},
        "kernel": {"name": "k_sample_tiles<f32>", "stages": stages,
                   "call_us_mean": c_mean * 1e3, "call_us_median": c_med * 1e3,
                   "call_us_p10": c_p10 * 1e3, "call_us_p90": c_p90 * 1e3,
                   "algorithmic_bytes": alg},
    }
    return res


def secondary(args, dev):
    import torch
    from speculative_decoding_verification_pipeline_amd import workloads as W
    from speculative_decoding_verification_pipeline_amd.sampler import Sampler
    out = {}
    steps = max(20, args.steps // 4)
    # low-entropy, B=4, V=32000: launch-bound
    w = W.low_entropy()
    s = Sampler(w.B, w.V, device=0)
    x = torch.from_numpy(w.logits).to(dev)
    p = sampling_params(w, dev)
    o = torch.empty(w.B, dtype=torch.int32, device=dev)
    ms, _ = time_graph([lambda: s.sample(x, p, out=o)], steps, 5)
    km = time_launches([lambda: s.sample(x, p, out=o)], steps)[0]
    st = stage_summary(time_stages(s, [lambda: s.sample(x, p, out=o)], steps, 2),
                       ["k_sample_tiles<f32>", "k_sample_rows<f32>"])
    out["low_entropy"] = {"us_per_call": ms / steps * 1e3, "call_us": km * 1e3, "stages": st,
                          "tokens_per_s": w.B * steps / (ms * 1e-3)}
    s.close()
    # grammar, B=256, V=152064 bf16 + mask
    w = W.grammar()
    nbytes = w.B * w.V * 2 + w.mask.nbytes
    R = max(2, -(-ROTATE_MIN // nbytes))
    base = torch.from_numpy(w.logits.view(np.int16)).to(dev).view(torch.bfloat16)
    bufs = [base] + [base.clone() for _ in range(R - 1)]
    prms = [sampling_params(w, dev, positions=np.full(w.B, r, np.int32)) for r in range(R)]
    for r in range(1, R):
        prms[r].grammar_mask = prms[0].grammar_mask.clone()
    s = Sampler(w.B, w.V, device=0)
    o = torch.empty(w.B, dtype=torch.int32, device=dev)
    fns = [(lambda x=bufs[r], pr=prms[r]: s.sample(x, pr, out=o)) for r in range(R)]
    ms, _ = time_graph(fns, steps, 5)
    km = time_launches(fns, steps)[0]
    st = stage_summary(time_stages(s, fns, steps, 2), ["k_sample_tiles<bf16>", "k_sample_rows<bf16>"])
    t_us = st["k_sample_tiles<bf16>"]["us_mean"]
    out["grammar"] = {"us_per_call": ms / steps * 1e3, "call_us": km * 1e3, "stages": st,
                      "tokens_per_s": w.B * steps / (ms * 1e-3), "bytes": nbytes,
                      "roofline": dict(fraction(nbytes, ms / steps * 1e-3),
                                       kernel=dict(name="k_sample_tiles<bf16>",
                                                   **fraction(nbytes, t_us * 1e-6)))}
    s.close()
    del bufs
    # speculative verification, 32 x (4 + 1) x 128256
    sw = W.speculative()
    nbytes = sw.target.nbytes
    R = max(2, -(-ROTATE_MIN // nbytes))
    tg = torch.from_numpy(sw.target).to(dev)
    qd = torch.from_numpy(sw.draft_probs).to(dev)
    tgs = [tg] + [tg.clone() for _ in range(R - 1)]
    dt = torch.from_numpy(sw.draft_tokens).to(dev)
    from speculative_decoding_verification_pipeline_amd.sampler import SamplingParams
    sp = SamplingParams(temperature=torch.from_numpy(sw.temperature).to(dev),
                        top_k=torch.from_numpy(sw.top_k).to(dev),
                        top_p=torch.from_numpy(sw.top_p).to(dev),
                        min_p=torch.from_numpy(sw.min_p).to(dev),
                        request_ids=torch.from_numpy(sw.request_ids).to(dev),
                        positions=torch.from_numpy(sw.positions).to(dev), seed=sw.seed)
    s = Sampler(sw.B, sw.V, max_draft=sw.G, device=0)
    ot = torch.empty(sw.B, sw.G + 1, dtype=torch.int32, device=dev)
    on = torch.empty(sw.B, dtype=torch.int32, device=dev)
    fns = [(lambda t=tgs[r]: s.spec_verify(t, qd, dt, sp, ot, on)) for r in range(R)]
    fns[0]()
    torch.cuda.synchronize()
    emitted = int((on + 1).sum().item())
    # a rejected sampling request reads its draft row at the rejected position
    # whole (the residual); every position reads one draft probability and token
    n_acc = on.cpu().numpy()
    rejected = int(np.sum((sw.temperature > 0) & (n_acc < sw.G)))
    ms, _ = time_graph(fns, steps, 5)
    km = time_launches(fns, steps)[0]
    st = stage_summary(time_stages(s, fns, steps, 4),
                       ["k_spec_tiles<f32>", "k_spec_rows<f32>", "k_spec_resid_tiles<f32>",
                        "k_spec_finish<f32>"])
    t_us = st["k_spec_tiles<f32>"]["us_mean"]
    nbytes_all = nbytes + rejected * sw.V * 4 + sw.B * sw.G * 4 * 2 + sw.B * (sw.G + 2) * 4
    out["speculative"] = {"us_per_call": ms / steps * 1e3, "call_us": km * 1e3, "stages": st,
                          "emitted_tokens_per_call": emitted,
                          "emitted_tokens_per_s": emitted * steps / (ms * 1e-3),
                          "bytes": nbytes_all, "rejected_sampling_requests": rejected,
                          "roofline": dict(fraction(nbytes_all, ms / steps * 1e-3),
                                           kernel=dict(name="k_spec_tiles<f32>",
                                                       **fraction(nbytes, t_us * 1e-6)))}
    # the same verification with greedy drafts (q one-hot, no draft rows read),
    # the emitted tokens appended to device-side sequences (positions = lengths)
    swg = W.speculative(greedy_draft=True)
    dg = torch.from_numpy(swg.draft_tokens).to(dev)
    seq_t = torch.zeros(sw.B, 1 << 16, dtype=torch.int32, device=dev)
    seq_l = torch.zeros(sw.B, dtype=torch.int32, device=dev)
    spg = SamplingParams(temperature=sp.temperature, request_ids=sp.request_ids, positions=seq_l,
                         seed=sw.seed)
    gfns = [(lambda t=tgs[r]: s.spec_verify(t, None, dg, spg, ot, on, seq_tokens=seq_t,
                                            seq_len=seq_l)) for r in range(R)]
    gfns[0]()
    torch.cuda.synchronize()
    g_emitted = int((on + 1).sum().item())
    seq_l.zero_()
    ms, _ = time_graph(gfns, steps, 5)
    st = stage_summary(time_stages(s, gfns, steps, 4),
                       ["k_spec_tiles<f32>", "k_spec_rows<f32>", "k_spec_resid_tiles<f32>",
                        "k_spec_finish<f32>"])
    gbytes = nbytes + swg.B * swg.G * 4 + swg.B * (swg.G + 2) * 4
    out["speculative_greedy_draft"] = {
        "us_per_call": ms / steps * 1e3, "stages": st, "emitted_tokens_per_call": g_emitted,
        "emitted_tokens_per_s": g_emitted * steps / (ms * 1e-3), "bytes": gbytes,
        "roofline": fraction(gbytes, ms / steps * 1e-3),
        "note": "no draft rows read; emitted tokens appended on the device"}
    s.close()
    del tgs
    # tree verification: 32 requests x 16-node draft trees x 128256 f32
    tw = W.tree()
    nbytes = tw.target.nbytes
    R = max(2, -(-ROTATE_MIN // nbytes))
    tt = torch.from_numpy(tw.target).to(dev)
    tts = [tt] + [tt.clone() for _ in range(R - 1)]
    tpar = torch.from_numpy(tw.parents).to(dev)
    ttok = torch.from_numpy(tw.tokens).to(dev)
    tp = SamplingParams(temperature=torch.from_numpy(tw.temperature).to(dev),
                        request_ids=torch.from_numpy(tw.request_ids).to(dev),
                        positions=torch.from_numpy(tw.positions).to(dev), seed=tw.seed)
    s = Sampler(tw.B, tw.V, max_draft=tw.N - 1, device=0)
    o1 = torch.empty(tw.B, tw.N, dtype=torch.int32, device=dev)
    o2 = torch.empty(tw.B, tw.N, dtype=torch.int32, device=dev)
    o3 = torch.empty(tw.B, dtype=torch.int32, device=dev)
    tfns = [(lambda t=tts[r]: s.tree_verify(t, tpar, ttok, tp, o1, o2, o3)) for r in range(R)]
    tfns[0]()
    torch.cuda.synchronize()
    t_emitted = int((o3 + 1).sum().item())
    ms, _ = time_graph(tfns, steps, 5)
    st = stage_summary(time_stages(s, tfns, steps, 5),
                       ["k_tree_paths", "k_tree_tiles<f32>", "k_tree_rows<f32>",
                        "k_tree_resid_tiles<f32>", "k_tree_finish<f32>"])
    out["tree"] = {"us_per_call": ms / steps * 1e3, "stages": st,
                   "emitted_tokens_per_call": t_emitted,
                   "emitted_tokens_per_s": t_emitted * steps / (ms * 1e-3), "bytes": nbytes,
                   "roofline": dict(fraction(nbytes, ms / steps * 1e-3),
                                    kernel=dict(name="k_tree_tiles<f32>",
                                                **fraction(nbytes, st["k_tree_tiles<f32>"]["us_mean"] * 1e-6)))}
    s.close()
    del tts
    # fused LM-head + Gumbel-max, hidden [64, 8192] x weight [128256, 8192] bf16
    B, K, V = 64, 8192, 128256
    gen = torch.Generator(device=dev).manual_seed(105)
    Hd = torch.randn(B, K, device=dev, generator=gen).to(torch.bfloat16)
    Wd = (torch.randn(V, K, device=dev, generator=gen) * 0.02).to(torch.bfloat16)
    T = torch.ones(B, device=dev)
    s = Sampler(B, V, hidden_size=K, device=0)
    o = torch.empty(B, dtype=torch.int32, device=dev)
    fn = [lambda: s.lmhead_sample(Hd, Wd, T, seed=0, out=o)]
    lsteps = max(10, steps // 4)
    ms, _ = time_graph(fn, lsteps, 3)
    km = time_launches(fn, lsteps)[0]
    st = stage_summary(time_stages(s, fn, lsteps, 2), ["k_lmhead", "k_lmhead_reduce"])
    g_us = st["k_lmhead"]["us_mean"]
    nbytes = V * K * 2 + B * K * 2
    # the same GEMM with the per-request pipeline in its epilogue: the
    # heterogeneous parameter recipe (penalties over 512 history ids, 16 bias
    # ids, mixed T / top-k / top-p / min-p); rows whose cuts fall outside the
    # tile candidates are selected over their whole row of z' (which the GEMM
    # kernel writes for rows with a filter)
    hw = W.heterogeneous(B=B, V=V)
    hp = sampling_params(hw, dev)
    lpath = torch.empty(B, dtype=torch.int32, device=dev)
    s.lmhead_sample_params(Hd, Wd, hp, out=o, path=lpath)
    torch.cuda.synchronize()
    lp = np.bincount(lpath.cpu().numpy(), minlength=3).tolist()
    pfn = [lambda: s.lmhead_sample_params(Hd, Wd, hp, out=o)]
    pms, _ = time_graph(pfn, lsteps, 3)
    pst = stage_summary(time_stages(s, pfn, lsteps, 5),
                        ["k_lmhead_proc", "k_lm_merge", "k_lm_slow", "k_lm_gumbel", "k_lm_pick"])
    out["lmhead_params"] = {"us_per_call": pms / lsteps * 1e3, "stages": pst,
                            "tokens_per_s": B * lsteps / (pms * 1e-3),
                            "rows_by_path": {"candidates": lp[0], "whole_row": lp[1],
                                             "unfiltered_or_greedy": lp[2]}}
    out["lmhead"] = {"us_per_call": ms / lsteps * 1e3, "call_us": km * 1e3, "stages": st,
                     "tokens_per_s": B * lsteps / (ms * 1e-3),
                     "gemm_kernel_gbs": nbytes / (g_us * 1e-6) / 1e9,
                     "gemm_kernel_hbm_frac": nbytes / (g_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                     "gemm_kernel_tflops": 2.0 * B * K * V / (g_us * 1e-6) / 1e12,
                     "whole_call_gbs": nbytes / (km * 1e-3) / 1e9}
    s.close()
    # unfiltered N(0, 1) rows at T = 1 (B = 64, V = 128256 f32): the row mass is
    # spread over the whole vocabulary, which sends rows to the exact whole-row path
    rng = np.random.default_rng(106)
    B, V = 64, 128256
    x = rng.standard_normal((B, V)).astype(np.float32)
    R = max(2, -(-ROTATE_MIN // x.nbytes))
    base = torch.from_numpy(x).to(dev)
    bufs = [base] + [base.clone() for _ in range(R - 1)]
    from speculative_decoding_verification_pipeline_amd.sampler import Debug, SamplingParams
    pr = SamplingParams(temperature=torch.ones(B, device=dev),
                        request_ids=torch.arange(B, dtype=torch.int32, device=dev),
                        positions=torch.zeros(B, dtype=torch.int32, device=dev), seed=0)
    s = Sampler(B, V, device=0)
    o = torch.empty(B, dtype=torch.int32, device=dev)
    path = torch.empty(B, dtype=torch.int32, device=dev)
    s.sample(bufs[0], pr, out=o, debug=Debug(path=path))
    torch.cuda.synchronize()
    whole_row = int((path == 1).sum().item())
    fns = [(lambda xx=bufs[r]: s.sample(xx, pr, out=o)) for r in range(R)]
    ms, _ = time_graph(fns, steps, 5)
    st = stage_summary(time_stages(s, fns, steps, 2), ["k_sample_tiles<f32>", "k_sample_rows<f32>"])
    out["unfiltered_normal"] = {"us_per_call": ms / steps * 1e3, "stages": st,
                                "tokens_per_s": B * steps / (ms * 1e-3),
                                "rows_on_whole_row_path": whole_row, "rows": B,
                                "roofline": fraction(x.nbytes, ms / steps * 1e-3)}
    s.close()
    del bufs
    return out


COPY_BYTES = 256 << 20


def counters_run(dev):
    """A plain device-to-device copy of COPY_BYTES (reads and writes that many
    bytes), then 5 headline calls on rotated buffers; the counter summary
    scales the sampler's FETCH_SIZE / WRITE_SIZE by what the copy reads."""
    import torch
    from speculative_decoding_verification_pipeline_amd import workloads as W
    from speculative_decoding_verification_pipeline_amd.sampler import Sampler
    a = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    log(f"bench: copied {COPY_BYTES} bytes")
    del a, b
    w = W.heterogeneous()
    R = max(2, -(-ROTATE_MIN // (w.B * w.V * 4)))
    base = torch.from_numpy(w.logits).to(dev)
    bufs = [base] + [base.clone() for _ in range(R - 1)]
    prms = [sampling_params(w, dev, positions=np.full(w.B, r, np.int32)) for r in range(R)]
    s = Sampler(w.B, w.V, device=0)
    out = torch.empty(w.B, dtype=torch.int32, device=dev)
    for r in range(5):
        s.sample(bufs[r + 1], prms[r + 1], out=out)
    torch.cuda.synchronize()
    log("bench: 5 headline calls done")


def counters_lmhead_run(dev):
    """The same known-size copy, then 3 fused LM-head calls at the full shape
    (hidden [64, 8192] x weight [128256, 8192] bf16; the weight, 2.1 GB, is far
    larger than the Infinity Cache, so every call streams it from HBM)."""
    import torch
    from speculative_decoding_verification_pipeline_amd.sampler import Sampler
    a = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    log(f"bench: copied {COPY_BYTES} bytes")
    del a, b
    B, K, V = 64, 8192, 128256
    gen = torch.Generator(device=dev).manual_seed(105)
    Hd = torch.randn(B, K, device=dev, generator=gen).to(torch.bfloat16)
    Wd = (torch.randn(V, K, device=dev, generator=gen) * 0.02).to(torch.bfloat16)
    T = torch.ones(B, device=dev)
    s = Sampler(B, V, hidden_size=K, device=0)
    o = torch.empty(B, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    for r in range(3):
        s.lmhead_sample(Hd, Wd, T, seed=r, out=o)
    torch.cuda.synchronize()
    log("bench: 3 lmhead calls done")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--counters", action="store_true",
                    help="for rocprofv3 --pmc runs: a device copy of known size (counter "
                         "scale), then a few headline calls; prints no JSON line")
    ap.add_argument("--counters-lmhead", action="store_true",
                    help="for rocprofv3 --pmc runs: the same copy, then a few full-size fused "
                         "LM-head calls; prints no JSON line")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "ss-sampler runs on one GPU; sharding across GPUs is not "
                                   "implemented (run with --gpus 1)"}))
        sys.exit(2)
    from speculative_decoding_verification_pipeline_amd import workloads as W
    counters = args.counters or args.counters_lmhead
    w = None if counters else W.heterogeneous()
    cpu = None
    if not counters and not args.no_cpu_baseline:
        # forked workers: before anything initialises the GPU
        log("bench: cpu baseline (oracle)")
        cpu = cpu_baseline(w, args.cpu_seconds)
        log(f"bench: cpu baseline {cpu['value']:.1f} tokens/s on {cpu['cores']} processes")
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda", 0)
    if args.counters:
        counters_run(dev)
        return
    if args.counters_lmhead:
        counters_lmhead_run(dev)
        return
    log("bench: headline (heterogeneous B=64 V=128256)")
    res = headline(args, dev, w)
    log(f"bench: headline done, {res['ms_per_step'] * 1e3:.2f} us per call in the graph "
        f"({res['roofline']['achieved']:.0f} GB/s), tile kernel "
        f"{res['roofline']['kernel']['us_mean']:.2f} us")
    if not args.no_secondary:
        log("bench: secondary configurations")
        res["secondary"] = secondary(args, dev)
    res["cpu_baseline"] = cpu
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
