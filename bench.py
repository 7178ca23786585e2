#!/usr/bin/env python3
"""Routed tokens/s of the MoE router + dispatch hot path on one MI355X.

One step = one moe_route_dispatch call -- the gate contraction, scoring,
selection and weights of moe_route, then the histogram, offsets,
permutation, inverse and load statistic (MaxVio) of moe_dispatch -- over
one batch of seeded synthetic tokens (hash workloads: moe_route_hash, whose
ids come from the token-id table and whose weights from the gathered gate
logits, one moe_route_hash_dispatch call; the capacity workload adds
moe_dispatch_capacity).
Inputs are resident in HBM before timing; each step routes a different copy
of x (rotating through copies totalling more than the 256 MB last-level
cache) so the gate reads x from HBM, not from cache.

The headline (`value`) is the gpt-oss-like configuration, T = 65536 tokens
(the largest one-GPU configuration).  The `configs` object times every other
routing configuration in the same run (Mixtral-, Qwen3-, DeepSeek-V3-,
DeepSeek-V4-like, the V4-like hash layer and the routing variants: selection
bias, OLMoE-like softmax, group max, Switch-like top-1 with a capacity,
per-group quota), each with its per-kernel times, binding roofline and the
oracle's throughput on the host.

Roofline of a kernel: its algorithmic HBM bytes and flops per launch give
t_bound = max(bytes / 8 TB/s, flops / MFMA peak of its dtype); the binding
bound is the larger term and frac = t_bound / measured average duration
(kernel start/stop HIP events the runtime sets on the launch stream).

Usage: python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-configs]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2516.6, "f32": 157.3}
LLC_BYTES = 256 << 20
HEADLINE = "gptoss_skew"
CONFIGS = ("mixtral", "qwen3_dynk", "dsv3_grouped", "dsv4", "dsv4_hash", "gptoss_skew",
           # routing variants on the same shapes
           "dsv4_bias", "olmoe", "dsv3_groupmax", "switch_top1", "grouped_quota")
METRIC = "routed tokens/sec (gate+select+dispatch) and % of MFMA/HBM roofline, 1 MI355X"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def host_threads():
    """Host cores this process may use: the affinity mask, or the machine's CPU
    share when OMP_NUM_THREADS states one."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS", "")
    return max(1, min(n, int(env))) if env.isdigit() else n


def kernel_work(w, T, R, R_valid, tile_bytes, producer_hist=False, beside_rows=0):
    """Algorithmic (HBM bytes, flops) per launch of each kernel: inputs read
    once, outputs written once.  tile_bytes: the dispatch's per-tile
    histogram data (written once, read once by the placement); with
    producer_hist the selection / hash kernel writes it (no disp_hist
    launch).  In a hash
    layer the gate's work is the method's -- x and W read once and k dot
    products per token (the table replaces the selection) -- not the dense
    contraction this design performs.  beside_rows: the hash layer's
    dispatch is placed inside the dot-product kernel (its free workgroups)
    from per-tile rows of counts of that many bytes, which the ids kernel
    writes."""
    xb = 2 if w.dtype == "bf16" else 4
    E, d, k = w.E, w.d, w.k
    kt = T * 4 if w.dynamic_k else 0
    dense = 2.0 * T * d * E
    ph = tile_bytes if producer_hist else 0
    return {
        "gate": (T * d * xb + E * d * xb, 2.0 * T * d * k) if w.hash_vocab
        else (T * d * xb + E * d * xb + T * E * 4, dense),
        # the gate kernel with the selection fused: no logits leave the chip
        "gate_select": (T * d * xb + E * d * xb + T * k * 8 + kt + tile_bytes, dense),
        # table rows, the k gathered logits, ids and weights
        "hash": (T * 4 + T * k * 4 + T * k * 4 + T * k * 8 + ph, 0.0),
        # the table's ids alone: token ids and table rows read, ids written
        # (+ the tiles' rows of counts)
        "hash_ids": (T * 4 + T * k * 4 + T * k * 4 + beside_rows, 0.0),
        # the hash layer's k dot products: x and W read once, ids read, the
        # k logits per token written once (+ the placement beside them: rows
        # of counts and ids read, inv, perm, counts and offsets written)
        "hash_dots": (T * d * xb + E * d * xb + T * k * 4 + T * k * 4
                      + (beside_rows + R * 4 + R * 4 + R_valid * 4 + E * 8 if beside_rows else 0),
                      2.0 * T * d * k),
        "select": (T * E * 4 + T * k * 8 + kt + ph, 0.0),
        # small batches: selection and the whole dispatch in one workgroup
        "select_dispatch": (T * E * 4 + T * k * 8 + kt + R * 4 + R_valid * 4 + E * 8, 0.0),
        "disp_hist": (R * 4 + tile_bytes, 0.0),
        "disp_scan": (2 * tile_bytes + E * 4, 0.0),
        "disp_scatter": (tile_bytes + E * 4 + R * 4 + R * 4 + R_valid * 4 + E * 8, 0.0),
        # capacity limit: ids and positions read, slots written, kept counts
        "capacity": (R * 12 + E * 8 + 4, 0.0),
    }


def roofline(nbytes, flops, us, dtype):
    """Binding bound of a kernel and its fraction of it."""
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
    peak_tf = MFMA_PEAK_TFLOPS[dtype]
    t_mfma = flops / (peak_tf * 1e12)
    t = us * 1e-6
    if t_mfma > t_hbm:
        return {"bound": "mfma", "achieved": round(flops / t / 1e12, 1), "peak": peak_tf,
                "unit": "TFLOP/s", "frac": round(t_mfma / t, 4),
                "hbm_frac": round(t_hbm / t, 4), "mfma_frac": round(t_mfma / t, 4)}
    return {"bound": "hbm", "achieved": round(nbytes / t / 1e9, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(t_hbm / t, 4), "hbm_frac": round(t_hbm / t, 4),
            "mfma_frac": round(t_mfma / t, 4)}


def pipeline_roofline(w, T, R, R_valid, step_us):
    """Lower bounds on a whole step at the MI355X peaks and the step's
    fraction of each: staged = the gate (max of its flops and bytes, logits
    written once) + the selection (logits read once, ids and weights
    written) + the dispatch (ids read; perm, inv, counts, offsets written)
    [+ the capacity limit]; fused = no logits hand-off, one pass over x and
    W.  A hash layer's bound is the method's: x and W once, table rows,
    k dot products per token, ids and weights, the dispatch."""
    xb = 2 if w.dtype == "bf16" else 4
    E, d, k = w.E, w.d, w.k
    bw = HBM_PEAK_GBS * 1e9
    peak = MFMA_PEAK_TFLOPS[w.dtype] * 1e12
    kt = T * 4 if w.dynamic_k else 0
    xw = T * d * xb + E * d * xb
    disp = R * 4 + R_valid * 4 + R * 4 + E * 8
    cap = R * 12 + E * 8 + 4 if w.capacity_factor else 0
    if w.hash_vocab:
        flops = 2.0 * T * d * k
        staged = max(flops / peak, (xw + T * 4 + T * k * 4 + T * k * 8) / bw) + disp / bw
        fused = staged
    else:
        flops = 2.0 * T * d * E
        staged = (max(flops / peak, (xw + T * E * 4) / bw) + (T * E * 4 + T * k * 8 + kt) / bw
                  + (disp + cap) / bw)
        fused = max(flops / peak, (xw + T * k * 8 + kt + disp + cap) / bw)
    return {"t_roof_staged_us": round(staged * 1e6, 3),
            "frac_staged": round(staged * 1e6 / step_us, 4),
            "t_roof_fused_us": round(fused * 1e6, 3), "frac_fused": round(fused * 1e6 / step_us, 4)}


def inputs_record(inp):
    """numpy's version and a sha256 of the synthetic input bytes, in name order."""
    import hashlib
    import numpy as np
    h = hashlib.sha256()
    for name in sorted(inp):
        a = inp[name]
        if isinstance(a, np.ndarray):
            h.update(name.encode())
            h.update(np.ascontiguousarray(a).tobytes())
    return {"numpy": np.__version__, "seed": 0, "sha256": h.hexdigest()}


def source_digest(files):
    """sha256 over the given source files, concatenated in order."""
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(path, workload, stage):
    """HBM bytes per launch from the committed counter summary, or None when
    there is none for this kernel or its sources (the kernel's file and the
    headers it is built with) changed since it was taken."""
    try:
        with open(path) as f:
            rec = json.load(f)[workload][stage]
        if source_digest(rec["sources"]) != rec["sha256"]:
            return None
        return rec["traffic_bytes"]
    except (OSError, KeyError, ValueError):
        return None


def cpu_baseline(w, inp, seconds, threads):
    """Time the oracle (gate + route + dispatch, fp64) on a bounded sample."""
    import numpy as np

    import oracle
    import workloads as wl

    def run_hash(n):  # table ids, the gate, the gathered weights, dispatch
        t0 = time.perf_counter()
        ids, _ = oracle.hash_ids(inp["token_ids"][:n], inp["tid2eid"], w.E)
        lg = oracle.gate(wl.rows(inp["x"], np.arange(n)), inp["W"], inp["logit_bias"],
                         nthreads=threads)
        oracle.weights_for_ids(lg, ids, score=w.score, renormalize=w.renormalize,
                               route_scale=w.route_scale)
        oracle.dispatch(ids, w.E)
        return time.perf_counter() - t0

    def run(n):
        if w.hash_vocab:
            return run_hash(n)
        sl = np.arange(n)
        kw = dict(score=w.score, logit_bias=inp["logit_bias"], select_bias=inp["select_bias"],
                  k_per_token=None if inp["k_per_token"] is None else inp["k_per_token"][:n],
                  n_groups=w.n_groups, topk_groups=w.topk_groups,
                  group_score=w.group_score if w.n_groups > 1 else None,
                  renormalize=w.renormalize, route_scale=w.route_scale,
                  k_per_group=w.k_per_group, nthreads=threads)
        t0 = time.perf_counter()
        oracle.route_full(wl.rows(inp["x"], sl), inp["W"], w.k, **kw)
        return time.perf_counter() - t0

    n0 = min(w.T, 256)
    t0 = run(n0)
    n = int(min(w.T, max(n0, n0 * seconds / max(t0, 1e-6))))
    t = run(n) if n > n0 else t0
    reps, total = 1, t
    while n == w.T and total < seconds:  # one pass is short: repeat it
        total += run(n)
        reps += 1
    what = ("hash ids + gate + gathered weights + dispatch" if w.hash_vocab
            else "gate + route + dispatch")
    return {"value": reps * n / total, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{'first %d of ' % n if n < w.T else 'all '}{w.T} tokens of the same "
                      f"workload x {reps} ({what}, fp64, {threads} host threads), {total:.1f} s"}


def combine_cpu_baseline(Yp, inv, weights, shared, seconds=3.0):
    """Time the oracle's combine (fp64, one thread) on the first tokens."""
    import oracle

    T = weights.shape[0]
    n = min(T, 64)
    while True:
        t0 = time.perf_counter()
        oracle.combine(Yp, inv[:n], weights[:n], shared[:n])
        t = time.perf_counter() - t0
        if t >= seconds / 4 or n == T:
            break
        n = min(T, n * 4)
    return {"value": n / t, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"first {n} of {T} tokens (combine, fp64), {t:.2f} s"}


class Case:
    """One workload on the GPU: inputs, rotating copies of x, outputs and the
    step (one pass of the hot path)."""

    def __init__(self, w, inp, dev):
        import numpy as np
        import torch

        import token_dispatch_amd as tda
        import workloads as wl

        self.w, self.inp, self.dev = w, inp, dev
        up = self.up
        x0 = up(inp["x"])
        xbytes = x0.numel() * x0.element_size()
        self.n_copies = max(1, min(64, math.ceil(3 * LLC_BYTES / xbytes)))
        self.xs = [x0] + [torch.roll(x0, shifts=97 * i, dims=0).contiguous()
                          for i in range(1, self.n_copies)]
        W = up(inp["W"])
        lb, sb, kpt = up(inp["logit_bias"]), up(inp["select_bias"]), up(inp["k_per_token"])
        T, E, k = w.T, w.E, w.k
        i32 = torch.int32
        self.ids = torch.empty((T, k), dtype=i32, device=dev)
        self.weights = torch.empty((T, k), dtype=torch.float32, device=dev)
        self.counts = torch.empty(E, dtype=i32, device=dev)
        self.offsets = torch.empty(E + 1, dtype=i32, device=dev)
        self.perm = torch.empty(T * k, dtype=i32, device=dev)
        self.inv = torch.empty(T * k, dtype=i32, device=dev)
        self.maxvio = torch.zeros(1, dtype=torch.float64, device=dev)
        pkw = dict(score=w.score, n_groups=w.n_groups, topk_groups=w.topk_groups,
                   group_score=w.group_score if w.n_groups > 1 else "max",
                   renormalize=w.renormalize, route_scale=w.route_scale,
                   k_per_group=w.k_per_group)
        dt = 1 if w.dtype == "bf16" else 0
        self.plan = ({"path": "hash", "kernels": None} if w.hash_vocab
                     else tda.route_dispatch_plan(T, w.d, E, k, dt, **pkw))
        ws_bytes = tda.route_dispatch_workspace_size(T, w.d, E, k, dt, **pkw)
        ws = torch.empty(max(1, ws_bytes), dtype=torch.uint8, device=dev)
        route_bytes = (tda.route_workspace_size(T, w.d, E, k, dt, **pkw) + 255) // 256 * 256
        rkw = dict(score=w.score, logit_bias=lb, select_bias=sb, k_per_token=kpt,
                   n_groups=w.n_groups, topk_groups=w.topk_groups,
                   group_score=w.group_score if w.n_groups > 1 else None,
                   renormalize=w.renormalize, route_scale=w.route_scale,
                   k_per_group=w.k_per_group)
        outs = dict(ids=self.ids, weights=self.weights, counts=self.counts,
                    offsets=self.offsets, perm=self.perm, inv=self.inv, maxvio=self.maxvio)
        xs, n = self.xs, self.n_copies

        # the call's arguments are checked and marshalled once; each step
        # passes the next copy of x (one moe_route_dispatch call: gate,
        # selection, dispatch)
        call = (None if w.hash_vocab else
                tda.prepare_route_dispatch(xs[0], W, k, workspace=ws, **outs, **rkw))

        def step(i):
            call(xs[i % n])

        if w.capacity_factor:  # the dispatch ends with the capacity limit
            C = wl.capacity(w)
            slot = torch.empty(T * k, dtype=i32, device=dev)
            kept = torch.empty(E, dtype=i32, device=dev)
            dropped = torch.empty(1, dtype=i32, device=dev)

            def step(i):  # noqa: F811 -- moe_route_dispatch, then the capacity limit
                call(xs[i % n])
                tda.dispatch_capacity(self.ids, E, C, self.offsets, self.inv, slot=slot,
                                      kept=kept, dropped=dropped)

        self.disp_ws = ws_bytes - route_bytes  # the dispatch's tile data
        if w.hash_vocab:
            tok, tab = up(inp["token_ids"]), up(inp["tid2eid"])
            hb = tda.route_hash_dispatch_workspace_size(T, w.d, E, k, dt, **pkw)
            hws = torch.empty(max(1, hb), dtype=torch.uint8, device=dev)
            self.disp_ws = hb - (tda.route_hash_workspace_size(T, w.d, E, k, dt, **pkw)
                                 + 255) // 256 * 256

            def step(i):  # noqa: F811 -- moe_route_hash_dispatch
                tda.route_hash_dispatch(tok, tab, E, x=xs[i % n], W=W, score=w.score,
                                        logit_bias=lb, renormalize=w.renormalize,
                                        route_scale=w.route_scale, workspace=hws, **outs)

        self.step = step
        self.xbytes = xbytes

    def up(self, a):
        import numpy as np
        import torch
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(self.dev).view(
                torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(self.dev)

    def timed(self, steps):
        """Average ms of `steps` steps between two events on the current stream."""
        import torch
        stream = torch.cuda.current_stream(self.dev)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ev0.record(stream)
        for i in range(steps):
            self.step(i)
        ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / steps

    def kernels(self, n_prof, traffic_path):
        """Per-kernel average times (library's start/stop events), bytes, flops
        and binding roofline; returns (stages, dominant stage)."""
        import torch

        import token_dispatch_amd as tda
        w = self.w
        tda.profile_enable(True)
        for i in range(n_prof):
            self.step(i)
        torch.cuda.synchronize()
        prof = tda.profile_read()
        tda.profile_enable(False)
        T, R = w.T, w.T * w.k
        self.R_valid = int(self.counts.sum().item())
        two = "disp_scan" not in prof or not prof["disp_scan"][1]
        tile_bytes = self.disp_ws if two else (self.disp_ws - 4 * w.E) // 2
        ran = {name for name, (_, n) in prof.items() if n}
        # a hash layer whose dot-product kernel placed the dispatch
        beside = bool(w.hash_vocab) and "hash_dots" in ran and "disp_scatter" not in ran
        work = kernel_work(w, T, R, self.R_valid, tile_bytes,
                           producer_hist="disp_hist" not in ran and not beside,
                           beside_rows=-(-R // 2048) * w.E * 4 if beside else 0)
        stages = {}
        for name, (ms, n) in prof.items():
            if n and name in work:
                us = ms / n * 1e3
                nbytes, flops = work[name]
                rf = roofline(nbytes, flops, us, w.dtype)
                stages[name] = {"avg_us": round(us, 3), "launches": n, "bytes": nbytes,
                                "flops": flops, **rf,
                                "traffic": measured_traffic(traffic_path, w.name, name)}
        dom = max(stages, key=lambda s: stages[s]["avg_us"])
        return stages, dom


def measure(w, inp, dev, args, *, headline):
    """Time one workload: K eager steps after W warm-up steps, per-kernel
    roofline, pipeline fractions; the headline also gets the single-step
    spread, HIP-graph replays and the combine / send-buffer measurements."""
    import numpy as np
    import torch

    import token_dispatch_amd as tda
    import workloads as wl

    case = Case(w, inp, dev)
    T, E, k = w.T, w.E, w.k
    warm = args.warmup if headline else max(args.warmup, 200)
    steps = args.steps if headline else max(args.steps, 100)
    log(f"[bench] {w.name}: T={T} d={w.d} E={E} k={k}; {case.n_copies} rotating copies of x "
        f"({case.xbytes / 1e6:.1f} MB each); plan {case.plan['path']} "
        f"({case.plan['kernels']} kernels); warmup {warm}, steps {steps}")
    out = {}
    if headline:
        # the headline's own extras first, at settled clocks: the spread of
        # single steps (each between its own pair of events) and the HIP-graph
        # replays
        settle(case, args.settle_ms)
        n_each = min(max(steps, 20), 200)
        stream = torch.cuda.current_stream(dev)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n_each)]
        for i, (a, b) in enumerate(evs):
            a.record(stream)
            case.step(i)
            b.record(stream)
        torch.cuda.synchronize()
        each = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
        out["step_us"] = {"n": n_each, "median": round(float(np.median(each)), 3),
                          "p10": round(float(np.percentile(each, 10)), 3),
                          "p90": round(float(np.percentile(each, 90)), 3)}
        if not args.no_graph:
            out["graph"] = graph_replay(case, max(steps, 20), dev, args.settle_ms)
    out["settle"] = settle(case, args.settle_ms)
    for i in range(warm):
        case.step(i)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ms_per_step = case.timed(steps)
    wall = time.perf_counter() - wall0
    log(f"[bench] {w.name}: {ms_per_step * 1e3:.2f} us/step (wall {wall / steps * 1e6:.2f} us)")
    out.update({"T": T, "d": w.d, "E": E, "k_max": k, "steps": steps, "warmup": warm,
                "ms_per_step": round(ms_per_step, 6),
                "tokens_per_s": round(T / (ms_per_step / 1e3), 1),
                "plan": case.plan["path"], "kernels_per_step": case.plan["kernels"]})
    if not headline and not args.no_graph:
        out["graph"] = graph_replay(case, steps, dev, args.settle_ms)

    stages, dom = case.kernels(min(steps, 100), args.traffic)
    for s, v in stages.items():
        log(f"[bench] {w.name}: {s:15s} {v['avg_us']:9.2f} us  {v['bound']} {v['achieved']} "
            f"{v['unit']} ({v['frac']:.3f})")
    d = stages[dom]
    out["stages"] = stages
    out["roofline"] = {"bound": d["bound"], "kernel": dom, "achieved": d["achieved"],
                       "peak": d["peak"], "unit": d["unit"], "frac": d["frac"],
                       "traffic": d["traffic"], "hbm_frac": d["hbm_frac"],
                       "mfma_frac": d["mfma_frac"]}
    out["pipeline"] = pipeline_roofline(w, T, T * k, case.R_valid, ms_per_step * 1e3)
    out["maxvio"] = round(float(case.maxvio.item()), 6)
    log(f"[bench] {w.name}: staged roofline {out['pipeline']['t_roof_staged_us']} us -> "
        f"pipeline fraction {out['pipeline']['frac_staged']}; MaxVio {out['maxvio']}")
    if headline and not args.no_combine and case.R_valid > 0:
        out.update(row_movement(case, dev, args))
    del case
    torch.cuda.empty_cache()
    return out


def settle(case, ms):
    """Untimed steps, back to back, for at least `ms` of wall time before the
    W warm-up steps: from an idle GPU the first few hundred gpt-oss-like
    steps run up to ~15 % slower (the fused kernel 78-88 us for ~30 ms of
    load, then 73.7-74.5 us for as long as the load lasts), a power-state
    ramp that W = 5 steps do not cover.  Returns the steps and time spent."""
    import torch
    t0 = time.perf_counter()
    n = 0
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(32):
            case.step(n)
            n += 1
        torch.cuda.synchronize()
    return {"steps": n, "ms": round((time.perf_counter() - t0) * 1e3, 1)}


def capture_graphs(case, dev):
    """HIP graphs of the step: one per copy of x (one step each), and one
    holding a step for every copy of x in order."""
    import torch
    n = case.n_copies
    cs = torch.cuda.Stream(dev)
    cs.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(cs):
        case.step(0)
    torch.cuda.current_stream(dev).wait_stream(cs)
    torch.cuda.synchronize()
    singles = []
    for i in range(n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            case.step(i)
        singles.append(g)
    many = torch.cuda.CUDAGraph()
    with torch.cuda.graph(many):
        for i in range(n):
            case.step(i)
    torch.cuda.synchronize()
    return singles, many


def time_enqueued(fn, reps, dev, warm=20):
    """(GPU us per rep between two events, host us per rep spent enqueuing)."""
    import torch
    stream = torch.cuda.current_stream(dev)
    for i in range(min(reps, warm)):
        fn(i)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    h0 = time.perf_counter()
    for i in range(reps):
        fn(i)
    h1 = time.perf_counter()
    ev1.record(stream)
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / reps * 1e3, (h1 - h0) / reps * 1e6


def graph_replay(case, steps, dev, settle_ms):
    """The same steps replayed from HIP graphs: one graph per step (one per
    copy of x), and one graph holding a step for every copy of x in order;
    with the host's enqueue time per step of each form.  The capture idles
    the GPU, so the clocks are settled again before the replays."""
    n = case.n_copies
    singles, many = capture_graphs(case, dev)
    settle(case, settle_ms)
    one, one_h = time_enqueued(lambda i: singles[i % n].replay(), steps, dev)
    reps = max(1, steps // n)
    multi, multi_h = time_enqueued(lambda i: many.replay(), reps, dev)
    eager, eager_h = time_enqueued(case.step, steps, dev)
    out = {"one_step_graphs_us": round(one, 3), "steps_per_graph": n,
           "multi_step_graph_us": round(multi / n, 3), "multi_step_replays": reps,
           "eager_us": round(eager, 3),
           "host_enqueue_us": {"one_step_graph": round(one_h, 2),
                               "multi_step_graph": round(multi_h / n, 2),
                               "eager": round(eager_h, 2)}}
    log(f"[bench] {case.w.name}: graph replay {out['one_step_graphs_us']} us/step "
        f"(one step per graph), {out['multi_step_graph_us']} us/step ({n} steps per graph), "
        f"eager {out['eager_us']}; host enqueue per step {out['host_enqueue_us']}")
    del singles, many
    return out


def graph_phases(case, dev, steps):
    """Eager steps, one-step graphs and a many-step graph, each phase
    between idle gaps of 30 ms (so that a kernel trace splits into phases),
    twice; GPU and host-enqueue microseconds per step of each."""
    n = case.n_copies
    singles, many = capture_graphs(case, dev)
    settle(case, 100.0)
    res = []
    for rep in range(2):
        for name, fn, reps, per in (
                ("eager", case.step, steps, 1),
                ("one_step_graphs", lambda i: singles[i % n].replay(), steps, 1),
                ("multi_step_graph", lambda i: many.replay(), max(1, steps // n), n)):
            time.sleep(0.03)
            g, h = time_enqueued(fn, reps, dev, warm=0)
            res.append({"phase": name, "round": rep, "steps": reps * per,
                        "gpu_us_per_step": round(g / per, 3),
                        "host_enqueue_us_per_step": round(h / per, 3)})
            log(f"[bench] {case.w.name}: {name}: {res[-1]['gpu_us_per_step']} us/step on the "
                f"GPU, host enqueue {res[-1]['host_enqueue_us_per_step']} us/step")
            time.sleep(0.03)
    del singles, many
    return res


def row_movement(case, dev, args):
    """The combine that follows the experts and the send buffer, each timed on
    its own on the step's dispatch (not part of a step): synthetic expert
    outputs in dispatch order plus a shared expert's output; rotating copies
    larger than the last-level cache."""
    import torch

    import token_dispatch_amd as tda
    import workloads as wl
    w, T, k = case.w, case.w.T, case.w.k
    R_valid = case.R_valid
    eb = 2 if w.dtype == "bf16" else 4
    Y_np, sh_np = wl.expert_outputs(w, R_valid), wl.shared_output(w)
    Y0 = case.up(Y_np)
    n_yc = max(1, min(16, math.ceil(3 * LLC_BYTES / (R_valid * w.d * eb))))
    Ys = [Y0] + [torch.roll(Y0, shifts=89 * i, dims=0).contiguous() for i in range(1, n_yc)]
    sh = case.up(sh_np)
    yout = torch.empty((T, w.d), dtype=Y0.dtype, device=dev)
    for i in range(20):
        tda.combine(Ys[i % n_yc], case.inv, case.weights, shared=sh, out=yout)
    torch.cuda.synchronize()
    tda.profile_enable(True)
    n_c = 50
    for i in range(n_c):
        tda.combine(Ys[i % n_yc], case.inv, case.weights, shared=sh, out=yout)
    torch.cuda.synchronize()
    cms, cn = tda.profile_read()["combine"]
    tda.profile_enable(False)
    c_us = cms / cn * 1e3
    cbytes = R_valid * w.d * eb + T * k * 8 + 2 * T * w.d * eb  # rows, inv+weights, shared, y
    c_gbs = cbytes / (c_us * 1e-6) / 1e9
    combine = {"kernel": "combine", "avg_us": round(c_us, 3), "launches": cn, "bytes": cbytes,
               "achieved": round(c_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
               "frac": round(c_gbs / HBM_PEAK_GBS, 4), "rows": R_valid, "d": w.d,
               "shared": True, "row_copies": n_yc}
    log(f"[bench] combine       {c_us:9.2f} us  {c_gbs:.1f} GB/s ({R_valid} rows of {w.d})")
    del Ys, Y0
    # the send buffer (token rows in dispatch order, the all-to-all's input
    # under expert parallelism), timed the same way
    x0 = case.up(case.inp["x"])
    n_xc = max(1, min(16, math.ceil(3 * LLC_BYTES / (T * w.d * eb))))
    xs = [x0] + [torch.roll(x0, shifts=89 * i, dims=0).contiguous() for i in range(1, n_xc)]
    sbuf = torch.empty((T * k, w.d), dtype=x0.dtype, device=dev)
    for i in range(20):
        tda.permute_rows(xs[i % n_xc], case.inv, k, T * k, out=sbuf)
    torch.cuda.synchronize()
    tda.profile_enable(True)
    for i in range(n_c):
        tda.permute_rows(xs[i % n_xc], case.inv, k, T * k, out=sbuf)
    torch.cuda.synchronize()
    pms, pn = tda.profile_read()["permute"]
    tda.profile_enable(False)
    p_us = pms / pn * 1e3
    pbytes = T * w.d * eb + R_valid * w.d * eb + T * k * 4  # rows in once, out once, inv
    p_gbs = pbytes / (p_us * 1e-6) / 1e9
    permute = {"kernel": "permute", "avg_us": round(p_us, 3), "launches": pn, "bytes": pbytes,
               "achieved": round(p_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
               "frac": round(p_gbs / HBM_PEAK_GBS, 4), "rows": R_valid, "d": w.d,
               "row_copies": n_xc}
    log(f"[bench] permute       {p_us:9.2f} us  {p_gbs:.1f} GB/s ({R_valid} rows of {w.d})")
    del sbuf, xs, x0
    if not args.no_cpu_baseline:
        combine["cpu_baseline"] = combine_cpu_baseline(
            Y_np, case.inv.cpu().numpy().reshape(T, k), case.weights.cpu().numpy(), sh_np)
    return {"combine": combine, "permute": permute}


def describe(w):
    import workloads as wl
    k = w.k
    return (f"{w.name}: T={w.T} tokens, d={w.d}, E={w.E}, "
            f"k={'/'.join(map(str, w.dynamic_k)) + ' per request' if w.dynamic_k else k}, "
            f"score={w.score}, groups={w.n_groups}/{w.topk_groups}, "
            + (f"hash ids from tid2eid[{w.hash_vocab}][{k}], " if w.hash_vocab else "")
            + f"dispatch over {w.E} experts"
            + (f" with capacity {wl.capacity(w)}" if w.capacity_factor else ""))


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--settle-ms", type=float, default=150.0,
                    help="untimed back-to-back steps for this long before the W warm-up "
                         "steps of every workload (power-state ramp)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--config-cpu-seconds", type=float, default=3.0)
    ap.add_argument("--no-configs", action="store_true",
                    help="time only --workload (no `configs` object)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-combine", action="store_true",
                    help="skip the separate measurement of the combine and send buffer")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager launches only (no HIP graph replay)")
    ap.add_argument("--graph-phases", action="store_true",
                    help="only time eager steps, one-step graphs and a many-step graph of "
                         "--workload, in phases between idle gaps (for a kernel trace)")
    ap.add_argument("--calibrate-copy-mb", type=float, default=0.0,
                    help="only run a plain device copy of this many MB (counter calibration)")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="JSON with counter-measured HBM bytes per launch (rocprofv3 --pmc)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the router and dispatch run on one device "
              "(no collectives); run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.calibrate_copy_mb > 0:
        # a plain copy of known size: what FETCH_SIZE / WRITE_SIZE read for
        # it scales the counters of the routing kernels
        n = int(args.calibrate_copy_mb * 1e6) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(max(1, args.steps)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n * 4, "launches": max(1, args.steps)}), flush=True)
        return

    import token_dispatch_amd as tda
    import workloads as wl

    tda.lib()  # fails loudly when the HIP library is not built
    dev = torch.device("cuda:0")
    threads = host_threads()
    w = wl.WORKLOADS[args.workload]

    # the headline's inputs first, then the other routing configurations
    # (their own warm-up and steps), then the headline: the configurations'
    # GPU work brings the clocks up, and no input generation idles the GPU
    # between them and the headline's W warm-up and K timed steps
    log(f"[bench] generating {w.name} inputs (T={w.T}, d={w.d}, E={w.E})")
    inp = wl.make_inputs(w)
    if args.graph_phases:
        res = graph_phases(Case(w, inp, dev), dev, max(args.steps, 96))
        print(json.dumps({"workload": describe(w), "graph_phases": res}), flush=True)
        return
    configs, config_inputs = {}, {}
    if not args.no_configs:
        shared = {}
        for name in CONFIGS:
            if name == w.name:
                continue
            cw = wl.WORKLOADS[name]
            key = (cw.T, cw.d, cw.E, cw.dtype)
            log(f"[bench] generating {name} inputs")
            cinp = wl.make_inputs(cw)
            if key in shared:  # the V4-like hash layer shares x and W with the V4-like one
                cinp["x"], cinp["W"] = shared[key]
            shared[key] = (cinp["x"], cinp["W"])
            res = measure(cw, cinp, dev, args, headline=False)
            res["workload"] = describe(cw)
            configs[name] = res
            config_inputs[name] = cinp
        shared.clear()

    head = measure(w, inp, dev, args, headline=True)
    configs[w.name] = {k: v for k, v in head.items() if k not in ("combine", "permute")}
    configs[w.name]["workload"] = describe(w)

    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] timing the CPU oracle on {threads} host threads")
        cpu = cpu_baseline(w, inp, args.cpu_seconds, threads)
        configs[w.name]["cpu_baseline"] = cpu
        for name, cinp in config_inputs.items():
            configs[name]["cpu_baseline"] = cpu_baseline(wl.WORKLOADS[name], cinp,
                                                         args.config_cpu_seconds, threads)

    ms = head["ms_per_step"]
    out = {
        "metric": METRIC,
        "value": round(w.T / (ms / 1e3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "timing": "eager launches on one stream",
        "settle": head["settle"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": describe(w), "T": w.T, "d": w.d, "E": w.E, "k_max": w.k},
        "step_us": head.get("step_us"),
        "graph": head.get("graph"),
        "inputs": inputs_record(inp),
        "stages": head["stages"],
        "pipeline": head["pipeline"],
        "maxvio": head["maxvio"],
        "roofline": head["roofline"],
        "combine": head.get("combine"),
        "permute": head.get("permute"),
        "cpu_baseline": cpu,
        "configs": configs,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
