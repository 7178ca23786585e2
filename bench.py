#!/usr/bin/env python3
"""Routed tokens/s of the MoE router + dispatch hot path on one MI355X.

One step = one moe_route_dispatch call -- the gate contraction, scoring,
selection and weights of moe_route, then the histogram, offsets,
permutation and inverse of moe_dispatch -- over one batch of seeded
synthetic tokens (hash workloads: moe_route_hash, whose ids come from the
token-id table and whose weights from the k gathered gate logits, then
moe_dispatch).  Inputs are resident in HBM before timing; each step
routes a different copy of x (rotating through copies totalling more than the
256 MB last-level cache) so the gate reads x from HBM, not from cache.

Prints one JSON line with the throughput, the dominant kernel's roofline
fraction (kernel time from HIP events recorded on the launch stream by the
library's per-kernel timing) and the CPU oracle's throughput on a bounded
sample of the same workload.  The combine that follows the experts (the
weighted sum of each token's expert outputs, moe_combine) is not part of a
step; it is timed separately on synthetic expert outputs in the step's
dispatch order and reported with its own HBM fraction ("combine"), and so
is the send buffer of token rows in dispatch order (moe_permute_rows,
"permute").

Usage: python bench.py [--steps K] [--warmup W] [--workload NAME]
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
MFMA_BF16_PEAK_TFLOPS = 2516.6
LLC_BYTES = 256 << 20


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def stage_bytes(w, T, R, R_valid, tile_bytes):
    """Algorithmic HBM bytes per launch of each kernel (inputs read once,
    outputs written once); tile_bytes: the dispatch's per-tile histogram
    data (written once, read once by the placement)."""
    xb = 2 if w.dtype == "bf16" else 4
    E, d, k = w.E, w.d, w.k
    return {
        "gate": T * d * xb + E * d * xb + T * E * 4,
        # the gate kernel with the selection fused: no logits leave the chip
        "gate_select": T * d * xb + E * d * xb + T * k * 8 + (T * 4 if w.dynamic_k else 0)
        + tile_bytes,
        "hash": T * 4 + T * k * 4 + T * d * xb + E * d * xb + T * k * 8,
        "select": T * E * 4 + T * k * 8 + (T * 4 if w.dynamic_k else 0),
        # small batches: selection and the whole dispatch in one workgroup
        "select_dispatch": T * E * 4 + T * k * 8 + (T * 4 if w.dynamic_k else 0)
        + R * 4 + R_valid * 4 + E * 8,
        "disp_hist": R * 4 + tile_bytes,
        "disp_scan": 2 * tile_bytes + E * 4,
        "disp_scatter": tile_bytes + E * 4 + R * 4 + R * 4 + R_valid * 4 + E * 8,
        # capacity limit: ids and positions read, slots written, kept counts
        "capacity": R * 12 + E * 8 + 4,
    }


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


def pipeline_roofline(w, T, R, R_valid, step_us):
    """Lower bounds on a whole step at the MI355X peaks (8 TB/s, 2.5 PFLOP/s
    bf16 / 157.3 TFLOP/s fp32) and the step's fraction of each: staged = the
    gate (max of its flops and its bytes, logits written once) + the
    selection (logits read once, ids and weights written) + the dispatch
    (ids read, perm, inv, counts and offsets written) [+ the capacity
    limit]; fused = no logits hand-off, one pass over x and W."""
    xb = 2 if w.dtype == "bf16" else 4
    E, d, k = w.E, w.d, w.k
    bw = HBM_PEAK_GBS * 1e9
    peak = (MFMA_BF16_PEAK_TFLOPS if w.dtype == "bf16" else 157.3) * 1e12
    flops = 2.0 * T * d * E
    kt = T * 4 if w.dynamic_k else 0
    xw = T * d * xb + E * d * xb
    disp = R * 4 + R_valid * 4 + R * 4 + E * 8
    cap = R * 12 + E * 8 + 4 if w.capacity_factor else 0
    staged = (max(flops / peak, (xw + T * E * 4) / bw) + (T * E * 4 + T * k * 8 + kt) / bw
              + (disp + cap) / bw)
    fused = max(flops / peak, (xw + T * k * 8 + kt + disp + cap) / bw)
    return {"t_roof_staged_us": round(staged * 1e6, 3), "frac_staged": round(staged * 1e6 / step_us, 4),
            "t_roof_fused_us": round(fused * 1e6, 3), "frac_fused": round(fused * 1e6 / step_us, 4)}


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
        lg = oracle.gate(wl.rows(inp["x"], np.arange(n)), inp["W"], inp["logit_bias"])
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
    return {"value": reps * n / total, "unit": "tokens/s",
            "cores": 1 if w.hash_vocab else threads, "kind": "oracle",
            "sample": f"{'first %d of ' % n if n < w.T else 'all '}{w.T} tokens of the same "
                      f"workload x {reps} ({what}, fp64), {total:.1f} s"}


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


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--workload", default="qwen3_dynk")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-combine", action="store_true",
                    help="skip the separate measurement of the combine kernel")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager launches only (no HIP graph replay)")
    ap.add_argument("--calibrate-copy-mb", type=float, default=0.0,
                    help="only run a plain device copy of this many MB (counter calibration)")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="JSON with counter-measured HBM bytes per launch (rocprofv3 --pmc)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the router and dispatch run on one device "
              "(no collectives); run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
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

    w = wl.WORKLOADS[args.workload]
    log(f"[bench] generating {w.name} inputs (T={w.T}, d={w.d}, E={w.E})")
    inp = wl.make_inputs(w)
    dev = torch.device("cuda:0")

    def up(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(
                torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    x0 = up(inp["x"])
    xbytes = x0.numel() * x0.element_size()
    n_copies = max(1, min(64, math.ceil(3 * LLC_BYTES / xbytes)))
    xs = [x0] + [torch.roll(x0, shifts=97 * i, dims=0).contiguous() for i in range(1, n_copies)]
    W = up(inp["W"])
    lb, sb, kpt = up(inp["logit_bias"]), up(inp["select_bias"]), up(inp["k_per_token"])
    T, E, k = w.T, w.E, w.k
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    weights = torch.empty((T, k), dtype=torch.float32, device=dev)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(T * k, dtype=torch.int32, device=dev)
    inv = torch.empty(T * k, dtype=torch.int32, device=dev)
    pkw = dict(score=w.score, n_groups=w.n_groups, topk_groups=w.topk_groups,
               group_score=w.group_score if w.n_groups > 1 else "max",
               renormalize=w.renormalize, route_scale=w.route_scale, k_per_group=w.k_per_group)
    dt = 1 if w.dtype == "bf16" else 0
    ws_bytes = tda.route_dispatch_workspace_size(T, w.d, E, k, dt, **pkw)
    ws = torch.empty(max(1, ws_bytes), dtype=torch.uint8, device=dev)
    route_bytes = (tda.route_workspace_size(T, w.d, E, k, dt, **pkw) + 255) // 256 * 256
    rkw = dict(score=w.score, logit_bias=lb, select_bias=sb, k_per_token=kpt,
               n_groups=w.n_groups, topk_groups=w.topk_groups,
               group_score=w.group_score if w.n_groups > 1 else None,
               renormalize=w.renormalize, route_scale=w.route_scale, k_per_group=w.k_per_group)

    def step(i):  # one moe_route_dispatch call: gate, selection, dispatch
        tda.route_dispatch(xs[i % n_copies], W, k, ids=ids, weights=weights, counts=counts,
                           offsets=offsets, perm=perm, inv=inv, workspace=ws, **rkw)

    if w.capacity_factor:  # the dispatch ends with the capacity limit
        C = wl.capacity(w)
        slot = torch.empty(T * k, dtype=torch.int32, device=dev)
        kept = torch.empty(E, dtype=torch.int32, device=dev)
        dropped = torch.empty(1, dtype=torch.int32, device=dev)

        def step(i):  # noqa: F811 -- moe_route_dispatch, then the capacity limit
            tda.route_dispatch(xs[i % n_copies], W, k, ids=ids, weights=weights, counts=counts,
                               offsets=offsets, perm=perm, inv=inv, workspace=ws, **rkw)
            tda.dispatch_capacity(ids, E, C, offsets, inv, slot=slot, kept=kept,
                                  dropped=dropped)

    disp_ws = ws_bytes - route_bytes  # the dispatch's tile data
    if w.hash_vocab:
        tok, tab = up(inp["token_ids"]), up(inp["tid2eid"])
        disp_ws = tda.dispatch_workspace_size(T, k, E)
        dws = torch.empty(max(1, disp_ws), dtype=torch.uint8, device=dev)
        hws = torch.empty(max(1, tda.route_hash_workspace_size(T, w.d, E, k, dt, **pkw)),
                          dtype=torch.uint8, device=dev)

        def step(i):  # noqa: F811 -- moe_route_hash then moe_dispatch
            tda.route_hash(tok, tab, E, x=xs[i % n_copies], W=W, score=w.score,
                           logit_bias=lb, renormalize=w.renormalize,
                           route_scale=w.route_scale, ids=ids, weights=weights,
                           workspace=hws)
            tda.dispatch(ids, E, counts=counts, offsets=offsets, perm=perm, inv=inv,
                         workspace=dws)

    log(f"[bench] {n_copies} rotating copies of x ({xbytes / 1e6:.1f} MB each); "
        f"warmup {args.warmup}, steps {args.steps}")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = ev0.elapsed_time(ev1)
    ms_per_step = ms_total / args.steps
    value = T / (ms_per_step / 1e3)
    log(f"[bench] {ms_per_step * 1e3:.2f} us/step (wall {wall / args.steps * 1e6:.2f} us/step)")

    # the spread of single steps: each of n_each steps between its own pair
    # of events (after the timed run; the pairs add a little per step)
    n_each = min(args.steps, 200)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n_each)]
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        step(i)
        b.record(stream)
    torch.cuda.synchronize()
    each_us = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
    step_spread = {"n": n_each, "median": round(float(np.median(each_us)), 3),
                   "p10": round(float(np.percentile(each_us, 10)), 3),
                   "p90": round(float(np.percentile(each_us, 90)), 3)}
    log(f"[bench] single steps: median {step_spread['median']} us, p10 {step_spread['p10']}, "
        f"p90 {step_spread['p90']}")

    # the same steps replayed from HIP graphs (one per copy of x): no Python
    # or launch-API cost between kernels
    graph_ms = None
    if not args.no_graph:
        graphs = []
        cs = torch.cuda.Stream(dev)
        cs.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(cs):
            step(0)
        torch.cuda.current_stream(dev).wait_stream(cs)
        torch.cuda.synchronize()
        for i in range(n_copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(i)
            graphs.append(g)
        for i in range(args.warmup):
            graphs[i % n_copies].replay()
        torch.cuda.synchronize()
        ev0.record(stream)
        for i in range(args.steps):
            graphs[i % n_copies].replay()
        ev1.record(stream)
        torch.cuda.synchronize()
        graph_ms = ev0.elapsed_time(ev1) / args.steps
        log(f"[bench] graph replay: {graph_ms * 1e3:.2f} us/step")

    # per-kernel times from HIP events the library records on the launch stream
    n_prof = min(args.steps, 100)
    tda.profile_enable(True)
    for i in range(n_prof):
        step(i)
    torch.cuda.synchronize()
    prof = tda.profile_read()
    tda.profile_enable(False)

    R = T * k
    R_valid = int(counts.sum().item())
    tile_bytes = disp_ws if "disp_scan" not in prof or not prof["disp_scan"][1] else (disp_ws - 4 * E) // 2
    sbytes = stage_bytes(w, T, R, R_valid, tile_bytes)
    stages = {}
    for name, (ms, n) in prof.items():
        if n:
            avg_us = ms / n * 1e3
            stages[name] = {"avg_us": round(avg_us, 3), "launches": n,
                            "bytes": sbytes.get(name),
                            "GBs": round(sbytes[name] / (avg_us * 1e-6) / 1e9, 1)
                            if name in sbytes else None}
    dom = max(stages, key=lambda s: stages[s]["avg_us"])
    dom_us = stages[dom]["avg_us"]
    achieved = sbytes[dom] / (dom_us * 1e-6) / 1e9
    traffic = measured_traffic(args.traffic, w.name, dom)
    gate_flops = 2.0 * T * w.d * E
    gs = "gate_select" if "gate_select" in stages else ("gate" if "gate" in stages else None)
    maxvio = float(counts.max().item()) / (R_valid / E) - 1.0 if R_valid else 0.0
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic,
                "gate_mfma_frac": round(gate_flops / (stages[gs]["avg_us"] * 1e-6) / 1e12
                                        / MFMA_BF16_PEAK_TFLOPS, 4) if gs else None}
    for s, v in stages.items():
        log(f"[bench] {s:13s} {v['avg_us']:9.2f} us  {v['GBs']} GB/s")
    pipeline = pipeline_roofline(w, T, R, R_valid, ms_per_step * 1e3)
    log(f"[bench] staged roofline {pipeline['t_roof_staged_us']} us -> pipeline fraction "
        f"{pipeline['frac_staged']}")

    # the combine that follows the experts, timed on its own (not part of a
    # step): synthetic expert outputs in this step's dispatch order plus a
    # shared expert's output; rotating copies of the rows keep them from
    # being served out of the last-level cache
    combine = permute = None
    if not args.no_combine and R_valid > 0:
        eb = 2 if w.dtype == "bf16" else 4
        Y_np, sh_np = wl.expert_outputs(w, R_valid), wl.shared_output(w)
        Y0 = up(Y_np)
        n_yc = max(1, min(16, math.ceil(3 * LLC_BYTES / (R_valid * w.d * eb))))
        Ys = [Y0] + [torch.roll(Y0, shifts=89 * i, dims=0).contiguous() for i in range(1, n_yc)]
        sh = up(sh_np)
        yout = torch.empty((T, w.d), dtype=Y0.dtype, device=dev)
        for i in range(20):
            tda.combine(Ys[i % n_yc], inv, weights, shared=sh, out=yout)
        torch.cuda.synchronize()
        tda.profile_enable(True)
        n_c = 50
        for i in range(n_c):
            tda.combine(Ys[i % n_yc], inv, weights, shared=sh, out=yout)
        torch.cuda.synchronize()
        cms, cn = tda.profile_read()["combine"]
        tda.profile_enable(False)
        c_us = cms / cn * 1e3
        cbytes = R_valid * w.d * eb + T * k * 8 + 2 * T * w.d * eb  # rows, inv+weights, shared, y
        c_gbs = cbytes / (c_us * 1e-6) / 1e9
        combine = {"kernel": "combine", "avg_us": round(c_us, 3), "launches": cn,
                   "bytes": cbytes, "achieved": round(c_gbs, 1), "peak": HBM_PEAK_GBS,
                   "unit": "GB/s", "frac": round(c_gbs / HBM_PEAK_GBS, 4), "rows": R_valid,
                   "d": w.d, "shared": True, "row_copies": n_yc}
        log(f"[bench] combine       {c_us:9.2f} us  {c_gbs:.1f} GB/s ({R_valid} rows of {w.d})")
        # the send buffer (token rows in dispatch order, the all-to-all's
        # input under expert parallelism), timed the same way
        x0 = up(inp["x"])
        n_xc = max(1, min(16, math.ceil(3 * LLC_BYTES / (T * w.d * eb))))
        xs = [x0] + [torch.roll(x0, shifts=89 * i, dims=0).contiguous() for i in range(1, n_xc)]
        sbuf = torch.empty((T * k, w.d), dtype=x0.dtype, device=dev)
        for i in range(20):
            tda.permute_rows(xs[i % n_xc], inv, k, T * k, out=sbuf)
        torch.cuda.synchronize()
        tda.profile_enable(True)
        for i in range(n_c):
            tda.permute_rows(xs[i % n_xc], inv, k, T * k, out=sbuf)
        torch.cuda.synchronize()
        pms, pn = tda.profile_read()["permute"]
        tda.profile_enable(False)
        p_us = pms / pn * 1e3
        # each token row read once, every placed route's row written once,
        # inv read
        pbytes = T * w.d * eb + R_valid * w.d * eb + T * k * 4
        p_gbs = pbytes / (p_us * 1e-6) / 1e9
        permute = {"kernel": "permute", "avg_us": round(p_us, 3), "launches": pn,
                   "bytes": pbytes, "achieved": round(p_gbs, 1), "peak": HBM_PEAK_GBS,
                   "unit": "GB/s", "frac": round(p_gbs / HBM_PEAK_GBS, 4), "rows": R_valid,
                   "d": w.d, "row_copies": n_xc}
        log(f"[bench] permute       {p_us:9.2f} us  {p_gbs:.1f} GB/s ({R_valid} rows of {w.d})")
        del sbuf, xs, x0
        if not args.no_cpu_baseline:
            combine["cpu_baseline"] = combine_cpu_baseline(
                Y_np, inv.cpu().numpy().reshape(T, k), weights.cpu().numpy(), sh_np)
        del Ys, Y0, Y_np

    cpu = None
    if not args.no_cpu_baseline:
        try:
            threads = min(16, len(os.sched_getaffinity(0)))
        except AttributeError:
            threads = min(16, os.cpu_count() or 1)
        log(f"[bench] timing the CPU oracle on {threads} threads (~{args.cpu_seconds:.0f} s)")
        cpu = cpu_baseline(w, inp, args.cpu_seconds, threads)

    out = {
        "metric": "routed tokens/sec (gate+select+dispatch) and % of MFMA/HBM roofline, 1 MI355X",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 6),
        "timing": "eager launches on one stream",
        "graph_ms_per_step": None if graph_ms is None else round(graph_ms, 6),
        "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": f"{w.name}: T={T} tokens, d={w.d}, E={E}, "
                               f"k={'/'.join(map(str, w.dynamic_k)) + ' per request' if w.dynamic_k else k}, "
                               f"score={w.score}, groups={w.n_groups}/{w.topk_groups}, "
                               + (f"hash ids from tid2eid[{w.hash_vocab}][{k}], "
                                  if w.hash_vocab else "")
                               + f"dispatch over {E} experts"
                               + (f" with capacity {wl.capacity(w)}" if w.capacity_factor else ""),
                   "T": T, "d": w.d, "E": E, "k_max": k, "x_copies": n_copies},
        "step_us": step_spread,
        "inputs": inputs_record(inp),
        "stages": stages,
        "pipeline": pipeline,
        "maxvio": round(maxvio, 4),
        "roofline": roofline,
        "combine": combine,
        "permute": permute,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
