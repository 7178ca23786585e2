"""Every token of every workload at full size, through the calls bench.py
times: moe_route_dispatch (gate, scoring, selection, weights, histogram,
offsets, permutation, inverse and MaxVio in one call; for the capacity
workload then moe_dispatch_capacity), and for the hash workload
moe_route_hash_dispatch.  Nothing is sampled: the oracle (fp64,
tokens split over host threads) routes every token and the acceptance rule
of tests/parity.py is applied to all of them; the dispatch arrays, the
capacity slots and MaxVio are compared bit for bit.

These are the shapes the kernels' plans take at full size (the reduced-T
tests take other plans: the gpt-oss-like gate fuses the selection and
writes 256 tiles x 128 experts of dispatch histograms only at T = 65536)."""
import os

import numpy as np
import pytest
import torch

import oracle
import token_dispatch_amd as tda
import workloads as wl
from tests.gpu_util import down, route_kwargs, say, up
from tests.parity import WTOL, check_dispatch, check_route, oracle_route

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def host_threads():
    """The host cores this process may use (the box's share when
    OMP_NUM_THREADS says so)."""
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS")
    return max(1, min(n, int(env))) if env and env.isdigit() else n


NT = host_threads()


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    tda.lib()


ROUTED = ["mixtral", "qwen3_dynk", "dsv3_grouped", "dsv4", "gptoss_skew", "dsv4_bias", "olmoe",
          "dsv3_groupmax", "grouped_quota", "switch_top1"]


@pytest.mark.parametrize("name", ROUTED)
def test_route_dispatch_every_token(name):
    w = wl.WORKLOADS[name]
    inp = wl.make_inputs(w)
    kw = route_kwargs(w)
    if kw["group_score"] is None:
        kw.pop("group_score")
    plan = tda.route_dispatch_plan(w.T, w.d, w.E, w.k, 1 if w.dtype == "bf16" else 0,
                                   **{key: v for key, v in kw.items() if key != "group_score"},
                                   group_score=kw.get("group_score") or "max")
    say("full size, every token", name, "T", w.T, "plan", plan["path"], plan["kernels"],
        "kernels")
    mv = torch.full((1,), -7.0, dtype=torch.float64, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    ids, wts, counts, offsets, perm, inv = tda.route_dispatch(
        up(inp["x"]), up(inp["W"]), w.k, logit_bias=up(inp["logit_bias"]),
        select_bias=up(inp["select_bias"]), k_per_token=up(inp["k_per_token"]), maxvio=mv,
        dev_err=err, **kw)
    slot = None
    if w.capacity_factor:
        slot, kept, dropped = tda.dispatch_capacity(ids, w.E, wl.capacity(w), offsets, inv)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    gids, gw = down(ids), down(wts)
    say("oracle on", NT, "threads")
    l64 = oracle.gate(inp["x"], inp["W"], inp["logit_bias"], nthreads=NT)
    ref = oracle_route(oracle, l64, w.k, score=w.score, select_bias=inp["select_bias"],
                       k_per_token=inp["k_per_token"], n_groups=w.n_groups,
                       topk_groups=w.topk_groups,
                       group_score=w.group_score if w.n_groups > 1 else None,
                       renormalize=w.renormalize, route_scale=w.route_scale,
                       k_per_group=w.k_per_group, nthreads=NT)
    stats = check_route(gids, gw, ref, oracle, score=w.score, renormalize=w.renormalize,
                        route_scale=w.route_scale, k_per_token=inp["k_per_token"],
                        n_groups=w.n_groups, topk_groups=w.topk_groups,
                        k_per_group=w.k_per_group, where=name)
    d = oracle.dispatch(gids, w.E)
    check_dispatch((counts, offsets, perm, inv), d)
    assert float(mv.item()) == oracle.maxvio(d["counts"])
    if slot is not None:
        c = oracle.capacity(gids, w.E, wl.capacity(w))
        np.testing.assert_array_equal(down(slot), c["slot"])
        np.testing.assert_array_equal(down(kept), c["kept"])
        assert int(dropped.item()) == c["dropped"]
    print(name, "every token:", stats, "maxvio", float(mv.item()), "plan", plan["path"])


def test_hash_every_token():
    w = wl.WORKLOADS["dsv4_hash"]
    inp = wl.make_inputs(w)
    say("hash, full size, every token")
    mv = torch.full((1,), -7.0, dtype=torch.float64, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    ids, wts, counts, offsets, perm, inv = tda.route_hash_dispatch(
        up(inp["token_ids"]), up(inp["tid2eid"]), w.E, x=up(inp["x"]), W=up(inp["W"]),
        score=w.score, renormalize=w.renormalize, route_scale=w.route_scale, maxvio=mv,
        dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    gids, gw = down(ids), down(wts)
    ref_ids, nerr = oracle.hash_ids(inp["token_ids"], inp["tid2eid"], w.E)
    assert nerr == 0
    np.testing.assert_array_equal(gids, ref_ids)
    l64 = oracle.gate(inp["x"], inp["W"], nthreads=NT)
    ref_w = oracle.weights_for_ids(l64, ref_ids, score=w.score, renormalize=w.renormalize,
                                   route_scale=w.route_scale)
    worst = float(np.max(np.abs(gw - ref_w)))
    assert worst <= WTOL, worst
    d = oracle.dispatch(gids, w.E)
    check_dispatch((counts, offsets, perm, inv), d)
    assert float(mv.item()) == oracle.maxvio(d["counts"])
    print("dsv4_hash every token: max |dw|", worst, "maxvio", float(mv.item()))


@pytest.mark.parametrize("T,k,E,skew", [(0, 4, 128, False), (1, 1, 8, False),
                                        (3000, 4, 128, True), (65536, 4, 128, True),
                                        (16384, 6, 384, False), (262144, 8, 384, True)])
def test_maxvio_matches_oracle(T, k, E, skew):
    """MaxVio from the dispatch kernels equals the oracle's on the same counts,
    bit for bit (the same fp64 expression), on every dispatch path."""
    rng = np.random.default_rng([T, k, E])
    if skew:
        e = (rng.zipf(1.3, size=(T, k)) - 1) % E
    else:
        e = rng.integers(0, E, size=(T, k))
    e = np.where(rng.random((T, k)) < 0.05, -1, e).astype(np.int32)
    say("maxvio", T, k, E, skew)
    mv = torch.full((1,), -7.0, dtype=torch.float64, device=DEV)
    counts, offsets, perm, inv = tda.dispatch(up(e), E, maxvio=mv)
    torch.cuda.synchronize()
    d = oracle.dispatch(e, E)
    check_dispatch((counts, offsets, perm, inv), d)
    assert float(mv.item()) == oracle.maxvio(d["counts"])


def test_maxvio_small_batch_path():
    """The one-workgroup route + dispatch kernel (Mixtral-like batch) writes
    MaxVio too."""
    w = wl.WORKLOADS["mixtral"]
    inp = wl.make_inputs(w, T=200)
    mv = torch.full((1,), -7.0, dtype=torch.float64, device=DEV)
    say("maxvio small path")
    ids, wts, counts, offsets, perm, inv = tda.route_dispatch(up(inp["x"]), up(inp["W"]), w.k,
                                                              score=w.score, maxvio=mv)
    torch.cuda.synchronize()
    assert float(mv.item()) == oracle.maxvio(down(counts))
