"""moe_route_dispatch_noalloc (the library's per-GPU scratch array in place of
a workspace) against moe_route_dispatch: the same outputs bit for bit --
ids, weights, counts, offsets, perm, inv, MaxVio, error count -- on two calls
in a row, the second with a smaller input (the array keeps the first call's
contents), on each path whose kernels use scratch (the gate's K-split
hand-off and the selection-written tile histograms, the fused gate + select
with its tile histograms, the three-kernel dispatch), and the oracle's
acceptance rule on the results.  Shapes needing more than the array holds
are rejected before anything is enqueued."""
import numpy as np
import pytest
import torch

import oracle
import token_dispatch_amd as tda
import workloads as wl
from tests.gpu_util import down, route_kwargs, say, up
from tests.parity import check_dispatch, check_route, oracle_route

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    tda.lib()


def outputs(T, k, E):
    i32 = torch.int32
    return dict(ids=torch.full((T, k), -9, dtype=i32, device=DEV),
                weights=torch.full((T, k), -9.0, dtype=torch.float32, device=DEV),
                counts=torch.full((E,), -9, dtype=i32, device=DEV),
                offsets=torch.full((E + 1,), -9, dtype=i32, device=DEV),
                perm=torch.full((T * k,), -9, dtype=i32, device=DEV),
                inv=torch.full((T * k,), -9, dtype=i32, device=DEV),
                maxvio=torch.full((1,), -9.0, dtype=torch.float64, device=DEV),
                dev_err=torch.zeros(1, dtype=i32, device=DEV))


def one_case(name, T):
    w = wl.WORKLOADS[name]
    inp = wl.make_inputs(w, T=T)
    kw = route_kwargs(w)
    if kw["group_score"] is None:
        kw.pop("group_score")
    kw.update(logit_bias=up(inp["logit_bias"]), select_bias=up(inp["select_bias"]),
              k_per_token=up(inp["k_per_token"]))
    x, W = up(inp["x"]), up(inp["W"])
    say("no-alloc", name, "T", T, "scratch",
        tda.route_dispatch_workspace_size(T, w.d, w.E, w.k, 1 if w.dtype == "bf16" else 0,
                                          **{key: v for key, v in route_kwargs(w).items()
                                             if v is not None}))
    a, b = outputs(T, w.k, w.E), outputs(T, w.k, w.E)
    tda.route_dispatch(x, W, w.k, **a, **kw)
    tda.route_dispatch_noalloc(x, W, w.k, **b, **kw)
    torch.cuda.synchronize()
    for key in a:
        t1, t2 = a[key], b[key]
        if key == "perm":
            n = int(a["offsets"][-1].item())
            t1, t2 = t1[:n], t2[:n]
        assert torch.equal(t1, t2), (name, T, key)
    l64 = oracle.gate(inp["x"], inp["W"], inp["logit_bias"], nthreads=8)
    ref = oracle_route(oracle, l64, w.k, score=w.score, select_bias=inp["select_bias"],
                       k_per_token=inp["k_per_token"], n_groups=w.n_groups,
                       topk_groups=w.topk_groups,
                       group_score=w.group_score if w.n_groups > 1 else None,
                       renormalize=w.renormalize, route_scale=w.route_scale,
                       k_per_group=w.k_per_group, nthreads=8)
    check_route(down(b["ids"]), down(b["weights"]), ref, oracle, score=w.score,
                renormalize=w.renormalize, route_scale=w.route_scale,
                k_per_token=inp["k_per_token"], n_groups=w.n_groups, topk_groups=w.topk_groups,
                k_per_group=w.k_per_group, where=f"noalloc {name}")
    d = oracle.dispatch(down(b["ids"]), w.E)
    check_dispatch((b["counts"], b["offsets"], b["perm"], b["inv"]), d)
    assert float(b["maxvio"].item()) == oracle.maxvio(d["counts"])


@pytest.mark.parametrize("name,T1,T2", [
    ("qwen3_dynk", 4096, 1000),      # 2 K-split partial arrays + selection-written histograms
    ("dsv3_grouped", 8192, 3000),    # 4 K-split partial arrays (33.5 MB) + dispatch
    ("gptoss_skew", 65536, 20000),   # fused gate + select with tile histograms
    ("dsv4", 16384, 5000),           # 2 K-split partial arrays (50 MB) + three-kernel dispatch
    ("mixtral", 256, 100),           # small batch: one-workgroup selection + dispatch
])
def test_noalloc_matches_route_dispatch_twice(name, T1, T2):
    one_case(name, T1)
    one_case(name, T2)


def test_noalloc_rejects_shapes_beyond_the_scratch():
    T, d, E, k = 65536, 7168, 1024, 8
    need = tda.route_dispatch_workspace_size(T, d, E, k)
    assert need > tda.NOALLOC_SCRATCH_BYTES
    x = torch.empty((T, d), dtype=torch.bfloat16, device=DEV)
    W = torch.empty((E, d), dtype=torch.bfloat16, device=DEV)
    o = outputs(T, k, E)
    with pytest.raises(tda.MoeError) as ei:
        tda.route_dispatch_noalloc(x, W, k, **o)
    assert ei.value.code == tda.MOE_EUNSUPPORTED and str(need) in str(ei.value)
