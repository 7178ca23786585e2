"""moe_route_dispatch equals moe_route followed by moe_dispatch, bit for bit,
on the shapes where the selection kernel writes the dispatch histograms
(Qwen3-like: 16-token tiles of 256 routes) and on those where it does not;
the fused results also match the oracle."""
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


def both(x, W, k, E, **kw):
    """(fused outputs, separate-call outputs, fused dev_err, separate dev_err)."""
    err1 = torch.zeros(1, dtype=torch.int32, device=DEV)
    err2 = torch.zeros(1, dtype=torch.int32, device=DEV)
    fused = tda.route_dispatch(x, W, k, dev_err=err1, **kw)
    ids, w = tda.route(x, W, k, dev_err=err2, **kw)
    sep = (ids, w) + tuple(tda.dispatch(ids, E))
    torch.cuda.synchronize()
    return fused, sep, int(err1.item()), int(err2.item())


def assert_same(fused, sep):
    """Bit-equal outputs; perm only over its defined prefix (offsets[E])."""
    n = int(fused[3][-1].item())
    assert int(sep[3][-1].item()) == n
    for name, a, b in zip(("ids", "weights", "counts", "offsets", "perm", "inv"), fused, sep):
        if name == "perm":
            a, b = a[:n], b[:n]
        assert torch.equal(a, b), name


@pytest.mark.parametrize("name,T,lpt", [("qwen3_dynk", None, None), ("qwen3_dynk", 4091, None),
                                        ("qwen3_dynk", 33, None), ("qwen3_dynk", None, "64"),
                                        ("qwen3_dynk", 4091, "64"), ("qwen3_dynk", 4091, "16"),
                                        ("mixtral", None, None), ("gptoss_skew", 3000, None),
                                        ("dsv3_grouped", 700, None), ("dsv4_bias", 500, None),
                                        ("olmoe", 1000, None), ("dsv3_groupmax", 700, None),
                                        ("grouped_quota", 700, None)])
def test_route_dispatch_matches_separate_calls_and_oracle(name, T, lpt, monkeypatch):
    """The fused call (selection-written dispatch histograms where the shape
    allows) against separate moe_route + moe_dispatch calls and the oracle;
    lpt: a forced selection segment width (16-wave workgroups at 64)."""
    if lpt:
        monkeypatch.setenv("MOE_SELECT_LPT", lpt)
    w = wl.WORKLOADS[name]
    inp = wl.make_inputs(w, T=T)
    say("route_dispatch", name, inp["x"].shape[0], lpt)
    kw = route_kwargs(w)
    if kw["group_score"] is None:
        kw.pop("group_score")
    kw.update(logit_bias=up(inp["logit_bias"]), select_bias=up(inp["select_bias"]),
              k_per_token=up(inp["k_per_token"]))
    fused, sep, e1, e2 = both(up(inp["x"]), up(inp["W"]), w.k, w.E, **kw)
    assert_same(fused, sep)
    assert e1 == e2 == 0
    l64 = oracle.gate(inp["x"], inp["W"], inp["logit_bias"])
    ref = oracle_route(oracle, l64, w.k, score=w.score, select_bias=inp["select_bias"],
                       k_per_token=inp["k_per_token"], n_groups=w.n_groups,
                       topk_groups=w.topk_groups,
                       group_score=w.group_score if w.n_groups > 1 else None,
                       renormalize=w.renormalize, route_scale=w.route_scale,
                       k_per_group=w.k_per_group)
    check_route(down(fused[0]), down(fused[1]), ref, oracle, score=w.score,
                renormalize=w.renormalize, route_scale=w.route_scale,
                k_per_token=inp["k_per_token"], n_groups=w.n_groups, topk_groups=w.topk_groups,
                k_per_group=w.k_per_group, where=name)
    check_dispatch(tuple(fused[2:]), oracle.dispatch(down(fused[0]), w.E))


@pytest.mark.parametrize("name,T", [("qwen3_dynk", 1000), ("mixtral", None),
                                    ("dsv3_grouped", 2000), ("gptoss_skew", 3000)])
def test_prepared_call_matches_route_dispatch(name, T):
    """A prepared moe_route_dispatch call (arguments marshalled once) equals
    route_dispatch() bit for bit on two different inputs in a row, and on a
    side stream; a wrong x is rejected on the host."""
    w = wl.WORKLOADS[name]
    inp = wl.make_inputs(w, T=T)
    kw = route_kwargs(w)
    if kw["group_score"] is None:
        kw.pop("group_score")
    kw.update(logit_bias=up(inp["logit_bias"]), select_bias=up(inp["select_bias"]),
              k_per_token=up(inp["k_per_token"]))
    x, W = up(inp["x"]), up(inp["W"])
    x2 = torch.roll(x, 7, 0).contiguous()
    mv = torch.zeros(1, dtype=torch.float64, device=DEV)
    say("prepared call", name, T)
    call = tda.prepare_route_dispatch(x, W, w.k, maxvio=mv, **kw)
    for xi in (x, x2):
        got = [t.clone() for t in call(xi) if t is not None]
        mv_got = mv.clone()
        mv_ref = torch.zeros(1, dtype=torch.float64, device=DEV)
        ref = [t for t in tda.route_dispatch(xi, W, w.k, maxvio=mv_ref, **kw) if t is not None]
        torch.cuda.synchronize()
        n = int(ref[3][-1].item())
        for i, (a, b) in enumerate(zip(got, ref)):
            if i == 4:  # perm: the first offsets[E] entries are defined
                a, b = a[:n], b[:n]
            assert torch.equal(a, b), (name, i)
        assert torch.equal(mv_got, mv_ref)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        got = [t.clone() for t in call(x) if t is not None]
    torch.cuda.current_stream().wait_stream(s)
    ref = [t for t in tda.route_dispatch(x, W, w.k, **kw) if t is not None]
    torch.cuda.synchronize()
    assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1])
    with pytest.raises(ValueError):
        call(x[:-1].contiguous())


def test_route_dispatch_select_only_and_bad_k():
    rng = np.random.default_rng(5)
    T, E, K = 4096, 128, 16
    lg = up(rng.standard_normal((T, E)).astype(np.float32))
    kpt = rng.choice([4, 8, 16], size=T).astype(np.int32)
    kpt[[3, 100, 4095]] = [0, 17, -2]
    say("route_dispatch select-only")
    fused, sep, e1, e2 = both(None, None, K, E, logits=lg, k_per_token=up(kpt))
    assert_same(fused, sep)
    assert e1 == e2 == 3
    assert np.all(down(fused[0])[[3, 100, 4095]] == -1)
    check_dispatch(tuple(fused[2:]), oracle.dispatch(down(fused[0]), E))


def test_route_dispatch_empty():
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    W = up(wl.f32_to_bf16_bits(np.ones((8, 64), np.float32)))
    say("route_dispatch empty")
    ids, wts, counts, offsets, perm, inv = tda.route_dispatch(x, W, 2)
    torch.cuda.synchronize()
    assert ids.shape == (0, 2)
    assert np.all(down(counts) == 0) and np.all(down(offsets) == 0)



@pytest.mark.parametrize("T,E,tile,ns,score,bias_groups,dynk", [
    (2000, 128, "256x128w8", "3", "softmax_topk", False, False),   # 16 lanes x 8, monotone
    (2000, 128, "256x128w8", "3", "sigmoid", True, True),          # biased, grouped, per-token k
    (1777, 124, "128x128w8", "4", "softmax", False, True),         # ragged T and E, padded tile
    (16500, 128, "256x128w8", "3", "sqrt_softplus", True, False),  # 8 lanes x 16
    (16500, 128, "128x128w8", "4", "softmax", False, True),
    # k = 4 compiled into the 256-row tiles' selection, tokens asking 1-4
    (2000, 128, "256x128w8", "3", "softmax_topk", False, "k4"),
    (16500, 128, "256x128w8", "3", "softmax", False, "k4"),
])
def test_fused_gate_select_matches_separate_kernels(T, E, tile, ns, score, bias_groups, dynk,
                                                    monkeypatch):
    """The gate kernel with the selection in its epilogue (whole-row tiles, no
    K split) against the gate kernel followed by the select kernel on the
    same plan: ids, weights, logits and the dispatch bit for bit; and the
    oracle."""
    monkeypatch.setenv("MOE_GATE_TILE", tile)
    monkeypatch.setenv("MOE_GATE_SPLITS", "1")
    monkeypatch.setenv("MOE_GATE_RB", "128")
    monkeypatch.setenv("MOE_GATE_NS", ns)
    rng = np.random.default_rng([T, E])
    d, k = 1024, (8 if dynk is True else 4)
    x = rng.standard_normal((T, d)).astype(np.float32)
    Wf = (rng.standard_normal((E, d)) / np.sqrt(d)).astype(np.float32)
    xb, Wb = wl.f32_to_bf16_bits(x), wl.f32_to_bf16_bits(Wf)
    lb = (0.1 * rng.standard_normal(E)).astype(np.float32)
    sb = (0.01 * rng.standard_normal(E)).astype(np.float32) if bias_groups else None
    kpt = (rng.choice([2, 4, 8], size=T).astype(np.int32) if dynk is True else
           rng.integers(1, 5, size=T).astype(np.int32) if dynk == "k4" else None)
    rkw = dict(score=score, select_bias=sb, k_per_token=kpt,
               n_groups=4 if bias_groups else 1, topk_groups=2 if bias_groups else None,
               group_score="top2_sum" if bias_groups else None, renormalize=True,
               route_scale=2.5 if bias_groups else 1.0)
    kw = {key: (up(v) if isinstance(v, np.ndarray) else v) for key, v in rkw.items()
          if v is not None}
    kw["logit_bias"] = up(lb)
    say("fused gate+select", T, E, tile, score, bias_groups, dynk)
    outs = []
    for fused in (True, False):
        if fused:
            monkeypatch.delenv("MOE_NO_FUSED_SELECT", raising=False)
        else:
            monkeypatch.setenv("MOE_NO_FUSED_SELECT", "1")
        tda.profile_enable(True)
        lg = torch.empty((T, E), dtype=torch.float32, device=DEV)
        r = tda.route_dispatch(up(xb), up(Wb), k, logits=lg, **kw)
        ids2, w2 = tda.route(up(xb), up(Wb), k, **kw)
        torch.cuda.synchronize()
        prof = tda.profile_read()
        tda.profile_enable(False)
        staged = (prof["gate_select"][1], prof["select"][1])
        assert staged == ((2, 0) if fused else (0, 2)), staged
        assert torch.equal(r[0], ids2) and torch.equal(r[1], w2)
        outs.append(tuple(r) + (lg,))
    assert_same(outs[0][:6], outs[1][:6])
    assert torch.equal(outs[0][6], outs[1][6]), "logits"
    ref = oracle_route(oracle, oracle.gate(xb, Wb, lb), k, **rkw)
    check_route(down(outs[0][0]), down(outs[0][1]), ref, oracle, score=score, renormalize=True,
                route_scale=rkw["route_scale"], k_per_token=kpt, n_groups=rkw["n_groups"],
                topk_groups=rkw["topk_groups"], where="fused gate+select")
    check_dispatch(tuple(outs[0][2:6]), oracle.dispatch(down(outs[0][0]), E))


@pytest.mark.parametrize("T,E,k,score,bias_groups,dynk,dt", [
    (256, 8, 2, "softmax", False, False, "f32"),       # Mixtral-like
    (33, 128, 16, "softmax", False, True, "bf16"),     # a few Qwen3-like tokens, per-token k
    (100, 64, 8, "sigmoid", True, False, "bf16"),      # biased, grouped
    (511, 30, 4, "sqrt_softplus", False, False, "f32"),  # E not a multiple of 4
    (256, 128, 8, "softmax_topk", False, True, "bf16"),  # exactly 2048 routes
    (1, 16, 3, "softmax", False, False, "f32"),
    (2049, 16, 1, "softmax", False, False, "f32"),     # 2049 routes: the regular path
])
def test_small_batch_route_dispatch(T, E, k, score, bias_groups, dynk, dt):
    """Small batches (T * k <= 2048, E <= 128): selection and the whole
    dispatch in one workgroup, against separate moe_route + moe_dispatch calls
    (bit for bit) and the oracle; invalid per-token k values count as
    errors."""
    rng = np.random.default_rng([T, E, k])
    d = 256
    x = rng.standard_normal((T, d)).astype(np.float32)
    Wf = (rng.standard_normal((E, d)) / np.sqrt(d)).astype(np.float32)
    if dt == "bf16":
        x, Wf = wl.f32_to_bf16_bits(x), wl.f32_to_bf16_bits(Wf)
    sb = (0.01 * rng.standard_normal(E)).astype(np.float32) if bias_groups else None
    kpt = rng.integers(1, k + 1, size=T).astype(np.int32) if dynk else None
    nbad = 0
    if dynk and T > 3:
        kpt[[1, 2]] = [0, k + 1]
        nbad = 2
    rkw = dict(score=score, select_bias=sb, k_per_token=kpt,
               n_groups=4 if bias_groups else 1, topk_groups=2 if bias_groups else None,
               group_score="top2_sum" if bias_groups else None, renormalize=True,
               route_scale=2.5 if bias_groups else 1.0)
    kw = {key: (up(v) if isinstance(v, np.ndarray) else v) for key, v in rkw.items()
          if v is not None}
    say("small route_dispatch", T, E, k, score, bias_groups, dynk, dt)
    tda.profile_enable(True)
    fused, sep, e1, e2 = both(up(x), up(Wf), k, E, **kw)
    prof = tda.profile_read()
    tda.profile_enable(False)
    small = T * k <= 2048
    assert prof["select_dispatch"][1] == (1 if small else 0), prof["select_dispatch"]
    assert_same(fused, sep)
    assert e1 == e2 == nbad
    ref = oracle_route(oracle, oracle.gate(x, Wf), k, **rkw)
    check_route(down(fused[0]), down(fused[1]), ref, oracle, score=score, renormalize=True,
                route_scale=rkw["route_scale"], k_per_token=kpt, n_groups=rkw["n_groups"],
                topk_groups=rkw["topk_groups"], where="small route_dispatch")
    check_dispatch(tuple(fused[2:6]), oracle.dispatch(down(fused[0]), E))


@pytest.mark.parametrize("seed", range(16))
def test_quota_random_shapes_every_path(seed):
    """Grouped top-k with a per-group quota (k_per_group) over random shapes:
    moe_route_dispatch (small, selection-histogram or separate path by shape)
    equals moe_route + moe_dispatch bit for bit, and both match the oracle."""
    rng = np.random.default_rng(500 + seed)
    E = int(rng.choice([8, 16, 32, 64, 96, 128, 256, 384]))
    G = int(rng.choice([g for g in (1, 2, 4, 8, 16) if E % g == 0]))
    gs = E // G
    kpg = int(rng.integers(1, min(gs, 4) + 2))
    k = int(rng.integers(1, min(32, G * min(kpg, gs)) + 1))
    T = int(rng.choice([5, 64, 129, 700, 2100]))
    d = int(rng.choice([64, 200, 256]))
    score = str(rng.choice(["softmax", "sigmoid", "sqrt_softplus"]))
    x = wl.f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    Wf = wl.f32_to_bf16_bits((rng.standard_normal((E, d)) / np.sqrt(d)).astype(np.float32))
    sb = (0.1 * rng.standard_normal(E)).astype(np.float32) if rng.random() < 0.5 else None
    kpt = rng.integers(1, k + 1, size=T).astype(np.int32) if rng.random() < 0.3 else None
    rkw = dict(score=score, select_bias=sb, k_per_token=kpt, n_groups=G, renormalize=True,
               route_scale=1.0, k_per_group=kpg)
    kw = {key: (up(v) if isinstance(v, np.ndarray) else v) for key, v in rkw.items()
          if v is not None}
    say("quota route_dispatch", seed, dict(E=E, G=G, kpg=kpg, k=k, T=T, d=d, score=score))
    fused, sep, e1, e2 = both(up(x), up(Wf), k, E, **kw)
    assert_same(fused, sep)
    assert e1 == e2 == 0
    ref = oracle_route(oracle, oracle.gate(x, Wf), k, **rkw)
    check_route(down(fused[0]), down(fused[1]), ref, oracle, score=score, renormalize=True,
                route_scale=1.0, k_per_token=kpt, n_groups=G, k_per_group=kpg,
                where=f"quota seed {seed}")
    check_dispatch(tuple(fused[2:6]), oracle.dispatch(down(fused[0]), E))


@pytest.mark.parametrize("path,T,d,E,k,G,kpg", [("fused", 32768, 512, 128, 4, 8, 1),
                                                 ("select_hist", 700, 2048, 128, 16, 16, 2),
                                                 ("select_super", 700, 2048, 128, 16, 16, 2)])
def test_quota_fused_paths(path, T, d, E, k, G, kpg, monkeypatch):
    """The gate kernel with the selection in its epilogue (whole-row 128 x 128
    tiles), and the select kernel writing the dispatch's tile histograms (read
    in full by the placement, or with super-tile sums), under a per-group
    quota: equal to separate moe_route + moe_dispatch calls bit for bit, and
    to the oracle on sampled tokens."""
    if path == "select_hist":
        monkeypatch.setenv("MOE_DISPATCH_NO_SUPER", "1")
    plan = tda.route_dispatch_plan(T, d, E, k, 1, score="sigmoid", n_groups=G, topk_groups=G,
                                   k_per_group=kpg)
    assert plan["path"] == path, plan
    rng = np.random.default_rng(77)
    x = wl.f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    Wf = wl.f32_to_bf16_bits((rng.standard_normal((E, d)) / np.sqrt(d)).astype(np.float32))
    sb = (0.1 * rng.standard_normal(E)).astype(np.float32)
    say("quota", path, T, d, E, k, G, kpg)
    fused, sep, e1, e2 = both(up(x), up(Wf), k, E, score="sigmoid", select_bias=up(sb),
                              n_groups=G, k_per_group=kpg)
    assert_same(fused, sep)
    assert e1 == e2 == 0
    pick = np.sort(rng.choice(T, size=min(T, 300), replace=False))
    ref = oracle_route(oracle, oracle.gate(wl.rows(x, pick), Wf), k, score="sigmoid",
                       select_bias=sb, n_groups=G, k_per_group=kpg)
    check_route(down(fused[0])[pick], down(fused[1])[pick], ref, oracle, score="sigmoid",
                n_groups=G, k_per_group=kpg, where=f"quota {path}")


@pytest.mark.parametrize("T,d,E,k,dyn", [
    (5000, 256, 384, 6, False),    # 16-token tiles of 96 routes (not whole chunks), 313 tiles
    (777, 128, 1000, 5, True),     # one-token wavefronts, 16-wave tiles of 80 routes, 10-bit ids
    (3001, 64, 100, 7, True),      # E not a multiple of 8, ragged last tile
    (20000, 64, 64, 32, False),    # 2048-route tiles (two chunks per wave)
    (1, 64, 256, 8, False),        # a single tile
    (16384, 512, 384, 6, True),    # DeepSeek-V4-like tile shape with empty slots
    (3000, 64, 1024, 8, True),     # the largest E: 10-bit ids, one thread per expert
    (70000, 64, 1024, 2, False),   # 4375 tiles of 32 routes: 66 super rows, S = 67
    (5000, 128, 512, 16, True),    # 16-wave tiles of 256 routes at E = 512
])
def test_super_tile_dispatch(T, d, E, k, dyn, monkeypatch):
    """The select-written tile histograms plus super-tile sums (zeroed by the
    gate kernel) against the same call with that path switched off and
    against the oracle's dispatch of the GPU's ids, bit for bit."""
    rng = np.random.default_rng([T, E, k])
    x = wl.f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    W = wl.f32_to_bf16_bits((rng.standard_normal((E, d)) / np.sqrt(d)).astype(np.float32))
    kpt = rng.integers(1, k + 1, size=T).astype(np.int32) if dyn else None
    plan = tda.route_dispatch_plan(T, d, E, k, 1, score="sigmoid")
    say("super-tile dispatch", T, d, E, k, dyn, plan["path"], plan["hist_tokens"])
    assert plan["path"] == "select_super", plan
    kw = dict(score="sigmoid", k_per_token=up(kpt))
    outs = []
    for off in (False, True):
        if off:
            monkeypatch.setenv("MOE_DISPATCH_NO_SUPER", "1")
        mv = torch.zeros(1, dtype=torch.float64, device=DEV)
        r = tda.route_dispatch(up(x), up(W), k, maxvio=mv, **kw)
        torch.cuda.synchronize()
        outs.append((r, mv))
    monkeypatch.delenv("MOE_DISPATCH_NO_SUPER", raising=False)
    (a, mva), (b, mvb) = outs
    assert_same(a, b)
    assert torch.equal(mva, mvb)
    d_ref = oracle.dispatch(down(a[0]), E)
    check_dispatch(tuple(a[2:]), d_ref)
    assert float(mva.item()) == oracle.maxvio(d_ref["counts"])


@pytest.mark.parametrize("waves", ["2", "4", "8"])
@pytest.mark.parametrize("name,T", [("qwen3_dynk", None), ("qwen3_dynk", 1001),
                                    ("dsv3_grouped", 3000), ("olmoe", 777),
                                    ("grouped_quota", 2049)])
def test_super_tile_select_workgroup_sizes(name, T, waves, monkeypatch):
    """Selection workgroups of 2, 4 or 8 waves (one dispatch tile each, of
    2, 4 or 8 wavefronts' tokens) on the super-tile path: the same ids and
    weights as the path without tile counting, and the oracle's dispatch of
    those ids, bit for bit."""
    w = wl.WORKLOADS[name]
    inp = wl.make_inputs(w, T=T)
    kw = route_kwargs(w)
    if kw["group_score"] is None:
        kw.pop("group_score")
    kw.update(logit_bias=up(inp["logit_bias"]), select_bias=up(inp["select_bias"]),
              k_per_token=up(inp["k_per_token"]))
    x, W = up(inp["x"]), up(inp["W"])
    monkeypatch.setenv("MOE_SELECT_SUPER_WAVES", waves)
    kw2 = {key: v for key, v in route_kwargs(w).items() if v is not None}
    plan = tda.route_dispatch_plan(w.T if T is None else T, w.d, w.E, w.k, 1, **kw2)
    say("super select waves", name, T, waves, plan["path"], plan["hist_tokens"])
    assert plan["path"] == "select_super", plan
    mv = torch.zeros(1, dtype=torch.float64, device=DEV)
    a = tda.route_dispatch(x, W, w.k, maxvio=mv, **kw)
    monkeypatch.delenv("MOE_SELECT_SUPER_WAVES")
    monkeypatch.setenv("MOE_DISPATCH_UNFUSED", "1")
    monkeypatch.setenv("MOE_DISPATCH_NO_SUPER", "1")
    ids, wts = tda.route(x, W, w.k, **kw)[:2]
    torch.cuda.synchronize()
    assert torch.equal(a[0], ids) and torch.equal(a[1], wts)
    d_ref = oracle.dispatch(down(a[0]), w.E)
    check_dispatch(tuple(a[2:]), d_ref)
    assert float(mv.item()) == oracle.maxvio(d_ref["counts"])


@pytest.mark.parametrize("group", ["1", "2", "4", "8"])
@pytest.mark.parametrize("name,T", [("dsv4", 9001), ("switch_top1", 16384), ("qwen3_dynk", 3001),
                                    ("dsv4_hash", 7777)])
def test_placement_tile_groups(name, T, group, monkeypatch):
    """Several dispatch tiles per placement workgroup (MOE_PLACE_GROUP; the
    super-tile size is rounded to a multiple of the group, a ragged last
    group included): the dispatch equals the oracle's dispatch of the GPU's
    ids, bit for bit, and the ids and weights do not change."""
    w = wl.WORKLOADS[name]
    inp = wl.make_inputs(w, T=T)
    say("placement groups", name, T, group)
    mv = torch.zeros(1, dtype=torch.float64, device=DEV)
    outs = []
    for g in ("1", group):
        monkeypatch.setenv("MOE_PLACE_GROUP", g)
        if w.hash_vocab:
            r = tda.route_hash_dispatch(up(inp["token_ids"]), up(inp["tid2eid"]), w.E,
                                        x=up(inp["x"]), W=up(inp["W"]), score=w.score,
                                        renormalize=w.renormalize, route_scale=w.route_scale,
                                        maxvio=mv)
        else:
            kw = route_kwargs(w)
            if kw["group_score"] is None:
                kw.pop("group_score")
            kw.update(logit_bias=up(inp["logit_bias"]), select_bias=up(inp["select_bias"]),
                      k_per_token=up(inp["k_per_token"]))
            r = tda.route_dispatch(up(inp["x"]), up(inp["W"]), w.k, maxvio=mv, **kw)
        torch.cuda.synchronize()
        outs.append(r)
    monkeypatch.delenv("MOE_PLACE_GROUP")
    a, b = outs
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    d_ref = oracle.dispatch(down(b[0]), w.E)
    check_dispatch(tuple(b[2:]), d_ref)
    assert float(mv.item()) == oracle.maxvio(d_ref["counts"])


@pytest.mark.parametrize("name,T", [("qwen3_dynk", None), ("qwen3_dynk", 4091), ("olmoe", 1000)])
def test_all_counts_placement_after_the_gate(name, T, monkeypatch):
    """With the super-tile sums switched off the select kernel's tile
    histograms go to the placement that reads every tile's counts: equal to
    separate calls and to the super-tile path, bit for bit."""
    w = wl.WORKLOADS[name]
    inp = wl.make_inputs(w, T=T)
    kw = route_kwargs(w)
    if kw["group_score"] is None:
        kw.pop("group_score")
    kw.update(logit_bias=up(inp["logit_bias"]), select_bias=up(inp["select_bias"]),
              k_per_token=up(inp["k_per_token"]))
    say("all-counts placement", name, inp["x"].shape[0])
    sup = tda.route_dispatch(up(inp["x"]), up(inp["W"]), w.k, **kw)
    monkeypatch.setenv("MOE_DISPATCH_NO_SUPER", "1")
    plan = tda.route_dispatch_plan(inp["x"].shape[0], w.d, w.E, w.k, 1,
                                   **{k2: v for k2, v in route_kwargs(w).items() if v is not None})
    assert plan["path"] == "select_hist", plan
    fused, sep, e1, e2 = both(up(inp["x"]), up(inp["W"]), w.k, w.E, **kw)
    assert_same(fused, sep)
    assert_same(fused, tuple(sup))
