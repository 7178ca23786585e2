"""GPU parity of moe_route (gate + scoring + selection + weights) with the oracle.

Compared element by element on seeded inputs under the acceptance rule of
tests/parity.py; all calls go through the C ABI."""
import math

import numpy as np
import pytest
import torch

import oracle
import token_dispatch_amd as tda
import workloads as wl
from tests.gpu_util import down, gpu_route, say, up
from tests.parity import check_dispatch, check_route, oracle_route

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    tda.lib()


def run_select_only(logits32, k, **kw):
    return tda.route(None, None, k, logits=up(logits32), **kw)


# ---- hand cases (tests/golden/hand_cases.json) --------------------------------

@pytest.mark.parametrize("name", ["A_softmax_renorm", "A_softmax_topk", "B_tie_rule",
                                  "C_grouped_biased", "F_dynamic_k"])
@pytest.mark.parametrize("mode", ["select_only", "gate_d1"])
def test_hand_cases(hand_cases, name, mode):
    c = hand_cases[name]
    l32 = np.array(c["logits"], np.float32)
    kw = dict(score=c["score"], renormalize=c.get("renormalize", True),
              route_scale=c.get("route_scale", 1.0))
    if "n_groups" in c:
        kw.update(n_groups=c["n_groups"], topk_groups=c["topk_groups"],
                  group_score=c["group_score"])
    sb = np.array(c["select_bias"], np.float32) if "select_bias" in c else None
    kpt = np.array(c["k_per_token"], np.int32) if "k_per_token" in c else None
    say("hand case", name, mode)
    if mode == "select_only":
        ids, w = run_select_only(l32, c["k"], select_bias=up(sb), k_per_token=up(kpt), **kw)
    else:  # d = 1: x = 1, W[:, 0] = logits of each token (one token per call)
        rows = []
        for t in range(l32.shape[0]):
            x = np.ones((1, 1), np.float32)
            W = l32[t][:, None].copy()
            rows.append(tda.route(up(x), up(W), c["k"], select_bias=up(sb),
                                  k_per_token=None if kpt is None else up(kpt[t:t + 1]),
                                  **kw))
        ids = torch.cat([r[0] for r in rows])
        w = torch.cat([r[1] for r in rows])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(down(ids), np.array(c["ids"]))
    np.testing.assert_allclose(down(w), np.array(c["weights"]), atol=2e-6, rtol=0)


def test_hand_case_d_sqrt_softplus(hand_cases):
    c = hand_cases["D_sqrt_softplus"]
    l32 = np.array([[math.log(math.expm1(s)) for s in c["softplus_values"]]], np.float32)
    for k in (2, 3):
        ids, w = run_select_only(l32, k, score="sqrt_softplus")
        np.testing.assert_array_equal(down(ids), c["k%d" % k]["ids"])
        np.testing.assert_allclose(down(w), c["k%d" % k]["weights"], atol=2e-6)


# ---- gate exactness on integer-valued inputs ------------------------------------

GATE_SHAPES = [(1, 1, 1), (5, 7, 3), (63, 64, 8), (65, 200, 65), (200, 1000, 128),
               (33, 136, 256), (70, 96, 384), (20, 64, 512), (9, 48, 1024), (300, 2048, 8)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T,d,E", GATE_SHAPES)
def test_gate_logits_exact_on_integers(dtype, T, d, E):
    rng = np.random.default_rng([T, d, E])
    x = rng.integers(-4, 5, size=(T, d)).astype(np.float32)
    W = rng.integers(-4, 5, size=(E, d)).astype(np.float32)
    lb = rng.integers(-3, 4, size=E).astype(np.float32)
    exp = (x.astype(np.int64) @ W.astype(np.int64).T + lb.astype(np.int64)).astype(np.float32)
    if dtype == "bf16":
        x, W = wl.f32_to_bf16_bits(x), wl.f32_to_bf16_bits(W)
    say("gate integer", dtype, T, d, E)
    _, _, logits = tda.route(up(x), up(W), 1, logit_bias=up(lb), return_logits=True)
    np.testing.assert_array_equal(down(logits), exp)


# ---- the routing workloads at reduced T (full d and E) ----------------------------

REDUCED = {"mixtral": 256, "qwen3_dynk": 700, "dsv3_grouped": 300, "dsv4": 260,
           "gptoss_skew": 600, "dsv4_bias": 260, "olmoe": 700, "dsv3_groupmax": 300,
           "grouped_quota": 300}


def route_case(w, inp):
    ids, wts, logits = gpu_route(w, inp)
    torch.cuda.synchronize()
    l64 = oracle.gate(inp["x"], inp["W"], inp["logit_bias"])
    # gate: fp32 accumulation of exact products, bounded by d * 2^-23 * sum|x w|
    xa = np.abs(wl.bf16_bits_to_f32(inp["x"]) if inp["x"].dtype == np.uint16 else inp["x"])
    Wa = np.abs(wl.bf16_bits_to_f32(inp["W"]) if inp["W"].dtype == np.uint16 else inp["W"])
    bound = w.d * 2.0 ** -23 * (xa.astype(np.float64) @ Wa.T.astype(np.float64)) + 1e-6
    assert np.all(np.abs(down(logits) - l64) <= bound)
    ref = oracle_route(oracle, l64, w.k, score=w.score, select_bias=inp["select_bias"],
                       k_per_token=inp["k_per_token"], n_groups=w.n_groups,
                       topk_groups=w.topk_groups,
                       group_score=w.group_score if w.n_groups > 1 else None,
                       renormalize=w.renormalize, route_scale=w.route_scale,
                       k_per_group=w.k_per_group)
    stats = check_route(down(ids), down(wts), ref, oracle, score=w.score,
                        renormalize=w.renormalize, route_scale=w.route_scale,
                        k_per_token=inp["k_per_token"], n_groups=w.n_groups,
                        topk_groups=w.topk_groups, k_per_group=w.k_per_group, where=w.name)
    return ids, stats


@pytest.mark.parametrize("name", list(REDUCED))
def test_workload_reduced(name):
    w = wl.WORKLOADS[name]
    inp = wl.make_inputs(w, T=REDUCED[name])
    say("workload", name, "T", REDUCED[name])
    ids, stats = route_case(w, inp)
    print(name, stats)
    d = tda.dispatch(ids, w.E)
    check_dispatch(d, oracle.dispatch(down(ids), w.E))


# ---- random small shapes --------------------------------------------------------

def random_case(seed):
    rng = np.random.default_rng(seed)
    E = int(rng.choice([1, 2, 3, 8, 31, 60, 64, 65, 96, 128, 200, 256, 320, 384, 512, 1024]))
    divisors = [g for g in range(1, min(E, 64) + 1) if E % g == 0]
    G = int(rng.choice(divisors)) if rng.random() < 0.5 else 1
    TG = int(rng.integers(1, G + 1))
    gs = E // G
    kmax = min(32, TG * gs)
    k = int(rng.integers(1, kmax + 1))
    score = str(rng.choice(list(tda.SCORES)))
    bias = rng.random() < 0.5
    rule = str(rng.choice(["max", "top2_sum"])) if gs >= 2 else "max"
    T = int(rng.choice([1, 2, 63, 64, 65, 130, 257]))
    d = int(rng.choice([1, 7, 16, 64, 136, 200]))
    dtype = str(rng.choice(["f32", "bf16"]))
    dyn = rng.random() < 0.3
    return dict(E=E, G=G, TG=TG, k=k, score=score, bias=bias, rule=rule, T=T, d=d,
                dtype=dtype, dyn=dyn, renorm=bool(rng.random() < 0.8),
                scale=float(rng.choice([1.0, 2.5])))


@pytest.mark.parametrize("seed", range(40))
def test_random_shapes(seed):
    c = random_case(seed)
    rng = np.random.default_rng(1000 + seed)
    x = rng.standard_normal((c["T"], c["d"])).astype(np.float32)
    W = (rng.standard_normal((c["E"], c["d"])) / np.sqrt(c["d"])).astype(np.float32) * 2
    if c["dtype"] == "bf16":
        x, W = wl.f32_to_bf16_bits(x), wl.f32_to_bf16_bits(W)
    sb = (0.1 * rng.standard_normal(c["E"])).astype(np.float32) if c["bias"] else None
    kpt = rng.integers(1, c["k"] + 1, size=c["T"]).astype(np.int32) if c["dyn"] else None
    say("random shape", seed, c)
    kw = dict(score=c["score"], n_groups=c["G"], topk_groups=c["TG"], group_score=c["rule"],
              renormalize=c["renorm"], route_scale=c["scale"])
    ids, wts, logits = tda.route(up(x), up(W), c["k"], select_bias=up(sb), k_per_token=up(kpt),
                                 return_logits=True, **kw)
    torch.cuda.synchronize()
    l64 = oracle.gate(x, W)
    ref = oracle_route(oracle, l64, c["k"], select_bias=sb, k_per_token=kpt, **kw)
    check_route(down(ids), down(wts), ref, oracle, score=c["score"], renormalize=c["renorm"],
                route_scale=c["scale"], k_per_token=kpt, n_groups=c["G"], topk_groups=c["TG"],
                where=str(c))
    check_dispatch(tda.dispatch(ids, c["E"]), oracle.dispatch(down(ids), c["E"]))


def test_select_only_matches_gate_path():
    w = wl.WORKLOADS["dsv3_grouped"]
    inp = wl.make_inputs(w, T=130)
    ids, wts, logits = gpu_route(w, inp)
    ids2, wts2 = tda.route(None, None, w.k, logits=logits, score=w.score,
                           select_bias=up(inp["select_bias"]), n_groups=w.n_groups,
                           topk_groups=w.topk_groups, group_score=w.group_score,
                           route_scale=w.route_scale)
    assert torch.equal(ids, ids2) and torch.equal(wts, wts2)


def test_bad_k_per_token_rows_and_dev_err():
    rng = np.random.default_rng(5)
    l = rng.standard_normal((6, 16)).astype(np.float32)
    kpt = np.array([1, 0, 4, 5, -2, 2], np.int32)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    ids, w = run_select_only(l, 4, k_per_token=up(kpt), dev_err=err)
    assert int(err.item()) == 3  # 0, 5 and -2 lie outside [1, 4]
    ids, w = down(ids), down(w)
    for t in (1, 3, 4):
        assert np.all(ids[t] == -1) and np.all(w[t] == 0)
    ref = oracle.route_logits(l.astype(np.float64), 4, k_per_token=kpt)
    np.testing.assert_array_equal(ids, ref["ids"])


def test_T0_and_determinism():
    w = wl.WORKLOADS["qwen3_dynk"]
    inp = wl.make_inputs(w, T=0)
    ids, wts = gpu_route(w, inp, return_logits=False)
    assert ids.shape == (0, w.k)
    inp = wl.make_inputs(w, T=1000)
    a = gpu_route(w, inp)
    b = gpu_route(w, inp)
    for u, v in zip(a, b):
        assert torch.equal(u, v)


# ---- full sizes, sampled tokens ------------------------------------------------------

@pytest.mark.parametrize("name", ["mixtral", "qwen3_dynk", "dsv3_grouped", "dsv4", "gptoss_skew",
                                  "dsv4_bias", "olmoe", "dsv3_groupmax", "grouped_quota"])
def test_workload_full_size_sampled(name):
    w = wl.WORKLOADS[name]
    inp = wl.make_inputs(w)
    say("full size", name, "T", w.T)
    ids, wts = gpu_route(w, inp, return_logits=False)
    torch.cuda.synchronize()
    gids, gw = down(ids), down(wts)
    rng = np.random.default_rng(99)
    n = min(w.T, 160)
    sample = np.unique(np.concatenate([rng.choice(w.T, n, replace=False),
                                       [0, w.T - 1, min(63, w.T - 1)]]))
    l64 = oracle.gate(wl.rows(inp["x"], sample), inp["W"], inp["logit_bias"])
    kpt = None if inp["k_per_token"] is None else inp["k_per_token"][sample]
    ref = oracle_route(oracle, l64, w.k, score=w.score, select_bias=inp["select_bias"],
                       k_per_token=kpt, n_groups=w.n_groups, topk_groups=w.topk_groups,
                       group_score=w.group_score if w.n_groups > 1 else None,
                       renormalize=w.renormalize, route_scale=w.route_scale,
                       k_per_group=w.k_per_group)
    stats = check_route(gids[sample], gw[sample], ref, oracle, score=w.score,
                        renormalize=w.renormalize, route_scale=w.route_scale, k_per_token=kpt,
                        n_groups=w.n_groups, topk_groups=w.topk_groups,
                        k_per_group=w.k_per_group, where=name)
    print(name, "sampled", stats)
    # properties at every token: row structure and weight sums
    kt = np.full(w.T, w.k) if inp["k_per_token"] is None else inp["k_per_token"]
    valid = gids >= 0
    assert np.all(valid.sum(axis=1) == kt)
    assert np.all((gids < w.E))
    if w.renormalize or w.score == "softmax_topk":
        np.testing.assert_allclose(gw.sum(axis=1), w.route_scale, atol=1e-5)
    srt = np.sort(np.where(valid, gids, -1 - np.arange(w.k)[None, :]), axis=1)
    assert np.all(srt[:, 1:] != srt[:, :-1])  # distinct experts per token
    d = tda.dispatch(ids, w.E)
    check_dispatch(d, oracle.dispatch(gids, w.E))


@pytest.mark.parametrize("splits", ["1", "2", "4", "8"])
def test_gate_k_split_matches_oracle(splits, monkeypatch):
    """Every K split of the gate (partial sums added in order by the select
    kernel) gives the oracle's routes; integer inputs stay bit-exact."""
    monkeypatch.setenv("MOE_GATE_SPLITS", splits)
    monkeypatch.setenv("MOE_GATE_TILE", "64x128")
    w = wl.WORKLOADS["qwen3_dynk"]
    inp = wl.make_inputs(w, T=520)
    say("gate split", splits)
    ids, stats = route_case(w, inp)
    rng = np.random.default_rng(int(splits))
    x = rng.integers(-4, 5, size=(130, 2048)).astype(np.float32)
    Wi = rng.integers(-4, 5, size=(128, 2048)).astype(np.float32)
    exp = (x.astype(np.int64) @ Wi.astype(np.int64).T).astype(np.float32)
    _, _, logits = tda.route(up(wl.f32_to_bf16_bits(x)), up(wl.f32_to_bf16_bits(Wi)), 4,
                             return_logits=True)
    np.testing.assert_array_equal(down(logits), exp)


@pytest.mark.parametrize("rb", ["128", "256", "512"])
@pytest.mark.parametrize("tile,d", [("32x64", 2880), ("64x128", 1000), ("128x128", 2056),
                                    ("32x256", 7168)])
def test_gate_stage_lengths_exact(rb, tile, d, monkeypatch):
    """Every stage length of the pipelined gate, on rows that end inside a
    stage (d * 2 bytes not a multiple of the stage): integer bf16 inputs make
    the fp32 result exact, so logits must equal the integer product."""
    monkeypatch.setenv("MOE_GATE_RB", rb)
    monkeypatch.setenv("MOE_GATE_TILE", tile)
    rng = np.random.default_rng([int(rb), d])
    T, E = 300, 136
    x = rng.integers(-3, 4, size=(T, d)).astype(np.float32)
    Wi = rng.integers(-3, 4, size=(E, d)).astype(np.float32)
    exp = (x.astype(np.int64) @ Wi.astype(np.int64).T).astype(np.float32)
    say("gate stage", rb, tile, d)
    _, _, logits = tda.route(up(wl.f32_to_bf16_bits(x)), up(wl.f32_to_bf16_bits(Wi)), 4,
                             return_logits=True)
    np.testing.assert_array_equal(down(logits), exp)


@pytest.mark.parametrize("tile,rb,ns", [
    ("256x256w8", "128", "2"), ("256x192w8", "128", "2"), ("128x384w8", "128", "2"),
    ("256x128w8", "128", "3"), ("128x256w8", "128", "3"), ("128x192w8", "128", "3"),
    ("128x128w8", "128", "4"), ("32x64w8", "256", "3"), ("32x64w8", "512", "2"),
    ("64x64w8", "128", "4"), ("64x64w8", "256", "3"), ("32x128w8", "256", "3"),
    ("32x128w8", "512", "2"), ("32x128w8", "128", "3"), ("128x192w8", "256", "2"),
    # 64-byte stages, deep rings; some split their load blocks unevenly
    ("128x192w8", "64", "5"), ("128x192w8", "64", "8"), ("256x192w8", "64", "4"),
    ("128x384w8", "64", "5"), ("256x256w8", "64", "3"), ("256x128w8", "64", "6"),
    ("64x64w8", "64", "7"), ("128x128w8", "64", "2"),
    # split rings: x three stages deep, W two (the tiles whose combined ring
    # fits only two deep)
    ("256x192w8", "128", "3/2"), ("128x384w8", "128", "3/2")])
@pytest.mark.parametrize("splits", ["1", "2"])
def test_gate_eight_wave_tiles_exact(tile, rb, ns, splits, monkeypatch):
    """Eight-wavefront tiles (4 x 2 or 2 x 4 waves) at each stage length and
    ring depth they take: ragged T, E and d, integer bf16 inputs, logits
    equal to the integer product."""
    monkeypatch.setenv("MOE_GATE_TILE", tile)
    monkeypatch.setenv("MOE_GATE_SPLITS", splits)
    monkeypatch.setenv("MOE_GATE_RB", rb)
    if ns == "3/2":
        monkeypatch.setenv("MOE_GATE_NSW", "2")
    else:
        monkeypatch.setenv("MOE_GATE_NS", ns)
        monkeypatch.setenv("MOE_GATE_NSW", "0")
    rng = np.random.default_rng([len(tile), int(splits), int(rb), len(ns)])
    T, E, d = 777, 420, 1480
    x = rng.integers(-3, 4, size=(T, d)).astype(np.float32)
    Wi = rng.integers(-3, 4, size=(E, d)).astype(np.float32)
    exp = (x.astype(np.int64) @ Wi.astype(np.int64).T).astype(np.float32)
    say("gate 8-wave", tile, rb, ns, splits)
    _, _, logits = tda.route(up(wl.f32_to_bf16_bits(x)), up(wl.f32_to_bf16_bits(Wi)), 4,
                             return_logits=True)
    np.testing.assert_array_equal(down(logits), exp)


def test_per_request_k_matches_per_token_k():
    """route() and route_dispatch() with a k per request equal the calls with
    the expanded per-token k, bit for bit (Qwen3-like requests of 256)."""
    w = wl.WORKLOADS["qwen3_dynk"]
    inp = wl.make_inputs(w, T=1024)
    kt = inp["k_per_token"]
    lens = [256] * 4
    say("per-request k")
    a = tda.route(up(inp["x"]), up(inp["W"]), w.k, k_per_token=up(kt))
    b = tda.route(up(inp["x"]), up(inp["W"]), w.k, k_per_request=kt[::256].copy(),
                  request_lens=lens)
    c = tda.route_dispatch(up(inp["x"]), up(inp["W"]), w.k, k_per_request=kt[::256].copy(),
                           request_lens=lens)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    assert torch.equal(a[0], c[0]) and torch.equal(a[1], c[1])
