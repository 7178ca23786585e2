"""Oracle pinned by closed forms, invariants and library reductions.

Closed forms: sigmoid(0) = 1/2, sigmoid(ln 3) = 3/4, softplus(ln(e^a - 1)) = a,
softmax of equal logits = 1/E.  Invariants: selected experts lie in kept
groups; one group == no group limit; monotone scores pick the same experts;
softmax-then-renorm equals softmax over the selected logits; renormalised
weights sum to route_scale.  Gate and dispatch reduce to numpy matmul,
argsort(kind="stable"), bincount and cumsum."""
import math

import numpy as np
import pytest

import workloads


def rand_logits(seed, T, E):
    return np.random.default_rng(seed).standard_normal((T, E))


# ---- scores ------------------------------------------------------------------

def test_sigmoid_closed_forms(orc):
    l = np.array([[0.0, math.log(3.0)]])
    r = orc.route_logits(l, k=2, score="sigmoid", renormalize=False)
    np.testing.assert_array_equal(r["ids"], [[1, 0]])
    np.testing.assert_allclose(r["weights"], [[0.75, 0.5]], atol=1e-15)


@pytest.mark.parametrize("a", [0.25, 1.0, 4.0, 9.0])
def test_sqrt_softplus_closed_form(orc, a):
    l = np.array([[math.log(math.expm1(a)), -5.0]])
    r = orc.route_logits(l, k=1, score="sqrt_softplus", renormalize=False)
    assert r["ids"][0, 0] == 0
    assert r["weights"][0, 0] == pytest.approx(math.sqrt(a), abs=1e-13)


@pytest.mark.parametrize("E", [1, 3, 8, 128])
def test_softmax_of_equal_logits(orc, E):
    r = orc.route_logits(np.full((1, E), 0.7), k=1, score="softmax", renormalize=False)
    assert r["ids"][0, 0] == 0
    assert r["weights"][0, 0] == pytest.approx(1.0 / E, rel=1e-14)


# ---- selection invariants ----------------------------------------------------

@pytest.mark.parametrize("E,G,TG,k", [(256, 8, 4, 8), (64, 8, 2, 6), (384, 8, 4, 6),
                                      (24, 3, 1, 4)])
def test_selected_experts_lie_in_kept_groups(orc, E, G, TG, k):
    rng = np.random.default_rng([E, G])
    l = rng.standard_normal((200, E))
    b = (0.1 * rng.standard_normal(E)).astype(np.float32)
    r = orc.route_logits(l, k=k, score="sigmoid", select_bias=b, n_groups=G,
                         topk_groups=TG, group_score="top2_sum", route_scale=2.5)
    gs = E // G
    g = r["g"]
    for t in range(l.shape[0]):
        kept = np.lexsort((np.arange(G), -g[t]))[:TG]
        assert set(r["ids"][t] // gs) <= set(kept.tolist())
        # dropped groups are masked to -inf in the selection quantity
        dropped = sorted(set(range(G)) - set(kept.tolist()))
        for γ in dropped:
            assert np.all(np.isneginf(r["q"][t, γ * gs:(γ + 1) * gs]))
    np.testing.assert_allclose(r["weights"].sum(axis=1), 2.5, atol=1e-12)


def test_one_group_equals_no_group_limit(orc):
    l = rand_logits(1, 100, 64)
    b = (0.1 * np.random.default_rng(2).standard_normal(64)).astype(np.float32)
    a = orc.route_logits(l, k=6, score="sigmoid", select_bias=b)
    c = orc.route_logits(l, k=6, score="sigmoid", select_bias=b, n_groups=8, topk_groups=8,
                         group_score="top2_sum")
    np.testing.assert_array_equal(a["ids"], c["ids"])
    np.testing.assert_array_equal(a["weights"], c["weights"])


def test_monotone_scores_pick_the_same_experts(orc):
    l = rand_logits(3, 300, 128) * 3.0
    ids = [orc.route_logits(l, k=8, score=s)["ids"]
           for s in ("softmax", "sigmoid", "sqrt_softplus", "softmax_topk")]
    for other in ids[1:]:
        np.testing.assert_array_equal(ids[0], other)
    # and they are the k largest logits in descending order
    exp = np.argsort(-l, axis=1, kind="stable")[:, :8]
    np.testing.assert_array_equal(ids[0], exp)


def test_softmax_renorm_equals_softmax_over_selected(orc):
    l = rand_logits(4, 300, 128) * 2.0
    a = orc.route_logits(l, k=8, score="softmax", renormalize=True)
    b = orc.route_logits(l, k=8, score="softmax_topk", renormalize=False)
    np.testing.assert_array_equal(a["ids"], b["ids"])
    np.testing.assert_allclose(a["weights"], b["weights"], atol=1e-12)


def test_k_equals_E_returns_all_sorted(orc):
    l = rand_logits(5, 50, 16)
    r = orc.route_logits(l, k=16, score="sigmoid", renormalize=False)
    np.testing.assert_array_equal(r["ids"], np.argsort(-l, axis=1, kind="stable"))
    assert np.all(np.isinf(r["margin_k"]))


@pytest.mark.parametrize("score", ["softmax", "sigmoid", "sqrt_softplus", "softmax_topk"])
@pytest.mark.parametrize("scale", [1.0, 2.5])
def test_renormalised_weights_sum_to_route_scale(orc, score, scale):
    l = rand_logits(6, 100, 32)
    r = orc.route_logits(l, k=5, score=score, renormalize=True, route_scale=scale)
    np.testing.assert_allclose(r["weights"].sum(axis=1), scale, atol=1e-12)
    assert np.all(r["weights"] > 0)


def test_two_expert_softmax_weight_is_sigmoid_of_gap(orc):
    l = rand_logits(7, 100, 8)
    r = orc.route_logits(l, k=2, score="softmax")
    for t in range(100):
        a, b = r["ids"][t]
        assert r["weights"][t, 0] == pytest.approx(1 / (1 + math.exp(-(l[t, a] - l[t, b]))),
                                                   abs=1e-14)


def test_k1_renorm_weight_is_route_scale(orc):
    l = rand_logits(8, 20, 8)
    r = orc.route_logits(l, k=1, score="sigmoid", route_scale=2.5)
    np.testing.assert_allclose(r["weights"], 2.5, atol=1e-15)


def test_weights_use_unbiased_scores(orc):
    """A large bias can move the choice but never the weights' values."""
    l = rand_logits(9, 50, 16)
    b = np.zeros(16, np.float32)
    b[3] = 10.0
    r = orc.route_logits(l, k=4, score="sigmoid", select_bias=b, renormalize=False)
    assert np.all(r["ids"][:, 0] == 3)
    ref = 1 / (1 + np.exp(-np.take_along_axis(l, r["ids"], axis=1)))
    np.testing.assert_allclose(r["weights"], ref, atol=1e-15)


def test_margins_are_sorted_logit_gaps(orc):
    l = rand_logits(10, 100, 32)
    r = orc.route_logits(l, k=4, score="softmax")
    s = -np.sort(-l, axis=1)
    np.testing.assert_allclose(r["margin_k"], s[:, 3] - s[:, 4], atol=0)
    np.testing.assert_allclose(r["margin_o"], np.diff(-s[:, :4], axis=1).min(axis=1), atol=0)


def test_dynamic_k_rows(orc):
    l = rand_logits(11, 64, 128)
    kpt = np.random.default_rng(12).choice([4, 8, 16], size=64).astype(np.int32)
    r = orc.route_logits(l, k=16, score="softmax", k_per_token=kpt)
    full = orc.route_logits(l, k=16, score="softmax")
    for t in range(64):
        kt = kpt[t]
        np.testing.assert_array_equal(r["ids"][t, :kt], full["ids"][t, :kt])
        assert np.all(r["ids"][t, kt:] == -1) and np.all(r["weights"][t, kt:] == 0)
        assert r["weights"][t].sum() == pytest.approx(1.0, abs=1e-12)


def test_bad_k_per_token_empties_row(orc):
    l = rand_logits(13, 4, 8)
    r = orc.route_logits(l, k=4, score="softmax", k_per_token=np.array([0, 2, 5, -1]))
    assert r["nbad"] == 3
    assert np.all(r["ids"][[0, 2, 3]] == -1) and np.all(r["weights"][[0, 2, 3]] == 0)
    assert np.all(r["ids"][1, :2] >= 0)


# ---- gate ----------------------------------------------------------------------

def test_gate_integer_inputs_exact(orc):
    rng = np.random.default_rng(14)
    x = rng.integers(-8, 9, size=(37, 300)).astype(np.float32)
    W = rng.integers(-8, 9, size=(11, 300)).astype(np.float32)
    exp = x.astype(np.int64) @ W.astype(np.int64).T
    np.testing.assert_array_equal(orc.gate(x, W), exp.astype(np.float64))
    np.testing.assert_array_equal(
        orc.gate(workloads.f32_to_bf16_bits(x), workloads.f32_to_bf16_bits(W)),
        exp.astype(np.float64))


def test_gate_matches_float64_matmul(orc):
    rng = np.random.default_rng(15)
    x = rng.standard_normal((20, 1000)).astype(np.float32)
    W = rng.standard_normal((9, 1000)).astype(np.float32)
    bias = rng.standard_normal(9).astype(np.float32)
    exp = x.astype(np.float64) @ W.astype(np.float64).T + bias.astype(np.float64)
    bound = 1000 * 2.0 ** -52 * (np.abs(x).astype(np.float64) @ np.abs(W).T.astype(np.float64))
    assert np.all(np.abs(orc.gate(x, W, bias) - exp) <= bound + 1e-300)


def test_gate_bf16_bits_equal_their_float_values(orc):
    rng = np.random.default_rng(16)
    xb = workloads.f32_to_bf16_bits(rng.standard_normal((5, 64)).astype(np.float32))
    Wb = workloads.f32_to_bf16_bits(rng.standard_normal((3, 64)).astype(np.float32))
    np.testing.assert_array_equal(
        orc.gate(xb, Wb), orc.gate(workloads.bf16_bits_to_f32(xb), workloads.bf16_bits_to_f32(Wb)))


# ---- hash ----------------------------------------------------------------------

def test_hash_arithmetic_table(orc):
    V, k, E = 1000, 6, 384
    tab = ((np.arange(V)[:, None] * k + np.arange(k)[None, :]) % E).astype(np.int32)
    tok = np.random.default_rng(17).integers(0, V, 500).astype(np.int32)
    ids, nerr = orc.hash_ids(tok, tab, E)
    assert nerr == 0
    np.testing.assert_array_equal(ids, (tok[:, None] * k + np.arange(k)[None, :]) % E)


def test_hash_errors(orc):
    tab = np.array([[0, 1], [2, 9], [3, -1]], np.int32)
    ids, nerr = orc.hash_ids(np.array([0, 1, 2, 3, -1]), tab, 4)
    np.testing.assert_array_equal(ids, [[0, 1], [2, -1], [3, -1], [-1, -1], [-1, -1]])
    assert nerr == 4


# ---- dispatch ------------------------------------------------------------------

@pytest.mark.parametrize("T,k,E", [(1, 1, 1), (7, 3, 5), (1000, 8, 256), (4096, 4, 128)])
def test_dispatch_is_stable_counting_sort(orc, T, k, E):
    rng = np.random.default_rng([T, k, E])
    w = rng.zipf(1.5, size=T * k) % E           # skewed
    ids = np.where(rng.random(T * k) < 0.1, -1, w).astype(np.int32).reshape(T, k)
    d = orc.dispatch(ids, E)
    flat = ids.reshape(-1)
    valid = np.nonzero(flat >= 0)[0]
    np.testing.assert_array_equal(d["counts"], np.bincount(flat[valid], minlength=E))
    np.testing.assert_array_equal(d["offsets"], np.concatenate([[0], np.cumsum(d["counts"])]))
    perm_ref = valid[np.argsort(flat[valid], kind="stable")]
    np.testing.assert_array_equal(d["perm"], perm_ref)
    inv = np.full(T * k, -1)
    inv[perm_ref] = np.arange(perm_ref.size)
    np.testing.assert_array_equal(d["inv"], inv)
    assert d["offsets"][E] == valid.size and d["nerr"] == 0


def test_dispatch_out_of_range_ids(orc):
    ids = np.array([[0, 5], [7, 1], [-3, 0]], np.int32)
    d = orc.dispatch(ids, 4)
    assert d["nerr"] == 2
    np.testing.assert_array_equal(d["counts"], [2, 1, 0, 0])
    np.testing.assert_array_equal(d["perm"], [0, 5, 3])


def test_maxvio(orc):
    assert orc.maxvio(np.full(8, 10, np.int32)) == 0.0
    one_hot = np.zeros(8, np.int32)
    one_hot[2] = 40
    assert orc.maxvio(one_hot) == pytest.approx(7.0)


def test_route_full_matches_parts(orc):
    w = workloads.WORKLOADS["dsv3_grouped"]
    inp = workloads.make_inputs(w.with_T(64).__class__(**{**w.__dict__, "T": 64, "d": 256}))
    kw = dict(score=w.score, select_bias=inp["select_bias"], n_groups=w.n_groups,
              topk_groups=w.topk_groups, group_score=w.group_score, route_scale=w.route_scale)
    full = orc.route_full(inp["x"], inp["W"], w.k, nthreads=3, **kw)
    parts = orc.route(inp["x"], inp["W"], w.k, **kw)
    np.testing.assert_array_equal(full["ids"], parts["ids"])
    np.testing.assert_array_equal(full["weights"], parts["weights"])
    d = orc.dispatch(parts["ids"], w.E)
    np.testing.assert_array_equal(full["perm"], d["perm"])
    np.testing.assert_array_equal(full["inv"], d["inv"])
