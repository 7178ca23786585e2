"""Pins of the oracle's selection margins -- the numbers that decide which
tokens the acceptance rule compares bit for bit and which it checks for
validity only (a gap below 1e-4 at the k-th or the group boundary).

The pages fix no margin; the acceptance rule measures a token's gap in the
units of the quantity the selection compares: the logit when the choice is a
monotone function of it, else q = score + selection bias ("DeepSeek-V3.2-Exp
- Select experts", Explanation: the bias only chooses).  Pinned here by

* hand-worked values (tests/golden/hand_cases.json, each with its
  derivation): the biased grouped case, a biased flat case whose slot gap in
  q units differs from its logit gap, and grouped top-k with a per-group
  quota (ferrox_moe route_top_k_grouped) with its group-cut gap and each
  group's last kept value;
* brute force for E <= 8 that never sorts: the selection is the subset that
  dominates every other (as in test_oracle_bruteforce), and each margin is
  the smallest difference over all PAIRS across the boundary it describes
  (selected vs. unselected candidate, kept vs. dropped group, two selected
  experts, kept vs. dropped member of one group) -- a characterisation of
  the same number that shares no step with the oracle's sorted neighbours.
"""
import itertools
import math

import numpy as np
import pytest

from tests.test_oracle_bruteforce import brute_route, dominant_subset, group_score_by_pairs

INF = math.inf


def _route(orc, c):
    kw = dict(score=c["score"], renormalize=c.get("renormalize", True),
              route_scale=c.get("route_scale", 1.0))
    if "select_bias" in c:
        kw["select_bias"] = np.array(c["select_bias"], np.float32)
    if "n_groups" in c:
        kw["n_groups"] = c["n_groups"]
        if c.get("k_per_group"):
            kw["k_per_group"] = c["k_per_group"]
        else:
            kw.update(topk_groups=c["topk_groups"], group_score=c["group_score"])
    if "k_per_token" in c:
        kw["k_per_token"] = np.array(c["k_per_token"], np.int32)
    return orc.route_logits(np.array(c["logits"], np.float64), c["k"], **kw)


def _none_inf(v):
    return [INF if x is None else x for x in v]


@pytest.mark.parametrize("name", ["A_softmax_renorm", "A_softmax_topk", "B_tie_rule",
                                  "C_grouped_biased", "F_dynamic_k", "G_grouped_quota",
                                  "H_sigmoid_bias_order"])
def test_hand_worked_margins(orc, hand_cases, name):
    c = hand_cases[name]
    r = _route(orc, c)
    np.testing.assert_array_equal(r["ids"], np.array(c["ids"]))
    np.testing.assert_allclose(r["weights"], np.array(c["weights"]), atol=1e-12, rtol=0)
    np.testing.assert_allclose(r["margin_k"], _none_inf(c["margin_k"]), atol=1e-12, rtol=0)
    np.testing.assert_allclose(r["margin_o"], _none_inf(c["margin_o"]), atol=1e-12, rtol=0)
    if "margin_g" in c:
        np.testing.assert_allclose(r["margin_g"], c["margin_g"], atol=1e-12, rtol=0)
    if "group_last_kept" in c:
        np.testing.assert_allclose(r["g"], c["group_last_kept"], atol=1e-12, rtol=0)


def test_quota_case_differs_from_flat(orc, hand_cases):
    c = dict(hand_cases["G_grouped_quota"])
    c.pop("n_groups")
    r = _route(orc, c)
    np.testing.assert_array_equal(r["ids"], c["ids_without_quota"])


def test_biased_slot_gap_is_in_q_units(orc, hand_cases):
    """Without the bias the same logits give the logit gap ln 3 as slot gap
    (monotone case); with it the q gap 0.25 -- the units change with the
    rule, as the acceptance rule reads them."""
    c = hand_cases["H_sigmoid_bias_order"]
    r = orc.route_logits(np.array(c["logits"]), c["k"], score="sigmoid")
    assert r["ids"][0].tolist() == [1, 0]
    assert r["margin_o"][0] == pytest.approx(math.log(3.0), abs=1e-12)


# ---- brute force over pairs -------------------------------------------------------

def pair_margins(q, S, cands):
    """(k-boundary gap, slot gap) as minima over pairs; +inf when empty."""
    rest = [j for j in cands if j not in S]
    mk = min((q[i] - q[j] for i in S for j in rest), default=INF)
    mo = min((abs(q[i] - q[j]) for i, j in itertools.combinations(S, 2)), default=INF)
    return mk, mo


CASES = [(E, k, G, TG) for E in (2, 3, 4, 6, 8) for k in range(1, E + 1)
         for G in (1, 2, 4) if E % G == 0 for TG in range(1, G + 1)
         if k <= TG * (E // G)]


@pytest.mark.parametrize("E,k,G,TG", CASES)
def test_margins_are_pairwise_minima(orc, E, k, G, TG):
    rng = np.random.default_rng([E, k, G, TG, 3])
    n = 25
    # distinct-ish continuous logits plus some exact ties
    l = np.round(rng.standard_normal((n, E)) * 4) / 4 + rng.choice([0.0, 0.01], size=(n, E))
    b = (0.25 * rng.standard_normal(E)).astype(np.float32)
    rules = ["max", "top2_sum"] if G > 1 and E // G >= 2 else ["max"]
    for rule in rules:
        for bias in (None, b):
            r = orc.route_logits(l, k=k, score="softmax_topk", select_bias=bias,
                                 n_groups=G, topk_groups=TG, group_score=rule)
            grouped = G > 1 and TG < G
            for t in range(n):
                q = list(l[t] + (0.0 if bias is None else bias.astype(np.float64)))
                S = brute_route(q, k, G, TG, rule)
                cands = list(range(E))
                mg = INF
                if grouped:
                    gs = E // G
                    g = [group_score_by_pairs(q[γ * gs:(γ + 1) * gs], rule) for γ in range(G)]
                    kept = dominant_subset(g, list(range(G)), TG)
                    cands = [e for e in range(E) if e // gs in kept]
                    mg = min(g[a] - g[c] for a in kept for c in range(G) if c not in kept)
                mk, mo = pair_margins(q, S, cands)
                where = (t, rule, bias is not None)
                assert r["margin_k"][t] == pytest.approx(mk, abs=1e-12), where
                assert r["margin_o"][t] == pytest.approx(mo, abs=1e-12), where
                assert r["margin_g"][t] == pytest.approx(mg, abs=1e-12), where


QUOTA = [(4, 2, 1, 2), (6, 3, 1, 2), (6, 2, 2, 3), (8, 4, 1, 3), (8, 2, 3, 5), (8, 4, 2, 6),
         (8, 2, 4, 4), (8, 1, 3, 3)]


@pytest.mark.parametrize("E,G,kpg,k", QUOTA)
@pytest.mark.parametrize("biased", [False, True])
def test_quota_margins_are_pairwise_minima(orc, E, G, kpg, k, biased):
    """With a per-group quota: each group keeps its dominant kpg-subset; the
    group-cut gap is the smallest kept-minus-dropped difference inside a
    group, a group's last kept value the smallest q it keeps (-inf when it
    keeps all), and the k gap / slot gap are pair minima over the kept."""
    rng = np.random.default_rng([E, G, kpg, k, int(biased)])
    n = 30
    l = np.round(rng.standard_normal((n, E)) * 4) / 4 + rng.choice([0.0, 0.02], size=(n, E))
    b = (0.25 * rng.standard_normal(E)).astype(np.float32) if biased else None
    r = orc.route_logits(l, k=k, score="softmax_topk", select_bias=b, n_groups=G,
                         k_per_group=kpg)
    gs = E // G
    for t in range(n):
        q = list(l[t] + (0.0 if b is None else b.astype(np.float64)))
        kept_all, mg, last = [], INF, []
        for γ in range(G):
            members = list(range(γ * gs, (γ + 1) * gs))
            if kpg >= gs:
                keep = members
                last.append(-INF)
            else:
                keep = dominant_subset(q, members, kpg)
                drop = [j for j in members if j not in keep]
                mg = min(mg, min(q[i] - q[j] for i in keep for j in drop))
                last.append(min(q[i] for i in keep))
            kept_all += keep
        S = dominant_subset(q, kept_all, k)
        mk, mo = pair_margins(q, S, kept_all)
        assert list(r["ids"][t]) == S, t
        assert r["margin_g"][t] == pytest.approx(mg, abs=1e-12), t
        np.testing.assert_allclose(r["g"][t], last, atol=1e-12)
        assert r["margin_k"][t] == pytest.approx(mk, abs=1e-12), t
        assert r["margin_o"][t] == pytest.approx(mo, abs=1e-12), t


@pytest.mark.parametrize("score", ["softmax", "sigmoid", "sqrt_softplus"])
def test_monotone_margins_in_logit_units(orc, score):
    """No bias and no group limit: every score is strictly increasing in the
    logit, so the margins are pair minima of the logits themselves."""
    rng = np.random.default_rng(len(score))
    l = rng.standard_normal((40, 8)) * 2
    r = orc.route_logits(l, k=3, score=score)
    for t in range(40):
        S = brute_route(list(l[t]), 3)
        mk, mo = pair_margins(list(l[t]), S, list(range(8)))
        assert r["margin_k"][t] == pytest.approx(mk, abs=1e-12)
        assert r["margin_o"][t] == pytest.approx(mo, abs=1e-12)
        assert math.isinf(r["margin_g"][t])


def test_threaded_oracle_equals_one_thread(orc):
    """The threaded entry points split tokens only: same results bit for bit."""
    rng = np.random.default_rng(4)
    x = rng.standard_normal((203, 300)).astype(np.float32)
    W = rng.standard_normal((40, 300)).astype(np.float32)
    lb = rng.standard_normal(40).astype(np.float32)
    a = orc.gate(x, W, lb)
    np.testing.assert_array_equal(orc.gate(x, W, lb, nthreads=7), a)
    b = (0.1 * rng.standard_normal(40)).astype(np.float32)
    kw = dict(score="sigmoid", select_bias=b, n_groups=8, topk_groups=3,
              k_per_token=rng.integers(1, 7, 203).astype(np.int32))
    one = orc.route_logits(a, 6, **kw)
    many = orc.route_logits(a, 6, nthreads=5, **kw)
    for key in ("ids", "weights", "margin_k", "margin_g", "margin_o", "margin_s", "q", "g"):
        np.testing.assert_array_equal(one[key], many[key], err_msg=key)
