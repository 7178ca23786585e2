"""Oracle selection pinned by brute force over every k-subset (E <= 8).

The oracle sorts; these tests never sort.  They enumerate all subsets and keep
the one that dominates the rest under the order (larger q first, lower id on
ties), for experts and for groups (group scores from every pair's sum), as
the DeepSeek-V3.2-Exp "Select experts" page describes the grouped choice and
the ferrox_moe docs describe plain top-k."""
import itertools
import math

import numpy as np
import pytest

# dyadic values: q = l + b is exact, so ties are exact on both sides
L_VALUES = np.array([-1.0, 0.0, 0.5, 1.0, 2.0])
B_VALUES = np.array([0.0, 0.25, -0.25])


def better(q, i, j):
    return q[i] > q[j] or (q[i] == q[j] and i < j)


def dominant_subset(q, cands, k):
    wins = []
    for S in itertools.combinations(cands, k):
        rest = [j for j in cands if j not in S]
        if all(better(q, i, j) for i in S for j in rest):
            wins.append(S)
    assert len(wins) == 1, wins
    S = wins[0]
    # slot order by counting how many members beat each member
    return sorted(S, key=lambda i: sum(better(q, j, i) for j in S))


def group_score_by_pairs(qg, rule):
    if rule == "max":
        return max(qg)
    return max(qg[i] + qg[j] for i in range(len(qg)) for j in range(len(qg)) if i < j)


def brute_route(q, k, G=1, TG=1, rule="max"):
    E = len(q)
    cands = list(range(E))
    if G > 1 and TG < G:
        gs = E // G
        g = [group_score_by_pairs(q[γ * gs:(γ + 1) * gs], rule) for γ in range(G)]
        kept = dominant_subset(g, list(range(G)), TG)
        cands = [e for e in range(E) if e // gs in kept]
    return dominant_subset(q, cands, k)


CASES = [(E, k, G, TG) for E in (1, 2, 3, 4, 6, 8) for k in range(1, E + 1)
         for G in (1, 2, 4) if E % G == 0 for TG in range(1, G + 1)
         if k <= TG * (E // G)]


@pytest.mark.parametrize("E,k,G,TG", CASES)
def test_selection_is_the_dominant_subset(orc, E, k, G, TG):
    rng = np.random.default_rng([E, k, G, TG])
    n = 40
    l = rng.choice(L_VALUES, size=(n, E))
    b = rng.choice(B_VALUES, size=E).astype(np.float32)
    for rule in (["max", "top2_sum"] if G > 1 and E // G >= 2 else ["max"]):
        for bias in (None, b):
            r = orc.route_logits(l, k=k, score="softmax_topk", select_bias=bias,
                                 n_groups=G, topk_groups=TG, group_score=rule,
                                 renormalize=True)
            qb = l + (0.0 if bias is None else bias.astype(np.float64))
            for t in range(n):
                exp = brute_route(list(qb[t]), k, G, TG, rule)
                assert list(r["ids"][t]) == exp, (t, l[t], bias, rule)


@pytest.mark.parametrize("E,k", [(4, 1), (5, 2), (8, 2), (8, 3), (8, 5)])
def test_sigmoid_bias_selection_by_brute_force(orc, E, k):
    """Sigmoid scores plus a selection bias, distinct values, no ties."""
    rng = np.random.default_rng([7, E, k])
    for _ in range(30):
        l = rng.permutation(L_VALUES.tolist() * 2)[:E].astype(np.float64)
        b = rng.choice(B_VALUES, size=E).astype(np.float32)
        r = orc.route_logits(l[None], k=k, score="sigmoid", select_bias=b)
        q = [1.0 / (1.0 + math.exp(-v)) + float(bb) for v, bb in zip(l, b)]
        assert list(r["ids"][0]) == brute_route(q, k)
