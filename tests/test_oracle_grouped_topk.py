"""Pins of the oracle's grouped top-k with a per-group quota (CPU): the
ferrox_moe item route_top_k_grouped splits the experts into contiguous
groups, keeps the k_per_group highest of each group by the flat rule's
score, then (optionally) the global top-k of those.  The pages print no
example, so the pins are hand-worked cases, special cases that reduce to the
flat rule, and brute force against an independent characterisation: keeping
at most k_per_group per group is a partition-matroid constraint, and the
two-step rule picks the unique k-subset of largest total q under it."""
import itertools

import numpy as np
import pytest

import oracle


def sig(x):
    return 1.0 / (1.0 + np.exp(-x))


def test_hand_case_one_per_group():
    # groups {0,1} {2,3} {4,5}; each keeps its best: 0 (5), 2 (1), 4 (3);
    # the global top-2 of those is 0, 4 (the flat top-2 would be 0, 1)
    l = np.array([[5.0, 4.0, 1.0, 0.0, 3.0, 2.0]])
    out = oracle.route_logits(l, 2, score="sigmoid", n_groups=3, k_per_group=1)
    assert out["ids"].tolist() == [[0, 4]]
    w = np.array([sig(5.0), sig(3.0)])
    np.testing.assert_allclose(out["weights"][0], w / w.sum(), rtol=1e-15)
    flat = oracle.route_logits(l, 2, score="sigmoid")
    assert flat["ids"].tolist() == [[0, 1]]
    # k = 3: every group's best, larger first
    out3 = oracle.route_logits(l, 3, score="sigmoid", n_groups=3, k_per_group=1)
    assert out3["ids"].tolist() == [[0, 4, 2]]
    # two per group keeps everything: the flat top-3
    out2 = oracle.route_logits(l, 3, score="sigmoid", n_groups=3, k_per_group=2)
    assert out2["ids"].tolist() == [[0, 1, 4]]


def test_hand_case_ties_and_bias():
    # equal q inside a group: the lower id is kept
    l = np.array([[1.0, 1.0, 0.0, 0.0]])
    out = oracle.route_logits(l, 2, score="softmax", n_groups=2, k_per_group=1)
    assert out["ids"].tolist() == [[0, 2]]
    # the selection bias moves the choice (q = s + b), not the weights
    b = np.array([0.0, 0.5, 0.0, 0.0], np.float32)
    outb = oracle.route_logits(l, 2, score="softmax", n_groups=2, k_per_group=1,
                               select_bias=b, renormalize=False)
    assert outb["ids"].tolist() == [[1, 2]]
    p = np.exp(l[0]) / np.exp(l[0]).sum()
    np.testing.assert_allclose(outb["weights"][0], [p[1], p[2]], rtol=1e-15)


@pytest.mark.parametrize("E,G,kpg,k", [(6, 3, 1, 2), (6, 2, 2, 3), (8, 4, 1, 3), (8, 2, 3, 5),
                                       (8, 4, 2, 8), (8, 8, 1, 4), (8, 1, 3, 3)])
@pytest.mark.parametrize("score", ["softmax", "sigmoid", "sqrt_softplus"])
def test_brute_force_matroid_optimum(E, G, kpg, k, score):
    rng = np.random.default_rng([E, G, kpg, k, len(score)])
    T = 40
    l = rng.standard_normal((T, E))
    sb = (rng.standard_normal(E) * 0.3).astype(np.float32) if score != "softmax" else None
    out = oracle.route_logits(l, k, score=score, n_groups=G, k_per_group=kpg, select_bias=sb)
    raw = oracle.route_logits(l, 1, score=score, select_bias=sb)["q"]  # q, no mask
    gs = E // G
    subsets = [c for c in itertools.combinations(range(E), k)
               if all(sum(1 for e in c if e // gs == g) <= kpg for g in range(G))]
    for t in range(T):
        best = max(subsets, key=lambda c: raw[t, list(c)].sum())
        assert sorted(out["ids"][t].tolist()) == sorted(best), (t, out["ids"][t], best)
        q = raw[t, out["ids"][t]]
        assert np.all(np.diff(q) <= 0)  # larger first


@pytest.mark.parametrize("score", ["softmax", "sigmoid"])
def test_reductions_to_the_flat_rule(score):
    rng = np.random.default_rng(7)
    l = rng.standard_normal((200, 32))
    flat = oracle.route_logits(l, 6, score=score)
    # a quota no group can fill, or one group: the flat top-k
    for G, kpg in [(4, 8), (4, 20), (1, 6), (1, 32)]:
        out = oracle.route_logits(l, 6, score=score, n_groups=G, k_per_group=kpg)
        assert np.array_equal(out["ids"], flat["ids"]), (G, kpg)
        np.testing.assert_allclose(out["weights"], flat["weights"], rtol=1e-14)


def test_full_quota_takes_exactly_kpg_per_group():
    rng = np.random.default_rng(8)
    E, G, kpg = 64, 8, 2
    l = rng.standard_normal((300, E))
    out = oracle.route_logits(l, G * kpg, score="sigmoid", n_groups=G, k_per_group=kpg)
    gs = E // G
    for t in range(300):
        cnt = np.bincount(out["ids"][t] // gs, minlength=G)
        assert np.all(cnt == kpg)
        for g in range(G):  # the group's two largest logits
            mine = np.sort(out["ids"][t][out["ids"][t] // gs == g])
            assert np.array_equal(mine, np.sort(np.argsort(-l[t, g * gs:(g + 1) * gs])[:kpg] + g * gs))


def test_quota_invariants_dynamic_k_and_weights():
    rng = np.random.default_rng(9)
    E, G, kpg, K = 128, 8, 2, 10
    T = 256
    l = rng.standard_normal((T, E))
    kt = rng.integers(1, K + 1, size=T).astype(np.int32)
    out = oracle.route_logits(l, K, score="softmax", n_groups=G, k_per_group=kpg,
                              k_per_token=kt)
    gs = E // G
    for t in range(T):
        row = out["ids"][t, :kt[t]]
        assert np.all(row >= 0) and np.all(out["ids"][t, kt[t]:] == -1)
        assert np.bincount(row // gs, minlength=G).max() <= kpg
        assert np.isfinite(out["margin_g"][t]) and out["margin_g"][t] >= 0
    # weights depend only on the ids (the same rule as every other selection)
    w = oracle.weights_for_ids(l, out["ids"], score="softmax")
    np.testing.assert_allclose(out["weights"], w, rtol=1e-14)
    # the prefix property of the greedy: k_t picks are the first k_t of K
    full = oracle.route_logits(l, K, score="softmax", n_groups=G, k_per_group=kpg)
    for t in range(T):
        assert np.array_equal(out["ids"][t, :kt[t]], full["ids"][t, :kt[t]])


def test_argument_checks():
    l = np.zeros((1, 8))
    with pytest.raises(ValueError):  # more than the groups keep
        oracle.route_logits(l, 5, n_groups=4, k_per_group=1)
    with pytest.raises(ValueError):  # no group limit together with a quota
        oracle.route_logits(l, 2, n_groups=4, topk_groups=2, k_per_group=1)
