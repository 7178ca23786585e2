"""The acceptance checker (tests/parity.py) on fabricated GPU outputs (CPU).

Rows the rule must accept (the oracle's own answer; another valid answer of
a near tie) and rows it must reject (a wrong id on a clear token, a clear
winner dropped in a near-tie token, a pick from a group that is clearly
out, experts inside a valid kept-group set that are not its top-k, a quota
exceeded or not optimal, a slot order reversed beyond 1e-4, a weight off by
more than 1e-4).  Weights of fabricated rows come from the oracle's own
weights_for_ids, so only the property under test differs."""
import numpy as np
import pytest

from tests.parity import NEAR, check_route, oracle_route


def fabricate(orc, ref, rows, *, score, renormalize=True, route_scale=1.0):
    """GPU outputs equal to the oracle's, with rows {t: ids} replaced."""
    ids = ref["ids"].copy()
    for t, r in rows.items():
        ids[t] = r
    w = orc.weights_for_ids(ref["logits"], ids, score=score, renormalize=renormalize,
                            route_scale=route_scale)
    return ids, w


def run(orc, ref, ids, w, **kw):
    return check_route(ids, w, ref, orc, **kw)


# ---- flat selection: a near tie at the k-th boundary --------------------------------

def flat_case(orc):
    # token 0: experts 1 and 2 tie within 5e-5 at the k = 2 boundary (near tie);
    # token 1: clear margins everywhere
    l = np.array([[3.0, 2.0, 2.0 - 5e-5, 0.0, -1.0, -2.0],
                  [0.0, 1.0, 2.0, 3.0, 4.0, 5.0]])
    return oracle_route(orc, l, 2, score="softmax")


def test_flat_oracle_answer_and_valid_alternative_pass(orc):
    ref = flat_case(orc)
    assert ref["margin_k"][0] < NEAR <= ref["margin_k"][1]
    st = run(orc, ref, *fabricate(orc, ref, {}, score="softmax"), score="softmax")
    assert st["near_tie"] == 1
    run(orc, ref, *fabricate(orc, ref, {0: [0, 2]}, score="softmax"), score="softmax")


def test_flat_dropped_clear_winner_fails(orc):
    """[1, 2] keeps both near-tie experts and drops expert 0, which is clearly
    above the boundary: each chosen expert is within 1e-4 of the boundary, so
    a one-sided check would pass it."""
    ref = flat_case(orc)
    with pytest.raises(AssertionError, match="k boundary"):
        run(orc, ref, *fabricate(orc, ref, {0: [1, 2]}, score="softmax"), score="softmax")


def test_flat_clear_token_wrong_id_fails(orc):
    ref = flat_case(orc)
    with pytest.raises(AssertionError, match="ids != oracle"):
        run(orc, ref, *fabricate(orc, ref, {1: [5, 3]}, score="softmax"), score="softmax")


def test_slot_order(orc):
    # token 0: selected experts 0, 1 within 5e-5 of each other (slot-order tie)
    l = np.array([[2.0, 2.0 - 5e-5, 0.0, -1.0]])
    ref = oracle_route(orc, l, 2, score="softmax")
    assert ref["margin_o"][0] < NEAR and ref["margin_k"][0] > NEAR
    run(orc, ref, *fabricate(orc, ref, {0: [1, 0]}, score="softmax"), score="softmax")
    l2 = np.array([[2.0, 1.0, 1.0 - 5e-5, -1.0]])  # near tie at k = 2; slots 0 and 1 clear
    ref2 = oracle_route(orc, l2, 2, score="softmax")
    run(orc, ref2, *fabricate(orc, ref2, {0: [0, 2]}, score="softmax"), score="softmax")
    with pytest.raises(AssertionError, match="slot order"):
        run(orc, ref2, *fabricate(orc, ref2, {0: [2, 0]}, score="softmax"), score="softmax")


def test_weight_error_fails(orc):
    ref = flat_case(orc)
    ids, w = fabricate(orc, ref, {}, score="softmax")
    w[1, 0] += 2e-4
    with pytest.raises(AssertionError, match="dw"):
        run(orc, ref, ids, w, score="softmax")
    ids, w = fabricate(orc, ref, {0: [0, 2]}, score="softmax")
    w[0, 1] += 2e-4
    with pytest.raises(AssertionError, match="near-tie weights"):
        run(orc, ref, ids, w, score="softmax")


# ---- group limit: a near tie between groups -------------------------------------------

def grouped_case(orc):
    # softmax_topk with a zero bias: q = l + 0 (not monotone: biased rule);
    # 4 groups of 2, keep 2, top-2 by the group score (sum of the two largest).
    # Groups 0 and 1 tie within 5e-5; group 2 is clearly kept, group 3 out.
    l = np.array([[1.0, 0.5, 1.0, 0.5 - 5e-5, 3.0, 2.0, -1.0, -2.0]])
    b = np.zeros(8, np.float32)
    kw = dict(score="softmax_topk", select_bias=b, n_groups=4, topk_groups=2,
              group_score="top2_sum")
    return oracle_route(orc, l, 2, **kw), kw


def test_group_near_tie_alternatives(orc):
    ref, kw = grouped_case(orc)
    assert ref["margin_g"][0] < NEAR
    ck = dict(score="softmax_topk", n_groups=4, topk_groups=2)
    assert ref["ids"][0].tolist() == [4, 5]
    run(orc, ref, *fabricate(orc, ref, {}, score="softmax_topk"), **ck)


def test_group_near_tie_wrong_picks_fail(orc):
    ref, kw = grouped_case(orc)
    ck = dict(score="softmax_topk", n_groups=4, topk_groups=2)
    # expert 0 lies in a near group, but within groups {2, 0} the top-2 is 4, 5
    with pytest.raises(AssertionError, match="group limit"):
        run(orc, ref, *fabricate(orc, ref, {0: [4, 0]}, score="softmax_topk"), **ck)
    # expert 6 lies in group 3, clearly dropped
    with pytest.raises(AssertionError, match="group limit"):
        run(orc, ref, *fabricate(orc, ref, {0: [4, 6]}, score="softmax_topk"), **ck)


def test_group_near_tie_choice_inside_the_near_groups(orc):
    # now the k boundary falls inside the near groups: keep {2, x}, x in {0, 1};
    # top-3 takes 4, 5 and the best of group x -- 0 (x = 0) or 2 (x = 1)
    l = np.array([[1.0, 0.5, 1.0, 0.5 - 5e-5, 3.0, 2.0, -1.0, -2.0]])
    kw = dict(score="softmax_topk", select_bias=np.zeros(8, np.float32), n_groups=4,
              topk_groups=2, group_score="top2_sum")
    ref = oracle_route(orc, l, 3, **kw)
    ck = dict(score="softmax_topk", n_groups=4, topk_groups=2)
    assert ref["ids"][0].tolist() == [4, 5, 0]
    run(orc, ref, *fabricate(orc, ref, {0: [4, 5, 2]}, score="softmax_topk"), **ck)
    with pytest.raises(AssertionError, match="group limit"):  # 1 < 0 in group 0
        run(orc, ref, *fabricate(orc, ref, {0: [4, 5, 1]}, score="softmax_topk"), **ck)


# ---- per-group quota --------------------------------------------------------------------

def test_quota_near_tie(orc):
    # 2 groups of 3, one per group, k = 2; group 0's best two tie within 5e-5
    l = np.array([[2.0, 2.0 - 5e-5, 0.0, 1.0, 0.5, -1.0]])
    ref = oracle_route(orc, l, 2, score="softmax_topk", n_groups=2, k_per_group=1)
    ck = dict(score="softmax_topk", n_groups=2, k_per_group=1)
    assert ref["margin_g"][0] < NEAR and ref["ids"][0].tolist() == [0, 3]
    run(orc, ref, *fabricate(orc, ref, {}, score="softmax_topk"), **ck)
    run(orc, ref, *fabricate(orc, ref, {0: [1, 3]}, score="softmax_topk"), **ck)
    with pytest.raises(AssertionError, match="quota"):  # two from group 0
        run(orc, ref, *fabricate(orc, ref, {0: [0, 1]}, score="softmax_topk"), **ck)
    with pytest.raises(AssertionError, match="quota"):  # 4 instead of 3 in group 1
        run(orc, ref, *fabricate(orc, ref, {0: [0, 4]}, score="softmax_topk"), **ck)
