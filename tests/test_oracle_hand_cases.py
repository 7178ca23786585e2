"""Oracle pinned to the hand-worked cases of tests/golden/hand_cases.json.

Each case cites the page passage whose rule it exercises and carries its own
derivation; the expected numbers are closed forms, not oracle output."""
import math

import numpy as np
import pytest

TOL = 1e-12


def _route(orc, c, **over):
    kw = dict(k=c["k"], score=c["score"], renormalize=c.get("renormalize", True),
              route_scale=c.get("route_scale", 1.0))
    if "select_bias" in c:
        kw["select_bias"] = np.array(c["select_bias"], np.float32)
    if "n_groups" in c:
        kw.update(n_groups=c["n_groups"], topk_groups=c["topk_groups"],
                  group_score=c["group_score"])
    if "k_per_token" in c:
        kw["k_per_token"] = np.array(c["k_per_token"], np.int32)
    kw.update(over)
    return orc.route_logits(np.array(c["logits"], np.float64), **kw)


@pytest.mark.parametrize("name", ["A_softmax_renorm", "A_softmax_topk", "B_tie_rule",
                                  "C_grouped_biased"])
def test_hand_case_ids_weights_margins(orc, hand_cases, name):
    c = hand_cases[name]
    r = _route(orc, c)
    np.testing.assert_array_equal(r["ids"], np.array(c["ids"]))
    np.testing.assert_allclose(r["weights"], np.array(c["weights"]), atol=TOL, rtol=0)
    np.testing.assert_allclose(r["margin_k"], np.array(c["margin_k"]), atol=TOL, rtol=0)
    if "margin_g" in c:
        np.testing.assert_allclose(r["margin_g"], np.array(c["margin_g"]), atol=TOL)
    if "group_scores" in c:
        np.testing.assert_allclose(r["g"], np.array(c["group_scores"]), atol=TOL)


def test_case_c_group_limit_matters(orc, hand_cases):
    """Dropping the group limit must change the answer to the cited one."""
    c = hand_cases["C_grouped_biased"]
    r = _route(orc, c, n_groups=1, topk_groups=1)
    np.testing.assert_array_equal(r["ids"], np.array(c["ids_without_groups"]))


def test_case_c_group_score_is_top2_not_max(orc, hand_cases):
    """With the max rule the kept groups would be {3, 1} and ids [7, 2]."""
    c = hand_cases["C_grouped_biased"]
    r = _route(orc, c, group_score="max")
    np.testing.assert_array_equal(r["ids"], [[7, 2]])


def test_case_a_softmax_probs(orc, hand_cases):
    c = hand_cases["A_softmax_renorm"]
    r = _route(orc, c, k=4, renormalize=False)
    # all four selected in order 1, 2, 0, 3 with the plain softmax probabilities
    np.testing.assert_array_equal(r["ids"], [[1, 2, 0, 3]])
    p = np.array(c["softmax_probs"])
    np.testing.assert_allclose(r["weights"][0], p[[1, 2, 0, 3]], atol=TOL)


@pytest.mark.parametrize("k", [2, 3])
def test_case_d_sqrt_softplus(orc, hand_cases, k):
    c = hand_cases["D_sqrt_softplus"]
    logits = np.array([[math.log(math.expm1(s)) for s in c["softplus_values"]]])
    r = orc.route_logits(logits, k=k, score="sqrt_softplus", renormalize=True)
    exp = c["k%d" % k]
    np.testing.assert_array_equal(r["ids"], exp["ids"])
    np.testing.assert_allclose(r["weights"], exp["weights"], atol=1e-12)


def test_case_e_hash_and_dispatch(orc, hand_cases):
    c = hand_cases["E_hash_dispatch"]
    ids, nerr = orc.hash_ids(np.array(c["token_ids"]), np.array(c["tid2eid"]), c["E"])
    assert nerr == 0
    np.testing.assert_array_equal(ids, c["ids"])
    w = orc.weights_for_ids(np.zeros((3, c["E"])), ids, score="sigmoid")
    np.testing.assert_allclose(w, c["weights_sigmoid_zero_logits"], atol=TOL)
    d = orc.dispatch(ids, c["E"])
    for key in ("counts", "offsets", "perm", "inv"):
        np.testing.assert_array_equal(d[key], c[key], err_msg=key)
    assert orc.maxvio(d["counts"]) == pytest.approx(c["maxvio"], abs=1e-15)


def test_case_f_dynamic_k(orc, hand_cases):
    c = hand_cases["F_dynamic_k"]
    r = _route(orc, c)
    np.testing.assert_array_equal(r["ids"], c["ids"])
    np.testing.assert_allclose(r["weights"], c["weights"], atol=TOL)
    d = orc.dispatch(r["ids"], 4)
    for key in ("counts", "offsets", "perm", "inv"):
        np.testing.assert_array_equal(d[key], c[key], err_msg=key)
