"""Pins of the oracle's combine (CPU): y[t] = sum_j w[t][j] * Yp[inv[t][j]]
(+ shared[t]).  Sources: the dynamic-k feature request ("Possible
Implementation": the output is the weighted sum of the selected experts'
outputs) and the ferrox_moe documentation (combine_expert_outputs: routed
plus shared outputs of a token).  The pages print no numeric example, so the
pins are a hand-worked case, identities and special cases that fix every
index, weight and term."""
import numpy as np
import pytest

import oracle


def bf16_bits(a):
    """bf16 bit patterns of float32 values that bf16 holds exactly."""
    b = np.ascontiguousarray(a, np.float32).view(np.uint32)
    assert np.all(b & 0xFFFF == 0), "value not exact in bf16"
    return (b >> 16).astype(np.uint16)


def test_hand_case():
    # Yp rows are the expert outputs in dispatch order; token 0 takes row 2
    # with weight 1/2 and row 0 with weight 1/4 plus its shared output of 1s;
    # token 1 takes row 1 with weight 1, and slot 1 is empty (inv -1) even
    # though its weight is 3.
    Yp = np.array([[1, 2, 3], [4, 5, 6], [7, 8, 9]], np.float32)
    inv = np.array([[2, 0], [1, -1]], np.int32)
    w = np.array([[0.5, 0.25], [1.0, 3.0]], np.float32)
    shared = np.array([[1, 1, 1], [0, 0, 0]], np.float32)
    y, nerr = oracle.combine(Yp, inv, w, shared)
    # 0.5*[7,8,9] + 0.25*[1,2,3] + [1,1,1] = [4.75, 5.5, 6.25]
    assert np.array_equal(y, [[4.75, 5.5, 6.25], [4.0, 5.0, 6.0]])
    assert nerr == 0
    y2, _ = oracle.combine(Yp, inv, w)  # no shared expert
    assert np.array_equal(y2, [[3.75, 4.5, 5.25], [4.0, 5.0, 6.0]])


def test_out_of_range_rows_are_counted_and_skipped():
    Yp = np.arange(6, dtype=np.float32).reshape(2, 3)
    inv = np.array([[1, 2], [5, -1], [-7, 0]], np.int32)
    w = np.ones((3, 2), np.float32)
    y, nerr = oracle.combine(Yp, inv, w)
    assert nerr == 2  # rows 2 and 5 do not exist (R = 2)
    assert np.array_equal(y, [[3, 4, 5], [0, 0, 0], [0, 1, 2]])


@pytest.mark.parametrize("k", [1, 2, 4])
def test_identity_experts_return_the_tokens(k):
    # every expert is the identity: row p of Yp is the hidden state of the
    # token that route perm[p] belongs to; with weights summing to one the
    # combine gives the token back (dyadic weights: exact), and with a shared
    # output s it gives x + s.  A wrong row index or a dropped slot breaks it.
    rng = np.random.default_rng(5)
    T, E, d = 37, 8, 5
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    ids[3, k - 1] = -1 if k > 1 else ids[3, 0]
    disp = oracle.dispatch(ids, E)
    x = rng.integers(-8, 9, size=(T, d)).astype(np.float32)
    Yp = x[disp["perm"] // k]
    valid = (disp["inv"].reshape(T, k) >= 0)
    w = np.where(valid, 1.0 / valid.sum(1, keepdims=True), 0.0).astype(np.float32)
    w[3] = np.where(valid[3], 1.0 if valid[3].sum() == 1 else 0.5, 0.0)
    y, nerr = oracle.combine(Yp, disp["inv"].reshape(T, k), w)
    wsum = w.sum(1, dtype=np.float64)[:, None]
    assert nerr == 0 and np.array_equal(y, wsum * x)
    s = rng.integers(-4, 5, size=(T, d)).astype(np.float32)
    y2, _ = oracle.combine(Yp, disp["inv"].reshape(T, k), w, s)
    assert np.array_equal(y2, wsum * x + s)


def test_relabelled_rows_give_the_same_result():
    # the combine depends on which row each slot names, not on where the rows
    # sit: moving the rows by a permutation and the slots with them changes
    # nothing (the sum over slots keeps its order, so bit for bit)
    rng = np.random.default_rng(6)
    T, k, d, R = 20, 3, 7, 45
    Yp = rng.standard_normal((R, d)).astype(np.float32)
    inv = rng.integers(-1, R, size=(T, k)).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    pi = rng.permutation(R)
    Yq = np.empty_like(Yp)
    Yq[pi] = Yp
    invq = np.where(inv >= 0, pi[np.maximum(inv, 0)], -1).astype(np.int32)
    a, _ = oracle.combine(Yp, inv, w)
    b, _ = oracle.combine(Yq, invq, w)
    assert np.array_equal(a, b)


def test_single_slot_is_a_gather_and_weights_are_linear():
    rng = np.random.default_rng(7)
    T, d, R = 16, 9, 10
    Yp = rng.standard_normal((R, d)).astype(np.float32)
    inv = rng.integers(0, R, size=(T, 1)).astype(np.int32)
    y, _ = oracle.combine(Yp, inv, np.ones((T, 1), np.float32))
    assert np.array_equal(y, Yp[inv[:, 0]].astype(np.float64))
    # scaling every weight by a power of two scales the routed sum exactly
    inv2 = rng.integers(0, R, size=(T, 3)).astype(np.int32)
    w = rng.random((T, 3)).astype(np.float32)
    a, _ = oracle.combine(Yp, inv2, w)
    b, _ = oracle.combine(Yp, inv2, (4 * w).astype(np.float32))
    assert np.array_equal(4 * a, b)


def test_bf16_inputs_match_their_float32_values():
    rng = np.random.default_rng(8)
    T, k, d, R = 11, 2, 6, 9
    Yp = rng.integers(-100, 101, size=(R, d)).astype(np.float32) / 8
    sh = rng.integers(-100, 101, size=(T, d)).astype(np.float32) / 4
    inv = rng.integers(-1, R, size=(T, k)).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    a, _ = oracle.combine(Yp, inv, w, sh)
    b, _ = oracle.combine(bf16_bits(Yp), inv, w, bf16_bits(sh))
    assert np.array_equal(a, b)
