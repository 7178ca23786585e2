"""Pins of the oracle's expert-parallel send layout (CPU): per-rank counts
and offsets for N ranks owning E/N contiguous experts, and the send buffer
of token rows in dispatch order.  The router survey page states that under
expert parallelism every routing choice becomes all-to-all traffic; the
layout taken is the dispatch order itself.  No numeric example is printed,
so the pins are a hand-worked case, special cases and invariants."""
import numpy as np
import pytest

import oracle


def test_hand_case():
    # E = 4 experts over N = 2 ranks: rank 0 owns experts 0-1, rank 1 owns 2-3
    ids = np.array([[3, 2], [3, 1], [1, 1]], np.int32)  # routes r = 0..5
    d = oracle.dispatch(ids, 4)
    assert d["counts"].tolist() == [0, 3, 1, 2] and d["perm"].tolist() == [3, 4, 5, 1, 0, 2]
    cnt, off = oracle.ep_layout(d["offsets"], 2)
    assert cnt.tolist() == [3, 3] and off.tolist() == [0, 3, 6]
    x = np.array([[10, 11], [20, 21], [30, 31]], np.float32)  # tokens 0..2
    rows = oracle.permute_rows(x, d["perm"], 2)
    # routes 3,4,5 belong to tokens 1,2,2; routes 1,0,2 to tokens 0,0,1
    assert rows.tolist() == [[20, 21], [30, 31], [30, 31], [10, 11], [10, 11], [20, 21]]


@pytest.mark.parametrize("N", [1, 2, 8, 64])
def test_rank_blocks_sum_the_expert_counts(N):
    rng = np.random.default_rng(N)
    E, T, k = 64, 400, 4
    ids = rng.integers(-1, E, size=(T, k)).astype(np.int32)
    d = oracle.dispatch(ids, E)
    cnt, off = oracle.ep_layout(d["offsets"], N)
    assert off[0] == 0 and off[-1] == d["offsets"][-1] and np.all(np.diff(off) == cnt)
    assert np.array_equal(cnt, d["counts"].reshape(N, E // N).sum(axis=1))
    if N == E:
        assert np.array_equal(cnt, d["counts"])


def test_send_rows_belong_to_their_rank_and_token():
    # every row in rank n's block is the hidden state of a token that routed
    # to one of rank n's experts; each token appears once per valid slot
    rng = np.random.default_rng(3)
    E, N, T, k, dd = 16, 4, 120, 3, 5
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    ids[rng.random((T, k)) < 0.1] = -1
    x = (np.arange(T, dtype=np.float32)[:, None] * 10 + np.arange(dd, dtype=np.float32))
    d = oracle.dispatch(ids, E)
    cnt, off = oracle.ep_layout(d["offsets"], N)
    rows = oracle.permute_rows(x, d["perm"], k)
    tok = (rows[:, 0] // 10).astype(int)
    flat = ids.reshape(-1)
    for n in range(N):
        for p in range(off[n], off[n + 1]):
            r = d["perm"][p]
            assert tok[p] == r // k and n * E // N <= flat[r] < (n + 1) * E // N
    assert np.array_equal(np.bincount(tok, minlength=T), (ids >= 0).sum(axis=1))


def test_rank_count_must_divide_the_experts():
    with pytest.raises(ValueError):
        oracle.ep_layout(np.zeros(9, np.int32), 3)
