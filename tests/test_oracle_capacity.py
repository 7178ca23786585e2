"""Pins of the oracle's capacity-limited dispatch (CPU).  The router survey
page names top-1 routing with a Switch-style capacity and gives no rule; the
reading taken: each expert keeps its first C routes in route order (the
order of the stable dispatch) and drops the rest; a kept route of expert e
with rank q goes to slot e*C + q.  The pages print no example, so the pins
are a hand-worked case, special cases and invariants."""
import numpy as np
import pytest

import oracle


def test_hand_case():
    # routes r = 0..7 (T = 4, k = 2): experts [2,0, 2,1, 2,2, -1,0]; C = 2
    ids = np.array([[2, 0], [2, 1], [2, 2], [-1, 0]], np.int32)
    out = oracle.capacity(ids, 3, 2)
    # expert 0: routes 1, 7 -> slots 0, 1; expert 1: route 3 -> slot 2;
    # expert 2: routes 0, 2 -> slots 4, 5, routes 4, 5 dropped
    assert out["slot"].tolist() == [4, 0, 5, 2, -1, -1, -1, 1]
    assert out["kept"].tolist() == [2, 1, 2]
    assert out["dropped"] == 2


@pytest.mark.parametrize("k,E", [(1, 8), (2, 16), (4, 128)])
def test_large_capacity_is_the_dispatch_rank(k, E):
    # with room for every route nothing is dropped and each route's slot is
    # its expert's block start plus its rank, the stable dispatch's position
    rng = np.random.default_rng(k * E)
    T = 300
    ids = rng.integers(-1, E, size=(T, k)).astype(np.int32)
    d = oracle.dispatch(ids, E)
    C = int(d["counts"].max())
    out = oracle.capacity(ids, E, C)
    flat = ids.reshape(-1)
    want = np.where(flat >= 0, flat * C + (d["inv"] - d["offsets"][np.maximum(flat, 0)]), -1)
    assert np.array_equal(out["slot"], want)
    assert np.array_equal(out["kept"], d["counts"]) and out["dropped"] == 0


def test_zero_capacity_drops_every_route():
    ids = np.array([[0, 1], [1, -1], [2, 0]], np.int32)
    out = oracle.capacity(ids, 4, 0)
    assert np.all(out["slot"] == -1) and out["kept"].tolist() == [0, 0, 0, 0]
    assert out["dropped"] == 5


@pytest.mark.parametrize("C", [1, 3, 17])
def test_invariants_on_skewed_routes(C):
    # kept + dropped = valid routes; kept slots are distinct, inside e's
    # block of C; the kept routes of an expert are its first routes in r
    rng = np.random.default_rng(C)
    T, k, E = 500, 2, 16
    ids = ((rng.zipf(1.5, size=(T, k)) - 1) % E).astype(np.int32)
    ids[rng.random((T, k)) < 0.05] = -1
    ids[7, 1] = 99  # an error: not a route
    out = oracle.capacity(ids, E, C)
    flat = ids.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    kept_mask = out["slot"] >= 0
    assert out["kept"].sum() + out["dropped"] == valid.sum() == kept_mask.sum() + out["dropped"]
    s = out["slot"][kept_mask]
    assert len(np.unique(s)) == len(s)
    assert np.all(s // C == flat[kept_mask])
    for e in range(E):
        r_e = np.nonzero(flat == e)[0]
        assert np.array_equal(np.nonzero(kept_mask & (flat == e))[0], r_e[:C])
        assert out["kept"][e] == min(len(r_e), C)
