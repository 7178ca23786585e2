"""GPU parity of moe_dispatch_capacity with the oracle (bit-exact slots,
kept counts and dropped count): each expert keeps its first C routes in
route order (the reading taken of the router survey's Switch-style
capacity, which states no rule)."""
import numpy as np
import pytest
import torch

import oracle
import token_dispatch_amd as tda
import workloads as wl
from tests.gpu_util import down, route_kwargs, say, up

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    tda.lib()


def capacity_case(ids, E, C):
    _, offsets, _, inv = tda.dispatch(up(ids), E)
    slot, kept, dropped = tda.dispatch_capacity(up(ids), E, C, offsets, inv)
    torch.cuda.synchronize()
    ref = oracle.capacity(ids, E, C)
    assert np.array_equal(down(slot), ref["slot"])
    assert np.array_equal(down(kept), ref["kept"])
    assert int(dropped.item()) == ref["dropped"]
    return slot, ref


@pytest.mark.parametrize("T,k,E,C", [(1, 1, 1, 0), (1, 1, 1, 1), (300, 1, 8, 10),
                                     (5000, 1, 128, 50), (4000, 2, 16, 300), (20000, 1, 128, 160),
                                     (777, 4, 384, 3), (3000, 8, 1024, 1)])
def test_capacity_random(T, k, E, C):
    rng = np.random.default_rng([T, k, E, C])
    ids = ((rng.zipf(1.4, size=(T, k)) - 1) % E).astype(np.int32)
    ids[rng.random((T, k)) < 0.05] = -1
    if T > 10:
        ids[3, 0] = E + 5  # an error: not a route, slot -1
    say("capacity", T, k, E, C)
    capacity_case(ids, E, C)


def test_capacity_empty():
    ids = torch.empty((0, 2), dtype=torch.int32, device=DEV)
    offsets = torch.zeros(9, dtype=torch.int32, device=DEV)
    inv = torch.empty(0, dtype=torch.int32, device=DEV)
    slot, kept, dropped = tda.dispatch_capacity(ids, 8, 4, offsets, inv)
    torch.cuda.synchronize()
    assert slot.numel() == 0 and int(kept.sum().item()) == 0 and int(dropped.item()) == 0


@pytest.mark.parametrize("T", [3000, None])
def test_switch_top1_route_capacity_combine(T):
    """Top-1 routing, the capacity limit and the combine over the [E*C][d]
    expert buffer: slots from the GPU's own ids, bit for bit the oracle's;
    the combine within its bound (rows of dropped routes are left out)."""
    w = wl.WORKLOADS["switch_top1"]
    if T is not None:
        w = w.with_T(T)
    C = wl.capacity(w)
    inp = wl.make_inputs(w)
    kw = route_kwargs(w)
    kw.pop("group_score")
    say("switch top-1", w.T, "C", C)
    ids, wts, counts, offsets, perm, inv = tda.route_dispatch(up(inp["x"]), up(inp["W"]), w.k,
                                                              **kw)
    slot, kept, dropped = tda.dispatch_capacity(ids, w.E, C, offsets, inv)
    torch.cuda.synchronize()
    gids = down(ids)
    ref = oracle.capacity(gids, w.E, C)
    assert np.array_equal(down(slot), ref["slot"]) and np.array_equal(down(kept), ref["kept"])
    assert int(dropped.item()) == ref["dropped"]
    if T is None:
        return
    Y = wl.expert_outputs(w, w.E * C)  # the experts' rows, [E*C][d]
    y = tda.combine(up(Y), slot, wts)
    torch.cuda.synchronize()
    out = down(y.view(torch.int16)).view(np.uint16)
    exact, nerr = oracle.combine(Y, ref["slot"].reshape(w.T, w.k), down(wts))
    assert nerr == 0
    got = wl.bf16_bits_to_f32(out).astype(np.float64)
    S, _ = oracle.combine(np.abs(wl.bf16_bits_to_f32(Y)), ref["slot"].reshape(w.T, w.k),
                          np.abs(down(wts)))
    delta = 3 * 2.0 ** -24 * S
    assert np.all(np.abs(got - exact) <= delta + 2.0 ** -8 * (np.abs(exact) + delta) + 1e-30)
