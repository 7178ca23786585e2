"""GPU parity of moe_route_hash and moe_dispatch with the oracle (bit-exact
ids and dispatch arrays; hash weights within 1e-4)."""
import numpy as np
import pytest
import torch

import oracle
import token_dispatch_amd as tda
import workloads as wl
from tests.gpu_util import down, say, up
from tests.parity import WTOL, check_dispatch

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    tda.lib()


# ---- hash routing ------------------------------------------------------------------

def hash_case(w, inp, sample=None):
    say("hash", w.name, "T", inp["token_ids"].shape[0])
    ids, wts = tda.route_hash(up(inp["token_ids"]), up(inp["tid2eid"]), w.E, x=up(inp["x"]),
                              W=up(inp["W"]), score=w.score, renormalize=w.renormalize,
                              route_scale=w.route_scale)
    torch.cuda.synchronize()
    gids, gw = down(ids), down(wts)
    ref_ids, nerr = oracle.hash_ids(inp["token_ids"], inp["tid2eid"], w.E)
    assert nerr == 0
    np.testing.assert_array_equal(gids, ref_ids)
    rows = np.arange(gids.shape[0]) if sample is None else sample
    l64 = oracle.gate(wl.rows(inp["x"], rows), inp["W"])
    ref_w = oracle.weights_for_ids(l64, ref_ids[rows], score=w.score,
                                   renormalize=w.renormalize, route_scale=w.route_scale)
    assert np.max(np.abs(gw[rows] - ref_w)) <= WTOL
    return ids


def test_hash_reduced():
    w = wl.WORKLOADS["dsv4_hash"]
    inp = wl.make_inputs(w, T=300)
    ids = hash_case(w, inp)
    check_dispatch(tda.dispatch(ids, w.E), oracle.dispatch(down(ids), w.E))


def test_hash_full_size_sampled():
    w = wl.WORKLOADS["dsv4_hash"]
    inp = wl.make_inputs(w)
    sample = np.unique(np.random.default_rng(3).choice(w.T, 200, replace=False))
    ids = hash_case(w, inp, sample)
    check_dispatch(tda.dispatch(ids, w.E), oracle.dispatch(down(ids), w.E))


@pytest.mark.parametrize("score", ["sigmoid", "sqrt_softplus", "softmax_topk", "softmax"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("gate", [True, False], ids=["gate-logits", "dot-products"])
def test_hash_scores_ragged_and_duplicates(score, dtype, gate):
    rng = np.random.default_rng([len(score), len(dtype)])
    T, d, E, k, V = 77, 100, 24, 5, 50
    tab = rng.integers(0, E, size=(V, k)).astype(np.int32)  # duplicates allowed
    tok = rng.integers(0, V, size=T).astype(np.int32)
    x = rng.standard_normal((T, d)).astype(np.float32)
    W = (rng.standard_normal((E, d)) / 10).astype(np.float32)
    lb = (0.5 * rng.standard_normal(E)).astype(np.float32)
    if dtype == "bf16":
        x, W = wl.f32_to_bf16_bits(x), wl.f32_to_bf16_bits(W)
    say("hash scores", score, dtype, gate)
    ws = None if gate else torch.empty(0, dtype=torch.uint8, device=DEV)
    ids, wts = tda.route_hash(up(tok), up(tab), E, x=up(x), W=up(W), score=score,
                              logit_bias=up(lb), route_scale=1.5, workspace=ws)
    ref_ids, _ = oracle.hash_ids(tok, tab, E)
    np.testing.assert_array_equal(down(ids), ref_ids)
    ref_w = oracle.weights_for_ids(oracle.gate(x, W, lb), ref_ids, score=score, route_scale=1.5)
    assert np.max(np.abs(down(wts) - ref_w)) <= WTOL


def test_hash_arithmetic_table_and_errors():
    V, k, E = 1000, 6, 384
    tab = ((np.arange(V)[:, None] * k + np.arange(k)[None, :]) % E).astype(np.int32)
    tab[7, 2] = E + 3      # bad entry
    tab[8, 0] = -5         # bad entry
    tok = np.random.default_rng(17).integers(0, V, 500).astype(np.int32)
    tok[:3] = [7, 8, V]    # two bad entries, one bad token id
    tok[3] = -1            # bad token id
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    ids, w = tda.route_hash(up(tok), up(tab), E, dev_err=err)
    assert w is None
    ref, nerr = oracle.hash_ids(tok, tab, E)
    np.testing.assert_array_equal(down(ids), ref)
    assert int(err.item()) == nerr == 4


# ---- dispatch ----------------------------------------------------------------------

def dispatch_case(ids_np, E, with_inv=True):
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = tda.dispatch(up(ids_np), E, with_inv=with_inv, dev_err=err)
    ref = oracle.dispatch(ids_np, E)
    check_dispatch(out, ref)
    assert int(err.item()) == ref["nerr"]
    return out


@pytest.mark.parametrize("T,k,E", [(1, 1, 1), (3, 2, 8), (1023, 1, 8), (1024, 1, 8), (1025, 1, 8),
                                   (4096, 16, 128), (8192, 8, 256), (16384, 6, 384),
                                   (2000, 3, 1024), (65536, 4, 128), (70000, 30, 1024),
                                   # 16-bit histograms: 64 groups of 8 experts, and
                                   # group counts that do not divide a wavefront
                                   (3000, 8, 512), (5000, 3, 40), (50000, 6, 24)])
def test_dispatch_random(T, k, E):
    rng = np.random.default_rng([T, k, E])
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    ids[rng.random((T, k)) < 0.05] = -1
    say("dispatch", T, k, E)
    dispatch_case(ids, E)


def test_dispatch_skew_and_single_expert():
    rng = np.random.default_rng(11)
    T, k, E = 50000, 4, 128
    ids = (rng.zipf(1.3, size=(T, k)) - 1) % E
    dispatch_case(ids.astype(np.int32), E)
    dispatch_case(np.full((3000, 2), 5, np.int32), 8)


def test_dispatch_errors_and_empty():
    ids = np.array([[0, 9], [-1, 3], [12, 0], [2, -7]], np.int32)
    dispatch_case(ids, 8)
    out = dispatch_case(np.full((5, 3), -1, np.int32), 4)
    assert int(down(out[1])[-1]) == 0
    counts, offsets, perm, inv = tda.dispatch(torch.empty((0, 4), dtype=torch.int32, device=DEV), 16)
    assert np.all(down(counts) == 0) and np.all(down(offsets) == 0)


def test_dispatch_without_inv_and_determinism():
    rng = np.random.default_rng(21)
    ids = up(rng.integers(0, 384, size=(16384, 6)).astype(np.int32))
    a = tda.dispatch(ids, 384, with_inv=False)
    b = tda.dispatch(ids, 384, with_inv=True)
    assert a[3] is None
    for u, v in zip(a[:3], b[:3]):
        assert torch.equal(u, v)
    c = tda.dispatch(ids, 384)
    for u, v in zip(b, c):
        assert torch.equal(u, v)
