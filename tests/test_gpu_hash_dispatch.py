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


@pytest.mark.parametrize("T,d,E,k,bad,slice_", [
    (77, 104, 24, 5, True, None),       # one slice wider than d (zero-filled), ragged T
    (1000, 7168, 384, 6, False, None),  # DeepSeek-V4-like rows: 38 slices of 192 columns,
                                        # the last one 64 wide
    (1000, 7168, 384, 6, False, "128"),  # 56 slices of 128 columns
    (2000, 2880, 128, 4, True, None),   # k = 4 compiled in (192-column slices)
    (900, 2880, 200, 5, True, None),    # k only at run time (192-column slices)
    (500, 1000, 500, 8, True, None),    # 64-column slices (E > 384), a partial last slice
    (500, 1000, 300, 8, True, "64"),    # 64-column slices below 384 experts
    (70000, 200, 64, 3, False, None),   # 2 slices (the second 8 wide) x 128 token chunks
    (3001, 256, 768, 1, False, None),   # the largest E of the kernel, k = 1
    (5, 64, 8, 8, True, None),          # fewer tokens than one wavefront's tile
])
def test_hash_dot_products_against_gate_path(T, d, E, k, bad, slice_, monkeypatch):
    """The hash layer's k dot products per token (W slices on chip, partial
    sums added in slice order) against the tiled gate contraction of every
    expert (MOE_HASH_DENSE) and the oracle: ids bit for bit, weights within
    2e-5 of each other and 1e-4 of the oracle, with a logit bias, duplicate
    table entries, and bad token ids and table entries."""
    rng = np.random.default_rng([T, d, E, k])
    V = 97
    tab = rng.integers(0, E, size=(V, k)).astype(np.int32)
    tok = rng.integers(0, V, size=T).astype(np.int32)
    if bad:
        tok[rng.choice(T, min(T, 3), replace=False)] = [-1, V, V + 5][:min(T, 3)]
        tab[rng.integers(0, V, 3), rng.integers(0, k, 3)] = [E, -3, E + 7]
    x = wl.f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    W = wl.f32_to_bf16_bits((rng.standard_normal((E, d)) / np.sqrt(d)).astype(np.float32))
    lb = (0.3 * rng.standard_normal(E)).astype(np.float32)
    say("hash dot products", T, d, E, k, bad, slice_)
    if slice_:
        monkeypatch.setenv("MOE_HASH_SLICE", slice_)
    outs = []
    for dense in (False, True):
        if dense:
            monkeypatch.setenv("MOE_HASH_DENSE", "1")
        err = torch.zeros(1, dtype=torch.int32, device=DEV)
        ids, wts = tda.route_hash(up(tok), up(tab), E, x=up(x), W=up(W), score="sqrt_softplus",
                                  logit_bias=up(lb), route_scale=1.5, dev_err=err)
        torch.cuda.synchronize()
        outs.append((down(ids), down(wts), int(err.item())))
    monkeypatch.delenv("MOE_HASH_DENSE")
    (ia, wa, ea), (ib, wb, eb) = outs
    ref_ids, nerr = oracle.hash_ids(tok, tab, E)
    np.testing.assert_array_equal(ia, ref_ids)
    np.testing.assert_array_equal(ib, ref_ids)
    assert ea == eb == nerr
    assert np.max(np.abs(wa - wb)) <= 2e-5
    ref_w = oracle.weights_for_ids(oracle.gate(x, W, lb), ref_ids, score="sqrt_softplus",
                                   route_scale=1.5)
    assert np.max(np.abs(wa - ref_w)) <= WTOL


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


@pytest.mark.parametrize("T,d,E,k,V,bad", [
    (16384, 7168, 384, 6, 129280, False),  # the DeepSeek-V4-like hash layer, full size
    (1000, 256, 384, 6, 5000, True),       # bad token ids and table entries
    (777, 64, 8, 1, 50, True),             # k = 1 (4-lane segments)
    (3001, 128, 100, 9, 700, False),       # 16-lane segments, E not a multiple of 8
    (513, 64, 1000, 17, 300, True),        # one token per wavefront, 10-bit ids
    (200, 32, 64, 32, 90, False),          # k = 32, duplicates in the table
])
def test_hash_dispatch_matches_separate_calls(T, d, E, k, V, bad):
    """moe_route_hash_dispatch (the hash kernel counting the dispatch tiles)
    equals moe_route_hash + moe_dispatch bit for bit, error counts included,
    and the oracle's ids and dispatch."""
    rng = np.random.default_rng([T, E, k])
    if k <= E and not (E == 64 and k == 32):
        tab = np.argsort(rng.random((V, E)), axis=1)[:, :k].astype(np.int32)
    else:
        tab = rng.integers(0, E, size=(V, k)).astype(np.int32)  # duplicates allowed
    tok = rng.integers(0, V, size=T).astype(np.int32)
    if bad:
        tok[rng.choice(T, 5, replace=False)] = rng.choice([-1, V, V + 3], 5)
        tab[rng.choice(V, 7, replace=False), rng.integers(0, k, 7)] = rng.choice([-2, E, E + 9], 7)
    x = wl.f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    W = wl.f32_to_bf16_bits((rng.standard_normal((E, d)) / np.sqrt(d)).astype(np.float32))
    say("hash dispatch", T, d, E, k, V, bad)
    e1 = torch.zeros(1, dtype=torch.int32, device=DEV)
    e2 = torch.zeros(1, dtype=torch.int32, device=DEV)
    m1 = torch.zeros(1, dtype=torch.float64, device=DEV)
    m2 = torch.zeros(1, dtype=torch.float64, device=DEV)
    a = tda.route_hash_dispatch(up(tok), up(tab), E, x=up(x), W=up(W), maxvio=m1, dev_err=e1)
    ids, wts = tda.route_hash(up(tok), up(tab), E, x=up(x), W=up(W), dev_err=e2)
    b = (ids, wts) + tuple(tda.dispatch(ids, E, maxvio=m2))
    torch.cuda.synchronize()
    n = int(a[3][-1].item())
    for name, u, v in zip(("ids", "weights", "counts", "offsets", "perm", "inv"), a, b):
        if name == "perm":
            u, v = u[:n], v[:n]
        assert torch.equal(u, v), name
    assert int(e1.item()) == int(e2.item()) and torch.equal(m1, m2)
    ref_ids, nerr = oracle.hash_ids(tok, tab, E)
    assert nerr == int(e1.item())
    np.testing.assert_array_equal(down(a[0]), ref_ids)
    d_ref = oracle.dispatch(ref_ids, E)
    check_dispatch(tuple(a[2:]), d_ref)
    assert float(m1.item()) == oracle.maxvio(d_ref["counts"])


@pytest.mark.parametrize("T,d,E,k,V,bad", [
    (3001, 7168, 384, 6, 9000, True),     # 228 slice workgroups + 28 placement, ragged tiles
    (20000, 7168, 384, 8, 30000, False),  # 79 tiles on 28 placement workgroups (3 rounds)
    (5000, 1024, 64, 8, 3000, False),     # a partial last slice, 20 tiles, 20 workgroups
    (2000, 512, 640, 5, 800, True),       # 64-column slices of 640 experts
    (700, 256, 128, 1, 100, False),       # k = 1, one tile
    (4096, 2048, 96, 7, 5000, True),      # odd k, E a multiple of 8 below 128
    (3000, 1024, 100, 6, 2000, False),    # E not a multiple of 8
])
def test_hash_dispatch_beside_the_dot_products(T, d, E, k, V, bad, monkeypatch):
    """The dispatch placed by the dot-product kernel's free workgroups
    (MOE_HASH_BESIDE=1) equals the placement kernel after the hash kernel
    (MOE_HASH_BESIDE=0) bit for bit -- ids, weights, counts, offsets, perm,
    inv, MaxVio and the error count -- and the oracle's ids and dispatch."""
    rng = np.random.default_rng([T, d, E, k])
    tab = np.argsort(rng.random((V, E)), axis=1)[:, :k].astype(np.int32)
    tok = rng.integers(0, V, size=T).astype(np.int32)
    if bad:
        tok[rng.choice(T, 5, replace=False)] = rng.choice([-1, V, V + 3], 5)
        tab[rng.choice(V, 7, replace=False), rng.integers(0, k, 7)] = rng.choice([-2, E, E + 9], 7)
    x = wl.f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    W = wl.f32_to_bf16_bits((rng.standard_normal((E, d)) / np.sqrt(d)).astype(np.float32))
    say("hash dispatch beside the dot products", T, d, E, k, V, bad)
    xg, Wg, tg, tabg = up(x), up(W), up(tok), up(tab)
    res = {}
    for mode in ("1", "0"):
        monkeypatch.setenv("MOE_HASH_BESIDE", mode)
        err = torch.zeros(1, dtype=torch.int32, device=DEV)
        mv = torch.full((1,), -7.0, dtype=torch.float64, device=DEV)
        tda.profile_enable(True)
        out = tda.route_hash_dispatch(tg, tabg, E, x=xg, W=Wg, maxvio=mv, dev_err=err)
        torch.cuda.synchronize()
        stages = {s for s, (_, n) in tda.profile_read().items() if n}
        tda.profile_enable(False)
        res[mode] = (out, err, mv, stages)
    (a, e1, m1, s1), (b, e2, m2, s2) = res["1"], res["0"]
    assert "disp_scatter" not in s1 and "hash_dots" in s1, s1  # placed beside
    assert "disp_scatter" in s2, s2
    n = int(a[3][-1].item())
    for name, u, v in zip(("ids", "weights", "counts", "offsets", "perm", "inv"), a, b):
        if name == "perm":
            u, v = u[:n], v[:n]
        assert torch.equal(u, v), name
    assert int(e1.item()) == int(e2.item()) and torch.equal(m1, m2)
    ref_ids, nerr = oracle.hash_ids(tok, tab, E)
    assert nerr == int(e1.item())
    np.testing.assert_array_equal(down(a[0]), ref_ids)
    d_ref = oracle.dispatch(ref_ids, E)
    check_dispatch(tuple(a[2:]), d_ref)
    assert float(m1.item()) == oracle.maxvio(d_ref["counts"])
