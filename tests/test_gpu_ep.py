"""GPU parity of the expert-parallel send layout (moe_ep_layout) and the send
buffer (moe_permute_rows) with the oracle, bit for bit: the rows are copies
and the layout is integer arithmetic."""
import numpy as np
import pytest
import torch

import oracle
import token_dispatch_amd as tda
import workloads as wl
from tests.gpu_util import down, say, up

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    tda.lib()


def as_dtype(a32, dtype):
    return wl.f32_to_bf16_bits(a32) if dtype == "bf16" else a32.astype(np.float32)


def to_f64(a):
    return wl.bf16_bits_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


def placed_rows(x, places, k, n_rows):
    """The oracle's rows for a placement: route r at row places[r]; returns
    (rows placed at, their expected contents)."""
    r = np.flatnonzero((places >= 0) & (places < n_rows)).astype(np.int32)
    order = np.argsort(places[r], kind="stable")
    return places[r][order], oracle.permute_rows(x, r[order], k)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T,k,E,d", [(1, 1, 1, 8), (300, 2, 16, 64), (2000, 8, 128, 2048),
                                     (333, 4, 384, 2880), (97, 3, 40, 100), (50, 6, 24, 7),
                                     (40, 70, 64, 1100), (5, 1, 8, 7168)])
def test_permute_rows(dtype, T, k, E, d):
    """Dispatch order: out[p] = x[perm[p] // k] (the oracle's definition, on
    the GPU's perm), written by the kernel from inv; rows past R untouched.
    Covers k above one wavefront of places and rows of one to four chunks
    with a ragged last one."""
    rng = np.random.default_rng([T, k, E, d])
    ids = rng.integers(-1, E, size=(T, k)).astype(np.int32)
    x = as_dtype(rng.standard_normal((T, d)).astype(np.float32), dtype)
    say("permute", dtype, T, k, E, d)
    _, offsets, perm, inv = tda.dispatch(up(ids), E)
    xt = up(x)
    out = torch.full((T * k, d), 7.0, dtype=xt.dtype, device=DEV)  # rows past R stay 7
    tda.permute_rows(xt, inv, k, T * k, out=out)
    torch.cuda.synchronize()
    R = int(offsets[-1].item())
    got = down(out.view(torch.int16)).view(np.uint16) if dtype == "bf16" else down(out)
    ref = oracle.permute_rows(x, down(perm)[:R], k)
    assert np.array_equal(to_f64(got[:R]), ref)
    assert np.all(to_f64(got[R:]) == 7.0)


@pytest.mark.parametrize("T,k,E,C", [(4096, 1, 128, 40), (1000, 2, 16, 100), (300, 4, 8, 1)])
def test_permute_rows_capacity_slots(T, k, E, C):
    """Expert-major rows [E*C][d] from the capacity limit's slots: kept
    routes' rows at e*C + rank (the oracle's capacity rule), other rows
    untouched, dropped routes nowhere."""
    d = 256
    rng = np.random.default_rng([T, k, E, C])
    ids = ((rng.zipf(1.4, size=(T, k)) - 1) % E).astype(np.int32)
    x = wl.f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    say("permute capacity", T, k, E, C)
    _, offsets, _, inv = tda.dispatch(up(ids), E)
    slot, _, _ = tda.dispatch_capacity(up(ids), E, C, offsets, inv)
    out = torch.zeros((E * C, d), dtype=torch.bfloat16, device=DEV)
    tda.permute_rows(up(x), slot, k, E * C, out=out)
    torch.cuda.synchronize()
    ref_slot = oracle.capacity(ids, E, C)["slot"]
    rows, ref = placed_rows(x, ref_slot.reshape(-1), k, E * C)
    got = down(out.view(torch.int16)).view(np.uint16)
    assert np.array_equal(to_f64(got[rows]), ref)
    rest = np.setdiff1d(np.arange(E * C), rows)
    assert np.all(got[rest] == 0)


def test_permute_unaligned_empty_and_errors():
    rng = np.random.default_rng(5)
    T, k, E, d = 64, 2, 8, 64
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    x = wl.f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    _, offsets, perm, inv = tda.dispatch(up(ids), E)
    big = up(np.concatenate([x.reshape(-1)[:1], x.reshape(-1)]))
    xu = big[1:].view(T, d)  # the same rows, 2 bytes off alignment: element copies
    say("permute unaligned")
    a = tda.permute_rows(up(x), inv, k, T * k)
    b = tda.permute_rows(xu, inv, k, T * k)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    # places past out_rows are counted and skipped
    places = np.arange(T * k, dtype=np.int32)[::-1].copy()
    places[::5] = -1
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    n_rows = 50
    say("permute out of range")
    c = torch.zeros((n_rows, d), dtype=torch.bfloat16, device=DEV)
    tda.permute_rows(up(x), up(places), k, n_rows, out=c, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == int(np.sum(places >= n_rows))
    rows, ref = placed_rows(x, places, k, n_rows)
    got = down(c.view(torch.int16)).view(np.uint16)
    assert np.array_equal(to_f64(got[rows]), ref)
    e = tda.permute_rows(torch.empty((0, 16), device=DEV),
                         torch.empty(0, dtype=torch.int32, device=DEV), 2, 0)
    assert e.shape == (0, 16)


@pytest.mark.parametrize("E,N", [(8, 1), (8, 2), (128, 8), (384, 8), (256, 256), (1024, 16)])
def test_ep_layout(E, N):
    rng = np.random.default_rng([E, N])
    T, k = 3000, 4
    ids = ((rng.zipf(1.3, size=(T, k)) - 1) % E).astype(np.int32)
    ids[rng.random((T, k)) < 0.05] = -1
    _, offsets, _, _ = tda.dispatch(up(ids), E)
    say("ep layout", E, N)
    cnt, off = tda.ep_layout(offsets, N)
    torch.cuda.synchronize()
    rc, ro = oracle.ep_layout(down(offsets), N)
    assert np.array_equal(down(cnt), rc) and np.array_equal(down(off), ro)


def test_ep_send_buffer_full_size():
    """Qwen3-like routes at full size: the send buffer checked on a sample of
    rows (the oracle's copy of each sampled route's token row), the layout
    bit for bit, over 8 ranks."""
    w = wl.WORKLOADS["qwen3_dynk"]
    T, k, E, d = w.T, w.k, w.E, w.d
    rng = np.random.default_rng(12)
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    kt = wl.request_k(0, T, w.dynamic_k, w.request_len)
    ids[np.arange(k)[None, :] >= kt[:, None]] = -1
    x = wl.make_inputs(w)["x"]
    _, offsets, perm, inv = tda.dispatch(up(ids), E)
    say("send buffer full size", T, k, d)
    out = tda.permute_rows(up(x), inv, k, T * k)
    cnt, off = tda.ep_layout(offsets, 8)
    torch.cuda.synchronize()
    R = int(offsets[-1].item())
    pick = np.sort(rng.choice(R, size=256, replace=False))
    got = down(out.view(torch.int16)).view(np.uint16)[pick]
    ref = oracle.permute_rows(x, down(perm)[pick], k)
    assert np.array_equal(to_f64(got), ref)
    rc, ro = oracle.ep_layout(down(offsets), 8)
    assert np.array_equal(down(cnt), rc) and np.array_equal(down(off), ro)


def test_row_movement_two_million_routes():
    """2.1 M routes (T = 262144, k = 8, E = 384): capacity slots, kept and
    dropped counts and the per-rank layout bit for bit, the send buffer on
    sampled rows."""
    T, k, E, d = 262144, 8, 384, 64
    rng = np.random.default_rng(41)
    ids = ((rng.zipf(1.2, size=(T, k)) - 1) % E).astype(np.int32)
    ids[rng.random((T, k)) < 0.02] = -1
    x = wl.f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    C = int(np.ceil(1.25 * T * k / E))
    say("row movement, 2.1 M routes")
    _, offsets, perm, inv = tda.dispatch(up(ids), E)
    slot, kept, dropped = tda.dispatch_capacity(up(ids), E, C, offsets, inv)
    out = tda.permute_rows(up(x), inv, k, T * k)
    cnt, off = tda.ep_layout(offsets, 16)
    torch.cuda.synchronize()
    rc = oracle.capacity(ids, E, C)
    assert np.array_equal(down(slot), rc["slot"]) and np.array_equal(down(kept), rc["kept"])
    assert int(dropped.item()) == rc["dropped"] > 0
    ro, rf = oracle.ep_layout(down(offsets), 16)
    assert np.array_equal(down(cnt), ro) and np.array_equal(down(off), rf)
    R = int(offsets[-1].item())
    pick = np.sort(rng.choice(R, size=512, replace=False))
    got = down(out.view(torch.int16)).view(np.uint16)[pick]
    assert np.array_equal(to_f64(got), oracle.permute_rows(x, down(perm)[pick], k))
