"""GPU parity of moe_combine with the oracle: y[t] = sum_j w[t][j] *
Yp[inv[t][j]] (+ shared[t]).

Bar (derived from the arithmetic, the pages fix no precision): the kernel
adds k_t + 1 terms in fp32 in slot order, so it is within (k + 2) * 2^-24 *
S of the exact sum, S = sum_j |w_j Y_j| + |shared| (the oracle evaluated on
absolute values); a bf16 result adds at most half an ulp, 2^-8 of its
magnitude.  Integer-valued inputs with dyadic weights make every partial sum
exact, and there the result must be bit for bit the oracle's."""
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


def to_f64(a):
    return wl.bf16_bits_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


def as_dtype(a32, dtype):
    return wl.f32_to_bf16_bits(a32) if dtype == "bf16" else a32.astype(np.float32)


def check_combine(y_gpu, Yp, inv, w, shared, k):
    """Element-wise bar against the oracle (see the module docstring)."""
    exact, nerr = oracle.combine(Yp, inv, w, shared)
    absY = np.abs(to_f64(Yp)).astype(np.float32)
    absS = None if shared is None else np.abs(to_f64(shared)).astype(np.float32)
    S, _ = oracle.combine(absY, inv, np.abs(w), absS)
    delta = (k + 2) * 2.0 ** -24 * S
    got = to_f64(y_gpu)
    tol = delta + (2.0 ** -8 * (np.abs(exact) + delta) if Yp.dtype == np.uint16 else 0.0)
    err = np.abs(got - exact)
    assert np.all(err <= tol + 1e-30), (float(err.max()), float((err - tol).max()))
    return exact, nerr


def rand_case(rng, T, k, R, d, dtype, empty=0.2):
    Yp = as_dtype(rng.standard_normal((R, d)).astype(np.float32), dtype)
    inv = rng.integers(0, R, size=(T, k)).astype(np.int32)
    inv[rng.random((T, k)) < empty] = -1
    w = rng.random((T, k)).astype(np.float32)
    return Yp, inv, w


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shared", [False, True], ids=["routed", "routed+shared"])
@pytest.mark.parametrize("T,k,R,d", [(1, 1, 1, 8), (37, 2, 50, 64), (130, 8, 700, 2048),
                                     (61, 16, 400, 2880), (9, 32, 300, 1000),
                                     (21, 4, 90, 100), (5, 3, 7, 7), (13, 2, 40, 2056),
                                     (17, 3, 60, 2888), (9, 1, 20, 4104), (6, 5, 30, 520)])
def test_combine_random(dtype, shared, T, k, R, d):
    """Several 16-byte passes per row, ragged rows (scalar units), every k;
    k <= 2 and k <= 4 (4 and 2 units per lane) with a ragged last chunk."""
    rng = np.random.default_rng([T, k, R, d])
    Yp, inv, w = rand_case(rng, T, k, R, d, dtype)
    sh = as_dtype(rng.standard_normal((T, d)).astype(np.float32), dtype) if shared else None
    say("combine", dtype, shared, T, k, R, d)
    y = tda.combine(up(Yp), up(inv), up(w), shared=up(sh))
    torch.cuda.synchronize()
    out = down(y.view(torch.int16)).view(np.uint16) if dtype == "bf16" else down(y)
    check_combine(out, Yp, inv, w, sh, k)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_combine_exact_on_integers(dtype):
    """Small integers and dyadic weights: every partial sum is exact, so the
    kernel's result equals the oracle's bit for bit."""
    rng = np.random.default_rng(3)
    T, k, R, d = 200, 6, 500, 256
    Yp = as_dtype(rng.integers(-8, 9, size=(R, d)).astype(np.float32), dtype)
    sh = as_dtype(rng.integers(-8, 9, size=(T, d)).astype(np.float32), dtype)
    inv = rng.integers(-1, R, size=(T, k)).astype(np.int32)
    w = rng.choice(np.array([0.25, 0.5, 1.0, 2.0], np.float32), size=(T, k))
    say("combine exact", dtype)
    y = tda.combine(up(Yp), up(inv), up(w), shared=up(sh))
    torch.cuda.synchronize()
    out = down(y.view(torch.int16)).view(np.uint16) if dtype == "bf16" else down(y)
    exact, _ = oracle.combine(Yp, inv, w, sh)
    assert np.array_equal(to_f64(out), exact)


def test_combine_errors_empty_slots_and_unaligned():
    rng = np.random.default_rng(4)
    T, k, R, d = 40, 4, 30, 64
    Yp, inv, w = rand_case(rng, T, k, R, d, "bf16")
    inv[0] = -1           # a token with no routed slot: y = shared
    inv[1, 2] = R         # no such row: counted, left out
    inv[2, 0] = R + 1000
    sh = as_dtype(rng.standard_normal((T, d)).astype(np.float32), "bf16")
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    say("combine errors")
    y = tda.combine(up(Yp), up(inv), up(w), shared=up(sh), dev_err=err)
    torch.cuda.synchronize()
    out = down(y.view(torch.int16)).view(np.uint16)
    _, nerr = check_combine(out, Yp, inv, w, sh, k)
    assert int(err.item()) == nerr == 2
    assert np.array_equal(out[0], sh[0])
    # rows that start off a 16-byte boundary take the one-element units
    big = up(np.concatenate([Yp.reshape(-1)[:1], Yp.reshape(-1)]))
    Yu = big[1:].view(R, d)  # the same rows, 2 bytes off alignment
    say("combine unaligned")
    y2 = tda.combine(Yu, up(inv), up(w), shared=up(sh))
    torch.cuda.synchronize()
    assert torch.equal(y2, y)


def test_combine_empty_shapes():
    w = torch.zeros((0, 4), dtype=torch.float32, device=DEV)
    inv = torch.zeros(0, dtype=torch.int32, device=DEV)
    Yp = torch.zeros((0, 16), dtype=torch.bfloat16, device=DEV)
    assert tda.combine(Yp, inv, w).shape == (0, 16)
    # R = 0: every slot is an error or empty; y is the shared output
    T, k, d = 5, 2, 16
    inv = torch.full((T * k,), -1, dtype=torch.int32, device=DEV)
    inv[3] = 0
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    sh = torch.randn((T, d), device=DEV).to(torch.bfloat16)
    y = tda.combine(Yp, inv, torch.ones((T, k), device=DEV), shared=sh, dev_err=err)
    torch.cuda.synchronize()
    assert torch.equal(y, sh) and int(err.item()) == 1


@pytest.mark.parametrize("name,T", [("qwen3_dynk", 1000), ("gptoss_skew", 700),
                                    ("dsv3_grouped", 300), ("mixtral", None)])
def test_combine_after_route_dispatch(name, T):
    """The layer round trip: route + dispatch on the GPU, expert outputs in
    dispatch order, then combine; checked against the oracle on the GPU's
    own inv and weights."""
    w = wl.WORKLOADS[name]
    inp = wl.make_inputs(w, T=T)
    Tn = inp["x"].shape[0]
    kw = route_kwargs(w)
    if kw["group_score"] is None:
        kw.pop("group_score")
    say("route_dispatch + combine", name, Tn)
    ids, wts, counts, offsets, perm, inv = tda.route_dispatch(
        up(inp["x"]), up(inp["W"]), w.k, logit_bias=up(inp["logit_bias"]),
        select_bias=up(inp["select_bias"]), k_per_token=up(inp["k_per_token"]), **kw)
    R = int(offsets[-1].item())
    Yp = wl.expert_outputs(w, R)
    sh = wl.shared_output(w, T=Tn)
    y = tda.combine(up(Yp), inv, wts, shared=up(sh))
    torch.cuda.synchronize()
    out = down(y.view(torch.int16)).view(np.uint16) if w.dtype == "bf16" else down(y)
    check_combine(out, Yp, down(inv).reshape(Tn, w.k), down(wts), sh, w.k)


@pytest.mark.parametrize("name,T", [("qwen3_dynk", None), ("gptoss_skew", 8192)])
def test_combine_full_size_sampled(name, T):
    """Full-size combine (the Qwen3-like shape the benchmark times; the
    gpt-oss-like rows at 8192 tokens); the oracle checks a sample of tokens,
    with the GPU's own dispatch inverse."""
    w = wl.WORKLOADS[name] if T is None else wl.WORKLOADS[name].with_T(T)
    T, k = w.T, w.k
    rng = np.random.default_rng(9)
    ids = rng.integers(0, w.E, size=(T, k)).astype(np.int32)
    if w.dynamic_k:
        kt = wl.request_k(0, T, w.dynamic_k, w.request_len)
        ids[np.arange(k)[None, :] >= kt[:, None]] = -1
    wts = rng.random((T, k)).astype(np.float32)
    _, offsets, _, inv = tda.dispatch(up(ids), w.E)
    R = int(offsets[-1].item())
    Yp = wl.expert_outputs(w, R)
    sh = wl.shared_output(w)
    say("combine full size", name, T, R, w.d)
    y = tda.combine(up(Yp), inv, up(wts), shared=up(sh))
    torch.cuda.synchronize()
    pick = np.sort(rng.choice(T, size=64, replace=False))
    inv_np = down(inv).reshape(T, k)
    out = down(y.view(torch.int16)).view(np.uint16)[pick]
    check_combine(out, Yp, inv_np[pick], wts[pick], wl.rows(sh, pick), k)


def test_identity_experts_round_trip_full_size():
    """Route + dispatch (Qwen3-like, full size), the send buffer as the
    experts' outputs (identity experts), then the combine with dyadic
    weights: with x small integers every sum is exact, so at every token
    y = (sum of the token's weights) * x, bit for bit."""
    w = wl.WORKLOADS["qwen3_dynk"]
    T, k, d = w.T, w.k, w.d
    rng = np.random.default_rng(17)
    x = wl.f32_to_bf16_bits(rng.integers(-4, 5, size=(T, d)).astype(np.float32))
    Wt = wl.make_inputs(w)["W"]
    kt = wl.request_k(0, T, w.dynamic_k, w.request_len)
    say("identity experts round trip", T, k, d)
    ids, _, _, offsets, _, inv = tda.route_dispatch(up(x), up(Wt), k, k_per_token=up(kt))
    R = int(offsets[-1].item())
    send = tda.permute_rows(up(x), inv, k, R)
    wts = rng.choice(np.array([0.5, 1.0], np.float32), size=(T, k))
    y = tda.combine(send, inv, up(wts))
    torch.cuda.synchronize()
    valid = down(inv).reshape(T, k) >= 0
    assert np.array_equal(valid.sum(axis=1), kt)
    wsum = np.where(valid, wts, 0).sum(axis=1).astype(np.float64)
    want = wsum[:, None] * wl.bf16_bits_to_f32(x).astype(np.float64)
    got = to_f64(down(y.view(torch.int16)).view(np.uint16))
    assert np.array_equal(got, want)
