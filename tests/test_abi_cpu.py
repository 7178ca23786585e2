"""The C-ABI library loads, exports every symbol its header declares, and
rejects bad arguments on the host (no GPU needed: nothing is enqueued)."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

import token_dispatch_amd as tda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_route.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(moe_\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    assert {"moe_route", "moe_route_workspace_size", "moe_route_hash",
            "moe_route_hash_workspace_size", "moe_dispatch", "moe_dispatch_workspace_size",
            "moe_route_dispatch", "moe_route_dispatch_workspace_size", "moe_last_error",
            "moe_abi_version"} <= set(names), names


def test_library_exports_every_declared_symbol():
    lib = tda.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(declared_functions()) <= set(tda.EXPORTS) | {"moe_abi_version"}


def test_abi_version():
    assert tda.lib().moe_abi_version() == tda.ABI_VERSION


def test_header_constants_match_binding():
    src = open(HEADER).read()
    consts = dict(re.findall(r"#define (MOE_\w+) \(?(-?\d+)\)?", src))
    assert int(consts["MOE_ABI_VERSION"]) == tda.ABI_VERSION
    assert int(consts["MOE_MAX_EXPERTS"]) == tda.MAX_EXPERTS
    assert int(consts["MOE_MAX_K"]) == tda.MAX_K
    assert int(consts["MOE_MAX_GROUPS"]) == tda.MAX_GROUPS
    for name, code in tda.SCORES.items():
        assert int(consts["MOE_SCORE_" + name.upper()]) == code
    for name, code in tda.GROUP_SCORES.items():
        assert int(consts["MOE_GROUP_" + name.upper()]) == code
    assert ctypes.sizeof(tda.RouteParams) == 48


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


def call_route(**over):
    kw = dict(T=16, d=64, E=8, k=2, dtype=1, score="softmax", n_groups=1, topk_groups=1,
              group_score="max", renormalize=True, route_scale=1.0)
    kw.update(over)
    p = tda.make_params(**kw)
    return tda.lib().moe_route(ctypes.byref(p), FAKE, FAKE, None, None, None, FAKE, FAKE,
                               FAKE, None, 0, None, None)


@pytest.mark.parametrize("over,code,text", [
    (dict(T=-1), tda.MOE_EINVAL, "T="),
    (dict(d=0), tda.MOE_EINVAL, "d="),
    (dict(E=0), tda.MOE_EINVAL, "E="),
    (dict(E=2048, k=2), tda.MOE_EUNSUPPORTED, "MOE_MAX_EXPERTS"),
    (dict(k=0), tda.MOE_EINVAL, "k="),
    (dict(k=9), tda.MOE_EINVAL, "exceeds E"),
    (dict(E=64, k=33), tda.MOE_EUNSUPPORTED, "MOE_MAX_K"),
    (dict(dtype=7), tda.MOE_EINVAL, "dtype"),
    (dict(n_groups=3), tda.MOE_EINVAL, "does not divide"),
    (dict(n_groups=4, topk_groups=5), tda.MOE_EINVAL, "topk_groups"),
    (dict(n_groups=4, topk_groups=0), tda.MOE_EINVAL, "topk_groups"),
    (dict(n_groups=4, topk_groups=1, k=3), tda.MOE_EINVAL, "kept groups"),
    (dict(n_groups=8, topk_groups=2, group_score="top2_sum"), tda.MOE_EINVAL, "at least 2"),
    (dict(route_scale=float("inf")), tda.MOE_EINVAL, "finite"),
    (dict(E=128, k=4, n_groups=128, topk_groups=4), tda.MOE_EUNSUPPORTED, "MOE_MAX_GROUPS"),
])
def test_route_rejects_bad_params(over, code, text):
    assert call_route(**over) == code
    assert text in tda.lib().moe_last_error().decode()


def test_route_rejects_half_select_only_and_missing_outputs():
    p = tda.make_params(16, 64, 8, 2)
    L = tda.lib()
    assert L.moe_route(ctypes.byref(p), FAKE, None, None, None, None, FAKE, FAKE, FAKE, None, 0,
                       None, None) == tda.MOE_EINVAL
    assert L.moe_route(ctypes.byref(p), None, None, None, None, None, None, FAKE, FAKE, None, 0,
                       None, None) == tda.MOE_EINVAL
    assert L.moe_route(ctypes.byref(p), FAKE, FAKE, None, None, None, FAKE, None, FAKE, None, 0,
                       None, None) == tda.MOE_EINVAL
    assert L.moe_route(None, FAKE, FAKE, None, None, None, FAKE, FAKE, FAKE, None, 0,
                       None, None) == tda.MOE_EINVAL
    # neither logits nor enough workspace for the gate hand-off
    assert L.moe_route(ctypes.byref(p), FAKE, FAKE, None, None, None, None, FAKE, FAKE, FAKE, 16,
                       None, None) == tda.MOE_EINVAL
    assert "workspace" in L.moe_last_error().decode()


def test_route_T0_is_a_noop():
    p = tda.make_params(0, 64, 8, 2)
    assert tda.lib().moe_route(ctypes.byref(p), FAKE, FAKE, None, None, None, None, None, None,
                               None, 0, None, None) == tda.MOE_OK
    assert tda.route_workspace_size(0, 64, 8, 2) == 0


def test_route_workspace_size_covers_the_hand_off():
    # at least one fp32 logit per (token, expert); a multiple of it (K split)
    for T, d, E, k in [(4096, 2048, 128, 16), (8192, 7168, 256, 8), (256, 1024, 8, 2),
                       (65536, 2880, 128, 4), (5, 7, 3, 1)]:
        n = tda.route_workspace_size(T, d, E, k)
        assert n >= T * E * 4 and n % (T * E * 4) == 0 and n // (T * E * 4) <= 8


def test_route_hash_validation():
    L = tda.lib()
    p = tda.make_params(4, 64, 8, 2, score="softmax", renormalize=False)
    assert L.moe_route_hash(ctypes.byref(p), FAKE, FAKE, 10, FAKE, FAKE, None, FAKE, FAKE, None,
                            0, None, None) == tda.MOE_EUNSUPPORTED
    p = tda.make_params(4, 64, 8, 2, score="sigmoid")
    assert L.moe_route_hash(ctypes.byref(p), FAKE, FAKE, 0, FAKE, FAKE, None, FAKE, FAKE, None,
                            0, None, None) == tda.MOE_EINVAL
    assert L.moe_route_hash(ctypes.byref(p), None, FAKE, 10, None, None, None, FAKE, None, None,
                            0, None, None) == tda.MOE_EINVAL
    p0 = tda.make_params(0, 64, 8, 2, score="sigmoid")
    assert L.moe_route_hash(ctypes.byref(p0), None, None, 10, None, None, None, None, None, None,
                            0, None, None) == tda.MOE_OK
    # bf16, k <= 8, E <= 768, d % 8 == 0: per-slice partial dot products of
    # the k table experts (slices of 192 columns up to 384 experts, else 64)
    n = tda.route_hash_workspace_size(16384, 7168, 384, 6, score="sqrt_softplus")
    assert n == 38 * 16384 * 6 * 4
    assert tda.route_hash_workspace_size(100, 7168, 500, 8) == 112 * 100 * 8 * 4
    assert tda.route_hash_workspace_size(100, 1000, 384, 2) == 6 * 100 * 2 * 4
    # otherwise the gate logits of every expert, per K split
    for args in [(16384, 7168, 384, 6, 0), (4096, 2048, 128, 9, 1), (100, 64, 1024, 4, 1),
                 (100, 60, 64, 4, 1)]:
        n = tda.route_hash_workspace_size(*args)
        te = args[0] * args[2] * 4
        assert n >= te and n % te == 0, args
    assert tda.route_hash_workspace_size(0, 64, 8, 2) == 0


def test_route_hash_dispatch_validation():
    """moe_route_hash_dispatch rejects bad calls before enqueueing anything;
    its workspace holds the gate hand-off (256-byte aligned) and then the
    larger of the dispatch's own workspace and the hash kernel's tile
    histograms plus super-tile sums."""
    L = tda.lib()
    T, d, E, k = 1000, 128, 384, 6
    p = tda.make_params(T, d, E, k, score="sqrt_softplus")
    n = tda.route_hash_dispatch_workspace_size(T, d, E, k, score="sqrt_softplus")
    route = (tda.route_hash_workspace_size(T, d, E, k, score="sqrt_softplus") + 255) // 256 * 256
    tiles = -(-T // 32)  # 8-lane token segments, 4 wavefronts: 32 tokens per tile
    S = int(np.ceil(np.sqrt(tiles)))
    hist = (tiles * E * 2 + 255) // 256 * 256
    assert n >= route + hist + -(-tiles // S) * E * 4
    assert n >= route + tda.dispatch_workspace_size(T, k, E)
    ws = ctypes.c_void_p(0x1000)

    def call(pp, x=FAKE, W=FAKE, counts=FAKE, offsets=FAKE, perm=FAKE, w=ws, nbytes=n,
             vocab=50):
        return L.moe_route_hash_dispatch(ctypes.byref(pp), FAKE, FAKE, vocab, x, W, None, FAKE,
                                         FAKE, counts, offsets, perm, None, None, w, nbytes,
                                         None, None)

    assert call(p, x=None, W=None) == tda.MOE_EINVAL
    assert "required" in L.moe_last_error().decode()
    assert call(p, counts=None) == tda.MOE_EINVAL
    assert call(p, perm=None) == tda.MOE_EINVAL
    assert call(p, nbytes=n - 1) == tda.MOE_EINVAL
    assert "workspace" in L.moe_last_error().decode()
    assert call(p, w=ctypes.c_void_p(0x1010)) == tda.MOE_EINVAL
    assert "aligned" in L.moe_last_error().decode()
    assert call(p, vocab=0) == tda.MOE_EINVAL
    big = tda.make_params(T, d, 4096, k, score="sqrt_softplus")
    assert call(big) in (tda.MOE_EINVAL, tda.MOE_EUNSUPPORTED)
    assert tda.route_hash_dispatch_workspace_size(0, d, E, k) >= 0


def test_dispatch_validation_and_workspace_size():
    L = tda.lib()
    # two tiles of 512 routes: a [2][64] histogram of 16-bit counts
    assert tda.dispatch_workspace_size(100, 8, 64) >= 2 * 64 * 2
    assert tda.dispatch_workspace_size(0, 8, 64) == 0
    assert tda.dispatch_workspace_size(-1, 8, 64) == 0
    ws = tda.dispatch_workspace_size(100, 8, 64)
    assert L.moe_dispatch(FAKE, 100, 8, 64, FAKE, FAKE, FAKE, None, None, FAKE, ws - 1, None,
                          None) == tda.MOE_EINVAL
    assert "workspace" in L.moe_last_error().decode()
    assert L.moe_dispatch(FAKE, 100, 0, 64, FAKE, FAKE, FAKE, None, None, FAKE, ws, None,
                          None) == tda.MOE_EINVAL
    assert L.moe_dispatch(FAKE, 100, 8, 4096, FAKE, FAKE, FAKE, None, None, FAKE, ws, None,
                          None) == tda.MOE_EUNSUPPORTED
    assert L.moe_dispatch(FAKE, 100, 8, 64, None, FAKE, FAKE, None, None, FAKE, ws, None,
                          None) == tda.MOE_EINVAL


def test_binding_rejects_host_tensors():
    import torch
    with pytest.raises(ValueError):
        tda.route(torch.zeros(4, 8), torch.zeros(2, 8), 1)


def test_dispatch_rejects_unaligned_workspace():
    L = tda.lib()
    ws = tda.dispatch_workspace_size(100, 8, 64)
    assert L.moe_dispatch(FAKE, 100, 8, 64, FAKE, FAKE, FAKE, None, None, ctypes.c_void_p(0x1004), ws,
                          None, None) == tda.MOE_EINVAL
    assert "aligned" in L.moe_last_error().decode()


@pytest.mark.parametrize("T,k,E", [(4096, 16, 128), (65536, 4, 128), (16384, 6, 384),
                                   (8192, 8, 256), (256, 2, 8), (70000, 30, 1024), (5, 3, 7)])
def test_dispatch_workspace_size_per_path(T, k, E):
    # two-kernel path (E % 8 == 0): one tile-major histogram of at most 32 Ki
    # 16-bit counts (the smallest tiles of 512, 1024 or 2048 routes that
    # fit), unless those tiles are fewer than 128 while 512-route tiles are
    # at least 128; otherwise 32-bit tile histograms, tile bases and totals
    # (tiles of 512 routes)
    n = tda.dispatch_workspace_size(T, k, E)
    R = T * k
    fits = [-(-R // t) for t in (512, 1024, 2048) if -(-R // t) * E <= 32768]
    two = E % 8 == 0 and fits and not (fits[0] < 128 and -(-R // 512) >= 128)
    if two:
        assert n == fits[0] * E * 2
    else:
        nt = -(-R // 512)
        assert n == (2 * nt + 1) * E * 4


def super_bytes(T, k, E, tokens):
    """Tile histograms (16-bit, 256-byte aligned) plus super-tile sums (int32)
    of the select-written super-tile path: S = ceil(sqrt(tiles))."""
    tiles = -(-T // tokens)
    S = 1
    while S * S < tiles:
        S += 1
    return -(-tiles * E * 2 // 256) * 256 + -(-tiles // S) * E * 4


def test_route_dispatch_workspace_size():
    # the gate hand-off (256-byte aligned), then the dispatch's data for the
    # largest of the paths the call may take (gate or select-only, aligned or
    # not): the dispatch's own workspace, tile histograms, or tile histograms
    # plus super-tile sums
    for T, d, E, k in [(4096, 2048, 128, 16), (65536, 2880, 128, 4), (256, 1024, 8, 2),
                       (16384, 7168, 384, 6), (5, 7, 4, 1)]:
        route = tda.route_workspace_size(T, d, E, k)
        route = (route + 255) // 256 * 256
        n = tda.route_dispatch_workspace_size(T, d, E, k)
        disp = tda.dispatch_workspace_size(T, k, E)
        plan = tda.route_dispatch_plan(T, d, E, k)
        assert n >= route + (disp if plan["path"] == "separate" else 0), (T, n)
        if plan["path"] == "select_super":
            assert n >= route + super_bytes(T, k, E, plan["hist_tokens"]), (T, n)
    # Qwen3-like shape: the gate hand-off holds whole T x E partial arrays
    # (one per K split); then 16-token tiles of 256 routes -> 256 histogram rows
    # of 128 16-bit counts and 16 super rows of 128 int32 sums
    route = tda.route_workspace_size(4096, 2048, 128, 16)
    assert route % (4096 * 128 * 4) == 0 and 1 <= route // (4096 * 128 * 4) <= 8
    assert tda.route_dispatch_plan(4096, 2048, 128, 16)["hist_tokens"] == 16
    assert tda.route_dispatch_workspace_size(4096, 2048, 128, 16) == \
        (route + 255) // 256 * 256 + 256 * 128 * 2 + 16 * 128 * 4


def test_route_dispatch_validation():
    L = tda.lib()
    p = tda.make_params(64, 128, 16, 2)
    n = tda.route_dispatch_workspace_size(64, 128, 16, 2)
    args = lambda counts, ws, nbytes: (ctypes.byref(p), FAKE, FAKE, None, None, None, None, FAKE,
                                       FAKE, counts, FAKE, FAKE, None, None, ws, nbytes, None,
                                       None)
    assert L.moe_route_dispatch(*args(None, ctypes.c_void_p(0x1000), n)) == tda.MOE_EINVAL
    assert "counts" in L.moe_last_error().decode()
    assert L.moe_route_dispatch(*args(FAKE, ctypes.c_void_p(0x1000), n - 1)) == tda.MOE_EINVAL
    assert "workspace" in L.moe_last_error().decode()
    assert L.moe_route_dispatch(*args(FAKE, ctypes.c_void_p(0x1010), n)) == tda.MOE_EINVAL
    assert "aligned" in L.moe_last_error().decode()
    bad = tda.make_params(64, 128, 16, 0)
    assert L.moe_route_dispatch(ctypes.byref(bad), FAKE, FAKE, None, None, None, None, FAKE, FAKE,
                                FAKE, FAKE, FAKE, None, None, FAKE, n, None,
                                None) == tda.MOE_EINVAL


def test_plan_constants_match_binding():
    src = open(HEADER).read()
    consts = dict(re.findall(r"#define (MOE_\w+) \(?(-?\d+)\)?", src))
    for i, name in enumerate(tda.PATHS):
        assert int(consts["MOE_PATH_" + name.upper()]) == i
    assert ctypes.sizeof(tda.PlanInfo) == 4 * len(tda.PLAN_FIELDS)
    for i, name in enumerate(tda.STAGES):
        assert int(consts["MOE_STAGE_" + name.upper()]) == i
    assert int(consts["MOE_NUM_STAGES"]) == len(tda.STAGES)


WORKLOAD_PLANS = {  # path, kernels per moe_route_dispatch call
    "mixtral": ("small", 2),
    "qwen3_dynk": ("select_super", 3),
    "dsv3_grouped": ("select_super", 3),
    "dsv4": ("select_super", 3),
    "gptoss_skew": ("fused", 2),
    "dsv4_bias": ("select_super", 3),
    "olmoe": ("select_super", 3),
    "dsv3_groupmax": ("select_super", 3),
    "switch_top1": ("select_super", 3),
    "grouped_quota": ("select_super", 3),
}


@pytest.mark.parametrize("name", sorted(WORKLOAD_PLANS))
def test_workload_plans(name):
    """The kernel sequence moe_route_dispatch takes for each workload shape."""
    import workloads as wl
    w = wl.WORKLOADS[name]
    kw = dict(score=w.score, n_groups=w.n_groups, topk_groups=w.topk_groups,
              group_score=w.group_score if w.n_groups > 1 else "max",
              renormalize=w.renormalize, route_scale=w.route_scale)
    plan = tda.route_dispatch_plan(w.T, w.d, w.E, w.k, 1 if w.dtype == "bf16" else 0, **kw)
    assert (plan["path"], plan["kernels"]) == WORKLOAD_PLANS[name], plan
    # unaligned x or W: the register-staged gate, no K split, no fused selection
    plan_u = tda.route_dispatch_plan(w.T, w.d, w.E, w.k, 1 if w.dtype == "bf16" else 0,
                                     aligned=False, **kw)
    assert plan_u["gate_stage_bytes"] == 0 and plan_u["gate_splits"] == 1
    assert plan_u["path"] != "fused"


def test_planner_invariants_on_random_shapes():
    """Every plan the host chooses is one the kernels are built for: the ring
    (one ring of x and W stages, or x three deep and W two) within 144 KB of
    LDS, tiles split into whole 16 x 16 blocks per wave,
    eight-wave tiles only for bf16, a K split of 1-8 that leaves every split
    some of K, fused selection only on whole-row unsplit tiles of <= 128
    experts, the small path only up to 2048 routes, and dispatch tiles the
    placement kernel takes."""
    rng = np.random.default_rng(11)
    paths = set()
    for _ in range(600):
        E = int(rng.choice([4, 8, 16, 30, 64, 100, 128, 160, 256, 384, 512, 1000]))
        k = int(rng.integers(1, min(E, 32) + 1))
        T = int(rng.choice([1, 7, 100, 255, 1000, 4096, 8192, 16384, 65536, 200000]))
        d = int(rng.choice([8, 64, 512, 1024, 2048, 2880, 4096, 7168]))
        dt = int(rng.integers(0, 2))
        G = int(rng.choice([g for g in (1, 2, 4, 8) if E % g == 0 and g <= E]))
        kw = dict(score="sigmoid", n_groups=G, topk_groups=G,
                  group_score="max", renormalize=True, route_scale=1.0)
        plan = tda.route_dispatch_plan(T, d, E, k, dt, **kw)
        paths.add(plan["path"])
        bm, bn, waves, S = plan["gate_bm"], plan["gate_bn"], plan["gate_waves"], plan["gate_splits"]
        assert waves in (4, 8) and (waves == 4 or dt == 1), plan
        assert bm % 32 == 0 and bn % 32 == 0, plan
        assert S in (1, 2, 4, 8), plan
        if plan["gate_stage_bytes"]:
            rb, ns = plan["gate_stage_bytes"], plan["gate_ring_depth"]
            assert rb in (64, 128, 256, 512) and 2 <= ns <= 8, plan
            lds = plan["gate_lds_bytes"]
            assert lds <= 144 * 1024, plan
            if lds != ns * (bm + bn) * rb:
                # split rings: x three stages deep, W two, only where three
                # stages of both would not fit
                assert lds == (3 * bm + 2 * bn) * rb and ns == 3 and rb == 128, plan
                assert waves == 8 and 3 * (bm + bn) * rb > 144 * 1024, plan
            assert (d * (2 if dt else 4) + rb - 1) // rb >= S, plan  # every split has K
        if plan["path"] == "fused":
            assert S == 1 and bn >= E and E <= 128 and dt == 1, plan
        if plan["path"] == "small":
            assert T * k <= 2048 and E <= 128 and plan["kernels"] == 2, plan
        if plan["path"] in ("select_hist", "fused") and plan["hist_tokens"]:
            assert plan["hist_tokens"] * k in (256, 512, 1024, 2048), plan
            assert -(-T * k // (plan["hist_tokens"] * k)) * E <= 32 * 1024, plan
        if plan["path"] == "select_super":
            assert 1 <= plan["hist_tokens"] * k <= 2048 and plan["gate_stage_bytes"], plan
            assert plan["kernels"] == 3, plan
        assert plan["select_lanes"] in (4, 8, 16, 64), plan
        assert plan["select_lanes"] * plan["select_experts_per_lane"] >= E, plan
    assert {"small", "separate", "select_super", "fused"} <= paths, paths


def test_combine_validation():
    # every check runs on the host before a launch; T = 0 or d = 0 launch nothing
    L = tda.lib()
    ok = (FAKE, 5, FAKE, FAKE, None, FAKE, None, None)  # Yp, R, inv, weights, shared, y, dev_err, stream
    assert L.moe_combine(0, 4, 16, 1, *ok) == tda.MOE_OK
    assert L.moe_combine(3, 4, 0, 1, *ok) == tda.MOE_OK
    assert L.moe_combine(-1, 4, 16, 1, *ok) == tda.MOE_EINVAL
    assert L.moe_combine(3, 0, 16, 1, *ok) == tda.MOE_EINVAL
    assert L.moe_combine(3, tda.MAX_K + 1, 16, 1, *ok) == tda.MOE_EUNSUPPORTED
    assert L.moe_combine(3, 4, 16, 2, *ok) == tda.MOE_EINVAL
    assert "dtype" in L.moe_last_error().decode()
    assert L.moe_combine(3, 4, -2, 1, *ok) == tda.MOE_EINVAL
    assert L.moe_combine(3, 4, 16, 1, FAKE, -1, FAKE, FAKE, None, FAKE, None, None) == tda.MOE_EINVAL
    assert L.moe_combine(3, 4, 16, 1, None, 5, FAKE, FAKE, None, FAKE, None, None) == tda.MOE_EINVAL
    assert "Yp" in L.moe_last_error().decode()
    assert L.moe_combine(3, 4, 16, 1, FAKE, 5, FAKE, FAKE, None, None, None, None) == tda.MOE_EINVAL
    assert L.moe_combine(3, 4, 16, 1, FAKE, 5, None, FAKE, None, FAKE, None, None) == tda.MOE_EINVAL
    assert L.moe_combine(1 << 30, 4, 16, 1, *ok) == tda.MOE_EUNSUPPORTED


def test_capacity_validation():
    L = tda.lib()
    d = (FAKE, FAKE, FAKE, FAKE, FAKE, None)  # offsets, inv, slot, kept, dropped, stream
    assert L.moe_dispatch_capacity(FAKE, -1, 1, 8, 4, *d) == tda.MOE_EINVAL
    assert L.moe_dispatch_capacity(FAKE, 10, 0, 8, 4, *d) == tda.MOE_EINVAL
    assert L.moe_dispatch_capacity(FAKE, 10, 1, 0, 4, *d) == tda.MOE_EINVAL
    assert L.moe_dispatch_capacity(FAKE, 10, 1, tda.MAX_EXPERTS + 1, 4, *d) == tda.MOE_EUNSUPPORTED
    assert L.moe_dispatch_capacity(FAKE, 10, 1, 8, -1, *d) == tda.MOE_EINVAL
    assert "capacity" in L.moe_last_error().decode()
    assert L.moe_dispatch_capacity(FAKE, 10, 1, 1024, 1 << 22, *d) == tda.MOE_EUNSUPPORTED
    assert L.moe_dispatch_capacity(FAKE, 10, 1, 8, 4, None, FAKE, FAKE, FAKE, FAKE, None) == tda.MOE_EINVAL
    assert L.moe_dispatch_capacity(None, 10, 1, 8, 4, *d) == tda.MOE_EINVAL


def test_permute_and_ep_layout_validation():
    L = tda.lib()
    assert L.moe_permute_rows(0, 2, 16, 1, FAKE, FAKE, 8, FAKE, None, None) == tda.MOE_OK
    assert L.moe_permute_rows(-1, 2, 16, 1, FAKE, FAKE, 8, FAKE, None, None) == tda.MOE_EINVAL
    assert L.moe_permute_rows(4, 0, 16, 1, FAKE, FAKE, 8, FAKE, None, None) == tda.MOE_EINVAL
    assert L.moe_permute_rows(4, 2, 16, 3, FAKE, FAKE, 8, FAKE, None, None) == tda.MOE_EINVAL
    assert L.moe_permute_rows(4, 2, -1, 1, FAKE, FAKE, 8, FAKE, None, None) == tda.MOE_EINVAL
    assert L.moe_permute_rows(4, 2, 16, 1, FAKE, FAKE, -1, FAKE, None, None) == tda.MOE_EINVAL
    assert L.moe_permute_rows(4, 2, 16, 1, FAKE, None, 8, FAKE, None, None) == tda.MOE_EINVAL
    assert L.moe_permute_rows(4, 2, 16, 1, None, FAKE, 8, FAKE, None, None) == tda.MOE_EINVAL
    assert L.moe_permute_rows(4, 2, 16, 1, FAKE, FAKE, 8, None, None, None) == tda.MOE_EINVAL
    assert "out" in L.moe_last_error().decode()
    assert L.moe_permute_rows(1 << 30, 4, 16, 1, FAKE, FAKE, 8, FAKE, None, None) == tda.MOE_EUNSUPPORTED
    assert L.moe_ep_layout(FAKE, 8, 3, FAKE, FAKE, None) == tda.MOE_EINVAL
    assert "divide" in L.moe_last_error().decode()
    assert L.moe_ep_layout(FAKE, 8, 0, FAKE, FAKE, None) == tda.MOE_EINVAL
    assert L.moe_ep_layout(FAKE, 0, 1, FAKE, FAKE, None) == tda.MOE_EINVAL
    assert L.moe_ep_layout(FAKE, 8, 2, FAKE, None, None) == tda.MOE_EINVAL


def test_k_per_group_validation():
    """Grouped top-k with a quota: rejected with a group limit, a negative
    quota or more experts than the groups keep; accepted otherwise."""
    L = tda.lib()

    def rc(**kw):
        base = dict(T=0, d=64, E=64, k=4, dtype=1, score="sigmoid", n_groups=8)
        base.update(kw)
        p = tda.make_params(**base)
        return L.moe_route_workspace_size(ctypes.byref(p)), L.moe_route(
            ctypes.byref(p), FAKE, FAKE, None, None, None, None, FAKE, FAKE, None, 0, None, None)

    assert rc(k_per_group=1)[1] == tda.MOE_OK
    assert rc(k_per_group=-1)[1] == tda.MOE_EINVAL
    assert rc(k_per_group=1, topk_groups=4)[1] == tda.MOE_EINVAL
    assert "topk_groups" in L.moe_last_error().decode()
    assert rc(k_per_group=1, k=9)[1] == tda.MOE_EINVAL  # 8 groups keep 8
    assert rc(k_per_group=1, k=8)[1] == tda.MOE_OK
    assert rc(k_per_group=20, k=32)[1] == tda.MOE_OK   # quota above the group size
    plan = tda.route_dispatch_plan(4096, 2048, 128, 8, 1, score="sigmoid", n_groups=16,
                                   topk_groups=16, k_per_group=1)
    assert plan["select_lanes"] >= 16  # a lane per group


def test_expand_request_k():
    """A k per request expands to its requests' tokens, in order (checked on
    host tensors against the workloads' own per-request draw)."""
    import workloads as wl
    lens = [256] * 16
    kt = wl.request_k(0, 4096, (4, 8, 16), 256)
    kr = kt[::256]
    got = tda.expand_request_k(kr, lens, "cpu")
    assert got.dtype == torch.int32 and np.array_equal(got.numpy(), kt)
    got = tda.expand_request_k([3, 1, 2], [2, 0, 3], "cpu")
    assert got.tolist() == [3, 3, 2, 2, 2]
    with pytest.raises(ValueError):
        tda.expand_request_k([3, 1], [2], "cpu")
    with pytest.raises(ValueError):
        tda._request_k(None, [2], None, 5, "cpu")
    with pytest.raises(ValueError):
        tda._request_k(None, [2], [4], 5, "cpu")
