"""CPU oracle for the MoE router and token dispatch -- TEST INFRASTRUCTURE.

A numpy front end over ``oracle.c`` (plain fp64 C, see ``oracle.h`` for the
sources it follows).  Only the tests, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import this package; the HIP library never
does, and this package never imports the HIP library.

bf16 inputs are numpy ``uint16`` arrays of bf16 bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_SOURCES = [os.path.join(_HERE, "oracle.c")]

SCORE = {"softmax": 0, "sigmoid": 1, "sqrt_softplus": 2, "softmax_topk": 3}
GROUP = {"max": 0, "top2_sum": 1}
DTYPE = {"f32": 0, "bf16": 1}


def build(verbose: bool = False) -> str:
    """Compile liboracle.so with gcc (fp64, no fast-math, no FMA contraction)."""
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
           "-Wall", "-Wextra", "-fPIC", "-shared", "-o", _LIB_PATH + ".tmp",
           *_SOURCES, "-lm", "-lpthread"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    global _lib
    _lib = None
    return _LIB_PATH


class _Params(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("score", ctypes.c_int32), ("n_groups", ctypes.c_int32),
                ("topk_groups", ctypes.c_int32), ("group_score", ctypes.c_int32),
                ("renormalize", ctypes.c_int32), ("route_scale", ctypes.c_double),
                ("k_per_group", ctypes.c_int32)]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        vp = ctypes.c_void_p
        i32 = ctypes.c_int32
        lib.orc_gate.argtypes = [ctypes.POINTER(_Params), vp, vp, vp, vp]
        lib.orc_gate.restype = None
        lib.orc_route_logits.argtypes = [ctypes.POINTER(_Params)] + [vp] * 11
        lib.orc_route_logits.restype = i32
        lib.orc_weights_for_ids.argtypes = [ctypes.POINTER(_Params), vp, vp, vp]
        lib.orc_weights_for_ids.restype = None
        lib.orc_hash_ids.argtypes = [i32, i32, i32, vp, vp, i32, vp]
        lib.orc_hash_ids.restype = i32
        lib.orc_dispatch.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp]
        lib.orc_dispatch.restype = i32
        lib.orc_maxvio.argtypes = [vp, i32]
        lib.orc_maxvio.restype = ctypes.c_double
        lib.orc_ep_layout.argtypes = [vp, i32, i32, vp, vp]
        lib.orc_ep_layout.restype = None
        lib.orc_permute_rows.argtypes = [i32, i32, i32, vp, vp, i32, vp]
        lib.orc_permute_rows.restype = None
        lib.orc_capacity.argtypes = [vp, i32, i32, i32, i32, vp, vp]
        lib.orc_capacity.restype = i32
        lib.orc_combine.argtypes = [i32, i32, i32, i32, vp, i32, vp, vp, vp, vp]
        lib.orc_combine.restype = i32
        lib.orc_route_full.argtypes = [ctypes.POINTER(_Params)] + [vp] * 11 + [i32]
        lib.orc_route_full.restype = i32
        lib.orc_gate_mt.argtypes = [ctypes.POINTER(_Params), vp, vp, vp, vp, i32]
        lib.orc_gate_mt.restype = None
        lib.orc_route_logits_mt.argtypes = [ctypes.POINTER(_Params)] + [vp] * 11 + [i32]
        lib.orc_route_logits_mt.restype = i32
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def _params(T, d, E, k, dtype="f32", score="softmax", n_groups=1, topk_groups=None,
            group_score="max", renormalize=True, route_scale=1.0, k_per_group=0):
    if topk_groups is None:
        topk_groups = n_groups
    return _Params(int(T), int(d), int(E), int(k), DTYPE[dtype], SCORE[score],
                   int(n_groups), int(topk_groups), GROUP[group_score],
                   int(bool(renormalize)), float(route_scale), int(k_per_group))


def _check_route_args(E, k, n_groups, topk_groups, group_score, k_per_group=0):
    if topk_groups is None:
        topk_groups = n_groups
    if k_per_group:
        if k_per_group < 0 or topk_groups != n_groups:
            raise ValueError("k_per_group > 0 takes no group limit (topk_groups = n_groups)")
        if k > n_groups * min(k_per_group, E // max(n_groups, 1)):
            raise ValueError("k exceeds the experts the groups keep")
    if E < 1 or k < 1:
        raise ValueError("need E >= 1 and k >= 1")
    if n_groups < 1 or E % n_groups:
        raise ValueError("n_groups must divide E")
    if not 1 <= topk_groups <= n_groups:
        raise ValueError("need 1 <= topk_groups <= n_groups")
    if k > topk_groups * (E // n_groups):
        raise ValueError("k exceeds the experts of the kept groups")
    if n_groups > 1 and group_score == "top2_sum" and E // n_groups < 2:
        raise ValueError("top2_sum needs groups of at least 2 experts")


def gate(x, W, logit_bias=None, dtype=None, nthreads=1):
    """fp64 logits[T][E] of x[T][d] and W[E][d] (float32, or uint16 = bf16 bits).
    nthreads > 1 splits the tokens over host threads (same results)."""
    if dtype is None:
        dtype = "bf16" if x.dtype == np.uint16 else "f32"
    npdt = np.uint16 if dtype == "bf16" else np.float32
    x = _c(x, npdt)
    W = _c(W, npdt)
    T, d = x.shape
    E = W.shape[0]
    assert W.shape[1] == d
    out = np.empty((T, E), dtype=np.float64)
    p = _params(T, d, E, 1, dtype)
    lb = _c(logit_bias, np.float32)
    if nthreads > 1:
        _load().orc_gate_mt(ctypes.byref(p), _ptr(x), _ptr(W), _ptr(lb), _ptr(out),
                            int(nthreads))
    else:
        _load().orc_gate(ctypes.byref(p), _ptr(x), _ptr(W), _ptr(lb), _ptr(out))
    return out


def route_logits(logits, k, score="softmax", select_bias=None, k_per_token=None,
                 n_groups=1, topk_groups=None, group_score=None, renormalize=True,
                 route_scale=1.0, k_per_group=0, nthreads=1):
    """Select and weight from fp64 logits.  Returns a dict with ids, weights,
    margin_k, margin_g, margin_s, margin_o, q (masked selection quantity),
    g (group scores; with k_per_group, each group's last kept q) and nbad
    (tokens with k_t outside [1, k]).  nthreads > 1 splits the tokens over
    host threads (same results)."""
    logits = _c(logits, np.float64)
    T, E = logits.shape
    if group_score is None or k_per_group:
        group_score = "top2_sum" if select_bias is not None and not k_per_group else "max"
    _check_route_args(E, k, n_groups, topk_groups, group_score, k_per_group)
    p = _params(T, 1, E, k, "f32", score, n_groups, topk_groups, group_score,
                renormalize, route_scale, k_per_group)
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    mk, mg, ms, mo = (np.empty(T, np.float64) for _ in range(4))
    q = np.empty((T, E), np.float64)
    g = np.full((T, n_groups), np.nan)
    args = (ctypes.byref(p), _ptr(logits), _ptr(_c(select_bias, np.float32)),
            _ptr(_c(k_per_token, np.int32)), _ptr(ids), _ptr(w), _ptr(mk), _ptr(mg),
            _ptr(ms), _ptr(mo), _ptr(q), _ptr(g))
    if nthreads > 1:
        nbad = _load().orc_route_logits_mt(*args, int(nthreads))
    else:
        nbad = _load().orc_route_logits(*args)
    return {"ids": ids, "weights": w, "margin_k": mk, "margin_g": mg,
            "margin_s": ms, "margin_o": mo, "q": q, "g": g, "nbad": int(nbad),
            "logits": logits}


def route(x, W, k, logit_bias=None, **kw):
    """Gate + selection + weights (fp64) for every row of x."""
    return route_logits(gate(x, W, logit_bias), k, **kw)


def weights_for_ids(logits, ids, score="softmax", renormalize=True, route_scale=1.0):
    logits = _c(logits, np.float64)
    ids = _c(ids, np.int32)
    T, E = logits.shape
    k = ids.shape[1]
    p = _params(T, 1, E, k, "f32", score, 1, 1, "max", renormalize, route_scale)
    w = np.empty((T, k), np.float64)
    _load().orc_weights_for_ids(ctypes.byref(p), _ptr(logits), _ptr(ids), _ptr(w))
    return w


def hash_ids(token_ids, tid2eid, E):
    """ids[T][k] from a row-major [vocab][k] table; returns (ids, n_errors)."""
    tok = _c(token_ids, np.int32)
    tab = _c(tid2eid, np.int32)
    V, k = tab.shape
    T = tok.shape[0]
    ids = np.empty((T, k), np.int32)
    nerr = _load().orc_hash_ids(T, k, E, _ptr(tok), _ptr(tab), V, _ptr(ids))
    return ids, int(nerr)


def dispatch(ids, E):
    """Stable counting sort of route indices by expert.

    Returns counts[E], offsets[E+1], perm[offsets[E]], inv[T*k], n_errors."""
    ids = _c(ids, np.int32)
    T, ks = ids.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    perm = np.full(max(T * ks, 1), -1, np.int32)
    inv = np.empty(max(T * ks, 1), np.int32)
    nerr = _load().orc_dispatch(_ptr(ids), T, ks, E, _ptr(counts), _ptr(offsets),
                                _ptr(perm), _ptr(inv))
    R = int(offsets[E])
    return {"counts": counts, "offsets": offsets, "perm": perm[:R].copy(),
            "inv": inv[:T * ks].copy(), "nerr": int(nerr)}


def ep_layout(offsets, N):
    """Per-rank send counts[N] and offsets[N+1] for N ranks owning E/N
    contiguous experts each (offsets[E+1] from dispatch)."""
    offsets = _c(offsets, np.int32)
    E = offsets.shape[0] - 1
    if N < 1 or E % N:
        raise ValueError("N must divide E")
    cnt = np.empty(N, np.int32)
    off = np.empty(N + 1, np.int32)
    _load().orc_ep_layout(_ptr(offsets), E, int(N), _ptr(cnt), _ptr(off))
    return cnt, off


def permute_rows(x, perm, k_stride):
    """out[p] = x[perm[p] // k_stride] (fp64) for every p of perm."""
    dtype = "bf16" if x.dtype == np.uint16 else "f32"
    x = _c(x, np.uint16 if dtype == "bf16" else np.float32)
    perm = _c(perm, np.int32)
    R = perm.shape[0]
    d = x.shape[1]
    out = np.empty((R, d), np.float64)
    _load().orc_permute_rows(int(k_stride), d, DTYPE[dtype], _ptr(x), _ptr(perm), R, _ptr(out))
    return out


def capacity(ids, E, C):
    """Capacity-limited dispatch: each expert keeps its first C routes in
    route order.  Returns slot[T*k] (e*C + rank, or -1), kept[E], dropped."""
    ids = _c(ids, np.int32)
    T, ks = ids.shape
    slot = np.empty(max(T * ks, 1), np.int32)
    kept = np.empty(max(E, 1), np.int32)
    dropped = _load().orc_capacity(_ptr(ids), T, ks, E, int(C), _ptr(slot), _ptr(kept))
    return {"slot": slot[:T * ks].copy(), "kept": kept[:E].copy(), "dropped": int(dropped)}


def combine(Yp, inv, weights, shared=None):
    """y[T][d] (fp64) = sum_j weights[t][j] * Yp[inv[t][j]] (+ shared[t]).

    Yp[R][d] are the expert outputs in dispatch order (float32, or uint16 =
    bf16 bits); inv[T][k] as returned by dispatch (-1: empty slot);
    weights[T][k] float32.  Returns (y, n_errors) -- n_errors counts slots
    with inv >= R."""
    dtype = "bf16" if Yp.dtype == np.uint16 else "f32"
    npdt = np.uint16 if dtype == "bf16" else np.float32
    Yp = _c(Yp, npdt)
    inv = _c(inv, np.int32)
    weights = _c(weights, np.float32)
    R, d = Yp.shape
    T, k = inv.shape
    assert weights.shape == (T, k)
    if shared is not None:
        shared = _c(shared, npdt)
        assert shared.shape == (T, d)
    y = np.empty((T, d), np.float64)
    nerr = _load().orc_combine(T, k, d, DTYPE[dtype], _ptr(Yp), R, _ptr(inv),
                               _ptr(weights), _ptr(shared), _ptr(y))
    return y, int(nerr)


def maxvio(counts):
    c = _c(counts, np.int32)
    return float(_load().orc_maxvio(_ptr(c), c.shape[0]))


def route_full(x, W, k, *, score, logit_bias=None, select_bias=None, k_per_token=None,
               n_groups=1, topk_groups=None, group_score=None, renormalize=True,
               route_scale=1.0, k_per_group=0, nthreads=None):
    """Whole path (gate + route + dispatch) on nthreads host threads."""
    dtype = "bf16" if x.dtype == np.uint16 else "f32"
    npdt = np.uint16 if dtype == "bf16" else np.float32
    x = _c(x, npdt)
    W = _c(W, npdt)
    T, d = x.shape
    E = W.shape[0]
    if group_score is None or k_per_group:
        group_score = "top2_sum" if select_bias is not None and not k_per_group else "max"
    _check_route_args(E, k, n_groups, topk_groups, group_score, k_per_group)
    if nthreads is None:
        nthreads = os.cpu_count() or 1
    p = _params(T, d, E, k, dtype, score, n_groups, topk_groups, group_score,
                renormalize, route_scale, k_per_group)
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    perm = np.empty(max(T * k, 1), np.int32)
    inv = np.empty(max(T * k, 1), np.int32)
    nbad = _load().orc_route_full(
        ctypes.byref(p), _ptr(x), _ptr(W), _ptr(_c(logit_bias, np.float32)),
        _ptr(_c(select_bias, np.float32)), _ptr(_c(k_per_token, np.int32)), _ptr(ids),
        _ptr(w), _ptr(counts), _ptr(offsets), _ptr(perm), _ptr(inv), int(nthreads))
    return {"ids": ids, "weights": w, "counts": counts, "offsets": offsets,
            "perm": perm[:int(offsets[E])].copy(), "inv": inv[:T * k].copy(),
            "nbad": int(nbad), "nthreads": int(nthreads)}
