"""MI355X MoE router and token dispatch: thin Python binding of libmoe_route.so.

Every step of the path runs in the library's HIP kernels.  This module only
checks shapes and dtypes, allocates outputs with torch (device memory), and
passes raw pointers plus torch's current HIP stream to the C ABI declared in
include/moe_route.h.  It raises if the library has not been built; there is
no fallback path.

    ids, weights = route(x, W, k=8, score="sigmoid", select_bias=b,
                         n_groups=8, topk_groups=4, route_scale=2.5)
    counts, offsets, perm, inv = dispatch(ids, E)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_route.so")

ABI_VERSION = 11
MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EDEVICE = 0, -1, -2, -3
MAX_EXPERTS, MAX_K, MAX_GROUPS = 1024, 32, 64
SCORES = {"softmax": 0, "sigmoid": 1, "sqrt_softplus": 2, "softmax_topk": 3}
GROUP_SCORES = {"max": 0, "top2_sum": 1}
EXPORTS = ("moe_route", "moe_route_workspace_size", "moe_route_hash",
           "moe_route_hash_workspace_size",
           "moe_dispatch_workspace_size", "moe_dispatch",
           "moe_route_dispatch", "moe_route_dispatch_workspace_size",
           "moe_route_dispatch_noalloc", "moe_route_hash_dispatch",
           "moe_route_hash_dispatch_workspace_size",
           "moe_route_dispatch_plan", "moe_combine", "moe_dispatch_capacity",
           "moe_permute_rows", "moe_ep_layout",
           "moe_profile_enable", "moe_profile_read",
           "moe_last_error", "moe_abi_version")
PATHS = ("separate", "select_hist", "fused", "small", "select_super")
PLAN_FIELDS = ("path", "gate_bm", "gate_bn", "gate_waves", "gate_splits", "gate_stage_bytes",
               "gate_ring_depth", "gate_lds_bytes", "select_lanes", "select_experts_per_lane",
               "hist_tokens", "kernels")
STAGES = ("gate", "select", "hash", "disp_hist", "disp_scan", "disp_scatter", "gate_select",
          "select_dispatch", "combine", "capacity", "permute", "ep_layout", "hash_ids",
          "hash_dots")


class MoeError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


class RouteParams(ctypes.Structure):
    """Mirror of moe_route_params."""
    _fields_ = [("T", ctypes.c_int32), ("d", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("dtype", ctypes.c_int32), ("score", ctypes.c_int32),
                ("n_groups", ctypes.c_int32), ("topk_groups", ctypes.c_int32),
                ("group_score", ctypes.c_int32), ("renormalize", ctypes.c_int32),
                ("route_scale", ctypes.c_float), ("k_per_group", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmoe_route.so (built by token_dispatch_amd._build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m token_dispatch_amd._build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, P = ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(RouteParams)
        L.moe_route.argtypes = [P] + [vp] * 9 + [ctypes.c_size_t, vp, vp]
        L.moe_route.restype = i32
        L.moe_route_workspace_size.argtypes = [P]
        L.moe_route_workspace_size.restype = ctypes.c_size_t
        L.moe_route_hash.argtypes = [P, vp, vp, i32, vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                                     vp, vp]
        L.moe_route_hash.restype = i32
        L.moe_route_hash_workspace_size.argtypes = [P]
        L.moe_route_hash_workspace_size.restype = ctypes.c_size_t
        L.moe_route_hash_dispatch.argtypes = [P, vp, vp, i32] + [vp] * 11 + [ctypes.c_size_t,
                                                                           vp, vp]
        L.moe_route_hash_dispatch.restype = i32
        L.moe_route_hash_dispatch_workspace_size.argtypes = [P]
        L.moe_route_hash_dispatch_workspace_size.restype = ctypes.c_size_t
        L.moe_dispatch_workspace_size.argtypes = [i32, i32, i32]
        L.moe_dispatch_workspace_size.restype = ctypes.c_size_t
        L.moe_dispatch.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                                   vp, vp]
        L.moe_dispatch.restype = i32
        L.moe_route_dispatch.argtypes = [P] + [vp] * 14 + [ctypes.c_size_t, vp, vp]
        L.moe_route_dispatch.restype = i32
        L.moe_route_dispatch_noalloc.argtypes = [P] + [vp] * 15
        L.moe_route_dispatch_noalloc.restype = i32
        L.moe_route_dispatch_workspace_size.argtypes = [P]
        L.moe_route_dispatch_workspace_size.restype = ctypes.c_size_t
        L.moe_route_dispatch_plan.argtypes = [P, i32, ctypes.POINTER(PlanInfo)]
        L.moe_route_dispatch_plan.restype = i32
        L.moe_combine.argtypes = [i32, i32, i32, i32, vp, i32, vp, vp, vp, vp, vp, vp]
        L.moe_combine.restype = i32
        L.moe_dispatch_capacity.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp]
        L.moe_dispatch_capacity.restype = i32
        L.moe_permute_rows.argtypes = [i32, i32, i32, i32, vp, vp, i32, vp, vp, vp]
        L.moe_permute_rows.restype = i32
        L.moe_ep_layout.argtypes = [vp, i32, i32, vp, vp, vp]
        L.moe_ep_layout.restype = i32
        L.moe_last_error.argtypes = []
        L.moe_last_error.restype = ctypes.c_char_p
        L.moe_profile_enable.argtypes = [i32]
        L.moe_profile_enable.restype = i32
        L.moe_profile_read.argtypes = [ctypes.POINTER(ctypes.c_double),
                                       ctypes.POINTER(ctypes.c_int64), i32]
        L.moe_profile_read.restype = i32
        L.moe_abi_version.argtypes = []
        L.moe_abi_version.restype = i32
        v = L.moe_abi_version()
        if v != ABI_VERSION:
            raise ImportError(f"libmoe_route ABI {v}, binding expects {ABI_VERSION}")
        _lib = L
    return _lib


def _check(rc: int):
    if rc != MOE_OK:
        raise MoeError(rc, lib().moe_last_error().decode())


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dev(t: torch.Tensor, name: str, dtype=None, shape=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return 0
    if t.dtype == torch.bfloat16:
        return 1
    raise ValueError(f"x and W must be float32 or bfloat16, got {t.dtype}")


def make_params(T, d, E, k, dtype=1, score="softmax", n_groups=1, topk_groups=None,
                group_score="max", renormalize=True, route_scale=1.0,
                k_per_group=0) -> RouteParams:
    return RouteParams(int(T), int(d), int(E), int(k), int(dtype), SCORES[score],
                       int(n_groups), int(n_groups if topk_groups is None else topk_groups),
                       GROUP_SCORES[group_score], int(bool(renormalize)), float(route_scale),
                       int(k_per_group))


def route_workspace_size(T, d, E, k, dtype=1, **kw) -> int:
    """Device bytes moe_route uses as its gate hand-off for these shapes."""
    p = make_params(T, d, E, k, dtype, **kw)
    return int(lib().moe_route_workspace_size(ctypes.byref(p)))


def expand_request_k(k_per_request, request_lens, device=None) -> torch.Tensor:
    """Per-token k [T] int32 from a k per request ("dynamic number of experts",
    a per-request hyperparameter): request i covers the next request_lens[i]
    tokens.  k_per_request: sequence or int tensor [n_req]; request_lens: a
    host sequence of token counts (so the result's size needs no device
    synchronisation)."""
    lens = [int(n) for n in request_lens]
    if any(n < 0 for n in lens):
        raise ValueError("request_lens must be >= 0")
    kr = torch.as_tensor(k_per_request, dtype=torch.int32, device=device)
    if kr.dim() != 1 or kr.numel() != len(lens):
        raise ValueError("k_per_request must have one entry per request")
    reps = torch.tensor(lens, dtype=torch.int64, device=kr.device)
    return torch.repeat_interleave(kr, reps, output_size=sum(lens)).contiguous()


def _request_k(k_per_token, k_per_request, request_lens, T, device):
    if k_per_request is None and request_lens is None:
        return k_per_token
    if k_per_request is None or request_lens is None:
        raise ValueError("k_per_request and request_lens go together")
    if k_per_token is not None:
        raise ValueError("give k_per_token or k_per_request, not both")
    if sum(int(n) for n in request_lens) != T:
        raise ValueError("request_lens must add up to T")
    return expand_request_k(k_per_request, request_lens, device)


def _route_args(x, W, k, score, logit_bias, select_bias, k_per_token, n_groups, topk_groups,
                group_score, renormalize, route_scale, logits, E, ids, weights, dev_err,
                return_logits, k_per_group=0):
    """Checks and output allocation shared by route() and route_dispatch()."""
    if group_score is None:
        group_score = "top2_sum" if select_bias is not None and not k_per_group else "max"
    if x is None:
        if W is not None or logits is None:
            raise ValueError("select-only mode needs x = W = None and logits")
        _dev(logits, "logits", torch.float32)
        T, E_ = logits.shape
        d, dt, device = 1, 1, logits.device
    else:
        _dev(x, "x")
        _dev(W, "W", x.dtype)
        T, d = x.shape
        E_ = W.shape[0]
        if W.shape[1] != d:
            raise ValueError("W must be [E][d] with the d of x")
        dt, device = _dtype_code(x), x.device
        if logits is None and return_logits:
            logits = torch.empty((T, E_), dtype=torch.float32, device=device)
        if logits is not None:
            _dev(logits, "logits", torch.float32, (T, E_))
    if E is not None and E != E_:
        raise ValueError("E does not match W / logits")
    for name, b in (("logit_bias", logit_bias), ("select_bias", select_bias)):
        if b is not None:
            _dev(b, name, torch.float32, (E_,))
    if k_per_token is not None:
        _dev(k_per_token, "k_per_token", torch.int32, (T,))
    if ids is None:
        ids = torch.empty((T, k), dtype=torch.int32, device=device)
    if weights is None:
        weights = torch.empty((T, k), dtype=torch.float32, device=device)
    _dev(ids, "ids", torch.int32, (T, k))
    _dev(weights, "weights", torch.float32, (T, k))
    if dev_err is not None:
        _dev(dev_err, "dev_err", torch.int32, (1,))
    p = make_params(T, d, E_, k, dt, score, n_groups, topk_groups, group_score, renormalize,
                    route_scale, k_per_group)
    return p, device, logits, ids, weights


def route(x: Optional[torch.Tensor], W: Optional[torch.Tensor], k: int, *,
          score: str = "softmax", logit_bias=None, select_bias=None, k_per_token=None,
          n_groups: int = 1, topk_groups: Optional[int] = None,
          group_score: Optional[str] = None, renormalize: bool = True,
          route_scale: float = 1.0, logits: Optional[torch.Tensor] = None,
          E: Optional[int] = None, ids=None, weights=None, workspace=None, dev_err=None,
          return_logits: bool = False, k_per_group: int = 0, k_per_request=None,
          request_lens=None):
    """Gate + score + (grouped) top-k + weights.  Returns (ids, weights[, logits]).

    x [T][d] and W [E][d] (float32 or bfloat16); or x = W = None with
    ``logits`` [T][E] float32 as the input (select-only mode).  The gate
    logits are written to ``logits`` when one is passed (or return_logits).
    ``workspace`` (uint8 device tensor) carries the gate's hand-off; it is
    allocated when not given.  group_score defaults to "top2_sum" when
    select_bias is given, else "max".  k_per_group > 0: grouped top-k with a
    quota (each group keeps its k_per_group best, then the top-k of those).
    k_per_request with request_lens: a k per request, expanded to k_per_token.
    """
    k_per_token = _request_k(k_per_token, k_per_request, request_lens,
                             (x if x is not None else logits).shape[0],
                             (x if x is not None else logits).device)
    p, device, logits, ids, weights = _route_args(
        x, W, k, score, logit_bias, select_bias, k_per_token, n_groups, topk_groups,
        group_score, renormalize, route_scale, logits, E, ids, weights, dev_err, return_logits,
        k_per_group)
    if workspace is None and x is not None:
        nbytes = int(lib().moe_route_workspace_size(ctypes.byref(p)))
        if nbytes:
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().moe_route(ctypes.byref(p), _p(x), _p(W), _p(logit_bias), _p(select_bias),
                           _p(k_per_token), _p(logits), _p(ids), _p(weights), _p(workspace),
                           ws_bytes, _p(dev_err), _stream(device)))
    return (ids, weights, logits) if return_logits else (ids, weights)


def route_dispatch_workspace_size(T, d, E, k, dtype=1, **kw) -> int:
    """Device bytes moe_route_dispatch needs for these shapes."""
    p = make_params(T, d, E, k, dtype, **kw)
    return int(lib().moe_route_dispatch_workspace_size(ctypes.byref(p)))


class PlanInfo(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int32) for name in PLAN_FIELDS]


def route_dispatch_plan(T, d, E, k, dtype=1, aligned=True, **kw) -> dict:
    """How moe_route_dispatch runs for these shapes (host-side planning only):
    {"path": "separate" | "select_hist" | "fused" | "small" | "select_super",
    gate tile,
    waves, splits, stage bytes, ring depth and LDS, selection lanes and
    experts per lane, tokens per counted dispatch tile, kernels per call}."""
    p = make_params(T, d, E, k, dtype, **kw)
    info = PlanInfo()
    _check(lib().moe_route_dispatch_plan(ctypes.byref(p), int(bool(aligned)),
                                         ctypes.byref(info)))
    out = {name: int(getattr(info, name)) for name in PLAN_FIELDS}
    out["path"] = PATHS[out["path"]]
    return out


def route_dispatch(x: Optional[torch.Tensor], W: Optional[torch.Tensor], k: int, *,
                   score: str = "softmax", logit_bias=None, select_bias=None,
                   k_per_token=None, n_groups: int = 1, topk_groups: Optional[int] = None,
                   group_score: Optional[str] = None, renormalize: bool = True,
                   route_scale: float = 1.0, logits: Optional[torch.Tensor] = None,
                   E: Optional[int] = None, ids=None, weights=None, counts=None, offsets=None,
                   perm=None, inv=None, with_inv: bool = True, workspace=None, dev_err=None,
                   k_per_group: int = 0, k_per_request=None, request_lens=None, maxvio=None,
                   _prepare: bool = False):
    """route() then dispatch() of its ids in one library call.  Returns
    (ids, weights, counts, offsets, perm, inv); ``workspace`` (256-byte
    aligned uint8 device tensor) is allocated when not given.  k_per_request
    with request_lens: a k per request, expanded to k_per_token.  maxvio:
    optional float64 device tensor [1] that receives the load statistic."""
    k_per_token = _request_k(k_per_token, k_per_request, request_lens,
                             (x if x is not None else logits).shape[0],
                             (x if x is not None else logits).device)
    p, device, logits, ids, weights = _route_args(
        x, W, k, score, logit_bias, select_bias, k_per_token, n_groups, topk_groups,
        group_score, renormalize, route_scale, logits, E, ids, weights, dev_err, False,
        k_per_group)
    E_, R = p.E, p.T * p.k
    if counts is None:
        counts = torch.empty(E_, dtype=torch.int32, device=device)
    if offsets is None:
        offsets = torch.empty(E_ + 1, dtype=torch.int32, device=device)
    if perm is None:
        perm = torch.empty(R, dtype=torch.int32, device=device)
    if inv is None and with_inv:
        inv = torch.empty(R, dtype=torch.int32, device=device)
    _dev(counts, "counts", torch.int32, (E_,))
    _dev(offsets, "offsets", torch.int32, (E_ + 1,))
    _dev(perm, "perm", torch.int32, (R,))
    if inv is not None:
        _dev(inv, "inv", torch.int32, (R,))
    if workspace is None:
        nbytes = int(lib().moe_route_dispatch_workspace_size(ctypes.byref(p)))
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    if maxvio is not None:
        _dev(maxvio, "maxvio", torch.float64, (1,))
    ws_bytes = workspace.numel() * workspace.element_size()
    args = [ctypes.byref(p), _p(x), _p(W), _p(logit_bias), _p(select_bias), _p(k_per_token),
            _p(logits), _p(ids), _p(weights), _p(counts), _p(offsets), _p(perm), _p(inv),
            _p(maxvio), _p(workspace), ws_bytes, _p(dev_err), _stream(device)]
    outs = (ids, weights, counts, offsets, perm, inv)
    if _prepare:  # (arguments, outputs, the tensors the arguments point into)
        return args, outs, (p, x, W, logit_bias, select_bias, k_per_token, logits, workspace,
                            maxvio, dev_err)
    _check(lib().moe_route_dispatch(*args))
    return outs


class PreparedRouteDispatch:
    """moe_route_dispatch with every argument checked and marshalled once,
    for loops that route batch after batch of the same shapes: ``call(x)``
    routes and dispatches x (same shape, dtype and device as the x it was
    prepared with) into the prepared outputs and returns them.  Only x and
    the current stream change between calls; the per-call host work is a
    few attribute checks and the library call."""

    def __init__(self, x: torch.Tensor, W: torch.Tensor, k: int, **kw):
        if x is None:
            raise ValueError("a prepared call needs x (the gate input)")
        self._args, self._outs, self._keep = route_dispatch(x, W, k, _prepare=True, **kw)
        self._shape, self._dtype, self._device = tuple(x.shape), x.dtype, x.device
        self._fn = lib().moe_route_dispatch

    def __call__(self, x: torch.Tensor):
        if (tuple(x.shape) != self._shape or x.dtype != self._dtype or
                x.device != self._device or not x.is_contiguous()):
            raise ValueError(f"x must be a contiguous {self._dtype} tensor of shape "
                             f"{self._shape} on {self._device}")
        args = self._args
        args[1] = x.data_ptr()
        args[17] = torch.cuda.current_stream(self._device).cuda_stream
        _check(self._fn(*args))
        return self._outs


def prepare_route_dispatch(x: torch.Tensor, W: torch.Tensor, k: int,
                           **kw) -> PreparedRouteDispatch:
    """route_dispatch() checked and marshalled once (same keyword arguments;
    pass the outputs and the workspace to keep them fixed); see
    PreparedRouteDispatch."""
    return PreparedRouteDispatch(x, W, k, **kw)


NOALLOC_SCRATCH_BYTES = 64 << 20


def route_dispatch_noalloc(x: Optional[torch.Tensor], W: Optional[torch.Tensor], k: int, *,
                           score: str = "softmax", logit_bias=None, select_bias=None,
                           k_per_token=None, n_groups: int = 1,
                           topk_groups: Optional[int] = None,
                           group_score: Optional[str] = None, renormalize: bool = True,
                           route_scale: float = 1.0, logits: Optional[torch.Tensor] = None,
                           E: Optional[int] = None, ids, weights, counts, offsets, perm,
                           inv=None, maxvio=None, dev_err=None, k_per_group: int = 0):
    """route_dispatch() through moe_route_dispatch_noalloc: the library's own
    per-GPU scratch array instead of a workspace, so the call allocates
    nothing.  Every output is the caller's (ids, weights, counts, offsets,
    perm required; inv, maxvio, dev_err optional).  Shapes needing more than
    NOALLOC_SCRATCH_BYTES of scratch raise MoeError (MOE_EUNSUPPORTED)."""
    p, device, logits, ids, weights = _route_args(
        x, W, k, score, logit_bias, select_bias, k_per_token, n_groups, topk_groups,
        group_score, renormalize, route_scale, logits, E, ids, weights, dev_err, False,
        k_per_group)
    E_, R = p.E, p.T * p.k
    _dev(counts, "counts", torch.int32, (E_,))
    _dev(offsets, "offsets", torch.int32, (E_ + 1,))
    _dev(perm, "perm", torch.int32, (R,))
    if inv is not None:
        _dev(inv, "inv", torch.int32, (R,))
    if maxvio is not None:
        _dev(maxvio, "maxvio", torch.float64, (1,))
    _check(lib().moe_route_dispatch_noalloc(
        ctypes.byref(p), _p(x), _p(W), _p(logit_bias), _p(select_bias), _p(k_per_token),
        _p(logits), _p(ids), _p(weights), _p(counts), _p(offsets), _p(perm), _p(inv),
        _p(maxvio), _p(dev_err), _stream(device)))
    return ids, weights, counts, offsets, perm, inv


def route_hash(token_ids: torch.Tensor, tid2eid: torch.Tensor, E: int, *, x=None, W=None,
               score: str = "sqrt_softplus", logit_bias=None, renormalize: bool = True,
               route_scale: float = 1.0, ids=None, weights=None, workspace=None,
               dev_err=None):
    """Hash routing: ids = tid2eid[token_ids] ([vocab][k] row-major table), plus
    weights from the k gathered gate logits when x and W are given.

    ``workspace`` (uint8 device tensor) holds the gate logits of every expert
    (the tiled gate contraction); it is allocated when not given.  An empty
    tensor asks for the k dot products per token instead."""
    _dev(token_ids, "token_ids", torch.int32)
    _dev(tid2eid, "tid2eid", torch.int32)
    T = token_ids.shape[0]
    vocab, k = tid2eid.shape
    device = token_ids.device
    d, dt = 1, 1
    if x is not None:
        _dev(x, "x")
        _dev(W, "W", x.dtype, (E, x.shape[1]))
        d, dt = x.shape[1], _dtype_code(x)
        if x.shape[0] != T:
            raise ValueError("x must have one row per token id")
    if logit_bias is not None:
        _dev(logit_bias, "logit_bias", torch.float32, (E,))
    if ids is None:
        ids = torch.empty((T, k), dtype=torch.int32, device=device)
    if weights is None and x is not None:
        weights = torch.empty((T, k), dtype=torch.float32, device=device)
    p = make_params(T, d, E, k, dt, score, 1, 1, "max", renormalize, route_scale)
    if workspace is None and x is not None:
        nbytes = int(lib().moe_route_hash_workspace_size(ctypes.byref(p)))
        if nbytes:
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    ws = None if not ws_bytes else workspace
    _check(lib().moe_route_hash(ctypes.byref(p), _p(token_ids), _p(tid2eid), vocab, _p(x),
                                _p(W), _p(logit_bias), _p(ids), _p(weights), _p(ws), ws_bytes,
                                _p(dev_err), _stream(device)))
    return ids, weights


def route_hash_dispatch(token_ids: torch.Tensor, tid2eid: torch.Tensor, E: int, *,
                        x: torch.Tensor, W: torch.Tensor, score: str = "sqrt_softplus",
                        logit_bias=None, renormalize: bool = True, route_scale: float = 1.0,
                        ids=None, weights=None, counts=None, offsets=None, perm=None, inv=None,
                        with_inv: bool = True, maxvio=None, workspace=None, dev_err=None):
    """route_hash() then dispatch() of its ids in one library call (the hash
    kernel also counts the dispatch tiles).  Returns (ids, weights, counts,
    offsets, perm, inv); ``workspace`` is allocated when not given."""
    _dev(token_ids, "token_ids", torch.int32)
    _dev(tid2eid, "tid2eid", torch.int32)
    T = token_ids.shape[0]
    vocab, k = tid2eid.shape
    device = token_ids.device
    _dev(x, "x")
    _dev(W, "W", x.dtype, (E, x.shape[1]))
    if x.shape[0] != T:
        raise ValueError("x must have one row per token id")
    d, dt = x.shape[1], _dtype_code(x)
    if logit_bias is not None:
        _dev(logit_bias, "logit_bias", torch.float32, (E,))
    R = T * k
    i32 = torch.int32
    ids = torch.empty((T, k), dtype=i32, device=device) if ids is None else ids
    weights = torch.empty((T, k), dtype=torch.float32, device=device) if weights is None else weights
    counts = torch.empty(E, dtype=i32, device=device) if counts is None else counts
    offsets = torch.empty(E + 1, dtype=i32, device=device) if offsets is None else offsets
    perm = torch.empty(R, dtype=i32, device=device) if perm is None else perm
    if inv is None and with_inv:
        inv = torch.empty(R, dtype=i32, device=device)
    _dev(ids, "ids", i32, (T, k))
    _dev(weights, "weights", torch.float32, (T, k))
    _dev(counts, "counts", i32, (E,))
    _dev(offsets, "offsets", i32, (E + 1,))
    _dev(perm, "perm", i32, (R,))
    if inv is not None:
        _dev(inv, "inv", i32, (R,))
    if maxvio is not None:
        _dev(maxvio, "maxvio", torch.float64, (1,))
    p = make_params(T, d, E, k, dt, score, 1, 1, "max", renormalize, route_scale)
    if workspace is None:
        nbytes = int(lib().moe_route_hash_dispatch_workspace_size(ctypes.byref(p)))
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().moe_route_hash_dispatch(ctypes.byref(p), _p(token_ids), _p(tid2eid), vocab,
                                         _p(x), _p(W), _p(logit_bias), _p(ids), _p(weights),
                                         _p(counts), _p(offsets), _p(perm), _p(inv), _p(maxvio),
                                         _p(workspace), ws_bytes, _p(dev_err), _stream(device)))
    return ids, weights, counts, offsets, perm, inv


def route_hash_dispatch_workspace_size(T, d, E, k, dtype=1, **kw) -> int:
    """Device bytes moe_route_hash_dispatch needs for these shapes."""
    p = make_params(T, d, E, k, dtype, **kw)
    return int(lib().moe_route_hash_dispatch_workspace_size(ctypes.byref(p)))


def route_hash_workspace_size(T, d, E, k, dtype=1, **kw) -> int:
    """Device bytes moe_route_hash uses for the gate logits of these shapes."""
    p = make_params(T, d, E, k, dtype, **kw)
    return int(lib().moe_route_hash_workspace_size(ctypes.byref(p)))


def dispatch_workspace_size(T: int, k_stride: int, E: int) -> int:
    return int(lib().moe_dispatch_workspace_size(T, k_stride, E))


def dispatch(ids: torch.Tensor, E: int, *, with_inv: bool = True, counts=None, offsets=None,
             perm=None, inv=None, workspace=None, dev_err=None, maxvio=None):
    """Stable grouping of routes by expert.  Returns (counts, offsets, perm, inv);
    perm has T*k_stride entries of which the first offsets[E] are set.  maxvio:
    optional float64 device tensor [1] that receives the load statistic
    max_e counts[e] / (R / E) - 1."""
    _dev(ids, "ids", torch.int32)
    T, ks = ids.shape
    device = ids.device
    R = T * ks
    if counts is None:
        counts = torch.empty(E, dtype=torch.int32, device=device)
    if offsets is None:
        offsets = torch.empty(E + 1, dtype=torch.int32, device=device)
    if perm is None:
        perm = torch.empty(R, dtype=torch.int32, device=device)
    if inv is None and with_inv:
        inv = torch.empty(R, dtype=torch.int32, device=device)
    ws_bytes = dispatch_workspace_size(T, ks, E)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=device)
    if maxvio is not None:
        _dev(maxvio, "maxvio", torch.float64, (1,))
    _check(lib().moe_dispatch(_p(ids), T, ks, E, _p(counts), _p(offsets), _p(perm), _p(inv),
                              _p(maxvio), _p(workspace), workspace.numel(), _p(dev_err),
                              _stream(device)))
    return counts, offsets, perm, inv


def permute_rows(x: torch.Tensor, inv: torch.Tensor, k_stride: int, out_rows: int, *,
                 out: Optional[torch.Tensor] = None,
                 dev_err: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Send buffer: out[inv[r]] = x[r // k_stride] for 0 <= inv[r] < out_rows
    (dispatch's inv: dispatch order; dispatch_capacity's slot: expert-major
    rows).  Rows no route is placed at are left as they are."""
    _dev(x, "x")
    if x.dim() != 2:
        raise ValueError("x must be [T][d]")
    T, d = x.shape
    dt = _dtype_code(x)
    _dev(inv, "inv", torch.int32)
    if inv.numel() != T * k_stride:
        raise ValueError(f"inv has {inv.numel()} entries, expected T*k_stride={T * k_stride}")
    if out is None:
        out = torch.empty((out_rows, d), dtype=x.dtype, device=x.device)
    _dev(out, "out", x.dtype, (out_rows, d))
    if dev_err is not None:
        _dev(dev_err, "dev_err", torch.int32)
    _check(lib().moe_permute_rows(T, int(k_stride), d, dt, _p(x), _p(inv), int(out_rows),
                                  _p(out), _p(dev_err), _stream(x.device)))
    return out


def ep_layout(offsets: torch.Tensor, n_ranks: int):
    """Per-rank (send_counts[N], send_offsets[N+1]) for N ranks of E/N experts."""
    _dev(offsets, "offsets", torch.int32)
    E = offsets.numel() - 1
    cnt = torch.empty(n_ranks, dtype=torch.int32, device=offsets.device)
    off = torch.empty(n_ranks + 1, dtype=torch.int32, device=offsets.device)
    _check(lib().moe_ep_layout(_p(offsets), E, int(n_ranks), _p(cnt), _p(off),
                               _stream(offsets.device)))
    return cnt, off


def dispatch_capacity(ids: torch.Tensor, E: int, capacity: int, offsets: torch.Tensor,
                      inv: torch.Tensor, *, slot=None, kept=None, dropped=None):
    """Capacity limit on a dispatch of ids (offsets, inv from dispatch): each
    expert keeps its first `capacity` routes in route order.  Returns
    (slot[T*k], kept[E], dropped[1]); slot = e*capacity + rank, or -1."""
    _dev(ids, "ids", torch.int32)
    T, ks = ids.shape
    device = ids.device
    _dev(offsets, "offsets", torch.int32)
    _dev(inv, "inv", torch.int32)
    if slot is None:
        slot = torch.empty(T * ks, dtype=torch.int32, device=device)
    if kept is None:
        kept = torch.empty(E, dtype=torch.int32, device=device)
    if dropped is None:
        dropped = torch.empty(1, dtype=torch.int32, device=device)
    _check(lib().moe_dispatch_capacity(_p(ids), T, ks, E, int(capacity), _p(offsets), _p(inv),
                                       _p(slot), _p(kept), _p(dropped), _stream(device)))
    return slot, kept, dropped


def combine(Yp: torch.Tensor, inv: torch.Tensor, weights: torch.Tensor, *,
            shared: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
            dev_err: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y[T][d] = sum_j weights[t][j] * Yp[inv[t][j]] (+ shared[t]).

    Yp[R][d] (float32 or bfloat16): expert outputs in dispatch order;
    inv[T][k] or [T*k] int32 from dispatch; weights[T][k] float32."""
    _dev(weights, "weights", torch.float32)
    T, k = weights.shape
    _dev(inv, "inv", torch.int32)
    if inv.numel() != T * k:
        raise ValueError(f"inv must have {T * k} entries, got {inv.numel()}")
    _dev(Yp, "Yp")
    if Yp.dim() != 2:
        raise ValueError("Yp must be [R][d]")
    R, d = Yp.shape
    dt = _dtype_code(Yp)
    if shared is not None:
        _dev(shared, "shared", Yp.dtype, (T, d))
    if out is None:
        out = torch.empty((T, d), dtype=Yp.dtype, device=Yp.device)
    _dev(out, "out", Yp.dtype, (T, d))
    _check(lib().moe_combine(T, k, d, dt, _p(Yp), R, _p(inv), _p(weights), _p(shared), _p(out),
                             _p(dev_err), _stream(Yp.device)))
    return out


def profile_enable(on: bool = True) -> None:
    """Start (clearing old records) or stop per-kernel event timing."""
    _check(lib().moe_profile_enable(int(bool(on))))


def profile_read() -> dict:
    """{stage: (total_ms, launches)} for the kernels timed since profile_enable."""
    n = len(STAGES)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    rc = lib().moe_profile_read(ms, cnt, n)
    if rc < 0:
        _check(rc)
    return {STAGES[i]: (ms[i], cnt[i]) for i in range(n)}
