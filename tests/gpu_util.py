"""Helpers for the GPU tests: device upload and the workload -> call mapping."""
from __future__ import annotations

import sys

import numpy as np
import torch

import token_dispatch_amd as tda


def say(*a):
    """Name the case before a GPU step (flushed, so a crash still shows it)."""
    print("[gpu]", *a, file=sys.stderr, flush=True)


def up(a, device="cuda:0"):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def down(t):
    return None if t is None else t.detach().cpu().numpy()


def route_kwargs(w):
    """Keyword arguments of the routing rule of a workloads.Workload."""
    return dict(score=w.score, n_groups=w.n_groups, topk_groups=w.topk_groups,
                group_score=w.group_score if w.n_groups > 1 and not w.k_per_group else None,
                renormalize=w.renormalize, route_scale=w.route_scale,
                k_per_group=w.k_per_group)


def gpu_route(w, inp, device="cuda:0", return_logits=True):
    kw = route_kwargs(w)
    if kw["group_score"] is None:
        kw.pop("group_score")
    return tda.route(up(inp["x"], device), up(inp["W"], device), w.k,
                     logit_bias=up(inp["logit_bias"], device),
                     select_bias=up(inp["select_bias"], device),
                     k_per_token=up(inp["k_per_token"], device),
                     return_logits=return_logits, **kw)
