"""Comparison of the HIP path's outputs with the oracle's (acceptance rule).

Expert ids must be bit-exact except on tokens whose selection margin at the
k-th boundary or at the kept-group boundary is below NEAR (1e-4, in units of
the quantity the selection compares: the logit when the choice is a monotone
function of it, else q = score + bias).  Such near-tie tokens are counted and
checked for validity: the GPU's row must be one that an exact selection could
return if the quantities within NEAR of each other were reordered --

* flat selection: no unchosen candidate beats a chosen one by more than NEAR
  (every expert clearly above the boundary is chosen, every chosen one is at
  most NEAR below it);
* group limit: some set of topk_groups groups -- all groups clearly above
  the kept-group boundary, the rest within NEAR of it -- contains every
  chosen expert, and within that set's experts the same exchange condition
  holds;
* per-group quota (a partition-matroid limit): at most k_per_group per
  group, and no feasible swap of a chosen expert for an unchosen one gains
  more than NEAR;

with slots in descending order up to NEAR, and weights equal to the oracle's
weights for the GPU's own ids.  Tokens whose selected experts are only
separated by less than NEAR inside the row (slot order) must select the same
set, in an order valid up to NEAR.  Weights: |GPU - oracle| <= 1e-4.
Dispatch arrays: bit-exact against the oracle's dispatch of the GPU's ids."""
from __future__ import annotations

import itertools

import numpy as np

NEAR = 1e-4
WTOL = 1e-4


def to_numpy(t):
    return t.detach().cpu().numpy()


def _order_ok(v, row):
    """Slots in descending compared quantity, up to NEAR."""
    return bool(np.all(v[row[:-1]] >= v[row[1:]] - NEAR))


def _exchange_ok(v, S, cands):
    """No candidate outside S exceeds the smallest chosen value by > NEAR."""
    rest = np.setdiff1d(cands, S, assume_unique=False)
    return rest.size == 0 or v[S].min() >= v[rest].max() - NEAR


def _group_limit_ok(q, g, S, n_groups, topk_groups):
    gs = q.shape[0] // n_groups
    gb = np.sort(g)[::-1][topk_groups - 1]
    must = [γ for γ in range(n_groups) if g[γ] > gb + NEAR]
    maybe = [γ for γ in range(n_groups) if abs(g[γ] - gb) <= NEAR]
    need = topk_groups - len(must)
    if need < 0 or need > len(maybe):
        return False
    for extra in itertools.combinations(maybe, need):
        kept = np.array(sorted(must + list(extra)))
        if not np.all(np.isin(S // gs, kept)):
            continue
        cands = (kept[:, None] * gs + np.arange(gs)[None, :]).reshape(-1)
        if _exchange_ok(q, S, cands):
            return True
    return False


def _quota_ok(q, S, n_groups, kpg):
    gs = q.shape[0] // n_groups
    cnt = np.bincount(S // gs, minlength=n_groups)
    if cnt.max() > kpg:
        return False
    out = np.setdiff1d(np.arange(q.shape[0]), S)
    for i in S:
        # j may replace i when its group has room, or is i's own group
        gj = out // gs
        feasible = (cnt[gj] < kpg) | (gj == i // gs)
        if np.any(q[out[feasible]] > q[i] + NEAR):
            return False
    return True


def check_route(gpu_ids, gpu_w, ref, orc, *, score, renormalize=True, route_scale=1.0,
                k_per_token=None, n_groups=1, topk_groups=None, k_per_group=0, where=""):
    """Compare a route result with oracle output `ref` (from oracle_route).

    Returns statistics; raises AssertionError on any violation."""
    ids = np.asarray(gpu_ids)
    w = np.asarray(gpu_w, dtype=np.float64)
    T, K = ids.shape
    assert ref["ids"].shape == (T, K), (ref["ids"].shape, ids.shape, where)
    mk, mg, mo = ref["margin_k"], ref["margin_g"], ref["margin_o"]
    near_tie = np.minimum(mk, mg) < NEAR
    order_tie = (~near_tie) & (mo < NEAR)
    exact = ~(near_tie | order_tie)
    kt_all = np.full(T, K) if k_per_token is None else np.asarray(k_per_token)
    # the quantity the selection compares
    vq = ref["logits"] if ref["monotone"] else ref["q_raw"]

    # 1. exact tokens: bit-exact ids, weights within WTOL
    bad = np.nonzero(exact & np.any(ids != ref["ids"], axis=1))[0]
    assert bad.size == 0, (f"{where}: {bad.size} tokens with ids != oracle (margins "
                           f"{mk[bad[:3]]}, {mg[bad[:3]]}); first t={bad[0]}: gpu "
                           f"{ids[bad[0]]} oracle {ref['ids'][bad[0]]}")
    dw = np.abs(w - ref["weights"])
    worst = float(dw[exact].max()) if exact.any() else 0.0
    assert worst <= WTOL, f"{where}: max |dw| = {worst:.3g} > {WTOL}"

    # 2. slot-order near-ties: same set, a valid order, weights follow the ids
    for t in np.nonzero(order_tie)[0]:
        kt = int(kt_all[t])
        assert sorted(ids[t]) == sorted(ref["ids"][t]), (where, t, ids[t], ref["ids"][t])
        assert _order_ok(vq[t], ids[t, :kt]), (where, t, "slot order")
        for j in range(K):
            jj = int(np.nonzero(ref["ids"][t] == ids[t, j])[0][0])
            assert abs(w[t, j] - ref["weights"][t, jj]) <= WTOL, (where, t)

    # 3. near-ties at the k-th or group boundary: validity
    nt_idx = np.nonzero(near_tie)[0]
    if nt_idx.size:
        kw = orc.weights_for_ids(ref["logits"][nt_idx], ids[nt_idx], score=score,
                                 renormalize=renormalize, route_scale=route_scale)
        assert np.all(np.abs(kw - w[nt_idx]) <= WTOL), f"{where}: near-tie weights"
        E = vq.shape[1]
        grouped = n_groups > 1 and (topk_groups or n_groups) < n_groups and not k_per_group
        for t in nt_idx:
            kt = int(kt_all[t])
            S = ids[t, :kt]
            assert len(set(S.tolist())) == kt and S.min() >= 0 and S.max() < E, (where, t, ids[t])
            assert np.all(ids[t, kt:] == -1), (where, t)
            assert _order_ok(vq[t], S), (where, t, "slot order")
            if k_per_group:
                assert _quota_ok(vq[t], S, n_groups, k_per_group), (where, t, "quota", ids[t])
            elif grouped:
                assert _group_limit_ok(vq[t], ref["g"][t], S, n_groups, topk_groups), \
                    (where, t, "group limit", ids[t], ref["ids"][t])
            else:
                assert _exchange_ok(vq[t], S, np.arange(E)), (where, t, "k boundary", ids[t],
                                                              ref["ids"][t])
    return {"tokens": int(T), "near_tie": int(near_tie.sum()), "order_tie": int(order_tie.sum()),
            "max_dw": worst}


def oracle_route(orc, logits64, k, *, score, select_bias=None, k_per_token=None, n_groups=1,
                 topk_groups=None, group_score=None, renormalize=True, route_scale=1.0,
                 k_per_group=0, nthreads=1):
    """oracle.route_logits plus what check_route needs: the unmasked
    selection quantity q_raw = score + bias and whether the choice is a
    monotone function of the logit."""
    ref = orc.route_logits(logits64, k, score=score, select_bias=select_bias,
                           k_per_token=k_per_token, n_groups=n_groups, topk_groups=topk_groups,
                           group_score=group_score, renormalize=renormalize,
                           route_scale=route_scale, k_per_group=k_per_group,
                           nthreads=nthreads)
    ref["q_raw"] = orc.route_logits(logits64, 1, score=score, select_bias=select_bias,
                                    nthreads=nthreads)["q"]
    grouped = n_groups > 1 and (topk_groups or n_groups) < n_groups
    ref["monotone"] = select_bias is None and not grouped and not k_per_group
    return ref


def check_dispatch(gpu, ref):
    counts, offsets, perm, inv = (to_numpy(a) if a is not None else None for a in gpu[:4])
    np.testing.assert_array_equal(counts, ref["counts"])
    np.testing.assert_array_equal(offsets, ref["offsets"])
    R = int(ref["offsets"][-1])
    np.testing.assert_array_equal(perm[:R], ref["perm"])
    if inv is not None:
        np.testing.assert_array_equal(inv, ref["inv"])
