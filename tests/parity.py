"""Comparison of the HIP path's outputs with the oracle's (acceptance rule).

Expert ids must be bit-exact except on tokens whose selection margin at the
k-th boundary or at the kept-group boundary is below NEAR (1e-4, in units of
the quantity the selection compares: the logit when the choice is a monotone
function of it, else q = score + bias).  Such tokens are counted and checked
for validity: distinct in-range ids, every chosen expert within NEAR of the
oracle's boundary (and its group within NEAR of the kept-group boundary), and
weights equal to the oracle's weights for the GPU's own ids.  Tokens whose
selected experts are only separated by less than NEAR inside the row (slot
order) must select the same set.  Weights: |GPU - oracle| <= 1e-4.
Dispatch arrays: bit-exact against the oracle's dispatch of the GPU's ids."""
from __future__ import annotations

import numpy as np

NEAR = 1e-4
WTOL = 1e-4


def to_numpy(t):
    return t.detach().cpu().numpy()


def check_route(gpu_ids, gpu_w, ref, orc, *, score, renormalize=True, route_scale=1.0,
                k_per_token=None, n_groups=1, topk_groups=None, k_per_group=0, where=""):
    """Compare a route result with oracle output `ref` (oracle.route_logits dict).

    Returns statistics; raises AssertionError on any violation."""
    ids = np.asarray(gpu_ids)
    w = np.asarray(gpu_w, dtype=np.float64)
    T, K = ids.shape
    assert ref["ids"].shape == (T, K), (ref["ids"].shape, ids.shape, where)
    mk, mg, mo = ref["margin_k"], ref["margin_g"], ref["margin_o"]
    near_tie = np.minimum(mk, mg) < NEAR
    order_tie = (~near_tie) & (mo < NEAR)
    exact = ~(near_tie | order_tie)

    # 1. exact tokens: bit-exact ids, weights within WTOL
    bad = np.nonzero(exact & np.any(ids != ref["ids"], axis=1))[0]
    assert bad.size == 0, (f"{where}: {bad.size} tokens with ids != oracle (margins "
                           f"{mk[bad[:3]]}, {mg[bad[:3]]}); first t={bad[0]}: gpu "
                           f"{ids[bad[0]]} oracle {ref['ids'][bad[0]]}")
    dw = np.abs(w - ref["weights"])
    worst = float(dw[exact].max()) if exact.any() else 0.0
    assert worst <= WTOL, f"{where}: max |dw| = {worst:.3g} > {WTOL}"

    # 2. slot-order near-ties: same set, weights follow the ids
    for t in np.nonzero(order_tie)[0]:
        assert sorted(ids[t]) == sorted(ref["ids"][t]), (where, t, ids[t], ref["ids"][t])
        for j in range(K):
            jj = int(np.nonzero(ref["ids"][t] == ids[t, j])[0][0])
            assert abs(w[t, j] - ref["weights"][t, jj]) <= WTOL, (where, t)

    # 3. near-ties at the k-th or group boundary: validity
    nt_idx = np.nonzero(near_tie)[0]
    if nt_idx.size:
        kw = orc.weights_for_ids(ref["logits"][nt_idx], ids[nt_idx], score=score,
                                 renormalize=renormalize, route_scale=route_scale)
        assert np.all(np.abs(kw - w[nt_idx]) <= WTOL), f"{where}: near-tie weights"
        monotone = ref.get("monotone", False)
        for i, t in enumerate(nt_idx):
            kt = K if k_per_token is None else int(k_per_token[t])
            row = ids[t, :kt]
            assert len(set(row.tolist())) == kt and row.min() >= 0, (where, t, ids[t])
            assert np.all(ids[t, kt:] == -1)
            if mg[t] < NEAR and k_per_group:
                # a near-tie at a group's cut: at most k_per_group per group,
                # each pick within NEAR of its group's last kept q and of the
                # global boundary (in the unmasked q)
                gs = ref["q"].shape[1] // n_groups
                assert np.bincount(row // gs, minlength=n_groups).max() <= k_per_group, (where, t)
                qr = ref["q_raw"][t]
                assert np.all(qr[row] >= ref["g"][t][row // gs] - NEAR), (where, t, "group cut")
                assert np.all(qr[row] >= ref["q_boundary"][t] - NEAR), (where, t, "k boundary")
            elif mg[t] < NEAR and n_groups > 1:
                g = ref["g"][t]
                gb = np.sort(g)[::-1][topk_groups - 1]
                gs = ref["q"].shape[1] // n_groups
                assert np.all(g[row // gs] >= gb - NEAR), (where, t, "group")
            else:
                qv = ref["logits"][t] if monotone else ref["q"][t]
                qb = ref["q_boundary"][t]
                assert np.all(qv[row] >= qb - NEAR), (where, t, "k boundary")
    return {"tokens": int(T), "near_tie": int(near_tie.sum()), "order_tie": int(order_tie.sum()),
            "max_dw": worst}


def oracle_route(orc, logits64, k, *, score, select_bias=None, k_per_token=None, n_groups=1,
                 topk_groups=None, group_score=None, renormalize=True, route_scale=1.0,
                 k_per_group=0):
    """oracle.route_logits plus the boundary value used by check_route (and,
    with a per-group quota, the unmasked q)."""
    ref = orc.route_logits(logits64, k, score=score, select_bias=select_bias,
                           k_per_token=k_per_token, n_groups=n_groups, topk_groups=topk_groups,
                           group_score=group_score, renormalize=renormalize,
                           route_scale=route_scale, k_per_group=k_per_group)
    if k_per_group:
        ref["q_raw"] = orc.route_logits(logits64, 1, score=score, select_bias=select_bias)["q"]
    grouped = n_groups > 1 and (topk_groups or n_groups) < n_groups
    monotone = select_bias is None and not grouped and not k_per_group
    T = logits64.shape[0]
    kt = np.full(T, k) if k_per_token is None else np.asarray(k_per_token)
    qb = np.empty(T)
    for t in range(T):
        qv = logits64[t] if monotone else ref["q"][t]
        kk = int(min(max(kt[t], 1), k))
        qb[t] = np.sort(qv)[::-1][kk - 1]
    ref["monotone"] = monotone
    ref["q_boundary"] = qb
    return ref


def check_dispatch(gpu, ref):
    counts, offsets, perm, inv = (to_numpy(a) if a is not None else None for a in gpu)
    np.testing.assert_array_equal(counts, ref["counts"])
    np.testing.assert_array_equal(offsets, ref["offsets"])
    R = int(ref["offsets"][-1])
    np.testing.assert_array_equal(perm[:R], ref["perm"])
    if inv is not None:
        np.testing.assert_array_equal(inv, ref["inv"])
