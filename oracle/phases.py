"""The PrefixFlow phases and the HARTS tree case, each as plain full attention.

PrefixFlow's schedule (PrefixFlow §3.1) reaches exactly the result of
training every trajectory [P || S_i] as an independent full sequence, so the
oracle computes that full-sequence result and slices it:

* Phase A (prefix forward): causal attention over the prefix alone.
* Phase B (one suffix at a time): the rows of trajectory [P || S_i] that
  belong to S_i.  Outputs O_S and LSE_S are those rows of the full
  trajectory.  The backward takes upstream [0_P ; dO_S]; the trajectory's
  dK, dV rows of the prefix are that suffix's gK^i, gV^i, and its suffix rows
  are dK_S, dV_S.  gK = sum_i gK^i, in suffix order (the accumulated
  gradient-KV cache of PrefixFlow §3.3 and §4.1).
* Phase C (prefix backward with injection): causal prefix backward under
  upstream dO_P, plus the accumulated gK, gV added to the prefix K/V
  gradients (PrefixFlow §4.1: hooks add the cached-leaf gradients to the live
  prefix K/V before the prefix graph is traversed).

`suffix_attention` evaluates only the suffix rows of each trajectory.  The
prefix rows carry zero upstream in Phase B, so they add nothing to any
gradient; `suffix_attention_full_rows` evaluates every row of every
trajectory, exactly as the definition reads, and a test checks that both
agree.

Trees (HARTS §2.1, §2.2 and §3): `tree_attention_direct` applies the ancestor
mask to the compact rows; `tree_attention_expanded` runs causal attention on
every root-to-leaf trajectory and sums the per-occurrence gradients back into
the shared compact rows (HARTS §3.4: gather backward sums into the shared
compact activations).

Test infrastructure only.
"""
from typing import Dict, List, Optional

import numpy as np

from .attention import attention_backward, attention_forward
from .masks import causal_mask, suffix_rows_mask, tree_ancestor_mask


def prefix_forward(q_p, k_p, v_p, scale, hmap, dtype=np.float64):
    """Phase A: (O_P [P, Hq, d], LSE_P [Hq, P])."""
    return attention_forward(q_p, k_p, v_p, causal_mask(q_p.shape[0]), scale, hmap, dtype)


def suffix_attention(k_p, v_p, q_s, k_s, v_s, do_s, cu_seqlens, scale, hmap,
                     dtype=np.float64, backward=True) -> Dict[str, np.ndarray]:
    """Phase B over the packed suffixes of one call.

    Returns o_s, lse_s and (if backward) dq_s, dk_s, dv_s, gk, gv where gk, gv
    [P, Hkv, d] are this call's prefix-side gradients summed over its suffixes.
    """
    p = k_p.shape[0]
    t, hq, d = q_s.shape
    hkv = k_p.shape[1]
    res = {
        "o_s": np.zeros((t, hq, d), dtype), "lse_s": np.zeros((hq, t), dtype),
    }
    if backward:
        res.update(dq_s=np.zeros((t, hq, d), dtype), dk_s=np.zeros((t, hkv, d), dtype),
                   dv_s=np.zeros((t, hkv, d), dtype), gk=np.zeros((p, hkv, d), dtype),
                   gv=np.zeros((p, hkv, d), dtype))
    for i in range(len(cu_seqlens) - 1):
        a, b = int(cu_seqlens[i]), int(cu_seqlens[i + 1])
        if b == a:
            continue
        k_traj = np.concatenate([k_p, k_s[a:b]], axis=0)
        v_traj = np.concatenate([v_p, v_s[a:b]], axis=0)
        vis = suffix_rows_mask(p, b - a)
        o, lse = attention_forward(q_s[a:b], k_traj, v_traj, vis, scale, hmap, dtype)
        res["o_s"][a:b] = o
        res["lse_s"][:, a:b] = lse
        if backward:
            dq, dk, dv = attention_backward(q_s[a:b], k_traj, v_traj, do_s[a:b], vis, scale,
                                            hmap, dtype)
            res["dq_s"][a:b] = dq
            res["dk_s"][a:b] = dk[p:]
            res["dv_s"][a:b] = dv[p:]
            res["gk"] += dk[:p]
            res["gv"] += dv[:p]
    return res


def suffix_attention_full_rows(q_p, k_p, v_p, q_s, k_s, v_s, do_s, cu_seqlens, scale, hmap,
                               dtype=np.float64) -> Dict[str, np.ndarray]:
    """Phase B by the literal definition: every row of each trajectory [P || S_i],
    upstream [0_P ; dO_S], then slicing.  Slow; for small tests."""
    p = k_p.shape[0]
    t, hq, d = q_s.shape
    hkv = k_p.shape[1]
    res = {k: None for k in ("o_s", "lse_s", "dq_s", "dk_s", "dv_s")}
    o_s = np.zeros((t, hq, d), dtype)
    lse_s = np.zeros((hq, t), dtype)
    dq_s = np.zeros((t, hq, d), dtype)
    dk_s = np.zeros((t, hkv, d), dtype)
    dv_s = np.zeros((t, hkv, d), dtype)
    gk = np.zeros((p, hkv, d), dtype)
    gv = np.zeros((p, hkv, d), dtype)
    for i in range(len(cu_seqlens) - 1):
        a, b = int(cu_seqlens[i]), int(cu_seqlens[i + 1])
        if b == a:
            continue
        q_traj = np.concatenate([q_p, q_s[a:b]], axis=0)
        k_traj = np.concatenate([k_p, k_s[a:b]], axis=0)
        v_traj = np.concatenate([v_p, v_s[a:b]], axis=0)
        do_traj = np.concatenate([np.zeros((p, hq, d), dtype), do_s[a:b]], axis=0)
        vis = causal_mask(p + b - a)
        o, lse = attention_forward(q_traj, k_traj, v_traj, vis, scale, hmap, dtype)
        dq, dk, dv = attention_backward(q_traj, k_traj, v_traj, do_traj, vis, scale, hmap, dtype)
        o_s[a:b], lse_s[:, a:b] = o[p:], lse[:, p:]
        dq_s[a:b], dk_s[a:b], dv_s[a:b] = dq[p:], dk[p:], dv[p:]
        gk += dk[:p]
        gv += dv[:p]
    res.update(o_s=o_s, lse_s=lse_s, dq_s=dq_s, dk_s=dk_s, dv_s=dv_s, gk=gk, gv=gv)
    return res


def prefix_backward_inject(q_p, k_p, v_p, do_p, gk_acc, gv_acc, scale, hmap,
                           dtype=np.float64):
    """Phase C: (dQ_P, dK_P, dV_P) with dK_P = dK_self + gK_acc, dV_P = dV_self + gV_acc.

    do_p=None means a zero upstream (a suffix-only loss above this layer)."""
    if do_p is None:
        do_p = np.zeros(q_p.shape, dtype)
    dq, dk, dv = attention_backward(q_p, k_p, v_p, do_p, causal_mask(q_p.shape[0]), scale,
                                    hmap, dtype)
    return dq, dk + gk_acc, dv + gv_acc


def tree_attention_direct(q, k, v, do, node_off, parent, scale, hmap, dtype=np.float64,
                          backward=True):
    vis = tree_ancestor_mask(node_off, parent)
    o, lse = attention_forward(q, k, v, vis, scale, hmap, dtype)
    out = {"o": o, "lse": lse}
    if backward:
        out["dq"], out["dk"], out["dv"] = attention_backward(q, k, v, do, vis, scale, hmap, dtype)
    return out


def tree_trajectories(node_off: np.ndarray, parent: np.ndarray) -> List[np.ndarray]:
    """Compact row indices of every root-to-leaf trajectory (leaves in node order)."""
    n = len(parent)
    has_child = np.zeros(n, dtype=bool)
    for v in range(1, n):
        has_child[parent[v]] = True
    trajs = []
    for leaf in range(n):
        if has_child[leaf]:
            continue
        path = []
        u = leaf
        while u >= 0:
            path.append(u)
            u = int(parent[u])
        rows = np.concatenate([np.arange(node_off[u], node_off[u + 1]) for u in reversed(path)])
        trajs.append(rows)
    return trajs


def tree_attention_expanded(q, k, v, do, node_off, parent, scale, hmap,
                            rng: Optional[np.random.Generator] = None, dtype=np.float64):
    """Trees by expansion into independent causal trajectories.

    The upstream dO of a compact row is split across the row's occurrences
    with random weights summing to one (any split gives the same compact
    gradients, since the backward is linear in the upstream)."""
    c, hq, d = q.shape
    hkv = k.shape[1]
    trajs = tree_trajectories(node_off, parent)
    occ = np.zeros(c, dtype=np.int64)
    for rows in trajs:
        occ[rows] += 1
    # random split weights per (trajectory, row)
    weights = []
    if rng is None:
        rng = np.random.Generator(np.random.PCG64(12345))
    remaining = np.ones(c, dtype)
    seen = np.zeros(c, dtype=np.int64)
    for rows in trajs:
        seen[rows] += 1
        last = seen[rows] == occ[rows]
        wr = np.where(last, remaining[rows], rng.uniform(0, 1, size=len(rows)) * remaining[rows])
        remaining[rows] -= wr
        weights.append(wr)
    o = np.full((c, hq, d), np.nan, dtype)
    lse = np.full((hq, c), np.nan, dtype)
    spread = 0.0
    dq = np.zeros((c, hq, d), dtype)
    dk = np.zeros((c, hkv, d), dtype)
    dv = np.zeros((c, hkv, d), dtype)
    for rows, wr in zip(trajs, weights):
        L = len(rows)
        vis = causal_mask(L)
        ot, lt = attention_forward(q[rows], k[rows], v[rows], vis, scale, hmap, dtype)
        # every occurrence of a row must give the same forward result
        prev = ~np.isnan(lse[0, rows])
        if prev.any():
            spread = max(spread, float(np.abs(o[rows][prev] - ot[prev]).max()))
        o[rows] = ot
        lse[:, rows] = lt
        do_t = do[rows].astype(dtype) * wr[:, None, None]
        dqt, dkt, dvt = attention_backward(q[rows], k[rows], v[rows], do_t, vis, scale, hmap,
                                           dtype)
        np.add.at(dq, rows, dqt)
        np.add.at(dk, rows, dkt)
        np.add.at(dv, rows, dvt)
    return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv,
            "forward_spread": spread}


def tree_window_attention(k_p, v_p, q, k, v, do, node_off, parent, scale, hmap,
                          dtype=np.float64, backward=True) -> Dict[str, np.ndarray]:
    """One sharing window of rollout trees over a cached prefix (HARTS §3.4,
    "Window-scoped reuse and backward": a producer forward caches the ancestor
    K/V once; the consumers of a window run only their uncached tokens, and
    their backward passes accumulate the gradients at that interface before
    the one producer backward).

    The window's compact rows (DFS preorder, node_off / parent as for trees)
    all sit after the P prefix positions of every trajectory they belong to,
    so a row sees every prefix key and, through the ancestor mask, its own
    node up to itself and every ancestor node (HARTS §2.2).  Full attention
    over [prefix ; window rows] with that mask gives o, lse of the window rows;
    the backward under upstream [0_P ; dO] gives dq, dk, dv of the window rows
    and, in the prefix rows of dK, dV, this window's gk, gv.
    """
    p = k_p.shape[0]
    c = q.shape[0]
    tvis = tree_ancestor_mask(node_off, parent)
    vis = np.concatenate([np.ones((c, p), dtype=bool), tvis], axis=1)      # [C, P + C]
    k_all = np.concatenate([k_p, k], axis=0)
    v_all = np.concatenate([v_p, v], axis=0)
    o, lse = attention_forward(q, k_all, v_all, vis, scale, hmap, dtype)
    out = {"o": o, "lse": lse}
    if backward:
        dq, dk_all, dv_all = attention_backward(q, k_all, v_all, do, vis, scale, hmap, dtype)
        out.update(dq=dq, dk=dk_all[p:], dv=dv_all[p:], gk=dk_all[:p], gv=dv_all[:p])
    return out



def tree_window_attention_ranges(k_c, v_c, ranges, q, k, v, do, node_off, parent, scale, hmap,
                                 dtype=np.float64, backward=True) -> Dict[str, np.ndarray]:
    """A sharing window whose cached rows are row ranges of a producer's
    compact rows (HARTS §3.4, "Window-scoped reuse and backward": the producer
    caches ancestor K/V; each internal node of a rollout tree can carry such a
    cache, so a consumer attached under node u reads the rows of u and of its
    ancestors).

    `ranges` lists (start, length) spans of k_c / v_c [C_prod, Hkv, d]; their
    rows, concatenated in list order, precede the window's rows in every
    window trajectory.  By the definition of the gather: gather those rows,
    run `tree_window_attention` over them, and add the gathered rows'
    gradients back into the producer rows they came from (the gather's
    backward sums into the shared rows).  gk, gv are [C_prod, Hkv, d]."""
    idx = [np.arange(int(s), int(s) + int(n)) for s, n in ranges]
    rows = np.concatenate(idx) if idx else np.zeros(0, dtype=np.int64)
    res = tree_window_attention(k_c[rows], v_c[rows], q, k, v, do, node_off, parent, scale, hmap,
                                dtype, backward)
    if backward:
        gk = np.zeros(k_c.shape, dtype)
        gv = np.zeros(v_c.shape, dtype)
        np.add.at(gk, rows, res["gk"])
        np.add.at(gv, rows, res["gv"])
        res["gk"], res["gv"] = gk, gv
    return res


def tree_backward_inject(q, k, v, do, node_off, parent, gk_acc, gv_acc, scale, hmap,
                         dtype=np.float64):
    """The producer backward of a rollout tree whose rows were read by consumer
    windows (HARTS §3.4: the consumers' interface gradients are accumulated
    before the one producer backward): the tree backward under upstream dO,
    with gK/gV added to the K/V gradients of the compact rows.
    Returns (dQ, dK + gK_acc, dV + gV_acc)."""
    if do is None:
        do = np.zeros(q.shape, dtype)
    r = tree_attention_direct(q, k, v, do, node_off, parent, scale, hmap, dtype)
    return r["dq"], r["dk"] + gk_acc, r["dv"] + gv_acc
