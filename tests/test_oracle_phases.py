"""Pins for the oracle's phase-level functions (Phase A/B/C and trees).

* Row identity: evaluating only suffix rows equals the literal full-trajectory
  definition (PrefixFlow §3.1, regrouping into four parts).
* Packed-graph formulation: one sequence [P; S_1; ...; S_N] with the flat
  group mask, differentiated by torch autograd, gives the prefix-side
  gradients summed over suffixes (the single-graph designs of PrefixFlow §2.2),
  so it pins superposition (§3.3) and Phase C's injection (§4.1) through an
  independent route.
* Closed form at Q = 0 (uniform attention) and the single-visible-key row.
* Trees: expansion into trajectories vs the direct ancestor mask; the preorder
  interval rule vs the ancestor definition on random trees; a depth-2 tree is
  a flat group; a chain is one causal sequence (HARTS §2.1, §2.2, §3).
"""
import math

import numpy as np
import pytest
import torch

from oracle import (
    head_map,
    prefix_backward_inject,
    prefix_forward,
    suffix_attention,
    suffix_attention_full_rows,
    tree_ancestor_mask,
    tree_attention_direct,
    tree_attention_expanded,
    tree_backward_inject,
    tree_trajectories,
    tree_window_attention,
    tree_window_attention_ranges,
)
from workloads.gen import (
    ancestor_row_ranges,
    node_depths,
    random_small_group,
    random_tree,
    random_tree_group,
    tree_layout,
)


def _group(seed=0, hq=4, hkv=2, d=8, p=5, lens=(1, 2, 4), scale_q=1.0):
    g = random_small_group(seed, hq, hkv, d, p, list(lens), "f32", scale_q=scale_q)
    return {k: (v.astype(np.float64) if v.dtype == np.float32 else v) for k, v in g.items()}


def test_suffix_rows_equal_full_trajectory_rows():
    g = _group(seed=1, lens=(3, 0, 5, 1))
    hmap = head_map(4, 2)
    a = suffix_attention(g["k_p"], g["v_p"], g["q_s"], g["k_s"], g["v_s"], g["do_s"],
                         g["cu_seqlens"], 0.3, hmap)
    b = suffix_attention_full_rows(g["q_p"], g["k_p"], g["v_p"], g["q_s"], g["k_s"], g["v_s"],
                                   g["do_s"], g["cu_seqlens"], 0.3, hmap)
    for key in ("o_s", "lse_s", "dq_s", "dk_s", "dv_s", "gk", "gv"):
        np.testing.assert_allclose(a[key], b[key], rtol=1e-13, atol=1e-13, err_msg=key)


def _flat_group_mask(p, cu):
    """Packed [P; S_1..S_N]: prefix causal; suffix i sees the prefix and itself causally."""
    t = int(cu[-1])
    n = p + t
    vis = np.zeros((n, n), dtype=bool)
    vis[:p, :p] = np.tril(np.ones((p, p), dtype=bool))
    for i in range(len(cu) - 1):
        a, b = p + int(cu[i]), p + int(cu[i + 1])
        vis[a:b, :p] = True
        vis[a:b, a:b] = np.tril(np.ones((b - a, b - a), dtype=bool))
    return vis


def _torch_packed(q, k, v, do, vis, scale, hmap):
    tq = torch.tensor(q, dtype=torch.float64, requires_grad=True)
    tk = torch.tensor(k, dtype=torch.float64, requires_grad=True)
    tv = torch.tensor(v, dtype=torch.float64, requires_grad=True)
    idx = torch.tensor(hmap)
    z = scale * torch.einsum("qhd,khd->hqk", tq, tk[:, idx, :])
    z = z.masked_fill(~torch.tensor(vis)[None], float("-inf"))
    o = torch.einsum("hqk,khd->qhd", torch.softmax(z, -1), tv[:, idx, :])
    lse = torch.logsumexp(z, -1)
    o.backward(torch.tensor(do))
    return o.detach().numpy(), lse.detach().numpy(), tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("lens,hq,hkv", [((1, 2, 4), 4, 2), ((3, 3), 2, 2), ((6, 0, 2, 5), 6, 2)])
def test_three_phases_equal_packed_graph(lens, hq, hkv):
    p = 6
    g = random_small_group(3, hq, hkv, 8, p, list(lens), "f32")
    cu = g["cu_seqlens"]
    hmap = head_map(hq, hkv)
    scale = 1 / math.sqrt(8)
    q = np.concatenate([g["q_p"], g["q_s"]]).astype(np.float64)
    k = np.concatenate([g["k_p"], g["k_s"]]).astype(np.float64)
    v = np.concatenate([g["v_p"], g["v_s"]]).astype(np.float64)
    do = np.concatenate([g["do_p"], g["do_s"]]).astype(np.float64)
    ro, rlse, rdq, rdk, rdv = _torch_packed(q, k, v, do, _flat_group_mask(p, cu), scale, hmap)
    # Phase A
    o_p, lse_p = prefix_forward(g["q_p"], g["k_p"], g["v_p"], scale, hmap)
    np.testing.assert_allclose(o_p, ro[:p], atol=1e-12)
    np.testing.assert_allclose(lse_p, rlse[:, :p], atol=1e-12)
    # Phase B
    b = suffix_attention(g["k_p"], g["v_p"], g["q_s"], g["k_s"], g["v_s"], g["do_s"], cu, scale,
                         hmap)
    np.testing.assert_allclose(b["o_s"], ro[p:], atol=1e-12)
    np.testing.assert_allclose(b["lse_s"], rlse[:, p:], atol=1e-12)
    np.testing.assert_allclose(b["dq_s"], rdq[p:], atol=1e-12)
    np.testing.assert_allclose(b["dk_s"], rdk[p:], atol=1e-12)
    np.testing.assert_allclose(b["dv_s"], rdv[p:], atol=1e-12)
    # Phase C with the accumulated gK/gV injected
    dq_p, dk_p, dv_p = prefix_backward_inject(g["q_p"], g["k_p"], g["v_p"], g["do_p"], b["gk"],
                                              b["gv"], scale, hmap)
    np.testing.assert_allclose(dq_p, rdq[:p], atol=1e-12)
    np.testing.assert_allclose(dk_p, rdk[:p], atol=1e-12)
    np.testing.assert_allclose(dv_p, rdv[:p], atol=1e-12)


def test_superposition_over_microbatch_splits():
    """Sum of per-call gK/gV is the same for every partition and order of the suffixes."""
    g = _group(seed=5, lens=(2, 3, 1, 4, 2))
    hmap = head_map(4, 2)
    cu = g["cu_seqlens"]

    def call(idx):
        rows = np.concatenate([np.arange(cu[i], cu[i + 1]) for i in idx])
        sub_cu = np.concatenate([[0], np.cumsum([cu[i + 1] - cu[i] for i in idx])])
        return suffix_attention(g["k_p"], g["v_p"], g["q_s"][rows], g["k_s"][rows],
                                g["v_s"][rows], g["do_s"][rows], sub_cu, 0.4, hmap)

    whole = call([0, 1, 2, 3, 4])
    for split in ([[0], [1], [2], [3], [4]], [[4, 2], [0, 3, 1]], [[1, 0], [2], [3, 4]]):
        gk = sum(call(s)["gk"] for s in split)
        gv = sum(call(s)["gv"] for s in split)
        np.testing.assert_allclose(gk, whole["gk"], atol=1e-13)
        np.testing.assert_allclose(gv, whole["gv"], atol=1e-13)


def test_closed_form_uniform_attention():
    """Q = 0: every visible key gets weight 1/n_q; dK = 0; dV_k = sum_{q sees k} dO_q / n_q."""
    p, lens = 4, (3, 2)
    g = _group(seed=9, p=p, lens=lens, scale_q=0.0)
    hmap = head_map(4, 2)
    cu = g["cu_seqlens"]
    b = suffix_attention(g["k_p"], g["v_p"], g["q_s"], g["k_s"], g["v_s"], g["do_s"], cu, 0.5,
                         hmap)
    gk_ref = np.zeros_like(b["gk"])
    gv_ref = np.zeros_like(b["gv"])
    dv_s_ref = np.zeros_like(b["dv_s"])
    for i in range(len(cu) - 1):
        for j in range(cu[i + 1] - cu[i]):
            r = cu[i] + j
            n = p + j + 1
            for h in range(4):
                kv = hmap[h]
                vis_v = np.concatenate([g["v_p"][:, kv], g["v_s"][cu[i]:r + 1, kv]]).astype(np.float64)
                np.testing.assert_allclose(b["o_s"][r, h], vis_v.mean(axis=0), atol=1e-13)
                assert abs(b["lse_s"][h, r] - math.log(n)) < 1e-13
                gv_ref[:, kv] += g["do_s"][r, h].astype(np.float64) / n
                dv_s_ref[cu[i]:r + 1, kv] += g["do_s"][r, h].astype(np.float64) / n
    np.testing.assert_allclose(b["gk"], 0.0, atol=1e-14)
    np.testing.assert_allclose(b["dk_s"], 0.0, atol=1e-14)
    np.testing.assert_allclose(b["gv"], gv_ref, atol=1e-12)
    np.testing.assert_allclose(b["dv_s"], dv_s_ref, atol=1e-12)


def test_closed_form_single_visible_key():
    """Row 0 of a causal prefix sees only key 0: O = V_0, LSE = s q.k, dQ = 0."""
    g = _group(seed=2, p=5)
    hmap = head_map(4, 2)
    o, lse = prefix_forward(g["q_p"], g["k_p"], g["v_p"], 0.6, hmap)
    dq, _, _ = prefix_backward_inject(g["q_p"], g["k_p"], g["v_p"], g["do_p"],
                                      np.zeros_like(g["k_p"]), np.zeros_like(g["v_p"]), 0.6, hmap)
    for h in range(4):
        np.testing.assert_allclose(o[0, h], g["v_p"][0, hmap[h]], atol=1e-14)
        assert abs(lse[h, 0] - 0.6 * g["q_p"][0, h] @ g["k_p"][0, hmap[h]]) < 1e-12
        np.testing.assert_allclose(dq[0, h], 0.0, atol=1e-14)


def test_phase_c_zero_upstream_is_injection():
    """With no prefix upstream, dQ_P = 0 and dK_P, dV_P are exactly the accumulators."""
    g = _group(seed=4, p=6)
    hmap = head_map(4, 2)
    rng = np.random.default_rng(0)
    gk, gv = rng.standard_normal(g["k_p"].shape), rng.standard_normal(g["v_p"].shape)
    dq, dk, dv = prefix_backward_inject(g["q_p"], g["k_p"], g["v_p"], None, gk, gv, 0.5, hmap)
    assert np.all(dq == 0)
    np.testing.assert_array_equal(dk, gk)
    np.testing.assert_array_equal(dv, gv)


def test_no_cross_suffix_leakage():
    g = _group(seed=6, lens=(3, 4, 2))
    hmap = head_map(4, 2)
    cu = g["cu_seqlens"]
    a = suffix_attention(g["k_p"], g["v_p"], g["q_s"], g["k_s"], g["v_s"], g["do_s"], cu, 0.5, hmap)
    k2 = g["k_s"].copy()
    k2[cu[1]:cu[2]] += 1.0                      # perturb suffix 1 only
    b = suffix_attention(g["k_p"], g["v_p"], g["q_s"], k2, g["v_s"], g["do_s"], cu, 0.5, hmap)
    for rows in (slice(cu[0], cu[1]), slice(cu[2], cu[3])):
        np.testing.assert_array_equal(a["o_s"][rows], b["o_s"][rows])
        np.testing.assert_array_equal(a["dq_s"][rows], b["dq_s"][rows])


# ----------------------------------------------------------------------------- trees

def _subtree_end(node_off, parent):
    n = len(parent)
    end = np.asarray(node_off[1:], dtype=np.int64).copy()
    for v in range(n - 1, 0, -1):
        end[parent[v]] = max(end[parent[v]], end[v])
    return end


def test_preorder_interval_rule_matches_ancestor_mask():
    """k visible to q  <=>  k <= q and q < subtree_end(node(k)), for trees in preorder."""
    for seed in range(200):
        rng = np.random.default_rng(seed)
        n = int(rng.integers(1, 12))
        node_off, parent = random_tree(seed, n, max_len=4)
        vis = tree_ancestor_mask(node_off, parent)
        end = _subtree_end(node_off, parent)
        c = int(node_off[-1])
        node = np.searchsorted(node_off, np.arange(c), side="right") - 1
        kend = end[node]
        rows = np.arange(c)
        rule = (rows[None, :] <= rows[:, None]) & (rows[:, None] < kend[None, :])
        np.testing.assert_array_equal(rule, vis, err_msg=f"seed {seed}")


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tree_expanded_equals_direct(seed):
    node_off, parent = random_tree(seed, 7, max_len=5)
    g = random_tree_group(seed, node_off, 4, 2, 8)
    hmap = head_map(4, 2)
    a = tree_attention_direct(g["q"], g["k"], g["v"], g["do"], node_off, parent, 0.35, hmap)
    b = tree_attention_expanded(g["q"], g["k"], g["v"], g["do"], node_off, parent, 0.35, hmap,
                                rng=np.random.default_rng(seed))
    assert b["forward_spread"] < 1e-13
    for key in ("o", "lse", "dq", "dk", "dv"):
        np.testing.assert_allclose(a[key], b[key], atol=1e-12, err_msg=key)


def test_depth2_tree_is_flat_group():
    p, lens = 5, (2, 3, 1)
    g = random_small_group(8, 4, 2, 8, p, list(lens), "f32")
    node_off = np.concatenate([[0], p + g["cu_seqlens"]]).astype(np.int32)
    parent = np.asarray([-1] + [0] * len(lens), dtype=np.int32)
    cat = lambda a, b: np.concatenate([g[a], g[b]])
    hmap = head_map(4, 2)
    t = tree_attention_direct(cat("q_p", "q_s"), cat("k_p", "k_s"), cat("v_p", "v_s"),
                              cat("do_p", "do_s"), node_off, parent, 0.5, hmap)
    o_p, _ = prefix_forward(g["q_p"], g["k_p"], g["v_p"], 0.5, hmap)
    b = suffix_attention(g["k_p"], g["v_p"], g["q_s"], g["k_s"], g["v_s"], g["do_s"],
                         g["cu_seqlens"], 0.5, hmap)
    dq_p, dk_p, dv_p = prefix_backward_inject(g["q_p"], g["k_p"], g["v_p"], g["do_p"], b["gk"],
                                              b["gv"], 0.5, hmap)
    np.testing.assert_allclose(t["o"][:p], o_p, atol=1e-13)
    np.testing.assert_allclose(t["o"][p:], b["o_s"], atol=1e-13)
    np.testing.assert_allclose(t["dq"], np.concatenate([dq_p, b["dq_s"]]), atol=1e-12)
    np.testing.assert_allclose(t["dk"], np.concatenate([dk_p, b["dk_s"]]), atol=1e-12)
    np.testing.assert_allclose(t["dv"], np.concatenate([dv_p, b["dv_s"]]), atol=1e-12)


def test_chain_tree_is_causal():
    node_off = np.asarray([0, 3, 5, 9], dtype=np.int32)
    parent = np.asarray([-1, 0, 1], dtype=np.int32)
    vis = tree_ancestor_mask(node_off, parent)
    np.testing.assert_array_equal(vis, np.tril(np.ones((9, 9), dtype=bool)))


def test_config5_tree_layout():
    """Root 4096, four children of 1024, four leaves of 256 under each: 21 nodes, 16 paths."""
    node_off, parent = tree_layout(((1, 4096), (4, 1024), (4, 256)))
    assert len(parent) == 21 and int(node_off[-1]) == 12288
    trajs = tree_trajectories(node_off, parent)
    assert len(trajs) == 16 and all(len(t) == 4096 + 1024 + 256 for t in trajs)
    assert sum(len(t) for t in trajs) == 86016
    end = _subtree_end(node_off, parent)
    assert end[0] == 12288 and end[1] == 4096 + 1024 + 4 * 256


def _window(seed, p, n_nodes=7, max_len=6, hq=4, hkv=2, d=8):
    node_off, parent = random_tree(seed, n_nodes, max_len=max_len, min_len=1)
    g = random_tree_group(seed, node_off, hq, hkv, d)
    rng = np.random.default_rng(seed + 77)
    g["k_p"] = rng.standard_normal((p, hkv, d))
    g["v_p"] = rng.standard_normal((p, hkv, d))
    return node_off, parent, {k: np.asarray(v, dtype=np.float64) for k, v in g.items()}


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tree_window_equals_flat_phase_b_per_trajectory(seed):
    """A window of trees over a prefix, by expansion: every root-to-leaf
    trajectory is one flat Phase-B suffix [P || path] (suffix_attention, the
    flat-suffix mask), with each compact row's upstream split at random over
    the trajectories that contain it.  Forward rows must agree with the
    compact result wherever they occur; compact dQ/dK/dV are the sums over
    occurrences, and gK/gV the sum over trajectories (linearity in dO)."""
    p = 6
    node_off, parent, g = _window(seed, p)
    hmap = head_map(4, 2)
    ref = tree_window_attention(g["k_p"], g["v_p"], g["q"], g["k"], g["v"], g["do"], node_off,
                                parent, 0.4, hmap)
    trajs = tree_trajectories(node_off, parent)
    c = int(node_off[-1])
    occ = np.zeros(c, dtype=np.int64)
    for rows in trajs:
        occ[rows] += 1
    rng = np.random.default_rng(seed + 5)
    left = np.ones(c)
    seen = np.zeros(c, dtype=np.int64)
    dq = np.zeros_like(g["q"])
    dk = np.zeros_like(g["k"])
    dv = np.zeros_like(g["v"])
    gk = np.zeros_like(g["k_p"])
    gv = np.zeros_like(g["v_p"])
    for rows in trajs:
        seen[rows] += 1
        w = np.where(seen[rows] == occ[rows], left[rows], rng.uniform(0, 1, len(rows)) * left[rows])
        left[rows] -= w
        r = suffix_attention(g["k_p"], g["v_p"], g["q"][rows], g["k"][rows], g["v"][rows],
                             g["do"][rows] * w[:, None, None], np.asarray([0, len(rows)]), 0.4,
                             hmap)
        np.testing.assert_allclose(r["o_s"], ref["o"][rows], atol=1e-12)
        np.testing.assert_allclose(r["lse_s"], ref["lse"][:, rows], atol=1e-12)
        np.add.at(dq, rows, r["dq_s"])
        np.add.at(dk, rows, r["dk_s"])
        np.add.at(dv, rows, r["dv_s"])
        gk += r["gk"]
        gv += r["gv"]
    np.testing.assert_allclose(left, 0.0, atol=1e-12)
    for name, got in (("dq", dq), ("dk", dk), ("dv", dv), ("gk", gk), ("gv", gv)):
        np.testing.assert_allclose(got, ref[name], atol=1e-11, err_msg=name)


def test_tree_window_chain_is_one_flat_suffix():
    """A chain of nodes is one trajectory: the window equals Phase B with one suffix."""
    p = 5
    node_off = np.asarray([0, 2, 5, 6, 9], dtype=np.int32)
    parent = np.asarray([-1, 0, 1, 2], dtype=np.int32)
    g = random_tree_group(3, node_off, 4, 2, 8)
    g = {k: np.asarray(v, dtype=np.float64) for k, v in g.items()}
    rng = np.random.default_rng(9)
    k_p, v_p = rng.standard_normal((p, 2, 8)), rng.standard_normal((p, 2, 8))
    hmap = head_map(4, 2)
    a = tree_window_attention(k_p, v_p, g["q"], g["k"], g["v"], g["do"], node_off, parent, 0.5,
                              hmap)
    b = suffix_attention(k_p, v_p, g["q"], g["k"], g["v"], g["do"], np.asarray([0, 9]), 0.5, hmap)
    for x, y in (("o", "o_s"), ("lse", "lse_s"), ("dq", "dq_s"), ("dk", "dk_s"), ("dv", "dv_s"),
                 ("gk", "gk"), ("gv", "gv")):
        np.testing.assert_allclose(a[x], b[y], atol=1e-12, err_msg=x)


def test_tree_window_without_prefix_is_a_tree():
    node_off, parent, g = _window(4, 0)
    hmap = head_map(4, 2)
    a = tree_window_attention(g["k_p"], g["v_p"], g["q"], g["k"], g["v"], g["do"], node_off,
                              parent, 0.3, hmap)
    b = tree_attention_expanded(g["q"], g["k"], g["v"], g["do"], node_off, parent, 0.3, hmap,
                                rng=np.random.default_rng(4))
    for key in ("o", "lse", "dq", "dk", "dv"):
        np.testing.assert_allclose(a[key], b[key], atol=1e-12, err_msg=key)
    assert a["gk"].shape[0] == 0



@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_window_over_producer_ancestors_equals_combined_tree(seed):
    """A consumer window attached under an internal node u of a producer tree,
    reading the rows of u and its ancestors as its cached rows, then the
    producer backward with the window's gK/gV injected, equals plain attention
    over the combined tree in which the consumer's root is a child of u (the
    ancestor mask over all compact rows, HARTS §2.2): the consumer rows'
    outputs and gradients, and the producer rows' outputs and gradients."""
    rng = np.random.default_rng(seed)
    node_off_p, parent_p = random_tree(50 + seed, 7, max_len=5, min_len=1)
    depth = node_depths(parent_p)
    cand = [v for v in range(len(parent_p)) if depth[v] >= 1]
    u = int(cand[seed % len(cand)])
    ranges = ancestor_row_ranges(node_off_p, parent_p, u)
    node_off_c, parent_c = random_tree(80 + seed, 5, max_len=4, min_len=1)
    hq, hkv, d = 4, 2, 8
    hmap = head_map(hq, hkv)
    cp, cc = int(node_off_p[-1]), int(node_off_c[-1])
    gp = {k: rng.standard_normal((cp, hq if k in ("q", "do") else hkv, d)) for k in "q k v do".split()}
    gc = {k: rng.standard_normal((cc, hq if k in ("q", "do") else hkv, d)) for k in "q k v do".split()}
    win = tree_window_attention_ranges(gp["k"], gp["v"], ranges, gc["q"], gc["k"], gc["v"],
                                       gc["do"], node_off_c, parent_c, 0.35, hmap)
    prod = tree_attention_direct(gp["q"], gp["k"], gp["v"], gp["do"], node_off_p, parent_p, 0.35,
                                 hmap)
    dq_p, dk_p, dv_p = tree_backward_inject(gp["q"], gp["k"], gp["v"], gp["do"], node_off_p,
                                            parent_p, win["gk"], win["gv"], 0.35, hmap)
    # the combined tree: producer nodes, then the consumer's, its root under u
    n_p = len(parent_p)
    parent = np.concatenate([parent_p, np.where(parent_c < 0, u, parent_c + n_p)]).astype(np.int32)
    node_off = np.concatenate([node_off_p, node_off_c[1:] + cp]).astype(np.int32)
    both = {k: np.concatenate([gp[k], gc[k]], axis=0) for k in gp}
    full = tree_attention_direct(both["q"], both["k"], both["v"], both["do"], node_off, parent,
                                 0.35, hmap)
    for key in ("o", "dq", "dk", "dv"):
        np.testing.assert_allclose(win[key], full[key][cp:], atol=1e-12, err_msg=key)
    np.testing.assert_allclose(win["lse"], full["lse"][:, cp:], atol=1e-12)
    np.testing.assert_allclose(prod["o"], full["o"][:cp], atol=1e-12)
    for key, got in (("dq", dq_p), ("dk", dk_p), ("dv", dv_p)):
        np.testing.assert_allclose(got, full[key][:cp], atol=1e-12, err_msg=key)
    # rows outside the ranges receive no gradient from the window
    used = np.zeros(cp, dtype=bool)
    for s, n in ranges:
        used[s:s + n] = True
    assert np.all(win["gk"][~used] == 0) and np.abs(win["gk"][used]).max() > 0


def test_forest_window_equals_separate_windows():
    """Several rollout trees over one cached prefix in one call (a forest: each
    root has parent -1) equal one window per tree: rows of different trees
    never see each other (HARTS §2.1), every tree sees the whole prefix, and
    the prefix-side gradients add."""
    p = 5
    hmap = head_map(4, 2)
    rng = np.random.default_rng(7)
    k_p, v_p = rng.standard_normal((p, 2, 8)), rng.standard_normal((p, 2, 8))
    trees = [random_tree(s, n, max_len=4, min_len=1) for s, n in ((1, 4), (2, 1), (3, 5))]
    groups = [{k: np.asarray(v, np.float64) for k, v in random_tree_group(s, t[0], 4, 2, 8).items()}
              for s, t in zip((1, 2, 3), trees)]
    parent, node_off, base_n, base_r = [], [0], 0, 0
    for no, pa in trees:
        parent += [x + base_n if x >= 0 else -1 for x in pa]
        node_off += [int(x) + base_r for x in no[1:]]
        base_n += len(pa)
        base_r += int(no[-1])
    parent = np.asarray(parent, np.int32)
    node_off = np.asarray(node_off, np.int32)
    cat = {k: np.concatenate([g[k] for g in groups], axis=0) for k in groups[0]}
    f = tree_window_attention(k_p, v_p, cat["q"], cat["k"], cat["v"], cat["do"], node_off, parent,
                              0.4, hmap)
    r0 = 0
    gk = np.zeros_like(k_p)
    for (no, pa), g in zip(trees, groups):
        r1 = r0 + int(no[-1])
        s = tree_window_attention(k_p, v_p, g["q"], g["k"], g["v"], g["do"], no, pa, 0.4, hmap)
        for key in ("o", "dq", "dk", "dv"):
            np.testing.assert_allclose(f[key][r0:r1], s[key], atol=1e-12, err_msg=key)
        np.testing.assert_allclose(f["lse"][:, r0:r1], s["lse"], atol=1e-12)
        gk += s["gk"]
        r0 = r1
    np.testing.assert_allclose(f["gk"], gk, atol=1e-12)
