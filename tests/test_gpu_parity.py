"""GPU parity of every entry point against the fp64 oracle, on small groups
that still span several tiles and ragged tails, plus the degenerate cases.

Tolerance: normwise max |x - y| / max |y| <= 2e-2 for bf16 groups and 1e-4
for fp32 groups, per output tensor.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import TOL, check, dev, host
from workloads.gen import (
    ancestor_row_ranges,
    forest,
    node_depths,
    random_small_group,
    random_tree,
    random_tree_group,
)

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import shared_prefix_attention_pf_amd as pf
    from shared_prefix_attention_pf_amd import group as G


def _desc(hq, hkv, d, dtype, q_to_kv=None):
    return pf.AttnDesc(hq, hkv, d, pf.PF_BF16 if dtype == "bf16" else pf.PF_F32, 0.0, q_to_kv)


SUFFIX_CASES = [
    # (hq, hkv, d, dtype, P, suffix lengths, head map)
    (8, 2, 128, "bf16", 300, [1, 77, 130, 0, 64], None),
    (4, 4, 128, "bf16", 64, [200], None),
    (8, 1, 128, "bf16", 129, [33, 257], None),
    (6, 2, 128, "bf16", 70, [50, 90], None),
    (4, 2, 128, "bf16", 0, [100, 30], None),
    (4, 2, 128, "bf16", 96, [40, 41], [1, 0, 0, 1]),
    # KV head counts that are neither a divisor nor a multiple of 8 (head-major
    # block order) and a multiple of 8 with two heads per XCD
    (6, 3, 128, "bf16", 130, [70, 33], None),
    (16, 16, 128, "bf16", 64, [40, 90], None),
    (2, 2, 64, "f32", 256, [64, 64, 64, 64], None),
    (4, 2, 128, "f32", 100, [3, 70, 0], None),
    # fp32 matrix-core kernels: several 128-key blocks and 32-row tiles with
    # ragged tails, query-head groups of 1, 2, 4 and 8, a permuted head map
    (8, 2, 128, "f32", 300, [1, 77, 130, 0, 64], None),
    (6, 3, 64, "f32", 130, [70, 33], None),
    (4, 2, 128, "f32", 96, [40, 41], [1, 0, 0, 1]),
    (8, 1, 64, "f32", 129, [33, 257], None),
    (3, 3, 128, "f32", 0, [100, 30], None),
    # one KV head with eight query heads over 1024 rows: the prefix blocks split
    # into eight query chunks, the own blocks into two
    (8, 1, 64, "f32", 200, [600, 424], None),
    # a one-row prefix and one-row suffixes
    (2, 1, 128, "f32", 1, [1, 2, 0, 1], None),
]


@pytest.mark.parametrize("case", SUFFIX_CASES, ids=lambda c: f"{c[3]}-h{c[0]}x{c[1]}-P{c[4]}-{c[5]}")
def test_suffix_phase_b(case):
    _suffix_case(case)


def _suffix_case(case):
    """Phase B (forward, backward with gK/gV accumulation) of one case against
    the oracle."""
    hq, hkv, d, dtype, p, lens, qmap = case
    print(f"\ncase {case}", flush=True)
    g = random_small_group(17, hq, hkv, d, p, lens, dtype)
    cu = g["cu_seqlens"]
    desc = _desc(hq, hkv, d, dtype, qmap)
    scale = 1.0 / math.sqrt(d)
    t = {k: dev(g[k], dtype) for k in ("k_p", "v_p", "q_s", "k_s", "v_s", "do_s")}
    o_s, lse_s = G.suffix_fwd(desc, t["k_p"], t["v_p"], cu, t["q_s"], t["k_s"], t["v_s"])
    gk = torch.zeros(p, hkv, d, dtype=torch.float32, device="cuda")
    gv = torch.zeros_like(gk)
    dq, dk, dv = G.suffix_bwd(desc, t["k_p"], t["v_p"], cu, t["q_s"], t["k_s"], t["v_s"], o_s,
                              lse_s, t["do_s"], gk, gv)
    torch.cuda.synchronize()
    hmap = oracle.head_map(hq, hkv, qmap)
    ref = oracle.suffix_attention(g["k_p"], g["v_p"], g["q_s"], g["k_s"], g["v_s"], g["do_s"], cu,
                                  scale, hmap)
    tol = TOL[dtype]
    check("O_S", host(o_s), ref["o_s"], tol)
    check("LSE_S", host(lse_s), ref["lse_s"], tol)
    check("dQ_S", host(dq), ref["dq_s"], tol)
    check("dK_S", host(dk), ref["dk_s"], tol)
    check("dV_S", host(dv), ref["dv_s"], tol)
    if p > 0:
        check("gK", host(gk), ref["gk"], tol)
        check("gV", host(gv), ref["gv"], tol)


@pytest.mark.parametrize("case", [SUFFIX_CASES[0], SUFFIX_CASES[2], SUFFIX_CASES[11],
                                  SUFFIX_CASES[15]],
                         ids=lambda c: f"{c[3]}-h{c[0]}x{c[1]}-P{c[4]}-{c[5]}")
def test_suffix_phase_b_min_workspace(case):
    """The backward with the smallest workspace (no dS buffer: dQ recomputes
    S and dP) against the oracle, and against the dS-buffer path."""
    hq, hkv, d, dtype, p, lens, qmap = case
    print(f"\ncase {case}", flush=True)
    g = random_small_group(17, hq, hkv, d, p, lens, dtype)
    cu = g["cu_seqlens"]
    rows = int(cu[-1])
    desc = _desc(hq, hkv, d, dtype, qmap)
    scale = 1.0 / math.sqrt(d)
    t = {k: dev(g[k], dtype) for k in ("k_p", "v_p", "q_s", "k_s", "v_s", "do_s")}
    o_s, lse_s = G.suffix_fwd(desc, t["k_p"], t["v_p"], cu, t["q_s"], t["k_s"], t["v_s"])
    n_min = pf.pf_workspace_size_min(pf.PF_OP_SUFFIX_BWD, desc, p, rows)
    n_full = pf.pf_workspace_size(pf.PF_OP_SUFFIX_BWD, desc, p, rows)
    assert n_full > n_min
    outs = []
    for n_ws in (n_min, n_full):
        ws = torch.empty(n_ws, dtype=torch.uint8, device="cuda")
        gk = torch.zeros(p, hkv, d, dtype=torch.float32, device="cuda")
        gv = torch.zeros_like(gk)
        dq, dk, dv = G.suffix_bwd(desc, t["k_p"], t["v_p"], cu, t["q_s"], t["k_s"], t["v_s"],
                                  o_s, lse_s, t["do_s"], gk, gv, ws=ws)
        torch.cuda.synchronize()
        outs.append({"dq": host(dq), "dk": host(dk), "dv": host(dv), "gk": host(gk),
                     "gv": host(gv)})
    hmap = oracle.head_map(hq, hkv, qmap)
    ref = oracle.suffix_attention(g["k_p"], g["v_p"], g["q_s"], g["k_s"], g["v_s"], g["do_s"], cu,
                                  scale, hmap)
    tol = TOL[dtype]
    mn = outs[0]
    check("dQ_S (min ws)", mn["dq"], ref["dq_s"], tol)
    check("dK_S (min ws)", mn["dk"], ref["dk_s"], tol)
    check("dV_S (min ws)", mn["dv"], ref["dv_s"], tol)
    check("gK (min ws)", mn["gk"], ref["gk"], tol)
    check("gV (min ws)", mn["gv"], ref["gv"], tol)
    # the two paths differ only in rounding (for bf16, dS is rounded to bf16
    # either way)
    for k in ("dq", "dk", "dv", "gk", "gv"):
        check(f"{k}: min ws vs dS buffer", mn[k], outs[1][k], tol)


PREFIX_CASES = [
    (8, 2, 128, "bf16", 300, True),
    (4, 4, 128, "bf16", 64, True),
    (8, 2, 128, "bf16", 257, False),
    (2, 2, 64, "f32", 256, True),
    (4, 2, 128, "f32", 77, False),
    (8, 2, 128, "f32", 300, True),
    (6, 2, 64, "f32", 257, False),
    # one KV head, eight query heads: the causal prefix's key blocks split into
    # four query chunks with partial planes
    (8, 1, 64, "f32", 1100, True),
]


@pytest.mark.parametrize("case", PREFIX_CASES, ids=lambda c: f"{c[3]}-h{c[0]}x{c[1]}-P{c[4]}-do{c[5]}")
def test_prefix_phases_a_and_c(case):
    _prefix_case(case)


def _prefix_case(case):
    """Phase A and Phase C (with injected accumulators) of one case against the
    oracle, with dK/dV in the input dtype and in fp32."""
    hq, hkv, d, dtype, p, with_do = case
    print(f"\ncase {case}", flush=True)
    g = random_small_group(23, hq, hkv, d, p, [1], dtype)
    desc = _desc(hq, hkv, d, dtype)
    scale = 1.0 / math.sqrt(d)
    rng = np.random.default_rng(5)
    gk_np = rng.standard_normal((p, hkv, d)).astype(np.float32)
    gv_np = rng.standard_normal((p, hkv, d)).astype(np.float32)
    t = {k: dev(g[k], dtype) for k in ("q_p", "k_p", "v_p", "do_p")}
    o_p, lse_p = G.prefix_fwd(desc, t["q_p"], t["k_p"], t["v_p"])
    gk, gv = torch.from_numpy(gk_np).cuda(), torch.from_numpy(gv_np).cuda()
    do_p = t["do_p"] if with_do else None
    res = {}
    for dkv_dtype in {desc.dtype, pf.PF_F32}:
        res[dkv_dtype] = G.prefix_bwd(desc, t["q_p"], t["k_p"], t["v_p"], o_p, lse_p, do_p, gk, gv,
                                      dkv_dtype)
    torch.cuda.synchronize()
    hmap = oracle.head_map(hq, hkv)
    ro, rlse = oracle.prefix_forward(g["q_p"], g["k_p"], g["v_p"], scale, hmap)
    rdq, rdk, rdv = oracle.prefix_backward_inject(g["q_p"], g["k_p"], g["v_p"],
                                                  g["do_p"] if with_do else None, gk_np, gv_np,
                                                  scale, hmap)
    tol = TOL[dtype]
    check("O_P", host(o_p), ro, tol)
    check("LSE_P", host(lse_p), rlse, tol)
    for dkv_dtype, (dq, dk, dv) in res.items():
        check(f"dQ_P[{dkv_dtype}]", host(dq), rdq, tol)
        check(f"dK_P[{dkv_dtype}]", host(dk), rdk, tol)
        check(f"dV_P[{dkv_dtype}]", host(dv), rdv, tol)
    if not with_do:
        assert torch.count_nonzero(res[desc.dtype][0]).item() == 0
        # fp32 outputs equal the accumulators exactly
        np.testing.assert_array_equal(host(res[pf.PF_F32][1]), gk_np)


@pytest.mark.parametrize("seed,hq,hkv,dtype", [(0, 8, 2, "bf16"), (1, 4, 4, "bf16"),
                                               (2, 2, 1, "f32"), (3, 8, 2, "bf16")])
def test_tree(seed, hq, hkv, dtype):
    _tree_case(seed, hq, hkv, dtype, 9, 90)


def test_tree_f32_many_tiles():
    """An fp32 tree of about 1500 rows with GQA 8/2 at head_dim 128: many
    key and query tiles under the tree mask, own key blocks split into query
    chunks, and the dS buffer."""
    _tree_case(5, 8, 2, "f32", 24, 120, d=128)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_maximum_sizes(dtype):
    """The limits the boundary accepts: PF_MAX_SEGMENTS suffixes in one call
    (ragged, a quarter of them empty) and a tree of PF_MAX_SEGMENTS nodes,
    PF_MAX_HEADS query heads as 128 per KV head and as one per KV head."""
    d = 128 if dtype == "bf16" else 64
    rng = np.random.Generator(np.random.PCG64(77))
    lens = rng.integers(0, 10, size=pf.PF_MAX_SEGMENTS)
    lens[rng.permutation(pf.PF_MAX_SEGMENTS)[:pf.PF_MAX_SEGMENTS // 4]] = 0
    _suffix_case((4, 2, d, dtype, 100, lens.tolist(), None))
    _tree_case(11, 4, 2, dtype, pf.PF_MAX_SEGMENTS, 6)
    for hkv in (2, pf.PF_MAX_HEADS):
        _suffix_case((pf.PF_MAX_HEADS, hkv, d, dtype, 40, [30, 0, 17], None))
        _prefix_case((pf.PF_MAX_HEADS, hkv, d, dtype, 45, True))


def _tree_case(seed, hq, hkv, dtype, n_nodes, max_len, d=None):
    """Tree forward and backward of a random tree against the oracle."""
    if d is None:
        d = 128 if dtype == "bf16" else 64
    node_off, parent = random_tree(seed, n_nodes, max_len=max_len, min_len=0)
    if n_nodes <= 16:
        print(f"\ntree seed {seed}: node_off {node_off.tolist()} parent {parent.tolist()}",
              flush=True)
    else:
        print(f"\ntree seed {seed}: {n_nodes} nodes, {int(node_off[-1])} rows", flush=True)
    g = random_tree_group(seed, node_off, hq, hkv, d, dtype)
    desc = _desc(hq, hkv, d, dtype)
    t = {k: dev(g[k], dtype) for k in ("q", "k", "v", "do")}
    o, lse = G.tree_fwd(desc, node_off, parent, t["q"], t["k"], t["v"])
    dq, dk, dv = G.tree_bwd(desc, node_off, parent, t["q"], t["k"], t["v"], o, lse, t["do"])
    torch.cuda.synchronize()
    ref = oracle.tree_attention_direct(g["q"], g["k"], g["v"], g["do"], node_off, parent,
                                       1.0 / math.sqrt(d), oracle.head_map(hq, hkv))
    tol = TOL[dtype]
    for name, got in (("O", o), ("LSE", lse), ("dQ", dq), ("dK", dk), ("dV", dv)):
        check(name, host(got), ref[name.lower()], tol)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_phase_c_and_tree_min_workspace(dtype):
    """Phase C and the tree backward with the smallest workspace (dQ recomputes
    S and dP) and with the full one (dQ from the stored dS), each against the
    oracle and against each other."""
    hq, hkv, p = 8, 2, 300
    d = 128 if dtype == "bf16" else 64
    g = random_small_group(23, hq, hkv, d, p, [1], dtype)
    desc = _desc(hq, hkv, d, dtype)
    scale = 1.0 / math.sqrt(d)
    hmap = oracle.head_map(hq, hkv)
    rng = np.random.default_rng(5)
    gk_np = rng.standard_normal((p, hkv, d)).astype(np.float32)
    gv_np = rng.standard_normal((p, hkv, d)).astype(np.float32)
    t = {k: dev(g[k], dtype) for k in ("q_p", "k_p", "v_p", "do_p")}
    o_p, lse_p = G.prefix_fwd(desc, t["q_p"], t["k_p"], t["v_p"])
    gk, gv = torch.from_numpy(gk_np).cuda(), torch.from_numpy(gv_np).cuda()
    n_min = pf.pf_workspace_size_min(pf.PF_OP_PREFIX_BWD, desc, p, p)
    n_full = pf.pf_workspace_size(pf.PF_OP_PREFIX_BWD, desc, p, p)
    assert n_full > n_min
    outs = []
    for n_ws in (n_min, n_full):
        ws = torch.empty(n_ws, dtype=torch.uint8, device="cuda")
        outs.append([host(x) for x in G.prefix_bwd(desc, t["q_p"], t["k_p"], t["v_p"], o_p, lse_p,
                                                   t["do_p"], gk, gv, ws=ws)])
    torch.cuda.synchronize()
    ref = oracle.prefix_backward_inject(g["q_p"], g["k_p"], g["v_p"], g["do_p"], gk_np, gv_np,
                                        scale, hmap)
    for name, mn, full, r in zip(("dQ_P", "dK_P", "dV_P"), outs[0], outs[1], ref):
        check(f"{name} (min ws)", mn, r, TOL[dtype])
        check(f"{name} (dS buffer)", full, r, TOL[dtype])
        check(f"{name}: min ws vs dS buffer", mn, full, TOL[dtype])

    node_off, parent = random_tree(4, 9, max_len=90, min_len=0)
    print(f"\ntree node_off {node_off.tolist()} parent {parent.tolist()}", flush=True)
    rows = int(node_off[-1])
    tg = random_tree_group(4, node_off, hq, hkv, d, dtype)
    tt = {k: dev(tg[k], dtype) for k in ("q", "k", "v", "do")}
    o, lse = G.tree_fwd(desc, node_off, parent, tt["q"], tt["k"], tt["v"])
    n_min = pf.pf_workspace_size_min(pf.PF_OP_TREE_BWD, desc, 0, rows)
    n_full = pf.pf_workspace_size(pf.PF_OP_TREE_BWD, desc, 0, rows)
    assert n_full > n_min
    outs = []
    for n_ws in (n_min, n_full):
        ws = torch.empty(n_ws, dtype=torch.uint8, device="cuda")
        outs.append([host(x) for x in G.tree_bwd(desc, node_off, parent, tt["q"], tt["k"],
                                                 tt["v"], o, lse, tt["do"], ws=ws)])
    torch.cuda.synchronize()
    ref = oracle.tree_attention_direct(tg["q"], tg["k"], tg["v"], tg["do"], node_off, parent,
                                       scale, hmap)
    for name, mn, full in zip(("dq", "dk", "dv"), outs[0], outs[1]):
        check(f"tree {name} (min ws)", mn, ref[name], TOL[dtype])
        check(f"tree {name} (dS buffer)", full, ref[name], TOL[dtype])
        check(f"tree {name}: min ws vs dS buffer", mn, full, TOL[dtype])


@pytest.mark.parametrize("d", [64, 128])
def test_tree_bwd_inject_f32(d):
    """The tree backward with gK/gV injected (a producer tree after its
    windows) for an fp32 tree against the oracle, with the full and the
    smallest workspace."""
    hq, hkv = 4, 2
    node_off, parent = random_tree(31, 9, max_len=70, min_len=1)
    rows = int(node_off[-1])
    print(f"\ntree node_off {node_off.tolist()} parent {parent.tolist()}", flush=True)
    tg = random_tree_group(31, node_off, hq, hkv, d, "f32")
    desc = _desc(hq, hkv, d, "f32")
    scale = 1.0 / math.sqrt(d)
    hmap = oracle.head_map(hq, hkv)
    rng = np.random.default_rng(9)
    gk_np = rng.standard_normal((rows, hkv, d)).astype(np.float32)
    gv_np = rng.standard_normal((rows, hkv, d)).astype(np.float32)
    t = {k: dev(tg[k], "f32") for k in ("q", "k", "v", "do")}
    o, lse = G.tree_fwd(desc, node_off, parent, t["q"], t["k"], t["v"])
    gk, gv = torch.from_numpy(gk_np).cuda(), torch.from_numpy(gv_np).cuda()
    rdq, rdk, rdv = oracle.tree_backward_inject(tg["q"], tg["k"], tg["v"], tg["do"], node_off,
                                                parent, gk_np, gv_np, scale, hmap)
    n_min = pf.pf_workspace_size_min(pf.PF_OP_TREE_BWD, desc, 0, rows)
    for ws in (None, torch.empty(n_min, dtype=torch.uint8, device="cuda")):
        dq, dk, dv = G.tree_bwd_inject(desc, node_off, parent, t["q"], t["k"], t["v"], o, lse,
                                       t["do"], gk, gv, ws=ws)
        torch.cuda.synchronize()
        what = "full ws" if ws is None else "min ws"
        check(f"dQ ({what})", host(dq), rdq, TOL["f32"])
        check(f"dK ({what})", host(dk), rdk, TOL["f32"])
        check(f"dV ({what})", host(dv), rdv, TOL["f32"])


@pytest.mark.parametrize("dtype,p", [("bf16", 300), ("bf16", 0), ("f32", 70)])
def test_tree_windows_over_a_prefix(dtype, p):
    """Two sharing windows of irregular rollout trees over one cached prefix:
    each window's outputs against the oracle, the prefix-side gradients
    accumulated over both windows, then the producer backward (Phase C with
    the accumulated gK/gV injected).  The first window's backward also runs
    with the smallest workspace (recompute dQ path)."""
    hq, hkv = 8, 2
    d = 128 if dtype == "bf16" else 64
    print(f"\ntree windows {dtype} P={p}", flush=True)
    g = random_small_group(41, hq, hkv, d, p, [1], dtype)
    desc = _desc(hq, hkv, d, dtype)
    scale = 1.0 / math.sqrt(d)
    hmap = oracle.head_map(hq, hkv)
    tol = TOL[dtype]
    t = {k: dev(g[k], dtype) for k in ("q_p", "k_p", "v_p", "do_p")}
    gk = torch.zeros(p, hkv, d, dtype=torch.float32, device="cuda")
    gv = torch.zeros_like(gk)
    gk_ref = np.zeros((p, hkv, d))
    gv_ref = np.zeros((p, hkv, d))
    for w, (seed, n_nodes, max_len) in enumerate(((5, 9, 90), (6, 12, 40))):
        node_off, parent = random_tree(seed, n_nodes, max_len=max_len, min_len=0)
        rows = int(node_off[-1])
        print(f"  window {w}: node_off {node_off.tolist()} parent {parent.tolist()}", flush=True)
        tg = random_tree_group(seed, node_off, hq, hkv, d, dtype)
        tt = {k: dev(tg[k], dtype) for k in ("q", "k", "v", "do")}
        o, lse = G.tree_suffix_fwd(desc, t["k_p"], t["v_p"], node_off, parent, tt["q"], tt["k"],
                                   tt["v"])
        if w == 0:
            n_min = pf.pf_workspace_size_min(pf.PF_OP_TREE_SUFFIX_BWD, desc, p, rows)
            ws = torch.empty(n_min, dtype=torch.uint8, device="cuda")
            gk0 = torch.zeros_like(gk)
            gv0 = torch.zeros_like(gv)
            mn = G.tree_suffix_bwd(desc, t["k_p"], t["v_p"], node_off, parent, tt["q"], tt["k"],
                                   tt["v"], o, lse, tt["do"], gk0, gv0, ws=ws)
        dq, dk, dv = G.tree_suffix_bwd(desc, t["k_p"], t["v_p"], node_off, parent, tt["q"],
                                       tt["k"], tt["v"], o, lse, tt["do"], gk, gv)
        torch.cuda.synchronize()
        ref = oracle.tree_window_attention(g["k_p"], g["v_p"], tg["q"], tg["k"], tg["v"],
                                           tg["do"], node_off, parent, scale, hmap)
        gk_ref += ref["gk"]
        gv_ref += ref["gv"]
        for name, got in (("O", o), ("LSE", lse), ("dQ", dq), ("dK", dk), ("dV", dv)):
            check(f"window {w} {name}", host(got), ref[name.lower()], tol)
        if w == 0:
            for name, got in zip(("dQ", "dK", "dV"), mn):
                check(f"window 0 {name} (min ws)", host(got), ref[name.lower()], tol)
            if p > 0:
                check("window 0 gK (min ws)", host(gk0), ref["gk"], tol)
        if p > 0:
            check(f"gK after window {w}", host(gk), gk_ref, tol)
            check(f"gV after window {w}", host(gv), gv_ref, tol)
    if p == 0:
        return
    # the producer backward with both windows' gradients injected
    o_p, lse_p = G.prefix_fwd(desc, t["q_p"], t["k_p"], t["v_p"])
    dq_p, dk_p, dv_p = G.prefix_bwd(desc, t["q_p"], t["k_p"], t["v_p"], o_p, lse_p, t["do_p"], gk,
                                    gv)
    torch.cuda.synchronize()
    rdq, rdk, rdv = oracle.prefix_backward_inject(g["q_p"], g["k_p"], g["v_p"], g["do_p"], gk_ref,
                                                  gv_ref, scale, hmap)
    check("producer dQ_P", host(dq_p), rdq, tol)
    check("producer dK_P", host(dk_p), rdk, tol)
    check("producer dV_P", host(dv_p), rdv, tol)


def _phase_b_run(desc, t, cu, p, calls):
    """Run Phase B as the given microbatches (lists of suffix indices); return gK, gV."""
    hkv, d = t["k_p"].shape[1], t["k_p"].shape[2]
    gk = torch.zeros(p, hkv, d, dtype=torch.float32, device="cuda")
    gv = torch.zeros_like(gk)
    for idx in calls:
        rows = torch.cat([torch.arange(cu[i], cu[i + 1]) for i in idx]).cuda()
        sub_cu = np.concatenate([[0], np.cumsum([cu[i + 1] - cu[i] for i in idx])]).astype(np.int32)
        q, k, v, do = (t[n].index_select(0, rows).contiguous() for n in ("q_s", "k_s", "v_s", "do_s"))
        o, lse = G.suffix_fwd(desc, t["k_p"], t["v_p"], sub_cu, q, k, v)
        G.suffix_bwd(desc, t["k_p"], t["v_p"], sub_cu, q, k, v, o, lse, do, gk, gv)
    torch.cuda.synchronize()
    return gk, gv


# Across microbatch splits only rounding differs.  In bf16 a different split
# moves a suffix's keys onto different 64-key block boundaries, which changes
# the running softmax maximum at which P is rounded to bf16 (and the bf16 O
# that D is built from), so splits agree to the size of the bf16 parity error,
# not bitwise.  In fp32 only the fp32 summation order differs.
SPLIT_TOL = {"bf16": 5e-3, "f32": 1e-5}


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_determinism_and_split_invariance(dtype):
    hq, hkv, p, lens = 8, 2, 520, [60, 130, 1, 200, 64, 90]
    d = 128
    g = random_small_group(31, hq, hkv, d, p, lens, dtype)
    cu = g["cu_seqlens"]
    desc = _desc(hq, hkv, d, dtype)
    t = {k: dev(g[k], dtype) for k in ("k_p", "v_p", "q_s", "k_s", "v_s", "do_s")}
    whole = [list(range(len(lens)))]
    gk1, gv1 = _phase_b_run(desc, t, cu, p, whole)
    gk2, gv2 = _phase_b_run(desc, t, cu, p, whole)
    assert torch.equal(gk1, gk2) and torch.equal(gv1, gv2), "re-run is not bitwise identical"
    ref = oracle.suffix_attention(g["k_p"], g["v_p"], g["q_s"], g["k_s"], g["v_s"], g["do_s"], cu,
                                  1.0 / math.sqrt(d), oracle.head_map(hq, hkv))
    check("gK whole vs oracle", host(gk1), ref["gk"], TOL[dtype])
    for split in ([[0], [1], [2], [3], [4], [5]], [[5, 3], [0, 2, 1], [4]]):
        gks, gvs = _phase_b_run(desc, t, cu, p, split)
        gks2, _ = _phase_b_run(desc, t, cu, p, split)
        assert torch.equal(gks, gks2), "re-run of a split is not bitwise identical"
        check(f"gK split {split}", host(gks), host(gk1), SPLIT_TOL[dtype])
        check(f"gV split {split}", host(gvs), host(gv1), SPLIT_TOL[dtype])
        check(f"gK split {split} vs oracle", host(gks), ref["gk"], TOL[dtype])


def test_no_cross_suffix_leakage():
    hq, hkv, d, p, lens = 4, 2, 128, 64, [70, 50, 90]
    g = random_small_group(37, hq, hkv, d, p, lens, "bf16")
    cu = g["cu_seqlens"]
    desc = _desc(hq, hkv, d, "bf16")
    t = {k: dev(g[k], "bf16") for k in ("k_p", "v_p", "q_s", "k_s", "v_s", "do_s")}

    def run(k_s):
        o, lse = G.suffix_fwd(desc, t["k_p"], t["v_p"], cu, t["q_s"], k_s, t["v_s"])
        gk = torch.zeros(p, hkv, d, dtype=torch.float32, device="cuda")
        dq, _, _ = G.suffix_bwd(desc, t["k_p"], t["v_p"], cu, t["q_s"], k_s, t["v_s"], o, lse,
                                t["do_s"], gk, torch.zeros_like(gk))
        return o, dq

    o1, dq1 = run(t["k_s"])
    k2 = t["k_s"].clone()
    k2[cu[1]:cu[2]] += 1.0
    o2, dq2 = run(k2)
    torch.cuda.synchronize()
    for a, b in ((0, 1), (2, 3)):
        sl = slice(int(cu[a]), int(cu[b]))
        assert torch.equal(o1[sl], o2[sl]) and torch.equal(dq1[sl], dq2[sl])
    assert not torch.equal(o1[cu[1]:cu[2]], o2[cu[1]:cu[2]])


def test_empty_call_is_noop():
    desc = _desc(4, 2, 128, "bf16")
    kp = torch.zeros(16, 2, 128, dtype=torch.bfloat16, device="cuda")
    empty_q = torch.zeros(0, 4, 128, dtype=torch.bfloat16, device="cuda")
    empty_k = torch.zeros(0, 2, 128, dtype=torch.bfloat16, device="cuda")
    gk = torch.full((16, 2, 128), 3.0, device="cuda")
    o, lse = G.suffix_fwd(desc, kp, kp, np.array([0, 0], np.int32), empty_q, empty_k, empty_k)
    G.suffix_bwd(desc, kp, kp, np.array([0, 0], np.int32), empty_q, empty_k, empty_k, o, lse,
                 empty_q, gk, gk.clone())
    torch.cuda.synchronize()
    assert o.shape[0] == 0 and torch.all(gk == 3.0)


@pytest.mark.parametrize("hq,hkv,dtype,d", [(8, 2, "bf16", 128), (16, 4, "bf16", 128),
                                            (8, 2, "f32", 128), (4, 1, "f32", 64)])
def test_windows_under_producer_nodes(hq, hkv, dtype, d):
    """Consumer windows attached under internal nodes of a producer rollout
    tree, each reading the rows of its node and the node's ancestors in place
    (row ranges of the producer's K/V, not 32-aligned), adding its gradients
    into those producer rows; then the producer's tree backward with the
    summed gradients injected.  Every output against the oracle (gather,
    window attention, scatter-add; tree backward plus the injection).  The
    first window's backward also runs with the smallest workspace (recompute
    dQ), and one range [0, P) equals the window over a flat prefix."""
    desc = _desc(hq, hkv, d, dtype)
    scale = 1.0 / math.sqrt(d)
    hmap = oracle.head_map(hq, hkv)
    tol = TOL[dtype]
    node_off_p, parent_p = random_tree(28, 10, max_len=120, min_len=20)
    depth = node_depths(parent_p)
    assert depth[7] == 2 and 8 in np.flatnonzero(parent_p == 7)   # a depth-2 internal node
    cp = int(node_off_p[-1])
    gp = random_tree_group(28, node_off_p, hq, hkv, d, dtype)
    tp = {k: dev(gp[k], dtype) for k in ("q", "k", "v", "do")}
    print(f"\nproducer node_off {node_off_p.tolist()} parent {parent_p.tolist()}", flush=True)
    o_p, lse_p = G.tree_fwd(desc, node_off_p, parent_p, tp["q"], tp["k"], tp["v"])
    gk = torch.zeros(cp, hkv, d, dtype=torch.float32, device="cuda")
    gv = torch.zeros_like(gk)
    gk_ref = np.zeros((cp, hkv, d))
    gv_ref = np.zeros((cp, hkv, d))
    for w, (u, seed, n_nodes, max_len) in enumerate(((7, 60, 8, 70), (9, 61, 11, 40))):
        ranges = ancestor_row_ranges(node_off_p, parent_p, u)
        node_off, parent = random_tree(seed, n_nodes, max_len=max_len, min_len=1)
        rows = int(node_off[-1])
        print(f"  window {w} under node {u}: ranges {ranges}, {rows} rows", flush=True)
        tg = random_tree_group(seed, node_off, hq, hkv, d, dtype)
        tt = {k: dev(tg[k], dtype) for k in ("q", "k", "v", "do")}
        o, lse = G.tree_suffix_fwd_ranges(desc, tp["k"], tp["v"], ranges, node_off, parent,
                                          tt["q"], tt["k"], tt["v"])
        if w == 0:
            nk = pf.pf_ranges_cached_keys([n for _, n in ranges])
            n_min = pf.pf_workspace_size_min(pf.PF_OP_TREE_SUFFIX_BWD, desc, nk, rows)
            ws = torch.empty(n_min, dtype=torch.uint8, device="cuda")
            gk0 = torch.zeros_like(gk)
            gv0 = torch.zeros_like(gv)
            mn = G.tree_suffix_bwd_ranges(desc, tp["k"], tp["v"], ranges, node_off, parent,
                                          tt["q"], tt["k"], tt["v"], o, lse, tt["do"], gk0, gv0,
                                          ws=ws)
        dq, dk, dv = G.tree_suffix_bwd_ranges(desc, tp["k"], tp["v"], ranges, node_off, parent,
                                              tt["q"], tt["k"], tt["v"], o, lse, tt["do"], gk, gv)
        torch.cuda.synchronize()
        ref = oracle.tree_window_attention_ranges(gp["k"], gp["v"], ranges, tg["q"], tg["k"],
                                                  tg["v"], tg["do"], node_off, parent, scale, hmap)
        gk_ref += ref["gk"]
        gv_ref += ref["gv"]
        for name, got in (("O", o), ("LSE", lse), ("dQ", dq), ("dK", dk), ("dV", dv)):
            check(f"window {w} {name}", host(got), ref[name.lower()], tol)
        if w == 0:
            for name, got in zip(("dQ", "dK", "dV"), mn):
                check(f"window 0 {name} (min ws)", host(got), ref[name.lower()], tol)
            check("window 0 gK (min ws)", host(gk0), ref["gk"], tol)
            check("window 0 gV (min ws)", host(gv0), ref["gv"], tol)
            # rows outside the ranges are never written
            used = np.zeros(cp, dtype=bool)
            for s, n in ranges:
                used[s:s + n] = True
            assert np.all(host(gk)[~used] == 0) and np.all(host(gv)[~used] == 0)
        check(f"gK after window {w}", host(gk), gk_ref, tol)
        check(f"gV after window {w}", host(gv), gv_ref, tol)
    # the producer backward with both windows' gradients injected
    dq_p, dk_p, dv_p = G.tree_bwd_inject(desc, node_off_p, parent_p, tp["q"], tp["k"], tp["v"],
                                         o_p, lse_p, tp["do"], gk, gv)
    torch.cuda.synchronize()
    rp = oracle.tree_attention_direct(gp["q"], gp["k"], gp["v"], gp["do"], node_off_p, parent_p,
                                      scale, hmap)
    rdq, rdk, rdv = oracle.tree_backward_inject(gp["q"], gp["k"], gp["v"], gp["do"], node_off_p,
                                                parent_p, gk_ref, gv_ref, scale, hmap)
    check("producer O", host(o_p), rp["o"], tol)
    check("producer dQ", host(dq_p), rdq, tol)
    check("producer dK (injected)", host(dk_p), rdk, tol)
    check("producer dV (injected)", host(dv_p), rdv, tol)
    # zero upstream: the injected gradients alone
    dq0, dk0, dv0 = G.tree_bwd_inject(desc, node_off_p, parent_p, tp["q"], tp["k"], tp["v"], o_p,
                                      lse_p, torch.empty(0, device="cuda"), gk, gv,
                                      dkv_dtype=pf.PF_F32)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dq0).item() == 0
    assert torch.equal(dk0, gk) and torch.equal(dv0, gv)
    # one range [0, P) of a flat prefix is the window over that prefix
    p = 300
    g = random_small_group(43, hq, hkv, d, p, [1], dtype)
    kp, vp = dev(g["k_p"], dtype), dev(g["v_p"], dtype)
    node_off, parent = random_tree(62, 6, max_len=50, min_len=1)
    tg = random_tree_group(62, node_off, hq, hkv, d, dtype)
    tt = {k: dev(tg[k], dtype) for k in ("q", "k", "v", "do")}
    o1, l1 = G.tree_suffix_fwd(desc, kp, vp, node_off, parent, tt["q"], tt["k"], tt["v"])
    o2, l2 = G.tree_suffix_fwd_ranges(desc, kp, vp, [(0, p)], node_off, parent, tt["q"], tt["k"],
                                      tt["v"])
    a1 = torch.zeros(p, hkv, d, device="cuda")
    b1 = torch.zeros_like(a1)
    a2 = torch.zeros_like(a1)
    b2 = torch.zeros_like(a1)
    r1 = G.tree_suffix_bwd(desc, kp, vp, node_off, parent, tt["q"], tt["k"], tt["v"], o1, l1,
                           tt["do"], a1, b1)
    r2 = G.tree_suffix_bwd_ranges(desc, kp, vp, [(0, p)], node_off, parent, tt["q"], tt["k"],
                                  tt["v"], o1, l1, tt["do"], a2, b2)
    torch.cuda.synchronize()
    for name, x, y in (("O", o2, o1), ("LSE", l2, l1), ("dQ", r2[0], r1[0]), ("dK", r2[1], r1[1]),
                       ("dV", r2[2], r1[2]), ("gK", a2, a1), ("gV", b2, b1)):
        check(f"one range vs flat prefix: {name}", host(x), host(y), 1e-6)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_forest_window_in_one_call(dtype):
    """Three rollout trees over one cached prefix in one call (a forest): each
    tree's rows against the oracle's forest window (rows of different trees
    never see each other), the prefix gradients against the oracle, and the
    same values as one call per tree to the dtype's bar."""
    hq, hkv, d, p = 8, 2, 128, 200
    desc = _desc(hq, hkv, d, dtype)
    scale = 1.0 / math.sqrt(d)
    hmap = oracle.head_map(hq, hkv)
    tol = TOL[dtype]
    g = random_small_group(44, hq, hkv, d, p, [1], dtype)
    kp, vp = dev(g["k_p"], dtype), dev(g["v_p"], dtype)
    trees = [random_tree(s, n, max_len=ml, min_len=1) for s, n, ml in ((70, 7, 60), (71, 1, 90),
                                                                      (72, 10, 30))]
    groups = [random_tree_group(s, t[0], hq, hkv, d, dtype) for s, t in zip((70, 71, 72), trees)]
    node_off, parent = forest(trees)
    print(f"\nforest node_off {node_off.tolist()} parent {parent.tolist()}", flush=True)
    cat = {k: np.concatenate([gg[k] for gg in groups], axis=0) for k in ("q", "k", "v", "do")}
    tt = {k: dev(cat[k], dtype) for k in cat}
    o, lse = G.tree_suffix_fwd(desc, kp, vp, node_off, parent, tt["q"], tt["k"], tt["v"])
    gk = torch.zeros(p, hkv, d, device="cuda")
    gv = torch.zeros_like(gk)
    dq, dk, dv = G.tree_suffix_bwd(desc, kp, vp, node_off, parent, tt["q"], tt["k"], tt["v"], o, lse,
                                   tt["do"], gk, gv)
    gk1 = torch.zeros_like(gk)
    gv1 = torch.zeros_like(gk)
    sep = []
    for (no, pa), gg in zip(trees, groups):
        ts = {k: dev(gg[k], dtype) for k in ("q", "k", "v", "do")}
        o1, l1 = G.tree_suffix_fwd(desc, kp, vp, no, pa, ts["q"], ts["k"], ts["v"])
        r1 = G.tree_suffix_bwd(desc, kp, vp, no, pa, ts["q"], ts["k"], ts["v"], o1, l1, ts["do"],
                               gk1, gv1)
        sep.append((o1, l1) + tuple(r1))
    torch.cuda.synchronize()
    ref = oracle.tree_window_attention(g["k_p"], g["v_p"], cat["q"], cat["k"], cat["v"], cat["do"],
                                       node_off, parent, scale, hmap)
    for name, got in (("O", o), ("LSE", lse), ("dQ", dq), ("dK", dk), ("dV", dv), ("gK", gk),
                      ("gV", gv)):
        check(f"forest {name}", host(got), ref[name.lower()], tol)
    cat_sep = [torch.cat([s[i] for s in sep], dim=1 if i == 1 else 0) for i in range(5)]
    for name, x, y in zip(("O", "LSE", "dQ", "dK", "dV"), (o, lse, dq, dk, dv), cat_sep):
        check(f"forest vs one call per tree: {name}", host(x), host(y), tol)
    check("forest vs one call per tree: gK", host(gk), host(gk1), tol)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_many_shuffled_ranges(dtype):
    """A window over 200 disjoint row ranges of 1-40 rows each (5 of them
    start on a 32-row boundary), listed out of row order, with empty ranges among them: every
    range a padded tile run of its own in the tile table, split key blocks,
    and gK/gV scattered back through the table.  Against the oracle's gather,
    window attention and scatter-add."""
    hq, hkv = 4, 2
    d = 128 if dtype == "bf16" else 64
    rng = np.random.default_rng(77)
    lens = rng.integers(1, 41, size=200)
    gaps = rng.integers(0, 5, size=200)
    starts = np.cumsum(np.concatenate([[3], (lens + gaps)[:-1]])) + gaps[0]
    cp = int(starts[-1] + lens[-1] + 7)
    order = rng.permutation(200)
    ranges = [(int(starts[i]), int(lens[i])) for i in order]
    ranges[5:5] = [(int(starts[0]), 0)]           # empty ranges are ignored
    ranges.append((cp, 0))
    print(f"\n{len(ranges)} ranges over {cp} producer rows, {sum(n for _, n in ranges)} cached",
          flush=True)
    gp = random_tree_group(78, np.array([0, cp], np.int32), hq, hkv, d, dtype)
    node_off, parent = random_tree(79, 6, max_len=60, min_len=1)
    tg = random_tree_group(79, node_off, hq, hkv, d, dtype)
    desc = _desc(hq, hkv, d, dtype)
    kc, vc = dev(gp["k"], dtype), dev(gp["v"], dtype)
    tt = {k: dev(tg[k], dtype) for k in ("q", "k", "v", "do")}
    o, lse = G.tree_suffix_fwd_ranges(desc, kc, vc, ranges, node_off, parent, tt["q"], tt["k"],
                                      tt["v"])
    gk = torch.zeros(cp, hkv, d, dtype=torch.float32, device="cuda")
    gv = torch.zeros_like(gk)
    dq, dk, dv = G.tree_suffix_bwd_ranges(desc, kc, vc, ranges, node_off, parent, tt["q"], tt["k"],
                                          tt["v"], o, lse, tt["do"], gk, gv)
    torch.cuda.synchronize()
    ref = oracle.tree_window_attention_ranges(gp["k"], gp["v"], ranges, tg["q"], tg["k"], tg["v"],
                                              tg["do"], node_off, parent, 1.0 / math.sqrt(d),
                                              oracle.head_map(hq, hkv))
    tol = TOL[dtype]
    for name, got in (("O", o), ("LSE", lse), ("dQ", dq), ("dK", dk), ("dV", dv), ("gK", gk),
                      ("gV", gv)):
        check(name, host(got), ref[name.lower()], tol)
    used = np.zeros(cp, dtype=bool)
    for s, n in ranges:
        used[s:s + n] = True
    assert np.all(host(gk)[~used] == 0) and np.all(host(gv)[~used] == 0)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_strided_layouts(dtype):
    """Phases A, B and C with every tensor a strided view, as a training step
    hands them over: Q/K/V sliced out of one fused projection output
    [T, Hq + 2 Hkv, d], dO and O with padded rows, dQ starting two heads into
    a wider buffer, dK/dV sharing one fused buffer.  Every output bitwise equal
    to the contiguous run (the arithmetic does not depend on strides) and
    within the bar of the oracle."""
    hq, hkv, d, p, lens = 8, 2, 128, 200, [70, 1, 130]
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    g = random_small_group(47, hq, hkv, d, p, lens, dtype)
    cu = g["cu_seqlens"]
    rows = int(cu[-1])
    desc = _desc(hq, hkv, d, dtype)
    t = {k: dev(g[k], dtype) for k in ("q_p", "k_p", "v_p", "do_p", "q_s", "k_s", "v_s", "do_s")}

    def fused(q, k, v):
        buf = torch.zeros(q.shape[0], hq + 2 * hkv, d, dtype=tdt, device="cuda")
        buf[:, :hq] = q
        buf[:, hq:hq + hkv] = k
        buf[:, hq + hkv:] = v
        return buf[:, :hq], buf[:, hq:hq + hkv], buf[:, hq + hkv:]

    def padded(n, heads, pad):
        return torch.full((n, heads, d + pad), 7.0, dtype=tdt, device="cuda")[:, :, :d]

    def fused_kv(n):
        buf = torch.full((n, 2 * hkv, d), 7.0, dtype=tdt, device="cuda")
        return buf[:, :hkv], buf[:, hkv:]

    qs, ks, vs = fused(t["q_s"], t["k_s"], t["v_s"])
    qp, kp, vp = fused(t["q_p"], t["k_p"], t["v_p"])
    do_s = padded(rows, hq, 8)
    do_s.copy_(t["do_s"])
    do_p = padded(p, hq, 8)
    do_p.copy_(t["do_p"])
    assert not qs.is_contiguous() and not do_s.is_contiguous()

    # Phase A
    o_p = padded(p, hq, 16)
    lse_p = torch.empty(hq, p, device="cuda")
    pf.pf_prefix_fwd(desc, p, qp, kp, vp, o_p, lse_p, G.workspace(pf.PF_OP_PREFIX_FWD, desc, p, p,
                                                                 "cuda"))
    # Phase B
    o_s = padded(rows, hq, 16)
    lse_s = torch.empty(hq, rows, device="cuda")
    pf.pf_suffix_attn_fwd(desc, p, kp, vp, cu, qs, ks, vs, o_s, lse_s,
                          G.workspace(pf.PF_OP_SUFFIX_FWD, desc, p, rows, "cuda"))
    dq_buf = torch.full((rows, hq + 4, d), 7.0, dtype=tdt, device="cuda")
    dq_s = dq_buf[:, 2:2 + hq]
    dk_s, dv_s = fused_kv(rows)
    gk = torch.zeros(p, hkv, d, device="cuda")
    gv = torch.zeros_like(gk)
    pf.pf_suffix_attn_bwd_accum(desc, p, kp, vp, cu, qs, ks, vs, o_s, lse_s, do_s, dq_s, dk_s,
                                dv_s, gk, gv, G.workspace(pf.PF_OP_SUFFIX_BWD, desc, p, rows,
                                                          "cuda"))
    # Phase C
    dq_p = padded(p, hq, 24)
    dk_p, dv_p = fused_kv(p)
    pf.pf_prefix_bwd_inject(desc, p, qp, kp, vp, o_p, lse_p, do_p, gk, gv, dq_p, dk_p, dv_p,
                            desc.dtype, G.workspace(pf.PF_OP_PREFIX_BWD, desc, p, p, "cuda"))
    torch.cuda.synchronize()

    # the same calls on contiguous tensors
    c_op, c_lp = G.prefix_fwd(desc, t["q_p"], t["k_p"], t["v_p"])
    c_os, c_ls = G.suffix_fwd(desc, t["k_p"], t["v_p"], cu, t["q_s"], t["k_s"], t["v_s"])
    c_gk = torch.zeros_like(gk)
    c_gv = torch.zeros_like(gk)
    c_dq, c_dk, c_dv = G.suffix_bwd(desc, t["k_p"], t["v_p"], cu, t["q_s"], t["k_s"], t["v_s"],
                                    c_os, c_ls, t["do_s"], c_gk, c_gv)
    c_dqp, c_dkp, c_dvp = G.prefix_bwd(desc, t["q_p"], t["k_p"], t["v_p"], c_op, c_lp, t["do_p"],
                                       c_gk, c_gv)
    torch.cuda.synchronize()
    for name, x, y in (("O_P", o_p, c_op), ("LSE_P", lse_p, c_lp), ("O_S", o_s, c_os),
                       ("LSE_S", lse_s, c_ls), ("dQ_S", dq_s, c_dq), ("dK_S", dk_s, c_dk),
                       ("dV_S", dv_s, c_dv), ("gK", gk, c_gk), ("gV", gv, c_gv),
                       ("dQ_P", dq_p, c_dqp), ("dK_P", dk_p, c_dkp), ("dV_P", dv_p, c_dvp)):
        assert torch.equal(x, y), f"{name}: strided run differs from the contiguous one"
    # nothing outside the views was written
    assert torch.all(dq_buf[:, :2] == 7.0) and torch.all(dq_buf[:, 2 + hq:] == 7.0)
    assert torch.all(o_s.as_strided((rows, hq, 16), (hq * (d + 16), d + 16, 1), d) == 7.0)
    scale = 1.0 / math.sqrt(d)
    hmap = oracle.head_map(hq, hkv)
    tol = TOL[dtype]
    ref = oracle.suffix_attention(g["k_p"], g["v_p"], g["q_s"], g["k_s"], g["v_s"], g["do_s"], cu,
                                  scale, hmap)
    for name, x, key in (("O_S", o_s, "o_s"), ("dQ_S", dq_s, "dq_s"), ("dK_S", dk_s, "dk_s"),
                         ("dV_S", dv_s, "dv_s"), ("gK", gk, "gk"), ("gV", gv, "gv")):
        check(name, host(x), ref[key], tol)
    rdq, rdk, rdv = oracle.prefix_backward_inject(g["q_p"], g["k_p"], g["v_p"], g["do_p"],
                                                  ref["gk"], ref["gv"], scale, hmap)
    check("dQ_P", host(dq_p), rdq, tol)
    check("dK_P", host(dk_p), rdk, tol)
    check("dV_P", host(dv_p), rdv, tol)
