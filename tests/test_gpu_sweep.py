"""Seeded random sweep of small groups against the fp64 oracle.

The fixed cases of test_gpu_parity.py pick shapes by hand; these draw them:
dtype and head_dim, KV heads and query-head group size, a permuted head map,
prefix lengths on and off the 32- and 64-key tile edges (0 included), one to
five suffixes of ragged lengths (0 and 1 included), a sharper softmax (Q
scaled by 3, so the running maximum moves and the lazy rescale runs), a
softmax scale of the caller's (0.05 or 0.2) or the 1/sqrt(d) default, and
the smallest workspace (recompute dQ) or the full one (dQ from stored dS).
Each draw is printed before it runs.  Tolerances as in test_gpu_parity.py.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import TOL, check, dev, host
from workloads.gen import ancestor_row_ranges, random_small_group, random_tree, random_tree_group

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import shared_prefix_attention_pf_amd as pf
    from shared_prefix_attention_pf_amd import group as G

EDGE_LENS = [0, 1, 2, 31, 32, 33, 63, 64, 65, 96, 127, 129, 200]


def _heads(rng):
    """(hq, hkv, head map or None): groups of 1-4 query heads, 1-8 KV heads."""
    hkv = int(rng.choice([1, 2, 3, 4, 8]))
    group = int(rng.choice([1, 2, 3, 4]))
    hq = hkv * group
    qmap = None
    if rng.random() < 0.4:
        # every KV head keeps exactly `group` query heads, in a shuffled order
        qmap = [int(x) for x in rng.permutation(np.repeat(np.arange(hkv), group))]
    return hq, hkv, qmap


def _dtype_dim(rng):
    if rng.random() < 0.55:
        return "bf16", 128
    return "f32", int(rng.choice([64, 128]))


def _desc(hq, hkv, d, dtype, qmap=None, softmax_scale=0.0):
    return pf.AttnDesc(hq, hkv, d, pf.PF_BF16 if dtype == "bf16" else pf.PF_F32, softmax_scale,
                       qmap)


def _scale(c):
    """the descriptor's softmax scale and the one the oracle applies"""
    return c["softmax_scale"], c["softmax_scale"] or 1.0 / math.sqrt(c["d"])


def draw_suffix_case(seed):
    rng = np.random.default_rng(9000 + seed)
    dtype, d = _dtype_dim(rng)
    hq, hkv, qmap = _heads(rng)
    p = int(rng.choice(EDGE_LENS + [257, 300]))
    n = int(rng.integers(1, 6))
    lens = [int(rng.choice(EDGE_LENS)) for _ in range(n)]
    if sum(lens) == 0:
        lens[0] = 1 + int(rng.integers(0, 90))
    scale_q = float(rng.choice([1.0, 3.0]))
    min_ws = bool(rng.random() < 0.35)
    # drawn last, so the fields above are the same as without it
    softmax_scale = float(rng.choice([0.0, 0.0, 0.05, 0.2]))
    return dict(dtype=dtype, d=d, hq=hq, hkv=hkv, qmap=qmap, p=p, lens=lens, scale_q=scale_q,
                min_ws=min_ws, softmax_scale=softmax_scale)


@pytest.mark.parametrize("seed", range(24))
def test_random_suffix_group(seed):
    """Phase B forward and backward (gK/gV added into nonzero accumulators)."""
    c = draw_suffix_case(seed)
    print(f"\nsweep suffix seed {seed}: {c}", flush=True)
    dtype, d, hq, hkv, p = c["dtype"], c["d"], c["hq"], c["hkv"], c["p"]
    g = random_small_group(500 + seed, hq, hkv, d, p, c["lens"], dtype, scale_q=c["scale_q"])
    cu = g["cu_seqlens"]
    rows = int(cu[-1])
    ds, scale = _scale(c)
    desc = _desc(hq, hkv, d, dtype, c["qmap"], ds)
    t = {k: dev(g[k], dtype) for k in ("k_p", "v_p", "q_s", "k_s", "v_s", "do_s")}
    o, lse = G.suffix_fwd(desc, t["k_p"], t["v_p"], cu, t["q_s"], t["k_s"], t["v_s"])
    rng = np.random.default_rng(seed)
    gk0 = rng.standard_normal((p, hkv, d)).astype(np.float32)
    gv0 = rng.standard_normal((p, hkv, d)).astype(np.float32)
    gk, gv = torch.from_numpy(gk0).cuda(), torch.from_numpy(gv0).cuda()
    ws = None
    if c["min_ws"]:
        ws = torch.empty(max(16, pf.pf_workspace_size_min(pf.PF_OP_SUFFIX_BWD, desc, p, rows)),
                         dtype=torch.uint8, device="cuda")
    dq, dk, dv = G.suffix_bwd(desc, t["k_p"], t["v_p"], cu, t["q_s"], t["k_s"], t["v_s"], o, lse,
                              t["do_s"], gk, gv, ws=ws)
    torch.cuda.synchronize()
    ref = oracle.suffix_attention(g["k_p"], g["v_p"], g["q_s"], g["k_s"], g["v_s"], g["do_s"], cu,
                                  scale, oracle.head_map(hq, hkv, c["qmap"]))
    tol = TOL[dtype]
    for name, got, key in (("O_S", o, "o_s"), ("LSE_S", lse, "lse_s"), ("dQ_S", dq, "dq_s"),
                           ("dK_S", dk, "dk_s"), ("dV_S", dv, "dv_s")):
        check(name, host(got), ref[key], tol)
    if p > 0:
        check("gK (accumulated)", host(gk), gk0 + ref["gk"], tol)
        check("gV (accumulated)", host(gv), gv0 + ref["gv"], tol)


def draw_prefix_case(seed):
    rng = np.random.default_rng(9500 + seed)
    dtype, d = _dtype_dim(rng)
    hq, hkv, qmap = _heads(rng)
    p = int(rng.choice([1, 2, 31, 33, 64, 65, 130, 255, 257, 384, 511]))
    c = dict(dtype=dtype, d=d, hq=hq, hkv=hkv, qmap=qmap, p=p,
             with_do=bool(rng.random() < 0.8), scale_q=float(rng.choice([1.0, 3.0])),
             min_ws=bool(rng.random() < 0.35))
    c["softmax_scale"] = float(rng.choice([0.0, 0.0, 0.05, 0.2]))
    return c


@pytest.mark.parametrize("seed", range(10))
def test_random_prefix_group(seed):
    """Phase A, then Phase C with random gK/gV injected (fp32 dK/dV out)."""
    c = draw_prefix_case(seed)
    print(f"\nsweep prefix seed {seed}: {c}", flush=True)
    dtype, d, hq, hkv, p = c["dtype"], c["d"], c["hq"], c["hkv"], c["p"]
    g = random_small_group(600 + seed, hq, hkv, d, p, [1], dtype, scale_q=c["scale_q"])
    ds, scale = _scale(c)
    desc = _desc(hq, hkv, d, dtype, c["qmap"], ds)
    hmap = oracle.head_map(hq, hkv, c["qmap"])
    rng = np.random.default_rng(seed)
    gk_np = rng.standard_normal((p, hkv, d)).astype(np.float32)
    gv_np = rng.standard_normal((p, hkv, d)).astype(np.float32)
    t = {k: dev(g[k], dtype) for k in ("q_p", "k_p", "v_p", "do_p")}
    o_p, lse_p = G.prefix_fwd(desc, t["q_p"], t["k_p"], t["v_p"])
    gk, gv = torch.from_numpy(gk_np).cuda(), torch.from_numpy(gv_np).cuda()
    ws = None
    if c["min_ws"]:
        ws = torch.empty(pf.pf_workspace_size_min(pf.PF_OP_PREFIX_BWD, desc, p, p),
                         dtype=torch.uint8, device="cuda")
    do_p = t["do_p"] if c["with_do"] else None
    dq, dk, dv = G.prefix_bwd(desc, t["q_p"], t["k_p"], t["v_p"], o_p, lse_p, do_p, gk, gv,
                              pf.PF_F32, ws=ws)
    torch.cuda.synchronize()
    ro, rlse = oracle.prefix_forward(g["q_p"], g["k_p"], g["v_p"], scale, hmap)
    rdq, rdk, rdv = oracle.prefix_backward_inject(g["q_p"], g["k_p"], g["v_p"],
                                                  g["do_p"] if c["with_do"] else None, gk_np,
                                                  gv_np, scale, hmap)
    tol = TOL[dtype]
    check("O_P", host(o_p), ro, tol)
    check("LSE_P", host(lse_p), rlse, tol)
    check("dQ_P", host(dq), rdq, tol)
    check("dK_P", host(dk), rdk, tol)
    check("dV_P", host(dv), rdv, tol)


def draw_window_case(seed):
    rng = np.random.default_rng(9800 + seed)
    dtype, d = _dtype_dim(rng)
    hq, hkv, qmap = _heads(rng)
    n_prod = int(rng.integers(1, 12))
    return dict(dtype=dtype, d=d, hq=hq, hkv=hkv, qmap=qmap, n_prod=n_prod,
                prod_len=int(rng.choice([20, 45, 80])), node=int(rng.integers(0, n_prod)),
                n_win=int(rng.integers(1, 10)), win_len=int(rng.choice([1, 30, 70])),
                min_ws=bool(rng.random() < 0.35))


@pytest.mark.parametrize("seed", range(10))
def test_random_window_under_a_producer_node(seed):
    """A consumer window under a random node of a random producer tree, reading
    that node's and its ancestors' rows in place; gK/gV added into the
    producer rows."""
    c = draw_window_case(seed)
    print(f"\nsweep window seed {seed}: {c}", flush=True)
    dtype, d, hq, hkv = c["dtype"], c["d"], c["hq"], c["hkv"]
    node_off_p, parent_p = random_tree(700 + seed, c["n_prod"], max_len=c["prod_len"], min_len=1)
    cp = int(node_off_p[-1])
    ranges = ancestor_row_ranges(node_off_p, parent_p, c["node"])
    node_off, parent = random_tree(800 + seed, c["n_win"], max_len=c["win_len"], min_len=1)
    print(f"  producer node_off {node_off_p.tolist()} parent {parent_p.tolist()}; ranges "
          f"{ranges}; window node_off {node_off.tolist()} parent {parent.tolist()}", flush=True)
    gp = random_tree_group(700 + seed, node_off_p, hq, hkv, d, dtype)
    tg = random_tree_group(800 + seed, node_off, hq, hkv, d, dtype)
    desc = _desc(hq, hkv, d, dtype, c["qmap"])
    kc, vc = dev(gp["k"], dtype), dev(gp["v"], dtype)
    tt = {k: dev(tg[k], dtype) for k in ("q", "k", "v", "do")}
    o, lse = G.tree_suffix_fwd_ranges(desc, kc, vc, ranges, node_off, parent, tt["q"], tt["k"],
                                      tt["v"])
    gk = torch.zeros(cp, hkv, d, dtype=torch.float32, device="cuda")
    gv = torch.zeros_like(gk)
    ws = None
    if c["min_ws"]:
        nk = pf.pf_ranges_cached_keys([n for _, n in ranges])
        ws = torch.empty(pf.pf_workspace_size_min(pf.PF_OP_TREE_SUFFIX_BWD, desc, nk,
                                                  int(node_off[-1])),
                         dtype=torch.uint8, device="cuda")
    dq, dk, dv = G.tree_suffix_bwd_ranges(desc, kc, vc, ranges, node_off, parent, tt["q"], tt["k"],
                                          tt["v"], o, lse, tt["do"], gk, gv, ws=ws)
    torch.cuda.synchronize()
    ref = oracle.tree_window_attention_ranges(gp["k"], gp["v"], ranges, tg["q"], tg["k"], tg["v"],
                                              tg["do"], node_off, parent, 1.0 / math.sqrt(d),
                                              oracle.head_map(hq, hkv, c["qmap"]))
    tol = TOL[dtype]
    for name, got in (("O", o), ("LSE", lse), ("dQ", dq), ("dK", dk), ("dV", dv), ("gK", gk),
                      ("gV", gv)):
        check(name, host(got), ref[name.lower()], tol)
    used = np.zeros(cp, dtype=bool)
    for s, n in ranges:
        used[s:s + n] = True
    assert np.all(host(gk)[~used] == 0) and np.all(host(gv)[~used] == 0)


def draw_tree_case(seed):
    rng = np.random.default_rng(9900 + seed)
    dtype, d = _dtype_dim(rng)
    hq, hkv, qmap = _heads(rng)
    return dict(dtype=dtype, d=d, hq=hq, hkv=hkv, qmap=qmap, n=int(rng.integers(1, 20)),
                max_len=int(rng.choice([1, 20, 64, 130])), min_len=int(rng.choice([0, 1])),
                min_ws=bool(rng.random() < 0.35),
                softmax_scale=float(rng.choice([0.0, 0.0, 0.05, 0.2])))


@pytest.mark.parametrize("seed", range(10))
def test_random_tree(seed):
    """Tree attention forward and backward over a random tree (node lengths
    from 0, fan-out random), and the backward with random gK/gV injected."""
    c = draw_tree_case(seed)
    print(f"\nsweep tree seed {seed}: {c}", flush=True)
    dtype, d, hq, hkv = c["dtype"], c["d"], c["hq"], c["hkv"]
    node_off, parent = random_tree(900 + seed, c["n"], max_len=c["max_len"], min_len=c["min_len"])
    rows = int(node_off[-1])
    print(f"  node_off {node_off.tolist()} parent {parent.tolist()}", flush=True)
    if rows == 0:
        pytest.skip("the drawn tree has no rows")
    tg = random_tree_group(900 + seed, node_off, hq, hkv, d, dtype)
    ds, scale = _scale(c)
    desc = _desc(hq, hkv, d, dtype, c["qmap"], ds)
    hmap = oracle.head_map(hq, hkv, c["qmap"])
    t = {k: dev(tg[k], dtype) for k in ("q", "k", "v", "do")}
    o, lse = G.tree_fwd(desc, node_off, parent, t["q"], t["k"], t["v"])
    ws = None
    if c["min_ws"]:
        ws = torch.empty(pf.pf_workspace_size_min(pf.PF_OP_TREE_BWD, desc, 0, rows),
                         dtype=torch.uint8, device="cuda")
    dq, dk, dv = G.tree_bwd(desc, node_off, parent, t["q"], t["k"], t["v"], o, lse, t["do"], ws=ws)
    rng = np.random.default_rng(seed)
    gk_np = rng.standard_normal((rows, hkv, d)).astype(np.float32)
    gv_np = rng.standard_normal((rows, hkv, d)).astype(np.float32)
    gk, gv = torch.from_numpy(gk_np).cuda(), torch.from_numpy(gv_np).cuda()
    iq, ik, iv = G.tree_bwd_inject(desc, node_off, parent, t["q"], t["k"], t["v"], o, lse, t["do"],
                                   gk, gv, dkv_dtype=pf.PF_F32, ws=ws)
    torch.cuda.synchronize()
    ref = oracle.tree_attention_direct(tg["q"], tg["k"], tg["v"], tg["do"], node_off, parent,
                                       scale, hmap)
    tol = TOL[dtype]
    for name, got in (("O", o), ("LSE", lse), ("dQ", dq), ("dK", dk), ("dV", dv)):
        check(name, host(got), ref[name.lower()], tol)
    rdq, rdk, rdv = oracle.tree_backward_inject(tg["q"], tg["k"], tg["v"], tg["do"], node_off,
                                                parent, gk_np, gv_np, scale, hmap)
    check("dQ (injected)", host(iq), rdq, tol)
    check("dK (injected, fp32 out)", host(ik), rdk, tol)
    check("dV (injected, fp32 out)", host(iv), rdv, tol)
