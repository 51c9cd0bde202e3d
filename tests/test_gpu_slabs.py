"""The dS-buffer backward in key slabs: a workspace of pf_workspace_size_sliced
bytes holds the dS of one slab of keys at a time (external keys, then own
keys, in 256-key blocks), and dQ is summed slab by slab in fp32.  Each backward
(Phase B, Phase C, a tree, a tree window) is checked against the fp64 oracle
for several slab widths, including slabs that hold only external keys, only
own keys, or both.  dK/dV and gK/gV come from the same per-key-block work as
with every key in the buffer, so they must be bitwise equal to that run; dQ
differs from it only by the order of its fp32 sums.  A workspace between two
slab sizes must run the widest slab that fits it.

Tolerance: normwise max |x - y| / max |y| <= 2e-2 (bf16)."""
import math

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import TOL, check, dev, host
from workloads.gen import random_small_group, random_tree, random_tree_group

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import shared_prefix_attention_pf_amd as pf
    from shared_prefix_attention_pf_amd import group as G

HQ, HKV, D = 8, 2, 128


def _desc():
    return pf.AttnDesc(HQ, HKV, D, pf.PF_BF16)


def _ws(n):
    return torch.empty(n, dtype=torch.uint8, device="cuda")


def test_phase_b_in_key_slabs():
    p, lens = 700, [1, 300, 130, 64, 257]
    g = random_small_group(31, HQ, HKV, D, p, lens, "bf16")
    cu = g["cu_seqlens"]
    rows = int(cu[-1])
    desc = _desc()
    t = {k: dev(g[k], "bf16") for k in ("k_p", "v_p", "q_s", "k_s", "v_s", "do_s")}
    o_s, lse_s = G.suffix_fwd(desc, t["k_p"], t["v_p"], cu, t["q_s"], t["k_s"], t["v_s"])

    def run(n_ws):
        gk = torch.zeros(p, HKV, D, dtype=torch.float32, device="cuda")
        gv = torch.zeros_like(gk)
        dq, dk, dv = G.suffix_bwd(desc, t["k_p"], t["v_p"], cu, t["q_s"], t["k_s"], t["v_s"],
                                  o_s, lse_s, t["do_s"], gk, gv, ws=_ws(n_ws))
        torch.cuda.synchronize()
        return {"dq": dq.cpu(), "dk": dk.cpu(), "dv": dv.cpu(), "gk": gk.cpu(), "gv": gv.cpu()}

    full = run(pf.pf_workspace_size(pf.PF_OP_SUFFIX_BWD, desc, p, rows))
    ref = oracle.suffix_attention(g["k_p"], g["v_p"], g["q_s"], g["k_s"], g["v_s"], g["do_s"], cu,
                                  1.0 / math.sqrt(D), oracle.head_map(HQ, HKV))
    names = {"dq": "dq_s", "dk": "dk_s", "dv": "dv_s", "gk": "gk", "gv": "gv"}
    # 768 external + 768 own keys in the store: slabs of 256 (six), 512 (the
    # second spans both kinds), 768 (one of each kind) and 1024
    for slab in (256, 512, 768, 1024):
        n_ws = pf.pf_workspace_size_sliced(pf.PF_OP_SUFFIX_BWD, desc, p, rows, slab)
        print(f"\nslab {slab}: workspace {n_ws} bytes", flush=True)
        out = run(n_ws)
        for k in ("dk", "dv", "gk", "gv"):
            assert torch.equal(out[k], full[k]), f"slab {slab}: {k} differs from every-key run"
        for k, r in names.items():
            check(f"slab {slab}: {k}", host(out[k]), ref[r], TOL["bf16"])
        check(f"slab {slab}: dq vs every key", host(out["dq"]), host(full["dq"]), TOL["bf16"])
        again = run(n_ws)
        for k in out:
            assert torch.equal(out[k], again[k]), f"slab {slab}: {k} not bitwise repeatable"


def test_phase_c_in_key_slabs_and_the_widest_fitting_slab():
    p = 1000
    g = random_small_group(37, HQ, HKV, D, p, [1], "bf16")
    desc = _desc()
    rng = np.random.default_rng(9)
    gk_np = rng.standard_normal((p, HKV, D)).astype(np.float32)
    gv_np = rng.standard_normal((p, HKV, D)).astype(np.float32)
    t = {k: dev(g[k], "bf16") for k in ("q_p", "k_p", "v_p", "do_p")}
    o_p, lse_p = G.prefix_fwd(desc, t["q_p"], t["k_p"], t["v_p"])
    gk, gv = torch.from_numpy(gk_np).cuda(), torch.from_numpy(gv_np).cuda()

    def run(n_ws):
        out = G.prefix_bwd(desc, t["q_p"], t["k_p"], t["v_p"], o_p, lse_p, t["do_p"], gk, gv,
                           ws=_ws(n_ws))
        torch.cuda.synchronize()
        return [x.cpu() for x in out]

    full = run(pf.pf_workspace_size(pf.PF_OP_PREFIX_BWD, desc, p, p))
    ref = oracle.prefix_backward_inject(g["q_p"], g["k_p"], g["v_p"], g["do_p"], gk_np, gv_np,
                                        1.0 / math.sqrt(D), oracle.head_map(HQ, HKV))
    size = {s: pf.pf_workspace_size_sliced(pf.PF_OP_PREFIX_BWD, desc, p, p, s)
            for s in (256, 512, 768)}
    runs = {}
    for slab in (256, 512, 768):
        print(f"\nslab {slab}: workspace {size[slab]} bytes", flush=True)
        out = run(size[slab])
        runs[slab] = out
        for name, x, f, r in zip(("dQ_P", "dK_P", "dV_P"), out, full, ref):
            check(f"slab {slab}: {name}", host(x), r, TOL["bf16"])
        assert torch.equal(out[1], full[1]) and torch.equal(out[2], full[2])
        check(f"slab {slab}: dQ_P vs every key", host(out[0]), host(full[0]), TOL["bf16"])
    # a workspace between two slab sizes runs the wider slab that fits it
    assert size[256] < size[512] < size[768]
    between = run(size[512] + (size[768] - size[512]) // 2)
    assert all(torch.equal(x, y) for x, y in zip(between, runs[512]))
    just_under = run(size[512] - 1)
    assert all(torch.equal(x, y) for x, y in zip(just_under, runs[256]))


def test_tree_and_tree_window_in_key_slabs():
    desc = _desc()
    scale = 1.0 / math.sqrt(D)
    hmap = oracle.head_map(HQ, HKV)
    node_off, parent = random_tree(6, 12, max_len=120, min_len=1)
    rows = int(node_off[-1])
    print(f"\ntree node_off {node_off.tolist()} parent {parent.tolist()}", flush=True)
    tg = random_tree_group(6, node_off, HQ, HKV, D, "bf16")
    tt = {k: dev(tg[k], "bf16") for k in ("q", "k", "v", "do")}
    o, lse = G.tree_fwd(desc, node_off, parent, tt["q"], tt["k"], tt["v"])
    full = [x.cpu() for x in G.tree_bwd(desc, node_off, parent, tt["q"], tt["k"], tt["v"], o, lse,
                                        tt["do"])]
    ref = oracle.tree_attention_direct(tg["q"], tg["k"], tg["v"], tg["do"], node_off, parent,
                                       scale, hmap)
    n_ws = pf.pf_workspace_size_sliced(pf.PF_OP_TREE_BWD, desc, 0, rows, 256)
    out = [x.cpu() for x in G.tree_bwd(desc, node_off, parent, tt["q"], tt["k"], tt["v"], o, lse,
                                       tt["do"], ws=_ws(n_ws))]
    for name, x, f in zip(("dq", "dk", "dv"), out, full):
        check(f"tree slab 256: {name}", host(x), ref[name], TOL["bf16"])
    assert torch.equal(out[1], full[1]) and torch.equal(out[2], full[2])

    # a window of the same tree over a cached prefix of 520 keys
    p = 520
    rng = np.random.default_rng(3)
    kp_np = rng.standard_normal((p, HKV, D)).astype(np.float32)
    vp_np = rng.standard_normal((p, HKV, D)).astype(np.float32)
    kp, vp = dev(kp_np, "bf16"), dev(vp_np, "bf16")
    kp_r, vp_r = host(kp), host(vp)     # the bf16-rounded values the kernels see
    ow, lw = G.tree_suffix_fwd(desc, kp, vp, node_off, parent, tt["q"], tt["k"], tt["v"])

    def run_window(n_ws):
        gk = torch.zeros(p, HKV, D, dtype=torch.float32, device="cuda")
        gv = torch.zeros_like(gk)
        dq, dk, dv = G.tree_suffix_bwd(desc, kp, vp, node_off, parent, tt["q"], tt["k"], tt["v"],
                                       ow, lw, tt["do"], gk, gv,
                                       ws=None if n_ws is None else _ws(n_ws))
        torch.cuda.synchronize()
        return [x.cpu() for x in (dq, dk, dv, gk, gv)]

    wfull = run_window(None)
    ref = oracle.tree_window_attention(kp_r, vp_r, tg["q"], tg["k"], tg["v"], tg["do"], node_off,
                                       parent, scale, hmap)
    for slab in (256, 768):
        n_ws = pf.pf_workspace_size_sliced(pf.PF_OP_TREE_SUFFIX_BWD, desc, p, rows, slab)
        wout = run_window(n_ws)
        for name, x in zip(("dq", "dk", "dv", "gk", "gv"), wout):
            check(f"window slab {slab}: {name}", host(x), ref[name], TOL["bf16"])
        for i in (1, 2, 3, 4):
            assert torch.equal(wout[i], wfull[i])
