"""GPU parity at the full measured sizes.

The GPU runs each workload exactly as the benchmark times it:
- the fp32 group of config 1;
- the 32/8-head group at P = 4096 with all 8 suffixes in one Phase-B call
  (config 2);
- the RAG-shaped varlen group at P = 16384: Phase A, Phase B in 4 calls
  adding into one gK/gV, Phase C (config 3);
- the 64-suffix group at P = 8192 in 8 microbatch calls (config 4);
- the 12288-row rollout tree (config 5);
- four irregular tree windows over a 4096-row prefix with the producer
  backward (config 6);
- the compact log-probabilities of the config-5 tree over a 151936-token
  vocabulary (config 7).

The fp64 oracle then recomputes whole KV-head groups (every query head that
reads the chosen KV head, every row), and each output slice is compared
normwise against it: 2e-2, the bf16 bar, and 1e-4 for fp32.  Heads are
independent, so a KV-head group is an exact sub-problem of the full call.

Invariants checked at full size, where the oracle cannot cover every head
or row:
- the prefix-side gradient of a call is the same whichever microbatch split
  produced it (up to fp32 summation order);
- the outputs are finite;
- every compact row's log-sum-exp lies in [max z, max z + ln V];
- every log-probability is at most 0;
- every row of dz sums to zero.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import TOL, check, dev, host
from tests.row_blocks import prefix_phases_by_row_blocks
from workloads import generate, get_config

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import shared_prefix_attention_pf_amd as pf
    from shared_prefix_attention_pf_amd import group as G


def _heads_of(cfg, g):
    gs = cfg.group_size
    return slice(g * gs, (g + 1) * gs)


def _phase_b(cfg, data, desc, calls):
    """Phase B as `calls` consecutive calls (lists of (first, last) suffixes),
    accumulating gK/gV.  Returns per-row outputs and the accumulators."""
    p, cu = cfg.prefix_len, data["cu_seqlens"]
    t = {k: dev(data[k], cfg.dtype) for k in ("k_p", "v_p", "q_s", "k_s", "v_s", "do_s")}
    rows = int(cu[-1])
    out = {"o": torch.empty_like(t["q_s"]), "dq": torch.empty_like(t["q_s"]),
           "dk": torch.empty_like(t["k_s"]), "dv": torch.empty_like(t["v_s"]),
           "lse": torch.empty(cfg.num_q_heads, rows, device="cuda")}
    gk = torch.zeros(p, cfg.num_kv_heads, cfg.head_dim, device="cuda")
    gv = torch.zeros_like(gk)
    for a, b in calls:
        r0, r1 = int(cu[a]), int(cu[b])
        sub = (cu[a:b + 1] - cu[a]).astype(np.int32)
        sl = slice(r0, r1)
        o, lse = G.suffix_fwd(desc, t["k_p"], t["v_p"], sub, t["q_s"][sl], t["k_s"][sl],
                              t["v_s"][sl])
        dq, dk, dv = G.suffix_bwd(desc, t["k_p"], t["v_p"], sub, t["q_s"][sl], t["k_s"][sl],
                                  t["v_s"][sl], o, lse, t["do_s"][sl], gk, gv)
        out["o"][sl], out["lse"][:, sl] = o, lse
        out["dq"][sl], out["dk"][sl], out["dv"][sl] = dq, dk, dv
    torch.cuda.synchronize()
    res = {k: host(v) for k, v in out.items()}
    res["gk"], res["gv"] = host(gk), host(gv)
    return res


def _check_phase_b_group(cfg, data, res, g):
    hs = _heads_of(cfg, g)
    scale = 1.0 / math.sqrt(cfg.head_dim)
    hmap = np.zeros(cfg.group_size, dtype=np.int64)
    print(f"  oracle Phase B, KV head {g}", flush=True)
    ref = oracle.suffix_attention(data["k_p"][:, g:g + 1], data["v_p"][:, g:g + 1],
                                  data["q_s"][:, hs], data["k_s"][:, g:g + 1],
                                  data["v_s"][:, g:g + 1], data["do_s"][:, hs],
                                  data["cu_seqlens"], scale, hmap)
    tol = TOL[cfg.dtype]
    check(f"O_S[g{g}]", res["o"][:, hs], ref["o_s"], tol)
    check(f"LSE_S[g{g}]", res["lse"][hs], ref["lse_s"], tol)
    check(f"dQ_S[g{g}]", res["dq"][:, hs], ref["dq_s"], tol)
    check(f"dK_S[g{g}]", res["dk"][:, g:g + 1], ref["dk_s"], tol)
    check(f"dV_S[g{g}]", res["dv"][:, g:g + 1], ref["dv_s"], tol)
    check(f"gK[g{g}]", res["gk"][:, g:g + 1], ref["gk"], tol)
    check(f"gV[g{g}]", res["gv"][:, g:g + 1], ref["gv"], tol)
    return ref


def _desc(cfg):
    return pf.AttnDesc(cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim,
                       pf.PF_BF16 if cfg.dtype == "bf16" else pf.PF_F32)


def test_config1_fp32_all_phases():
    """The fp32 group of config 1 (2 heads, d 64, P 256, 4 suffixes of 64) as
    the benchmark generates it: Phase A, Phase B and Phase C with the
    accumulated gK/gV, every head against the oracle at the fp32 bar."""
    cfg = get_config(1)
    print(f"\ngenerating config {cfg.cid}", flush=True)
    data = generate(cfg)
    desc = pf.AttnDesc(cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, pf.PF_F32)
    res = _phase_b(cfg, data, desc, [(0, cfg.n_suffix)])
    q_p, k_p, v_p, do_p = (dev(data[k], cfg.dtype) for k in ("q_p", "k_p", "v_p", "do_p"))
    o_p, lse_p = G.prefix_fwd(desc, q_p, k_p, v_p)
    gk = torch.from_numpy(res["gk"].astype(np.float32)).cuda()
    gv = torch.from_numpy(res["gv"].astype(np.float32)).cuda()
    dq_p, dk_p, dv_p = G.prefix_bwd(desc, q_p, k_p, v_p, o_p, lse_p, do_p, gk, gv)
    torch.cuda.synchronize()
    scale = 1.0 / math.sqrt(cfg.head_dim)
    hmap = oracle.head_map(cfg.num_q_heads, cfg.num_kv_heads)
    tol = TOL[cfg.dtype]
    ref = oracle.suffix_attention(data["k_p"], data["v_p"], data["q_s"], data["k_s"], data["v_s"],
                                  data["do_s"], data["cu_seqlens"], scale, hmap)
    check("O_S", res["o"], ref["o_s"], tol)
    check("LSE_S", res["lse"], ref["lse_s"], tol)
    check("dQ_S", res["dq"], ref["dq_s"], tol)
    check("dK_S", res["dk"], ref["dk_s"], tol)
    check("dV_S", res["dv"], ref["dv_s"], tol)
    check("gK", res["gk"], ref["gk"], tol)
    check("gV", res["gv"], ref["gv"], tol)
    ro, rl = oracle.prefix_forward(data["q_p"], data["k_p"], data["v_p"], scale, hmap)
    check("O_P", host(o_p), ro, tol)
    check("LSE_P", host(lse_p), rl, tol)
    rdq, rdk, rdv = oracle.prefix_backward_inject(data["q_p"], data["k_p"], data["v_p"],
                                                  data["do_p"], ref["gk"], ref["gv"], scale, hmap)
    check("dQ_P", host(dq_p), rdq, tol)
    check("dK_P", host(dk_p), rdk, tol)
    check("dV_P", host(dv_p), rdv, tol)


@pytest.mark.parametrize("cid", [2, 9])
def test_config2_all_phases_full_size(cid):
    """Phase A, one Phase-B call over all 8 suffixes, Phase C with the
    accumulated gK/gV injected: the benchmark's step at config 2 (bf16) and at
    config 9 (the same shapes in fp32)."""
    cfg = get_config(cid)
    print(f"\ngenerating config {cfg.cid}", flush=True)
    data = generate(cfg)
    desc = _desc(cfg)
    n = cfg.n_suffix
    res = _phase_b(cfg, data, desc, [(0, n)])
    # Phase A and Phase C on the GPU, C with the GPU's accumulators
    q_p, k_p, v_p, do_p = (dev(data[k], cfg.dtype) for k in ("q_p", "k_p", "v_p", "do_p"))
    o_p, lse_p = G.prefix_fwd(desc, q_p, k_p, v_p)
    gk = torch.from_numpy(res["gk"].astype(np.float32)).cuda()
    gv = torch.from_numpy(res["gv"].astype(np.float32)).cuda()
    dq_p, dk_p, dv_p = G.prefix_bwd(desc, q_p, k_p, v_p, o_p, lse_p, do_p, gk, gv)
    torch.cuda.synchronize()
    o_p, lse_p, dq_p, dk_p, dv_p = (host(x) for x in (o_p, lse_p, dq_p, dk_p, dv_p))
    for x in (res["o"], res["dq"], res["dk"], res["dv"], res["gk"], o_p, dq_p, dk_p, dv_p):
        assert np.all(np.isfinite(x))
    scale = 1.0 / math.sqrt(cfg.head_dim)
    hmap = np.zeros(cfg.group_size, dtype=np.int64)
    tol = TOL[cfg.dtype]
    for g in (0, 5):
        ref_b = _check_phase_b_group(cfg, data, res, g)
        hs = _heads_of(cfg, g)
        print(f"  oracle Phase A/C, KV head {g}", flush=True)
        ro, rl = oracle.prefix_forward(data["q_p"][:, hs], data["k_p"][:, g:g + 1],
                                       data["v_p"][:, g:g + 1], scale, hmap)
        check(f"O_P[g{g}]", o_p[:, hs], ro, tol)
        check(f"LSE_P[g{g}]", lse_p[hs], rl, tol)
        rdq, rdk, rdv = oracle.prefix_backward_inject(
            data["q_p"][:, hs], data["k_p"][:, g:g + 1], data["v_p"][:, g:g + 1],
            data["do_p"][:, hs], ref_b["gk"], ref_b["gv"], scale, hmap)
        check(f"dQ_P[g{g}]", dq_p[:, hs], rdq, tol)
        check(f"dK_P[g{g}]", dk_p[:, g:g + 1], rdk, tol)
        check(f"dV_P[g{g}]", dv_p[:, g:g + 1], rdv, tol)


def test_config4_microbatches_full_size():
    """Phase B of 64 suffixes at P = 8192 as 8 calls of 8 (the benchmark's
    split): oracle on one KV-head group, and the accumulated gK/gV of a
    different split (2 calls of 32) agree to fp32 summation order."""
    cfg = get_config(4)
    print(f"\ngenerating config {cfg.cid}", flush=True)
    data = generate(cfg)
    desc = _desc(cfg)
    calls = [tuple(int(x) for x in mb) for mb in data["microbatches"]]
    res = _phase_b(cfg, data, desc, calls)
    _check_phase_b_group(cfg, data, res, 3)
    res2 = _phase_b(cfg, data, desc, [(0, 32), (32, 64)])
    for name in ("gk", "gv"):
        rel = np.abs(res2[name] - res[name]).max() / np.abs(res[name]).max()
        print(f"  {name}: split 8x8 vs 2x32 max rel diff {rel:.2e}", flush=True)
        assert rel < 1e-5
    for name in ("o", "dq", "dk", "dv"):
        assert np.array_equal(res[name], res2[name]), f"{name} depends on the split"


@pytest.mark.timeout(1200)
def test_config3_varlen_full_size():
    """The RAG-shaped group as the benchmark runs it: Phase A at P = 16384,
    Phase B of 16 varlen suffixes in 4 calls adding into one gK/gV, and
    Phase C with that gK/gV injected (the full workspace, so the backward
    stores dS: the largest dS buffer of any workload, Hq x P^2 bf16).  For one
    KV-head group (its 4 query heads, every row) the fp64 oracle recomputes
    every Phase-B output, the gK/gV accumulated over the 4 calls (against the
    oracle over all 16 suffixes at once), and Phase A / Phase C, assembled from
    the oracle over blocks of 2048 prefix rows (tests/row_blocks.py)."""
    cfg = get_config(3)
    print(f"\ngenerating config {cfg.cid}", flush=True)
    data = generate(cfg)
    desc = _desc(cfg)
    p = cfg.prefix_len
    calls = [tuple(int(x) for x in mb) for mb in data["microbatches"]]
    assert len(calls) == 4
    res = _phase_b(cfg, data, desc, calls)
    q_p, k_p, v_p, do_p = (dev(data[k], cfg.dtype) for k in ("q_p", "k_p", "v_p", "do_p"))
    o_p, lse_p = G.prefix_fwd(desc, q_p, k_p, v_p)
    gk = torch.from_numpy(res["gk"].astype(np.float32)).cuda()
    gv = torch.from_numpy(res["gv"].astype(np.float32)).cuda()
    ws_c = G.workspace(pf.PF_OP_PREFIX_BWD, desc, p, p, "cuda")
    assert ws_c.numel() > pf.pf_workspace_size_min(pf.PF_OP_PREFIX_BWD, desc, p, p)
    dq_p, dk_p, dv_p = G.prefix_bwd(desc, q_p, k_p, v_p, o_p, lse_p, do_p, gk, gv, ws=ws_c)
    torch.cuda.synchronize()
    del ws_c, q_p, k_p, v_p, do_p, gk, gv
    o_p, lse_p, dq_p, dk_p, dv_p = (host(x) for x in (o_p, lse_p, dq_p, dk_p, dv_p))
    for x in (res["o"], res["dq"], res["dk"], res["dv"], res["gk"], res["gv"], o_p, lse_p, dq_p,
              dk_p, dv_p):
        assert np.all(np.isfinite(x))
    g = 6
    hs = _heads_of(cfg, g)
    scale = 1.0 / math.sqrt(cfg.head_dim)
    hmap = np.zeros(cfg.group_size, dtype=np.int64)
    tol = TOL[cfg.dtype]
    # every Phase-B output of the group, and gK/gV summed over all 16 suffixes
    ref_b = _check_phase_b_group(cfg, data, res, g)
    torch.cuda.empty_cache()

    def progress(r0, r1):
        print(f"  oracle prefix rows [{r0}, {r1}), KV head {g}", flush=True)

    kp, vp = data["k_p"][:, g:g + 1], data["v_p"][:, g:g + 1]
    ro, rl, rdq, rdk, rdv = prefix_phases_by_row_blocks(
        data["q_p"][:, hs], kp, vp, data["do_p"][:, hs], ref_b["gk"], ref_b["gv"], scale, hmap,
        2048, progress)
    check(f"O_P[g{g}]", o_p[:, hs], ro, tol)
    check(f"LSE_P[g{g}]", lse_p[hs], rl, tol)
    check(f"dQ_P[g{g}]", dq_p[:, hs], rdq, tol)
    check(f"dK_P[g{g}]", dk_p[:, g:g + 1], rdk, tol)
    check(f"dV_P[g{g}]", dv_p[:, g:g + 1], rdv, tol)


def test_config5_tree_full_size():
    """The 12288-row rollout tree, forward and backward in one call each:
    oracle (ancestor mask over the compact rows) on one KV-head group."""
    cfg = get_config(5)
    print(f"\ngenerating config {cfg.cid}", flush=True)
    data = generate(cfg)
    desc = _desc(cfg)
    node_off, parent = data["node_off"], data["parent"]
    q, k, v, do = (dev(data[n], cfg.dtype) for n in ("q", "k", "v", "do"))
    o, lse = G.tree_fwd(desc, node_off, parent, q, k, v)
    dq, dk, dv = G.tree_bwd(desc, node_off, parent, q, k, v, o, lse, do)
    torch.cuda.synchronize()
    o, lse, dq, dk, dv = (host(x) for x in (o, lse, dq, dk, dv))
    g = 2
    hs = _heads_of(cfg, g)
    scale = 1.0 / math.sqrt(cfg.head_dim)
    hmap = np.zeros(cfg.group_size, dtype=np.int64)
    print(f"  oracle tree, KV head {g}", flush=True)
    ref = oracle.tree_attention_direct(data["q"][:, hs], data["k"][:, g:g + 1],
                                       data["v"][:, g:g + 1], data["do"][:, hs], node_off, parent,
                                       scale, hmap)
    tol = TOL[cfg.dtype]
    check("O", o[:, hs], ref["o"], tol)
    check("LSE", lse[hs], ref["lse"], tol)
    check("dQ", dq[:, hs], ref["dq"], tol)
    check("dK", dk[:, g:g + 1], ref["dk"], tol)
    check("dV", dv[:, g:g + 1], ref["dv"], tol)


def test_config6_tree_windows_full_size():
    """Phase A, four irregular tree windows over the 4096-row prefix (each a
    forward and a backward call adding into one gK/gV), then Phase C with that
    gK/gV injected: the benchmark's step at config 6.  The oracle recomputes
    one KV-head group through every window and both prefix phases."""
    cfg = get_config(6)
    print(f"\ngenerating config {cfg.cid}", flush=True)
    data = generate(cfg)
    desc = _desc(cfg)
    p = cfg.prefix_len
    q_p, k_p, v_p, do_p = (dev(data[k], cfg.dtype) for k in ("q_p", "k_p", "v_p", "do_p"))
    o_p, lse_p = G.prefix_fwd(desc, q_p, k_p, v_p)
    gk = torch.zeros(p, cfg.num_kv_heads, cfg.head_dim, device="cuda")
    gv = torch.zeros_like(gk)
    outs = []
    for wd in data["windows"]:
        q, k, v, do = (dev(wd[n], cfg.dtype) for n in ("q", "k", "v", "do"))
        o, lse = G.tree_suffix_fwd(desc, k_p, v_p, wd["node_off"], wd["parent"], q, k, v)
        dq, dk, dv = G.tree_suffix_bwd(desc, k_p, v_p, wd["node_off"], wd["parent"], q, k, v, o,
                                       lse, do, gk, gv)
        outs.append((o, lse, dq, dk, dv))
    dq_p, dk_p, dv_p = G.prefix_bwd(desc, q_p, k_p, v_p, o_p, lse_p, do_p, gk, gv)
    torch.cuda.synchronize()
    outs = [tuple(host(x) for x in w) for w in outs]
    o_p, lse_p, dq_p, dk_p, dv_p, gk, gv = (host(x) for x in (o_p, lse_p, dq_p, dk_p, dv_p, gk,
                                                                gv))
    for x in (o_p, dq_p, dk_p, dv_p, gk, gv):
        assert np.all(np.isfinite(x))
    g = 5
    hs = _heads_of(cfg, g)
    scale = 1.0 / math.sqrt(cfg.head_dim)
    hmap = np.zeros(cfg.group_size, dtype=np.int64)
    tol = TOL[cfg.dtype]
    kp, vp = data["k_p"][:, g:g + 1], data["v_p"][:, g:g + 1]
    ref_gk = np.zeros((p, 1, cfg.head_dim))
    ref_gv = np.zeros_like(ref_gk)
    for w, (wd, (o, lse, dq, dk, dv)) in enumerate(zip(data["windows"], outs)):
        assert np.all(np.isfinite(dq)) and np.all(np.isfinite(dk))
        print(f"  oracle window {w} ({int(wd['node_off'][-1])} rows), KV head {g}", flush=True)
        ref = oracle.tree_window_attention(kp, vp, wd["q"][:, hs], wd["k"][:, g:g + 1],
                                           wd["v"][:, g:g + 1], wd["do"][:, hs], wd["node_off"],
                                           wd["parent"], scale, hmap)
        check(f"O[w{w}]", o[:, hs], ref["o"], tol)
        check(f"LSE[w{w}]", lse[hs], ref["lse"], tol)
        check(f"dQ[w{w}]", dq[:, hs], ref["dq"], tol)
        check(f"dK[w{w}]", dk[:, g:g + 1], ref["dk"], tol)
        check(f"dV[w{w}]", dv[:, g:g + 1], ref["dv"], tol)
        ref_gk += ref["gk"]
        ref_gv += ref["gv"]
    check("gK (4 windows)", gk[:, g:g + 1], ref_gk, tol)
    check("gV (4 windows)", gv[:, g:g + 1], ref_gv, tol)
    # the benchmark runs the four trees as one call (a forest over the prefix)
    from workloads.gen import forest
    no, pa = forest([(wd["node_off"], wd["parent"]) for wd in data["windows"]])
    cat = {n: np.concatenate([wd[n] for wd in data["windows"]], axis=0)
           for n in ("q", "k", "v", "do")}
    tt = {n: dev(x, cfg.dtype) for n, x in cat.items()}
    fgk = torch.zeros(p, cfg.num_kv_heads, cfg.head_dim, device="cuda")
    fgv = torch.zeros_like(fgk)
    fo, flse = G.tree_suffix_fwd(desc, k_p, v_p, no, pa, tt["q"], tt["k"], tt["v"])
    fdq, fdk, fdv = G.tree_suffix_bwd(desc, k_p, v_p, no, pa, tt["q"], tt["k"], tt["v"], fo, flse,
                                      tt["do"], fgk, fgv)
    torch.cuda.synchronize()
    r0 = 0
    for w, (o, lse, dq, dk, dv) in enumerate(outs):
        r1 = r0 + o.shape[0]
        for name, x, y in (("O", fo[r0:r1], o), ("dQ", fdq[r0:r1], dq), ("dK", fdk[r0:r1], dk),
                           ("dV", fdv[r0:r1], dv), ("LSE", flse[:, r0:r1], lse)):
            check(f"one call vs window {w}: {name}", host(x), y, tol)
        r0 = r1
    check("one call gK (g)", host(fgk)[:, g:g + 1], ref_gk, tol)
    check("one call gV (g)", host(fgv)[:, g:g + 1], ref_gv, tol)
    print(f"  oracle Phase A/C, KV head {g}", flush=True)
    ro, rl = oracle.prefix_forward(data["q_p"][:, hs], kp, vp, scale, hmap)
    check("O_P", o_p[:, hs], ro, tol)
    check("LSE_P", lse_p[hs], rl, tol)
    rdq, rdk, rdv = oracle.prefix_backward_inject(data["q_p"][:, hs], kp, vp, data["do_p"][:, hs],
                                                  ref_gk, ref_gv, scale, hmap)
    check("dQ_P", dq_p[:, hs], rdq, tol)
    check("dK_P", dk_p[:, g:g + 1], rdk, tol)
    check("dV_P", dv_p[:, g:g + 1], rdv, tol)


def test_config7_compact_logprob_full_size():
    """Compact log-probabilities of the config-5 tree's 12288 rows over a
    151936-token vocabulary, logits drawn on the device from the seed as the
    benchmark draws them.  The oracle recomputes sampled rows (the root, rows
    of every tree level, the last row); properties hold for every row."""
    cfg = get_config(7)
    print(f"\ngenerating config {cfg.cid}", flush=True)
    data = generate(cfg)
    c, v = int(data["node_off"][-1]), cfg.logprob_vocab
    s_pos = len(data["m"])
    gen = torch.Generator(device="cuda")
    gen.manual_seed(cfg.seed)
    z = (torch.randn(c, v, generator=gen, device="cuda") * 3.0).to(torch.bfloat16)
    ints = {k: torch.from_numpy(data[k]).cuda() for k in ("row_ptr", "pos", "y")}
    lse = torch.empty(c, device="cuda")
    logp = torch.full((s_pos,), 7.0, device="cuda")
    dz = torch.empty_like(z)
    pf.pf_compact_logprob_fwd(z, ints["row_ptr"], ints["pos"], ints["y"], lse, logp)
    pf.pf_compact_logprob_bwd(z, lse, ints["row_ptr"], ints["pos"], ints["y"],
                              torch.from_numpy(data["dlogp"]).cuda(), dz)
    torch.cuda.synchronize()
    # properties over every row and position
    zmax = z.float().amax(dim=1)
    assert torch.all(lse >= zmax - 1e-3).item()
    assert torch.all(lse <= zmax + math.log(v) + 1e-3).item()
    assert torch.all(logp <= 1e-3).item(), "a log-probability above 0 (or a position not written)"
    dzf = dz.float()
    row_sum = dzf.sum(dim=1).abs()
    row_abs = dzf.abs().sum(dim=1)
    worst = (row_sum / row_abs.clamp_min(1e-30)).max().item()
    print(f"  max |sum dz| / sum |dz| over rows: {worst:.2e}", flush=True)
    assert worst < 1e-2
    # sampled rows against the oracle
    node_off = data["node_off"]
    rows = sorted({0, int(node_off[1]) - 1, int(node_off[1]), int(node_off[5]) - 1,
                   int(node_off[5]) + 7, c // 2, c - 1})
    rp, ps = data["row_ptr"], data["pos"]
    tol = TOL["bf16"]
    for r in rows:
        zr = z[r:r + 1].float().cpu().double().numpy()
        sub_ptr = np.asarray([0, rp[r + 1] - rp[r]], dtype=np.int32)
        sub_pos = ps[rp[r]:rp[r + 1]]
        ref = oracle.compact_logprob(zr, sub_ptr, sub_pos, data["y"], data["dlogp"])
        print(f"  oracle row {r} ({len(sub_pos)} positions)", flush=True)
        check(f"lse[{r}]", lse[r:r + 1].cpu().double().numpy(), ref["lse"], tol)
        check(f"logp[row {r}]", logp[torch.from_numpy(sub_pos.astype(np.int64)).cuda()]
              .cpu().double().numpy(), ref["logp"][sub_pos], tol)
        check(f"dz[{r}]", dz[r:r + 1].float().cpu().double().numpy(), ref["dz"], tol)


@pytest.mark.timeout(1200)
def test_config8_windows_under_producer_full_size():
    """Per-node caches at the measured size: the producer tree (10240 compact
    rows), its forward; 8 windows, each hung under a depth-2 node and reading
    the 3584 rows of that node and its ancestors in place, adding into the
    producer rows' gK/gV; the producer backward with them injected.  The
    oracle recomputes one KV-head group: every window (gather, window
    attention, scatter-add), the accumulated gK/gV, and the producer's
    forward and injected backward."""
    cfg = get_config(8)
    print(f"\ngenerating config {cfg.cid}", flush=True)
    data = generate(cfg)
    desc = _desc(cfg)
    node_off, parent = data["node_off"], data["parent"]
    c = int(node_off[-1])
    t = {n: dev(data[n], cfg.dtype) for n in ("q", "k", "v", "do")}
    o_c, lse_c = G.tree_fwd(desc, node_off, parent, t["q"], t["k"], t["v"])
    gk = torch.zeros(c, cfg.num_kv_heads, cfg.head_dim, device="cuda")
    gv = torch.zeros_like(gk)
    outs = []
    for wd in data["windows"]:
        tw = {n: dev(wd[n], cfg.dtype) for n in ("q", "k", "v", "do")}
        o, lse = G.tree_suffix_fwd_ranges(desc, t["k"], t["v"], wd["ranges"], wd["node_off"],
                                          wd["parent"], tw["q"], tw["k"], tw["v"])
        dq, dk, dv = G.tree_suffix_bwd_ranges(desc, t["k"], t["v"], wd["ranges"], wd["node_off"],
                                              wd["parent"], tw["q"], tw["k"], tw["v"], o, lse,
                                              tw["do"], gk, gv)
        outs.append(tuple(host(x) for x in (o, lse, dq, dk, dv)))
    dq_c, dk_c, dv_c = G.tree_bwd_inject(desc, node_off, parent, t["q"], t["k"], t["v"], o_c,
                                         lse_c, t["do"], gk, gv)
    torch.cuda.synchronize()
    o_c, dq_c, dk_c, dv_c, gk, gv = (host(x) for x in (o_c, dq_c, dk_c, dv_c, gk, gv))
    for x in (o_c, dq_c, dk_c, dv_c, gk, gv):
        assert np.all(np.isfinite(x))
    g = 3
    hs = _heads_of(cfg, g)
    scale = 1.0 / math.sqrt(cfg.head_dim)
    hmap = np.zeros(cfg.group_size, dtype=np.int64)
    tol = TOL[cfg.dtype]
    kc, vc = data["k"][:, g:g + 1], data["v"][:, g:g + 1]
    ref_gk = np.zeros((c, 1, cfg.head_dim))
    ref_gv = np.zeros_like(ref_gk)
    for w, (wd, (o, lse, dq, dk, dv)) in enumerate(zip(data["windows"], outs)):
        print(f"  oracle window {w} under node {wd['under']} ({int(wd['node_off'][-1])} rows), "
              f"KV head {g}", flush=True)
        ref = oracle.tree_window_attention_ranges(kc, vc, wd["ranges"], wd["q"][:, hs],
                                                  wd["k"][:, g:g + 1], wd["v"][:, g:g + 1],
                                                  wd["do"][:, hs], wd["node_off"], wd["parent"],
                                                  scale, hmap)
        check(f"O[w{w}]", o[:, hs], ref["o"], tol)
        check(f"LSE[w{w}]", lse[hs], ref["lse"], tol)
        check(f"dQ[w{w}]", dq[:, hs], ref["dq"], tol)
        check(f"dK[w{w}]", dk[:, g:g + 1], ref["dk"], tol)
        check(f"dV[w{w}]", dv[:, g:g + 1], ref["dv"], tol)
        ref_gk += ref["gk"]
        ref_gv += ref["gv"]
    check("gK (8 windows)", gk[:, g:g + 1], ref_gk, tol)
    check("gV (8 windows)", gv[:, g:g + 1], ref_gv, tol)
    print(f"  oracle producer tree, KV head {g}", flush=True)
    rp = oracle.tree_attention_direct(data["q"][:, hs], kc, vc, data["do"][:, hs], node_off,
                                      parent, scale, hmap, backward=False)
    check("producer O", o_c[:, hs], rp["o"], tol)
    rdq, rdk, rdv = oracle.tree_backward_inject(data["q"][:, hs], kc, vc, data["do"][:, hs],
                                                node_off, parent, ref_gk, ref_gv, scale, hmap)
    check("producer dQ", dq_c[:, hs], rdq, tol)
    check("producer dK (injected)", dk_c[:, g:g + 1], rdk, tol)
    check("producer dV (injected)", dv_c[:, g:g + 1], rdv, tol)
