"""The Phase-B backward without a workspace (pf_suffix_attn_bwd_accum_noalloc).

It must give what pf_suffix_attn_bwd_accum gives, to the dtype's bar, for two
calls in a row on one GPU (the second smaller, so the static scratch still
holds the first call's tables and D / LSE), and both must match the oracle.
A repeated call must be bitwise identical to the first: nothing a call reads
from the scratch survives from an earlier call.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import TOL, check, dev, host
from workloads.gen import random_small_group

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import shared_prefix_attention_pf_amd as pf
    from shared_prefix_attention_pf_amd import group as G


def _run_case(seed, hq, hkv, p, lens, dtype="bf16", d=128):
    g = random_small_group(seed, hq, hkv, d, p, lens, dtype)
    cu = g["cu_seqlens"]
    t = {k: dev(g[k], dtype) for k in ("k_p", "v_p", "q_s", "k_s", "v_s", "do_s")}
    desc = pf.AttnDesc(hq, hkv, d, pf.PF_BF16 if dtype == "bf16" else pf.PF_F32)
    print(f"\ncase seed {seed}: {dtype}, Hq {hq}, Hkv {hkv}, d {d}, P {p}, suffixes {lens}",
          flush=True)
    o, lse = G.suffix_fwd(desc, t["k_p"], t["v_p"], cu, t["q_s"], t["k_s"], t["v_s"])
    # the workspace entry point
    gk_w = torch.zeros(p, hkv, d, device="cuda")
    gv_w = torch.zeros_like(gk_w)
    dq_w, dk_w, dv_w = G.suffix_bwd(desc, t["k_p"], t["v_p"], cu, t["q_s"], t["k_s"], t["v_s"],
                                    o, lse, t["do_s"], gk_w, gv_w)
    # the no-alloc entry point, twice
    outs = []
    for _ in range(2):
        gk = torch.zeros(p, hkv, d, device="cuda")
        gv = torch.zeros_like(gk)
        dq, dk, dv = (torch.empty_like(t["q_s"]), torch.empty_like(t["k_s"]),
                      torch.empty_like(t["v_s"]))
        pf.pf_suffix_attn_bwd_accum_noalloc(desc, p, t["k_p"], t["v_p"], cu, t["q_s"], t["k_s"],
                                            t["v_s"], o, lse, t["do_s"], dq, dk, dv, gk, gv)
        outs.append((dq, dk, dv, gk, gv))
    torch.cuda.synchronize()
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b), "a repeated no-alloc call changed its result"
    scale = 1.0 / math.sqrt(d)
    ref = oracle.suffix_attention(g["k_p"], g["v_p"], g["q_s"], g["k_s"], g["v_s"], g["do_s"], cu,
                                  scale, oracle.head_map(hq, hkv))
    tol = TOL[dtype]
    names = ("dQ_S", "dK_S", "dV_S", "gK", "gV")
    keys = ("dq_s", "dk_s", "dv_s", "gk", "gv")
    for name, key, x, w in zip(names, keys, outs[0], (dq_w, dk_w, dv_w, gk_w, gv_w)):
        x, w = host(x), host(w)
        check(f"{name} no-alloc vs workspace call", x, w, tol)
        check(f"{name} no-alloc vs oracle", x, ref[key], tol)
        check(f"{name} workspace call vs oracle", w, ref[key], tol)


def test_noalloc_matches_the_workspace_entry_point_twice():
    _run_case(11, 16, 4, 700, [300, 129, 0, 257])
    _run_case(12, 8, 2, 130, [64, 33])


def test_noalloc_fp32_matches_the_workspace_entry_point_twice():
    _run_case(13, 8, 2, 300, [200, 65], dtype="f32")
    _run_case(14, 4, 4, 70, [33], dtype="f32", d=64)
