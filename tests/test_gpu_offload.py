"""Dormant prefix activations offloaded to one pinned host pool between Phase A
and Phase C.  Phase C from offloaded tensors must match the fp64 oracle, and be
bitwise that of a run that keeps them in HBM (with a prefetch and with the
demand load); the device memory they held is released while Phase B runs;
one pool serves group after group with no further pinned allocation; a pool
too small keeps what does not fit on the device, with the same results."""
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
    from shared_prefix_attention_pf_amd.offload import PinnedPool

HQ, HKV, D, P, LENS = 8, 2, 128, 1024, [300, 200]


def _group(seed):
    g = random_small_group(seed, HQ, HKV, D, P, LENS, "bf16")
    t = {k: dev(g[k], "bf16") for k in ("q_p", "k_p", "v_p", "do_p", "q_s", "k_s", "v_s",
                                         "do_s")}
    return g, t


def _dormant_bytes():
    return 2 * P * HQ * D * 2 + HQ * P * 4


def _run(g, t, mode, pool=None):
    """Phase A, B, C of one group; mode: resident, prefetch or demand."""
    cu = g["cu_seqlens"]
    desc = pf.AttnDesc(HQ, HKV, D, pf.PF_BF16)
    o_p, lse_p = G.prefix_fwd(desc, t["q_p"], t["k_p"], t["v_p"])
    holder = None
    released = 0
    if mode == "resident":
        q_p = t["q_p"]
    else:
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        # right after Phase A: Q_P was read by it, O_P and LSE_P produced by it
        holder = pool.offload({"q_p": t.pop("q_p"), "o_p": o_p, "lse_p": lse_p})
        del o_p, lse_p
        torch.cuda.synchronize()
        # the allocator retires blocks freed behind a stream at its next call
        torch.empty(1, device="cuda")
        released = before - torch.cuda.memory_allocated()
    gk = torch.zeros(P, HKV, D, dtype=torch.float32, device="cuda")
    gv = torch.zeros_like(gk)
    o_s, lse_s = G.suffix_fwd(desc, t["k_p"], t["v_p"], cu, t["q_s"], t["k_s"], t["v_s"])
    dq_s, _, _ = G.suffix_bwd(desc, t["k_p"], t["v_p"], cu, t["q_s"], t["k_s"], t["v_s"], o_s,
                              lse_s, t["do_s"], gk, gv)
    if holder is not None:
        if mode == "prefetch":
            holder.prefetch()
        back = holder.get()
        q_p, o_p, lse_p = back["q_p"], back["o_p"], back["lse_p"]
        t["q_p"] = q_p
    dq_p, dk_p, dv_p = G.prefix_bwd(desc, q_p, t["k_p"], t["v_p"], o_p, lse_p, t["do_p"], gk, gv)
    torch.cuda.synchronize()
    return [x.cpu() for x in (dq_s, o_p, dq_p, dk_p, dv_p)], released


def _oracle(g):
    scale = 1.0 / math.sqrt(D)
    hmap = oracle.head_map(HQ, HKV)
    rb = oracle.suffix_attention(g["k_p"], g["v_p"], g["q_s"], g["k_s"], g["v_s"], g["do_s"],
                                 g["cu_seqlens"], scale, hmap)
    ro, _ = oracle.prefix_forward(g["q_p"], g["k_p"], g["v_p"], scale, hmap)
    rdq, rdk, rdv = oracle.prefix_backward_inject(g["q_p"], g["k_p"], g["v_p"], g["do_p"], rb["gk"],
                                                  rb["gv"], scale, hmap)
    return ro, rdq, rdk, rdv


def test_offload_matches_the_oracle_and_the_resident_run():
    g, t = _group(51)
    ref, _ = _run(g, t, "resident")
    pool = PinnedPool.for_footprint(_dormant_bytes())
    ro, rdq, rdk, rdv = _oracle(g)
    tol = TOL["bf16"]
    for mode in ("prefetch", "demand"):
        got, released = _run(g, t, mode, pool)
        print(f"\n{mode}: released {released} bytes of HBM during Phase B", flush=True)
        # Q_P and O_P (1024 x 8 x 128 bf16 each) and LSE_P (8 x 1024 fp32)
        assert released >= 2 * P * HQ * D * 2
        for a, b in zip(ref, got):
            assert torch.equal(a, b), f"{mode}: results differ from the resident run"
        _, o_p, dq_p, dk_p, dv_p = got
        check(f"{mode}: O_P (back from the pool)", host(o_p), ro, tol)
        check(f"{mode}: dQ_P", host(dq_p), rdq, tol)
        check(f"{mode}: dK_P", host(dk_p), rdk, tol)
        check(f"{mode}: dV_P", host(dv_p), rdv, tol)
    assert pool.live_bytes() == 0 and pool.resident_fallbacks == 0
    assert pool.pinned_allocations == 1


def test_one_pool_serves_group_after_group():
    """Three groups in turn through one 1.5x pool, the next group's offload
    issued before the previous group's tensors come back (two groups live at
    once would need 2x, so part of the second stays resident); every group's
    Phase C against the oracle; one pinned allocation in all."""
    pool = PinnedPool.for_footprint(_dormant_bytes())
    tol = TOL["bf16"]
    desc = pf.AttnDesc(HQ, HKV, D, pf.PF_BF16)
    groups = [_group(60 + i) for i in range(3)]
    held = []
    for i, (g, t) in enumerate(groups):
        o_p, lse_p = G.prefix_fwd(desc, t["q_p"], t["k_p"], t["v_p"])
        held.append(pool.offload({"q_p": t["q_p"], "o_p": o_p, "lse_p": lse_p}))
        del o_p, lse_p
        if i >= 1:
            # the previous group's Phase C
            gp, tp = groups[i - 1]
            back = held[i - 1].get()
            _phase_c_check(desc, gp, tp, back, tol, f"group {i - 1}")
    gp, tp = groups[-1]
    _phase_c_check(desc, gp, tp, held[-1].get(), tol, "group 2")
    print(f"\npool: {pool.capacity} bytes, {pool.bytes_offloaded} offloaded, "
          f"{pool.resident_fallbacks} tensors kept resident", flush=True)
    assert pool.pinned_allocations == 1 and pool.live_bytes() == 0
    assert pool.bytes_offloaded >= 2 * _dormant_bytes()


def _phase_c_check(desc, g, t, back, tol, name):
    cu = g["cu_seqlens"]
    gk = torch.zeros(P, HKV, D, dtype=torch.float32, device="cuda")
    gv = torch.zeros_like(gk)
    o_s, lse_s = G.suffix_fwd(desc, t["k_p"], t["v_p"], cu, t["q_s"], t["k_s"], t["v_s"])
    G.suffix_bwd(desc, t["k_p"], t["v_p"], cu, t["q_s"], t["k_s"], t["v_s"], o_s, lse_s,
                 t["do_s"], gk, gv)
    dq_p, dk_p, dv_p = G.prefix_bwd(desc, back["q_p"], t["k_p"], t["v_p"], back["o_p"],
                                    back["lse_p"], t["do_p"], gk, gv)
    torch.cuda.synchronize()
    ro, rdq, rdk, rdv = _oracle(g)
    check(f"{name}: O_P", host(back["o_p"]), ro, tol)
    check(f"{name}: dQ_P", host(dq_p), rdq, tol)
    check(f"{name}: dK_P", host(dk_p), rdk, tol)
    check(f"{name}: dV_P", host(dv_p), rdv, tol)


def test_pool_too_small_keeps_tensors_resident():
    g, t = _group(52)
    ref, _ = _run(g, t, "resident")
    pool = PinnedPool(P * HQ * 4 + 1024)        # room for LSE_P only
    got, _ = _run(g, t, "prefetch", pool)
    assert pool.resident_fallbacks == 2
    for a, b in zip(ref, got):
        assert torch.equal(a, b)
