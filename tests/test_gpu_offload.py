"""Dormant prefix activations offloaded to pinned host memory between Phase A
and Phase C: the Phase C results must be bitwise those of a run that keeps
them in HBM, with a prefetch and with the demand load; the device memory
they held is released while Phase B runs."""
import math

import numpy as np
import pytest
import torch

from tests.gpu_util import dev
from workloads.gen import random_small_group

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import shared_prefix_attention_pf_amd as pf
    from shared_prefix_attention_pf_amd import group as G
    from shared_prefix_attention_pf_amd.offload import DormantPrefix


def _run(prefetch: str):
    hq, hkv, d, p, lens = 8, 2, 128, 1024, [300, 200]
    g = random_small_group(51, hq, hkv, d, p, lens, "bf16")
    cu = g["cu_seqlens"]
    desc = pf.AttnDesc(hq, hkv, d, pf.PF_BF16)
    t = {k: dev(g[k], "bf16") for k in ("q_p", "k_p", "v_p", "do_p", "q_s", "k_s", "v_s",
                                         "do_s")}
    o_p, lse_p = G.prefix_fwd(desc, t["q_p"], t["k_p"], t["v_p"])
    holder = None
    released = 0
    if prefetch != "resident":
        q_p = t.pop("q_p")
        holder = DormantPrefix({"q_p": q_p, "o_p": o_p, "lse_p": lse_p})
        del q_p, o_p, lse_p
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        holder.offload()
        torch.cuda.synchronize()
        # the allocator retires blocks freed behind a stream at its next call
        torch.empty(1, device="cuda")
        released = before - torch.cuda.memory_allocated()
    gk = torch.zeros(p, hkv, d, dtype=torch.float32, device="cuda")
    gv = torch.zeros_like(gk)
    o_s, lse_s = G.suffix_fwd(desc, t["k_p"], t["v_p"], cu, t["q_s"], t["k_s"], t["v_s"])
    dq_s, _, _ = G.suffix_bwd(desc, t["k_p"], t["v_p"], cu, t["q_s"], t["k_s"], t["v_s"], o_s,
                              lse_s, t["do_s"], gk, gv)
    if holder is not None:
        if prefetch == "prefetch":
            holder.prefetch()
        back = holder.get()
        q_p, o_p, lse_p = back["q_p"], back["o_p"], back["lse_p"]
    else:
        q_p = t["q_p"]
    dq_p, dk_p, dv_p = G.prefix_bwd(desc, q_p, t["k_p"], t["v_p"], o_p, lse_p, t["do_p"], gk, gv)
    torch.cuda.synchronize()
    return [x.cpu() for x in (dq_s, dq_p, dk_p, dv_p)], released


def test_offload_is_bitwise_transparent():
    ref, _ = _run("resident")
    for mode in ("prefetch", "demand"):
        got, released = _run(mode)
        print(f"\n{mode}: released {released} bytes of HBM during Phase B", flush=True)
        # Q_P and O_P (1024 x 8 x 128 bf16 each) and LSE_P (8 x 1024 fp32)
        assert released >= 2 * 1024 * 8 * 128 * 2
        for a, b in zip(ref, got):
            assert torch.equal(a, b), f"{mode}: results differ from the resident run"
