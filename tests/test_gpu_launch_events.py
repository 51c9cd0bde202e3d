"""The launch-events hook (pf_set_launch_events_hook): kernels launched with
caller-owned start/stop events compute exactly what a plain launch computes,
and every event pair times one kernel inside the interval that brackets the
calls."""
import numpy as np
import pytest
import torch

from tests.gpu_util import dev
from workloads.gen import random_small_group

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import shared_prefix_attention_pf_amd as pf
    from shared_prefix_attention_pf_amd import group as G


def _phase_b(desc, g, t, p, hkv, d):
    cu = g["cu_seqlens"]
    o, lse = G.suffix_fwd(desc, t["k_p"], t["v_p"], cu, t["q_s"], t["k_s"], t["v_s"])
    gk = torch.zeros(p, hkv, d, dtype=torch.float32, device="cuda")
    gv = torch.zeros_like(gk)
    dq, dk, dv = G.suffix_bwd(desc, t["k_p"], t["v_p"], cu, t["q_s"], t["k_s"], t["v_s"], o, lse,
                              t["do_s"], gk, gv)
    return (o, lse, dq, dk, dv, gk, gv)


def test_launch_events_hook_times_each_kernel_and_changes_nothing():
    hq, hkv, d, p, lens = 8, 2, 128, 300, [1, 77, 130, 0, 64]
    print(f"\ncase hq={hq} hkv={hkv} P={p} suffixes={lens}", flush=True)
    g = random_small_group(23, hq, hkv, d, p, lens, "bf16")
    desc = pf.AttnDesc(hq, hkv, d, pf.PF_BF16)
    t = {k: dev(g[k], "bf16") for k in ("k_p", "v_p", "q_s", "k_s", "v_s", "do_s")}
    plain = _phase_b(desc, g, t, p, hkv, d)
    torch.cuda.synchronize()

    pool = [torch.cuda.Event(enable_timing=True) for _ in range(64)]
    for e in pool:
        e.record()
    torch.cuda.synchronize()
    spans = []

    def events(label, stream):
        a, b = pool.pop(), pool.pop()
        spans.append((label, a, b))
        return a.cuda_event, b.cuda_event

    outer0, outer1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    pf.pf_set_launch_events_hook(events)
    try:
        outer0.record()
        timed = _phase_b(desc, g, t, p, hkv, d)
        outer1.record()
        torch.cuda.synchronize()
    finally:
        pf.pf_set_launch_events_hook(None)

    for x, y in zip(plain, timed):
        assert torch.equal(x, y), "a kernel launched with events computed something else"
    labels = [s[0] for s in spans]
    print(f"  launches: {labels}", flush=True)
    for need in ("pf_fwd_bf16", "pf_bwd_dkv_bf16"):
        assert need in labels
    total = outer0.elapsed_time(outer1)
    times = [a.elapsed_time(b) for _, a, b in spans]
    print(f"  kernel ms {np.round(times, 4).tolist()}, bracket {total:.4f} ms", flush=True)
    assert all(x > 0 for x in times)
    assert sum(times) <= total * 1.01 + 1e-3
    # the events follow launch order on the stream
    for (_, _, b), (_, a2, _) in zip(spans, spans[1:]):
        assert b.elapsed_time(a2) >= -1e-3

    # removing the hook restores plain launches (no event is consumed)
    left = len(pool)
    _phase_b(desc, g, t, p, hkv, d)
    torch.cuda.synchronize()
    assert len(pool) == left
