#!/usr/bin/env python3
"""Benchmark of the group attention hot path on one MI355X.

One step = the whole path over one synthetic group: zero the fp32 gK/gV
accumulators, Phase A (prefix causal forward), Phase B (suffix forward and
backward over the cached prefix, accumulating gK/gV; one call per
microbatch) and Phase C (prefix backward with gK/gV injected).  For the tree
workload a step is the tree forward and backward.

Printed JSON (one line): `value` is the Phase-B forward+backward throughput
in algorithmic TFLOP/s (12 * head_dim FLOPs per visible (query, key) pair
per query head: 4 forward, 8 backward; the backward's recompute of the
scores is not counted), with inputs resident in HBM.  The timed steps record
HIP events at the phase boundaries only.  `roofline` is for the kernel with
the largest share of the step; its launch time comes from a separate pass
over the same steps that records HIP events on the kernel's own stream
around every launch (issued behind a queue of untimed steps, so the host's
event bookkeeping never leaves the GPU idle).  `cpu_baseline` is the CPU
oracle (fp32 numpy): dense attention over whole trajectories, timed on a
bounded sample of the same workload.
"""
import argparse
import gc
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3        # MI355X dense fp32 MFMA
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=2,
                    help="workload (1..9; 6 is tree windows over a cached prefix, 7 compact "
                         "log-probabilities, 8 windows under a producer tree's nodes, 9 the "
                         "headline group in fp32); 2 is the headline")
    ap.add_argument("--separate-windows", action="store_true",
                    help="config 6: one call per window instead of the four trees in one call")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample (0 disables)")
    ap.add_argument("--json-out", default=None)
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the timed steps, run a plain elementwise copy of this many MiB "
                         "(3 launches); its HBM counter readings scale the attention kernels' ones")
    ap.add_argument("--traffic-summary", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "OUT_MD"),
                    default=None,
                    help="no GPU work: turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of "
                         "this script into the traffic summary that later runs report")
    ap.add_argument("--stats-summary", nargs=2, metavar=("STATS_CSV", "OUT_MD"), default=None,
                    help="no GPU work: turn a rocprofv3 --kernel-trace --stats csv of this script "
                         "into a kernel-time summary")
    ap.add_argument("--offload", action="store_true",
                    help="flat configs: measure the dormant-prefix offload instead (Q_P, O_P, "
                         "LSE_P to pinned host memory during Phase B, prefetched before Phase C)")
    ap.add_argument("--counter-summary", nargs="+", metavar="RUN_DIR_OR_OUT_MD", default=None,
                    help="no GPU work: turn rocprofv3 --pmc runs of SQ_ counters (their output "
                         "directories, then the output file) into a per-kernel counter summary")
    ap.add_argument("--pmc-command", default="",
                    help="with --traffic-summary / --stats-summary: the profiling commands, "
                         "recorded in the summary")
    return ap.parse_args()


# ---------------------------------------------------------------- work counts

def flat_pairs(p, lens):
    """Visible (query, key) pairs per query head of Phase B and of Phase A/C."""
    lens = np.asarray(lens, dtype=np.int64)
    return int(np.sum(lens * p + lens * (lens + 1) // 2)), p * (p + 1) // 2


def tree_pairs(node_off, parent):
    n = len(parent)
    depth_rows = np.zeros(n, dtype=np.int64)   # rows of strict ancestors
    for v in range(1, n):
        u = parent[v]
        depth_rows[v] = depth_rows[u] + (node_off[u + 1] - node_off[u])
    total = 0
    for v in range(n):
        ln = int(node_off[v + 1] - node_off[v])
        total += ln * int(depth_rows[v]) + ln * (ln + 1) // 2
    return total


def ranges_window_pairs(w):
    """Visible pairs per query head of a window under a producer node: every
    row sees every cached row of its ranges, plus its tree pairs."""
    return int(w["node_off"][-1]) * sum(n for _, n in w["ranges"]) + tree_pairs(w["node_off"],
                                                                                 w["parent"])


def window_pairs(p, node_off, parent):
    """Visible pairs per query head of a tree window over a P-row prefix: every
    row sees the whole prefix, plus its tree pairs."""
    return int(node_off[-1]) * p + tree_pairs(node_off, parent)


# ---------------------------------------------------------------- GPU side

class KernelTimer:
    """Launch-hook consumer: HIP events around every kernel, on its own stream.

    Within one phase the step enqueues nothing but library calls, so the event
    that ends one kernel also starts the next one on the same stream: one event
    per launch boundary instead of two.  A kernel's time then includes the
    launch gap before it, which errs on the long side.  Setting `phase` starts
    fresh events, since the step records its own phase events in between.
    `reserve` events are created (and recorded once) up front, so the timed
    region only re-records existing events."""

    def __init__(self, torch, reserve=0, streams=()):
        self.torch = torch
        self.open = {}
        self.spans = []          # (label, phase, start_event, end_event)
        # streams the library is called on, wrapped before any launch so the
        # hook creates no stream objects while kernels are being enqueued
        self.streams = {s.cuda_stream: s for s in streams}
        self.last_end = {}       # stream -> end event of the previous kernel, this phase
        self._phase = None
        self.reserve = reserve
        self.pool = []
        self.refill()

    def refill(self):
        """Drops recorded spans and makes `reserve` events ready for reuse."""
        torch = self.torch
        self.open, self.spans, self.last_end = {}, [], {}
        self.pool = [torch.cuda.Event(enable_timing=True) for _ in range(self.reserve)]
        for e in self.pool:
            e.record()
        if self.reserve:
            torch.cuda.synchronize()

    @property
    def phase(self):
        return self._phase

    @phase.setter
    def phase(self, name):
        # set by the step before each phase's calls
        self._phase = name
        self.last_end = {}

    def _record(self, s):
        ev = self.pool.pop() if self.pool else self.torch.cuda.Event(enable_timing=True)
        ev.record(s)
        return ev

    def __call__(self, label, stream, end):
        torch = self.torch
        if stream not in self.streams:
            self.streams[stream] = torch.cuda.ExternalStream(stream) if stream else \
                torch.cuda.default_stream()
        s = self.streams[stream]
        if end == 0:
            ev = self.last_end.pop(stream, None)
            self.open[(label, stream)] = ev if ev is not None else self._record(s)
        else:
            ev = self._record(s)
            self.spans.append((label, self.phase, self.open.pop((label, stream)), ev))
            self.last_end[stream] = ev

    def summary(self):
        out = {}
        for label, phase, a, b in self.spans:
            ms = a.elapsed_time(b)
            t = out.setdefault(label, {"launches": 0, "total_ms": 0.0, "phases": {}})
            t["launches"] += 1
            t["total_ms"] += ms
            t["phases"][phase] = t["phases"].get(phase, 0) + 1
            t.setdefault("phase_total_ms", {})
            t["phase_total_ms"][phase] = t["phase_total_ms"].get(phase, 0.0) + ms
        for t in out.values():
            t["avg_ms"] = t["total_ms"] / t["launches"]
            # average launch time within each phase the kernel runs in
            t["phase_avg_ms"] = {p: round(t["phase_total_ms"].pop(p) / n, 4)
                                 for p, n in t["phases"].items()}
            del t["phase_total_ms"]
        return out


def run_gpu(cfg, data, steps, warmup, copy_mib=0, separate_windows=False):
    import torch

    import shared_prefix_attention_pf_amd as pf

    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    pdt = pf.PF_BF16 if cfg.dtype == "bf16" else pf.PF_F32
    desc = pf.AttnDesc(cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, pdt)

    def to_dev(x):
        return torch.from_numpy(np.ascontiguousarray(x)).to(tdt).to(dev)

    stream = torch.cuda.current_stream()
    res = {}
    timer = KernelTimer(torch, reserve=64 * (min(steps, 10) + 1), streams=(stream,))
    if cfg.is_ranges:
        # producer tree forward, the windows under its nodes, producer backward
        node_off, parent = data["node_off"], data["parent"]
        q_c, k_c, v_c, do_c = (to_dev(data[n]) for n in ("q", "k", "v", "do"))
        c = q_c.shape[0]
        o_c = torch.empty_like(q_c)
        lse_c = torch.empty(cfg.num_q_heads, c, device=dev)
        dq_c, dk_c, dv_c = torch.empty_like(q_c), torch.empty_like(k_c), torch.empty_like(v_c)
        gk = torch.empty(c, cfg.num_kv_heads, cfg.head_dim, device=dev)
        gv = torch.empty_like(gk)
        wins = []
        for wd in data["windows"]:
            w = {n: to_dev(wd[n]) for n in ("q", "k", "v", "do")}
            rw = w["q"].shape[0]
            w.update(node_off=wd["node_off"], parent=wd["parent"],
                     starts=[s for s, _ in wd["ranges"]], lens=[n for _, n in wd["ranges"]],
                     o=torch.empty_like(w["q"]), lse=torch.empty(cfg.num_q_heads, rw, device=dev),
                     dq=torch.empty_like(w["q"]), dk=torch.empty_like(w["k"]),
                     dv=torch.empty_like(w["v"]))
            wins.append(w)
        ws_bytes = max(pf.pf_workspace_size(op, desc, pf.pf_ranges_cached_keys(w["lens"]),
                                            int(w["node_off"][-1]))
                       for w in wins for op in (pf.PF_OP_TREE_SUFFIX_FWD, pf.PF_OP_TREE_SUFFIX_BWD))
        ws_bytes = max(ws_bytes, pf.pf_workspace_size(pf.PF_OP_TREE_BWD, desc, 0, c),
                       pf.pf_workspace_size(pf.PF_OP_TREE_FWD, desc, 0, c))
        ws = torch.empty(max(16, ws_bytes), dtype=torch.uint8, device=dev)

        def step(ev=None):
            gk.zero_()
            gv.zero_()
            timer.phase = "A"
            if ev:
                ev[0].record(stream)
            pf.pf_tree_attn_fwd(desc, node_off, parent, q_c, k_c, v_c, o_c, lse_c, ws)
            if ev:
                ev[1].record(stream)
            timer.phase = "B"
            for w in wins:
                pf.pf_tree_suffix_attn_fwd_ranges(desc, k_c, v_c, w["starts"], w["lens"],
                                                  w["node_off"], w["parent"], w["q"], w["k"],
                                                  w["v"], w["o"], w["lse"], ws)
                pf.pf_tree_suffix_attn_bwd_accum_ranges(
                    desc, k_c, v_c, w["starts"], w["lens"], w["node_off"], w["parent"], w["q"],
                    w["k"], w["v"], w["o"], w["lse"], w["do"], w["dq"], w["dk"], w["dv"], gk, gv,
                    ws)
            timer.phase = "C"
            if ev:
                ev[2].record(stream)
            pf.pf_tree_attn_bwd_inject(desc, node_off, parent, q_c, k_c, v_c, o_c, lse_c, do_c, gk,
                                       gv, dq_c, dk_c, dv_c, pdt, ws)
            if ev:
                ev[3].record(stream)
        phase_names = ("A", "B", "C")
    elif cfg.is_windows:
        p = cfg.prefix_len
        q_p, k_p, v_p, do_p = (to_dev(data[n]) for n in ("q_p", "k_p", "v_p", "do_p"))
        o_p = torch.empty_like(q_p)
        lse_p = torch.empty(cfg.num_q_heads, p, device=dev)
        dq_p, dk_p, dv_p = torch.empty_like(q_p), torch.empty_like(k_p), torch.empty_like(v_p)
        gk = torch.empty(p, cfg.num_kv_heads, cfg.head_dim, device=dev)
        gv = torch.empty_like(gk)
        wins = []
        for wd in data["windows"]:
            w = {n: to_dev(wd[n]) for n in ("q", "k", "v", "do")}
            c = w["q"].shape[0]
            w.update(node_off=wd["node_off"], parent=wd["parent"], o=torch.empty_like(w["q"]),
                     lse=torch.empty(cfg.num_q_heads, c, device=dev), dq=torch.empty_like(w["q"]),
                     dk=torch.empty_like(w["k"]), dv=torch.empty_like(w["v"]))
            wins.append(w)
        if not separate_windows and cfg.window_calls == 1 and len(wins) > 1:
            # every window's tree in one call: a forest over the prefix
            from workloads.gen import forest
            no, pa = forest([(w["node_off"], w["parent"]) for w in wins])
            one = {n: torch.cat([w[n] for w in wins]) for n in ("q", "k", "v", "do", "o", "dq",
                                                                 "dk", "dv")}
            one.update(node_off=no, parent=pa,
                       lse=torch.empty(cfg.num_q_heads, int(no[-1]), device=dev))
            wins = [one]
        max_c = max(int(w["node_off"][-1]) for w in wins)
        ws_bytes = max(pf.pf_workspace_size(op, desc, p, max_c) for op in
                       (pf.PF_OP_TREE_SUFFIX_FWD, pf.PF_OP_TREE_SUFFIX_BWD))
        ws_bytes = max(ws_bytes, pf.pf_workspace_size(pf.PF_OP_PREFIX_BWD, desc, p, p))
        ws = torch.empty(max(16, ws_bytes), dtype=torch.uint8, device=dev)

        def step(ev=None):
            gk.zero_()
            gv.zero_()
            timer.phase = "A"
            if ev:
                ev[0].record(stream)
            pf.pf_prefix_fwd(desc, p, q_p, k_p, v_p, o_p, lse_p, ws)
            if ev:
                ev[1].record(stream)
            timer.phase = "B"
            for w in wins:
                pf.pf_tree_suffix_attn_fwd(desc, p, k_p, v_p, w["node_off"], w["parent"], w["q"],
                                           w["k"], w["v"], w["o"], w["lse"], ws)
                pf.pf_tree_suffix_attn_bwd_accum(desc, p, k_p, v_p, w["node_off"], w["parent"],
                                                 w["q"], w["k"], w["v"], w["o"], w["lse"],
                                                 w["do"], w["dq"], w["dk"], w["dv"], gk, gv, ws)
            timer.phase = "C"
            if ev:
                ev[2].record(stream)
            pf.pf_prefix_bwd_inject(desc, p, q_p, k_p, v_p, o_p, lse_p, do_p, gk, gv, dq_p, dk_p,
                                    dv_p, pdt, ws)
            if ev:
                ev[3].record(stream)
        phase_names = ("A", "B", "C")
    elif cfg.is_tree:
        node_off, parent = data["node_off"], data["parent"]
        q, k, v, do = (to_dev(data[n]) for n in ("q", "k", "v", "do"))
        c = q.shape[0]
        o = torch.empty_like(q)
        lse = torch.empty(cfg.num_q_heads, c, device=dev)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws_f = torch.empty(max(16, pf.pf_workspace_size(pf.PF_OP_TREE_FWD, desc, 0, c)),
                           dtype=torch.uint8, device=dev)
        ws_b = torch.empty(max(16, pf.pf_workspace_size(pf.PF_OP_TREE_BWD, desc, 0, c)),
                           dtype=torch.uint8, device=dev)

        def step(ev=None):
            timer.phase = "tree"
            if ev:
                ev[0].record(stream)
            pf.pf_tree_attn_fwd(desc, node_off, parent, q, k, v, o, lse, ws_f)
            pf.pf_tree_attn_bwd(desc, node_off, parent, q, k, v, o, lse, do, dq, dk, dv, ws_b)
            if ev:
                ev[1].record(stream)
                ev[2].record(stream)
                ev[3].record(stream)
        phase_names = ("tree",)
    else:
        p = cfg.prefix_len
        cu = data["cu_seqlens"]
        q_p, k_p, v_p, do_p = (to_dev(data[n]) for n in ("q_p", "k_p", "v_p", "do_p"))
        q_s, k_s, v_s, do_s = (to_dev(data[n]) for n in ("q_s", "k_s", "v_s", "do_s"))
        t_rows = q_s.shape[0]
        o_p = torch.empty_like(q_p)
        lse_p = torch.empty(cfg.num_q_heads, p, device=dev)
        o_s = torch.empty_like(q_s)
        lse_s = torch.empty(cfg.num_q_heads, t_rows, device=dev)
        dq_s, dk_s, dv_s = torch.empty_like(q_s), torch.empty_like(k_s), torch.empty_like(v_s)
        dq_p, dk_p, dv_p = torch.empty_like(q_p), torch.empty_like(k_p), torch.empty_like(v_p)
        gk = torch.empty(p, cfg.num_kv_heads, cfg.head_dim, device=dev)
        gv = torch.empty_like(gk)
        mbs = []
        for a, b in data["microbatches"]:
            r0, r1 = int(cu[a]), int(cu[b])
            sub_cu = (cu[a:b + 1] - cu[a]).astype(np.int32)
            sl = slice(r0, r1)
            mbs.append(dict(cu=sub_cu, q=q_s[sl], k=k_s[sl], v=v_s[sl], do=do_s[sl], o=o_s[sl],
                            lse=lse_s[:, sl], dq=dq_s[sl], dk=dk_s[sl], dv=dv_s[sl]))
        max_rows = max(int(m["cu"][-1]) for m in mbs)
        ws_bytes = max(pf.pf_workspace_size(op, desc, p, max_rows) for op in
                       (pf.PF_OP_SUFFIX_FWD, pf.PF_OP_SUFFIX_BWD))
        ws_bytes = max(ws_bytes, pf.pf_workspace_size(pf.PF_OP_PREFIX_BWD, desc, p, p))
        ws = torch.empty(max(16, ws_bytes), dtype=torch.uint8, device=dev)
        # LSE slices of a [Hq, rows] array are not contiguous: give each
        # microbatch its own contiguous LSE buffer
        for m in mbs:
            m["lse"] = torch.empty(cfg.num_q_heads, int(m["cu"][-1]), device=dev)

        def step(ev=None):
            gk.zero_()
            gv.zero_()
            timer.phase = "A"
            if ev:
                ev[0].record(stream)
            pf.pf_prefix_fwd(desc, p, q_p, k_p, v_p, o_p, lse_p, ws)
            if ev:
                ev[1].record(stream)
            timer.phase = "B"
            for m in mbs:
                pf.pf_suffix_attn_fwd(desc, p, k_p, v_p, m["cu"], m["q"], m["k"], m["v"], m["o"],
                                      m["lse"], ws)
                pf.pf_suffix_attn_bwd_accum(desc, p, k_p, v_p, m["cu"], m["q"], m["k"], m["v"],
                                            m["o"], m["lse"], m["do"], m["dq"], m["dk"], m["dv"],
                                            gk, gv, ws)
            timer.phase = "C"
            if ev:
                ev[2].record(stream)
            pf.pf_prefix_bwd_inject(desc, p, q_p, k_p, v_p, o_p, lse_p, do_p, gk, gv, dq_p, dk_p,
                                    dv_p, pdt, ws)
            if ev:
                ev[3].record(stream)
        phase_names = ("A", "B", "C")

    def phases_of(evs):
        n = len(evs)
        if cfg.is_tree:
            return {"tree": sum(e[0].elapsed_time(e[1]) for e in evs) / n}
        return {"A": sum(e[0].elapsed_time(e[1]) for e in evs) / n,
                "B": sum(e[1].elapsed_time(e[2]) for e in evs) / n,
                "C": sum(e[2].elapsed_time(e[3]) for e in evs) / n}

    # timed region: K steps with HIP events at the phase boundaries only (no
    # per-kernel events: an event record between two kernels adds its own
    # cost, and host-side bookkeeping per launch can leave the GPU idle)
    # (the collection and the event creation come before the warm-up, so the
    # GPU goes from the warm-up steps to the timed ones without an idle gap)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    gc.collect()
    gc.disable()
    try:
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            step(evs[i])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    finally:
        gc.enable()
    phase_ms = phases_of(evs)
    res["wall_ms_per_step"] = wall * 1e3 / steps
    res["phase_ms"] = phase_ms
    # the headline phase step by step: its median and fastest step
    key = (0, 1) if cfg.is_tree else (1, 2)
    in_order = [e[key[0]].elapsed_time(e[key[1]]) for e in evs]
    per_step = sorted(in_order)
    res["headline_phase_ms_median"] = float(np.median(per_step))
    res["headline_phase_ms_min"] = per_step[0]
    res["headline_phase_ms_steps"] = [round(x, 4) for x in in_order]
    res["steps_total_ms"] = evs[0][0].elapsed_time(evs[-1][3])
    res["kernels"], res["kernel_pass"] = kernel_pass(torch, pf, timer, step, phases_of, phase_ms,
                                                     min(steps, 10))
    if copy_mib > 0:
        copy_probe(torch, copy_mib)
    res["device"] = torch.cuda.get_device_name(0)
    res["cus"] = torch.cuda.get_device_properties(0).multi_processor_count
    return res


def kernel_pass(torch, pf, timer, step, phases_of, timed_phase_ms, n_steps, lead=3, tries=2):
    """Per-kernel launch times, from steps run after the timed region with the
    launch hook recording HIP events around every kernel.  `lead` untimed steps
    are queued first, so the GPU has several milliseconds of work ahead of the
    host while the hook's bookkeeping runs.  The pass is repeated once if its
    Phase-B (or tree) time is more than 5 % above the timed region's, and the
    pass closer to the timed region is kept; both are reported."""
    key = "tree" if "tree" in timed_phase_ms else "B"
    best = None
    passes = []
    for _ in range(tries):
        timer.refill()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n_steps)]
        torch.cuda.synchronize()
        gc.collect()
        gc.disable()
        try:
            for _ in range(lead):
                step()
            pf.pf_set_launch_hook(timer)
            try:
                for i in range(n_steps):
                    step(evs[i])
            finally:
                pf.pf_set_launch_hook(None)
            torch.cuda.synchronize()
        finally:
            gc.enable()
        ph = phases_of(evs)
        summ = timer.summary()
        passes.append({k: round(v, 4) for k, v in ph.items()})
        if best is None or ph[key] < best[0][key]:
            best = (ph, summ)
        if ph[key] <= 1.05 * timed_phase_ms[key]:
            break
    info = {"steps": n_steps, "lead_steps": lead, "passes_phase_ms": passes,
            "kept_phase_ms": {k: round(v, 4) for k, v in best[0].items()}}
    return best[1], info


# ---------------------------------------------------------------- HBM traffic from counters

# launch-hook label -> substring of the kernel symbol in rocprofv3 output
KERNEL_SYMBOL = {"pf_fwd_bf16": "fwd_kernel", "pf_bwd_dq_bf16": "bwd_dq_kernel",
                 "pf_bwd_dq_ds_bf16": "bwd_dq_ds_kernel", "pf_bwd_dkv_bf16": "bwd_dkv_kernel",
                 "pf_fwd_f32": "fwd_f32_kernel", "pf_bwd_dq_f32": "dq_f32_kernel",
                 "pf_bwd_dkv_f32": "dkv_f32_kernel", "pf_bwd_dq_ds_f32": "dq_ds_f32_kernel",
                 "pf_prep_dsum": "prep_dsum_kernel",
                 "pf_partials": "partial_sums_kernel", "pf_logprob_fwd": "logprob_fwd_kernel",
                 "pf_logprob_bwd": "logprob_bwd_kernel"}
COPY_SYMBOL = "neg_kernel"       # the elementwise copy run by --copy-probe-mib


# Each kernel family's own source file; the rest of csrc/ (launch code, shared
# headers, the prep kernels) is common to every family.
FAMILY_SOURCES = {"bf16": "pf_attn_bf16.hip", "f32": "pf_attn_f32.hip",
                  "logprob": "pf_logprob.hip"}


def config_family(cid):
    from workloads import get_config
    cfg = get_config(cid)
    return "logprob" if cfg.is_logprob else cfg.dtype


def kernel_source_hash(family):
    """sha256 over the sources a kernel family's launches depend on (its own
    file and the common ones): a stored traffic figure only applies to the
    kernels it was measured on."""
    import hashlib
    others = {f for fam, f in FAMILY_SOURCES.items() if fam != family}
    h = hashlib.sha256()
    cdir = os.path.join(ROOT, "shared_prefix_attention_pf_amd", "csrc")
    for name in sorted(os.listdir(cdir)):
        if name.endswith((".hip", ".cpp", ".h")) and name not in others:
            with open(os.path.join(cdir, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def source_hash_line(cid):
    fam = config_family(cid)
    return f"kernel sources sha256 ({fam} family): `{kernel_source_hash(fam)}`"


def traffic_path(cid):
    return os.path.join(ROOT, "profiles", f"hbm_traffic_config{cid}.md")


def copy_probe(torch, mib):
    """A plain elementwise copy (dst = -src) of `mib` MiB of fp32, launched 3
    times: reads exactly mib MiB and writes mib MiB per launch."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def plain_name(name):
    """A kernel name as the profiler printed it, with the identifiers of a
    symbol it could not demangle (a template over __bf16 stays mangled) joined
    by '::', so that names like prep_dsum_kernel can be found in it."""
    import re
    if not name.startswith("_Z"):
        return name
    parts = []
    for m in re.finditer(r"\d+", name):
        ident = name[m.end():m.end() + int(m.group(0))]
        if len(ident) == int(m.group(0)) and re.fullmatch(r"[A-Za-z_]\w*", ident):
            parts.append(ident)
    return "::".join(parts) if parts else name


def _counter_means(run_dir, counter):
    """{kernel symbol: mean of `counter` per dispatch} from a rocprofv3 csv run."""
    import csv
    import glob
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {run_dir}")
    per = {}
    for fn in files:
        with open(fn) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                key = (fn, r["Dispatch_Id"])
                kname = plain_name(r["Kernel_Name"])
                per.setdefault(kname, {}).setdefault(key, 0.0)
                per[kname][key] += float(r["Counter_Value"])
    return {k: (sum(v.values()) / len(v), len(v)) for k, v in per.items()}


def _pick(means, sub, whole=False):
    """Mean counter value per dispatch over the kernels whose name contains
    `sub` (as a whole identifier when `whole`: fwd_kernel must not match
    logprob_fwd_kernel)."""
    import re
    pat = re.compile(r"(?<![A-Za-z0-9_])" + re.escape(sub) + r"(?![A-Za-z0-9_])")
    hits = [(k, v) for k, v in means.items() if (pat.search(k) if whole else sub in k)]
    if not hits:
        return None
    tot = sum(v[0] * v[1] for _, v in hits)
    n = sum(v[1] for _, v in hits)
    return tot / n, n


def traffic_summary(fetch_dir, write_dir, out_md, cid, copy_mib, command):
    """Writes the per-launch HBM read/write bytes of every attention kernel,
    each counter scaled by the ratio of known to counted bytes of the copy."""
    fetch = _counter_means(fetch_dir, "FETCH_SIZE")
    write = _counter_means(write_dir, "WRITE_SIZE")
    known_kib = copy_mib * 1024.0
    cf, cw = _pick(fetch, COPY_SYMBOL), _pick(write, COPY_SYMBOL)
    if cf is None or cw is None:
        raise SystemExit("the copy probe's dispatches are missing from the counter runs")
    f_fac, w_fac = known_kib / cf[0], known_kib / cw[0]
    lines = [f"# HBM traffic per launch, config {cid} (rocprofv3 FETCH_SIZE / WRITE_SIZE)", "",
             "Commands (run from the repository root on one MI355X):", "", "```", command.strip(),
             "```", "",
             f"Copy probe: `dst = -src` over {copy_mib} MiB of fp32 (reads and writes exactly "
             f"{copy_mib} MiB per launch).", "",
             f"- copy FETCH_SIZE {cf[0]:.1f} KiB per launch -> fetch scale {f_fac:.4f}",
             f"- copy WRITE_SIZE {cw[0]:.1f} KiB per launch -> write scale {w_fac:.4f}", "",
             "| label | kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | "
             "read bytes (scaled) | write bytes (scaled) |", "|---|---|---|---|---|---|---|"]
    for label, sym in KERNEL_SYMBOL.items():
        fk, wk = _pick(fetch, sym, whole=True), _pick(write, sym, whole=True)
        if fk is None or wk is None:
            continue
        rb, wb = fk[0] * 1024 * f_fac, wk[0] * 1024 * w_fac
        lines.append(f"| {label} | {sym} | {fk[1]} | {fk[0]:.1f} | {wk[0]:.1f} | {rb:.6g} | {wb:.6g} |")
    lines += ["", source_hash_line(cid), ""]
    with open(out_md, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


def stats_summary(stats_csv, out_md, cid, command):
    """Kernel-time table from rocprofv3's kernel_stats.csv."""
    import csv
    rows = list(csv.DictReader(open(stats_csv)))
    lines = [f"# Kernel times, config {cid} (rocprofv3 --kernel-trace --stats)", "",
             "Command (run from the repository root on one MI355X):", "", "```", command.strip(),
             "```", "", "| kernel | calls | total (us) | average (us) | min (us) | max (us) | share |",
             "|---|---|---|---|---|---|---|"]
    for r in rows:
        name = plain_name(r["Name"])
        m = re.search(r"\w*kernel\w*(<\d+>)?", name)
        short = m.group(0) if m else name[:60]
        fn = re.search(r"\w+Functor", name)
        if fn:
            short += f" ({fn.group(0)})"
        lines.append(f"| {short} | {r['Calls']} | {float(r['TotalDurationNs']) / 1e3:.1f} | "
                     f"{float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                     f"{float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f}% |")
    # a kernel built in several template forms (one per call kind) is one
    # launch label to bench.py's per-kernel pass: its combined average
    forms = {}
    for r in rows:
        m = re.search(r"(\w*kernel\w*)<\d+>", plain_name(r["Name"]))
        if m:
            f = forms.setdefault(m.group(1), [0, 0.0])
            f[0] += int(r["Calls"])
            f[1] += float(r["TotalDurationNs"])
    comb = [f"- {k} (all forms): {n} calls, average {t / n / 1e3:.1f} us" for k, (n, t) in
            sorted(forms.items()) if n]
    if comb:
        lines += ["", "Combined over template forms (what bench.py's per-kernel pass averages):",
                  ""] + comb
    lines += ["", source_hash_line(cid), ""]
    with open(out_md, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


# phases a single-call group step launches each kernel in (full workspace)
# the phases a flat group's step launches each kernel in, in launch order
PHASES_OF = {"fwd_kernel": ("A", "B"), "bwd_dkv_kernel": ("B", "C"),
             "bwd_dq_ds_kernel": ("B", "C"), "prep_dsum_kernel": ("B", "C"),
             "partial_sums_kernel": ("B", "C"), "fwd_f32_kernel": ("A", "B"),
             "dkv_f32_kernel": ("B", "C"), "dq_ds_f32_kernel": ("B", "C")}


def counter_summary(run_dirs, out_md, cid, command):
    """Per-kernel SQ counter table (last dispatch of each kernel and phase) from
    rocprofv3 --pmc runs of one bench step, with the derived shares of the
    shader clock: MFMA busy, and per wave the time issuing or waiting."""
    import csv
    import glob
    per = {}        # (kernel, k-th dispatch of it) -> {counter: value}
    for d in run_dirs:
        for fn in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            disp = {}
            for r in csv.DictReader(open(fn)):
                m = re.search(r"(\w+_kernel)", plain_name(r["Kernel_Name"]))
                if not m or m.group(1) not in KERNEL_SYMBOL.values():
                    continue
                did = int(r["Dispatch_Id"])
                disp.setdefault(did, [m.group(1), {}])
                c = disp[did][1]
                c[r["Counter_Name"]] = c.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            seen = {}
            for did in sorted(disp):
                k, c = disp[did]
                seen.setdefault(k, []).append(c)
            for k, lst in seen.items():
                # one step of a single-call group launches each kernel once in
                # each phase that uses it, in phase order; keep the last step's
                phases = PHASES_OF.get(k, ("B",))
                for ph, c in zip(phases, lst[-len(phases):]):
                    per.setdefault((k, ph), {}).update(c)
    names = ["SQ_CYCLES", "SQ_BUSY_CU_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_MFMA",
             "SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_WAVE_CYCLES", "SQ_WAIT_ANY",
             "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY", "SQ_VALU_MFMA_COEXEC_CYCLES"]
    lines = [f"# SQ counters per kernel, config {cid} (rocprofv3 --pmc)", "",
             "Commands (run from the repository root on one MI355X):", "", "```", command.strip(),
             "```", "",
             "Raw counters are summed over the chip. Derived: clock = SQ_CYCLES / 32 shader "
             "engines / kernel time; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs / "
             "(SQ_CYCLES / 32); wave shares = SQ_ACTIVE_INST_ANY, SQ_WAIT_ANY (at an "
             "s_waitcnt) and SQ_WAIT_INST_ANY (instruction not yet issuable) over "
             "SQ_WAVE_CYCLES.", "",
             "| kernel (phase) | " + " | ".join(names) +
             " | VALU / MFMA | MFMA busy | issuing | at s_waitcnt | waiting to issue |",
             "|---" * (len(names) + 6) + "|"]
    for (k, ph), c in sorted(per.items()):
        vals = [c.get(n) for n in names]
        cyc = c.get("SQ_CYCLES")
        mf = c.get("SQ_VALU_MFMA_BUSY_CYCLES")
        wc = c.get("SQ_WAVE_CYCLES")

        def share(x):
            return f"{100 * x / wc:.0f}%" if x is not None and wc else "-"
        busy = f"{100 * mf / 1024 / (cyc / 32):.0f}%" if mf is not None and cyc else "-"
        vpm = (f"{(c['SQ_INSTS_VALU'] - c['SQ_INSTS_MFMA']) / c['SQ_INSTS_MFMA']:.2f}"
               if c.get("SQ_INSTS_MFMA") and c.get("SQ_INSTS_VALU") is not None else "-")
        lines.append(f"| {k} ({ph}) | " + " | ".join("-" if v is None else f"{v:.4g}" for v in vals)
                     + f" | {vpm} | {busy} | {share(c.get('SQ_ACTIVE_INST_ANY'))} | "
                     f"{share(c.get('SQ_WAIT_ANY'))} | {share(c.get('SQ_WAIT_INST_ANY'))} |")
    lines += ["", source_hash_line(cid), ""]
    with open(out_md, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


def load_traffic(cid, label):
    """HBM bytes per launch of `label` from the stored counter summary, or None
    when there is none or the kernel sources changed since it was taken."""
    path = traffic_path(cid)
    if not os.path.exists(path):
        return None, "no counter summary"
    text = open(path).read()
    if source_hash_line(cid) not in text:
        return None, "kernel sources changed since the counters were taken"
    for ln in text.splitlines():
        cells = [c.strip() for c in ln.strip().strip("|").split("|")]
        if len(cells) == 7 and cells[0] == label:
            return float(cells[5]) + float(cells[6]), os.path.relpath(path, ROOT)
    return None, f"{label} missing from the counter summary"


# ---------------------------------------------------------------- CPU oracle baseline

def cpu_baseline(cfg, data, target_s, group_flops, compact, expanded):
    """The oracle as it stands (fp32 numpy, every core BLAS gets) on the dense
    baseline the method replaces: every trajectory [P || S_i] of a flat group,
    and every root-to-leaf trajectory of a tree, trained as an independent
    causal sequence (forward and backward over its whole L x L score matrix;
    `suffix_attention_full_rows`, `tree_attention_expanded`).  That yields the
    group's Phase A, B and C results.  Tree windows use the oracle's
    per-window dense attention over [prefix ; window rows].

    Timed on whole KV-head groups until about target_s seconds; heads are
    independent, so the whole group's time is the sample's scaled by
    Hkv / groups done (exact in work).  `value` is the group's algorithmic
    TFLOP (Phases A + B + C, or the tree) per second of oracle time."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        pools = threadpool_info()
        threads = max((p.get("num_threads", 1) for p in pools), default=1)
        blas = ",".join(sorted({p.get("internal_api", "?") for p in pools}))
    except Exception:
        threads, blas = os.cpu_count(), "unknown"
    g = cfg.group_size
    d = cfg.head_dim
    scale = 1.0 / math.sqrt(d)
    hmap = np.zeros(g, dtype=np.int64)
    done_groups, elapsed = 0, 0.0
    for kvh in range(cfg.num_kv_heads):
        heads = slice(kvh * g, (kvh + 1) * g)
        kv = slice(kvh, kvh + 1)
        t0 = time.perf_counter()
        if cfg.is_ranges:
            oracle.tree_attention_direct(data["q"][:, heads], data["k"][:, kv], data["v"][:, kv],
                                         data["do"][:, heads], data["node_off"], data["parent"],
                                         scale, hmap, dtype=np.float32)
            for w in data["windows"]:
                oracle.tree_window_attention_ranges(data["k"][:, kv], data["v"][:, kv],
                                                    w["ranges"], w["q"][:, heads], w["k"][:, kv],
                                                    w["v"][:, kv], w["do"][:, heads],
                                                    w["node_off"], w["parent"], scale, hmap,
                                                    dtype=np.float32)
        elif cfg.is_windows:
            q_ph = data["q_p"][:, heads]
            oracle.prefix_forward(q_ph, data["k_p"][:, kv], data["v_p"][:, kv], scale, hmap,
                                  dtype=np.float32)
            zero = np.zeros((cfg.prefix_len, 1, d), np.float32)
            oracle.prefix_backward_inject(q_ph, data["k_p"][:, kv], data["v_p"][:, kv],
                                          data["do_p"][:, heads], zero, zero, scale, hmap,
                                          dtype=np.float32)
            for w in data["windows"]:
                oracle.tree_window_attention(data["k_p"][:, kv], data["v_p"][:, kv],
                                             w["q"][:, heads], w["k"][:, kv], w["v"][:, kv],
                                             w["do"][:, heads], w["node_off"], w["parent"], scale,
                                             hmap, dtype=np.float32)
        elif cfg.is_tree:
            oracle.tree_attention_expanded(data["q"][:, heads], data["k"][:, kv],
                                           data["v"][:, kv], data["do"][:, heads],
                                           data["node_off"], data["parent"], scale, hmap,
                                           dtype=np.float32)
        else:
            oracle.suffix_attention_full_rows(data["q_p"][:, heads], data["k_p"][:, kv],
                                              data["v_p"][:, kv], data["q_s"][:, heads],
                                              data["k_s"][:, kv], data["v_s"][:, kv],
                                              data["do_s"][:, heads], data["cu_seqlens"], scale,
                                              hmap, dtype=np.float32)
        elapsed += time.perf_counter() - t0
        done_groups += 1
        if elapsed >= target_s:
            break
    full_s = elapsed * cfg.num_kv_heads / done_groups
    what = ("dense fwd+bwd of every root-to-leaf trajectory" if cfg.is_tree else
            "dense producer tree fwd+bwd and every window over its gathered ancestor rows"
            if cfg.is_ranges else
            "dense prefix fwd+bwd and every window over [prefix ; window rows]" if cfg.is_windows
            else
            "dense fwd+bwd of every trajectory [P || S_i], all rows")
    return {
        "value": group_flops / full_s / 1e12, "unit": "TFLOP/s", "cores": int(threads),
        "kind": "oracle",
        "sample": f"{what} of config {cfg.cid} on {done_groups} of {cfg.num_kv_heads} KV-head "
                  f"groups ({done_groups * g} query heads), fp32 numpy, {elapsed:.1f} s; value = "
                  f"the group's algorithmic FLOPs / the group time scaled from the sample",
        "seconds": elapsed, "os_cpu_count": os.cpu_count(),
        "affinity_cpus": len(os.sched_getaffinity(0)), "blas": blas,
        "full_workload_seconds_extrapolated": full_s,
        "group_tokens_per_s": {"compact": compact / full_s, "expanded": expanded / full_s},
    }


def run_logprob(cfg, data, args):
    """Compact log-probabilities (forward + backward) of one tree's compact rows:
    HBM-bound, so the line reports GB/s against the 8 TB/s HBM peak."""
    import torch

    import oracle
    import shared_prefix_attention_pf_amd as pf

    dev = torch.device("cuda:0")
    c, v = int(data["node_off"][-1]), cfg.logprob_vocab
    s_pos = len(data["m"])
    gen = torch.Generator(device=dev)
    gen.manual_seed(cfg.seed)
    z = (torch.randn(c, v, generator=gen, device=dev) * 3.0).to(torch.bfloat16)
    ints = {k: torch.from_numpy(data[k]).to(dev) for k in ("row_ptr", "pos", "y")}
    dl = torch.from_numpy(data["dlogp"]).to(dev)
    lse = torch.empty(c, device=dev)
    logp = torch.empty(s_pos, device=dev)
    dz = torch.empty_like(z)
    stream = torch.cuda.current_stream()
    timer = KernelTimer(torch, reserve=4 * (args.steps + 1))

    def step():
        pf.pf_compact_logprob_fwd(z, ints["row_ptr"], ints["pos"], ints["y"], lse, logp)
        pf.pf_compact_logprob_bwd(z, lse, ints["row_ptr"], ints["pos"], ints["y"], dl, dz)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    timer.phase = "logprob"
    pf.pf_set_launch_hook(timer)
    try:
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(args.steps):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    finally:
        pf.pf_set_launch_hook(None)
    ms = e0.elapsed_time(e1) / args.steps
    if args.copy_probe_mib > 0:
        copy_probe(torch, args.copy_probe_mib)
    eb = 2
    # algorithmic bytes: the logits read once forward, read and dz written once
    # backward, plus the per-position index, target and gradient arrays
    per_pos = 4 * 4
    fwd_bytes = c * v * eb + c * 4 + s_pos * per_pos + (c + 1) * 4
    bwd_bytes = 2 * c * v * eb + c * 4 + s_pos * per_pos + (c + 1) * 4
    value = (fwd_bytes + bwd_bytes) / (ms * 1e-3) / 1e9
    kern = timer.summary()
    dom = max(kern, key=lambda k: kern[k]["total_ms"])
    dom_bytes = bwd_bytes if dom == "pf_logprob_bwd" else fwd_bytes
    achieved = dom_bytes / (kern[dom]["avg_ms"] * 1e-3) / 1e9
    traffic, traffic_src = load_traffic(cfg.cid, dom)
    cpu = None
    if args.cpu_seconds > 0:
        print("[bench] timing the CPU oracle", flush=True)
        zs = z.float().cpu().numpy()
        rp, ps, ys = data["row_ptr"], data["pos"], data["y"]
        rows, t_cpu = 0, 0.0
        while rows < c and t_cpu < args.cpu_seconds:
            r1 = min(c, rows + 16)
            sub_ptr = (rp[rows:r1 + 1] - rp[rows]).astype(np.int32)
            sub_pos = ps[rp[rows]:rp[r1]]
            t0 = time.perf_counter()
            oracle.compact_logprob(zs[rows:r1], sub_ptr, sub_pos, ys, data["dlogp"])
            t_cpu += time.perf_counter() - t0
            rows = r1
        sample_bytes = 3 * rows * v * eb
        # numpy's elementwise exp and sums run on one thread
        cpu = {"value": sample_bytes / t_cpu / 1e9, "unit": "GB/s", "cores": 1,
               "kind": "oracle",
               "sample": f"compact log-prob fwd+bwd of {rows} of {c} rows (fp64 numpy; bytes "
                         f"counted as bf16 logits read twice and dz written once), {t_cpu:.1f} s"}
    out = {
        "metric": "compact log-prob fwd+bwd HBM GB/s (algorithmic bytes)",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"config {cfg.cid}: {cfg.name}", "rows": c, "vocab": v,
                   "positions": s_pos},
        "wall_ms_per_step": round(wall * 1e3 / args.steps, 4),
        "kernels": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv)
                        for kk, vv in kv.items()} for k, kv in kern.items()},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": traffic, "traffic_unit": "bytes per launch",
                     "traffic_source": traffic_src, "algorithmic_bytes_per_launch": dom_bytes,
                     "avg_launch_ms": round(kern[dom]["avg_ms"], 4)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def run_offload(cfg, data, args):
    """Dormant prefix offload at a flat config: copy rates each way, how much of
    the device-to-host copy Phase B hides, and Phase B's peak HBM with the
    dormant tensors resident or offloaded.  Prints one JSON line."""
    import torch

    import shared_prefix_attention_pf_amd as pf
    from shared_prefix_attention_pf_amd import group as G
    from shared_prefix_attention_pf_amd.offload import PinnedPool

    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    pdt = pf.PF_BF16 if cfg.dtype == "bf16" else pf.PF_F32
    desc = pf.AttnDesc(cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, pdt)
    t = {k: torch.from_numpy(np.ascontiguousarray(data[k])).to(tdt).to(dev)
         for k in ("q_p", "k_p", "v_p", "do_p", "q_s", "k_s", "v_s", "do_s")}
    cu = data["cu_seqlens"]
    p = cfg.prefix_len
    rows = int(cu[-1])
    ws = G.workspace(pf.PF_OP_SUFFIX_BWD, desc, p, rows, dev)
    gk = torch.zeros(p, cfg.num_kv_heads, cfg.head_dim, device=dev)
    gv = torch.zeros_like(gk)
    cs = torch.cuda.current_stream()

    def phase_b():
        o_s, lse_s = G.suffix_fwd(desc, t["k_p"], t["v_p"], cu, t["q_s"], t["k_s"], t["v_s"],
                                  ws=ws)
        G.suffix_bwd(desc, t["k_p"], t["v_p"], cu, t["q_s"], t["k_s"], t["v_s"], o_s, lse_s,
                     t["do_s"], gk, gv, ws=ws)

    def ev():
        return torch.cuda.Event(enable_timing=True)

    res = {}
    reps = max(3, args.steps)
    for _ in range(args.warmup):
        phase_b()
    # Phase A's outputs; Phase B reads none of Q_P, O_P, LSE_P
    o_p, lse_p = G.prefix_fwd(desc, t["q_p"], t["k_p"], t["v_p"])
    q_keep = t["q_p"].clone()          # Q_P of the later whole-group runs
    dormant = {"q_p": t.pop("q_p"), "o_p": o_p, "lse_p": lse_p}
    del o_p, lse_p
    nbytes = sum(x.numel() * x.element_size() for x in dormant.values())

    def steady_phase_b(key):
        # peak HBM over `reps` Phase-B steps, from a synchronized start
        torch.cuda.synchronize()
        torch.empty(1, device=dev)  # lets the allocator retire stream-deferred frees
        torch.cuda.reset_peak_memory_stats()
        a, b = ev(), ev()
        a.record(cs)
        for _ in range(reps):
            phase_b()
        b.record(cs)
        torch.cuda.synchronize()
        res[f"phase_b_ms_{key}"] = a.elapsed_time(b) / reps
        res[f"phase_b_peak_mib_{key}"] = torch.cuda.max_memory_allocated() / 2**20

    # dormant tensors resident through Phase B
    steady_phase_b("resident")
    # one pinned pool of about 1.5x the dormant bytes, allocated once
    pool = PinnedPool.for_footprint(nbytes)
    cps = pool.copy_stream
    # copy rates, each alone
    torch.cuda.synchronize()
    a, b = ev(), ev()
    a.record(cps)
    holder = pool.offload(dormant, cs)
    b.record(cps)
    torch.cuda.synchronize()
    res["d2h_ms"] = a.elapsed_time(b)
    a, b = ev(), ev()
    a.record(cps)
    holder.prefetch()
    b.record(cps)
    torch.cuda.synchronize()
    res["h2d_ms"] = a.elapsed_time(b)
    dormant = holder.get()
    del holder
    # Phase B with the offload running beside it on the copy stream: one
    # untimed round (its first time through this path can stall the host for
    # milliseconds), then `reps` timed rounds, each offloading and bringing
    # the tensors back; median and range reported
    beside, done = [], []
    for i in range(reps + 1):
        torch.cuda.synchronize()
        a, b, c0, c1 = ev(), ev(), ev(), ev()
        c0.record(cs)
        holder = pool.offload(dormant, cs)
        # the copy stream's event right behind the copies (recorded before
        # Phase B is enqueued, so host time spent enqueuing Phase B does not
        # count)
        c1.record(cps)
        del dormant
        a.record(cs)
        phase_b()
        b.record(cs)
        torch.cuda.synchronize()
        if i > 0:
            beside.append(a.elapsed_time(b))
            done.append(c0.elapsed_time(c1))
        if i < reps:
            dormant = holder.get()
            del holder
            torch.cuda.synchronize()
    res["phase_b_ms_beside_d2h"] = round(float(np.median(beside)), 4)
    res["d2h_done_ms_after_phase_b_start"] = round(float(np.median(done)), 4)
    res["d2h_done_ms_after_phase_b_start_range"] = [round(min(done), 4), round(max(done), 4)]
    res["d2h_rounds"] = reps
    # dormant tensors in host memory through Phase B
    steady_phase_b("offloaded")
    # Phase C's inputs come back
    holder.prefetch()
    holder.get()
    del holder
    torch.cuda.synchronize()
    # whole groups through the same pool: Phase A, offload right after it,
    # Phase B, prefetch, Phase C; no further pinned allocation
    n_groups = max(4, args.steps)
    desc_c = desc
    a, b = ev(), ev()
    a.record(cs)
    for _ in range(n_groups):
        o_p, lse_p = G.prefix_fwd(desc_c, q_keep, t["k_p"], t["v_p"])
        hg = pool.offload({"q_p": q_keep, "o_p": o_p, "lse_p": lse_p}, cs)
        del o_p, lse_p
        gk.zero_()
        gv.zero_()
        phase_b()
        hg.prefetch()
        back = hg.get(cs)
        G.prefix_bwd(desc_c, back["q_p"], t["k_p"], t["v_p"], back["o_p"], back["lse_p"],
                     t["do_p"], gk, gv)
        del back, hg
    b.record(cs)
    torch.cuda.synchronize()
    res["group_ms_through_pool"] = a.elapsed_time(b) / n_groups

    # Two layers of one group, in a trainer's order: both layers' Phase A (each
    # offloading its dormant tensors right after it), both layers' Phase B,
    # then the prefix backward in reverse layer order with the next layer's
    # prefetch issued before this layer's Phase C, so that the copy back runs
    # beside it (PrefixFlow §4.2: prefetched before the matching prefix-backward
    # layer).  The same sequence with the tensors resident is the comparison.
    # The pool holds both layers' tensors (1.5x of two layers).
    pool2 = PinnedPool.for_footprint(2 * nbytes, copy_stream=cps)

    def two_layers(offload):
        held = []
        for _ in range(2):
            o_p, lse_p = G.prefix_fwd(desc_c, q_keep, t["k_p"], t["v_p"])
            tens = {"q_p": q_keep, "o_p": o_p, "lse_p": lse_p}
            held.append(pool2.offload(tens, cs) if offload else tens)
            del o_p, lse_p, tens
        for _ in range(2):
            phase_b()
        if offload:
            held[1].prefetch()
        for layer in (1, 0):
            if offload:
                if layer == 1:
                    held[0].prefetch()
                back = held[layer].get(cs)
            else:
                back = held[layer]
            G.prefix_bwd(desc_c, back["q_p"], t["k_p"], t["v_p"], back["o_p"], back["lse_p"],
                         t["do_p"], gk, gv)
            del back

    for mode in (False, True):
        two_layers(mode)
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record(cs)
        for _ in range(reps):
            two_layers(mode)
        b.record(cs)
        torch.cuda.synchronize()
        res["two_layer_ms_offloaded" if mode else "two_layer_ms_resident"] = \
            a.elapsed_time(b) / reps
    out = {
        "metric": "dormant prefix offload across Phase B (host link)",
        "config": {"workload": f"config {cfg.cid}: {cfg.name}"},
        "dormant_bytes": nbytes,
        "d2h_gbs": round(nbytes / (res["d2h_ms"] * 1e-3) / 1e9, 2),
        "h2d_gbs": round(nbytes / (res["h2d_ms"] * 1e-3) / 1e9, 2),
        "phase_b_time_ratio_beside_d2h": round(res["phase_b_ms_beside_d2h"] /
                                               res["phase_b_ms_resident"], 4),
        "d2h_hidden_by_phase_b": res["d2h_done_ms_after_phase_b_start"] <=
                                 res["phase_b_ms_beside_d2h"],
        "phase_b_peak_hbm_saved_mib": round(res["phase_b_peak_mib_resident"] -
                                            res["phase_b_peak_mib_offloaded"], 2),
        "pool_bytes": pool.capacity, "pool_over_dormant": round(pool.capacity / nbytes, 3),
        "pinned_allocations": pool.pinned_allocations,
        "groups_through_pool": n_groups + reps + 2,
        "resident_fallbacks": pool.resident_fallbacks,
        "two_layer_pool_fallbacks": pool2.resident_fallbacks,
        "two_layer_overhead_ratio": round(res["two_layer_ms_offloaded"] /
                                          res["two_layer_ms_resident"], 4),
        **{k: (round(v, 4) if isinstance(v, float) else v) for k, v in res.items()},
    }
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path runs on one GPU: heads, groups or suffixes would shard across GPUs, "
              "none of which is built here)", file=sys.stderr)
        sys.exit(2)
    if args.stats_summary:
        stats_summary(args.stats_summary[0], args.stats_summary[1], args.config, args.pmc_command)
        return
    if args.counter_summary:
        counter_summary(args.counter_summary[:-1], args.counter_summary[-1], args.config,
                        args.pmc_command)
        return
    if args.traffic_summary:
        fdir, wdir, out_md = args.traffic_summary
        traffic_summary(fdir, wdir, out_md, args.config, args.copy_probe_mib, args.pmc_command)
        return
    from workloads import generate, get_config
    cfg = get_config(args.config)
    print(f"[bench] generating config {cfg.cid} ({cfg.name})", flush=True)
    data = generate(cfg)
    if cfg.is_logprob:
        print("[bench] running GPU steps", flush=True)
        run_logprob(cfg, data, args)
        return
    if args.offload:
        if cfg.is_tree or cfg.is_windows:
            raise SystemExit("--offload measures a flat group (configs 1-4)")
        print("[bench] measuring the dormant-prefix offload", flush=True)
        run_offload(cfg, data, args)
        return
    print("[bench] running GPU steps", flush=True)
    gres = run_gpu(cfg, data, args.steps, args.warmup, args.copy_probe_mib, args.separate_windows)
    d, hq = cfg.head_dim, cfg.num_q_heads
    if cfg.is_ranges:
        from oracle import tree_trajectories
        pairs_b = sum(ranges_window_pairs(w) for w in data["windows"])
        pairs_a = tree_pairs(data["node_off"], data["parent"])
        compact = int(data["node_off"][-1]) + sum(int(w["node_off"][-1]) for w in data["windows"])
        expanded = int(sum(sum(n for _, n in w["ranges"]) + len(t) for w in data["windows"]
                           for t in tree_trajectories(w["node_off"], w["parent"])))
        b_ms = gres["phase_ms"]["B"]
    elif cfg.is_windows:
        from oracle import tree_trajectories
        p = cfg.prefix_len
        pairs_b = sum(window_pairs(p, w["node_off"], w["parent"]) for w in data["windows"])
        pairs_a = p * (p + 1) // 2
        compact = p + sum(int(w["node_off"][-1]) for w in data["windows"])
        expanded = int(sum(p + len(t) for w in data["windows"]
                           for t in tree_trajectories(w["node_off"], w["parent"])))
        b_ms = gres["phase_ms"]["B"]
    elif cfg.is_tree:
        pairs_b = tree_pairs(data["node_off"], data["parent"])
        pairs_a = 0
        compact = int(data["node_off"][-1])
        from oracle import tree_trajectories
        expanded = int(sum(len(t) for t in tree_trajectories(data["node_off"], data["parent"])))
        b_ms = gres["phase_ms"]["tree"]
    else:
        lens = np.diff(data["cu_seqlens"])
        pairs_b, pairs_a = flat_pairs(cfg.prefix_len, lens)
        compact = cfg.prefix_len + int(lens.sum())
        expanded = int(np.sum(cfg.prefix_len + lens))
        b_ms = gres["phase_ms"]["B"]
    flops_b = 12.0 * d * pairs_b * hq
    step_ms = sum(gres["phase_ms"].values())
    value = flops_b / (b_ms * 1e-3) / 1e12
    # the same phase by other conventions: the median and fastest step, and the
    # FlashAttention count (backward 10 d per pair: dQ's product included)
    extra = {"value_median_step": round(flops_b / (gres["headline_phase_ms_median"] * 1e-3) / 1e12, 3),
             "value_fastest_step": round(flops_b / (gres["headline_phase_ms_min"] * 1e-3) / 1e12, 3),
             "value_fa_convention": round(14.0 / 12.0 * value, 3),
             "headline_phase_ms_steps": gres["headline_phase_ms_steps"]}

    # roofline of the kernel with the largest total time
    kern = gres["kernels"]
    dom = max(kern, key=lambda k: kern[k]["total_ms"])
    # algorithmic FLOPs of each matrix kernel per visible (query, key) pair per
    # query head: forward 4d (S = QK^T, O = PV); dQ kernels 2d (dQ = dS K; the
    # recompute of S and dP is not counted); dK/dV kernel 6d (dV, dP, dK)
    per_pair = {"pf_fwd_bf16": 4, "pf_bwd_dq_bf16": 2, "pf_bwd_dq_ds_bf16": 2,
                "pf_bwd_dkv_bf16": 6, "pf_fwd_f32": 4, "pf_bwd_dq_f32": 2,
                "pf_bwd_dq_ds_f32": 2, "pf_bwd_dkv_f32": 6}
    # a kernel launched in a phase covers every visible pair of that phase
    phase_pairs = {"A": pairs_a, "B": pairs_b, "C": pairs_a, "tree": pairs_b}
    for label, kn in kern.items():
        if label not in per_pair:
            continue
        flops = (sum(per_pair[label] * d * hq * phase_pairs[ph] for ph in kn["phases"]) *
                 gres["kernel_pass"]["steps"])
        kn["algorithmic_flops_per_launch"] = flops / kn["launches"]
        kn["tflops"] = flops / (kn["total_ms"] * 1e-3) / 1e12
    if dom in per_pair:
        kn = kern[dom]
        flops_per_launch = kn["algorithmic_flops_per_launch"]
        achieved = flops_per_launch / (kn["avg_ms"] * 1e-3) / 1e12
        peak = PEAK_BF16_TFLOPS if "bf16" in dom else PEAK_F32_TFLOPS
        traffic, traffic_src = load_traffic(cfg.cid, dom)
        roofline = {"bound": "mfma", "kernel": dom,
                    "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                    "frac": round(achieved / peak, 4),
                    "traffic": None if traffic is None else round(traffic),
                    "traffic_unit": "bytes per launch", "traffic_source": traffic_src,
                    "avg_launch_ms": round(kn["avg_ms"], 4),
                    "algorithmic_flops_per_launch": flops_per_launch}
    else:
        roofline = {"bound": "hbm", "kernel": dom, "achieved": None, "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": None, "traffic": None}

    # the group's algorithmic work: Phase A forward (4d per pair), Phase B
    # forward and backward (12d), Phase C backward (8d); or the tree (12d)
    group_flops = flops_b + 12.0 * d * pairs_a * hq
    cpu = None
    if args.cpu_seconds > 0:
        print("[bench] timing the CPU oracle", flush=True)
        cpu = cpu_baseline(cfg, data, args.cpu_seconds, group_flops, compact, expanded)

    peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
    out = {
        "metric": (f"suffix attn fwd+bwd TFLOP/s & % {cfg.dtype} MFMA peak; group tokens/s vs "
                   "oracle"),
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {
            "workload": f"config {cfg.cid}: {cfg.name}",
            "num_q_heads": hq, "num_kv_heads": cfg.num_kv_heads, "head_dim": d,
            "prefix_len": cfg.prefix_len,
            "suffix_lens": (None if cfg.is_tree or cfg.is_windows or cfg.is_ranges else
                            np.diff(data["cu_seqlens"]).astype(int).tolist()),
            "microbatches": (len(data["windows"]) if cfg.is_windows or cfg.is_ranges else
                             None if cfg.is_tree else len(data["microbatches"])),
            "window_rows": ([int(w["node_off"][-1]) for w in data["windows"]]
                            if cfg.is_windows or cfg.is_ranges else None),
            "window_calls": (None if not cfg.is_windows else
                             len(data["windows"]) if args.separate_windows or
                             cfg.window_calls != 1 else 1),
            "cached_ranges": ([w["ranges"] for w in data["windows"]] if cfg.is_ranges else None),
            "parallelism": "single GPU",
        },
        f"pct_of_{cfg.dtype}_peak": round(100.0 * value / peak, 2),
        "phase_ms": {k: round(v, 4) for k, v in gres["phase_ms"].items()},
        "phase_b_gflop": round(flops_b / 1e9, 2),
        "group_tokens_per_s": {"compact": round(compact / (step_ms * 1e-3), 1),
                               "expanded": round(expanded / (step_ms * 1e-3), 1)},
        "wall_ms_per_step": round(gres["wall_ms_per_step"], 4),
        "steps_total_ms_per_step": round(gres["steps_total_ms"] / args.steps, 4),
        "kernels": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv)
                        for kk, vv in v.items()} for k, v in kern.items()},
        "kernel_pass": gres["kernel_pass"],
        "roofline": roofline,
        "cpu_baseline": cpu,
        "device": gres["device"], "compute_units": gres["cus"],
    }
    out["group_tflops"] = round(group_flops / (step_ms * 1e-3) / 1e12, 3)
    out.update(extra)
    # the D / LSE pre-pass (HBM-bound): dO and O read (bf16), D and LSE log2(e)
    # written (fp32), per row and query head of the Phase-B call
    kd = kern.get("pf_prep_dsum")
    if kd and "B" in kd.get("phase_avg_ms", {}) and not (cfg.is_tree or cfg.is_ranges):
        # Phase-B rows, over the Phase-B launches of one step (one per call)
        per_step = kd["phases"]["B"] / gres["kernel_pass"]["steps"]
        rows_b = (compact - cfg.prefix_len) / per_step
        nbytes = rows_b * hq * (2 * d * (2 if cfg.dtype == "bf16" else 4) + 8)
        out["prep_dsum_phase_b_gbs"] = round(nbytes / (kd["phase_avg_ms"]["B"] * 1e-3) / 1e9, 1)
    if cpu:
        # the same group on both sides: algorithmic TFLOP/s and group tokens/s
        ratio = out["group_tflops"] / cpu["value"] if cpu["value"] > 0 else None
        out["gpu_over_oracle"] = round(ratio, 1) if ratio else None
    line = json.dumps(out)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(line + "\n")
    print(line, flush=True)


if __name__ == "__main__":
    main()
