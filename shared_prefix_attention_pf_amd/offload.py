"""Dormant prefix activations in pinned host memory across the Phase A -> B ->
C boundary ("PrefixFlow: Training-Time KV Caching for Schedule-Level Prefix
Reuse in LLM RL Training": §3.2, challenge C2, the prefix K/V and gK/gV are
hot during Phase B while the other saved prefix tensors are dormant until the
delayed prefix backward; §4.2, they are moved to a pinned host pool after
they are produced and prefetched asynchronously before the prefix backward
that needs them, with a demand load when no prefetch was issued).

At the attention boundary the dormant tensors are the ones only Phase C reads:
Q_P, O_P and LSE_P (K_P and V_P stay resident: every Phase-B call reads them).
`DormantPrefix.offload` copies them to pinned host buffers on a copy stream,
ordered after the producing work by an event, and drops the device copies
once the copy is done; `prefetch` copies them back on the copy stream; `get`
makes the compute stream wait for that copy and returns the device tensors.
If `get` is called without a prefetch, the copy is issued then (the demand
load).  Device memory and streams come from torch; nothing here computes.
Streams keep the default priority.
"""
from typing import Dict, Optional

import torch


class DormantPrefix:
    def __init__(self, tensors: Dict[str, torch.Tensor],
                 copy_stream: Optional[torch.cuda.Stream] = None):
        self.dev: Optional[Dict[str, torch.Tensor]] = dict(tensors)
        self.meta = {k: (t.shape, t.dtype, t.device) for k, t in tensors.items()}
        # pinned host buffers, allocated once per holder
        self.host = {k: torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
                     for k, t in tensors.items()}
        self.copy_stream = copy_stream or torch.cuda.Stream()
        self._ready: Optional[torch.cuda.Event] = None
        self._offloaded: Optional[torch.cuda.Event] = None

    def offload(self, compute_stream: Optional[torch.cuda.Stream] = None) -> None:
        """Copy the tensors to host after the work queued so far on
        `compute_stream`, then release the device copies."""
        cs = compute_stream or torch.cuda.current_stream()
        produced = torch.cuda.Event()
        produced.record(cs)
        self.copy_stream.wait_event(produced)
        with torch.cuda.stream(self.copy_stream):
            for k, t in self.dev.items():
                self.host[k].copy_(t, non_blocking=True)
                # the caching allocator must not hand this memory out again
                # before the copy stream has read it
                t.record_stream(self.copy_stream)
        self._offloaded = torch.cuda.Event()
        self._offloaded.record(self.copy_stream)
        self.dev = None

    def prefetch(self) -> None:
        """Start the host-to-device copy on the copy stream."""
        if self.dev is not None:
            return
        with torch.cuda.stream(self.copy_stream):
            self.dev = {}
            for k, (shape, dtype, device) in self.meta.items():
                t = torch.empty(shape, dtype=dtype, device=device)
                t.copy_(self.host[k], non_blocking=True)
                self.dev[k] = t
        self._ready = torch.cuda.Event()
        self._ready.record(self.copy_stream)

    def get(self, compute_stream: Optional[torch.cuda.Stream] = None) -> Dict[str, torch.Tensor]:
        """The device tensors, usable on `compute_stream` (prefetching on
        demand if no prefetch was issued)."""
        cs = compute_stream or torch.cuda.current_stream()
        if self.dev is None:
            self.prefetch()
        if self._ready is not None:
            cs.wait_event(self._ready)
            for t in self.dev.values():
                t.record_stream(cs)
            self._ready = None
        return self.dev

    def host_bytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in self.host.values())
