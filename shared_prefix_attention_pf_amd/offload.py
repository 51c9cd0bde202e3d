"""Dormant prefix activations in one pinned host pool across the Phase A -> B ->
C boundary ("PrefixFlow: Training-Time KV Caching for Schedule-Level Prefix
Reuse in LLM RL Training": §3.2, challenge C2, the prefix K/V and gK/gV are
hot during Phase B while the other saved prefix tensors are dormant until the
delayed prefix backward; §4.2, "Pinned pool and transfers": they go to a
pinned host pool of about 1.5 times the saved footprint right after they are
produced, and come back ahead of the prefix backward that needs them, with a
demand load when no prefetch was issued).

At the attention boundary the dormant tensors are the ones only Phase C reads:
Q_P, O_P and LSE_P (K_P and V_P stay resident: every Phase-B call reads them).

`PinnedPool` owns one pinned host buffer (allocated once, through torch's
pinned allocator, i.e. hipHostMalloc) and one copy stream.  `offload` places
each tensor in a slot of the buffer, taken in ring order, and copies it there
on the copy stream after the work already queued on the compute stream (call
it right after Phase A); the device copies are then dropped.  `prefetch` copies
them back on the copy stream; `get` makes the compute stream wait for that copy
(issuing it first if no prefetch was made: the demand load) and hands the
slots back to the pool.  Because every copy into or out of the buffer runs on
the one copy stream, a slot's next offload is ordered after the host-to-device
copy that last read it.  A tensor that does not fit in the free part of the
ring stays on the device (counted in `resident_fallbacks`): the result is the
same, only the HBM saving is lost.  Nothing here computes; streams keep the
default priority.
"""
from typing import Dict, List, Optional, Tuple

import torch

_ALIGN = 256


def _round(n: int) -> int:
    return (n + _ALIGN - 1) // _ALIGN * _ALIGN


class RingSlots:
    """First-in first-out placement of byte slots in a buffer of `capacity`
    bytes (host logic only).  Live slots are kept in allocation order; their
    offsets increase, wrap to 0 at most once, and increase again, so the free
    space is [head, capacity) and [0, tail) when they have not wrapped, and
    [head, tail) when they have (tail = the oldest live slot, head = the end of
    the newest).  Slots may be freed in any order; space behind an older live
    slot is reused once that slot is freed."""

    def __init__(self, capacity: int):
        self.capacity = capacity
        self.live: List[Tuple[int, int]] = []    # (offset, size), allocation order

    def alloc(self, nbytes: int) -> Optional[int]:
        n = _round(max(int(nbytes), 1))
        if n > self.capacity:
            return None
        if not self.live:
            start = 0
        else:
            tail = self.live[0][0]
            last_off, last_n = self.live[-1]
            head = last_off + last_n
            if last_off >= tail:          # not wrapped: free [head, cap) and [0, tail)
                if head + n <= self.capacity:
                    start = head
                elif n <= tail:
                    start = 0
                else:
                    return None
            elif head + n <= tail:        # wrapped: free [head, tail)
                start = head
            else:
                return None
        self.live.append((start, n))
        return start

    def free(self, offset: int) -> None:
        for i, (o, _) in enumerate(self.live):
            if o == offset:
                del self.live[i]
                return
        raise KeyError(offset)

    def used(self) -> int:
        return sum(n for _, n in self.live)


class PinnedPool:
    """A ring of byte slots in one pinned host buffer, reused group after group."""

    def __init__(self, capacity_bytes: int, copy_stream: Optional[torch.cuda.Stream] = None):
        self.capacity = _round(max(int(capacity_bytes), _ALIGN))
        self.buf = torch.empty(self.capacity, dtype=torch.uint8, pin_memory=True)
        self.copy_stream = copy_stream or torch.cuda.Stream()
        self.ring = RingSlots(self.capacity)
        self.pinned_allocations = 1              # pinned buffers ever allocated
        self.resident_fallbacks = 0              # tensors that did not fit and stayed on device
        self.bytes_offloaded = 0

    @classmethod
    def for_footprint(cls, footprint_bytes: int, headroom: float = 1.5,
                      copy_stream: Optional[torch.cuda.Stream] = None) -> "PinnedPool":
        """A pool of headroom x one group's dormant bytes (PrefixFlow §4.2: about 1.5x)."""
        return cls(int(footprint_bytes * headroom) + 8 * _ALIGN, copy_stream)

    def _alloc(self, nbytes: int) -> Optional[int]:
        return self.ring.alloc(nbytes)

    def _free(self, offset: int) -> None:
        self.ring.free(offset)

    def host_view(self, offset: int, shape, dtype) -> torch.Tensor:
        n = torch.Size(shape).numel() * torch.empty(0, dtype=dtype).element_size()
        return self.buf[offset:offset + n].view(dtype).view(shape)

    def live_bytes(self) -> int:
        return self.ring.used()

    def offload(self, tensors: Dict[str, torch.Tensor],
                compute_stream: Optional[torch.cuda.Stream] = None) -> "DormantPrefix":
        """Move `tensors` (contiguous device tensors) to the pool after the work
        queued so far on `compute_stream`; returns their holder."""
        return DormantPrefix(self, tensors, compute_stream)


class DormantPrefix:
    """One group's dormant tensors: in pool slots while offloaded."""

    def __init__(self, pool: PinnedPool, tensors: Dict[str, torch.Tensor],
                 compute_stream: Optional[torch.cuda.Stream] = None):
        self.pool = pool
        self.meta = {k: (t.shape, t.dtype, t.device) for k, t in tensors.items()}
        self.slots: Dict[str, int] = {}
        self.dev: Dict[str, torch.Tensor] = {}
        self._ready: Optional[torch.cuda.Event] = None
        cs = compute_stream or torch.cuda.current_stream()
        produced = torch.cuda.Event()
        produced.record(cs)
        cps = pool.copy_stream
        cps.wait_event(produced)
        for k, t in tensors.items():
            if not t.is_contiguous():
                raise ValueError(f"{k}: only contiguous tensors can be offloaded")
            off = pool._alloc(t.numel() * t.element_size())
            if off is None:
                pool.resident_fallbacks += 1
                self.dev[k] = t
                continue
            self.slots[k] = off
            with torch.cuda.stream(cps):
                pool.host_view(off, t.shape, t.dtype).copy_(t, non_blocking=True)
                # the caching allocator must not hand this memory out again
                # before the copy stream has read it
                t.record_stream(cps)
            pool.bytes_offloaded += t.numel() * t.element_size()

    def offloaded_keys(self):
        return sorted(self.slots)

    def prefetch(self) -> None:
        """Start the host-to-device copies on the pool's copy stream."""
        if not self.slots or self._ready is not None:
            return
        cps = self.pool.copy_stream
        with torch.cuda.stream(cps):
            for k, off in self.slots.items():
                shape, dtype, device = self.meta[k]
                t = torch.empty(shape, dtype=dtype, device=device)
                t.copy_(self.pool.host_view(off, shape, dtype), non_blocking=True)
                self.dev[k] = t
        self._ready = torch.cuda.Event()
        self._ready.record(cps)

    def get(self, compute_stream: Optional[torch.cuda.Stream] = None) -> Dict[str, torch.Tensor]:
        """The device tensors, usable on `compute_stream`; the pool slots are
        free for the next group (its copies queue behind this one's on the
        copy stream)."""
        cs = compute_stream or torch.cuda.current_stream()
        if self.slots and self._ready is None:
            self.prefetch()
        if self._ready is not None:
            cs.wait_event(self._ready)
            for k in self.slots:
                self.dev[k].record_stream(cs)
            for off in self.slots.values():
                self.pool._free(off)
            self.slots = {}
            self._ready = None
        return dict(self.dev)
