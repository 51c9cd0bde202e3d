"""The pinned pool's slot placement (host logic only): slots never overlap,
stay inside the buffer, are reused after they are freed, and a request that
does not fit is refused rather than placed over a live slot."""
import random

import pytest

torch = pytest.importorskip("torch")
from shared_prefix_attention_pf_amd.offload import RingSlots  # noqa: E402


def _check(ring):
    spans = sorted(ring.live)
    for (o, n) in spans:
        assert 0 <= o and o + n <= ring.capacity
    for (a, n), (b, _) in zip(spans, spans[1:]):
        assert a + n <= b, "live slots overlap"


def test_full_ring_refuses_instead_of_overlapping():
    r = RingSlots(100 * 256)
    a = r.alloc(60 * 256)
    b = r.alloc(40 * 256)
    assert (a, b) == (0, 60 * 256)
    r.free(a)
    c = r.alloc(50 * 256)          # wraps to the front
    assert c == 0
    d = r.alloc(10 * 256)          # fills [50, 60)
    assert d == 50 * 256
    assert r.alloc(256) is None    # full: head meets the oldest live slot
    _check(r)
    r.free(b)
    assert r.alloc(40 * 256) == 60 * 256
    _check(r)


@pytest.mark.parametrize("seed", range(20))
def test_random_groups_never_overlap(seed):
    """Groups of three tensors offloaded and brought back in order, with up to
    two groups live at once, in a 1.5x pool: every placement valid."""
    rng = random.Random(seed)
    sizes = [rng.randrange(1, 50) * 256 for _ in range(3)]
    cap = int(1.5 * sum(sizes)) + 8 * 256
    r = RingSlots(cap)
    live_groups = []
    placed = refused = 0
    for _ in range(200):
        if live_groups and (len(live_groups) == 2 or rng.random() < 0.5):
            for off in live_groups.pop(0):
                if off is not None:
                    r.free(off)
        else:
            offs = [r.alloc(s) for s in sizes]
            placed += sum(o is not None for o in offs)
            refused += sum(o is None for o in offs)
            live_groups.append(offs)
        _check(r)
    assert placed > refused
