"""The row-block assembly of Phase A / Phase C used by the full-size GPU tests
equals the dense oracle (PrefixFlow §3.1, §3.3: causal prefix rows over the
rows before them are suffixes over a cached prefix, and K/V gradients add)."""
import math

import numpy as np
import pytest

from oracle import head_map, prefix_backward_inject, prefix_forward
from tests.row_blocks import prefix_phases_by_row_blocks
from workloads.gen import random_small_group


@pytest.mark.parametrize("p,block", [(37, 8), (16, 16), (9, 20)])
def test_row_blocks_equal_dense_prefix_phases(p, block):
    g = random_small_group(3, 4, 2, 8, p, [], "f32")
    q, k, v, do = (g[n].astype(np.float64) for n in ("q_p", "k_p", "v_p", "do_p"))
    rng = np.random.Generator(np.random.PCG64(4))
    gk, gv = rng.standard_normal((2, p, 2, 8))
    hmap = head_map(4, 2)
    scale = 1.0 / math.sqrt(8)
    o, lse = prefix_forward(q, k, v, scale, hmap)
    dq, dk, dv = prefix_backward_inject(q, k, v, do, gk, gv, scale, hmap)
    bo, blse, bdq, bdk, bdv = prefix_phases_by_row_blocks(q, k, v, do, gk, gv, scale, hmap, block)
    for name, x, y in (("O", bo, o), ("LSE", blse, lse), ("dQ", bdq, dq), ("dK", bdk, dk),
                       ("dV", bdv, dv)):
        err = np.abs(x - y).max() / np.abs(y).max()
        assert err < 1e-12, f"{name}: {err}"
