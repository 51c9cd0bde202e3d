"""Phase A and Phase C of a long prefix, assembled from oracle calls on row blocks.

The fp64 oracle's dense Phase A / Phase C hold several P x P matrices per
query head (about 10 GB at P = 16384).  The same results follow from the
oracle's own Phase-B function applied to blocks of prefix rows: prefix rows
[r0, r1) see keys [0, r0) in full and keys [r0, r1) causally, which is a
suffix of r1 - r0 rows over a cached prefix of r0 rows (PrefixFlow §3.1
and §4.1: a suffix sees every cached token, then its own tokens causally).
Their outputs are rows of the causal prefix attention, and because the
backward is linear in the upstream gradient (PrefixFlow §3.3), the prefix
rows' K/V gradients are the sum over blocks of each block's cached-side
gradient (keys before r0) and its own-key gradient (keys in the block).

Only sums of oracle outputs happen here; `tests/test_oracle_phases.py` checks
this assembly against the dense oracle at a small size.
"""
import numpy as np

import oracle


def prefix_phases_by_row_blocks(q_p, k_p, v_p, do_p, gk_acc, gv_acc, scale, hmap, block,
                                progress=None):
    """(O_P, LSE_P, dQ_P, dK_P, dV_P) of one causal prefix with gK/gV injected,
    as oracle.prefix_forward and oracle.prefix_backward_inject define them."""
    p, hq, d = q_p.shape
    hkv = k_p.shape[1]
    o = np.zeros((p, hq, d))
    lse = np.zeros((hq, p))
    dq = np.zeros((p, hq, d))
    dk = np.zeros((p, hkv, d))
    dv = np.zeros((p, hkv, d))
    for r0 in range(0, p, block):
        r1 = min(p, r0 + block)
        if progress:
            progress(r0, r1)
        ref = oracle.suffix_attention(k_p[:r0], v_p[:r0], q_p[r0:r1], k_p[r0:r1], v_p[r0:r1],
                                      do_p[r0:r1], np.asarray([0, r1 - r0], np.int32), scale,
                                      hmap)
        o[r0:r1] = ref["o_s"]
        lse[:, r0:r1] = ref["lse_s"]
        dq[r0:r1] = ref["dq_s"]
        dk[:r0] += ref["gk"]
        dv[:r0] += ref["gv"]
        dk[r0:r1] += ref["dk_s"]
        dv[r0:r1] += ref["dv_s"]
    return o, lse, dq, dk + gk_acc, dv + gv_acc
