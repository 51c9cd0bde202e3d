"""Compact log-probability recovery, written out from its definition.

HARTS §3.5 ("Compact log-probability recovery"): every semantic position s of
the original trajectories has a compact row m(s) and a next-token target y_s;
its log-probability is

    lambda_s = z[m(s), y_s] - log sum_v exp z[m(s), v]

so the logits are kept only per compact row (C x V), never per position
(S x V).  The backward gives each position's own contribution to its row:

    dz[c, v] = sum over s with m(s) = c of  dlambda_s * (1[v = y_s] - softmax(z_c)[v])

(the pages: the backward sums each position's own gradient into its compact
row instead of scaling one gradient by a reuse count).  Positions are given
grouped by row, as (row_ptr, pos): the positions of row c are
pos[row_ptr[c] : row_ptr[c + 1]].

Test infrastructure only (see the package docstring).
"""
from typing import Dict

import numpy as np


def row_logsumexp(z: np.ndarray) -> np.ndarray:
    """[C] natural-log sum of exp over each row of z [C, V], max-shifted."""
    z = np.asarray(z, dtype=np.float64)
    m = z.max(axis=1)
    return m + np.log(np.exp(z - m[:, None]).sum(axis=1))


def compact_logprob(z, row_ptr, pos, y, dlogp=None) -> Dict[str, np.ndarray]:
    """lse [C], logp [S] (position order) and, given dlogp [S], dz [C, V] (fp64)."""
    z = np.asarray(z, dtype=np.float64)
    c, v = z.shape
    s = len(y)
    lse = row_logsumexp(z)
    logp = np.full(s, np.nan)
    for r in range(c):
        for i in range(int(row_ptr[r]), int(row_ptr[r + 1])):
            p = int(pos[i])
            logp[p] = z[r, int(y[p])] - lse[r]
    out = {"lse": lse, "logp": logp}
    if dlogp is not None:
        dlogp = np.asarray(dlogp, dtype=np.float64)
        prob = np.exp(z - lse[:, None])
        dz = np.zeros_like(z)
        for r in range(c):
            for i in range(int(row_ptr[r]), int(row_ptr[r + 1])):
                p = int(pos[i])
                dz[r] -= dlogp[p] * prob[r]
                dz[r, int(y[p])] += dlogp[p]
        out["dz"] = dz
    return out
