"""Dense masked attention, forward and backward, written out from the definition.

For query head h reading KV head g = map(h) and softmax scale s:

    Z = s * Q K^T, with invisible (q, k) pairs set to -inf
    A = row-softmax(Z);  O = A V;  LSE_q = m_q + ln sum_k exp(Z_qk - m_q)

and for an upstream gradient dO:

    dV = A^T dO;  dA = dO V^T;  D_q = sum_k A_qk dA_qk
    dZ = A * (dA - D);  dQ = s dZ K;  dK = s dZ^T Q

with dK, dV of a KV head summed over every query head that reads it.  This is
the plain full-sequence attention that the PrefixFlow page's three-phase
schedule reproduces exactly (PrefixFlow §3.1 "Overall Three-Phase Schedule",
§3.3 "The Training-Time KV Boundary").  A row that sees no key gets O = 0,
LSE = -inf and contributes no gradient.

Test infrastructure only (see the package docstring).
"""
from typing import Optional, Sequence

import numpy as np


def head_map(num_q_heads: int, num_kv_heads: int,
             q_to_kv: Optional[Sequence[int]] = None) -> np.ndarray:
    """KV head read by each query head.  Default: contiguous groups h // (Hq/Hkv)."""
    if q_to_kv is None:
        if num_q_heads % num_kv_heads:
            raise ValueError("num_q_heads must be a multiple of num_kv_heads")
        g = num_q_heads // num_kv_heads
        return np.arange(num_q_heads) // g
    m = np.asarray(q_to_kv, dtype=np.int64)
    if m.shape != (num_q_heads,) or m.min() < 0 or m.max() >= num_kv_heads:
        raise ValueError("bad head map")
    return m


def _softmax_rows(z: np.ndarray, visible: np.ndarray):
    """Row softmax of z over visible entries: (A, LSE).  Fully masked rows -> 0, -inf."""
    zm = np.where(visible, z, -np.inf)
    m = zm.max(axis=1)
    live = np.isfinite(m)
    shift = np.where(live, m, 0.0)
    e = np.where(visible, np.exp(zm - shift[:, None]), 0.0)
    l = e.sum(axis=1)
    a = np.where(live[:, None], e / np.where(live, l, 1.0)[:, None], 0.0)
    lse = np.where(live, shift + np.log(np.where(live, l, 1.0)), -np.inf)
    return a, lse


def attention_forward(q, k, v, visible, scale, hmap, dtype=np.float64):
    """q [Lq, Hq, d]; k, v [Lk, Hkv, d]; visible [Lq, Lk] bool.

    Returns o [Lq, Hq, d] and lse [Hq, Lq] (natural log).
    """
    lq, hq, d = q.shape
    o = np.zeros((lq, hq, d), dtype=dtype)
    lse = np.zeros((hq, lq), dtype=dtype)
    for h in range(hq):
        g = int(hmap[h])
        qh = q[:, h, :].astype(dtype)
        kg = k[:, g, :].astype(dtype)
        vg = v[:, g, :].astype(dtype)
        z = dtype(scale) * (qh @ kg.T)
        a, lse[h] = _softmax_rows(z, visible)
        o[:, h, :] = a @ vg
    return o, lse


def attention_backward(q, k, v, do, visible, scale, hmap, dtype=np.float64):
    """Gradients of sum(dO * O) with respect to q, k, v (same shapes as inputs)."""
    lq, hq, d = q.shape
    lk, hkv, _ = k.shape
    dq = np.zeros((lq, hq, d), dtype=dtype)
    dk = np.zeros((lk, hkv, d), dtype=dtype)
    dv = np.zeros((lk, hkv, d), dtype=dtype)
    for h in range(hq):
        g = int(hmap[h])
        qh = q[:, h, :].astype(dtype)
        kg = k[:, g, :].astype(dtype)
        vg = v[:, g, :].astype(dtype)
        doh = do[:, h, :].astype(dtype)
        z = dtype(scale) * (qh @ kg.T)
        a, _ = _softmax_rows(z, visible)
        dv[:, g, :] += a.T @ doh
        da = doh @ vg.T
        dsum = (a * da).sum(axis=1)
        dz = a * (da - dsum[:, None])
        dq[:, h, :] = dtype(scale) * (dz @ kg)
        dk[:, g, :] += dtype(scale) * (dz.T @ qh)
    return dq, dk, dv
