"""Pins for the oracle's core attention (forward and backward).

Each test checks the oracle against something other than itself: central
finite differences, torch's fp64 autograd and its SDPA math path, scipy's
logsumexp, hand-derived closed forms, and invariants of the softmax.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

from oracle import attention_backward, attention_forward, head_map
from oracle.masks import causal_mask, suffix_rows_mask

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _random_mask(rng, lq, lk):
    vis = rng.uniform(size=(lq, lk)) < 0.6
    vis[np.arange(lq), rng.integers(0, lk, size=lq)] = True  # no fully masked row
    return vis


def _loss(q, k, v, do, vis, scale, hmap):
    o, _ = attention_forward(q, k, v, vis, scale, hmap)
    return float((o * do).sum())


@pytest.mark.parametrize("hq,hkv", [(2, 2), (4, 2), (3, 1)])
def test_finite_difference_directional(hq, hkv):
    """<grad, R> matches the central difference of sum(dO * O) along R, per input."""
    rng = np.random.default_rng(7 + hq)
    lq, lk, d = 5, 7, 8
    q, k, v = _rand(rng, lq, hq, d), _rand(rng, lk, hkv, d), _rand(rng, lk, hkv, d)
    do = _rand(rng, lq, hq, d)
    vis = _random_mask(rng, lq, lk)
    scale = 0.37
    hmap = head_map(hq, hkv)
    dq, dk, dv = attention_backward(q, k, v, do, vis, scale, hmap)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        r = _rand(rng, *x.shape)
        xp, xm = x + h * r, x - h * r
        args_p = dict(q=q, k=k, v=v)
        args_m = dict(q=q, k=k, v=v)
        args_p[name], args_m[name] = xp, xm
        fd = (_loss(do=do, vis=vis, scale=scale, hmap=hmap, **args_p)
              - _loss(do=do, vis=vis, scale=scale, hmap=hmap, **args_m)) / (2 * h)
        an = float((g * r).sum())
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (name, fd, an)


def test_finite_difference_every_element():
    """Full Jacobian-vector check, element by element, on a tiny causal case."""
    rng = np.random.default_rng(3)
    l, hq, hkv, d = 4, 2, 1, 3
    q, k, v = _rand(rng, l, hq, d), _rand(rng, l, hkv, d), _rand(rng, l, hkv, d)
    do = _rand(rng, l, hq, d)
    vis = causal_mask(l)
    hmap = head_map(hq, hkv)
    dq, dk, dv = attention_backward(q, k, v, do, vis, 0.8, hmap)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            ap = dict(q=q, k=k, v=v)
            am = dict(q=q, k=k, v=v)
            ap[name], am[name] = xp, xm
            fd = (_loss(do=do, vis=vis, scale=0.8, hmap=hmap, **ap)
                  - _loss(do=do, vis=vis, scale=0.8, hmap=hmap, **am)) / (2 * h)
            assert abs(fd - g[idx]) < 1e-7, (name, idx, fd, g[idx])


def _torch_reference(q, k, v, do, vis, scale, hmap):
    """torch fp64 autograd through an explicit masked softmax."""
    tq = torch.tensor(q, dtype=torch.float64, requires_grad=True)
    tk = torch.tensor(k, dtype=torch.float64, requires_grad=True)
    tv = torch.tensor(v, dtype=torch.float64, requires_grad=True)
    idx = torch.tensor(hmap, dtype=torch.long)
    kk = tk[:, idx, :].permute(1, 0, 2)             # [Hq, Lk, d]
    vv = tv[:, idx, :].permute(1, 0, 2)
    qq = tq.permute(1, 0, 2)                        # [Hq, Lq, d]
    z = scale * torch.matmul(qq, kk.transpose(1, 2).contiguous())
    z = z.masked_fill(~torch.tensor(vis)[None], float("-inf"))
    lse = torch.logsumexp(z, dim=-1)
    o = torch.matmul(torch.softmax(z, dim=-1), vv).permute(1, 0, 2)
    o.backward(torch.tensor(do, dtype=torch.float64))
    return (o.detach().numpy(), lse.detach().numpy(), tq.grad.numpy(), tk.grad.numpy(),
            tv.grad.numpy())


@pytest.mark.parametrize("hq,hkv", [(4, 4), (4, 2), (6, 3)])
def test_against_torch_autograd(hq, hkv):
    rng = np.random.default_rng(11 * hq + hkv)
    lq, lk, d = 9, 13, 16
    q, k, v = _rand(rng, lq, hq, d), _rand(rng, lk, hkv, d), _rand(rng, lk, hkv, d)
    do = _rand(rng, lq, hq, d)
    vis = _random_mask(rng, lq, lk)
    hmap = head_map(hq, hkv)
    o, lse = attention_forward(q, k, v, vis, 0.25, hmap)
    dq, dk, dv = attention_backward(q, k, v, do, vis, 0.25, hmap)
    ro, rlse, rdq, rdk, rdv = _torch_reference(q, k, v, do, vis, 0.25, hmap)
    for a, b in ((o, ro), (lse, rlse), (dq, rdq), (dk, rdk), (dv, rdv)):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


def test_against_torch_sdpa_math():
    """torch's SDPA (math backend, fp64, boolean mask) forward and backward."""
    rng = np.random.default_rng(5)
    hq, hkv, lq, lk, d = 4, 2, 6, 10, 8
    q, k, v = _rand(rng, lq, hq, d), _rand(rng, lk, hkv, d), _rand(rng, lk, hkv, d)
    do = _rand(rng, lq, hq, d)
    vis = suffix_rows_mask(lk - lq, lq)
    hmap = head_map(hq, hkv)
    scale = 1.0 / math.sqrt(d)
    o, _ = attention_forward(q, k, v, vis, scale, hmap)
    dq, dk, dv = attention_backward(q, k, v, do, vis, scale, hmap)
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    rep = hq // hkv
    qq = tq.permute(1, 0, 2)[None]
    kk = tk.repeat_interleave(rep, dim=1).permute(1, 0, 2)[None]
    vv = tv.repeat_interleave(rep, dim=1).permute(1, 0, 2)[None]
    with torch.nn.attention.sdpa_kernel(torch.nn.attention.SDPBackend.MATH):
        ro = torch.nn.functional.scaled_dot_product_attention(
            qq, kk, vv, attn_mask=torch.tensor(vis), scale=scale)
    ro = ro[0].permute(1, 0, 2)
    ro.backward(torch.tensor(do))
    np.testing.assert_allclose(o, ro.detach().numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-11, atol=1e-12)


def test_lse_is_logsumexp():
    rng = np.random.default_rng(8)
    q, k, v = _rand(rng, 7, 2, 4), _rand(rng, 9, 1, 4), _rand(rng, 9, 1, 4)
    vis = _random_mask(rng, 7, 9)
    _, lse = attention_forward(q, k, v, vis, 0.5, head_map(2, 1))
    for h in range(2):
        z = 0.5 * q[:, h, :] @ k[:, 0, :].T
        ref = scipy.special.logsumexp(np.where(vis, z, -np.inf), axis=1)
        np.testing.assert_allclose(lse[h], ref, rtol=1e-14, atol=1e-14)


def test_golden_hand_derived_example():
    """A 1-query, 3-key example whose softmax weights are 1/6, 2/6, 3/6 by construction."""
    with open(os.path.join(GOLDEN, "softmax_three_keys.json")) as f:
        g = json.load(f)
    q = np.asarray(g["q"], dtype=np.float64).reshape(1, 1, -1)
    k = np.asarray(g["k"], dtype=np.float64).reshape(3, 1, -1)
    v = np.asarray(g["v"], dtype=np.float64).reshape(3, 1, -1)
    do = np.asarray(g["do"], dtype=np.float64).reshape(1, 1, -1)
    vis = np.ones((1, 3), dtype=bool)
    hmap = head_map(1, 1)
    o, lse = attention_forward(q, k, v, vis, g["scale"], hmap)
    dq, dk, dv = attention_backward(q, k, v, do, vis, g["scale"], hmap)
    exp = g["expected"]
    np.testing.assert_allclose(o.ravel(), exp["o"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse.ravel(), [math.log(exp["lse_exp"])], rtol=0, atol=1e-15)
    ln2, ln3 = math.log(2.0), math.log(3.0)
    dq_ref = [exp["dq_coeff_ln2"] * ln2 + exp["dq_coeff_ln3"] * ln3, 0.0]
    np.testing.assert_allclose(dq.ravel(), dq_ref, rtol=0, atol=1e-15)
    np.testing.assert_allclose(dk[:, 0, 0], exp["dk_first_component"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(dk[:, 0, 1], 0.0, atol=1e-15)
    np.testing.assert_allclose(dv[:, 0, 0], exp["dv_first_component"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(dv[:, 0, 1], 0.0, atol=1e-15)


def test_invariants():
    """Row-constant score shifts leave O and dV unchanged; sum_k dK_k = 0; V = 1 gives O = 1."""
    rng = np.random.default_rng(21)
    hq, hkv, lq, lk, d = 4, 2, 6, 8, 5
    q, k, v = _rand(rng, lq, hq, d), _rand(rng, lk, hkv, d), _rand(rng, lk, hkv, d)
    do = _rand(rng, lq, hq, d)
    vis = _random_mask(rng, lq, lk)
    hmap = head_map(hq, hkv)
    o, lse = attention_forward(q, k, v, vis, 0.7, hmap)
    dq, dk, dv = attention_backward(q, k, v, do, vis, 0.7, hmap)
    c = _rand(rng, d)
    k2 = k + c[None, None, :]
    o2, lse2 = attention_forward(q, k2, v, vis, 0.7, hmap)
    _, _, dv2 = attention_backward(q, k2, v, do, vis, 0.7, hmap)
    np.testing.assert_allclose(o2, o, atol=1e-12)
    np.testing.assert_allclose(dv2, dv, atol=1e-12)
    for h in range(hq):
        np.testing.assert_allclose(lse2[h] - lse[h], 0.7 * q[:, h, :] @ c, atol=1e-12)
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-12)
    ones, _ = attention_forward(q, k, np.ones_like(v), vis, 0.7, hmap)
    np.testing.assert_allclose(ones, 1.0, atol=1e-14)


def test_gqa_equals_mha_with_repeated_kv():
    rng = np.random.default_rng(4)
    hq, hkv, lq, lk, d = 6, 2, 5, 7, 4
    q, k, v = _rand(rng, lq, hq, d), _rand(rng, lk, hkv, d), _rand(rng, lk, hkv, d)
    do = _rand(rng, lq, hq, d)
    vis = _random_mask(rng, lq, lk)
    g = head_map(hq, hkv)
    o, lse = attention_forward(q, k, v, vis, 0.5, g)
    dq, dk, dv = attention_backward(q, k, v, do, vis, 0.5, g)
    kr, vr = k[:, g, :], v[:, g, :]
    ident = np.arange(hq)
    o2, lse2 = attention_forward(q, kr, vr, vis, 0.5, ident)
    dq2, dkr, dvr = attention_backward(q, kr, vr, do, vis, 0.5, ident)
    np.testing.assert_allclose(o, o2, atol=1e-14)
    np.testing.assert_allclose(lse, lse2, atol=1e-14)
    np.testing.assert_allclose(dq, dq2, atol=1e-14)
    for j in range(hkv):
        np.testing.assert_allclose(dk[:, j], dkr[:, g == j].sum(axis=1), atol=1e-13)
        np.testing.assert_allclose(dv[:, j], dvr[:, g == j].sum(axis=1), atol=1e-13)


def test_explicit_head_map():
    """A permuted head map equals the contiguous map on permuted query heads."""
    rng = np.random.default_rng(6)
    hq, hkv, lq, lk, d = 4, 2, 3, 5, 4
    q, k, v = _rand(rng, lq, hq, d), _rand(rng, lk, hkv, d), _rand(rng, lk, hkv, d)
    do = _rand(rng, lq, hq, d)
    vis = _random_mask(rng, lq, lk)
    m = np.array([1, 0, 0, 1])
    perm = np.argsort(m, kind="stable")            # heads reading kv 0 first
    o, _ = attention_forward(q, k, v, vis, 0.5, head_map(hq, hkv, m))
    o2, _ = attention_forward(q[:, perm], k, v, vis, 0.5, head_map(hq, hkv))
    np.testing.assert_allclose(o[:, perm], o2, atol=1e-14)
    _, dk, _ = attention_backward(q, k, v, do, vis, 0.5, head_map(hq, hkv, m))
    _, dk2, _ = attention_backward(q[:, perm], k, v, do[:, perm], vis, 0.5, head_map(hq, hkv))
    np.testing.assert_allclose(dk, dk2, atol=1e-13)


def test_fully_masked_row_convention():
    q, k, v = np.ones((2, 1, 2)), np.ones((3, 1, 2)), np.ones((3, 1, 2))
    vis = np.array([[True, False, False], [False, False, False]])
    o, lse = attention_forward(q, k, v, vis, 1.0, head_map(1, 1))
    assert np.all(o[1] == 0) and lse[0, 1] == -np.inf
    dq, dk, dv = attention_backward(q, k, v, np.ones((2, 1, 2)), vis, 1.0, head_map(1, 1))
    assert np.all(dq[1] == 0)
