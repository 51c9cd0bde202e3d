"""Pins of the compact log-probability oracle (HARTS §3.5), none comparing
the oracle with itself: torch's log_softmax and autograd on the expanded
per-position logits (the definition the compact form must reproduce), scipy's
logsumexp, and the grouping helper against a direct scan."""
import numpy as np
import pytest
import torch
from scipy.special import logsumexp

from oracle.logprob import compact_logprob, row_logsumexp
from workloads.gen import positions_by_row


def _case(seed, c=7, v=53, s=23):
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((c, v)) * 3.0
    m = rng.integers(0, c, size=s)
    y = rng.integers(0, v, size=s)
    dl = rng.standard_normal(s)
    return z, m, y, dl


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_matches_expanded_log_softmax_and_autograd(seed):
    """Expanded logits z[m(s)] per position, torch log_softmax and autograd:
    the gather's backward sums every position's gradient into its row."""
    z, m, y, dl = _case(seed)
    row_ptr, pos = positions_by_row(m, z.shape[0])
    ref = compact_logprob(z, row_ptr, pos, y, dl)
    zt = torch.tensor(z, dtype=torch.float64, requires_grad=True)
    lp = torch.log_softmax(zt[torch.tensor(m)], dim=-1)
    lam = lp.gather(1, torch.tensor(y)[:, None])[:, 0]
    (lam * torch.tensor(dl)).sum().backward()
    np.testing.assert_allclose(ref["logp"], lam.detach().numpy(), atol=1e-12)
    np.testing.assert_allclose(ref["dz"], zt.grad.numpy(), atol=1e-12)


def test_rows_without_positions_have_zero_gradient():
    z, m, y, dl = _case(5, c=9)
    m = np.where(m == 3, 4, m)           # row 3 read by no position
    row_ptr, pos = positions_by_row(m, z.shape[0])
    ref = compact_logprob(z, row_ptr, pos, y, dl)
    assert np.all(ref["dz"][3] == 0.0)


def test_row_logsumexp_matches_scipy():
    z = np.random.default_rng(3).standard_normal((5, 1000)) * 20
    np.testing.assert_allclose(row_logsumexp(z), logsumexp(z, axis=1), rtol=1e-14)


def test_grouping_by_row():
    m = np.asarray([2, 0, 2, 1, 0, 2])
    row_ptr, pos = positions_by_row(m, 4)
    assert row_ptr.tolist() == [0, 2, 3, 6, 6]
    assert pos.tolist() == [1, 4, 3, 0, 2, 5]
