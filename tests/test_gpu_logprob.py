"""GPU parity of the compact log-probability calls against the fp64 oracle
(HARTS §3.5), on ragged vocabularies, shared rows, repeated targets, unread
rows and out-of-range indices.

Tolerance: normwise max |x - y| / max |y| <= 1e-4 (fp32 logits) and 2e-2
(bf16 logits, whose dz is stored in bf16)."""
import numpy as np
import pytest
import torch

from oracle.logprob import compact_logprob
from tests.gpu_util import TOL, check
from workloads.gen import random_logprob_case

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import shared_prefix_attention_pf_amd as pf


def _dev_logits(z, dtype, pad_to=None):
    """z on the device in dtype, inside rows of pad_to elements (a strided view)."""
    c, v = z.shape
    width = pad_to or v
    t = torch.zeros(c, width, dtype=torch.bfloat16 if dtype == "bf16" else torch.float32,
                    device="cuda")
    t[:, :v] = torch.from_numpy(z).to(t.dtype).cuda()
    return t[:, :v]


CASES = [(37, 1000, 120, "f32", None), (50, 4099, 200, "bf16", 4104), (9, 64, 40, "bf16", None),
         (16, 152000, 64, "bf16", None), (12, 3001, 30, "f32", 3004),
         # fewer than eight columns (no whole vector), exactly one vector, and
         # a vocabulary whose backward chunks end in a partial group
         (7, 5, 20, "bf16", 8), (6, 8, 12, "f32", None), (11, 6150, 50, "bf16", 6152)]


@pytest.mark.parametrize("c,v,s,dtype,pad", CASES, ids=lambda x: str(x))
def test_compact_logprob(c, v, s, dtype, pad):
    print(f"\ncase C={c} V={v} S={s} {dtype} pad={pad}", flush=True)
    g = random_logprob_case(c + v + s, c, v, s, dtype)
    z = _dev_logits(g["z"], dtype, pad)
    ints = {k: torch.from_numpy(g[k]).cuda() for k in ("row_ptr", "pos", "y")}
    lse = torch.empty(c, device="cuda")
    logp = torch.full((s,), -7.0, device="cuda")
    pf.pf_compact_logprob_fwd(z, ints["row_ptr"], ints["pos"], ints["y"], lse, logp)
    dl = torch.from_numpy(g["dlogp"]).cuda()
    dz = torch.empty(c, pad or v, dtype=z.dtype, device="cuda")[:, :v]
    pf.pf_compact_logprob_bwd(z, lse, ints["row_ptr"], ints["pos"], ints["y"], dl, dz)
    torch.cuda.synchronize()
    ref = compact_logprob(g["z"], g["row_ptr"], g["pos"], g["y"], g["dlogp"])
    tol = TOL[dtype]
    check("lse", lse.cpu().double().numpy(), ref["lse"], tol)
    check("logp", logp.cpu().double().numpy(), ref["logp"], tol)
    check("dz", dz.float().cpu().double().numpy(), ref["dz"], tol)
    # a row no position reads has a zero gradient
    assert torch.count_nonzero(dz[c - 1].float()).item() == 0


def test_out_of_range_indices_are_skipped():
    """A target past the vocabulary gives NaN and no gradient; a position index
    past the end is skipped, so the position it replaced is neither written
    nor differentiated; everything else matches the oracle."""
    c, v, s = 6, 256, 10
    g = random_logprob_case(3, c, v, s, "f32")
    bad = int(g["pos"][0])               # its target moves past the vocabulary
    skipped = int(g["pos"][-1])          # its slot in pos gets an index past the end
    y = g["y"].copy()
    y[bad] = v + 5
    pos = g["pos"].copy()
    pos[-1] = s + 100
    z = _dev_logits(g["z"], "f32")
    rp, pp, yy = (torch.from_numpy(a).cuda() for a in (g["row_ptr"], pos, y))
    lse = torch.empty(c, device="cuda")
    logp = torch.full((s,), -7.0, device="cuda")
    pf.pf_compact_logprob_fwd(z, rp, pp, yy, lse, logp)
    dz = torch.empty_like(z)
    pf.pf_compact_logprob_bwd(z, lse, rp, pp, yy, torch.from_numpy(g["dlogp"]).cuda(), dz)
    torch.cuda.synchronize()
    out = logp.cpu().numpy()
    assert np.isnan(out[bad]) and out[skipped] == -7.0
    # the oracle with both positions contributing nothing
    dl = g["dlogp"].astype(np.float64).copy()
    dl[[bad, skipped]] = 0.0
    y_ok = g["y"].copy()
    ref = compact_logprob(g["z"], g["row_ptr"], g["pos"], y_ok, dl)
    ok = np.ones(s, dtype=bool)
    ok[[bad, skipped]] = False
    check("logp (valid positions)", out[ok].astype(np.float64), ref["logp"][ok], TOL["f32"])
    check("dz", dz.cpu().double().numpy(), ref["dz"], TOL["f32"])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_masked_vocabulary_columns(dtype):
    """Logits of -inf (a padded vocabulary masked out, and scattered masked
    columns, one whole 8-column vector among them) add nothing to the row's
    sum and get a zero gradient; the rest matches the oracle.  Targets stay on
    unmasked columns."""
    c, v, s, v_real = 10, 9000, 60, 8190
    g = random_logprob_case(77, c, v, s, dtype)
    z = g["z"].copy()
    z[:, v_real:] = -np.inf
    z[:, 1000:1008] = -np.inf
    z[:, 5::97] = -np.inf
    y = (g["y"] % v_real).astype(np.int32)
    keep = np.ones(v, dtype=bool)
    keep[v_real:] = False
    keep[1000:1008] = False
    keep[5::97] = False
    y = np.where(keep[y], y, 11).astype(np.int32)
    zd = _dev_logits(z, dtype)
    rp, pp, yy = (torch.from_numpy(a).cuda() for a in (g["row_ptr"], g["pos"], y))
    lse = torch.empty(c, device="cuda")
    logp = torch.empty(s, device="cuda")
    pf.pf_compact_logprob_fwd(zd, rp, pp, yy, lse, logp)
    dz = torch.empty_like(zd)
    pf.pf_compact_logprob_bwd(zd, lse, rp, pp, yy, torch.from_numpy(g["dlogp"]).cuda(), dz)
    torch.cuda.synchronize()
    ref = compact_logprob(z, g["row_ptr"], g["pos"], y, g["dlogp"])
    tol = TOL[dtype]
    check("lse", lse.cpu().double().numpy(), ref["lse"], tol)
    check("logp", logp.cpu().double().numpy(), ref["logp"], tol)
    got = dz.float().cpu().double().numpy()
    check("dz", got, ref["dz"], tol)
    assert np.all(got[:, ~keep] == 0.0)
