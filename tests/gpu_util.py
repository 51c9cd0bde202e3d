"""Shared helpers of the GPU parity tests (device transfer and error norms)."""
import numpy as np
import torch

TOL = {"bf16": 2e-2, "f32": 1e-4}


def dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    """Device tensor holding exactly the (dtype-representable) values of x."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t
    return t.cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def normwise(x, y) -> float:
    """max |x - y| / max |y| (the max-relative-error measure of the parity bar)."""
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    den = np.abs(y).max() if y.size else 0.0
    num = np.abs(x - y).max() if y.size else 0.0
    return float(num / den) if den > 0 else float(num)


def check(name, got, ref, tol):
    err = normwise(got, ref)
    print(f"  {name}: normwise err {err:.3e} (tol {tol:.0e})", flush=True)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    assert err <= tol, f"{name}: normwise error {err:.3e} > {tol:.0e}"
    return err
