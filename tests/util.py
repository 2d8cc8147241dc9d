"""Helpers for the GPU parity tests: host<->device marshalling and error reports."""
from __future__ import annotations

import numpy as np

# tolerances (max-abs error against the fp64 oracle fed the same input values)
TOL_F32 = 1e-5
TOL_BF16_O = 2e-2
TOL_BF16_LSE = 1e-3


def dev(x: np.ndarray, bf16: bool | None = None):
    """numpy -> torch CUDA tensor.  uint16 arrays are bf16 bit patterns."""
    import torch
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def host(t) -> np.ndarray:
    """torch tensor -> float64 numpy (bf16 upcast exactly)."""
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def max_err(got: np.ndarray, want: np.ndarray):
    """Max-abs error over entries where ``want`` is not NaN, with its index.
    -inf must match exactly (rows without keys)."""
    sel = ~np.isnan(want)
    g, w = got[sel], want[sel]
    inf_ok = np.array_equal(np.isneginf(g), np.isneginf(w))
    fin = np.isfinite(w)
    if not fin.any():
        return 0.0, None, inf_ok
    diff = np.where(fin, np.abs(np.where(fin, g, 0) - np.where(fin, w, 0)), 0.0)
    diff = np.where(np.isnan(g) & fin, np.inf, diff)
    k = int(np.argmax(diff))
    idx = tuple(int(i[k]) for i in np.nonzero(sel))
    return float(diff[k]), idx, inf_ok


def assert_close(name: str, got: np.ndarray, want: np.ndarray, tol: float):
    err, where, inf_ok = max_err(got, want)
    print(f"  {name}: max|err| = {err:.3e} at {where} (tol {tol:g})", flush=True)
    assert inf_ok, f"{name}: -inf pattern differs"
    assert err <= tol, f"{name}: max|err| {err:.3e} at {where} > {tol:g}"
