"""Host <-> device plumbing for the GPU tests (no attention arithmetic)."""
from __future__ import annotations

import numpy as np

import oracle

BF16_TOL = 2e-2
F32_TOL = 1e-5


def dev(arr):
    import torch
    arr = np.ascontiguousarray(arr)
    if arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16).copy()).cuda().view(torch.bfloat16)
    return torch.from_numpy(arr.copy()).cuda()


def host(t):
    import torch
    if t.dtype == torch.bfloat16:
        return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.detach().cpu().numpy()


def host_f64(t):
    return oracle.to_f64(host(t))


def tol_for(dtype: str) -> float:
    return BF16_TOL if dtype == "bf16" else F32_TOL


def compare(got, want, tol, what=""):
    """Max-abs contract plus the normalised diagnostics (printed)."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - want)
    rms = np.sqrt(np.mean(want ** 2)) if want.size else 0.0
    mx = float(err.max()) if err.size else 0.0
    print(f"[{what}] max|d|={mx:.3e} max|d|/rms={mx / rms if rms else 0:.3e} "
          f"rms|d|/rms={np.sqrt(np.mean(err ** 2)) / rms if rms else 0:.3e}")
    assert mx <= tol, f"{what}: max abs error {mx} > {tol}"
    return mx


def compare_lse(got, want, tol=1e-3, what="lse"):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    ninf = np.isneginf(want)
    assert np.array_equal(np.isneginf(got), ninf), f"{what}: -inf pattern differs"
    if (~ninf).any():
        d = np.abs(got[~ninf] - want[~ninf]).max()
        assert d <= tol, f"{what}: {d}"
