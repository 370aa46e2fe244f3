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


GUARD_BYTE = 0xA5


class Guarded:
    """A device buffer between two guard bands (a 256-byte band before it,
    4 KiB after), filled with GUARD_BYTE, to catch writes outside the
    buffer.  The buffer itself starts as NaN (float types; caught by the
    finite check of any row left unwritten), as zeros (`zero=True`, the
    workspace rule) or as GUARD_BYTE (integer types).  The lead band keeps
    the buffer 256-byte aligned (torch allocations are)."""

    LEAD = 256
    TRAIL = 4096

    def __init__(self, shape, dtype, zero=False):
        import torch
        self.shape = tuple(shape)
        n = 1
        for s in self.shape:
            n *= s
        esz = torch.empty(0, dtype=dtype).element_size()
        self.nbytes = n * esz
        self.raw = torch.full((self.LEAD + self.nbytes + self.TRAIL,), GUARD_BYTE,
                              dtype=torch.uint8, device="cuda")
        body = self.raw[self.LEAD:self.LEAD + self.nbytes]
        self.t = body.view(dtype).view(self.shape)
        if zero:
            self.t.zero_()
        elif dtype.is_floating_point:
            self.t.fill_(float("nan"))

    def check(self, what=""):
        import torch
        torch.cuda.synchronize()
        lead = self.raw[:self.LEAD]
        trail = self.raw[self.LEAD + self.nbytes:]
        assert bool((lead == GUARD_BYTE).all()), f"{what}: write before the buffer"
        assert bool((trail == GUARD_BYTE).all()), f"{what}: write after the buffer"


def guarded_workspace(nbytes):
    """A zero-filled workspace inside guard bands (None if nbytes is 0)."""
    import torch
    if nbytes == 0:
        return None
    return Guarded((nbytes,), torch.uint8, zero=True)
