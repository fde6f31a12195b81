"""Helpers shared by the GPU parity tests (marshalling and the tolerance)."""
from __future__ import annotations

import sys

import numpy as np

import quant_matvec_amd as kq

# Per-row acceptance: |y_gpu - y_ref| <= 1e-4 * sum_j |W_ij x_j| + 1e-6, with
# y_ref and the sum from the binary64 oracle.
REL_TOL = 1e-4
ABS_TOL = 1e-6


def torch():
    import torch as _t
    return _t


def dev(a: np.ndarray):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(a)).to("cuda")


def host(t) -> np.ndarray:
    torch().cuda.synchronize()
    return t.detach().cpu().numpy()


def note(msg: str) -> None:
    """Name the case on stdout before it runs on the GPU (flushed)."""
    print("[case] " + msg, flush=True)
    sys.stdout.flush()


def gpu_matvec(fmt, w_np, rows, cols, x_np, ldx=None, ldy=None):
    """Run kq_matvec on copies of the host arrays; returns y [ntok, rows]."""
    t = torch()
    x_np = np.atleast_2d(x_np).astype(np.float32)
    ntok = x_np.shape[0]
    ldx = ldx or cols
    ldy = ldy or rows
    xp = np.zeros((ntok, ldx), np.float32)
    xp[:, :cols] = x_np
    w = dev(w_np.reshape(-1))
    x = dev(xp)
    y = t.full((ntok, ldy), float("nan"), dtype=t.float32, device="cuda")
    kq.kq_matvec(fmt, w, rows, cols, x, y, ntok=ntok, ldx=ldx, ldy=ldy)
    out = host(y)
    if ldy > rows:
        assert np.isnan(out[:, rows:]).all(), "kernel wrote past rows"
    return out[:, :rows]


def check_tol(y, y_ref, s, what=""):
    y = np.asarray(y, np.float64)
    err = np.abs(y - y_ref)
    bound = REL_TOL * s + ABS_TOL
    bad = ~(err <= bound)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError("%s: %d of %d outputs outside tolerance; first %s: gpu %r ref %r bound %r"
                             % (what, int(bad.sum()), bad.size, tuple(i), y[tuple(i)], y_ref[tuple(i)],
                                bound[tuple(i)]))
    ratio = err / bound
    return float(ratio.max()) if ratio.size else 0.0
