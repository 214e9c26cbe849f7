"""Shared helpers for the GPU parity tests (device transfer and tolerance checks)."""
import sys

import numpy as np

TOL = 2e-3   # |y - y_ref| <= TOL * sum |w| |x| per output


def announce(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def dev(a, dtype=None):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint32:
        t = torch.from_numpy(a.view(np.int32))
    else:
        t = torch.from_numpy(a)
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def x_dev(x, bf16):
    import torch
    t = dev(x.astype(np.float32))
    return t.to(torch.bfloat16) if bf16 else t


def check_tol(y, y_ref, bound, what, tol=TOL):
    y = np.asarray(y, dtype=np.float64)
    err = np.abs(y - y_ref)
    lim = tol * bound + 1e-30
    bad = err > lim
    ratio = float((err / lim).max()) if err.size else 0.0
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} outputs over tolerance; "
                           f"worst err/tol {ratio:.3f}")
    assert np.isfinite(y).all(), f"{what}: non-finite output"
    return ratio


def sigmoid(z):
    """1 / (1 + e^-z) without overflow for large |z|."""
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(-np.abs(z))
    return np.where(z >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def silu(z):
    return np.asarray(z, dtype=np.float64) * sigmoid(z)
