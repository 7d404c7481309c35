"""Parity metric shared by the GPU tests.

For each independent unit (sequence, head) and each compared tensor X:
err = max|X_gpu - X_ref| / max|X_ref| over that unit's elements; a test reports
the largest err over units.  Elementwise relative error is not used because
bf16 outputs near zero have no relative accuracy; this is the per-unit scale.
"""
import numpy as np
import torch

TOL_BF16 = 2e-2
TOL_F32 = 1e-4


def to64(x):
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def unit_err_fixed(x, ref):
    """x, ref: [B, H, ...]; one unit per (b, h)."""
    x, ref = to64(x), to64(ref)
    B, H = ref.shape[:2]
    d = np.abs(x - ref).reshape(B * H, -1).max(1)
    s = np.abs(ref).reshape(B * H, -1).max(1)
    return float((d / np.maximum(s, 1e-300)).max())


def unit_err_varlen(x, ref, cu):
    """x, ref: [1, H, Ttot, d]; one unit per (sequence, head)."""
    x, ref = to64(x), to64(ref)
    cu = [int(c) for c in to64(cu)]
    worst = 0.0
    for n in range(len(cu) - 1):
        a, b = cu[n], cu[n + 1]
        if b == a:
            continue
        d = np.abs(x[0, :, a:b] - ref[0, :, a:b]).reshape(ref.shape[1], -1).max(1)
        s = np.abs(ref[0, :, a:b]).reshape(ref.shape[1], -1).max(1)
        worst = max(worst, float((d / np.maximum(s, 1e-300)).max()))
    return worst
