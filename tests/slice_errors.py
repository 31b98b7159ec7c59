"""Per-slice relative Frobenius errors, computed in fp64: the parity measure of the GPU tests.

A slice is one (sequence, value head): its boundary state [dv, dk] and its per-token outputs
[n, dv].  The error of a slice is |X_gpu - X_ref|_F / |X_ref|_F, or the absolute error
|X_gpu - X_ref|_F when the reference slice is zero.
"""
import numpy as np
import torch


def np64(t):
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu", torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def _ratio(num, den):
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), num)


def state_errors(S_gpu, S_ref):
    """[B, Hv] errors of states [B, Hv, dv, dk]."""
    a, b = np64(S_gpu), np64(S_ref)
    B, Hv = b.shape[:2]
    diff = np.linalg.norm((a - b).reshape(B, Hv, -1), axis=-1)
    return _ratio(diff, np.linalg.norm(b.reshape(B, Hv, -1), axis=-1))


def output_errors(o_gpu, o_ref, cu):
    """[B, Hv] errors of packed outputs [T, Hv, dv] over the sequences of cu (empty ones: 0)."""
    a, b = np64(o_gpu), np64(o_ref)
    cu = np.asarray(cu, dtype=np.int64)
    B, Hv = len(cu) - 1, b.shape[1]
    out = np.zeros((B, Hv))
    for s in range(B):
        lo, hi = int(cu[s]), int(cu[s + 1])
        if hi == lo:
            continue
        d = np.sqrt(np.sum((a[lo:hi] - b[lo:hi]) ** 2, axis=(0, 2)))
        out[s] = _ratio(d, np.sqrt(np.sum(b[lo:hi] ** 2, axis=(0, 2))))
    return out
