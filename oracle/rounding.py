"""Rounding points of the replay contract (oracle side; test infrastructure only).

bf16 keeps 8 significant bits and the fp32 exponent range.  The oracle rounds an
fp64 value straight to the nearest bf16, ties to even, without passing through
fp32 (no double rounding).
"""
from __future__ import annotations

import numpy as np


def round_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value (ties to even), as float64."""
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    finite = np.isfinite(x) & (x != 0)
    xf = x[finite]
    m, e = np.frexp(xf)                     # xf = m * 2**e, 0.5 <= |m| < 1
    # bf16 normal numbers have exponents >= -126, i.e. frexp exponent >= -125;
    # below that the spacing stays at 2**-133 (subnormal range).
    e_eff = np.maximum(e, -125)
    scaled = np.ldexp(xf, 8 - e_eff)        # |scaled| < 2**8 for normals
    r = np.ldexp(np.rint(scaled), e_eff - 8)   # np.rint rounds half to even
    # values beyond the largest bf16 (0x7F7F) overflow to infinity
    big = np.abs(r) > np.ldexp(255.0, 127 - 7)
    r[big] = np.copysign(np.inf, r[big])
    out[finite] = r
    return out


def round_f32(x) -> np.ndarray:
    """Round float64 values to the nearest float32 value (ties to even), as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
