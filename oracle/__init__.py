"""CPU oracle for the Tail-Replay GDN state rebuild -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline``
leg may import this package.  The product path (``linear_attention_state_amd``)
never imports it and shares no code with it.

Contents
--------
* :func:`gdn` -- fp64 token-by-token Gated DeltaNet recurrence (C, OpenMP), the
  plain definition of Eq. (1) in section 2.3 of the reading notes
  "Tail-Replay：混合 LLM 前缀缓存的短尾重放机制".
* :func:`gdn_mirror` -- a second, independent numpy implementation of the same
  recurrence for tiny shapes (cross-check of the C code's indexing).
* :func:`tail_length` -- the replay length k = ceil(r m) (same notes, section 2.1
  symbol table and the worked example in section 2.2).
* :func:`group` -- one group's chain of LA layers replayed from the cached FA
  hidden vectors (section 2.2 steps 2-3), with the layer body described in
  ``chain.py``.
* :func:`round_bf16` / :func:`round_f32` -- the rounding points of the contract.

Every function here is pinned by tests/test_oracle.py or tests/test_oracle_group.py
to closed forms, invariants or library routines outside this package.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

from .rounding import round_bf16, round_f32  # noqa: F401
from .tail import tail_length, tail_range  # noqa: F401
from .mirror import gdn_mirror  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "_gdn_oracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (-O2, OpenMP).  Returns the library path."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def open_library(path):
    """Load a compiled oracle library (the default one, or a test's modified copy)."""
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int32)
    lib.oracle_gdn.argtypes = [dp, dp, dp, dp, dp, ip, ctypes.c_int32, ctypes.c_int32,
                               ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                               ctypes.c_double, dp, dp, dp]
    lib.oracle_gdn.restype = ctypes.c_int
    lib.oracle_num_threads.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is None:
            _lib = open_library(build())
    return _lib


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def _dptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double)) if a is not None else None


def gdn(q, k, v, g, beta, cu_seqlens, q_scale=1.0, state_in=None, want_o=True, lib=None):
    """fp64 GDN recurrence over packed sequences.

    q, k: [T, Hqk, dk]; v: [T, Hv, dv]; g, beta: [T, Hv]; cu_seqlens: [B+1].
    Inputs are converted exactly to float64 (bf16 and fp32 values are representable).
    Returns (state_out [B, Hv, dv, dk], o [T, Hv, dv] or None).
    """
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    g = np.ascontiguousarray(g, dtype=np.float64)
    beta = np.ascontiguousarray(beta, dtype=np.float64)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    T, Hqk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    B = cu.shape[0] - 1
    assert k.shape == q.shape and v.shape[0] == T and g.shape == (T, Hv) and beta.shape == (T, Hv)
    assert cu[0] == 0 and cu[-1] == T
    s_in = None
    if state_in is not None:
        s_in = np.ascontiguousarray(state_in, dtype=np.float64)
        assert s_in.shape == (B, Hv, dv, dk)
    s_out = np.empty((B, Hv, dv, dk), dtype=np.float64)
    o = np.empty((T, Hv, dv), dtype=np.float64) if want_o else None
    rc = (lib or _load()).oracle_gdn(_dptr(q), _dptr(k), _dptr(v), _dptr(g), _dptr(beta),
                            cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                            B, Hqk, Hv, dk, dv, float(q_scale), _dptr(s_in), _dptr(s_out), _dptr(o))
    if rc != 0:
        raise RuntimeError("oracle_gdn failed with code %d" % rc)
    return s_out, o


from .chain import group  # noqa: E402,F401
