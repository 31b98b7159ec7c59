"""ctypes loader for libtailreplay.so (the C ABI in include/tailreplay.h).

Loading fails loudly when the library has not been built: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtailreplay.so")

TR_OK, TR_ERR_INVALID_ARG, TR_ERR_UNSUPPORTED, TR_ERR_WORKSPACE, TR_ERR_HIP = range(5)
TR_BF16, TR_F32 = 0, 1
TR_NOALLOC_SCRATCH_BYTES = 64 << 20   # the header's TR_NOALLOC_SCRATCH_BYTES
TR_SCHEDULE_AUTO, TR_SCHEDULE_FUSED, TR_SCHEDULE_SPLIT = 0, 1, 2

# Every symbol the header declares: (name, restype, argtypes).
_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_f32 = ctypes.c_float
_sz = ctypes.c_size_t


class LaWeights(ctypes.Structure):
    """Mirror of tr_la_weights."""
    _fields_ = [("w_qk", _vp), ("w_v", _vp), ("w_a", _vp), ("w_b", _vp), ("w_o", _vp), ("rms_gain", _vp)]


SIGNATURES = {
    "tr_last_error": (ctypes.c_char_p, []),
    "tr_version": (ctypes.c_char_p, []),
    "tr_tail_length": (_i64, [_i64, _i32, _i32]),
    "tr_tail_seqlens": (ctypes.c_int, [_vp, _i32, _i32, _i32, _vp, _vp]),
    "tr_gdn_replay": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                     _i32, _i32, _i32, _i32, _i32, _i32, ctypes.c_int, _f32,
                                     _vp, _vp, _vp, _vp, _sz, _vp]),
    "tr_gdn_replay_noalloc": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                             _i32, _i32, _i32, _i32, _i32, _i32, ctypes.c_int, _f32,
                                             _vp, _vp, _vp, _vp]),
    "tr_gdn_replay_workspace_size": (_sz, [_vp, _i32, _i32, _i32, _i32, _i32, ctypes.c_int]),
    "tr_gdn_set_schedule": (ctypes.c_int, [ctypes.c_int]),
    "tr_gdn_get_schedule": (ctypes.c_int, []),
    "tr_gdn_transition": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, ctypes.c_int,
                                         _vp, _vp, _vp, _sz, _vp]),
    "tr_gdn_transition_workspace_size": (_sz, [_vp, _i32, _i32, _i32, _i32, ctypes.c_int]),
    "tr_state_compose": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp]),
    "tr_gdn_decode": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, ctypes.c_int, _f32,
                                     _vp, _vp, _vp]),
    "tr_la_layer_inputs_workspace_size": (_sz, [_i32, _i32, _i32]),
    "tr_la_layer_inputs": (ctypes.c_int, [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32,
                                          _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "tr_rmsnorm": (ctypes.c_int, [_vp, _vp, _i32, _i32, _i32, _f32, _vp, _vp]),
    "tr_la_project": (ctypes.c_int, [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                     _vp, _vp, _vp, _vp, _vp, _vp]),
    "tr_la_output_residual": (ctypes.c_int, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp]),
    "tr_group_replay_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "tr_group_replay": (ctypes.c_int, [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32,
                                       _vp, _vp, _sz, _vp]),
}

_lock = threading.Lock()
_lib = None


class TailReplayError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("status %d: %s" % (status, message))
        self.status = status


def lib() -> ctypes.CDLL:
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise ImportError("libtailreplay.so is not built (%s); run `python -m "
                                  "linear_attention_state_amd.build` first" % LIB_PATH)
            handle = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(handle, name)
                fn.restype = res
                fn.argtypes = args
            _lib = handle
    return _lib


def check(status: int) -> None:
    if status != TR_OK:
        raise TailReplayError(status, lib().tr_last_error().decode())
