"""C-ABI checks that need no GPU: the library loads, exports every symbol the header
declares, does tail selection in exact integers, and rejects bad arguments on the host
before any HIP call."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tailreplay.h")

L = pytest.importorskip("linear_attention_state_amd")
from linear_attention_state_amd import _lib as C  # noqa: E402  (status and schedule codes)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tr_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = L.lib()
    names = declared_functions()
    assert "tr_gdn_replay" in names and "tr_group_replay" in names and "tr_tail_length" in names
    for name in names:
        assert hasattr(lib, name), name
    # the Python binding knows the signature of every declared function
    from linear_attention_state_amd._lib import SIGNATURES
    assert sorted(SIGNATURES) == names


def test_tail_length_matches_oracle():
    rng = np.random.default_rng(3)
    for m in list(rng.integers(0, 1 << 40, size=500)) + [0, 1, 10000, 32768, 131072]:
        for rn, rd in ((5, 100), (10, 100), (1, 7), (7, 7)):
            assert L.tail_length(int(m), rn, rd) == oracle.tail_length(int(m), rn, rd)


def test_tail_seqlens_worked_example():
    cu, starts = L.tail_seqlens([10000, 32768, 4096], 5, 100)
    assert cu.tolist() == [0, 500, 500 + 1639, 500 + 1639 + 205]
    assert starts.tolist() == [9500, 32768 - 1639, 4096 - 205]


def test_tail_rejects_bad_ratio():
    with pytest.raises(ValueError):
        L.tail_length(100, 0, 100)
    with pytest.raises(ValueError):
        L.tail_length(100, 101, 100)
    with pytest.raises(ValueError):
        L.tail_length(-1, 5, 100)


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation first


def call_gdn(**over):
    cu = (ctypes.c_int32 * 3)(0, 5, 9)
    args = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, cu_h=ctypes.cast(cu, ctypes.c_void_p), cu_d=FAKE,
                B=2, T=9, Hqk=2, Hv=4, dk=128, dv=128, dt=0, q_scale=1.0, s_in=None, s_out=FAKE, o=FAKE,
                ws=None, ws_bytes=0)
    args.update(over)
    lib = L.lib()
    st = lib.tr_gdn_replay(args["q"], args["k"], args["v"], args["g"], args["beta"], args["cu_h"], args["cu_d"],
                           args["B"], args["T"], args["Hqk"], args["Hv"], args["dk"], args["dv"], args["dt"],
                           args["q_scale"], args["s_in"], args["s_out"], args["o"], args["ws"], args["ws_bytes"],
                           None)
    return st, lib.tr_last_error().decode()


@pytest.mark.parametrize("over,status", [
    (dict(B=0), 1),
    (dict(T=-1), 1),
    (dict(Hv=3), 1),                       # not a multiple of Hqk
    (dict(Hqk=0), 1),
    (dict(dk=96), 2),
    (dict(dv=256), 2),
    (dict(dt=7), 1),
    (dict(q_scale=0.0), 1),
    (dict(q_scale=float("nan")), 1),
    (dict(q=None), 1),
    (dict(s_out=None), 1),
    (dict(cu_d=None), 1),
    (dict(T=10), 1),                       # cu[B] != T
])
def test_gdn_rejects_bad_arguments(over, status):
    st, msg = call_gdn(**over)
    assert st == status and msg


def _ws_size(cu, B, Hv=4, dv=128, dt=0):
    arr = (ctypes.c_int32 * len(cu))(*cu)
    return L.lib().tr_gdn_replay_workspace_size(ctypes.cast(arr, ctypes.c_void_p), B, 2, Hv, 128, dv, dt)


def test_gdn_schedule_and_workspace_query():
    lib = L.lib()
    prev = lib.tr_gdn_get_schedule()
    try:
        assert lib.tr_gdn_set_schedule(7) == C.TR_ERR_INVALID_ARG and lib.tr_last_error()
        assert lib.tr_gdn_set_schedule(C.TR_SCHEDULE_AUTO) == C.TR_OK
        assert lib.tr_gdn_get_schedule() == C.TR_SCHEDULE_AUTO
        # few heads: the split schedule, whose records grow with the chunks and the heads
        n1 = _ws_size([0, 5, 9], 2)
        n2 = _ws_size([0, 500, 900], 2)
        assert 0 < n1 < n2 and n2 % 16 == 0
        assert _ws_size([0, 5, 9], 2, Hv=8) == 2 * n1
        assert _ws_size([0, 5, 9], 2, dt=1) == 0            # fp32 inputs: token path, no workspace
        assert _ws_size([0, 5, 9], 2, Hv=128) == 0          # many heads: fused
        assert lib.tr_gdn_set_schedule(C.TR_SCHEDULE_FUSED) == C.TR_OK
        assert _ws_size([0, 5, 9], 2) == 0
        assert lib.tr_gdn_set_schedule(C.TR_SCHEDULE_SPLIT) == C.TR_OK
        assert _ws_size([0, 5, 9], 2, Hv=128) > 0
        assert _ws_size([0, 5, 9], 0) == 0 and lib.tr_last_error()   # invalid: B = 0
        # a missing or short workspace is rejected before anything is enqueued
        assert lib.tr_gdn_set_schedule(C.TR_SCHEDULE_AUTO) == C.TR_OK
        st, msg = call_gdn()
        assert st == C.TR_ERR_WORKSPACE and "workspace" in msg
        st, msg = call_gdn(ws=FAKE, ws_bytes=n1 - 1)
        assert st == C.TR_ERR_WORKSPACE
        st, msg = call_gdn(ws=ctypes.c_void_p(0x1008), ws_bytes=n1)
        assert st == C.TR_ERR_INVALID_ARG and "aligned" in msg
    finally:
        lib.tr_gdn_set_schedule(prev)


def test_gdn_rejects_bad_cu_seqlens():
    for bad in ((1, 5, 9), (0, 6, 5)):
        cu = (ctypes.c_int32 * 3)(*bad)
        st, msg = call_gdn(cu_h=ctypes.cast(cu, ctypes.c_void_p), T=bad[-1])
        assert st == 1 and "cu_seqlens" in msg


def call_transition(**over):
    cu = (ctypes.c_int32 * 3)(0, 5, 9)
    args = dict(k=FAKE, g=FAKE, beta=FAKE, cu_h=ctypes.cast(cu, ctypes.c_void_p), cu_d=FAKE,
                B=2, T=9, Hqk=2, Hv=4, d=128, dt=0, phi=FAKE)
    args.update(over)
    lib = L.lib()
    st = lib.tr_gdn_transition(args["k"], args["g"], args["beta"], args["cu_h"], args["cu_d"], args["B"], args["T"],
                               args["Hqk"], args["Hv"], args["d"], args["dt"], args["phi"], None, None)
    return st, lib.tr_last_error().decode()


@pytest.mark.parametrize("over,status", [
    (dict(B=0), 1), (dict(Hv=3), 1), (dict(d=96), 2), (dict(dt=5), 1), (dict(k=None), 1),
    (dict(phi=None), 1), (dict(cu_d=None), 1), (dict(T=8), 1),
])
def test_transition_rejects_bad_arguments(over, status):
    st, msg = call_transition(**over)
    assert st == status and "tr_gdn_transition" in msg


def test_state_compose_rejects_bad_arguments():
    lib = L.lib()
    other = ctypes.c_void_p(0x2000)
    cases = [((FAKE, FAKE, None, None, other, 0, 128, 128), 1),          # N < 1
             ((FAKE, FAKE, None, None, other, 4, 96, 128), 2),           # unsupported dv
             ((None, FAKE, None, None, other, 4, 128, 128), 1),          # null S_c
             ((FAKE, other, None, None, FAKE, 4, 128, 128), 1),          # out aliases S_c
             ((other, FAKE, None, None, FAKE, 4, 128, 128), 1)]          # out aliases phi
    for args, status in cases:
        st = lib.tr_state_compose(*args, None)
        assert st == status and "tr_state_compose" in lib.tr_last_error().decode()


def test_decode_rejects_bad_arguments():
    lib = L.lib()
    base = [FAKE, FAKE, FAKE, FAKE, FAKE, 2, 2, 4, 128, 128, 0, 1.0, FAKE, FAKE, None]
    for idx, val, status in [(5, 0, 1), (7, 3, 1), (8, 32, 2), (10, 9, 1), (11, -1.0, 1), (12, None, 1), (0, None, 1)]:
        args = list(base)
        args[idx] = val
        st = lib.tr_gdn_decode(*args)
        assert st == status and "tr_gdn_decode" in lib.tr_last_error().decode(), (idx, val)
