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
                B=2, T=9, Hqk=2, Hv=4, dk=128, dv=128, dt=0, q_scale=1.0, s_in=None, s_out=FAKE, o=FAKE)
    args.update(over)
    lib = L.lib()
    st = lib.tr_gdn_replay(args["q"], args["k"], args["v"], args["g"], args["beta"], args["cu_h"], args["cu_d"],
                           args["B"], args["T"], args["Hqk"], args["Hv"], args["dk"], args["dv"], args["dt"],
                           args["q_scale"], args["s_in"], args["s_out"], args["o"], None)
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


def test_gdn_rejects_bad_cu_seqlens():
    for bad in ((1, 5, 9), (0, 6, 5)):
        cu = (ctypes.c_int32 * 3)(*bad)
        st, msg = call_gdn(cu_h=ctypes.cast(cu, ctypes.c_void_p), T=bad[-1])
        assert st == 1 and "cu_seqlens" in msg
