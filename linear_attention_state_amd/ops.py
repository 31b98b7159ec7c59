"""Python binding of the Tail-Replay C ABI (argument marshalling only).

Every function checks tensor dtypes, shapes and devices, allocates outputs with torch
(device memory and streams are all torch provides), and calls the matching
``tr_*`` entry point on the current torch stream.  All arithmetic runs in the HIP
library.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import torch

from ._lib import LaWeights, TR_BF16, TR_F32, check, lib

_DT = {torch.bfloat16: TR_BF16, torch.float32: TR_F32}


def _ptr(t: Optional[torch.Tensor]):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def tail_length(m: int, r_num: int, r_den: int) -> int:
    """k = ceil(m r_num / r_den) replayed tokens for a hit of m matched tokens."""
    k = lib().tr_tail_length(int(m), int(r_num), int(r_den))
    if k < 0:
        raise ValueError(lib().tr_last_error().decode())
    return int(k)


def tail_seqlens(m: Sequence[int], r_num: int, r_den: int):
    """Packed tail offsets for several hits: (cu_seqlens [B+1] int32, tail starts [B] int64), host."""
    mm = torch.tensor(list(m), dtype=torch.int64)
    cu = torch.empty(len(m) + 1, dtype=torch.int32)
    starts = torch.empty(len(m), dtype=torch.int64)
    check(lib().tr_tail_seqlens(_ptr(mm), len(m), int(r_num), int(r_den), _ptr(cu), _ptr(starts)))
    return cu, starts


_SCHEDULES = {"auto": 0, "fused": 1, "split": 2}


def set_gdn_schedule(schedule: str) -> None:
    """Process-wide schedule of the bf16 recurrence: "auto" (split for few heads), "fused"
    or "split" (tr_gdn_set_schedule)."""
    _need(schedule in _SCHEDULES, "schedule must be one of %s" % sorted(_SCHEDULES))
    check(lib().tr_gdn_set_schedule(_SCHEDULES[schedule]))


def get_gdn_schedule() -> str:
    code = lib().tr_gdn_get_schedule()
    return {v: k for k, v in _SCHEDULES.items()}[code]


def gdn_replay_workspace_size(cu_seqlens, Hqk: int, Hv: int, dk: int, dv: int, dtype) -> int:
    """Bytes of workspace tr_gdn_replay needs for this request (0 for none)."""
    cu = cu_seqlens.to(torch.int32).cpu().contiguous()
    n = lib().tr_gdn_replay_workspace_size(_ptr(cu), cu.numel() - 1, Hqk, Hv, dk, dv, _DT[dtype])
    msg = lib().tr_last_error().decode()
    _need(not msg, msg)
    return int(n)


def gdn_replay(q, k, v, g, beta, cu_seqlens, q_scale: float = 1.0, state_in=None,
               want_o: bool = True, cu_seqlens_dev=None, state_out=None, o=None, workspace=None, stream=None):
    """Varlen GDN recurrence (tr_gdn_replay).  Returns (state_out [B,Hv,dv,dk] fp32, o or None).

    q, k [T, Hqk, dk], v [T, Hv, dv] in bf16 (chunked MFMA path) or fp32; g, beta [T, Hv]
    fp32; cu_seqlens [B+1] int32 on the host; state_in optional [B, Hv, dv, dk] fp32.
    workspace: a uint8 device tensor of at least gdn_replay_workspace_size() bytes, or None
    to allocate one when the schedule needs it.
    """
    _need(q.is_cuda and k.is_cuda and v.is_cuda and g.is_cuda and beta.is_cuda, "inputs must be on the GPU")
    _need(q.dtype == k.dtype == v.dtype and q.dtype in _DT, "q, k, v must share dtype bf16 or fp32")
    _need(g.dtype == torch.float32 and beta.dtype == torch.float32, "g and beta must be fp32")
    for t in (q, k, v, g, beta):
        _need(t.is_contiguous(), "inputs must be contiguous")
    _need(q.dim() == 3 and k.shape == q.shape and v.dim() == 3, "q, k: [T, Hqk, dk]; v: [T, Hv, dv]")
    T, Hqk, dk = q.shape
    _, Hv, dv = v.shape
    _need(v.shape[0] == T and g.shape == (T, Hv) and beta.shape == (T, Hv), "shape mismatch")
    cu = cu_seqlens.to(torch.int32).cpu().contiguous()
    B = cu.numel() - 1
    if cu_seqlens_dev is None:
        cu_seqlens_dev = cu.to(q.device)
    _need(cu_seqlens_dev.dtype == torch.int32 and cu_seqlens_dev.numel() == B + 1, "cu_seqlens_dev")
    if state_in is not None:
        _need(state_in.is_cuda and state_in.dtype == torch.float32 and state_in.is_contiguous()
              and tuple(state_in.shape) == (B, Hv, dv, dk), "state_in must be [B, Hv, dv, dk] fp32")
    if state_out is None:
        state_out = torch.empty((B, Hv, dv, dk), dtype=torch.float32, device=q.device)
    if want_o and o is None:
        o = torch.empty((T, Hv, dv), dtype=q.dtype, device=q.device)
    if not want_o:
        o = None
    if workspace is None:
        need = lib().tr_gdn_replay_workspace_size(_ptr(cu), B, Hqk, Hv, dk, dv, _DT[q.dtype])
        if need:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0
    if workspace is not None:
        _need(workspace.is_cuda and workspace.is_contiguous(), "workspace must be a contiguous device tensor")
        ws_bytes = workspace.numel() * workspace.element_size()
    st = lib().tr_gdn_replay(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu), _ptr(cu_seqlens_dev),
                             B, T, Hqk, Hv, dk, dv, _DT[q.dtype], float(q_scale),
                             _ptr(state_in), _ptr(state_out), _ptr(o), _ptr(workspace), ws_bytes, _stream(stream))
    check(st)
    return state_out, o


def gdn_replay_noalloc(q, k, v, g, beta, cu_seqlens, cu_seqlens_dev, state_out, o=None, q_scale: float = 1.0,
                       state_in=None, stream=None):
    """tr_gdn_replay_noalloc: tr_gdn_replay with the split schedule's records in the library's
    static device scratch.  Every buffer is the caller's (cu_seqlens on the host and its device
    copy, state_out [B, Hv, dv, dk] fp32, o [T, Hv, dv] or None for state-only); nothing is
    allocated.  Returns (state_out, o)."""
    _need(q.is_cuda and k.is_cuda and v.is_cuda and g.is_cuda and beta.is_cuda, "inputs must be on the GPU")
    _need(q.dtype == k.dtype == v.dtype and q.dtype in _DT, "q, k, v must share dtype bf16 or fp32")
    _need(g.dtype == torch.float32 and beta.dtype == torch.float32, "g and beta must be fp32")
    for t in (q, k, v, g, beta):
        _need(t.is_contiguous(), "inputs must be contiguous")
    _need(q.dim() == 3 and k.shape == q.shape and v.dim() == 3, "q, k: [T, Hqk, dk]; v: [T, Hv, dv]")
    T, Hqk, dk = q.shape
    _, Hv, dv = v.shape
    _need(v.shape[0] == T and g.shape == (T, Hv) and beta.shape == (T, Hv), "shape mismatch")
    _need(cu_seqlens.device.type == "cpu" and cu_seqlens.dtype == torch.int32 and cu_seqlens.is_contiguous(),
          "cu_seqlens: int32 on the host")
    B = cu_seqlens.numel() - 1
    _need(cu_seqlens_dev.is_cuda and cu_seqlens_dev.dtype == torch.int32 and cu_seqlens_dev.numel() == B + 1,
          "cu_seqlens_dev: its int32 device copy")
    _need(state_out.is_cuda and state_out.dtype == torch.float32 and state_out.is_contiguous()
          and tuple(state_out.shape) == (B, Hv, dv, dk), "state_out must be [B, Hv, dv, dk] fp32")
    if state_in is not None:
        _need(state_in.is_cuda and state_in.dtype == torch.float32 and state_in.is_contiguous()
              and tuple(state_in.shape) == (B, Hv, dv, dk), "state_in must be [B, Hv, dv, dk] fp32")
    if o is not None:
        _need(o.is_cuda and o.dtype == q.dtype and o.is_contiguous() and tuple(o.shape) == (T, Hv, dv),
              "o must be [T, Hv, dv] in the input dtype")
    check(lib().tr_gdn_replay_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens),
                                      _ptr(cu_seqlens_dev), B, T, Hqk, Hv, dk, dv, _DT[q.dtype], float(q_scale),
                                      _ptr(state_in), _ptr(state_out), _ptr(o), _stream(stream)))
    return state_out, o


def gdn_transition_workspace_size(cu_seqlens, Hqk: int, Hv: int, d: int, dtype) -> int:
    """Bytes of workspace tr_gdn_transition needs for this request (0 for none)."""
    cu = cu_seqlens.to(torch.int32).cpu().contiguous()
    n = lib().tr_gdn_transition_workspace_size(_ptr(cu), cu.numel() - 1, Hqk, Hv, d, _DT[dtype])
    msg = lib().tr_last_error().decode()
    _need(not msg, msg)
    return int(n)


def gdn_transition(k, g, beta, cu_seqlens, cu_seqlens_dev=None, phi_out=None, separate_decay: bool = False,
                   workspace=None, stream=None):
    """Transition products of the packed spans (tr_gdn_transition): the recurrence from S = I
    with zero values.  k [T, Hqk, d] bf16 or fp32; g, beta [T, Hv] fp32.  Returns Phi
    [B, Hv, d, d], or with separate_decay (phi, log_scale [B, Hv]) where Phi = exp(log_scale) phi.
    workspace: a uint8 device tensor of at least gdn_transition_workspace_size() bytes, or None
    to allocate one when the request needs it."""
    _need(k.is_cuda and g.is_cuda and beta.is_cuda, "inputs must be on the GPU")
    _need(k.dtype in _DT and g.dtype == torch.float32 and beta.dtype == torch.float32, "dtypes")
    for t in (k, g, beta):
        _need(t.is_contiguous(), "inputs must be contiguous")
    _need(k.dim() == 3, "k: [T, Hqk, d]")
    T, Hqk, d = k.shape
    _need(g.dim() == 2 and g.shape[0] == T and beta.shape == g.shape, "g, beta: [T, Hv]")
    Hv = g.shape[1]
    cu = cu_seqlens.to(torch.int32).cpu().contiguous()
    B = cu.numel() - 1
    if cu_seqlens_dev is None:
        cu_seqlens_dev = cu.to(k.device)
    if phi_out is None:
        phi_out = torch.empty((B, Hv, d, d), dtype=torch.float32, device=k.device)
    _need(phi_out.is_cuda and phi_out.dtype == torch.float32 and phi_out.is_contiguous()
          and tuple(phi_out.shape) == (B, Hv, d, d), "phi_out must be [B, Hv, d, d] fp32")
    log_scale = torch.empty((B, Hv), dtype=torch.float32, device=k.device) if separate_decay else None
    if workspace is None:
        need = lib().tr_gdn_transition_workspace_size(_ptr(cu), B, Hqk, Hv, d, _DT[k.dtype])
        if need:
            workspace = torch.empty(need, dtype=torch.uint8, device=k.device)
    ws_bytes = 0
    if workspace is not None:
        _need(workspace.is_cuda and workspace.is_contiguous(), "workspace must be a contiguous device tensor")
        ws_bytes = workspace.numel() * workspace.element_size()
    check(lib().tr_gdn_transition(_ptr(k), _ptr(g), _ptr(beta), _ptr(cu), _ptr(cu_seqlens_dev),
                                  B, T, Hqk, Hv, d, _DT[k.dtype], _ptr(phi_out), _ptr(log_scale),
                                  _ptr(workspace), ws_bytes, _stream(stream)))
    return (phi_out, log_scale) if separate_decay else phi_out


def state_compose(S_c, phi, S_hat=None, out=None, log_scale=None, stream=None):
    """out = exp(log_scale) S_c @ phi (+ S_hat) over the leading dimensions (tr_state_compose), fp32."""
    _need(S_c.is_cuda and S_c.dtype == torch.float32 and S_c.is_contiguous(), "S_c: fp32 contiguous on the GPU")
    dv, dk = S_c.shape[-2], S_c.shape[-1]
    N = S_c.numel() // (dv * dk)
    _need(phi.is_cuda and phi.dtype == torch.float32 and phi.is_contiguous()
          and tuple(phi.shape) == tuple(S_c.shape[:-2]) + (dk, dk), "phi: [..., dk, dk] fp32")
    if S_hat is not None:
        _need(S_hat.is_cuda and S_hat.dtype == torch.float32 and S_hat.is_contiguous()
              and S_hat.shape == S_c.shape, "S_hat: same shape as S_c")
    if log_scale is not None:
        _need(log_scale.is_cuda and log_scale.dtype == torch.float32 and log_scale.is_contiguous()
              and log_scale.numel() == N, "log_scale: one fp32 per matrix")
    if out is None:
        out = torch.empty_like(S_c)
    _need(out.is_cuda and out.dtype == torch.float32 and out.is_contiguous() and out.shape == S_c.shape, "out")
    check(lib().tr_state_compose(_ptr(S_c), _ptr(phi), _ptr(log_scale), _ptr(S_hat), _ptr(out), N, dv, dk,
                                 _stream(stream)))
    return out


def gdn_decode(q, k, v, g, beta, state, q_scale: float = 1.0, want_o: bool = True, o=None, stream=None):
    """One recurrence step per (sequence, value head), state updated in place (tr_gdn_decode).
    q, k [B, Hqk, dk], v [B, Hv, dv] bf16 or fp32; g, beta [B, Hv] fp32; state [B, Hv, dv, dk]."""
    _need(q.is_cuda and k.is_cuda and v.is_cuda and g.is_cuda and beta.is_cuda and state.is_cuda, "GPU tensors")
    _need(q.dtype == k.dtype == v.dtype and q.dtype in _DT, "q, k, v must share dtype bf16 or fp32")
    _need(g.dtype == torch.float32 and beta.dtype == torch.float32 and state.dtype == torch.float32, "fp32")
    for t in (q, k, v, g, beta, state):
        _need(t.is_contiguous(), "inputs must be contiguous")
    B, Hqk, dk = q.shape
    _, Hv, dv = v.shape
    _need(k.shape == q.shape and v.shape[0] == B and g.shape == (B, Hv) and beta.shape == (B, Hv)
          and tuple(state.shape) == (B, Hv, dv, dk), "shape mismatch")
    if want_o and o is None:
        o = torch.empty((B, Hv, dv), dtype=q.dtype, device=q.device)
    if not want_o:
        o = None
    check(lib().tr_gdn_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), B, Hqk, Hv, dk, dv,
                              _DT[q.dtype], float(q_scale), _ptr(state), _ptr(o), _stream(stream)))
    return o


def _weights_struct(w: dict) -> LaWeights:
    return LaWeights(w["w_qk"].data_ptr(), w["w_v"].data_ptr(), w["w_a"].data_ptr(), w["w_b"].data_ptr(),
                     w["w_o"].data_ptr() if w.get("w_o") is not None else None,
                     w["rms_gain"].data_ptr() if w.get("rms_gain") is not None else None)


def _check_weights(w: dict, d, Hqk, Hv, dk, dv, need_o):
    shapes = {"w_qk": (2 * Hqk * dk, d), "w_v": (Hv * dv, d), "w_a": (Hv, d), "w_b": (Hv, d)}
    if need_o:
        shapes["w_o"] = (d, Hv * dv)
    for name, shp in shapes.items():
        t = w[name]
        _need(t.is_cuda and t.dtype == torch.bfloat16 and t.is_contiguous() and tuple(t.shape) == shp,
              "%s must be contiguous bf16 %s on the GPU" % (name, shp))
    if w.get("rms_gain") is not None:
        t = w["rms_gain"]
        _need(t.is_cuda and t.dtype == torch.bfloat16 and t.numel() == d, "rms_gain must be bf16 [d_model]")


def la_layer_inputs(x, weights: Sequence[dict], Hqk, Hv, dk, dv, rms_eps=1e-6, stream=None):
    """Projections in front of one LA layer for G blocks (tr_la_layer_inputs).

    x [G, n, d_model] bf16; weights: G dicts.  Returns q, k, v (bf16), g, beta (fp32) with
    G*n rows each.
    """
    _need(x.is_cuda and x.dtype == torch.bfloat16 and x.is_contiguous() and x.dim() == 3, "x: [G, n, d] bf16")
    G, n, d = x.shape
    _need(len(weights) == G, "one weight set per block")
    for w in weights:
        _check_weights(w, d, Hqk, Hv, dk, dv, need_o=False)
    dev = x.device
    q = torch.empty((G * n, Hqk, dk), dtype=torch.bfloat16, device=dev)
    k = torch.empty_like(q)
    v = torch.empty((G * n, Hv, dv), dtype=torch.bfloat16, device=dev)
    g = torch.empty((G * n, Hv), dtype=torch.float32, device=dev)
    beta = torch.empty_like(g)
    ws = int(lib().tr_la_layer_inputs_workspace_size(G, n, d))
    work = torch.empty(max(ws, 1), dtype=torch.uint8, device=dev)
    structs = [_weights_struct(w) for w in weights]
    arr = (ctypes.POINTER(LaWeights) * G)(*[ctypes.pointer(s) for s in structs])
    check(lib().tr_la_layer_inputs(_ptr(x), ctypes.cast(arr, ctypes.c_void_p), G, n, d, Hqk, Hv, dk, dv,
                                   float(rms_eps), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                   _ptr(work), ws, _stream(stream)))
    return q, k, v, g, beta


def rmsnorm(x, gains: Sequence, rms_eps=1e-6, y=None, stream=None):
    """y = bf16(x / sqrt(mean(x^2) + eps) * gain) per block (tr_rmsnorm); gains: G tensors or None."""
    _need(x.is_cuda and x.dtype == torch.bfloat16 and x.is_contiguous() and x.dim() == 3, "x: [G, n, d] bf16")
    G, n, d = x.shape
    _need(len(gains) == G, "one gain (or None) per block")
    for t in gains:
        if t is not None:
            _need(t.is_cuda and t.dtype == torch.bfloat16 and t.numel() == d, "gain must be bf16 [d_model]")
    if y is None:
        y = torch.empty_like(x)
    arr = (ctypes.c_void_p * G)(*[t.data_ptr() if t is not None else None for t in gains])
    check(lib().tr_rmsnorm(_ptr(x), ctypes.cast(arr, ctypes.c_void_p), G, n, d, float(rms_eps), _ptr(y),
                           _stream(stream)))
    return y


def la_project(y, weights: Sequence[dict], Hqk, Hv, dk, dv, out=None, stream=None):
    """q, k, v, g, beta from a normalised hidden y [G, n, d] (tr_la_project)."""
    _need(y.is_cuda and y.dtype == torch.bfloat16 and y.is_contiguous() and y.dim() == 3, "y: [G, n, d] bf16")
    G, n, d = y.shape
    _need(len(weights) == G, "one weight set per block")
    for w in weights:
        _check_weights(w, d, Hqk, Hv, dk, dv, need_o=False)
    dev = y.device
    if out is None:
        out = (torch.empty((G * n, Hqk, dk), dtype=torch.bfloat16, device=dev),
               torch.empty((G * n, Hqk, dk), dtype=torch.bfloat16, device=dev),
               torch.empty((G * n, Hv, dv), dtype=torch.bfloat16, device=dev),
               torch.empty((G * n, Hv), dtype=torch.float32, device=dev),
               torch.empty((G * n, Hv), dtype=torch.float32, device=dev))
    q, k, v, g, beta = out
    structs = [_weights_struct(w) for w in weights]
    arr = (ctypes.POINTER(LaWeights) * G)(*[ctypes.pointer(s) for s in structs])
    check(lib().tr_la_project(_ptr(y), ctypes.cast(arr, ctypes.c_void_p), G, n, d, Hqk, Hv, dk, dv,
                              _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _stream(stream)))
    return out


def la_output_residual(x_in, o, weights: Sequence[dict], Hv, dv, x_out=None, stream=None):
    """x_out = bf16(x_in + o Wo^T) per block (tr_la_output_residual)."""
    _need(x_in.is_cuda and x_in.dtype == torch.bfloat16 and x_in.is_contiguous() and x_in.dim() == 3, "x_in")
    G, n, d = x_in.shape
    _need(o.is_cuda and o.dtype == torch.bfloat16 and o.is_contiguous() and o.numel() == G * n * Hv * dv, "o")
    _need(len(weights) == G, "one weight set per block")
    for w in weights:
        t = w["w_o"]
        _need(t.is_cuda and t.dtype == torch.bfloat16 and t.is_contiguous() and tuple(t.shape) == (d, Hv * dv), "w_o")
    if x_out is None:
        x_out = torch.empty_like(x_in)
    structs = [_weights_struct(w) for w in weights]
    arr = (ctypes.POINTER(LaWeights) * G)(*[ctypes.pointer(s) for s in structs])
    check(lib().tr_la_output_residual(_ptr(x_in), _ptr(o), ctypes.cast(arr, ctypes.c_void_p), G, n, d, Hv, dv,
                                      _ptr(x_out), _stream(stream)))
    return x_out


class GroupReplay:
    """Reusable tr_group_replay call: holds the weight table and the workspace."""

    def __init__(self, weights: Sequence[Sequence[dict]], n_tokens, d_model, Hqk, Hv, dk, dv,
                 rms_eps=1e-6, device="cuda"):
        self.G, self.L = len(weights), len(weights[0])
        self.dims = (n_tokens, d_model, Hqk, Hv, dk, dv)
        self.rms_eps = float(rms_eps)
        for gi, row in enumerate(weights):
            _need(len(row) == self.L, "every group needs L layers")
            for li, w in enumerate(row):
                _check_weights(w, d_model, Hqk, Hv, dk, dv, need_o=li < self.L - 1)
        self._structs = (LaWeights * (self.G * self.L))(
            *[_weights_struct(w) for row in weights for w in row])
        self._keep = weights
        ws = int(lib().tr_group_replay_workspace_size(self.G, self.L, n_tokens, d_model, Hqk, Hv, dk, dv))
        self.workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=device)
        self.ws_bytes = ws

    def __call__(self, h_tail, states_out=None, stream=None):
        n, d, Hqk, Hv, dk, dv = self.dims
        _need(h_tail.is_cuda and h_tail.dtype == torch.bfloat16 and h_tail.is_contiguous()
              and tuple(h_tail.shape) == (self.G, n, d), "h_tail must be [G, n, d_model] bf16")
        if states_out is None:
            states_out = torch.empty((self.G, self.L, Hv, dv, dk), dtype=torch.float32, device=h_tail.device)
        check(lib().tr_group_replay(_ptr(h_tail), ctypes.cast(self._structs, ctypes.c_void_p), self.G, self.L,
                                    n, d, Hqk, Hv, dk, dv, self.rms_eps, _ptr(states_out),
                                    _ptr(self.workspace), self.ws_bytes, _stream(stream)))
        return states_out


def group_replay(h_tail, weights, Hqk, Hv, dk, dv, rms_eps=1e-6):
    """One-shot tr_group_replay: states [G, L, Hv, dv, dk] fp32."""
    G, n, d = h_tail.shape
    return GroupReplay(weights, n, d, Hqk, Hv, dk, dv, rms_eps, device=h_tail.device)(h_tail)
