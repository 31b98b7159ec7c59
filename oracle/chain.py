"""Group-chain oracle: replay one group's LA layers from cached FA hiddens.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Method (reading notes "Tail-Replay：混合 LLM 前缀缓存的短尾重放机制", section 2.2
steps 2-3 and section 2.4): for every group, take the cached FA output hidden
vectors of the tail, h_{m-k+1..m}; start every LA layer of the group from a zero
state; run the hidden vectors through the group's LA layers in order; keep each
layer's boundary state.  Groups are independent.  Section 2.5: the FFN after the
group's last layer is not needed; the pages give no FFN shape, so no FFN is
modelled, and the last layer's output projection and residual are dead work too.

Layer body (the pages name only k_i, v_i, alpha_i, beta_i as "produced by the
in-group computation", section 2.1 symbol table; the body below is the plainest
Gated DeltaNet layer with the stated widths):

  y  = bf16( x / sqrt(mean(x^2) + eps) * gain )          RMSNorm, gain = 1 if absent
  q|k = y Wqk^T ;  v = bf16(y Wv^T) ;  za = y Wa^T ;  zb = y Wb^T
  q  = bf16( q_h / sqrt(|q_h|^2 + 1e-6) * dk^-1/2 )       per head h
  k  = bf16( k_h / sqrt(|k_h|^2 + 1e-6) )                 per head h
  g  = f32( -softplus(za) ) = f32(log alpha) ;  beta = f32( sigmoid(zb) )
  S, o = GDN recurrence from the zero state (``oracle.gdn``)
  x  <- bf16( x + bf16(o) Wo^T )                          all but the last layer

Weights are [out, in] row-major.  bf16(...) / f32(...) mark the points where the
library stores a tensor in that type; between them everything is float64.

Pins: tests/test_oracle_group.py checks the chain against a constructed case with
a closed-form answer (one-hot keys and saturated gates give exact key-value
recall), the projections on exact weights whose every output has a closed form
(orientation, head order, per-head L2 norm, q scale, gate maps against numpy's
logaddexp and scipy's expit), RMSNorm with a gain in closed form, RMSNorm / L2-norm
invariants, residual pass-through, scale invariance of the first layer, and gate
ranges.  Random-weight projections are otherwise numpy's float64 matmul.
"""
from __future__ import annotations

import numpy as np

from .rounding import round_bf16, round_f32

L2_EPS = 1e-6


def softplus(z):
    z = np.asarray(z, dtype=np.float64)
    return np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))


def sigmoid(z):
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(-np.abs(z))
    return np.where(z >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def rmsnorm(x, gain, eps):
    x = np.asarray(x, dtype=np.float64)
    y = x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    if gain is not None:
        y = y * np.asarray(gain, dtype=np.float64)
    return y


def l2norm_heads(x, n_heads, d_head):
    xs = x.reshape(x.shape[0], n_heads, d_head)
    return xs / np.sqrt(np.sum(xs * xs, axis=-1, keepdims=True) + L2_EPS)


def layer_inputs(x, w, Hqk, Hv, dk, dv, eps):
    """Projections of one LA layer: returns bf16-valued q, k, v and fp32-valued g, beta."""
    return project(round_bf16(rmsnorm(x, w.get("rms_gain"), eps)), w, Hqk, Hv, dk, dv)


def project(y, w, Hqk, Hv, dk, dv):
    """The projections of one LA layer from its normalised hidden y (bf16 values)."""
    y = np.asarray(y, dtype=np.float64)
    qk = y @ np.asarray(w["w_qk"], dtype=np.float64).T
    q = round_bf16(l2norm_heads(qk[:, : Hqk * dk], Hqk, dk) * dk ** -0.5)
    k = round_bf16(l2norm_heads(qk[:, Hqk * dk:], Hqk, dk))
    v = round_bf16(y @ np.asarray(w["w_v"], dtype=np.float64).T).reshape(-1, Hv, dv)
    za = y @ np.asarray(w["w_a"], dtype=np.float64).T
    zb = y @ np.asarray(w["w_b"], dtype=np.float64).T
    g = round_f32(-softplus(za))
    beta = round_f32(sigmoid(zb))
    return q, k, v, g, beta


def group(h_tail, weights, Hqk, Hv, dk, dv, rms_eps=1e-6, return_trace=False):
    """Replay every group's LA layers from its cached hidden vectors.

    h_tail: [G, n, d_model] (bf16 values); weights: list (len G) of lists (len L) of
    dicts with keys w_qk [2*Hqk*dk, d], w_v [Hv*dv, d], w_a [Hv, d], w_b [Hv, d],
    w_o [d, Hv*dv] and optional rms_gain [d].
    Returns states [G, L, Hv, dv, dk] (and, with return_trace, the per-layer inputs).
    """
    from . import gdn  # late import: the package initialises this module first

    h_tail = np.asarray(h_tail, dtype=np.float64)
    G, n, _ = h_tail.shape
    L = len(weights[0])
    states = np.zeros((G, L, Hv, dv, dk))
    trace = []
    cu = np.array([0, n], dtype=np.int32)
    for gi in range(G):
        x = h_tail[gi]
        tr = []
        for li in range(L):
            w = weights[gi][li]
            q, k, v, g, beta = layer_inputs(x, w, Hqk, Hv, dk, dv, rms_eps)
            last = li == L - 1
            S, o = gdn(q, k, v, g, beta, cu, q_scale=1.0, want_o=not last)
            states[gi, li] = S[0]
            if return_trace:
                tr.append(dict(x=x, q=q, k=k, v=v, g=g, beta=beta, o=o))
            if not last:
                ob = round_bf16(o).reshape(n, Hv * dv)
                x = round_bf16(x + ob @ np.asarray(w["w_o"], dtype=np.float64).T)
        trace.append(tr)
    return (states, trace) if return_trace else states
