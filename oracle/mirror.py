"""Independent numpy implementation of the GDN recurrence (test infrastructure only).

A second CPU implementation, written separately from ``gdn_oracle.c``, used to
cross-check the C code's pointer arithmetic (packing, head mapping, state layout)
on tiny shapes.  It forms the transition operator as an explicit dk x dk matrix,
T_t = alpha_t (I - beta_t k_t k_t^T), and applies it from the right to the
dv x dk state (reading notes "Tail-Replay：混合 LLM 前缀缓存的短尾重放机制",
section 2.3, Eq. (1) and the layout remark after it).  Cost is O(dk^2 dv) per
token, so keep shapes tiny.
"""
from __future__ import annotations

import numpy as np


def gdn_mirror(q, k, v, g, beta, cu_seqlens, q_scale=1.0, state_in=None):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    T, Hqk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    B = len(cu_seqlens) - 1
    group_size = Hv // Hqk
    states = np.zeros((B, Hv, dv, dk))
    outs = np.zeros((T, Hv, dv))
    eye = np.eye(dk)
    for b in range(B):
        for h in range(Hv):
            qk_head = h // group_size
            S = np.zeros((dv, dk)) if state_in is None else np.array(state_in[b, h], dtype=np.float64)
            for t in range(int(cu_seqlens[b]), int(cu_seqlens[b + 1])):
                kv = k[t, qk_head]
                trans = np.exp(g[t, h]) * (eye - beta[t, h] * np.outer(kv, kv))
                S = S @ trans + beta[t, h] * np.outer(v[t, h], kv)
                outs[t, h] = S @ (q_scale * q[t, qk_head])
            states[b, h] = S
    return states, outs
