"""A numpy model of the chunked bf16 GDN replay's rounding points (test infrastructure).

The library's bf16 path evaluates the recurrence of reading notes "Tail-Replay：混合 LLM 前缀缓存
的短尾重放机制", section 2.3, Eq. (1), in 64-token chunks (the WY form): per chunk, with gamma
the in-chunk cumulative log decay,
    L     = strictly lower part of diag(beta) (K K^T) o exp(gamma_i - gamma_j)
    A     = (I + L)^{-1}                       (diagonal 16x16 blocks, then block merges)
    U0    = A diag(beta) V,   W = A diag(beta e^gamma) K
    U'    = U0 - W S^T
    O     = diag(q_scale e^gamma) Q S^T + P U',  P = q_scale (Q K^T) o exp(gamma_i - gamma_j), j <= i
    S    <- e^{gamma_last} S + U'^T diag(exp(gamma_last - gamma)) K.
This model follows those steps with a rounding switch at each place where the kernel rounds
(bf16 MFMA operands, fp32 accumulation), so that the effect of each precision choice can be
measured on the CPU against the fp64 oracle:
  "exact"    no rounding at all (fp64): checks the chunked algebra itself;
  "plan"     the kernel's plan: fp32 accumulation, the diagonal inverse blocks to fp32
             accuracy, A's unit diagonal applied exactly in fp32, P and U' split hi / lo in
             P U', U' diag(dec) split hi / lo in the state update, S single bf16 in W S^T
             and Q S^T, outputs stored as bf16;
  "all_bf16" every matrix operand rounded once to bf16, the unit diagonal folded into the
             bf16 operands, no hi / lo splits (outputs stored as bf16);
and, with mode "plan", `drop` takes single choices out of the plan.
It shares nothing with the HIP sources; only the oracle's rounding helpers are used.
"""
from __future__ import annotations

import numpy as np

from oracle.rounding import round_bf16, round_f32

CH = 64          # tokens per chunk (the kernel's); chunk_replay takes others for the algebra pin
BLK = 16         # diagonal block size of the inverse


def _ident(x):
    return np.asarray(x, dtype=np.float64)


def _split(x, b):
    """hi / lo bf16 pair of an fp32 array: x ~ hi + lo."""
    hi = b(x)
    return hi, b(x - hi)


def _inverse(L, f, b, mode):
    CH = L.shape[0]
    """A = (I + L)^{-1} for a strictly lower triangular 64x64 L: the 16x16 diagonal blocks
    first, then block column j of A - I by merges A_ij = -A_ii sum_{k=j}^{i-1} L_ik A_kj.
    Returns N = A - I (fp32 values) as the kernel forms it."""
    n_b = CH // BLK
    blk = lambda M, i, j: M[BLK * i:BLK * (i + 1), BLK * j:BLK * (j + 1)]  # noqa: E731
    I16 = np.eye(BLK)
    N = np.zeros((CH, CH))
    D = []
    for i in range(n_b):
        Di = np.linalg.inv(I16 + blk(L, i, i))          # fp32-accurate (hi / lo products on the GPU)
        Di = Di if mode == "exact" else f(Di)
        D.append(Di)
        blk(N, i, i)[...] = np.tril(Di, -1)
    Db = [b(Di) for Di in D]                            # bf16 merge operands
    Lb = b(L)                                           # off-diagonal blocks of L in bf16
    for j in range(n_b - 1):
        Aj = {j: Db[j]}
        for i in range(j + 1, n_b):
            acc = f(sum(blk(Lb, i, kk) @ Aj[kk] for kk in range(j, i)))
            t = b(-acc)
            full = f(Db[i] @ t)                         # block (i, j) of A - I, fp32
            blk(N, i, j)[...] = full
            Aj[i] = b(full)
    return N


def chunk_replay(q, k, v, g, beta, q_scale=1.0, mode="plan", state=None, drop=(), ch=CH):
    """Replay one (sequence, head) in chunks.  q, k: [T, dk]; v: [T, dv]; g, beta: [T]
    (values exactly representable, e.g. bf16 inputs as float64).  Returns (S [dv, dk], O [T, dv]).
    `ch` is the chunk length (a multiple of 16; the kernel's is 64).
    `drop` takes single choices out of the plan: "unit_diag" (fold A's unit diagonal into the
    bf16 operands), "split_pu" (P and U' single bf16 in P U'), "split_update" (U' diag(dec)
    single bf16 in the state update)."""
    if mode == "all_bf16":
        mode, drop = "plan", ("unit_diag", "split_pu", "split_update")
    if mode == "exact":
        f = b = _ident
    else:
        f, b = round_f32, round_bf16
    T, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dv, dk)) if state is None else np.array(state, dtype=np.float64)
    O = np.zeros((T, dv))
    CH = ch
    for c0 in range(0, T, CH):
        n = min(CH, T - c0)
        qc = np.zeros((CH, dk)); kc = np.zeros((CH, dk)); vc = np.zeros((CH, dv))
        gc = np.zeros(CH); bc = np.zeros(CH)
        qc[:n], kc[:n], vc[:n], gc[:n], bc[:n] = q[c0:c0 + n], k[c0:c0 + n], v[c0:c0 + n], g[c0:c0 + n], beta[c0:c0 + n]
        gam = f(np.cumsum(gc)) if mode == "exact" else np.cumsum(gc.astype(np.float32)).astype(np.float64)
        eg = f(np.exp(gam))
        decay = f(np.exp(gam[:, None] - gam[None, :]))   # exp(gamma_i - gamma_j)
        raw = f(kc @ kc.T)
        L = f(np.tril(bc[:, None] * decay * raw, -1))
        bg = f(bc * eg)
        if "unit_diag" in drop:
            A = np.eye(CH) + _inverse(L, f, b, mode)
            U0 = f(b(A * bc[None, :]) @ vc)
            Wn = b(-f(b(A * bg[None, :]) @ kc))
        else:
            N = _inverse(L, f, b, mode)
            Nb, Nbg = b(N * bc[None, :]), b(N * bg[None, :])
            U0 = f(Nb @ vc + bc[:, None] * vc)           # unit diagonal exactly, in fp32
            Wn = b(-f(Nbg @ kc + bg[:, None] * kc))
        Sb = b(S)
        Up = f(U0 + Wn @ Sb.T)                           # U' = U0 - W S^T
        Y = f(qc @ Sb.T)
        P = f(q_scale * np.tril(f(qc @ kc.T) * decay))
        qeg = f(q_scale * eg)
        if mode == "plan" and "split_pu" not in drop:
            Ph, Pl = _split(P, b)
            Uh, Ul = _split(Up, b)
            PU = f(Ph @ Uh + Ph @ Ul + Pl @ Uh)
        else:
            PU = f(b(P) @ b(Up))
        O[c0:c0 + n] = b(f(qeg[:, None] * Y + PU))[:n]
        dec = f(np.exp(gam[-1] - gam))
        X = f(Up * dec[:, None])
        if mode == "plan" and "split_update" not in drop:
            Xh, Xl = _split(X, b)
            upd = f(Xh.T @ kc + Xl.T @ kc)
        else:
            upd = f(b(X).T @ kc)
        S = f(eg[-1] * S + upd)
    return S, O
