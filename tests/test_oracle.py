"""Pins for the fp64 GDN oracle (CPU only).

Each test checks the oracle against something other than its own formula: a
closed form, an invariant of the recurrence, a textbook special case, or an
independent implementation.  Recurrence: reading notes "Tail-Replay：混合 LLM
前缀缓存的短尾重放机制", section 2.3, Eq. (1) (state stored dv x dk, operator
applied from the right); read-out o_t = S_t q_t after the update (the pages print
none; this is the plain reading).

Shapes deliberately use dv != dk so that a transposed state or operand fails.
"""
import numpy as np
import pytest

import oracle

RNG = np.random.default_rng(1234)


def unit_rows(n, d, rng=RNG):
    x = rng.standard_normal((n, d))
    return x / np.linalg.norm(x, axis=1, keepdims=True)


def one_seq(T, dk, dv, rng=RNG, beta=None, g=None, unit_k=True):
    q = rng.standard_normal((T, 1, dk))
    k = (unit_rows(T, dk, rng) if unit_k else rng.standard_normal((T, dk)))[:, None, :]
    v = rng.standard_normal((T, 1, dv))
    if g is None:
        g = -np.log1p(np.exp(rng.standard_normal((T, 1)) - 1.0))
    if beta is None:
        beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, 1))))
    return q, k, v, np.asarray(g, float).reshape(T, 1), np.asarray(beta, float).reshape(T, 1)


def cu(*lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


def test_beta_zero_is_pure_decay():
    # beta = 0: S_m = (prod alpha) S_a and o_t = (prod_{u<=t} alpha_u) S_a q_t (post-update read-out)
    T, dk, dv = 37, 7, 5
    q, k, v, g, _ = one_seq(T, dk, dv)
    beta = np.zeros((T, 1))
    Sa = RNG.standard_normal((1, 1, dv, dk))
    S, o = oracle.gdn(q, k, v, g, beta, cu(T), q_scale=0.75, state_in=Sa)
    decay = np.exp(np.cumsum(g[:, 0]))
    np.testing.assert_allclose(S[0, 0], decay[-1] * Sa[0, 0], rtol=1e-13, atol=1e-15)
    expect_o = decay[:, None] * (0.75 * (q[:, 0, :] @ Sa[0, 0].T))
    np.testing.assert_allclose(o[:, 0, :], expect_o, rtol=1e-12, atol=1e-14)


def test_orthonormal_recall():
    # alpha = beta = 1, orthonormal keys, zero start: S = sum_i v_i k_i^T, so S k_j = v_j.
    dk, dv = 8, 5
    Q, _ = np.linalg.qr(RNG.standard_normal((dk, dk)))
    keys = Q.T                                  # rows orthonormal
    T = dk
    v = RNG.standard_normal((T, 1, dv))
    k = keys[:, None, :]
    q = keys[:, None, :].copy()                 # read each token's own key back
    S, o = oracle.gdn(q, k, v, np.zeros((T, 1)), np.ones((T, 1)), cu(T))
    np.testing.assert_allclose(S[0, 0], v[:, 0, :].T @ keys, atol=1e-13)
    np.testing.assert_allclose(S[0, 0] @ keys.T, v[:, 0, :].T, atol=1e-13)
    # post-update read-out of the key just written returns its value exactly
    np.testing.assert_allclose(o[:, 0, :], v[:, 0, :], atol=1e-13)


def test_single_step_on_key_and_complement():
    # One token with a unit key fixes the new state completely through two facts:
    #   S_t k   = alpha (1 - beta) S_{t-1} k + beta v     (the key direction)
    #   S_t x   = alpha S_{t-1} x      for every x orthogonal to k
    dk, dv = 9, 4
    for beta_val in (0.0, 0.3, 1.0, 1.7, 2.0):
        q, k, v, g, _ = one_seq(1, dk, dv)
        beta = np.array([[beta_val]])
        S0 = RNG.standard_normal((1, 1, dv, dk))
        S, _ = oracle.gdn(q, k, v, g, beta, cu(1), state_in=S0)
        a = np.exp(g[0, 0])
        kk = k[0, 0]
        np.testing.assert_allclose(S[0, 0] @ kk, a * (1 - beta_val) * (S0[0, 0] @ kk) + beta_val * v[0, 0],
                                   rtol=1e-12, atol=1e-13)
        basis = np.linalg.svd(kk[None, :])[2][1:]          # orthonormal complement of k
        np.testing.assert_allclose(S[0, 0] @ basis.T, a * (S0[0, 0] @ basis.T), rtol=1e-12, atol=1e-13)


def test_linearity_and_transition_operator():
    # F(S_a, v) = S_a Phi + F(0, v) with Phi = T_{a+1} ... T_m = F(I, v = 0) (notes section 2.3
    # derivation: S_m = (T_m...T_{a+1}) S_a + S_hat_m, written here in the dv x dk layout).
    T, dk, dv = 29, 6, 4
    q, k, v, g, beta = one_seq(T, dk, dv, unit_k=False)
    Sa = RNG.standard_normal((1, 1, dv, dk))
    S_full, o_full = oracle.gdn(q, k, v, g, beta, cu(T), state_in=Sa)
    S_hat, o_hat = oracle.gdn(q, k, v, g, beta, cu(T))
    S_err, o_err = oracle.gdn(q, k, np.zeros_like(v), g, beta, cu(T), state_in=Sa)
    np.testing.assert_allclose(S_full, S_hat + S_err, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(o_full, o_hat + o_err, rtol=1e-12, atol=1e-12)
    # Phi from the identity start with a square state
    q2 = q.copy()
    Phi, _ = oracle.gdn(q2, k, np.zeros((T, 1, dk)), g, beta, cu(T), state_in=np.eye(dk)[None, None])
    np.testing.assert_allclose(S_err[0, 0], Sa[0, 0] @ Phi[0, 0], rtol=1e-12, atol=1e-12)
    # the error term is exactly the dropped state carried through the tail
    np.testing.assert_allclose(S_full[0, 0] - S_hat[0, 0], Sa[0, 0] @ Phi[0, 0], rtol=1e-11, atol=1e-12)


def test_contraction_bound():
    # unit keys, beta in [0, 2], v = 0: ||S_m||_F <= (prod alpha) ||S_a||_F (notes section 2.3)
    T, dk, dv = 50, 8, 6
    for trial in range(5):
        q, k, v, g, _ = one_seq(T, dk, dv)
        beta = RNG.uniform(0.0, 2.0, size=(T, 1))
        Sa = RNG.standard_normal((1, 1, dv, dk))
        S, _ = oracle.gdn(q, k, np.zeros_like(v), g, beta, cu(T), state_in=Sa)
        bound = np.exp(np.sum(g)) * np.linalg.norm(Sa)
        assert np.linalg.norm(S) <= bound * (1 + 1e-12)
    # with non-unit keys (beta |k|^2 > 2) the operator can expand: the bound is a real condition
    q, k, v, g, _ = one_seq(T, dk, dv)
    S, _ = oracle.gdn(q, 3.0 * k, np.zeros_like(v), np.zeros((T, 1)), np.ones((T, 1)), cu(T), state_in=Sa)
    assert np.linalg.norm(S) > np.linalg.norm(Sa)


def test_householder_product():
    # alpha = 1, beta = 2, unit keys, v = 0: each step right-multiplies by the Householder
    # reflector H_i = I - 2 k_i k_i^T, so S_m = S_a H_1 H_2 ... H_m and the norm is preserved.
    T, dk, dv = 12, 7, 3
    q, k, v, _, _ = one_seq(T, dk, dv)
    Sa = RNG.standard_normal((1, 1, dv, dk))
    S, _ = oracle.gdn(q, k, np.zeros_like(v), np.zeros((T, 1)), 2 * np.ones((T, 1)), cu(T), state_in=Sa)
    P = np.eye(dk)
    for t in range(T):
        kk = k[t, 0]
        P = P @ (np.eye(dk) - 2.0 * np.outer(kk, kk))
    np.testing.assert_allclose(S[0, 0], Sa[0, 0] @ P, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(np.linalg.norm(S), np.linalg.norm(Sa), rtol=1e-12)


def test_scalar_case_closed_form():
    # dk = dv = 1: s_t = a_t s_{t-1} + b_t with a_t = alpha_t (1 - beta_t k_t^2), b_t = beta_t v_t k_t,
    # whose solution is s_m = (prod a) s_0 + sum_j (prod_{u>j} a_u) b_j.
    T = 40
    q, k, v, g, beta = one_seq(T, 1, 1, unit_k=False)
    s0 = np.array([[[[0.8]]]])
    S, o = oracle.gdn(q, k, v, g, beta, cu(T), state_in=s0)
    a = np.exp(g[:, 0]) * (1 - beta[:, 0] * k[:, 0, 0] ** 2)
    b = beta[:, 0] * v[:, 0, 0] * k[:, 0, 0]
    expect = np.prod(a) * 0.8 + sum(np.prod(a[j + 1:]) * b[j] for j in range(T))
    np.testing.assert_allclose(S[0, 0, 0, 0], expect, rtol=1e-12)


def test_state_passing_split():
    # F(x[0:n]) = F(x[p:n], state = F(x[0:p]).S) for any split point p
    T, dk, dv = 45, 6, 5
    q, k, v, g, beta = one_seq(T, dk, dv)
    S_all, o_all = oracle.gdn(q, k, v, g, beta, cu(T))
    for p in (0, 1, 17, 44, 45):
        S1, o1 = oracle.gdn(q[:p], k[:p], v[:p], g[:p], beta[:p], cu(p))
        S2, o2 = oracle.gdn(q[p:], k[p:], v[p:], g[p:], beta[p:], cu(T - p), state_in=S1)
        np.testing.assert_allclose(S2, S_all, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(np.concatenate([o1, o2]), o_all, rtol=1e-12, atol=1e-13)


def test_packing_and_head_mapping():
    # Packed varlen with grouped heads equals per-sequence, per-head single calls where
    # value head h reads query/key head h // (Hv / Hqk).
    lens = (5, 0, 11, 3)
    T, Hqk, Hv, dk, dv = sum(lens), 2, 6, 4, 3
    q = RNG.standard_normal((T, Hqk, dk))
    k = unit_rows(T * Hqk, dk).reshape(T, Hqk, dk)
    v = RNG.standard_normal((T, Hv, dv))
    g = -RNG.uniform(0.0, 0.5, size=(T, Hv))
    beta = RNG.uniform(0.0, 1.0, size=(T, Hv))
    S0 = RNG.standard_normal((len(lens), Hv, dv, dk))
    S, o = oracle.gdn(q, k, v, g, beta, cu(*lens), q_scale=0.5, state_in=S0)
    c = cu(*lens)
    for b in range(len(lens)):
        sl = slice(c[b], c[b + 1])
        for h in range(Hv):
            j = h // (Hv // Hqk)
            Sb, ob = oracle.gdn(q[sl, j:j + 1], k[sl, j:j + 1], v[sl, h:h + 1], g[sl, h:h + 1],
                                beta[sl, h:h + 1], cu(lens[b]), q_scale=0.5, state_in=S0[b:b + 1, h:h + 1])
            np.testing.assert_array_equal(Sb[0, 0], S[b, h])
            np.testing.assert_array_equal(ob[:, 0], o[sl, h])
    # the empty sequence leaves its state untouched
    np.testing.assert_array_equal(S[1], S0[1])


def test_matches_independent_mirror():
    lens = (7, 13)
    T, Hqk, Hv, dk, dv = sum(lens), 1, 2, 5, 4
    q = RNG.standard_normal((T, Hqk, dk))
    k = unit_rows(T, dk).reshape(T, 1, dk)
    v = RNG.standard_normal((T, Hv, dv))
    g = -RNG.uniform(0.0, 1.0, size=(T, Hv))
    beta = RNG.uniform(0.0, 2.0, size=(T, Hv))
    S0 = RNG.standard_normal((2, Hv, dv, dk))
    S, o = oracle.gdn(q, k, v, g, beta, cu(*lens), q_scale=1.3, state_in=S0)
    Sm, om = oracle.gdn_mirror(q, k, v, g, beta, cu(*lens), q_scale=1.3, state_in=S0)
    np.testing.assert_allclose(S, Sm, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(o, om, rtol=1e-12, atol=1e-12)


def test_q_scale_only_scales_outputs():
    T, dk, dv = 20, 6, 6
    q, k, v, g, beta = one_seq(T, dk, dv)
    S1, o1 = oracle.gdn(q, k, v, g, beta, cu(T), q_scale=1.0)
    S2, o2 = oracle.gdn(q, k, v, g, beta, cu(T), q_scale=0.125)
    np.testing.assert_array_equal(S1, S2)
    np.testing.assert_allclose(o2, 0.125 * o1, rtol=1e-14)


def test_rejects_bad_head_grouping():
    q = np.zeros((2, 2, 4)); v = np.zeros((2, 3, 4)); gb = np.zeros((2, 3))
    with pytest.raises(RuntimeError):
        oracle.gdn(q, q, v, gb, gb, cu(2))
