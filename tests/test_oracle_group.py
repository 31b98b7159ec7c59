"""Pins for the group-chain oracle (CPU only).

The chain (reading notes "Tail-Replay：混合 LLM 前缀缓存的短尾重放机制", section 2.2
steps 2-3): every LA layer of a group starts from a zero state and the cached FA
hidden vectors run through the group's layers in order.  The layer body is the
one stated in oracle/chain.py.
"""
import numpy as np

import oracle
from oracle import chain as og

RNG = np.random.default_rng(77)


def _recall_case():
    """Two layers, d_model = 16, one head, dk = dv = 8, 8 tokens.

    Token t's hidden vector is 4 e_t.  Layer 1 reads key e_t and query e_{t-1}
    (query e_7 for t = 0); saturated gates make alpha = beta = 1 exactly, so the
    state is sum_t v_t e_t^T and o_t = s v_{t-1} (0 for t = 0), s = bf16(8^-1/2).
    W_o copies o into hidden dims 8..15.  Layer 2 reads the same keys and takes its
    values from dims 8..15, so its state column t is the RMS-normalised layer-1
    output of token t -- which needs the residual, its sign and the read-out order.
    """
    d, dk, n = 16, 8, 8
    V1 = RNG.choice([-4.0, -2.0, -1.0, 0.0, 1.0, 2.0, 4.0], size=(n, dk))
    h = np.zeros((1, n, d))
    h[0, np.arange(n), np.arange(n)] = 4.0
    wq = np.zeros((dk, d)); wk = np.zeros((dk, d))
    for t in range(n):
        wk[t, t] = 1.0
        wq[(t - 1) % n, t] = 1.0
    w1 = dict(w_qk=np.concatenate([wq, wk]), w_v=np.zeros((dk, d)),
              w_a=np.zeros((1, d)), w_b=np.zeros((1, d)), w_o=np.zeros((d, dk)))
    w1["w_v"][:, :n] = V1.T / 4.0
    w1["w_a"][0, :n] = -30.0
    w1["w_b"][0, :n] = 30.0
    w1["w_o"][8 + np.arange(dk), np.arange(dk)] = 1.0
    w2 = {k: v.copy() for k, v in w1.items()}
    w2["w_v"] = np.zeros((dk, d))
    w2["w_v"][np.arange(dk), 8 + np.arange(dk)] = 1.0
    return h, [[w1, w2]], V1


def test_recall_through_the_chain():
    h, weights, V1 = _recall_case()
    S = og.group(h, weights, Hqk=1, Hv=1, dk=8, dv=8)
    # layer 1: exact key-value recall
    np.testing.assert_array_equal(S[0, 0, 0], V1.T)
    # layer 2: column t is the normalised layer-1 output o_t = s v_{t-1} (o_0 = 0)
    s = oracle.round_bf16(np.array([8 ** -0.5]))[0]
    o1 = np.zeros_like(V1)
    o1[1:] = s * V1[:-1]
    rms = np.sqrt((16.0 + np.sum(o1 ** 2, axis=1)) / 16.0 + 1e-6)
    expect = oracle.round_bf16(o1 / rms[:, None])
    np.testing.assert_array_equal(S[0, 1, 0], expect.T)


def test_layer_input_invariants():
    d, Hqk, Hv, dk, dv, n = 64, 2, 4, 16, 8, 33
    x = oracle.round_bf16(RNG.standard_normal((n, d)) * 3.0)
    w = dict(w_qk=oracle.round_bf16(RNG.standard_normal((2 * Hqk * dk, d)) * 0.1),
             w_v=oracle.round_bf16(RNG.standard_normal((Hv * dv, d)) * 0.1),
             w_a=oracle.round_bf16(RNG.standard_normal((Hv, d)) * 0.1),
             w_b=oracle.round_bf16(RNG.standard_normal((Hv, d)) * 0.1))
    q, k, v, g, beta = og.layer_inputs(x, w, Hqk, Hv, dk, dv, 1e-6)
    # unit RMS after normalisation (before bf16 rounding)
    y = og.rmsnorm(x, None, 1e-6)
    np.testing.assert_allclose(np.mean(y * y, axis=1), 1.0, rtol=1e-5)
    # per-head norms: |k| = 1, |q| = dk^-1/2, up to bf16 rounding of the entries
    np.testing.assert_allclose(np.linalg.norm(k, axis=-1), 1.0, rtol=8e-3)
    np.testing.assert_allclose(np.linalg.norm(q, axis=-1), dk ** -0.5, rtol=8e-3)
    assert np.all(g < 0) and np.all((beta > 0) & (beta < 1))
    # gate maps: softplus(0) = ln 2, sigmoid(0) = 1/2, and their large-argument limits
    np.testing.assert_allclose(og.softplus(np.array([0.0, 50.0, -50.0])), [np.log(2), 50.0, np.exp(-50.0)], rtol=1e-14)
    np.testing.assert_allclose(og.sigmoid(np.array([0.0, 40.0, -40.0])), [0.5, 1.0, np.exp(-40.0)], rtol=1e-14)
    assert q.shape == (n, Hqk, dk) and v.shape == (n, Hv, dv) and g.shape == (n, Hv)


def _random_weights(L, d, Hqk, Hv, dk, dv, std=0.05):
    def w(*s):
        return oracle.round_bf16(RNG.standard_normal(s) * std)
    return [dict(w_qk=w(2 * Hqk * dk, d), w_v=w(Hv * dv, d), w_a=w(Hv, d), w_b=w(Hv, d), w_o=w(d, Hv * dv))
            for _ in range(L)]


def test_zero_output_projection_passes_the_hidden_through():
    d, Hqk, Hv, dk, dv, n = 32, 1, 2, 8, 8, 21
    h = oracle.round_bf16(RNG.standard_normal((2, n, d)))
    ws = []
    for gi in range(2):
        layer = _random_weights(1, d, Hqk, Hv, dk, dv)[0]
        layer["w_o"] = np.zeros_like(layer["w_o"])
        ws.append([layer, layer])
    S = og.group(h, ws, Hqk, Hv, dk, dv)
    np.testing.assert_array_equal(S[:, 1], S[:, 0])
    # groups are independent: replaying group 1 alone gives the same states
    S1 = og.group(h[1:], ws[1:], Hqk, Hv, dk, dv)
    np.testing.assert_array_equal(S1[0], S[1])


def test_first_layer_is_scale_invariant():
    d, Hqk, Hv, dk, dv, n = 32, 1, 2, 8, 8, 25
    h = oracle.round_bf16(RNG.standard_normal((1, n, d)))
    ws = [_random_weights(1, d, Hqk, Hv, dk, dv)]
    S_a = og.group(h, ws, Hqk, Hv, dk, dv)
    S_b = og.group(2.0 * h, ws, Hqk, Hv, dk, dv)
    assert np.linalg.norm(S_a - S_b) <= 1e-2 * np.linalg.norm(S_a)


def test_projection_values_on_exact_weights():
    # Weights whose rows pick single hidden coordinates (or the pair (3, 4) of them), so every
    # projected value has a closed form: pins the [out, in] orientation of each weight, the
    # order of the q heads then the k heads, the per-head L2 norm, the q scale dk^-1/2, the
    # head-major split of v, and the gate maps against independent library routines.
    from scipy.special import expit
    d, Hqk, Hv, dk, dv = 16, 2, 2, 4, 4
    y = np.array([[1.0, -2.0, 0.5, 4.0, -1.0, 3.0, 2.0, -0.25, 0.75, 1.5, -3.0, 0.125, 2.5, -0.5, 1.25, -4.0],
                  [0.5, 1.0, -1.5, 2.0, 3.0, -0.75, 0.25, 1.0, -2.0, 0.5, 1.0, -1.0, 0.375, 2.0, -2.5, 1.0]])
    assert np.array_equal(oracle.round_bf16(y), y)
    # q head h and k head h: 3 y[a] + 4 y[b] in column 0, y[c] in column 1 (others 0)
    picks = {("q", 0): (0, 1, 2), ("q", 1): (3, 4, 5), ("k", 0): (6, 7, 8), ("k", 1): (9, 10, 11)}
    w_qk = np.zeros((2 * Hqk * dk, d))
    for (kind, h), (a, b, c) in picks.items():
        row = (0 if kind == "q" else Hqk * dk) + h * dk
        w_qk[row, a], w_qk[row, b], w_qk[row + 1, c] = 3.0, 4.0, 1.0
    perm = np.array([5, 2, 7, 0, 12, 15, 1, 9])          # v output j reads y[perm[j]]
    w_v = np.zeros((Hv * dv, d)); w_v[np.arange(Hv * dv), perm] = 1.0
    w_a = np.zeros((Hv, d)); w_a[0, 3], w_a[1, 10] = 1.0, 0.5      # za = (y3, y10 / 2)
    w_b = np.zeros((Hv, d)); w_b[0, 13], w_b[1, 14] = 2.0, 1.0     # zb = (2 y13, y14)
    q, k, v, g, beta = og.project(y, dict(w_qk=w_qk, w_v=w_v, w_a=w_a, w_b=w_b), Hqk, Hv, dk, dv)
    for t in range(2):
        for (kind, h), (a, b, c) in picks.items():
            x0, x1 = 3.0 * y[t, a] + 4.0 * y[t, b], y[t, c]
            nrm = np.sqrt(x0 * x0 + x1 * x1 + og.L2_EPS)
            scale = dk ** -0.5 if kind == "q" else 1.0
            expect = oracle.round_bf16(np.array([x0, x1, 0.0, 0.0]) / nrm * scale)
            got = (q if kind == "q" else k)[t, h]
            np.testing.assert_array_equal(got, expect)
        np.testing.assert_array_equal(v[t].reshape(-1), y[t, perm])
        za = np.array([y[t, 3], y[t, 10] / 2.0])
        zb = np.array([2.0 * y[t, 13], y[t, 14]])
        np.testing.assert_allclose(g[t], -np.logaddexp(0.0, za), rtol=1e-7)
        np.testing.assert_allclose(beta[t], expit(zb), rtol=1e-7)


def test_rmsnorm_closed_form():
    # RMS of (3, 4, 0, 0) is 2.5; the gain multiplies after the normalisation
    x = np.array([[3.0, 4.0, 0.0, 0.0]])
    gain = np.array([1.0, 2.0, 3.0, 4.0])
    y = og.rmsnorm(x, gain, 0.0)
    np.testing.assert_allclose(y, [[1.2, 3.2, 0.0, 0.0]], rtol=1e-15)
