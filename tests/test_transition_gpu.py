"""GPU parity of the transition product, the state composition and the long-sequence
fidelity figures, through the C ABI.

The recurrence is linear in its starting state (reading notes "Tail-Replay：混合 LLM 前缀缓存的
短尾重放机制", section 2.3: S_m is the start carried through the span's operators plus the
replay from zero).  So Phi = tr_gdn_transition (the recurrence from I with zero values),
E_m = S_a Phi is the exact error of replaying from zero, and S_m = S_a Phi + S_hat_m.

Tolerances (relative Frobenius error per (sequence, head) slice): replayed states 2e-3 for
bf16 inputs; Phi and the composition 1e-5 (both are fp32 arithmetic on exactly converted
inputs, for either input type).
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from linear_attention_state_amd import (gdn_replay, gdn_transition, gdn_transition_workspace_size, state_compose,
                                        tail_seqlens)

pytestmark = pytest.mark.gpu


def rel(a, b):
    a = np.asarray(a, np.float64); b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / nb if nb > 0 else np.linalg.norm(a - b)


def np64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def oracle_phi(k, g, beta, cu, d):
    """Phi from the oracle: the recurrence from I with zero queries and values."""
    T, Hqk, _ = k.shape
    Hv = g.shape[1]
    B = len(cu) - 1
    eye = np.broadcast_to(np.eye(d), (B, Hv, d, d)).copy()
    S, _ = oracle.gdn(np.zeros((T, Hqk, d)), k, np.zeros((T, Hv, d)), g, beta, cu, state_in=eye, want_o=False)
    return S


def oracle_phi_separated(k, g, beta, cu, d):
    """(phi, log_scale) from the oracle: the same recurrence with every g = 0, and sum(g)."""
    phi = oracle_phi(k, np.zeros_like(g), beta, cu, d)
    ls = np.stack([g[cu[b]:cu[b + 1]].sum(axis=0) for b in range(len(cu) - 1)])
    return phi, ls


PHI_TOL = 1e-5


@pytest.mark.parametrize("d,dtype,tol", [(128, torch.bfloat16, PHI_TOL), (64, torch.bfloat16, PHI_TOL),
                                         (128, torch.float32, PHI_TOL), (64, torch.float32, PHI_TOL)])
def test_transition_matches_oracle(d, dtype, tol):
    lens = [130, 64, 1, 0, 77]
    inp = synthetic.gdn_inputs(lens, 2, 4, d, d, dtype=dtype, seed=11)
    dev = inp.to("cuda")
    phi = gdn_transition(dev.k, dev.g, dev.beta, inp.cu_seqlens)
    torch.cuda.synchronize()
    ref = oracle_phi(np64(inp.k), np64(inp.g), np64(inp.beta), inp.cu_seqlens.numpy(), d)
    worst = max(rel(np64(phi[b, h]), ref[b, h]) for b in range(len(lens)) for h in range(4))
    print("transition d=%d %s: worst err %.3e" % (d, dtype, worst), flush=True)
    assert worst <= tol
    # an empty span is the identity
    assert np.array_equal(np64(phi[3, 0]), np.eye(d))
    # the decay kept apart: Phi = exp(log_scale) psi
    psi, ls = gdn_transition(dev.k, dev.g, dev.beta, inp.cu_seqlens, separate_decay=True)
    torch.cuda.synchronize()
    psi_ref, ls_ref = oracle_phi_separated(np64(inp.k), np64(inp.g), np64(inp.beta), inp.cu_seqlens.numpy(), d)
    worst = max(rel(np64(psi[b, h]), psi_ref[b, h]) for b in range(len(lens)) for h in range(4))
    assert worst <= tol
    np.testing.assert_allclose(np64(ls), ls_ref, rtol=1e-5, atol=1e-6)
    for b in range(len(lens)):
        for h in range(4):
            assert rel(np.exp(np64(ls[b, h])) * np64(psi[b, h]), ref[b, h]) <= tol


@pytest.mark.parametrize("lens,Hv,min_segments", [([4000], 1, 16), ([1639, 900, 0, 1639], 4, 2)])
def test_transition_in_segments(lens, Hv, min_segments):
    # Few (sequence, head) pairs: every span is cut into segments that run side by side and are
    # multiplied in order.  One 4,000-token span on one head takes the most segments (16, of
    # 250 tokens); the packed case mixes several segments per span with an empty span.
    d = 128
    inp = synthetic.gdn_inputs(lens, 1, Hv, d, d, seed=17)
    n_ws = gdn_transition_workspace_size(inp.cu_seqlens, 1, Hv, d, torch.bfloat16)
    assert n_ws >= min_segments * len(lens) * Hv * d * d * 4
    dev = inp.to("cuda")
    psi, ls = gdn_transition(dev.k, dev.g, dev.beta, inp.cu_seqlens, separate_decay=True)
    torch.cuda.synchronize()
    psi_ref, ls_ref = oracle_phi_separated(np64(inp.k), np64(inp.g), np64(inp.beta), inp.cu_seqlens.numpy(), d)
    worst = max(rel(np64(psi[b, h]), psi_ref[b, h]) for b in range(len(lens)) for h in range(Hv))
    print("segments %s x %d heads: worst psi err %.3e" % (lens, Hv, worst), flush=True)
    assert worst <= PHI_TOL
    np.testing.assert_allclose(np64(ls), ls_ref, rtol=1e-5, atol=1e-5)
    if 0 in lens:
        assert np.array_equal(np64(psi[lens.index(0), 0]), np.eye(d))


@pytest.mark.parametrize("case", range(6))
def test_transition_random_configurations(case):
    # Seeded draws: 1-6 spans of 0-2,500 tokens, Hqk in {1, 2} with 1, 2 or 4 value heads each,
    # d in {64, 128}, bf16 or fp32 keys, the decay applied or kept apart.  Whether and how the
    # spans are cut into segments follows from the draw.
    rng = np.random.default_rng(3000 + case)
    lens = [int(x) for x in rng.integers(0, 2501, size=int(rng.integers(1, 7)))]
    Hqk = int(rng.choice([1, 2]))
    Hv = Hqk * int(rng.choice([1, 2, 4]))
    d = int(rng.choice([64, 128]))
    dtype = torch.float32 if rng.integers(0, 2) else torch.bfloat16
    separate = bool(rng.integers(0, 2))
    inp = synthetic.gdn_inputs(lens, Hqk, Hv, d, d, dtype=dtype, seed=3100 + case)
    dev = inp.to("cuda")
    label = "lens %s Hqk %d Hv %d d %d %s separate %s" % (lens, Hqk, Hv, d, dtype, separate)
    cu = inp.cu_seqlens.numpy()
    if separate:
        psi, ls = gdn_transition(dev.k, dev.g, dev.beta, inp.cu_seqlens, separate_decay=True)
        torch.cuda.synchronize()
        ref, ls_ref = oracle_phi_separated(np64(inp.k), np64(inp.g), np64(inp.beta), cu, d)
        np.testing.assert_allclose(np64(ls), ls_ref, rtol=1e-5, atol=1e-5, err_msg=label)
        got = psi
    else:
        got = gdn_transition(dev.k, dev.g, dev.beta, inp.cu_seqlens)
        torch.cuda.synchronize()
        ref = oracle_phi(np64(inp.k), np64(inp.g), np64(inp.beta), cu, d)
    worst = max(rel(np64(got[b, h]), ref[b, h]) for b in range(len(lens)) for h in range(Hv))
    print("%s: worst %.2e" % (label, worst), flush=True)
    assert worst <= PHI_TOL, label


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_transition_of_reflectors(dtype):
    # alpha = 1 and beta = 2 make every factor I - 2 k k^T a Householder reflector (for unit
    # keys): nothing decays, so every rounding stays in the product.  2,000 tokens on two heads
    # are cut into 16 segments and multiplied back, and Phi must still match the oracle.
    d, lens, H = 128, [2000], 2
    inp = synthetic.gdn_inputs(lens, H, H, d, d, dtype=dtype, seed=23)
    g = torch.zeros_like(inp.g)
    beta = torch.full_like(inp.beta, 2.0)
    n_ws = gdn_transition_workspace_size(inp.cu_seqlens, H, H, d, dtype)
    assert n_ws >= 16 * H * d * d * 4
    phi = gdn_transition(inp.k.cuda(), g.cuda(), beta.cuda(), inp.cu_seqlens)
    torch.cuda.synchronize()
    ref = oracle_phi(np64(inp.k), np64(g), np64(beta), inp.cu_seqlens.numpy(), d)
    worst = max(rel(np64(phi[0, h]), ref[0, h]) for h in range(H))
    print("reflectors %s: worst err %.3e" % (dtype, worst), flush=True)
    assert worst <= PHI_TOL
    if dtype == torch.float32:
        # unit keys to fp32 rounding: the product stays orthogonal to about the same accuracy
        for h in range(H):
            P = np64(phi[0, h])
            assert np.linalg.norm(P.T @ P - np.eye(d)) / np.sqrt(d) <= 1e-4


def test_compose_matches_definition():
    gen = torch.Generator(device="cpu").manual_seed(3)
    S_c = torch.randn((6, 128, 128), generator=gen)
    phi = torch.randn((6, 128, 128), generator=gen) * 0.1
    S_hat = torch.randn((6, 128, 128), generator=gen)
    out = state_compose(S_c.cuda(), phi.cuda(), S_hat.cuda())
    out2 = state_compose(S_c.cuda(), phi.cuda())
    torch.cuda.synchronize()
    ref = S_c.double().numpy() @ phi.double().numpy()
    assert rel(np64(out), ref + S_hat.double().numpy()) <= 1e-5
    assert rel(np64(out2), ref) <= 1e-5
    # out may alias S_hat (in-place accumulation)
    acc = S_hat.cuda().contiguous()
    state_compose(S_c.cuda(), phi.cuda(), acc, out=acc)
    torch.cuda.synchronize()
    assert rel(np64(acc), ref + S_hat.double().numpy()) <= 1e-5
    # dv != dk, both head sizes, and a log scale
    for dv, dk, N in ((64, 128, 3), (128, 64, 5), (64, 64, 9)):
        A = torch.randn((N, dv, dk), generator=gen)
        P = torch.randn((N, dk, dk), generator=gen) * 0.1
        ref = A.double().numpy() @ P.double().numpy()
        assert rel(np64(state_compose(A.cuda(), P.cuda())), ref) <= 1e-5
        ls = -torch.rand((N,), generator=gen) * 3
        got = state_compose(A.cuda(), P.cuda(), log_scale=ls.cuda())
        assert rel(np64(got), np.exp(ls.double().numpy())[:, None, None] * ref) <= 1e-5


def test_checkpoint_composition_on_gpu():
    # a prefix of 700 tokens, then a span of 300: S_m = S_a Phi + S_hat (all from the GPU)
    a, n = 700, 300
    inp = synthetic.gdn_inputs([a + n], 2, 4, 128, 128, seed=5)
    dev = inp.to("cuda")
    sl = lambda t, lo, hi: t[lo:hi].contiguous()  # noqa: E731
    cu_a = torch.tensor([0, a], dtype=torch.int32)
    cu_n = torch.tensor([0, n], dtype=torch.int32)
    S_a, _ = gdn_replay(sl(dev.q, 0, a), sl(dev.k, 0, a), sl(dev.v, 0, a), sl(dev.g, 0, a), sl(dev.beta, 0, a),
                        cu_a, want_o=False)
    tail = [sl(t, a, a + n) for t in (dev.q, dev.k, dev.v, dev.g, dev.beta)]
    S_hat, _ = gdn_replay(*tail, cu_n, want_o=False)
    phi = gdn_transition(tail[1], tail[3], tail[4], cu_n)
    S_m, _ = gdn_replay(dev.q, dev.k, dev.v, dev.g, dev.beta, inp.cu_seqlens, want_o=False)
    S_comp = state_compose(S_a, phi, S_hat)
    torch.cuda.synchronize()
    S_ref, _ = oracle.gdn(np64(inp.q), np64(inp.k), np64(inp.v), np64(inp.g), np64(inp.beta),
                          inp.cu_seqlens.numpy(), want_o=False)
    for h in range(4):
        e_comp = rel(np64(S_comp[0, h]), S_ref[0, h])
        e_full = rel(np64(S_m[0, h]), S_ref[0, h])
        print("head %d: composed %.3e, single pass %.3e" % (h, e_comp, e_full), flush=True)
        assert e_comp <= 2e-3 and e_full <= 2e-3


def test_full_prefix_fidelity_32k():
    # One 32,768-token sequence from zero, 16 heads, dk = dv = 128, bf16: the full-prefix state
    # S_m and the tail replays S_hat_m at r = 5% and 10% through the same kernel.  Four heads
    # are checked against the oracle; the fidelity ratio |S_m - S_hat_m| / |S_m| is compared
    # with the exact one, |S_a Phi| / |S_m| from the oracle.
    m, H = 32768, 16
    heads = [0, 5, 10, 15]
    inp = synthetic.gdn_inputs([m], H, H, 128, 128, seed=21)
    dev = inp.to("cuda")
    cu_m = torch.tensor([0, m], dtype=torch.int32)
    S_m, _ = gdn_replay(dev.q, dev.k, dev.v, dev.g, dev.beta, cu_m, want_o=False)
    torch.cuda.synchronize()
    f = {name: np64(getattr(inp, name))[:, heads] for name in ("q", "k", "v", "g", "beta")}
    # oracle: the prefix up to the 10% tail start, then each piece by state passing
    k10 = int(tail_seqlens([m], 10, 100)[0][1])
    k05 = int(tail_seqlens([m], 5, 100)[0][1])
    a10, a05 = m - k10, m - k05

    def orc(lo, hi, state=None):
        S, _ = oracle.gdn(f["q"][lo:hi], f["k"][lo:hi], f["v"][lo:hi], f["g"][lo:hi], f["beta"][lo:hi],
                          np.array([0, hi - lo], np.int32), state_in=state, want_o=False)
        return S

    S_a10 = orc(0, a10)
    S_a05 = orc(a10, a05, S_a10)
    S_m_ref = orc(a05, m, S_a05)
    for i, h in enumerate(heads):
        e = rel(np64(S_m[0, h]), S_m_ref[0, i])
        print("32K full recurrence head %d: err %.3e" % (h, e), flush=True)
        assert e <= 2e-3
    for r, a, S_a in ((5, a05, S_a05), (10, a10, S_a10)):
        k = m - a
        tail = [t[a:].contiguous() for t in (dev.q, dev.k, dev.v, dev.g, dev.beta)]
        cu_k = torch.tensor([0, k], dtype=torch.int32)
        S_hat, _ = gdn_replay(*tail, cu_k, want_o=False)
        # the decay product exp(sum g) leaves the fp32 range at r = 10%: keep it apart
        psi, ls = gdn_transition(tail[1], tail[3], tail[4], cu_k, separate_decay=True)
        S_a_dev = torch.zeros_like(S_m)
        for i, h in enumerate(heads):
            S_a_dev[0, h] = torch.from_numpy(S_a[0, i]).float()
        E = state_compose(S_a_dev, psi, log_scale=ls)
        torch.cuda.synchronize()
        psi_ref, ls_ref = oracle_phi_separated(f["k"][a:], f["g"][a:], f["beta"][a:], np.array([0, k], np.int32), 128)
        for i, h in enumerate(heads):
            # exact truncation error |S_a Phi| / |S_m|, Phi = exp(ls) psi, in log space
            log_exact = ls_ref[0, i] + np.log(np.linalg.norm(S_a[0, i] @ psi_ref[0, i])) \
                - np.log(np.linalg.norm(S_m_ref[0, i]))
            measured = np.linalg.norm(np64(S_m[0, h]) - np64(S_hat[0, h])) / np.linalg.norm(np64(S_m[0, h]))
            e_psi = rel(np64(psi[0, h]), psi_ref[0, i])
            e_ls = abs(float(ls[0, h]) - ls_ref[0, i]) / abs(ls_ref[0, i])
            print("r = %d%%, head %d: |S_m - S_hat|/|S_m| = %.3e (exact truncation 10^%.1f), psi err %.3e, "
                  "log-scale err %.1e" % (r, h, measured, log_exact / np.log(10), e_psi, e_ls), flush=True)
            # the truncation is negligible here, so the measured ratio is kernel rounding
            assert measured <= 3e-3 and log_exact < np.log(1e-6)
            assert e_psi <= PHI_TOL and e_ls <= 1e-5
            # the GPU's E_m = S_a Phi, where fp32 can hold it
            E_ref = np.exp(ls_ref[0, i]) * (S_a[0, i] @ psi_ref[0, i])
            if np.linalg.norm(E_ref) > 1e-30:
                assert rel(np64(E[0, h]), E_ref) <= 1e-4
