"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a copy of the C oracle's source (a dropped term, a
wrong sign, a wrong index, a pre-update read-out, ...), compiles the copy on the
CPU, and checks that at least one pin in test_oracle.py fails against it.  The
unmodified oracle must pass all of them.
"""
import os
import subprocess

import numpy as np
import pytest

import oracle
from tests import test_oracle as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "gdn_oracle.c")

MUTANTS = {
    "decay_outside_delta": ("row[c] = alpha * (row[c] - bt * sk * kt[c]) + bt * vt[r] * kt[c];",
                            "row[c] = alpha * row[c] - bt * sk * kt[c] + bt * vt[r] * kt[c];"),
    "delta_sign": ("row[c] = alpha * (row[c] - bt * sk * kt[c])",
                   "row[c] = alpha * (row[c] + bt * sk * kt[c])"),
    "write_without_beta": ("+ bt * vt[r] * kt[c];", "+ vt[r] * kt[c];"),
    "write_with_decay": ("+ bt * vt[r] * kt[c];", "+ alpha * bt * vt[r] * kt[c];"),
    "erase_without_beta": ("(row[c] - bt * sk * kt[c])", "(row[c] - sk * kt[c])"),
    "gate_not_exponentiated": ("const double alpha = exp(g[(size_t)t * Hv + h]);",
                               "const double alpha = 1.0 + g[(size_t)t * Hv + h];"),
    "head_mapping_modulo": ("const int32_t j = h / per_qk;", "const int32_t j = h % Hqk;"),
    "q_scale_dropped": ("ot[r] = q_scale * acc;", "ot[r] = acc;"),
    "readout_uses_key": ("acc += row[c] * qt[c];", "acc += row[c] * kt[c];"),
    "state_in_ignored": ("if (state_in)\n", "if (0)\n"),
}


def _build_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, name
    path = tmp_path / (name + ".c")
    path.write_text(src.replace(old, new))
    lib = tmp_path / (name + ".so")
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-o", str(lib), str(path), "-lm"])
    return oracle.open_library(str(lib))


def _pin_functions():
    return [getattr(pins, n) for n in dir(pins) if n.startswith("test_")]


def _failures(monkeypatch, lib):
    monkeypatch.setattr(oracle, "_lib", lib)
    failed = []
    for fn in _pin_functions():
        pins.RNG = np.random.default_rng(1234)
        try:
            fn()
        except (AssertionError, RuntimeError):
            failed.append(fn.__name__)
    return failed


def test_unmodified_oracle_passes_every_pin(monkeypatch):
    assert _failures(monkeypatch, oracle._load()) == []


def test_pre_update_readout_is_caught(tmp_path, monkeypatch):
    # move the read-out in front of the state update (o_t = S_{t-1} q_t)
    src = open(SRC).read()
    start = src.index("            for (int32_t r = 0; r < dv; ++r) {\n                double* row = S")
    end = src.index("            if (o) {")
    end_o = src.index("        memcpy(state_out")
    update, readout = src[start:end], src[end:end_o]
    close = readout.rindex("        }\n")          # end of the token loop body
    mutated = src[:start] + readout[:close] + update + readout[close:] + src[end_o:]
    path = tmp_path / "pre_update.c"
    path.write_text(mutated)
    lib = tmp_path / "pre_update.so"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-o", str(lib), str(path), "-lm"])
    assert _failures(monkeypatch, oracle.open_library(str(lib)))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(tmp_path, monkeypatch, name):
    old, new = MUTANTS[name]
    lib = _build_mutant(tmp_path, name, old, new)
    failed = _failures(monkeypatch, lib)
    assert failed, "no pin caught mutant %s" % name


# ---- the group-chain oracle (Python) ----------------------------------------------------------
import importlib.util  # noqa: E402
import sys  # noqa: E402

from tests import test_oracle_group as group_pins  # noqa: E402

CHAIN_SRC = os.path.join(os.path.dirname(oracle.__file__), "chain.py")
CHAIN_MUTANTS = {
    "residual_sign": ("x = round_bf16(x + ob @", "x = round_bf16(x - ob @"),
    "residual_dropped": ("x = round_bf16(x + ob @", "x = round_bf16(0 * x + ob @"),
    "q_k_swapped": ("q = round_bf16(l2norm_heads(qk[:, : Hqk * dk], Hqk, dk) * dk ** -0.5)\n    k = round_bf16(l2norm_heads(qk[:, Hqk * dk:], Hqk, dk))",
                    "k = round_bf16(l2norm_heads(qk[:, : Hqk * dk], Hqk, dk))\n    q = round_bf16(l2norm_heads(qk[:, Hqk * dk:], Hqk, dk) * dk ** -0.5)"),
    "no_rmsnorm": ("y = x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)", "y = x"),
    "gate_sign": ("g = round_f32(-softplus(za))", "g = round_f32(softplus(za))"),
    "no_key_norm": ("k = round_bf16(l2norm_heads(qk[:, Hqk * dk:], Hqk, dk))", "k = round_bf16(qk[:, Hqk * dk:].reshape(-1, Hqk, dk))"),
    "q_scale_dropped": ("q = round_bf16(l2norm_heads(qk[:, : Hqk * dk], Hqk, dk) * dk ** -0.5)",
                        "q = round_bf16(l2norm_heads(qk[:, : Hqk * dk], Hqk, dk))"),
    "gate_weights_swapped": ('za = y @ np.asarray(w["w_a"], dtype=np.float64).T\n    zb = y @ np.asarray(w["w_b"], dtype=np.float64).T',
                             'za = y @ np.asarray(w["w_b"], dtype=np.float64).T\n    zb = y @ np.asarray(w["w_a"], dtype=np.float64).T'),
    "beta_softplus": ("beta = round_f32(sigmoid(zb))", "beta = round_f32(softplus(zb))"),
    "rms_gain_ignored": ("        y = y * np.asarray(gain, dtype=np.float64)", "        y = y * 1.0"),
    "heads_interleaved": ("    xs = x.reshape(x.shape[0], n_heads, d_head)",
                          "    xs = x.reshape(x.shape[0], d_head, n_heads).transpose(0, 2, 1)"),
    "states_from_previous_layer": ("S, o = gdn(q, k, v, g, beta, cu, q_scale=1.0, want_o=not last)",
                                   "S, o = gdn(q, k, v, g, beta, cu, q_scale=1.0, want_o=not last, "
                                   "state_in=states[gi, li - 1:li] if li else None)"),
}


def _chain_mutant(name, old, new):
    src = open(CHAIN_SRC).read()
    assert src.count(old) == 1, name
    spec = importlib.util.spec_from_loader("oracle._chain_mutant_" + name, loader=None)
    mod = importlib.util.module_from_spec(spec)
    mod.__package__ = "oracle"
    sys.modules[spec.name] = mod
    exec(compile(src.replace(old, new), CHAIN_SRC, "exec"), mod.__dict__)
    return mod


def _group_failures(monkeypatch, mod):
    monkeypatch.setattr(group_pins, "og", mod)
    failed = []
    for name in dir(group_pins):
        if name.startswith("test_"):
            group_pins.RNG = np.random.default_rng(77)
            try:
                getattr(group_pins, name)()
            except (AssertionError, RuntimeError, ValueError):
                failed.append(name)
    return failed


def test_unmodified_chain_passes_every_pin(monkeypatch):
    assert _group_failures(monkeypatch, _chain_mutant("identity", "L2_EPS = 1e-6", "L2_EPS = 1e-6")) == []


@pytest.mark.parametrize("name", sorted(CHAIN_MUTANTS))
def test_planted_chain_mistake_is_caught(monkeypatch, name):
    old, new = CHAIN_MUTANTS[name]
    assert _group_failures(monkeypatch, _chain_mutant(name, old, new)), "no pin caught %s" % name
