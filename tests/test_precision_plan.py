"""The precision plan of the chunked bf16 replay, reproduced on the CPU.

tests/precision_model.py follows the chunked (WY) form of reading notes "Tail-Replay：混合 LLM
前缀缓存的短尾重放机制", section 2.3, Eq. (1), with a rounding switch at each place where the
GPU kernel rounds.  Against the fp64 token recurrence (the oracle), on a single-hit tail
(1,639 tokens, dk = dv = 128, the workload's input distributions):
  - without rounding, the chunked algebra equals the token recurrence to fp64 rounding;
  - with the kernel's plan (fp32 accumulation, hi / lo splits where it splits), states and
    outputs stay within the bf16 tolerances (2e-3 and 3e-3 relative Frobenius);
  - with every operand rounded once to bf16 and no splits, the state error is several times
    the plan's: the splits are what keeps the states accurate.
The figures are printed (pytest -s) and listed in the design notes.
"""
import numpy as np
import pytest

import oracle
import synthetic
from precision_model import chunk_replay

TOKENS = 1639          # the 5% tail of a 32,768-token prefix
HEADS = 2


def rel(a, b):
    return np.linalg.norm(a - b) / np.linalg.norm(b)


@pytest.fixture(scope="module")
def case():
    inp = synthetic.gdn_inputs([TOKENS], HEADS, HEADS, 128, 128, seed=31)
    arr = {n: getattr(inp, n).to(dtype=__import__("torch").float64).numpy() for n in ("q", "k", "v", "g", "beta")}
    S_ref, O_ref = oracle.gdn(arr["q"], arr["k"], arr["v"], arr["g"], arr["beta"], inp.cu_seqlens.numpy())
    return arr, S_ref, O_ref


def errors(case, mode, drop=()):
    arr, S_ref, O_ref = case
    es, eo = [], []
    for h in range(HEADS):
        S, O = chunk_replay(arr["q"][:, h], arr["k"][:, h], arr["v"][:, h], arr["g"][:, h], arr["beta"][:, h],
                            mode=mode, drop=drop)
        es.append(rel(S, S_ref[0, h]))
        eo.append(rel(O, O_ref[:, h]))
    print("precision model %-8s %-24s: worst state %.3e, worst output %.3e"
          % (mode, "-".join(drop) or "", max(es), max(eo)), flush=True)
    return max(es), max(eo)


def test_chunked_algebra_is_the_token_recurrence(case):
    es, eo = errors(case, "exact")
    assert es < 1e-10 and eo < 1e-10


@pytest.mark.parametrize("ch", [16, 32])
def test_chunked_algebra_holds_at_other_chunk_lengths(case, ch):
    # the WY form does not depend on the chunk length: without rounding, chunks of 16 and 32
    # tokens (one diagonal block; two blocks and one merge) give the token recurrence too
    arr, S_ref, O_ref = case
    for h in range(HEADS):
        S, O = chunk_replay(arr["q"][:, h], arr["k"][:, h], arr["v"][:, h], arr["g"][:, h], arr["beta"][:, h],
                            mode="exact", ch=ch)
        assert rel(S, S_ref[0, h]) < 1e-10 and rel(O, O_ref[:, h]) < 1e-10


def test_plan_meets_the_bf16_tolerances(case):
    es, eo = errors(case, "plan")
    assert es <= 2e-3 and eo <= 3e-3


def test_splits_carry_the_state_accuracy(case):
    es_plan, eo_plan = errors(case, "plan")
    es_bf16, _ = errors(case, "all_bf16")
    assert es_bf16 > 3 * es_plan
    # each choice alone: the state-update split and the exact unit diagonal carry the
    # states, the P U' split the outputs
    es_upd, _ = errors(case, "plan", drop=("split_update",))
    es_diag, _ = errors(case, "plan", drop=("unit_diag",))
    _, eo_pu = errors(case, "plan", drop=("split_pu",))
    assert es_upd > 1.5 * es_plan and es_diag > 1.5 * es_plan and eo_pu > eo_plan
