"""Replay-length rule k = ceil(r m) (reading notes "Tail-Replay：混合 LLM 前缀缓存的短尾重放机制",
section 2.1 symbol table; worked example in section 2.2), oracle side."""
import math
import os

import numpy as np

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def load_golden():
    rows = []
    with open(os.path.join(HERE, "golden", "tail_worked_example.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                rows.append([int(x) for x in line.split()])
    return rows


def test_worked_example_from_the_pages():
    for m, rn, rd, first, last in load_golden():
        lo, hi = oracle.tail_range(m, rn, rd)
        assert (lo + 1, hi) == (first, last)          # 0-based [lo, hi) -> 1-based [lo+1, hi]
        assert oracle.tail_length(m, rn, rd) == last - first + 1


def test_ceiling_matches_real_arithmetic():
    # the exact-fraction ceiling agrees with ceil() of the real product wherever the float
    # product is exact or far from an integer
    rng = np.random.default_rng(5)
    for m in list(rng.integers(1, 200_000, size=2000)) + [1, 2, 19, 20, 21, 32768, 131072]:
        m = int(m)
        for rn, rd in ((5, 100), (10, 100), (1, 3), (1, 1)):
            k = oracle.tail_length(m, rn, rd)
            assert k == -((-m * rn) // rd)
            assert 1 <= k <= m
            assert k - 1 < m * rn / rd <= k


def test_workload_lengths():
    assert oracle.tail_length(32768, 5, 100) == 1639      # 1638.4 rounds up
    assert oracle.tail_length(32768, 10, 100) == 3277     # 3276.8 rounds up
    assert oracle.tail_length(100, 5, 100) == 5           # exact products do not round up
    assert oracle.tail_length(0, 5, 100) == 0
    assert math.ceil(0.05 * 131072) == oracle.tail_length(131072, 5, 100) == 6554
