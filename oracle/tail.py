"""Replay-length rule (oracle side; test infrastructure only).

Reading notes "Tail-Replay：混合 LLM 前缀缓存的短尾重放机制", section 2.1 (symbol
table): the number of replayed tokens is k = ceil(r m) for a matched prefix of m
tokens and replay ratio r; section 2.2 step 2 takes the cached hidden vectors
h_{m-k+1..m} (1-based), and its worked example replays positions 9,501-10,000 for
m = 10,000, r = 5%.

r is given as an exact fraction r_num / r_den so that the ceiling is exact.
"""
from __future__ import annotations

from fractions import Fraction


def tail_length(m: int, r_num: int, r_den: int) -> int:
    """k = ceil(r * m) with r = r_num / r_den in (0, 1]; 0 for m == 0."""
    if m < 0 or r_den <= 0 or r_num <= 0 or r_num > r_den:
        raise ValueError("need m >= 0 and 0 < r <= 1")
    prod = Fraction(m) * Fraction(r_num, r_den)
    k = prod.numerator // prod.denominator
    if k * prod.denominator != prod.numerator:
        k += 1
    return k


def tail_range(m: int, r_num: int, r_den: int) -> tuple[int, int]:
    """0-based half-open token range [m - k, m) of the replayed tail."""
    k = tail_length(m, r_num, r_den)
    return m - k, m
