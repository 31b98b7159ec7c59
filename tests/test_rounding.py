"""The oracle's fp64 -> bf16 rounding, pinned against torch's fp32 -> bf16 cast on values where
no double rounding can occur (every fp32 value), including ties, subnormals and overflow."""
import numpy as np
import torch

import oracle


def test_matches_torch_on_fp32_values():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2**32, size=200_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    # add exact ties: fp32 values whose low 16 bits are 0x8000
    ties = ((rng.integers(0, 2**16, size=5000, dtype=np.uint64) << 16) | 0x8000).astype(np.uint32).view(np.float32)
    x = np.concatenate([x, ties[np.isfinite(ties)], np.float32([1e-40, -3e-39, 3.4e38, 65504.0, 1.0, -0.0])])
    expect = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.round_bf16(x.astype(np.float64))
    np.testing.assert_array_equal(got, expect)


def test_direct_rounding_avoids_double_rounding():
    # 1 + 2^-8 + 2^-30 is just above the bf16 tie between 1 and 1 + 2^-7: the correct result
    # rounds up, while rounding through fp32 first would land on the tie and round to even (1.0)
    x = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert oracle.round_bf16(np.array([x]))[0] == 1.0 + 2.0 ** -7
