"""The exponent-mismatch protocol of the GPU tests, checked on the CPU.

A GPU exponent that differs from the oracle's is accepted only at a rounding
boundary of the fast-mode formula ([G] Methodik 1), and never above it by more
than rounding.
"""
import numpy as np

import oracle as O
from gpu_util import exponent_is_valid

U2 = 2 * O.U32  # 0.5 * 4 u32


def test_boundary_accepts_only_the_two_neighbours_below():
    # a row of one 1.0 has log2(sum) = 0, so z = P' - 2 u32: choose P' to put z
    # just above, just below, and well away from the integer 50
    row = np.array([1.0])
    above = 50.0 + U2 + 2.0 ** -45  # z = 50 + 2^-45
    assert exponent_is_valid(row, 50, above)
    assert exponent_is_valid(row, 49, above)
    assert not exponent_is_valid(row, 51, above)  # floor(z) + 1: breaks the bound
    below = 50.0 + U2 - 2.0 ** -45  # z = 50 - 2^-45
    assert exponent_is_valid(row, 49, below)
    assert exponent_is_valid(row, 50, below)
    assert not exponent_is_valid(row, 51, below)
    assert not exponent_is_valid(row, 48, below)
    away = 50.0 + U2 + 2.0 ** -30  # z = 50 + 2^-30: only floor(z)
    assert exponent_is_valid(row, 50, away)
    assert not exponent_is_valid(row, 49, away)
    assert not exponent_is_valid(row, 51, away)


def test_zero_row_takes_exponent_zero():
    assert exponent_is_valid(np.zeros(5), 0, 40.0)
    assert not exponent_is_valid(np.zeros(5), 1, 40.0)
