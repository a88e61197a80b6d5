"""Steps 3-5 fused into one launch (all moduli of a 64 x 64 tile of C per block,
reconstructed in registers; OZ2_FUSED=1): C bit-exact against the oracle on
ragged shapes, N from 2 to 20, both modes, FP64 and binary32 operands, and the
longest inner dimension the fused form takes (64 x 1024 k, where one modulus'
int32 sums reach the end of the residue step's range)."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_util import assert_bitwise_equal, run_ws

pytestmark = pytest.mark.gpu


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


CASES = [
    (1, 1, 1, 8, "fast"),
    (64, 64, 64, 8, "fast"),
    (70, 130, 200, 2, "fast"),
    (257, 63, 129, 14, "fast"),
    (300, 200, 500, 16, "fast"),
    (300, 200, 500, 16, "accurate"),
    (129, 300, 1000, 18, "fast"),
    (100, 90, 777, 20, "accurate"),
    (520, 520, 260, 14, "fast"),
]


@pytest.mark.parametrize("m,n,k,N,mode", CASES)
@pytest.mark.parametrize("single", [False, True])
def test_fused_matches_oracle(monkeypatch, m, n, k, N, mode, single):
    monkeypatch.setenv("OZ2_FUSED", "1")
    A, B = W.spread_case(m, n, k, 1.0, seed=m * 7 + n * 3 + k + N)
    if single:
        A, B = A.astype(np.float32), B.astype(np.float32)
    emul = O.os2_sgemm if single else O.os2_dgemm
    ref = emul(A, B, N, mode)["C"]
    assert_bitwise_equal(run_ws(A, B, N, mode), ref, f"fused {m}x{n}x{k} N={N} {mode}")


def test_fused_longest_inner_dimension_and_fallback(monkeypatch):
    # k = 65536: 1024 stages of 64 per modulus, the fused form's limit; one
    # beyond it the two-launch form runs instead and must agree as well
    monkeypatch.setenv("OZ2_FUSED", "1")
    for k in (65536, 65536 + 128):
        A, B = W.spread_case(40, 70, k, 0.5, seed=k % 97)
        ref = O.os2_dgemm(A, B, 16)["C"]
        assert_bitwise_equal(run_ws(A, B, 16), ref, f"fused k={k}")


def test_fused_equals_two_launch_form(monkeypatch):
    A, B = W.spread_case(1024, 768, 512, 1.0, seed=5)
    monkeypatch.setenv("OZ2_FUSED", "0")
    C2 = run_ws(A, B, 14)
    monkeypatch.setenv("OZ2_FUSED", "1")
    C1 = run_ws(A, B, 14)
    assert_bitwise_equal(C1, C2, "fused vs two launches")
