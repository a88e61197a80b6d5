"""GPU parity of the single-precision path (ozaki2_sgemm) against the oracle.

[G] ("Improved Scaling for Fast Mode of Ozaki Scheme II", section Zentrale
Beiträge) evaluates the scheme for SGEMM as well as DGEMM. The binary32 inputs
are widened exactly, so exponents, int8 residues, int32 products and reduced
residues must match the oracle bit for bit as in the FP64 path, and C must be
the oracle's single rounding of X * 2^-(e_i + f_j) to binary32, bit for bit.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_util import assert_bitwise_equal, full_parity, run_debug, run_ws
import rns_emulated_fp64_amd as oz

pytestmark = pytest.mark.gpu


def f32(pair):
    A, B = pair
    return A.astype(np.float32), B.astype(np.float32)


@pytest.mark.parametrize("N", [2, 6, 8, 9, 14, 16, 18])
def test_sgemm_ragged_fast(N):
    A, B = f32(W.spread_case(300, 290, 500, 1.0, seed=200 + N))
    g, r, _ = full_parity(A, B, N)
    assert g["C"].dtype == np.float32


@pytest.mark.parametrize("N", [8, 16, 20])
def test_sgemm_ragged_accurate(N):
    A, B = f32(W.spread_case(270, 333, 260, 1.5, seed=300 + N))
    full_parity(A, B, N, "accurate")


@pytest.mark.parametrize("shape", [(1, 1, 1), (1, 7, 3), (33, 17, 129), (64, 64, 1)])
def test_sgemm_tiny_shapes(shape):
    m, n, k = shape
    A, B = f32(W.uniform_case(m, n, k, seed=m * 5 + k))
    full_parity(A, B, 8)
    full_parity(A, B, 8, "accurate")


def test_sgemm_leading_dimensions():
    A, B = f32(W.spread_case(257, 130, 190, 0.5, seed=4))
    full_parity(A, B, 8, lda=300, ldb=211, ldc=260)


def test_sgemm_special_values():
    A, B = f32(W.spread_case(260, 140, 300, 1.0, seed=9))
    A[3, 7] = np.inf
    A[5] = 0.0
    A[8] *= np.float32(2.0 ** 100)
    A[9] *= np.float32(2.0 ** -125)      # partly subnormal binary32 entries
    B[11, 4] = np.nan
    B[:, 2] = 0.0
    B[:, 6] = np.float32(1e-40) * np.sign(B[:, 6])  # subnormal column
    for mode in ("fast", "accurate"):
        g, r, _ = full_parity(A, B, 8, mode)
        assert np.all(np.isnan(g["C"][3])) and np.all(np.isnan(g["C"][:, 4]))
        assert np.all(g["C"][5][~np.isnan(g["C"][5])] == 0.0)


def test_sgemm_overflow_and_underflow_of_results():
    # products beyond binary32's range round to +-inf, tiny ones into the
    # subnormals or to zero, exactly as the single rounding prescribes
    A, B = f32(W.uniform_case(40, 30, 64, seed=12))
    A[:10] *= np.float32(2.0 ** 70)
    B[:, :8] *= np.float32(2.0 ** 60)
    A[10:20] *= np.float32(2.0 ** -70)
    B[:, 8:16] *= np.float32(2.0 ** -70)
    g, r, _ = full_parity(A, B, 8)
    C = g["C"]
    assert np.any(np.isinf(C[:10, :8]))
    tiny = np.abs(C[10:20, 8:16])
    assert np.any((tiny > 0) & (tiny < np.finfo(np.float32).tiny))


def test_sgemm_config_4096_n8():
    # the single-precision workload at full size, in the benchmark's launch configuration
    A, B = W.make("sgemm_spread1.0_4096_n8")
    N = 8
    g = run_debug(A, B, N, want_prod=False, want_res=False)
    e, f = g["e"].tolist(), g["f"].tolist()
    rng = np.random.default_rng(7)
    rows = np.sort(rng.choice(4096, 24, replace=False)).tolist()
    cols = np.sort(rng.choice(4096, 24, replace=False)).tolist()
    A64, B64 = A.astype(np.float64), B.astype(np.float64)
    Pp = O.scaling_constant(math.prod(O.choose_moduli(N)))
    oe = O.fast_exponents_rows(A64[rows], Pp)
    of = O.fast_exponents_rows(B64[:, cols].T, Pp)
    assert sum(a != b for a, b in zip(oe, [e[i] for i in rows])) <= 1
    assert sum(a != b for a, b in zip(of, [f[j] for j in cols])) <= 1
    Ai = O.scaled_integers(A64[rows], [e[i] for i in rows])
    Bi = O.scaled_integers(B64[:, cols].T, [f[j] for j in cols])
    ref = O.unscale_f32(Ai.dot(Bi.T), [e[i] for i in rows], [f[j] for j in cols])
    assert_bitwise_equal(g["C"][np.ix_(rows, cols)], ref, "sampled C")
    assert_bitwise_equal(run_ws(A, B, N), g["C"], "ws vs debug")
    # accuracy on the sampled rows: at least that of native binary32
    exact = A64[rows] @ B64
    scale = np.abs(A64[rows]) @ np.abs(B64)
    ecw = float(np.max(np.abs(g["C"][rows].astype(np.float64) - exact) / scale))
    native = float(np.max(np.abs((A[rows] @ B).astype(np.float64) - exact) / scale))
    print(f"4096^3 SGEMM N=8: E_cw {ecw:.3e}, native binary32 {native:.3e}")
    assert ecw <= native


def test_sgemm_torch_wrapper():
    A, B = f32(W.spread_case(70, 90, 110, 1.0, seed=21))
    C = oz.sgemm(torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda(), 8).cpu().numpy()
    assert_bitwise_equal(C, O.os2_sgemm(A, B, 8)["C"], "torch sgemm")
