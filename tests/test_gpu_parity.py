"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Bar: exponents equal (with the documented boundary protocol), int8 residues,
int32 residue products and reduced residues bit-exact, and C bit-exact: the
GPU reconstructs the exact integer and rounds it once to nearest-even, the
same RN(X) * 2^-(e_i + f_j) the oracle computes with Python integers.

Pages: [Q] the Qiita article on Ozaki Scheme II (steps 1-5); [G] "Improved
Scaling for Fast Mode of Ozaki Scheme II" (section Methodik).
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_util import (assert_bitwise_equal, full_parity, reconcile_exponents, run_debug, run_ws, stream_handle,
                      device_colmajor)
import rns_emulated_fp64_amd as oz

pytestmark = pytest.mark.gpu


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oz.lib()


def test_config_u64_n8():
    # 64^3, U(-1,1), N = 8, fast mode
    A, B = W.make("u64_n8")
    g, r, mism = full_parity(A, B, 8)
    assert mism == 0


@pytest.mark.parametrize("N", [2, 8, 14, 16, 18, 20])
def test_ragged_several_tiles_fast(N):
    # m, n span two 256-row/column tiles and k a ragged 128-wide tail
    A, B = W.spread_case(300, 290, 500, 1.0, seed=N)
    full_parity(A, B, N)


@pytest.mark.parametrize("N", [8, 14, 16, 20])
def test_ragged_accurate(N):
    A, B = W.spread_case(270, 333, 260, 1.5, seed=100 + N)
    full_parity(A, B, N, "accurate")


@pytest.mark.parametrize("shape", [(1, 1, 1), (1, 7, 3), (5, 1, 200), (33, 17, 129), (64, 64, 1)])
def test_tiny_shapes(shape):
    m, n, k = shape
    A, B = W.uniform_case(m, n, k, seed=m * 7 + k)
    full_parity(A, B, 14)
    full_parity(A, B, 16, "accurate")


@pytest.mark.parametrize("shape", [(70000, 3, 5), (3, 70000, 5), (300, 66000, 2)])
def test_extreme_aspect_ratios(shape):
    # n above 65535 exceeds one grid dimension: the kernels that put columns
    # on the grid's y axis loop over them; m this large gives a long row of
    # tiles and a single column tile
    m, n, k = shape
    A, B = W.uniform_case(m, n, k, seed=m % 1000 + n % 1000)
    full_parity(A, B, 16, want_prod=False)


def test_leading_dimensions():
    A, B = W.spread_case(257, 130, 190, 0.5, seed=3)
    g, r, _ = full_parity(A, B, 16, lda=263, ldb=200, ldc=300)
    # entries beyond m in each column of C are left alone
    pad = g["C_padding"][:130, 257:]
    assert np.all(np.isnan(pad))


def test_max_inner_dimension():
    # k = 2^17 - 1, the largest k for which int32 sums stay exact ([Q] step 3)
    k = (1 << 17) - 1
    A, B = W.uniform_case(6, 5, k, seed=4)
    A[0] = 1.0
    B[:, 0] = -1.0
    full_parity(A, B, 16, want_prod=True)


@pytest.mark.parametrize("k,mode", [(1 << 16, "fast"), ((1 << 16) + 64, "fast"), ((1 << 17) + 4321, "fast"),
                                    (400000, "fast"), ((1 << 17) + 4321, "accurate")])
def test_long_inner_dimension_in_blocks(k, mode):
    # Beyond 2^17 terms the int32 sums are no longer exact ([Q] step 3: larger
    # inner dimensions are computed in blocks); the GEMM runs blocks of at most
    # 1024 stages of 64 terms, each adding its residues to the earlier ones, so
    # 2^16 is the longest single block and 2^16 + 64 the shortest split one.
    A, B = W.uniform_case(40, 24, k, seed=k % 97)
    A[0] = 1.0
    B[:, 0] = 1.0  # an all-ones row times an all-ones column: |Q| hits its bound
    full_parity(A, B, 16, mode, want_prod=False)


def test_special_values_and_zero_lines():
    A, B = W.spread_case(70, 66, 90, 1.0, seed=5)
    A[3] = 0.0
    B[:, 5] = 0.0
    A[7, 11] = np.inf
    A[9, 2] = np.nan
    B[4, 8] = -np.inf
    A[20] *= 2.0 ** 900
    A[21] *= 2.0 ** -900
    B[:, 30] *= 2.0 ** -1000   # subnormal entries
    A[40, :] = 0.0
    A[40, 17] = 5e-324         # a lone subnormal
    g, r, _ = full_parity(A, B, 16)
    C = g["C"]
    assert np.all(np.isnan(C[7])) and np.all(np.isnan(C[9])) and np.all(np.isnan(C[:, 8]))
    assert np.all(C[3, [j for j in range(66) if j != 8]] == 0.0)
    full_parity(A, B, 14, "accurate")


def test_k_zero_and_empty():
    dA = torch.zeros(1, dtype=torch.float64, device="cuda")
    dC = torch.full((4, 5), float("nan"), dtype=torch.float64, device="cuda")
    st = oz.ozaki2_dgemm(5, 4, 0, dA.data_ptr(), 5, dA.data_ptr(), 1, dC.data_ptr(), 5, 16, 0, stream_handle())
    assert st == 0
    torch.cuda.synchronize()
    assert torch.all(dC == 0)
    dC.fill_(float("nan"))
    st = oz.ozaki2_dgemm(0, 4, 3, dA.data_ptr(), 1, dA.data_ptr(), 3, dC.data_ptr(), 1, 16, 0, stream_handle())
    assert st == 0
    torch.cuda.synchronize()
    assert torch.all(torch.isnan(dC))


def test_cached_workspace_entry_and_determinism():
    A, B = W.spread_case(400, 300, 700, 1.0, seed=6)
    dA, dB = device_colmajor(A), device_colmajor(B)
    outs = []
    for _ in range(2):
        dC = torch.empty((300, 400), dtype=torch.float64, device="cuda")
        st = oz.ozaki2_dgemm(400, 300, 700, dA.data_ptr(), 400, dB.data_ptr(), 700, dC.data_ptr(), 400, 16, 0,
                             stream_handle())
        assert st == 0
        outs.append(dC.cpu().numpy().T.copy())
    assert_bitwise_equal(outs[0], outs[1], "rerun")
    r = O.os2_dgemm(A, B, 16)
    assert_bitwise_equal(outs[0], r["C"], "C via ozaki2_dgemm")
    # a different, larger problem grows the cached workspace
    A2, B2 = W.spread_case(600, 520, 900, 1.0, seed=7)
    dA2, dB2 = device_colmajor(A2), device_colmajor(B2)
    dC2 = torch.empty((520, 600), dtype=torch.float64, device="cuda")
    assert oz.ozaki2_dgemm(600, 520, 900, dA2.data_ptr(), 600, dB2.data_ptr(), 900, dC2.data_ptr(), 600, 14, 1,
                           stream_handle()) == 0
    assert_bitwise_equal(dC2.cpu().numpy().T.copy(), O.os2_dgemm(A2, B2, 14, "accurate")["C"], "grown ws")


def test_non_default_stream():
    A, B = W.spread_case(128, 96, 256, 1.0, seed=8)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        C = oz.dgemm(torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda(), 16)
    s.synchronize()
    r = O.os2_dgemm(B.T, A.T, 16)  # the binding multiplies B^T A^T in column-major terms
    assert_bitwise_equal(C.cpu().numpy(), r["C"].T, "torch wrapper")


def test_config_spread05_1024_n14():
    # 1024^3, phi = 0.5, N = 14: full parity and the accuracy gate
    A, B = W.make("spread0.5_1024_n14")
    g, r, mism = full_parity(A, B, 14, want_prod=False)
    hi, lo = O.dd_gemm(A, B)
    err = O.error_metrics(g["C"], hi, lo, A, B)
    native = O.error_metrics(A @ B, hi, lo, A, B)
    # the GPU's own FP64 product (hipBLAS through torch.mm), run only as a comparator
    Cn = (torch.from_numpy(A).cuda() @ torch.from_numpy(B).cuda()).cpu().numpy()
    native_gpu = O.error_metrics(Cn, hi, lo, A, B)
    print("1024^3 N=14:", err, "native:", native, "native GPU:", native_gpu, "exponent mismatches:", mism)
    assert err["E_cw"] <= 1e-14
    # [Q] 行列積の回数と性能: about 14 moduli reach the accuracy of native FP64
    assert err["E_cw"] <= 4 * native["E_cw"] and err["E_cw"] <= 4 * native_gpu["E_cw"]
    # proposed vs the stand-in for the original rule on the same operands (logged)
    go = run_debug(A, B, 14, "original", want_prod=False, want_res=False)
    erro = O.error_metrics(go["C"], hi, lo, A, B)
    print("1024^3 N=14 original-rule stand-in:", erro)


def _sampled_exact_check(A, B, C, e, f, rows, cols):
    """C[i, j] == RN(exact scaled dot) * 2^-(e_i + f_j) on sampled entries."""
    Ai = O.scaled_integers(A[rows], [e[i] for i in rows])
    Bi = O.scaled_integers(np.asarray(B)[:, cols].T, [f[j] for j in cols])
    Y = Ai.dot(Bi.T)
    ref = O.unscale(Y, [e[i] for i in rows], [f[j] for j in cols])
    assert_bitwise_equal(C[np.ix_(rows, cols)], ref, "sampled C")


@pytest.mark.parametrize("mode", ["fast", "accurate"])
def test_config_spread1_4096_n16(mode):
    # The headline workload at full size, in the launch configuration the
    # benchmark times: every exponent (mismatch protocol), every int8 residue
    # of A and B, every int32 residue product, every reduced residue and every
    # entry of C against the oracle's os2_dgemm, bit for bit.
    A, B = W.make("spread1.0_4096_n16")
    N = 16
    g, r, mismatches = full_parity(A, B, N, mode, want_prod=True)
    print(f"4096^3 N=16 {mode}: exponent mismatches {mismatches}")
    C_ws = run_ws(A, B, N, mode)
    assert_bitwise_equal(C_ws, g["C"], "ws vs debug")
    rng = np.random.default_rng(1)
    rows = np.sort(rng.choice(4096, 24, replace=False)).tolist()
    hi, lo = O.dd_gemm(A[rows], B)
    err = O.error_metrics(g["C"][rows], hi, lo, A[rows], B)
    print(f"4096^3 N=16 {mode}:", err)
    assert err["E_cw"] <= 1e-14


def test_config_scale_sweep_2048_n14():
    # A = alpha*ones and alpha*U(-1,1), alpha = 2^s: C(alpha) == alpha*C(1) bit
    # for bit and CRT succeeds at every alpha ([G] Methodik 2, Problemstellung).
    ones, ua, B = W.scale_sweep_case(2048)
    rng = np.random.default_rng(2)
    rows = np.sort(rng.choice(2048, 8, replace=False)).tolist()
    cols = np.sort(rng.choice(2048, 8, replace=False)).tolist()
    for A in (ones, ua):
        base = run_debug(A, B, 14, want_prod=False, want_res=False)
        for s in (-64, -32, 0, 32, 64):
            As = np.ldexp(A, s)
            g = run_debug(As, B, 14, want_prod=False, want_res=False)
            assert np.array_equal(g["e"], base["e"] - s)
            assert_bitwise_equal(g["C"], np.ldexp(base["C"], s), f"scale 2^{s}")
        _sampled_exact_check(A, B, base["C"], base["e"].tolist(), base["f"].tolist(), rows, cols)


def test_scale_sweep_original_rule_stand_in():
    # The comparison stand-in for the original fast-mode rule ([G] Problemstellung;
    # not printed on the pages): its GPU exponents follow the oracle's binary32
    # rule (summation order may move a few by one), it collapses at alpha = 2^64
    # and is not scale invariant, while the proposed rule is. Logged, not gated
    # on accuracy.
    ones, ua, B = W.scale_sweep_case(2048)
    Pp = O.scaling_constant(math.prod(O.choose_moduli(14)))
    for A in (ones, ua):
        prev = None
        for s in (-64, -32, 0, 32, 64):
            As = np.ldexp(A, s)
            g = run_debug(As, B, 14, "original", want_prod=False, want_res=False)
            oe = O.original_exponents_rows(As, Pp)
            ge = g["e"].tolist()
            diff = [a - b for a, b in zip(ge, oe)]
            assert all(abs(d) <= 1 for d in diff) and sum(d != 0 for d in diff) <= 20, s
            if s == 64:
                assert all(v == O.EXP_COLLAPSE for v in ge) and np.all(g["C"] == 0.0)
            print(f"original rule, {'ones' if A is ones else 'U'}, alpha=2^{s}: e[0]={ge[0]}, "
                  f"C[0,0]={g['C'][0, 0]!r}")
            prev = ge


def test_config_spread1_16384_n18():
    # 16384^3, N = 18 (2 GiB per operand; |x| reaches 2^69.7, beyond int64):
    # every column exponent of B and the sampled rows' exponents of A (mismatch
    # protocol), the int8 residues of the sampled rows of A and columns of B,
    # and whole sampled rows of C bit for bit against os2_dgemm(A[rows], B),
    # plus the accuracy gate on three of them.
    A, B = W.make("spread1.0_16384_n18")
    m, k = A.shape
    n = B.shape[1]
    N = 18
    rng = np.random.default_rng(3)
    rows = np.sort(rng.choice(m, 6, replace=False)).tolist()
    cols = np.sort(rng.choice(n, 6, replace=False)).tolist()
    dA = device_colmajor(A)
    dB = device_colmajor(B)
    dC = torch.empty((n, m), dtype=torch.float64, device="cuda")
    wbytes = oz.ozaki2_debug_workspace_size(m, n, k, N, 0)
    ws = torch.empty(wbytes, dtype=torch.uint8, device="cuda")
    e = torch.empty(m, dtype=torch.int32, device="cuda")
    f = torch.empty(n, dtype=torch.int32, device="cuda")
    ra = torch.empty((N, m, k), dtype=torch.int8, device="cuda")
    rb = torch.empty((N, n, k), dtype=torch.int8, device="cuda")
    st = oz.ozaki2_dgemm_debug(m, n, k, dA.data_ptr(), m, dB.data_ptr(), k, dC.data_ptr(), m, N, 0, ws.data_ptr(),
                               wbytes, e.data_ptr(), f.data_ptr(), ra.data_ptr(), rb.data_ptr(), None, None,
                               stream_handle())
    assert st == 0
    torch.cuda.synchronize()
    del ws, dA, dB
    RA_s = ra[:, rows, :].cpu().numpy()
    RB_s = rb[:, cols, :].cpu().numpy()
    del ra, rb
    C_rows = dC[:, rows].cpu().numpy().T  # whole rows of C
    ge = e.cpu().numpy()
    gf = f.cpu().numpy()
    del dC
    r = O.os2_dgemm(A[rows], B, N)
    er, ne = reconcile_exponents(ge[rows], r["e"], A[rows], N, "fast")
    ef, nf = reconcile_exponents(gf, r["f"], B.T, N, "fast")
    if ne or nf:
        r = O.os2_dgemm(A[rows], B, N, e=er, f=ef)
    print(f"16384^3 N=18: exponent mismatches {ne + nf} of {len(rows) + n}")
    assert np.array_equal(RA_s, r["RA"]), "residues of the sampled rows of A differ"
    assert np.array_equal(RB_s, r["RB"][:, cols, :]), "residues of the sampled columns of B differ"
    assert_bitwise_equal(C_rows, r["C"], "sampled rows of C at 16384^3")
    P = math.prod(O.choose_moduli(N))
    assert np.all(2 * np.abs(r["X"]) <= P - 1)
    hi, lo = O.dd_gemm(A[rows[:3]], B)
    err = O.error_metrics(C_rows[:3], hi, lo, A[rows[:3]], B)
    print("16384^3 N=18:", err)
    assert err["E_cw"] <= 1e-14
