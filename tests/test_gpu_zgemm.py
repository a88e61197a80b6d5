"""GPU parity of complex products (ozaki2_zgemm / ozaki2_cgemm) against the oracle.

[G] ("Improved Scaling for Fast Mode of Ozaki Scheme II") closes with the
remark that the approach carries over to complex products (ZGEMM/CGEMM). The
GPU path forms, per modulus, the three products of Gauss' trick on residue
planes of the real parts, imaginary parts and their sums; exponents, those
residue planes, the int32 products, their residues and C must all equal the
oracle's os2_zgemm bit for bit.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_util import INT32_MIN, assert_bitwise_equal, reconcile_exponents, stream_handle
import rns_emulated_fp64_amd as oz

pytestmark = pytest.mark.gpu


def complex_case(m, n, k, seed, phi=1.0):
    rng = np.random.default_rng(seed)
    parts = [W.spread_matrix(rng, shape, phi) for shape in ((m, k), (m, k), (k, n), (k, n))]
    return parts[0] + 1j * parts[1], parts[2] + 1j * parts[3]


def dev_complex(X, ld, single):
    """Column-major interleaved copy of complex X (rows x cols), leading dimension ld."""
    rows, cols = X.shape
    t = np.zeros((max(cols, 1), max(ld, 1), 2), dtype=np.float32 if single else np.float64)
    t[:cols, :rows, 0] = X.real.T
    t[:cols, :rows, 1] = X.imag.T
    return torch.from_numpy(t).cuda()


def run_complex(A, B, N, single=False, lda=None, ldb=None, ldc=None, want_prod=True):
    m, k = A.shape
    n = B.shape[1]
    lda, ldb, ldc = lda or max(m, 1), ldb or max(k, 1), ldc or max(m, 1)
    dA, dB = dev_complex(A, lda, single), dev_complex(B, ldb, single)
    dC = torch.full((max(n, 1), ldc, 2), float("nan"), dtype=torch.float32 if single else torch.float64,
                    device="cuda")
    wb = oz.ozaki2_zgemm_workspace_size(m, n, k, N, debug=True)
    ws = torch.empty(max(wb, 1), dtype=torch.uint8, device="cuda")
    e = torch.empty(max(m, 1), dtype=torch.int32, device="cuda")
    f = torch.empty(max(n, 1), dtype=torch.int32, device="cuda")
    ra = torch.empty((3 * N, m, k), dtype=torch.int8, device="cuda")
    rb = torch.empty((3 * N, n, k), dtype=torch.int8, device="cuda")
    prod = torch.empty((3 * N, n, m) if want_prod else (1,), dtype=torch.int32, device="cuda")
    red = torch.empty((3 * N, n, m), dtype=torch.uint8, device="cuda")
    fn = oz.ozaki2_cgemm_debug if single else oz.ozaki2_zgemm_debug
    st = fn(m, n, k, dA.data_ptr(), lda, dB.data_ptr(), ldb, dC.data_ptr(), ldc, N, oz.FAST, ws.data_ptr(), wb,
            e.data_ptr(), f.data_ptr(), ra.data_ptr(), rb.data_ptr(), prod.data_ptr() if want_prod else None,
            red.data_ptr(), stream_handle())
    assert st == 0, oz.status_string(st)
    torch.cuda.synchronize()
    c = dC.cpu().numpy()
    C = (c[:n, :m, 0] + 1j * c[:n, :m, 1]).T.astype(np.complex64 if single else np.complex128)
    out = dict(C=C, C_re=c[:n, :m, 0].T.copy(), C_im=c[:n, :m, 1].T.copy(), pad=c[:n, m:, :],
               e=e[:m].cpu().numpy(), f=f[:n].cpu().numpy(), RA=ra.cpu().numpy(), RB=rb.cpu().numpy(),
               red=red.cpu().numpy())
    if want_prod:
        out["Q"] = prod.cpu().numpy()
    return out


def complex_parity(A, B, N, single=False, **kw):
    g = run_complex(A, B, N, single, **kw)
    r = O.os2_zgemm(A, B, N, single=single)
    Ar = np.concatenate([A.real, A.imag], axis=1)
    Br = np.concatenate([B.real.T, B.imag.T], axis=1)
    e, ne = reconcile_exponents(g["e"], r["e"], Ar, N, "fast")
    f, nf = reconcile_exponents(g["f"], r["f"], Br, N, "fast")
    if ne or nf:
        r = O.os2_zgemm(A, B, N, e=e, f=f, single=single)
    okr = np.array([v is not None for v in r["e"]])
    okc = np.array([v is not None for v in r["f"]])
    for l in range(N):
        for gi, (ka, kb) in enumerate((("RAr", "RBr"), ("RAi", "RBi"), ("RAs", "RBs"))):
            assert np.array_equal(g["RA"][3 * l + gi][okr], r[ka][l][okr]), f"A residues l={l} g={gi}"
            assert np.array_equal(g["RB"][3 * l + gi][okc], r[kb][l][okc]), f"B residues l={l} g={gi}"
            sel = np.ix_(okr, okc)
            if "Q" in g:
                assert np.array_equal(g["Q"][3 * l + gi].T[sel], r["T"][l][gi][sel]), f"products l={l} g={gi}"
            assert np.array_equal(g["red"][3 * l + gi].T[sel], r["cT"][l][gi][sel]), f"reduced l={l} g={gi}"
    assert_bitwise_equal(g["C_re"], np.ascontiguousarray(r["C"].real), "Re C")
    assert_bitwise_equal(g["C_im"], np.ascontiguousarray(r["C"].imag), "Im C")
    return g, r


@pytest.mark.parametrize("N", [2, 8, 14, 16, 18, 20])
def test_zgemm_ragged(N):
    A, B = complex_case(300, 290, 260, seed=400 + N)
    complex_parity(A, B, N)


@pytest.mark.parametrize("N", [6, 8, 16, 18])
def test_cgemm_ragged(N):
    A, B = complex_case(270, 260, 200, seed=500 + N)
    g, r = complex_parity(A.astype(np.complex64), B.astype(np.complex64), N, single=True)
    assert g["C_re"].dtype == np.float32


@pytest.mark.parametrize("N", [8, 16])
@pytest.mark.parametrize("single", [False, True])
def test_zgemm_exact_zero_parts(N, single):
    # A = (1 + i) X and B = (1 + i) Y give A B = 2i X Y: the real part is exactly
    # zero although T1 = T2 is not, and must come out as +0 like RN(0); the
    # imaginary part of a zero row is zero from zero residues
    rng = np.random.default_rng(5)
    X = W.spread_matrix(rng, (70, 90), 1.0)
    Y = W.spread_matrix(rng, (90, 50), 1.0)
    X[4, :] = 0.0
    A, B = (1 + 1j) * X, (1 + 1j) * Y
    g, r = complex_parity(A, B, N, single)
    assert np.all(g["C_re"] == 0) and not np.any(np.signbit(g["C_re"]))
    assert np.all(g["C_im"][4] == 0) and not np.any(np.signbit(g["C_im"][4]))


@pytest.mark.parametrize("shape", [(1, 1, 1), (1, 7, 3), (33, 17, 129), (64, 64, 1)])
def test_zgemm_tiny_shapes(shape):
    A, B = complex_case(*shape, seed=sum(shape))
    complex_parity(A, B, 16)
    complex_parity(A.astype(np.complex64), B.astype(np.complex64), 8, single=True)


def test_zgemm_leading_dimensions_and_special_values():
    A, B = complex_case(257, 130, 190, seed=31)
    A[3, 5] = complex(np.inf, 1.0)
    A[7] = 0.0
    A[9] *= 2.0 ** 300
    B[4, 11] = complex(0.0, np.nan)
    B[:, 2] = 0.0
    B[:, 8] *= 2.0 ** -600
    g, r = complex_parity(A, B, 16, lda=300, ldb=211, ldc=260)
    assert np.all(np.isnan(g["C_re"][3])) and np.all(np.isnan(g["C_im"][:, 11]))
    assert np.all(np.isnan(g["pad"]))  # rows m..ldc of C untouched


def test_zgemm_full_512_accuracy():
    A, B = complex_case(512, 512, 512, seed=41)
    g, r = complex_parity(A, B, 16, want_prod=False)
    rr = [O.dd_gemm(X, Y) for X, Y in ((A.real, B.real), (A.imag, B.imag), (A.real, B.imag), (A.imag, B.real))]
    ref_r = (rr[0][0] - rr[1][0]) + (rr[0][1] - rr[1][1])
    ref_i = (rr[2][0] + rr[3][0]) + (rr[2][1] + rr[3][1])
    scale = np.abs(A) @ np.abs(B)
    ecw = lambda C: float(np.max(np.maximum(np.abs(C.real - ref_r), np.abs(C.imag - ref_i)) / scale))
    print(f"512^3 ZGEMM N=16: E_cw {ecw(g['C']):.3e}, native complex128 {ecw(A @ B):.3e}")
    assert ecw(g["C"]) <= ecw(A @ B)


def test_zgemm_k_zero_and_ws_entry():
    A, B = complex_case(40, 30, 0, seed=2)
    dC = torch.full((30, 40, 2), 5.0, dtype=torch.float64, device="cuda")
    st = oz.ozaki2_zgemm(40, 30, 0, 1 << 20, 40, 1 << 20, 1, dC.data_ptr(), 40, 8, oz.FAST, stream_handle())
    assert st == 0
    torch.cuda.synchronize()
    assert torch.all(dC == 0.0)
    # the workspace entry point gives the debug entry point's bits
    A, B = complex_case(100, 90, 80, seed=3)
    g = run_complex(A, B, 8, want_prod=False)
    dA, dB = dev_complex(A, 100, False), dev_complex(B, 80, False)
    dC = torch.empty((90, 100, 2), dtype=torch.float64, device="cuda")
    wb = oz.ozaki2_zgemm_workspace_size(100, 90, 80, 8)
    ws = torch.empty(wb, dtype=torch.uint8, device="cuda")
    st = oz.ozaki2_zgemm_ws(100, 90, 80, dA.data_ptr(), 100, dB.data_ptr(), 80, dC.data_ptr(), 100, 8, oz.FAST,
                            ws.data_ptr(), wb, stream_handle())
    assert st == 0
    torch.cuda.synchronize()
    c = dC.cpu().numpy()
    assert_bitwise_equal(c[:, :, 0].T.copy(), g["C_re"], "ws Re")
    assert_bitwise_equal(c[:, :, 1].T.copy(), g["C_im"], "ws Im")


def test_zgemm_config_4096_n16():
    # the complex workload at full size, in the benchmark's launch configuration
    A, B = W.make("zgemm_spread1.0_4096_n16")
    m, k = A.shape
    n = B.shape[1]
    N = 16
    dA, dB = dev_complex(A, m, False), dev_complex(B, k, False)
    dC = torch.empty((n, m, 2), dtype=torch.float64, device="cuda")
    wb = oz.ozaki2_zgemm_workspace_size(m, n, k, N, debug=True)
    ws = torch.empty(wb, dtype=torch.uint8, device="cuda")
    e = torch.empty(m, dtype=torch.int32, device="cuda")
    f = torch.empty(n, dtype=torch.int32, device="cuda")
    st = oz.ozaki2_zgemm_debug(m, n, k, dA.data_ptr(), m, dB.data_ptr(), k, dC.data_ptr(), m, N, oz.FAST,
                               ws.data_ptr(), wb, e.data_ptr(), f.data_ptr(), None, None, None, None, stream_handle())
    assert st == 0
    del ws
    wb2 = oz.ozaki2_zgemm_workspace_size(m, n, k, N)
    ws2 = torch.empty(wb2, dtype=torch.uint8, device="cuda")
    dC2 = torch.empty((n, m, 2), dtype=torch.float64, device="cuda")
    st = oz.ozaki2_zgemm_ws(m, n, k, dA.data_ptr(), m, dB.data_ptr(), k, dC2.data_ptr(), m, N, oz.FAST,
                            ws2.data_ptr(), wb2, stream_handle())
    assert st == 0
    torch.cuda.synchronize()
    assert torch.equal(dC.view(torch.int64), dC2.view(torch.int64)), "ws vs debug"
    del ws2, dC2
    ge, gf = e.cpu().numpy().tolist(), f.cpu().numpy().tolist()
    rng = np.random.default_rng(11)
    rows = np.sort(rng.choice(m, 12, replace=False)).tolist()
    cols = np.sort(rng.choice(n, 12, replace=False)).tolist()
    Pp = O.scaling_constant(math.prod(O.choose_moduli(N)))
    oe = O.complex_exponents_rows(A.real[rows], A.imag[rows], Pp)
    of = O.complex_exponents_rows(B.real[:, cols].T, B.imag[:, cols].T, Pp)
    assert sum(a != b for a, b in zip(oe, [ge[i] for i in rows])) <= 1
    assert sum(a != b for a, b in zip(of, [gf[j] for j in cols])) <= 1
    er, fc = [ge[i] for i in rows], [gf[j] for j in cols]
    Xr, Xi = O.exact_complex_scaled_product(A[rows], B[:, cols], er, fc)
    Cs = dC[cols][:, rows].cpu().numpy()  # [col][row][part]
    ref_r = O.unscale(Xr, er, fc)
    ref_i = O.unscale(Xi, er, fc)
    assert_bitwise_equal(np.ascontiguousarray(Cs[:, :, 0].T), ref_r, "sampled Re C")
    assert_bitwise_equal(np.ascontiguousarray(Cs[:, :, 1].T), ref_i, "sampled Im C")


@pytest.mark.parametrize("single", [False, True])
def test_complex_torch_wrappers(single):
    # row-major torch complex tensors: the wrapper swaps the operands, the
    # result must equal the oracle's C bit for bit
    A, B = complex_case(70, 90, 110, seed=31)
    if single:
        A, B = A.astype(np.complex64), B.astype(np.complex64)
    dA, dB = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    fn = oz.cgemm if single else oz.zgemm
    C = fn(dA, dB, 16).cpu().numpy()
    r = O.os2_zgemm(A.astype(np.complex128), B.astype(np.complex128), 16, single=single)
    assert_bitwise_equal(np.ascontiguousarray(C.real), np.ascontiguousarray(r["C"].real), "torch Re C")
    assert_bitwise_equal(np.ascontiguousarray(C.imag), np.ascontiguousarray(r["C"].imag), "torch Im C")
    # a caller-provided output and workspace give the same bits
    out = torch.empty((70, 90), dtype=dA.dtype, device="cuda")
    ws = torch.empty(oz.ozaki2_zgemm_workspace_size(90, 70, 110, 16), dtype=torch.uint8, device="cuda")
    fn(dA, dB, 16, out=out, workspace=ws)
    assert np.array_equal(out.cpu().numpy().view(np.uint8), C.view(np.uint8))


def test_torch_wrapper_rejects_bad_out():
    dA = torch.zeros((8, 5), dtype=torch.float64, device="cuda")
    dB = torch.zeros((5, 6), dtype=torch.float64, device="cuda")
    for bad in (torch.empty((6, 8), dtype=torch.float64, device="cuda"),
                torch.empty((8, 6), dtype=torch.float32, device="cuda"),
                torch.empty((6, 8), dtype=torch.float64, device="cuda").t()):
        with pytest.raises(ValueError):
            oz.dgemm(dA, dB, 8, out=bad)
    with pytest.raises(TypeError):
        oz.zgemm(dA, dB, 8)
