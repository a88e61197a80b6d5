"""Helpers shared by the GPU tests: move operands to the device, call the
C ABI (through the thin binding), bring intermediates back, and compare with
the oracle following the exponent-mismatch protocol.

Exponents are compared for equality. A GPU exponent may differ from the
oracle's only where the floor argument of the scaling formula lies within a
few ulps of an integer (the two sides sum the squares in different orders and
use different log2 routines). Such a row is accepted only if its exponent is
valid to 60 digits; the oracle then re-splits with the GPU exponents and every
later stage must still match bit for bit."""
from __future__ import annotations

import math

import mpmath
import numpy as np
import torch

import oracle as O
import rns_emulated_fp64_amd as oz

INT32_MIN = -(2 ** 31)


def device_colmajor(X: np.ndarray, ld: int | None = None) -> torch.Tensor:
    """Column-major copy of X (rows x cols) on the GPU with leading dimension ld
    (float32 for a float32 X, else float64)."""
    rows, cols = X.shape
    ld = max(rows, 1) if ld is None else ld
    dt = torch.float32 if X.dtype == np.float32 else torch.float64
    t = torch.zeros((max(cols, 1), ld), dtype=dt)
    if rows and cols:
        t[:cols, :rows] = torch.from_numpy(np.ascontiguousarray(X.T))
    return t.cuda()


def stream_handle() -> int:
    return torch.cuda.current_stream().cuda_stream


def run_debug(A, B, N, mode="fast", lda=None, ldb=None, ldc=None, want_prod=True, want_res=True):
    """One ozaki2_dgemm_debug call (ozaki2_sgemm_debug for float32 operands);
    returns numpy copies of C and intermediates."""
    single = A.dtype == np.float32
    m, k = A.shape
    n = B.shape[1]
    md = oz.MODES[mode]
    lda = max(m, 1) if lda is None else lda
    ldb = max(k, 1) if ldb is None else ldb
    ldc = max(m, 1) if ldc is None else ldc
    dA = device_colmajor(A, lda)
    dB = device_colmajor(B, ldb)
    dC = torch.full((max(n, 1), ldc), float("nan"), dtype=torch.float32 if single else torch.float64,
                    device="cuda")
    wbytes = oz.ozaki2_debug_workspace_size(m, n, k, N, md)
    ws = torch.empty(max(wbytes, 1), dtype=torch.uint8, device="cuda")
    e = torch.empty(max(m, 1), dtype=torch.int32, device="cuda")
    f = torch.empty(max(n, 1), dtype=torch.int32, device="cuda")
    ra = torch.empty((N, m, k) if want_res else (1,), dtype=torch.int8, device="cuda")
    rb = torch.empty((N, n, k) if want_res else (1,), dtype=torch.int8, device="cuda")
    prod = torch.empty((N, n, m) if want_prod else (1,), dtype=torch.int32, device="cuda")
    red = torch.empty((N, n, m), dtype=torch.uint8, device="cuda")
    debug = oz.ozaki2_sgemm_debug if single else oz.ozaki2_dgemm_debug
    st = debug(m, n, k, dA.data_ptr(), lda, dB.data_ptr(), ldb, dC.data_ptr(), ldc, N, md,
               ws.data_ptr(), wbytes, e.data_ptr(), f.data_ptr(),
               ra.data_ptr() if want_res else None, rb.data_ptr() if want_res else None,
               prod.data_ptr() if want_prod else None, red.data_ptr(), stream_handle())
    assert st == 0, oz.status_string(st)
    torch.cuda.synchronize()
    out = dict(C=dC[:n, :m].cpu().numpy().T.copy() if n and m else np.zeros((m, n), dtype=A.dtype),
               e=e[:m].cpu().numpy(), f=f[:n].cpu().numpy(), red=red.cpu().numpy())
    if want_res:
        out["RA"] = ra.cpu().numpy()
        out["RB"] = rb.cpu().numpy()
    if want_prod:
        out["Q"] = prod.cpu().numpy()
    out["C_padding"] = dC.cpu().numpy()
    return out


def run_ws(A, B, N, mode="fast"):
    """ozaki2_dgemm_ws (ozaki2_sgemm_ws for float32) on freshly uploaded operands; returns C (numpy)."""
    single = A.dtype == np.float32
    m, k = A.shape
    n = B.shape[1]
    md = oz.MODES[mode]
    dA = device_colmajor(A)
    dB = device_colmajor(B)
    dC = torch.empty((max(n, 1), max(m, 1)), dtype=torch.float32 if single else torch.float64, device="cuda")
    wbytes = oz.ozaki2_workspace_size(m, n, k, N, md)
    ws = torch.empty(max(wbytes, 1), dtype=torch.uint8, device="cuda")
    fn = oz.ozaki2_sgemm_ws if single else oz.ozaki2_dgemm_ws
    st = fn(m, n, k, dA.data_ptr(), max(m, 1), dB.data_ptr(), max(k, 1), dC.data_ptr(), max(m, 1),
            N, md, ws.data_ptr(), wbytes, stream_handle())
    assert st == 0, oz.status_string(st)
    torch.cuda.synchronize()
    return dC[:n, :m].cpu().numpy().T.copy()


def to_oracle_exponents(v: np.ndarray) -> list:
    return [None if int(x) == INT32_MIN else int(x) for x in v]


def exponent_is_valid(row: np.ndarray, e: int, Pp: float) -> bool:
    """Is e the fast-mode exponent of row, up to rounding at the boundary?

    z = P' - 0.5 (log2 sum row^2 + 4 u32) is evaluated at 60 digits. Away
    from an integer e must be floor(z). Within 2^-40 of an integer n (where
    the two sides' summation orders and log2 routines may round z to either
    side) e may be n - 1 or n, never n + 1: an exponent above floor(z + 2^-40)
    would break the bound of [G] Methodik by more than rounding.
    """
    with mpmath.workdps(60):
        s = mpmath.fsum(mpmath.mpf(float(x)) ** 2 for x in row)
        if s == 0:
            return e == 0
        z = mpmath.mpf(Pp) - (mpmath.log(s, 2) + 4 * mpmath.mpf(O.U32)) / 2
        n = int(mpmath.nint(z))
        if abs(z - n) < mpmath.mpf(2) ** -40:
            return e in (n - 1, n)
        return e == int(mpmath.floor(z))


def reconcile_exponents(gpu_e: np.ndarray, orc_e: list, X: np.ndarray, N: int, mode: str):
    """Protocol: equality expected; a mismatch must be a valid boundary case."""
    ge = to_oracle_exponents(gpu_e)
    bad = [i for i, (a, b) in enumerate(zip(ge, orc_e)) if a != b]
    if bad:
        assert mode == "fast", f"accurate-mode exponent mismatch at rows {bad[:8]}"
        Pp = O.scaling_constant(math.prod(O.choose_moduli(N)))
        for i in bad:
            assert orc_e[i] is not None and ge[i] is not None
            assert abs(ge[i] - orc_e[i]) == 1
            assert exponent_is_valid(X[i], ge[i], Pp), (i, ge[i], orc_e[i])
    return ge, len(bad)


def assert_bitwise_equal(a: np.ndarray, b: np.ndarray, what: str):
    assert a.shape == b.shape, (what, a.shape, b.shape)
    na, nb = np.isnan(a), np.isnan(b)
    assert np.array_equal(na, nb), f"{what}: NaN positions differ"
    assert a.dtype == b.dtype, (what, a.dtype, b.dtype)
    bits = np.uint32 if a.dtype == np.float32 else np.uint64
    av = np.where(na, a.dtype.type(0), a).view(bits)
    bv = np.where(nb, b.dtype.type(0), b).view(bits)
    if not np.array_equal(av, bv):
        idx = np.argwhere(av != bv)
        i = tuple(idx[0])
        raise AssertionError(f"{what}: {len(idx)} entries differ, first at {i}: {a[i]!r} vs {b[i]!r}")


def full_parity(A, B, N, mode="fast", **kw):
    """Debug run on the GPU vs the oracle at every stage; returns (gpu, oracle, mismatches).
    float32 operands go through ozaki2_sgemm_debug and the oracle's os2_sgemm."""
    emul = O.os2_sgemm if A.dtype == np.float32 else O.os2_dgemm
    g = run_debug(A, B, N, mode, **kw)
    r = emul(A, B, N, mode)
    e, ne = reconcile_exponents(g["e"], r["e"], A.astype(np.float64), N, mode)
    f, nf = reconcile_exponents(g["f"], r["f"], np.asarray(B, dtype=np.float64).T, N, mode)
    if ne or nf:
        r = emul(A, B, N, mode, e=e, f=f)
    okr = np.array([v is not None for v in r["e"]])
    okc = np.array([v is not None for v in r["f"]])
    assert np.array_equal(g["RA"][:, okr, :], r["RA"][:, okr, :]), "int8 residues of A differ"
    assert np.array_equal(g["RB"][:, okc, :], r["RB"][:, okc, :]), "int8 residues of B differ"
    if "Q" in g:
        Qg = g["Q"].transpose(0, 2, 1)
        assert np.array_equal(Qg[:, okr][:, :, okc], r["Q"][:, okr][:, :, okc]), "int32 residue products differ"
    cg = g["red"].transpose(0, 2, 1)
    assert np.array_equal(cg[:, okr][:, :, okc], r["c"][:, okr][:, :, okc]), "reduced residues differ"
    assert_bitwise_equal(g["C"], r["C"], "C")
    return g, r, ne + nf
