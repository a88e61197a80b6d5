"""Pins of the oracle's scaling constant, accurate-mode exponents and error
metrics (no GPU).

Each test states the planted mistake it was checked against: the mistake was
written into a scratch copy of the oracle function and the test failed on it.

Pages: [Q] the Qiita article on the Chinese remainder theorem and Ozaki
Scheme II; [G] "Improved Scaling for Fast Mode of Ozaki Scheme II".
"""
import math
from fractions import Fraction

import mpmath
import numpy as np
import pytest

import oracle as O
import workloads as W


# ---------------------------------------------------------------- P'
def test_scaling_constant_splits_the_range_condition_evenly():
    """P' is the largest double with 2^(2 P') <= (P - 1) / 2.

    [G] Methodik 1: with mu_i = 2^e_i and nu_j = 2^f_j each at most
    2^P' / ||row||, 2 mu ||a|| ||b|| nu <= 2 * 2^(2P') <= P - 1 ([Q] section
    時計の針で見る定理の中身: integers in (-P/2, P/2] are told apart).
    The integer part of 2P' is the bit length of (P - 1) / 2 minus one, which
    is exact integer arithmetic; the fractional part is compared at 120 digits
    (2^(2P') is irrational, so no finite Fraction holds it), where the working
    error is below 2^-390 and every margin below is above 2^-60.
    Planted: P' = 0.5 log2(P) (fails the bound) and P' = 0.5 log2((P-1)/2) - 2^-40
    (fails maximality).
    """
    for n in range(2, 21):
        P = math.prod(O.choose_moduli(n))
        H = Fraction(P - 1, 2)
        Pp = O.scaling_constant(P)
        two_pp = Fraction(Pp) * 2
        ip = math.floor(two_pp)
        assert ip == ((P - 1) // 2).bit_length() - 1, n  # exact: 2^ip <= (P-1)/2 < 2^(ip+1)
        nxt = Fraction(math.nextafter(Pp, math.inf)) * 2
        with mpmath.workdps(120):
            v = mpmath.mpf(2) ** (mpmath.mpf(two_pp.numerator) / two_pp.denominator)
            w = mpmath.mpf(2) ** (mpmath.mpf(nxt.numerator) / nxt.denominator)
            h = mpmath.mpf(H.numerator) / H.denominator
            assert v <= h * (1 - mpmath.mpf(2) ** -60), n
            assert w > h, n


def test_scaling_constant_worked_example_separates_the_readings():
    """A row of 3022 ones with 14 moduli gets e = 48.

    From first principles: e is the largest integer with
    2^(2e) * 3022 * 2^(4 u32) <= (P - 1) / 2; checked here in Python integers
    (2^(4 u32) < 1 + 2^-20 changes nothing at this margin). P' = 0.5 log2(P)
    would give 49, so this example tells the two readings apart, which the
    k = 2048 example (49 either way) does not.
    Planted: P' = 0.5 log2(P) gives 49.
    """
    P = math.prod(O.choose_moduli(14))
    Pp = O.scaling_constant(P)
    k = 3022
    e = O.fast_exponents_rows(np.ones((2, k)), Pp)
    assert e == [48, 48]
    H = (P - 1) // 2
    assert (1 << 96) * k * (1 + Fraction(1, 1 << 20)) <= H < (1 << 98) * k


# ---------------------------------------------------------------- accurate mode
def _accurate_from_first_principles(A, B, Pp):
    """Row/column exponents of the accurate-mode reading, computed with Python
    integers and Fractions only (no numpy arithmetic on the values):
    r_i = least integer with max_h |a_ih| < 2^r_i; Abar = ceil(|a| 2^(6 - r));
    W = Abar Bbar exactly; R_i = max_j W_ij; and e_i the LARGEST integer with
    2^(2 e_i + 2 r_i - 12) * R_i * 2^(4 u32) <= 2^(2 P'), i.e. the sufficient
    condition 2 sum_h |a'_ih||b'_hj| <= P - 1 split evenly, as in fast mode.
    The 2^(4 u32) and 2^(2P') factors are compared at 80 digits."""
    m, k = A.shape
    n = B.shape[1]

    def r_of(vals):
        mx = max((abs(Fraction(float(x))) for x in vals), default=Fraction(0))
        if mx == 0:
            return None
        r = 0
        while Fraction(2) ** r <= mx:
            r += 1
        while Fraction(2) ** (r - 1) > mx:
            r -= 1
        return r

    ra = [r_of(A[i]) for i in range(m)]
    cb = [r_of(B[:, j]) for j in range(n)]

    def bar(x, r):
        if r is None:
            return 0
        v = abs(Fraction(float(x))) * Fraction(2) ** (6 - r)
        return math.ceil(v)

    Ab = [[bar(A[i, h], ra[i]) for h in range(k)] for i in range(m)]
    Bb = [[bar(B[h, j], cb[j]) for h in range(k)] for j in range(n)]
    Wm = [[sum(a * b for a, b in zip(Ab[i], Bb[j])) for j in range(n)] for i in range(m)]
    R = [max(Wm[i]) if n else 0 for i in range(m)]
    C = [max(Wm[i][j] for i in range(m)) if m else 0 for j in range(n)]

    def largest(r, Rv):
        if Rv == 0:
            return 0
        with mpmath.workdps(80):
            lim = 2 * mpmath.mpf(Pp) - 4 * mpmath.mpf(O.U32) - mpmath.log(Rv, 2) - 2 * r + 12
            e = int(mpmath.floor(lim / 2))
            assert abs(lim / 2 - mpmath.nint(lim / 2)) > mpmath.mpf(2) ** -40, "boundary case: pick other data"
            return e

    return [largest(r, v) for r, v in zip(ra, R)], [largest(c, v) for c, v in zip(cb, C)]


@pytest.mark.parametrize("phi,N", [(0.5, 8), (1.0, 14), (2.0, 16)])
def test_accurate_exponents_are_the_largest_that_satisfy_the_bound(phi, N):
    """Maximality of the accurate-mode exponents ([G] Problemstellung, mode 1:
    one extra INT8 GEMM gives a tighter bound; the rule is our reading).

    The oracle's exponents must equal the largest integers that satisfy the
    reading's sufficient condition, recomputed from first principles (so one
    more bit on any row or column breaks it), and the exact range condition
    must hold on the truncated integers.
    Planted: '+ 5' for '+ 6' in the exponent; r_i one too large; R_i taken as
    the row sum of W instead of its maximum -- each fails here.
    """
    A, B = W.spread_case(12, 10, 40, phi, seed=21)
    A[3] = 0.0          # zero row: exponent 0
    B[:, 4] *= 2.0 ** 30  # a loud column
    P = math.prod(O.choose_moduli(N))
    Pp = O.scaling_constant(P)
    e, f, _ = O.accurate_exponents(A, B, Pp)
    we, wf = _accurate_from_first_principles(A, B, Pp)
    assert e == we
    assert f == wf
    Ai = np.abs(O.scaled_integers(A, e))
    Bi = np.abs(O.scaled_integers(B.T, f))
    assert np.all(2 * Ai.dot(Bi.T) <= P - 1)


def test_accurate_mode_is_about_as_accurate_as_fast_mode():
    """[G] Ergebnisse: the proposed fast mode reaches about the accuracy of the
    accurate mode. Pinned as E_cw(accurate) <= 2 E_cw(fast) over spreads
    phi in {0.5, 1, 2} and N in {8, 12, 14} on 48 x 512 x 40 products.
    Planted: every accurate exponent one smaller (e.g. '+ 5' for '+ 6') gives
    ratios up to about 3 and fails.
    """
    for phi in (0.5, 1.0, 2.0):
        A, B = W.spread_case(48, 40, 512, phi, seed=3)
        hi, lo = O.dd_gemm(A, B)
        for N in (8, 12, 14):
            ef = O.error_metrics(O.os2_dgemm(A, B, N, "fast")["C"], hi, lo, A, B)["E_cw"]
            ea = O.error_metrics(O.os2_dgemm(A, B, N, "accurate")["C"], hi, lo, A, B)["E_cw"]
            assert ea <= 2.0 * ef, (phi, N, ea, ef)


# ---------------------------------------------------------------- metrics
def test_error_metrics_hand_worked_2x2():
    """E_cw, E_el, E_nw on a 2 x 2 case worked by hand.

    A = [[1, -2], [0, 0]], B = [[3, 1], [1, 1]]: A B = [[1, -1], [0, 0]] and
    |A||B| = [[5, 3], [0, 0]]. The reference is the double-double
    hi + lo with hi = A B and lo(0,0) = 2^-54. C = [[1 + 2^-52, -1], [0, 0]]:
      |C - ref| = [[2^-52 - 2^-54, 0], [0, 0]] = [[3 * 2^-54, 0], [0, 0]];
      E_cw = max(3 * 2^-54 / 5, 0 / 3, 0/0 -> 0, 0/0 -> 0) = 3 * 2^-54 / 5;
      E_el = 3 * 2^-54 / |1| (the (1, *) entries are 0/0 -> 0);
      E_nw = ||diff||_F / ||ref||_F = 3 * 2^-54 / sqrt(2).
    A nonzero error where |A||B| = 0 counts as infinite.
    Planted: dropping lo (E_cw = 2^-52 / 5), normalising E_cw by |A B|
    (3 * 2^-54), and 0/0 -> NaN each fail here.
    """
    A = np.array([[1.0, -2.0], [0.0, 0.0]])
    B = np.array([[3.0, 1.0], [1.0, 1.0]])
    hi = np.array([[1.0, -1.0], [0.0, 0.0]])
    lo = np.array([[2.0 ** -54, 0.0], [0.0, 0.0]])
    C = np.array([[1.0 + 2.0 ** -52, -1.0], [0.0, 0.0]])
    m = O.error_metrics(C, hi, lo, A, B)
    d = 3.0 * 2.0 ** -54
    assert m["E_cw"] == d / 5.0
    assert m["E_el"] == d
    assert m["E_nw"] == pytest.approx(d / math.sqrt(2.0), rel=1e-15)
    C2 = C.copy()
    C2[1, 1] = 2.0 ** -1000
    assert O.error_metrics(C2, hi, lo, A, B)["E_cw"] == math.inf


# ---------------------------------------------------------------- CRT range check
@pytest.mark.parametrize("moduli,p_check", [([3, 5, 7], 11), ([256, 255], 253), ([4, 3, 5, 7], 11)])
def test_range_flags_brute_force(moduli, p_check):
    """Every integer Y in [-2P, 2P]: the flag is set exactly when Y lies outside
    (-P/2, P/2] ([Q] section 時計の針で見る定理の中身: such Y is read back as
    another number). Planted: a lift to [0, P) instead of (-P/2, P/2] flags
    the negative half and fails here (and in the table-edge test below)."""
    P = math.prod(moduli)
    Y = np.arange(-2 * P, 2 * P + 1, dtype=np.int64)
    c = np.stack([np.mod(Y, p) for p in moduli]).astype(np.int64)
    flags = O.crt_range_flags(c, np.mod(Y, p_check), moduli, p_check)
    outside = ~((2 * Y > -P) & (2 * Y <= P))
    assert np.array_equal(flags.astype(bool), outside)


def test_range_flags_with_the_table_edges():
    # N = 16 and its check modulus, the 17th of the table (191 in the footnote's order)
    N = 16
    moduli = O.choose_moduli(N)
    pc = O.check_modulus(N)
    assert pc == 191
    P = math.prod(moduli)
    H = P // 2
    Y = [0, 1, -1, H, -H + 1, H - 1, H + 1, -H, P, -P, 3 * H, 190 * P + 5]
    want = [0, 0, 0, 0, 0, 0, 1, 1, 1, 1, 1, 1]
    c = np.array([[y % p for y in Y] for p in moduli], dtype=object)
    flags = O.crt_range_flags(c, np.array([y % pc for y in Y], dtype=object), moduli, pc)
    assert flags.tolist() == want


def test_range_flags_catch_a_planted_exponent_error():
    # one bit too many on every row of a ones product: the reconstruction wraps
    # (X != Y everywhere) and the flags say so; with the right exponents none is set
    k, N = 2048, 14
    A = np.ones((4, k))
    B = np.ones((k, 4))
    moduli = O.choose_moduli(N)
    pc = O.check_modulus(N)
    e, f = O.exponents(A, B, N, "fast")
    for shift, want in ((0, 0), (1, 1)):
        ee = [v + shift for v in e]
        r = O.os2_dgemm(A, B, N, e=ee, f=f)
        Y = O.exact_scaled_product(A, B, r["e"], r["f"])
        flags = O.crt_range_flags(r["c"], np.mod(Y, pc), moduli, pc)
        assert np.all(flags == want)
        assert np.array_equal(flags.astype(bool), r["X"] != Y)
