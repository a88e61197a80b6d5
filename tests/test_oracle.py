"""Pins of the CPU oracle against the pages and the mathematics (no GPU).

Every test here checks the oracle against something other than itself: the
values the pages print (tests/golden/*.json, each with its citation), closed
forms, brute force on tiny inputs, exact rational arithmetic, or a library
routine computing the same textbook quantity. Together they are meant to fail
on a dropped term, a wrong sign or index, or a transposed operand anywhere in
the oracle.

Pages: [Q] the Qiita article on the Chinese remainder theorem and Ozaki
Scheme II; [G] "Improved Scaling for Fast Mode of Ozaki Scheme II".
"""
import itertools
import json
import math
import os
from fractions import Fraction

import mpmath
import numpy as np
import pytest

import oracle as O
import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as fh:
        return json.load(fh)


# ---------------------------------------------------------------- tables
def test_sunzi_tables_and_answer():
    g = gold("sunzi.json")
    t = O.crt_tables(g["moduli"])
    assert t["P"] == g["P_yanmu"]
    assert t["M"] == g["M_yanshu"]
    assert t["G"] == g["G_jishu"]
    assert t["K"] == g["K_chenglv"]
    assert t["W"] == g["W_yongshu"]
    s = sum(w * r for w, r in zip(t["W"], g["residues"]))
    assert s == g["weighted_sum"]
    assert s - g["turns_removed"] * t["P"] == g["answer"]
    c = np.array(g["residues"], dtype=np.uint8).reshape(3, 1)
    assert O.crt(c, t)[0] == g["answer"]
    assert O.garner(c, g["moduli"])[0] == g["answer"]


def test_worked_inverse():
    w = gold("sunzi.json")["worked_inverse"]
    k = O.dayan_qiuyi(w["jishu"], w["dingmu"])
    assert k == w["chenglv"]
    assert w["yanshu"] * k == w["yongshu"]


def test_dayan_qiuyi_against_modular_inverse():
    # The procedure is the extended Euclidean algorithm; Python's pow(g, -1, p)
    # computes the same inverse independently.
    for p in range(2, 300):
        for g in range(1, p):
            if math.gcd(g, p) == 1:
                assert O.dayan_qiuyi(g, p) == pow(g, -1, p), (g, p)
    with pytest.raises(ValueError):
        O.dayan_qiuyi(4, 8)


def test_weights_advance_one_clock():
    # Each 用数 is 1 on its own clock and 0 on every other one.
    for n in (2, 8, 16, 20):
        t = O.crt_tables(O.choose_moduli(n))
        for l, w in enumerate(t["W"]):
            for j, p in enumerate(t["moduli"]):
                assert w % p == (1 if j == l else 0)
            assert 0 < w < t["P"]


def test_moduli_match_implementation_table():
    g = gold("moduli.json")
    assert O.choose_moduli(20) == g["implementation_order"]
    for n in range(1, 21):
        assert O.choose_moduli(n) == g["implementation_order"][:n]
    mods = g["implementation_order"]
    for a, b in itertools.combinations(mods, 2):
        assert math.gcd(a, b) == 1
    assert sum(1 for p in mods if p % 2 == 0) == 1
    for p, factors in g["composites"].items():
        assert math.prod(factors) == int(p) and int(p) in mods


def test_log2P_values_printed():
    g = gold("moduli.json")
    P16 = math.prod(O.choose_moduli(16))
    assert abs(math.log2(P16) - g["log2P_first16_implementation"]) < 0.05
    assert round(math.log2(math.prod(g["article_list_16_without_241"]))) == g["log2P_article_list"]
    lo, hi = g["primes_only_16_range"]
    primes = [p for p in range(lo, hi + 1) if all(p % d for d in range(2, int(p ** 0.5) + 1))]
    assert len(primes) == 16
    assert round(math.log2(math.prod(primes))) == g["log2P_primes_only"]
    # each modulus adds a little under 8 bits ([Q] section 行列積の回数と性能)
    for p in O.choose_moduli(20):
        assert 7.4 < math.log2(p) <= 8


def test_scaling_constant_definition():
    # P' is the largest double not above 0.5*log2((P-1)/2).
    for n in range(2, 21):
        P = math.prod(O.choose_moduli(n))
        d = O.scaling_constant(P)
        with mpmath.workdps(100):
            v = mpmath.log(mpmath.mpf(P - 1) / 2, 2) / 2
            assert mpmath.mpf(d) <= v
            assert mpmath.mpf(math.nextafter(d, math.inf)) > v


# ---------------------------------------------------------------- CRT
def _brute(moduli):
    t = O.crt_tables(moduli)
    P = t["P"]
    xs = np.arange(-(P // 2) + (1 if P % 2 == 0 else 0), P // 2 + 1, dtype=np.int64)
    assert len(xs) == P
    c = np.stack([np.mod(xs, p) for p in moduli]).astype(np.uint8)
    return xs, c, t


@pytest.mark.parametrize("moduli", [[3, 5, 7], [4, 3, 5, 7], [256, 255], [7, 11, 13, 16], [256, 3, 5]])
def test_crt_round_trip_brute_force(moduli):
    # [Q] section 定理が保証すること: every residue tuple has exactly one
    # integer in a range of P consecutive integers (here the symmetric one).
    xs, c, t = _brute(moduli)
    X = O.crt(c, t)
    assert np.all(X.astype(np.int64) == xs)
    G = O.garner(c, moduli)
    assert np.all(G.astype(np.int64) == xs)
    # distinct tuples == P
    assert len({tuple(col) for col in c.T.tolist()}) == t["P"]


def test_non_coprime_clocks_distinguish_only_four():
    # [Q] section 時計の針で見る定理の中身: clocks with 2 and 4 marks both
    # return to 0 at 4, so only 4 numbers can be told apart.
    tuples = {(x % 2, x % 4) for x in range(100)}
    assert len(tuples) == 4


def test_symmetric_residue_ranges():
    g = gold("moduli.json")
    xs = np.arange(-1000, 1001, dtype=np.float64).reshape(1, -1)
    r7 = O.split(xs, [0], [7])[0, 0]
    lo, hi = g["symmetric_example"]["range"]
    assert r7.min() == lo and r7.max() == hi
    assert np.all(np.mod(xs[0] - r7, 7) == 0)
    mods = O.choose_moduli(20)
    R = O.split(xs, [0], mods)
    assert R.min() >= g["int8_range"][0] and R.max() <= g["int8_range"][1]
    for l, p in enumerate(mods):
        assert np.all(np.mod(xs[0] - R[l, 0], p) == 0)
        if p % 2:
            assert np.abs(R[l, 0]).max() <= (p - 1) // 2
    # 256: residue 128 is stored as -128 (the same clock position)
    r256 = O.split(np.array([[128.0, -128.0, 127.0, 384.0, -129.0]]), [0], [256])[0, 0]
    assert r256.tolist() == [-128, -128, 127, -128, 127]


def test_int32_exactness_limit():
    # [Q] section 誤差のないINT8行列積(手順3): |int8 * int8| <= 16384 and the sum
    # stays in int32 while the inner dimension is below 2^17.
    klim = gold("moduli.json")["int32_exact_k_limit"]
    assert klim == 2 ** 17
    assert 128 * 128 * (klim - 1) < 2 ** 31 <= 128 * 128 * klim
    RA = np.full((1, 1, 4), -128, dtype=np.int8)
    RB = np.full((1, 1, 4), -128, dtype=np.int8)
    assert O.residue_products(RA, RB)[0, 0, 0] == 4 * 16384


def test_split_round_trip_and_homomorphism():
    A, B = W.spread_case(40, 24, 72, 1.0, seed=3)
    for N in (8, 14, 18):
        r = O.os2_dgemm(A, B, N)
        t = r["tables"]
        Ai = O.scaled_integers(A, r["e"])
        cA = np.stack([np.mod(r["RA"][l].astype(np.int64), p) for l, p in enumerate(r["moduli"])]).astype(np.uint8)
        assert np.all(O.crt(cA, t) == Ai)  # |A'| < P/2, so CRT returns A'
        Y = O.exact_scaled_product(A, B, r["e"], r["f"])
        for l, p in enumerate(r["moduli"]):
            assert np.all(np.mod(r["Q"][l].astype(object), p) == np.mod(Y, p))
        assert np.all(2 * np.abs(Y) <= t["P"] - 1)
        assert np.all(r["X"] == Y)
        assert np.all(O.garner(r["c"], r["moduli"]) == Y)


def test_product_orientation():
    # A non-square case where a transposed operand would give the wrong shape or values.
    A, B = W.uniform_case(5, 3, 9, seed=11)
    r = O.os2_dgemm(A, B, 16)
    assert r["C"].shape == (5, 3)
    hi, lo = O.dd_gemm(A, B)
    assert np.max(np.abs(r["C"] - hi)) < 1e-14


# ---------------------------------------------------------------- exponents
def test_exponent_worked_example_ones():
    # A = ones, k = 2048, N = 14: floor(P' - 0.5*(log2(2048) + 4u32)) = 49.
    P = math.prod(O.choose_moduli(14))
    Pp = O.scaling_constant(P)
    e = O.fast_exponents_rows(np.ones((3, 2048)), Pp)
    assert e == [49, 49, 49]
    assert math.floor(Pp - 0.5 * (math.log2(2048) + 4 * O.U32)) == 49


def test_exponent_exact_characterization():
    # e_i = floor(P' - 0.5*(log2(sum_h a_ih^2) + 4 u32)) evaluated at 60 digits.
    rng = np.random.default_rng(5)
    P = math.prod(O.choose_moduli(16))
    Pp = O.scaling_constant(P)
    for phi in (0.0, 1.0, 4.0):
        X = W.spread_matrix(rng, (64, 300), phi)
        X[3] = 0.0
        X[4, :] = 0.0
        X[4, 7] = 2.0 ** -1070  # subnormal-only row
        X[5] *= 2.0 ** 600      # would overflow a plain sum of squares
        e = O.fast_exponents_rows(X, Pp)
        with mpmath.workdps(60):
            for i, row in enumerate(X):
                if not np.any(row):
                    assert e[i] == 0
                    continue
                s = mpmath.fsum(mpmath.mpf(float(x)) ** 2 for x in row)
                z = mpmath.mpf(Pp) - (mpmath.log(s, 2) + 4 * mpmath.mpf(O.U32)) / 2
                fl = int(mpmath.floor(z))
                if abs(z - mpmath.nint(z)) > mpmath.mpf(2) ** -30:
                    assert e[i] == fl, (i, e[i], z)
                else:
                    assert e[i] in (fl, fl - 1)


def test_fast_mode_cauchy_schwarz_invariant():
    # [G] section Methodik, 1.: 2 mu_i ||a_i|| ||b_j|| nu_j <= P - 1, checked on
    # the truncated integers in the form actually needed: 2 sum |a'||b'| <= P-1.
    A, B = W.spread_case(24, 20, 160, 2.0, seed=7)
    for N in (6, 10, 14, 16):
        P = math.prod(O.choose_moduli(N))
        e, f = O.exponents(A, B, N, "fast")
        Ai = np.abs(O.scaled_integers(A, e))
        Bi = np.abs(O.scaled_integers(B.T, f))
        assert np.all(2 * Ai.dot(Bi.T) <= P - 1)
        # maximality: one more bit on a row breaks the norm condition
        # 2^(2(e+1)) ||a||^2 <= 2^(2P') (the characterization test pins e itself)
        Pp = O.scaling_constant(P)
        for i in range(A.shape[0]):
            s = sum(Fraction(float(x)) ** 2 for x in A[i])
            assert float(Fraction(2) ** (2 * (e[i] + 1)) * s) > 2.0 ** (2 * Pp) * 2.0 ** (-4 * O.U32) * 0.999999


def test_scale_invariance_exponents_and_result():
    # [G] section Methodik, 2.: with A -> 2^s A the log2(alpha) term cancels;
    # here bit for bit: e(2^s A) = e(A) - s and C(2^s A) = 2^s C(A).
    _, ua, b = W.scale_sweep_case(size=48, seed=0)
    for A in (np.ones((48, 48)), ua):
        base = O.os2_dgemm(A, b, 14)
        for s in (-64, -32, 0, 32, 64):
            As = np.ldexp(A, s)
            r = O.os2_dgemm(As, b, 14)
            assert r["e"] == [v - s for v in base["e"]]
            assert r["f"] == base["f"]
            assert np.array_equal(r["C"], np.ldexp(base["C"], s))
            Y = O.exact_scaled_product(As, b, r["e"], r["f"])
            assert np.all(r["X"] == Y)  # CRT succeeds at every alpha


def test_scale_invariance_extreme_exponents():
    A, B = W.uniform_case(8, 6, 32, seed=2)
    base = O.os2_dgemm(A, B, 16)
    for s in (-900, -500, 500, 900):
        r = O.os2_dgemm(np.ldexp(A, s), B, 16)
        assert r["e"] == [v - s for v in base["e"]]
        assert np.array_equal(r["C"], np.ldexp(base["C"], s))


def test_accurate_mode_invariants():
    A, B = W.spread_case(32, 28, 200, 1.5, seed=9)
    A[2] = 0.0
    for N in (8, 14, 16):
        P = math.prod(O.choose_moduli(N))
        r = O.os2_dgemm(A, B, N, "accurate")
        assert r["e"][2] == 0
        Ai = np.abs(O.scaled_integers(A, r["e"]))
        Bi = np.abs(O.scaled_integers(B.T, r["f"]))
        assert np.all(2 * Ai.dot(Bi.T) <= P - 1)
        assert np.all(r["X"] == O.exact_scaled_product(A, B, r["e"], r["f"]))
        # Abar, Bbar are upper bounds of |A|, |B| on the 2^(r-6) grid
        ra, cb, abar, bbar = O.accurate_bound_operands(A, B)
        assert abar.max() <= 64 and bbar.max() <= 64
        assert np.all(np.ldexp(abar, (ra - 6)[:, None]) >= np.abs(A))
        for s in (-40, 40):
            rs = O.os2_dgemm(np.ldexp(A, s), B, N, "accurate")
            # the zero row keeps exponent 0; every other row shifts by -s
            assert rs["e"] == [0 if i == 2 else v - s for i, v in enumerate(r["e"])]
            assert np.array_equal(rs["C"], np.ldexp(r["C"], s))


# ---------------------------------------------------------------- results
def test_small_integers_give_the_exact_product():
    rng = np.random.default_rng(4)
    A = rng.integers(-3, 4, (30, 50)).astype(np.float64)
    B = rng.integers(-3, 4, (50, 20)).astype(np.float64)
    exact = (A.astype(np.int64) @ B.astype(np.int64)).astype(np.float64)
    for N, mode in ((8, "fast"), (14, "fast"), (14, "accurate")):
        assert np.array_equal(O.os2_dgemm(A, B, N, mode)["C"], exact)
    k = 2048
    C = O.os2_dgemm(np.ones((4, k)), np.ones((k, 3)), 14)["C"]
    assert np.all(C == k)


def test_zero_rows_and_nonfinite():
    A, B = W.uniform_case(6, 5, 12, seed=1)
    A[1] = 0.0
    B[:, 2] = 0.0
    A[3, 4] = np.inf
    B[7, 4] = np.nan
    r = O.os2_dgemm(A, B, 14)
    C = r["C"]
    assert np.all(C[1, [0, 1, 3]] == 0.0)
    assert np.all(C[[0, 2, 4, 5], 2] == 0.0)
    assert np.all(np.isnan(C[3])) and np.all(np.isnan(C[:, 4]))
    good = np.ix_([0, 2, 4, 5], [0, 1, 3])
    hi, lo = O.dd_gemm(A[[0, 2, 4, 5]], B[:, [0, 1, 3]])
    assert np.max(np.abs(C[good] - hi)) < 1e-14
    # accurate mode: the Inf/NaN lines take no part in the bound product
    ra = O.os2_dgemm(A, B, 14, "accurate")
    assert ra["e"][3] is None and ra["f"][4] is None
    assert all(v is not None for i, v in enumerate(ra["e"]) if i != 3)
    assert np.all(np.isnan(ra["C"][3])) and np.all(np.isnan(ra["C"][:, 4]))
    assert np.max(np.abs(ra["C"][good] - hi)) < 1e-14


def test_dd_gemm_against_exact_fractions():
    rng = np.random.default_rng(8)
    A = W.spread_matrix(rng, (5, 9), 3.0)
    B = W.spread_matrix(rng, (9, 4), 3.0)
    hi, lo = O.dd_gemm(A, B)
    for i in range(5):
        for j in range(4):
            ex = O.exact_dot(A[i], B[:, j])
            absum = sum(abs(Fraction(float(a)) * Fraction(float(b))) for a, b in zip(A[i], B[:, j]))
            err = abs(Fraction(hi[i, j]) + Fraction(lo[i, j]) - ex)
            assert err <= absum * Fraction(1, 2 ** 100)
            assert hi[i, j] == float(ex) or err > 0


def test_error_gate_and_comparison_with_native():
    # [Q] section 行列積の回数と性能: 14-15 moduli reach about the accuracy of
    # native DGEMM; the componentwise error stays below 1e-14 for N >= 14.
    for phi in (0.5, 1.0):
        A, B = W.spread_case(96, 80, 512, phi, seed=1)
        hi, lo = O.dd_gemm(A, B)
        native = O.error_metrics(A @ B, hi, lo, A, B)["E_cw"]
        for N in (14, 15, 16, 18):
            e = O.error_metrics(O.os2_dgemm(A, B, N)["C"], hi, lo, A, B)["E_cw"]
            assert e <= 1e-14
            if N >= 15:
                assert e <= 4 * native + 1e-16
        e8 = O.error_metrics(O.os2_dgemm(A, B, 8)["C"], hi, lo, A, B)["E_cw"]
        assert 1e-12 < e8 < 1e-6  # about 28 bits per element at N = 8


def test_planted_exponent_error_is_detected():
    # A mistake planted in the oracle (one bit too many on every row) must be
    # caught by the exact range check: CRT then wraps and X != Y.
    k, N = 2048, 14
    A = np.ones((4, k))
    B = np.ones((k, 4))
    e, f = O.exponents(A, B, N, "fast")
    r = O.os2_dgemm(A, B, N, e=[v + 1 for v in e], f=f)
    Y = O.exact_scaled_product(A, B, r["e"], r["f"])
    assert np.all(2 * np.abs(Y) > r["tables"]["P"] - 1)
    assert not np.any(r["X"] == Y)
    assert not np.any(r["C"] == k)


# --------------------------------------------------------------------------
# Single precision: one rounding of X * 2^-s to binary32
# --------------------------------------------------------------------------
def test_round_to_f32_against_exact_doubles():
    # when X * 2^-s is exactly a double (|X| < 2^53, no double underflow), the
    # binary32 rounding of that double is the single rounding we want
    rng = np.random.default_rng(11)
    for _ in range(4000):
        X = int(rng.integers(-(2 ** 53) + 1, 2 ** 53))
        s = int(rng.integers(-100, 221))
        want = np.float32(np.ldexp(np.float64(X), -s))
        got = O.round_to_f32(X, s)
        assert np.float32(got).view(np.uint32) == want.view(np.uint32), (X, s)


def test_round_to_f32_ties_subnormals_overflow():
    r = O.round_to_f32
    assert r(2 ** 24 + 1, 0) == 2.0 ** 24            # tie to even (down)
    assert r(2 ** 24 + 3, 0) == 2.0 ** 24 + 4        # tie to even (up)
    assert r(2 ** 60 + 2 ** 36, 0) == 2.0 ** 60      # tie far above 2^53, to even
    assert r(2 ** 60 + 2 ** 36 + 1, 0) == 2.0 ** 60 + 2 ** 37  # just above the tie
    tiny = np.float32(2.0 ** -149)
    assert r(1, 149) == tiny and r(1, 150) == 0.0    # 2^-150 ties to the even zero
    assert r(3, 151) == tiny                         # 0.75 quantum rounds up
    assert r(3, 150) == np.float32(2.0 ** -148)      # 1.5 quanta tie to 2 quanta
    assert r(2 ** 200 + 1, 200 + 126 + 23) == tiny * np.float32(2.0 ** 0)  # huge X, deep subnormal
    big = float(np.finfo(np.float32).max)            # (2 - 2^-23) * 2^127
    assert r(int(big), 0) == np.float32(big)
    assert r(int(big) + 2 ** 103, 0) == np.float32(np.inf)  # tie above max rounds to even = inf
    assert r(int(big) + 2 ** 103 - 1, 0) == np.float32(big)
    assert r(-(2 ** 24 + 1), 0) == -(2.0 ** 24) and r(0, 5) == 0.0


def test_sgemm_small_integers_and_nonfinite():
    rng = np.random.default_rng(2)
    A = rng.integers(-3, 4, (20, 30)).astype(np.float32)
    B = rng.integers(-3, 4, (30, 9)).astype(np.float32)
    A[4] = 0.0
    A[7, 3] = np.inf
    r = O.os2_sgemm(A, B, 8)
    C = r["C"]
    assert C.dtype == np.float32
    exact = A.astype(np.float64) @ B.astype(np.float64)
    ok = np.ones(20, bool)
    ok[7] = False
    assert np.array_equal(C[ok], exact[ok].astype(np.float32))
    assert np.all(np.isnan(C[7])) and np.all(C[4] == 0.0)
    # the binary32 result is the double result of the same X rounded once more
    # only where that cannot double-round: here all values are small integers
    assert np.array_equal(C[ok], r["C64"][ok].astype(np.float32))


def test_sgemm_accuracy_against_native_fp32():
    # [G] Zentrale Beiträge: the scheme is evaluated for SGEMM; with 8 moduli it
    # is at least as accurate as native binary32 on moderately spread data,
    # and 9 moduli are needed for the wider spread
    rng = np.random.default_rng(5)
    n = 160
    for phi, N in ((0.5, 8), (1.0, 8), (2.0, 9)):
        A = ((rng.random((n, n)) - 0.5) * np.exp(phi * rng.standard_normal((n, n)))).astype(np.float32)
        B = ((rng.random((n, n)) - 0.5) * np.exp(phi * rng.standard_normal((n, n)))).astype(np.float32)
        A64, B64 = A.astype(np.float64), B.astype(np.float64)
        ref = A64 @ B64
        scale = np.abs(A64) @ np.abs(B64)
        ecw = lambda C: float(np.max(np.abs(C.astype(np.float64) - ref) / scale))
        assert ecw(O.os2_sgemm(A, B, N)["C"]) <= ecw(A @ B), (phi, N)
        # and never worse than the final binary32 rounding allows
        assert ecw(O.os2_sgemm(A, B, 10)["C"]) <= 2.0 ** -24


# --------------------------------------------------------------------------
# Complex products: Gauss' three products per modulus, exact in residues
# --------------------------------------------------------------------------
def _complex_case(m, n, k, seed, phi=1.0):
    rng = np.random.default_rng(seed)
    parts = [W.spread_matrix(rng, shape, phi) for shape in ((m, k), (m, k), (k, n), (k, n))]
    return parts[0] + 1j * parts[1], parts[2] + 1j * parts[3]


def test_sym_mod_ranges():
    for p in (3, 173, 255, 256):
        x = np.arange(-3 * p, 3 * p)
        r = O.sym_mod(x, p).astype(np.int64)
        assert np.all((r - x) % p == 0)
        lo, hi = (-(p - 1) // 2, (p - 1) // 2) if p % 2 else (-p // 2, p // 2 - 1)
        assert r.min() == lo and r.max() == hi


@pytest.mark.parametrize("N", [4, 8, 16, 18])
def test_complex_rns_equals_plain_definition(N):
    A, B = _complex_case(11, 9, 23, seed=N)
    A[2] = 0.0
    A[5, 3] = complex(np.inf, 0.0)
    B[4, 6] = complex(0.0, np.nan)
    r = O.os2_zgemm(A, B, N)
    assert r["e"][5] is None and r["f"][6] is None and r["e"][2] == 0
    okr = [v is not None for v in r["e"]]
    okc = [v is not None for v in r["f"]]
    A0 = np.where(np.array(okr)[:, None], A, 0.0)
    B0 = np.where(np.array(okc)[None, :], B, 0.0)
    e0 = [v if v is not None else 0 for v in r["e"]]
    f0 = [v if v is not None else 0 for v in r["f"]]
    Xr, Xi = O.exact_complex_scaled_product(A0, B0, e0, f0)
    for i in range(11):
        for j in range(9):
            if okr[i] and okc[j]:
                assert int(r["Xr"][i, j]) == Xr[i, j] and int(r["Xi"][i, j]) == Xi[i, j]
                s = -(e0[i] + f0[j])
                assert r["C"][i, j].real == math.ldexp(float(Xr[i, j]), s)
                assert r["C"][i, j].imag == math.ldexp(float(Xi[i, j]), s)
            else:
                assert np.isnan(r["C"][i, j].real) and np.isnan(r["C"][i, j].imag)
    # the residues of both parts are the CRT images of the exact parts
    for l, p in enumerate(r["moduli"]):
        for i in range(11):
            for j in range(9):
                if okr[i] and okc[j]:
                    assert r["cr"][l, i, j] == Xr[i, j] % p and r["ci"][l, i, j] == Xi[i, j] % p


def test_complex_gaussian_integers_give_the_exact_product():
    rng = np.random.default_rng(3)
    A = rng.integers(-3, 4, (14, 40)) + 1j * rng.integers(-3, 4, (14, 40))
    B = rng.integers(-3, 4, (40, 10)) + 1j * rng.integers(-3, 4, (40, 10))
    assert np.array_equal(O.os2_zgemm(A, B, 8)["C"], A @ B)
    assert np.array_equal(O.os2_zgemm(A, B, 8, single=True)["C"], (A @ B).astype(np.complex64))


def test_complex_exponents_keep_both_parts_in_range():
    # 2 ||a_i'|| ||b_j'|| <= P - 1 on the truncated integers (complex 2-norms),
    # which bounds |Re| and |Im| of every product entry by (P - 1) / 2
    A, B = _complex_case(20, 16, 64, seed=5, phi=2.0)
    for N in (6, 14, 16):
        r = O.os2_zgemm(A, B, N)
        P = r["tables"]["P"]
        ar, ai = O.scaled_integers(A.real, r["e"]), O.scaled_integers(A.imag, r["e"])
        br, bi = O.scaled_integers(B.real.T, r["f"]), O.scaled_integers(B.imag.T, r["f"])
        na = [sum(int(x) ** 2 for x in ar[i]) + sum(int(x) ** 2 for x in ai[i]) for i in range(20)]
        nb = [sum(int(x) ** 2 for x in br[j]) + sum(int(x) ** 2 for x in bi[j]) for j in range(16)]
        for i in range(20):
            for j in range(16):
                assert 4 * na[i] * nb[j] <= (P - 1) ** 2
                assert 2 * abs(int(r["Xr"][i, j])) <= P - 1 and 2 * abs(int(r["Xi"][i, j])) <= P - 1


def test_complex_scale_law():
    A, B = _complex_case(9, 7, 30, seed=8)
    base = O.os2_zgemm(A, B, 14)["C"]
    for s in (-40, 40):
        got = O.os2_zgemm(np.ldexp(A.real, s) + 1j * np.ldexp(A.imag, s), B, 14)["C"]
        assert np.array_equal(got, np.ldexp(base.real, s) + 1j * np.ldexp(base.imag, s))


def test_complex_accuracy_against_native():
    A, B = _complex_case(48, 40, 300, seed=9)
    rr = [O.dd_gemm(X, Y) for X, Y in ((A.real, B.real), (A.imag, B.imag), (A.real, B.imag), (A.imag, B.real))]
    ref_r = (rr[0][0] - rr[1][0]) + (rr[0][1] - rr[1][1])
    ref_i = (rr[2][0] + rr[3][0]) + (rr[2][1] + rr[3][1])
    scale = np.abs(A) @ np.abs(B)
    ecw = lambda C: float(np.max(np.maximum(np.abs(C.real - ref_r), np.abs(C.imag - ref_i)) / scale))
    assert ecw(O.os2_zgemm(A, B, 16)["C"]) <= ecw(A @ B)
    assert ecw(O.os2_zgemm(A, B, 16)["C"]) <= 1e-15
    assert ecw(O.os2_zgemm(A, B, 8, single=True)["C"].astype(np.complex128)) <= \
        ecw((A.astype(np.complex64) @ B.astype(np.complex64)).astype(np.complex128))


# --------------------------------------------------------------------------
# The stand-in for the original fast-mode rule ([G] Problemstellung): pinned
# only by the behaviour [G] describes, not by values
# --------------------------------------------------------------------------
def test_original_rule_lacks_scale_invariance_and_fails_at_the_ends():
    Pp = O.scaling_constant(math.prod(O.choose_moduli(14)))
    rng = np.random.default_rng(4)
    U = rng.uniform(-1.0, 1.0, (6, 2048))
    base = O.original_exponents_rows(U, Pp)
    prop = O.fast_exponents_rows(U, Pp)
    # at moderate scale it picks about the proposed exponent (no margin: at most one more)
    assert all(0 <= b - p <= 1 for b, p in zip(base, prop))
    # large alpha: the binary32 sum overflows and the bit width collapses (mu = 0)
    big = O.original_exponents_rows(np.ldexp(U, 64), Pp)
    assert big == [O.EXP_COLLAPSE] * 6
    # tiny alpha: the binary32 squares underflow and mu is unbounded
    tiny = O.original_exponents_rows(np.ldexp(U, -90), Pp)
    assert tiny == [O.EXP_FLOOD] * 6
    # the proposed rule is exact over the same range
    for s in (64, -66, -90):
        assert O.fast_exponents_rows(np.ldexp(U, s), Pp) == [p - s for p in prop]
    # zero rows stay zero in both
    assert O.original_exponents_rows(np.zeros((2, 9)), Pp) == [0, 0]
