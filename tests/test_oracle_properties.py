"""Property tests of the CPU oracle on random small inputs (Hypothesis).

Each property is checked against a computation that does not go through the
oracle's own arithmetic: exact Python integers and Fractions for the
truncated scaled integers and their dot products, Python's three-argument
pow for modular inverses, and the defining congruences of the Chinese
remainder theorem. Random subsets of the moduli table and random shapes,
values, moduli counts and power-of-two scalings are drawn, so a dropped term,
a wrong sign or index or a transposed operand anywhere along the oracle's
path fails on some example.

Pages: [Q] the Qiita article on the Chinese remainder theorem and Ozaki
Scheme II (steps 1-5; sections 時計の針で見る定理の中身, 定理が保証すること and
秦九韶の大衍求一術); [G]
"Improved Scaling for Fast Mode of Ozaki Scheme II" (section Methodik).
"""
import math
from fractions import Fraction

import numpy as np
from hypothesis import given, settings
from hypothesis import strategies as st

import oracle as O

H1 = O.choose_moduli(20)
SETTINGS = settings(max_examples=150, deadline=None)


def exact_trunc(x: float, e: int) -> int:
    """trunc(x * 2^e) toward zero, exactly."""
    return int(Fraction(x) * Fraction(2) ** e)


def sym_range(r: int, p: int) -> bool:
    return (-128 <= r <= 127) if p == 256 else (-(p - 1) // 2 <= r <= (p - 1) // 2)


moduli_subsets = st.lists(st.sampled_from(H1), min_size=2, max_size=8, unique=True)
# entries with a spread of exponents (+-[0.5, 1) times 2^-40 .. 2^40), some
# zeros; products stay far from the subnormal range, where the final
# power-of-two scaling rounds a second time
entries = st.one_of(
    st.just(0.0),
    st.builds(lambda sg, m, k: sg * math.ldexp(m, k), st.sampled_from([-1.0, 1.0]),
              st.floats(0.5, 1.0, exclude_max=True), st.integers(-40, 40)),
)


@st.composite
def matrices(draw, max_rows=4, max_cols=6):
    r = draw(st.integers(1, max_rows))
    c = draw(st.integers(1, max_cols))
    return np.array(draw(st.lists(st.lists(entries, min_size=c, max_size=c), min_size=r, max_size=r)),
                    dtype=np.float64)


@st.composite
def products(draw):
    m = draw(st.integers(1, 4))
    k = draw(st.integers(1, 6))
    n = draw(st.integers(1, 4))
    A = np.array(draw(st.lists(st.lists(entries, min_size=k, max_size=k), min_size=m, max_size=m)))
    B = np.array(draw(st.lists(st.lists(entries, min_size=n, max_size=n), min_size=k, max_size=k)))
    return A.astype(np.float64), B.astype(np.float64)


@SETTINGS
@given(moduli_subsets, st.data())
def test_crt_and_garner_recover_every_integer_of_the_symmetric_range(moduli, data):
    # [Q] section 定理が保証すること: residues determine one integer in a range
    # of P consecutive integers; the oracle reads the range as (-P/2, P/2]
    P = math.prod(moduli)
    X = data.draw(st.integers(-((P - 1) // 2), P // 2))
    c = np.array([[X % p] for p in moduli], dtype=np.int64)
    tables = O.crt_tables(moduli)
    assert int(O.crt(c, tables)[0]) == X
    assert int(O.garner(c, moduli)[0]) == X


@SETTINGS
@given(moduli_subsets)
def test_weights_are_the_unit_vectors_of_the_residues(moduli):
    # [Q] 秦九韶の大衍求一術: the 用数 W_l is 1 mod p_l and 0 mod every other
    # modulus; the 乗率 is the inverse of the 奇数 mod p_l
    t = O.crt_tables(moduli)
    for l, p in enumerate(moduli):
        assert t["K"][l] == pow(t["G"][l], -1, p)
        for j, q in enumerate(moduli):
            assert t["W"][l] % q == (1 if j == l else 0)


@SETTINGS
@given(matrices(), st.integers(2, 20))
def test_split_residues_are_the_symmetric_residues_of_the_scaled_integers(X, N):
    # [Q] steps 1 and 2: trunc(x * 2^e) reduced mod each p into the symmetric range
    moduli = H1[:N]
    Pp = O.scaling_constant(math.prod(moduli))
    e = O.fast_exponents_rows(X, Pp)
    R = O.split(X, e, moduli)
    for i in range(X.shape[0]):
        for h in range(X.shape[1]):
            x = exact_trunc(float(X[i, h]), e[i])
            for l, p in enumerate(moduli):
                r = int(R[l, i, h])
                assert sym_range(r, p) and (x - r) % p == 0, (i, h, p, x, r)


def check_plain_definition(A, B, N, mode):
    moduli = H1[:N]
    P = math.prod(moduli)
    r = O.os2_dgemm(A, B, N, mode)
    e, f, C = r["e"], r["f"], r["C"]
    m, k = A.shape
    n = B.shape[1]
    for i in range(m):
        for j in range(n):
            a = [exact_trunc(float(A[i, h]), e[i]) for h in range(k)]
            b = [exact_trunc(float(B[h, j]), f[j]) for h in range(k)]
            Y = sum(x * y for x, y in zip(a, b))
            # [G] Methodik: the scaling keeps 2 sum |a'||b'| <= P - 1, so the
            # CRT recovers Y exactly ([Q] step 4)
            assert 2 * sum(abs(x) * abs(y) for x, y in zip(a, b)) <= P - 1
            assert int(r["X"][i, j]) == Y
            for l, p in enumerate(moduli):
                assert int(r["c"][l, i, j]) == Y % p  # residue homomorphism ([Q] step 3)
            want = math.ldexp(float(Y), -(e[i] + f[j]))  # float(int) rounds to nearest-even
            assert np.float64(C[i, j]).view(np.uint64) == np.float64(want).view(np.uint64), (i, j, C[i, j], want)


@SETTINGS
@given(products(), st.integers(2, 20))
def test_fast_mode_equals_the_plain_definition(AB, N):
    A, B = AB
    check_plain_definition(A, B, N, "fast")


@SETTINGS
@given(products(), st.integers(2, 20))
def test_accurate_mode_equals_the_plain_definition(AB, N):
    A, B = AB
    check_plain_definition(A, B, N, "accurate")


@SETTINGS
@given(products(), st.integers(8, 20), st.integers(-200, 200))
def test_power_of_two_scaling_passes_through_exactly(AB, N, s):
    # [G] Methodik 2: e(2^s A) = e(A) - s for every nonzero row (a zero row
    # gets 0 either way), hence C(2^s A) = 2^s C(A) bit for bit
    A, B = AB
    r0 = O.os2_dgemm(A, B, N)
    r1 = O.os2_dgemm(np.ldexp(A, s), B, N)
    nonzero = np.any(A != 0.0, axis=1)
    assert [x - s if nz else 0 for x, nz in zip(r0["e"], nonzero)] == list(r1["e"])
    assert list(r0["f"]) == list(r1["f"])
    np.testing.assert_array_equal(np.ldexp(r0["C"], s), r1["C"])
