"""Plain CPU oracle for Ozaki Scheme II FP64 matrix-product emulation.

TEST INFRASTRUCTURE ONLY. This module checks the HIP implementation and is
not part of it: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it. It shares no code, table
or constant generator with ``rns_emulated_fp64_amd``; the only common module
is ``workloads.py``, which draws random inputs and holds none of the method.

Pages followed (cited by title and section):
  [Q] "8ビットの整数で53ビットの倍精度を組み立てる。中国剰余定理をGPUに載せた
      Ozaki Scheme II" (Qiita article on the Chinese remainder theorem and
      Ozaki Scheme II)
  [G] "Improved Scaling for Fast Mode of Ozaki Scheme II" (technical summary,
      German)

What the method computes, step by step ([Q] section 行列積への当てはめ方):
  1. scale each row of A and each column of B by a power of two and cut the
     fraction off (steps 1 and 5, section 2の累乗による整数化(手順1と5));
  2. take the residues of those integers modulo N pairwise-coprime moduli
     <= 256, stored as int8 in a symmetric range (step 2);
  3. multiply the residue matrices, one integer product per modulus, exact in
     int32 (step 3, section 誤差のないINT8行列積(手順3));
  4. rebuild each entry by the Chinese remainder theorem in more than double
     precision (step 4, section 高い精度での復元(手順4));
  5. undo the powers of two (step 5).

Every function below is one of those steps written out plainly, with Python
integers wherever exactness matters. The heavy loops that need exact 128-bit
integers or double-double sums live in ``oracle_core.c`` (compiled by gcc).

Readings taken where the pages are silent:
  * u32, the unit roundoff of binary32, is 2**-24; the margin "4 u32" of [G]
    is kept verbatim.
  * P'_prop (a precomputed constant in [G] section Methodik) is
    0.5 * log2((P - 1) / 2), rounded down to a double: the sufficient
    condition 2 mu ||a|| ||b|| nu <= P - 1 split evenly between row and column.
  * sum_h a_ih^2 is evaluated in FP64 on the row scaled by 2**-g, where 2**g
    is the smallest power of two above max_h |a_ih|, in ascending h; the
    exponent g is added back exactly. This is the same quantity as the plain
    sum, but cannot overflow or underflow, and it makes the scale invariance
    of [G] (section Methodik, 2.) hold bit for bit.
  * log2 is applied only to the significand f in [1, 2) of that sum, and the
    binary exponent is split off exactly, so no rounding depends on it.
  * "cut off" is truncation toward zero.
  * The original fast-mode rule [G] criticises is not printed; the stand-in
    original_exponents_rows (binary32 sums, no margin) is for comparisons
    only and PARITY UNPINNED beyond its stated failure directions.
  * Single precision ([G] section Zentrale Beiträge names SGEMM): the same
    steps on the binary32 inputs widened exactly to doubles, and one rounding
    of X * 2^-(e+f) to binary32 (os2_sgemm, round_to_f32).
  * Complex products ([G] closing remark, future work there): one exponent
    per row/column from the complex 2-norm, parts truncated separately, and
    Gauss' three products per modulus, which are exact in residues
    (os2_zgemm; fast mode only).
  * Accurate mode ([Q] section 2の累乗による整数化, [G] section
    Problemstellung) is read as: bound |A| and |B| from above by 6-bit
    integers on the row/column maxima, form their product with one extra
    integer GEMM, and choose each row's exponent from the largest entry of its
    row of that product (and likewise for columns). PARITY UNPINNED as to the
    exact rule: the pages print no algorithm or value for it; only its
    invariants are pinned (the range condition holds exactly, the scale law,
    the bound operands really bound |A| and |B|).
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from fractions import Fraction

import numpy as np

U32 = 2.0 ** -24  # unit roundoff of IEEE binary32
MAX_MODULI = 20

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "_oracle_core.so")
_SRC = os.path.join(_HERE, "oracle_core.c")


# --------------------------------------------------------------------------
# The compiled core (gcc, OpenMP)
# --------------------------------------------------------------------------
def build_core() -> str:
    """Compile oracle_core.c with gcc (never fast-math, no FP contraction)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=gnu11",
           "-shared", "-fPIC", _SRC, "-o", _SO + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_SO + ".tmp", _SO)
    return _SO


_core = None


def core():
    global _core
    if _core is None:
        if not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
            build_core()
        lib = ctypes.CDLL(_SO)
        i64, p = ctypes.c_int64, ctypes.c_void_p
        lib.orc_split.argtypes = [i64, i64, p, i64, i64, p, ctypes.c_int, p, p]
        lib.orc_split.restype = ctypes.c_int
        lib.orc_scaled_ints.argtypes = [i64, i64, p, i64, i64, p, p, p]
        lib.orc_scaled_ints.restype = ctypes.c_int
        lib.orc_dd_gemm.argtypes = [i64, i64, i64, p, i64, p, i64, p, p]
        lib.orc_dd_gemm.restype = None
        _core = lib
    return _core


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


# --------------------------------------------------------------------------
# Step 2 tables: moduli and CRT weights
# --------------------------------------------------------------------------
def choose_moduli(count: int, largest: int = 256) -> list[int]:
    """The `count` largest pairwise-coprime integers <= `largest`, greedily.

    [Q] section 256以下の法の選び方(手順2): pick integers up to 256 that are
    pairwise coprime and as large as possible; primes are not required, only
    one even modulus can be used and 256 is the best one. Walking down from 256
    and keeping every integer coprime to all kept so far gives exactly the
    implementation order in the article's footnote on the moduli table.
    """
    chosen: list[int] = []
    x = largest
    while len(chosen) < count:
        if x < 2:
            raise ValueError("not enough pairwise-coprime moduli")
        if all(math.gcd(x, c) == 1 for c in chosen):
            chosen.append(x)
        x -= 1
    return chosen


def dayan_qiuyi(g: int, p: int) -> int:
    """Qin Jiushao's 大衍求一術: the multiplier k with g*k = 1 (mod p).

    [Q] section 秦九韶の大衍求一術: four cells; top right holds g mod p
    (the 奇数), bottom right the modulus p (定母), top left 1, bottom left 0.
    Divide the larger right-hand number by the smaller and replace it by the
    remainder, adding quotient * (the other left number) to the left number on
    the divided side. When the bottom right reaches 1, the last division of the
    top is taken with quotient (top - 1) so that 1 stays on top. Stop when the
    top right is 1: the top left is the 乗率.
    """
    if p < 2 or math.gcd(g, p) != 1:
        raise ValueError("g must be invertible modulo p")
    tr, br, tl, bl = g % p, p, 1, 0
    while tr != 1:
        if br == 1:
            tl += (tr - 1) * bl
            tr = 1
        elif br > tr:
            q, br = divmod(br, tr)
            bl += q * tl
        else:
            q, tr = divmod(tr, br)
            tl += q * bl
    return tl % p


def crt_tables(moduli) -> dict:
    """Qin Jiushao's quantities for a set of moduli ([Q] table in 秦九韶の大衍求一術).

    P   衍母  product of all moduli
    M   衍数  P / p_l
    G   奇数  M_l mod p_l
    K   乗率  multiplier with G_l * K_l = 1 mod p_l
    W   用数  M_l * K_l: advances clock l by one and leaves the others alone
    """
    moduli = [int(p) for p in moduli]
    P = math.prod(moduli)
    M = [P // p for p in moduli]
    G = [m % p for m, p in zip(M, moduli)]
    K = [dayan_qiuyi(g, p) for g, p in zip(G, moduli)]
    W = [m * k for m, k in zip(M, K)]
    return dict(moduli=moduli, P=P, M=M, G=G, K=K, W=W)


def scaling_constant(P: int) -> float:
    """P'_prop = 0.5 * log2((P - 1) / 2), rounded down to a double.

    [G] section Methodik, 1.: the sufficient condition
    2 mu_i ||a_i|| ||b_j|| nu_j <= P - 1 split evenly between the row and the
    column factor (the 0.5 in the printed exponent). Rounding down keeps the
    condition intact.
    """
    import mpmath

    with mpmath.workdps(80):
        v = mpmath.log(mpmath.mpf(P - 1) / 2, 2) / 2
        d = float(v)
        if mpmath.mpf(d) > v:
            d = math.nextafter(d, -math.inf)
    return d


# --------------------------------------------------------------------------
# Step 1: exponents
# --------------------------------------------------------------------------
def _frexp_exponent(x: np.ndarray) -> np.ndarray:
    """g with x < 2**g <= 2x for x > 0 (numpy.frexp's exponent); 0 for x == 0."""
    return np.frexp(x)[1].astype(np.int64)


def row_sumsq(X: np.ndarray):
    """For every row of X: (s, g, finite) with sum_h x_h^2 = s * 4**g.

    g is the frexp exponent of max_h |x_h| (so |x_h| * 2**-g < 1); the scaled
    entries are squared and summed in FP64 in ascending h, one rounding per
    product and per sum. Rows holding Inf or NaN are reported as not finite.
    """
    X = np.asarray(X, dtype=np.float64)
    amax = np.max(np.abs(X), axis=1) if X.shape[1] else np.zeros(X.shape[0])
    finite = np.isfinite(amax)
    g = np.where(finite, _frexp_exponent(np.where(finite, amax, 0.0)), 0)
    Xs = np.ldexp(np.where(finite[:, None], X, 0.0), -g[:, None])
    s = np.zeros(X.shape[0])
    for h in range(X.shape[1]):
        col = Xs[:, h]
        s = s + col * col
    return s, g, finite


def exponent_from_bound(s: float, Pp: float) -> int:
    """floor(P' - 0.5 * (log2(s) + 4 u32)) for s > 0, with log2 split exactly.

    [G] section Methodik, 1.: mu_i = 2^floor(P'_prop - 0.5*(log2(sum a^2) + 4u32)).
    Writing s = f * 2^E with f in [1, 2) and E = 2h + q (q in {0, 1}), the
    argument equals (P' - 0.5 q) - 0.5 (log2 f + 4 u32) - h, and h comes out
    of the floor exactly.
    """
    m, E1 = math.frexp(s)  # s = m * 2^E1, m in [0.5, 1)
    f, E = 2.0 * m, E1 - 1
    q = E % 2
    h = (E - q) // 2
    return math.floor((Pp - 0.5 * q) - 0.5 * (math.log2(f) + 4.0 * U32)) - h


NONFINITE = None  # marker in exponent lists for rows/columns holding Inf or NaN


def fast_exponents_rows(X: np.ndarray, Pp: float) -> list:
    """Proposed fast-mode exponent e_i for every row of X ([G] Methodik, 1.).

    A zero row gets 0; a row holding Inf/NaN gets NONFINITE.
    """
    s, g, finite = row_sumsq(X)
    out = []
    for si, gi, fi in zip(s, g, finite):
        if not fi:
            out.append(NONFINITE)
        elif si == 0.0:
            out.append(0)
        else:
            out.append(exponent_from_bound(float(si), Pp) - int(gi))
    return out


def fast_exponents(A: np.ndarray, B: np.ndarray, Pp: float):
    """(e for rows of A, f for columns of B) in the proposed fast mode."""
    return fast_exponents_rows(A, Pp), fast_exponents_rows(np.asarray(B).T, Pp)


# Stand-in for the original fast-mode rule ([G] Problemstellung criticises it
# but the pages do not print it; PARITY UNPINNED beyond its stated behaviour):
# squares of the binary32-rounded entries summed in binary32 in ascending h,
# e = floor(P' - 0.5 * log2(sum)) in binary32 with no margin and no exponent
# split. A sum that overflows gives mu = 0 (EXP_COLLAPSE: every integer is 0);
# a nonzero line whose sum underflows to zero leaves mu unbounded (EXP_FLOOD).
EXP_COLLAPSE, EXP_FLOOD = -2000, 2000


def original_exponents_rows(X: np.ndarray, Pp: float) -> list:
    X = np.asarray(X, dtype=np.float64)
    out = []
    with np.errstate(over="ignore", under="ignore"):
        for row in X:
            if not np.all(np.isfinite(row)):
                out.append(NONFINITE)
                continue
            a = row.astype(np.float32)
            s = np.float32(0.0)
            for v in a:
                s = np.float32(s + np.float32(v * v))
            if not np.any(row != 0.0):
                out.append(0)
            elif s == 0.0:
                out.append(EXP_FLOOD)
            elif not np.isfinite(s):
                out.append(EXP_COLLAPSE)
            else:
                out.append(int(np.floor(np.float32(Pp) - np.float32(0.5) * np.log2(s))))
    return out


def accurate_bound_operands(A: np.ndarray, B: np.ndarray):
    """6-bit integer upper bounds of |A| and |B| (accurate mode, our reading).

    r_i = frexp exponent of max_h |a_ih| (so |a_ih| < 2^r_i) and
    Abar_ih = ceil(|a_ih| * 2^(6 - r_i)) in [0, 64]; columns of B likewise.
    """
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    # Rows of A / columns of B holding Inf or NaN become NaN lines of C
    # whatever the exponents; they take no part in the bound product.
    A = np.where(np.all(np.isfinite(A), axis=1)[:, None], A, 0.0)
    B = np.where(np.all(np.isfinite(B), axis=0)[None, :], B, 0.0)
    ra = _frexp_exponent(np.max(np.abs(A), axis=1)) if A.shape[1] else np.zeros(A.shape[0], np.int64)
    cb = _frexp_exponent(np.max(np.abs(B), axis=0)) if B.shape[0] else np.zeros(B.shape[1], np.int64)
    abar = np.ceil(np.ldexp(np.abs(A), (6 - ra)[:, None]))
    bbar = np.ceil(np.ldexp(np.abs(B), (6 - cb)[None, :]))
    return ra, cb, abar, bbar


def accurate_exponents(A: np.ndarray, B: np.ndarray, Pp: float):
    """Exponents from one extra integer GEMM W = Abar * Bbar (accurate mode).

    Since sum_h |a_ih||b_hj| <= 2^(r_i + c_j - 12) W_ij and
    W_ij <= sqrt(R_i C_j) with R_i = max_j W_ij, C_j = max_i W_ij, the choice
    e_i = floor(P' + 6 - r_i - 0.5 (log2 R_i + 4 u32)) (f_j alike) keeps
    2 sum_h |a'_ih||b'_hj| <= P - 1. W is exact in FP64 (entries < 2^53).
    Returns (e, f, W).
    """
    ra, cb, abar, bbar = accurate_bound_operands(A, B)
    W = abar @ bbar  # integer-valued, exact
    R = W.max(axis=1) if W.shape[1] else np.zeros(W.shape[0])
    C = W.max(axis=0) if W.shape[0] else np.zeros(W.shape[1])
    finA = np.all(np.isfinite(A), axis=1)
    finB = np.all(np.isfinite(B), axis=0)
    e = [NONFINITE if not fi else (0 if Ri == 0 else exponent_from_bound(float(Ri), Pp) + 6 - int(ri))
         for Ri, ri, fi in zip(R, ra, finA)]
    f = [NONFINITE if not fi else (0 if Cj == 0 else exponent_from_bound(float(Cj), Pp) + 6 - int(cj))
         for Cj, cj, fi in zip(C, cb, finB)]
    return e, f, W


# --------------------------------------------------------------------------
# Steps 1-2: integerization and residues
# --------------------------------------------------------------------------
def _exp_array(e) -> np.ndarray:
    return np.array([0 if v is None else v for v in e], dtype=np.int32)


def _rows_view(X: np.ndarray):
    """(array, row stride, column stride) in elements, for the C core."""
    X = np.asarray(X, dtype=np.float64)
    if not (X.flags.c_contiguous or X.flags.f_contiguous):
        X = np.ascontiguousarray(X)
    rs, hs = (s // 8 for s in X.strides)
    return X, rs, hs


def split(X: np.ndarray, e, moduli) -> np.ndarray:
    """Residues of trunc(x_rh * 2^e_r) mod each p, symmetric range, int8 [N][rows][cols].

    [Q] steps 1 and 2. Rows with a NONFINITE exponent must not be passed.
    """
    X, rs, hs = _rows_view(X)
    rows, cols = X.shape
    ee = _exp_array(e)
    mods = np.array(moduli, dtype=np.int32)
    out = np.empty((len(mods), rows, cols), dtype=np.int8)
    rc = core().orc_split(rows, cols, _ptr(X), rs, hs, _ptr(ee), len(mods), _ptr(mods), _ptr(out))
    if rc != 0:
        raise OverflowError("scaled integer not finite or >= 2^126")
    return out


def scaled_integers(X: np.ndarray, e) -> np.ndarray:
    """trunc(x_rh * 2^e_r) as an object array of exact Python ints."""
    X, rs, hs = _rows_view(X)
    rows, cols = X.shape
    ee = _exp_array(e)
    hi = np.empty((rows, cols), dtype=np.int64)
    lo = np.empty((rows, cols), dtype=np.int64)
    rc = core().orc_scaled_ints(rows, cols, _ptr(X), rs, hs, _ptr(ee), _ptr(hi), _ptr(lo))
    if rc != 0:
        raise OverflowError("scaled integer not finite or >= 2^126")
    return hi.astype(object) * (1 << 63) + lo.astype(object)


# --------------------------------------------------------------------------
# Step 3: one exact integer product per modulus
# --------------------------------------------------------------------------
INT32_BLOCK = (1 << 17) - 1  # inner-dimension block for which int8 x int8 sums fit int32


def residue_products(RA: np.ndarray, RB: np.ndarray) -> np.ndarray:
    """Q^(l) = RA^(l) RB^(l)^T for each modulus, exact, int64 [N][m][n].

    [Q] section 誤差のないINT8行列積(手順3): int8 x int8 products are at most
    128*128 = 16384 in magnitude, so the sums fit int32 while the inner
    dimension is below 2^17; larger inner dimensions are split into blocks.
    Each block product is formed by an FP64 matrix product, which is exact
    because every partial sum is an integer below 2^31 < 2^53, and the blocks
    are added in int64. RA is [N][m][k], RB is [N][n][k] (B's columns as rows).
    """
    k = RA.shape[2]
    Q = np.zeros((RA.shape[0], RA.shape[1], RB.shape[1]), dtype=np.int64)
    for l in range(RA.shape[0]):
        for h0 in range(0, k, INT32_BLOCK):
            a = RA[l][:, h0:h0 + INT32_BLOCK].astype(np.float64)
            b = RB[l][:, h0:h0 + INT32_BLOCK].astype(np.float64)
            qb = (a @ b.T).astype(np.int64)
            assert np.all(np.abs(qb) < (1 << 31)), "int32 overflow in a block product"
            Q[l] += qb
    return Q


def reduce_products(Q: np.ndarray, moduli) -> np.ndarray:
    """c^(l) = Q^(l) mod p_l in [0, p_l), uint8 [N][m][n]."""
    c = np.empty(Q.shape, dtype=np.uint8)
    for l, p in enumerate(moduli):
        c[l] = np.mod(Q[l], p)
    return c


# --------------------------------------------------------------------------
# Step 4: Chinese remainder reconstruction
# --------------------------------------------------------------------------
def crt(c: np.ndarray, tables: dict) -> np.ndarray:
    """X = (sum_l W_l c_l) mod P, lifted to (-P/2, P/2]; object array of ints.

    [Q] section 繰り上がりのない計算: add each weight (用数) as many times as
    its clock shows, and remove whole turns of P; section 時計の針で見る定理の
    中身: read the upper half of the range as negative numbers.
    """
    P = tables["P"]
    acc = np.zeros(c.shape[1:], dtype=object)
    for l, w in enumerate(tables["W"]):
        acc = acc + c[l].astype(object) * w
    X = acc % P
    return np.where(2 * X > P, X - P, X)


def garner(c: np.ndarray, moduli) -> np.ndarray:
    """Same reconstruction by mixed-radix (Garner) digits, independent of the weights."""
    moduli = [int(p) for p in moduli]
    P = math.prod(moduli)
    digits = []
    for l, p in enumerate(moduli):
        v = c[l].astype(object)
        radix = 1
        partial = np.zeros(c.shape[1:], dtype=object)
        for d, q in zip(digits, moduli[:l]):
            partial = partial + d * radix
            radix *= q
        digits.append(((v - partial) * pow(radix % p, -1, p)) % p if l else v % p)
    X = np.zeros(c.shape[1:], dtype=object)
    radix = 1
    for d, p in zip(digits, moduli):
        X = X + d * radix
        radix *= p
    return np.where(2 * X > P, X - P, X)


def check_modulus(num_moduli: int) -> int:
    """The redundant modulus of the range check: the next one of the table."""
    return choose_moduli(num_moduli + 1)[num_moduli]


def crt_range_flags(c: np.ndarray, c_check: np.ndarray, moduli, p_check: int) -> np.ndarray:
    """CRT-range failure flags: 0 where the reconstruction agrees with one more clock, 1 where not.

    [Q] section 時計の針で見る定理の中身: an integer Y outside (-P/2, P/2] is read
    back as X = Y - j P, another number. With the residue c_check of the same
    integer modulo a further modulus p_check (coprime to every p_l), X and Y
    differ modulo p_check whenever 0 < |j| < p_check, so the flag is exactly
    "X != Y" for such j. c holds the residues in [0, p_l) ([N][...]), c_check
    the check residues in [0, p_check).
    """
    X = crt(c, crt_tables(moduli))
    return np.where((X - np.asarray(c_check).astype(object)) % p_check == 0, 0, 1).astype(np.uint8)


# --------------------------------------------------------------------------
# Step 5 and the whole pipeline
# --------------------------------------------------------------------------
def unscale(X: np.ndarray, e, f) -> np.ndarray:
    """C_ij = RN(X_ij) * 2^-(e_i + f_j); NaN where a row or column was not finite."""
    Xf = X.astype(np.float64)  # Python int -> double is correctly rounded
    ee = _exp_array(e).astype(np.int64)
    ff = _exp_array(f).astype(np.int64)
    C = np.ldexp(Xf, -(ee[:, None] + ff[None, :]))
    bad_r = np.array([v is None for v in e], dtype=bool)
    bad_c = np.array([v is None for v in f], dtype=bool)
    C[bad_r, :] = np.nan
    C[:, bad_c] = np.nan
    return C


def exponents(A, B, num_moduli: int, mode: str = "fast"):
    moduli = choose_moduli(num_moduli)
    Pp = scaling_constant(math.prod(moduli))
    if mode == "fast":
        return fast_exponents(A, B, Pp)
    if mode == "accurate":
        e, f, _ = accurate_exponents(A, B, Pp)
        return e, f
    if mode == "original":
        return original_exponents_rows(A, Pp), original_exponents_rows(np.asarray(B).T, Pp)
    raise ValueError(mode)


def os2_dgemm(A, B, num_moduli: int, mode: str = "fast", e=None, f=None) -> dict:
    """Whole emulation on the CPU, keeping every intermediate.

    A is (m, k), B is (k, n). Exponents may be supplied (e.g. to re-split with
    exponents taken from elsewhere after checking them). Rows/columns with
    Inf/NaN give NaN rows/columns of C.
    """
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    moduli = choose_moduli(num_moduli)
    tables = crt_tables(moduli)
    if e is None or f is None:
        e0, f0 = exponents(A, B, num_moduli, mode)
        e = e0 if e is None else e
        f = f0 if f is None else f
    okr = np.array([v is not None for v in e], dtype=bool)
    okc = np.array([v is not None for v in f], dtype=bool)
    A0 = np.where(okr[:, None], A, 0.0)
    B0 = np.where(okc[None, :], B, 0.0)
    RA = split(A0, e, moduli)
    RB = split(B0.T, f, moduli)
    Q = residue_products(RA, RB)
    c = reduce_products(Q, moduli)
    X = crt(c, tables)
    C = unscale(X, e, f)
    return dict(moduli=moduli, tables=tables, e=e, f=f, RA=RA, RB=RB, Q=Q, c=c, X=X, C=C)


# --------------------------------------------------------------------------
# Single precision ([G] section Zentrale Beiträge: the scheme evaluated for
# SGEMM as well as DGEMM)
# --------------------------------------------------------------------------
# Reading: the same steps on binary32 inputs (every binary32 value is a double,
# so the exponents, the split and the integer product are those of the FP64
# path on the widened inputs), and the result is the binary32 value nearest to
# X * 2^-(e_i + f_j), rounded once, ties to even, subnormals included.
F32_MANT = 24          # significand bits of binary32
F32_MIN_EXP = -149     # exponent of the smallest subnormal
F32_MAX = float(np.finfo(np.float32).max)


def round_to_f32(X: int, s: int) -> np.float32:
    """RN_binary32(X * 2^-s) for an integer X, by integer arithmetic."""
    if X == 0:
        return np.float32(0.0)
    sign = -1 if X < 0 else 1
    mag = -X if X < 0 else X
    b = mag.bit_length()
    # place of the last kept bit, in units of mag: 24 significant bits, but
    # never below the subnormal quantum 2^-149 (= 2^(s - 149) in units of mag)
    shift = max(b - F32_MANT, s + F32_MIN_EXP)
    if shift <= 0:
        q = mag << -shift
    else:
        q, r = divmod(mag, 1 << shift)
        half = 1 << (shift - 1)
        if r > half or (r == half and (q & 1)):
            q += 1
    v = math.ldexp(float(q), shift - s)  # q < 2^25: exact as a double
    if v > F32_MAX:
        return np.float32(sign * np.inf)
    return np.float32(sign * v)


def unscale_f32(X: np.ndarray, e, f) -> np.ndarray:
    """C_ij = RN_binary32(X_ij * 2^-(e_i + f_j)); NaN rows/columns as unscale."""
    m, n = X.shape
    C = np.empty((m, n), dtype=np.float32)
    for i in range(m):
        for j in range(n):
            if e[i] is None or f[j] is None:
                C[i, j] = np.float32(np.nan)
            else:
                C[i, j] = round_to_f32(int(X[i, j]), e[i] + f[j])
    return C


def os2_sgemm(A, B, num_moduli: int, mode: str = "fast", e=None, f=None) -> dict:
    """The emulation for binary32 A (m, k) and B (k, n): os2_dgemm's steps on
    the exactly widened inputs, then one rounding to binary32."""
    A = np.asarray(A, dtype=np.float32)
    B = np.asarray(B, dtype=np.float32)
    r = os2_dgemm(A.astype(np.float64), B.astype(np.float64), num_moduli, mode, e=e, f=f)
    r["C64"] = r["C"]
    r["C"] = unscale_f32(r["X"], r["e"], r["f"])
    return r


# --------------------------------------------------------------------------
# Complex products ([G] closing remark: the approach also applies to complex
# products, ZGEMM/CGEMM, left there as future work)
# --------------------------------------------------------------------------
# Reading (where the pages are silent):
#  * A = Ar + i Ai, B = Br + i Bi. Row i of A takes one exponent, from its
#    complex 2-norm sum_h (ar^2 + ai^2), with the formula of [G] Methodik;
#    column j of B likewise. By Cauchy-Schwarz, 2 mu ||a_i|| ||b_j|| nu <= P - 1
#    bounds both the real and the imaginary part of the exact integer product
#    by (P - 1) / 2.
#  * The two parts are truncated separately: ar' = trunc(2^e ar), ai' likewise.
#  * Xr = sum_h ar'br' - ai'bi' and Xi = sum_h ar'bi' + ai'br' exactly, and
#    C = RN(Xr) 2^-(e+f) + i RN(Xi) 2^-(e+f) (binary32 parts: one rounding
#    each, as round_to_f32).
#  * In residues the three products of Gauss' trick are exact: per modulus
#    T1 = ar'br', T2 = ai'bi', T3 = (ar' + ai')(br' + bi'), and
#    Xr = T1 - T2, Xi = T3 - T1 - T2 (mod p), so three integer GEMMs per
#    modulus give both parts with no rounding at all.
#  * Only the fast mode is defined for complex operands.
def sym_mod(x: np.ndarray, p: int) -> np.ndarray:
    """x mod p in the symmetric range of [Q] step 2, as int8 (for p = 256 the
    class of 128 is stored as -128)."""
    h = (p - 1) // 2 if p % 2 else p // 2
    return (np.mod(np.asarray(x, dtype=np.int64) + h, p) - h).astype(np.int8)


def complex_exponents_rows(Xr: np.ndarray, Xi: np.ndarray, Pp: float) -> list:
    """Fast-mode exponent of each row of a complex matrix from sum_h (re^2 + im^2)."""
    return fast_exponents_rows(np.concatenate([np.asarray(Xr, np.float64), np.asarray(Xi, np.float64)], axis=1), Pp)


def os2_zgemm(A, B, num_moduli: int, e=None, f=None, single: bool = False) -> dict:
    """The emulation of a complex product C = A B (A (m, k), B (k, n) complex),
    with every intermediate: residue planes of the real parts, imaginary parts
    and their sums, the three products per modulus and their residues, the
    residues of both parts, the exact parts Xr, Xi and C. single: binary32
    parts (inputs widened exactly, each part rounded once to binary32)."""
    cdt = np.complex64 if single else np.complex128
    A = np.asarray(A, dtype=cdt).astype(np.complex128)
    B = np.asarray(B, dtype=cdt).astype(np.complex128)
    moduli = choose_moduli(num_moduli)
    tables = crt_tables(moduli)
    Pp = scaling_constant(tables["P"])
    if e is None:
        e = complex_exponents_rows(A.real, A.imag, Pp)
    if f is None:
        f = complex_exponents_rows(B.real.T, B.imag.T, Pp)
    okr = np.array([v is not None for v in e], dtype=bool)
    okc = np.array([v is not None for v in f], dtype=bool)
    A0 = np.where(okr[:, None], A, 0.0)
    B0 = np.where(okc[None, :], B, 0.0)
    RAr, RAi = split(A0.real, e, moduli), split(A0.imag, e, moduli)
    RBr, RBi = split(B0.real.T, f, moduli), split(B0.imag.T, f, moduli)
    RAs = np.stack([sym_mod(RAr[l].astype(np.int64) + RAi[l], p) for l, p in enumerate(moduli)])
    RBs = np.stack([sym_mod(RBr[l].astype(np.int64) + RBi[l], p) for l, p in enumerate(moduli)])
    T1 = residue_products(RAr, RBr)
    T2 = residue_products(RAi, RBi)
    T3 = residue_products(RAs, RBs)
    T = np.stack([T1, T2, T3], axis=1)  # [N][3][m][n]
    cT = np.stack([reduce_products(T[:, g], moduli) for g in range(3)], axis=1)
    cr = reduce_products(T1 - T2, moduli)
    ci = reduce_products(T3 - T1 - T2, moduli)
    Xr = crt(cr, tables)
    Xi = crt(ci, tables)
    Cr, Ci = (unscale_f32(Xr, e, f), unscale_f32(Xi, e, f)) if single else (unscale(Xr, e, f), unscale(Xi, e, f))
    C = np.empty(Cr.shape, dtype=np.complex64 if single else np.complex128)
    C.real[...] = Cr
    C.imag[...] = Ci
    return dict(moduli=moduli, tables=tables, e=e, f=f, RAr=RAr, RAi=RAi, RAs=RAs, RBr=RBr, RBi=RBi,
                RBs=RBs, T=T, cT=cT, cr=cr, ci=ci, Xr=Xr, Xi=Xi, C=C)


def exact_complex_scaled_product(A, B, e, f):
    """(Xr, Xi) from the plain definition: exact sums of products of the
    truncated scaled parts, with Python integers (small cases only)."""
    A = np.asarray(A, dtype=np.complex128)
    B = np.asarray(B, dtype=np.complex128)
    ar, ai = scaled_integers(A.real, e), scaled_integers(A.imag, e)
    br, bi = scaled_integers(B.real.T, f), scaled_integers(B.imag.T, f)
    return ar.dot(br.T) - ai.dot(bi.T), ar.dot(bi.T) + ai.dot(br.T)


def exact_scaled_product(A, B, e, f) -> np.ndarray:
    """Plain definition: Y_ij = sum_h trunc(2^e_i a_ih) trunc(2^f_j b_hj), exact ints.

    When 2|Y_ij| <= P - 1 the CRT recovers Y exactly ([Q] section
    定理が保証すること), so the emulation returns RN(Y_ij) 2^-(e_i + f_j).
    """
    Ai = scaled_integers(np.asarray(A, dtype=np.float64), e)
    Bi = scaled_integers(np.asarray(B, dtype=np.float64).T, f)
    return Ai.dot(Bi.T)


# --------------------------------------------------------------------------
# Accuracy yardsticks
# --------------------------------------------------------------------------
def dd_gemm(A, B):
    """(hi, lo): double-double A @ B, TwoProd + TwoSum in ascending h."""
    A = np.asfortranarray(A, dtype=np.float64)
    B = np.asfortranarray(B, dtype=np.float64)
    m, k = A.shape
    n = B.shape[1]
    hi = np.empty((m, n), dtype=np.float64, order="F")
    lo = np.empty((m, n), dtype=np.float64, order="F")
    core().orc_dd_gemm(m, n, k, _ptr(A), max(m, 1), _ptr(B), max(k, 1), _ptr(hi), _ptr(lo))
    return hi, lo


def exact_dot(a_row, b_col) -> Fraction:
    """Exact sum of a_h * b_h as a Fraction (tiny inputs only)."""
    return sum((Fraction(float(x)) * Fraction(float(y)) for x, y in zip(a_row, b_col)), Fraction(0))


def error_metrics(C, ref_hi, ref_lo, A, B) -> dict:
    """Componentwise, elementwise and normwise errors of C against hi + lo.

    E_cw = max |C - ref| / (|A||B|) (0/0 counts as 0), the measure that stays
    bounded for every FP64 method; E_el = max |C - ref| / |ref|; E_nw is the
    Frobenius ratio.
    """
    C = np.asarray(C, dtype=np.float64)
    diff = np.abs((C - ref_hi) - ref_lo)
    absprod = np.abs(np.asarray(A)) @ np.abs(np.asarray(B))
    with np.errstate(divide="ignore", invalid="ignore"):
        cw = np.where(absprod > 0, diff / absprod, np.where(diff == 0, 0.0, np.inf))
        el = np.where(np.abs(ref_hi) > 0, diff / np.abs(ref_hi), np.where(diff == 0, 0.0, np.inf))
    nref = np.linalg.norm(ref_hi)
    return dict(E_cw=float(np.max(cw)) if cw.size else 0.0,
                E_el=float(np.max(el)) if el.size else 0.0,
                E_nw=float(np.linalg.norm(diff) / nref) if nref > 0 else 0.0)
