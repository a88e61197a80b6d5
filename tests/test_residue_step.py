"""Host-side check of the rounding argument behind the GEMM epilogue's residue
step (step 3 of [Q] "8ビットの整数で53ビットの倍精度を組み立てる", section
誤差のないINT8行列積(手順3): each int32 product is reduced mod p_l).

The kernel forms k = round(q / p) as the low word of one FP64 FMA,
t = RN(q * RN(1/p) + 1.5 * 2^52), and then r = q - k p with a 24-bit multiply.
That is valid when RN of the exact value q * RN(1/p) + 1.5 * 2^52 lands on
1.5 * 2^52 + round(q / p) (spacing 1 there), and |k| < 2^23. The test evaluates
the exact rational q * RN(1/p), rounds it to the nearest integer with ties to
even (what the FMA does), and compares with the exactly rounded q / p on the
values where the argument is tightest: the ends of |q| <= 2^30 + 128 and the
points next to every half-integer of q / p."""
from fractions import Fraction
import random

import pytest

import oracle as O

Q_MAX = (1 << 30) + 128  # 1024 stages of 64 terms of at most 2^14, plus a carried residue


def round_half_even(x: Fraction) -> int:
    f = x.numerator // x.denominator
    rem = x - f
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and f % 2 == 1):
        f += 1
    return f


def samples(p: int, rnd: random.Random):
    qs = {0, 1, -1, Q_MAX, -Q_MAX, Q_MAX - 1, -Q_MAX + 1}
    for _ in range(300):
        qs.add(rnd.randint(-Q_MAX, Q_MAX))
    # next to the half-integers of q / p, near zero and near the ends
    for base in (0, Q_MAX // p - 3, -(Q_MAX // p) + 3, rnd.randint(-(Q_MAX // p), Q_MAX // p)):
        for k in range(base, base + 3):
            for d in (-1, 0, 1):
                qs.add(k * p + p // 2 + d)
                qs.add(k * p - p // 2 + d)
    return [q for q in qs if -Q_MAX <= q <= Q_MAX]


@pytest.mark.parametrize("p", O.choose_moduli(20))
def test_fma_rounding_gives_the_symmetric_residue(p):
    pinv = Fraction(1.0 / p)  # RN(1/p): Python's float division is correctly rounded
    half = 128 if p == 256 else (p - 1) // 2
    rnd = random.Random(p)
    for q in samples(p, rnd):
        k = round_half_even(q * pinv)
        assert k == round_half_even(Fraction(q, p)), (p, q)
        assert abs(k) < (1 << 23)  # inside the 24-bit multiplier's signed range
        r = q - k * p
        assert -half <= r <= half and (r - q) % p == 0, (p, q, r)
