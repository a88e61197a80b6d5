/*
 * oracle_core.c -- exact-integer and double-double loops of the CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY. This file belongs to the oracle that checks the
 * HIP implementation; only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load it. It shares no code with the
 * library and is compiled by gcc, never by hipcc.
 *
 * Pages followed:
 *   [Q] "8ビットの整数で53ビットの倍精度を組み立てる。中国剰余定理をGPUに載せた
 *       Ozaki Scheme II" (Qiita article)
 *
 * Everything here is deliberately plain: one element at a time, in the order
 * the definition gives, with __int128 for exact integers. Build with
 * -O2 -fopenmp -ffp-contract=off (never fast-math): the double-double
 * reference relies on every product and sum being rounded separately.
 */
#include <math.h>
#include <stdint.h>

/*
 * Steps 1 and 2 of [Q] (sections "2の累乗による整数化(手順1と5)" and
 * "256以下の法の選び方(手順2)"): scale each row by its power of two, cut off
 * the fraction toward zero, and store the residue of the resulting integer
 * modulo every p in the symmetric range the article gives: for odd p the
 * residues run from -(p-1)/2 to (p-1)/2 (7 -> -3..3), and for p = 256 from
 * -128 to 127 (128 and -128 are the same residue).
 *
 * x[r, h] sits at X[r*rs + h*hs]. out is [nmod][rows][cols], row-major.
 * Returns 0, or -1 if some scaled value is not finite or |x| >= 2^126
 * (outside what __int128 holds exactly).
 */
int orc_split(int64_t rows, int64_t cols, const double *X, int64_t rs, int64_t hs,
              const int32_t *e, int nmod, const int32_t *moduli, int8_t *out)
{
    int bad = 0;
#pragma omp parallel for reduction(| : bad) schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t h = 0; h < cols; ++h) {
            double x = trunc(ldexp(X[r * rs + h * hs], e[r]));
            if (!isfinite(x) || fabs(x) >= 0x1p126) {
                bad = 1;
                continue;
            }
            __int128 xi = (__int128)x; /* exact: x is an integer below 2^126 */
            for (int l = 0; l < nmod; ++l) {
                int p = moduli[l];
                int v = (int)(xi % p); /* sign of xi, |v| < p */
                if (v < 0)
                    v += p; /* 0 <= v < p */
                if (v > (p - 1) / 2)
                    v -= p; /* symmetric range */
                out[((int64_t)l * rows + r) * cols + h] = (int8_t)v;
            }
        }
    }
    return bad ? -1 : 0;
}

/*
 * The integers themselves: xs[r][h] = trunc(x[r,h] * 2^e[r]) as two int64
 * halves, value = hi * 2^63 + lo with 0 <= lo < 2^63 (exact for |x| < 2^126).
 * Used by the plain-definition check (exact dot products in Python).
 */
int orc_scaled_ints(int64_t rows, int64_t cols, const double *X, int64_t rs, int64_t hs,
                    const int32_t *e, int64_t *hi, int64_t *lo)
{
    int bad = 0;
#pragma omp parallel for reduction(| : bad) schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t h = 0; h < cols; ++h) {
            double x = trunc(ldexp(X[r * rs + h * hs], e[r]));
            if (!isfinite(x) || fabs(x) >= 0x1p126) {
                bad = 1;
                continue;
            }
            __int128 xi = (__int128)x;
            __int128 two63 = (__int128)1 << 63;
            __int128 q = xi / two63, rem = xi % two63;
            if (rem < 0) {
                rem += two63;
                q -= 1;
            }
            hi[r * cols + h] = (int64_t)q;
            lo[r * cols + h] = (int64_t)rem;
        }
    }
    return bad ? -1 : 0;
}

/*
 * Double-double reference product, the accuracy yardstick: for every (i, j)
 * the sum over h of a_ih * b_hj, each product split exactly with an FMA
 * (TwoProd) and accumulated with TwoSum in ascending h. A is m x k at
 * A[i + h*lda], B is k x n at B[h + j*ldb] (column-major); hi and lo are
 * m x n column-major with leading dimension m.
 */
void orc_dd_gemm(int64_t m, int64_t n, int64_t k, const double *A, int64_t lda,
                 const double *B, int64_t ldb, double *hi, double *lo)
{
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t j = 0; j < n; ++j) {
        for (int64_t i = 0; i < m; ++i) {
            double sh = 0.0, sl = 0.0;
            for (int64_t h = 0; h < k; ++h) {
                double a = A[i + h * lda], b = B[h + j * ldb];
                double p = a * b;
                double pe = fma(a, b, -p); /* a*b = p + pe exactly */
                double s = sh + p;         /* TwoSum(sh, p) */
                double bb = s - sh;
                double se = (sh - (s - bb)) + (p - bb);
                se += sl + pe;
                double t = s + se; /* renormalise */
                sl = se - (t - s);
                sh = t;
            }
            hi[i + j * m] = sh;
            lo[i + j * m] = sl;
        }
    }
}
