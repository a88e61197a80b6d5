// kernels.hip -- gfx950 (MI355X) kernels of the Ozaki Scheme II FP64 GEMM
// emulation.
//
// Pages: [Q] Qiita article "8ビットの整数で53ビットの倍精度を組み立てる。中国剰余
// 定理をGPUに載せたOzaki Scheme II", section "Ozaki Scheme IIのGPU実装" (steps 1-5);
// [G] "Improved Scaling for Fast Mode of Ozaki Scheme II", section Methodik.
//
// Phases and the bound each one lives under:
//   norms + exponents  (step 1, [G] Methodik)          HBM: reads A and B once
//   residue split      (steps 1 + 2)                    HBM / FP64 VALU
//   INT8 GEMMs         (step 3), one per modulus        INT8 MFMA
//   CRT + unscale      (steps 4 + 5)                    HBM / FP64 VALU
//
// Compiled with -ffp-contract=off: every product and sum below rounds on its
// own unless an fma() is written out, which the exact integer arithmetic
// relies on.
#include <float.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <type_traits>

#include <hip/hip_ext.h>

#include "common.h"

namespace oz2 {

// Launch with optional timing events. hipExtLaunchKernelGGL attaches them to
// the dispatch itself (start: the kernel's start time, stop: its end time),
// so a timed launch puts no marker packets in the stream.
#define OZ2_LAUNCH(ev, kern, grid, block, shm, stream, ...)                                            \
    do {                                                                                             \
        if ((ev).start || (ev).stop)                                                                 \
            hipExtLaunchKernelGGL(kern, grid, block, shm, stream, (ev).start, (ev).stop, 0, __VA_ARGS__); \
        else                                                                                         \
            hipLaunchKernelGGL(kern, grid, block, shm, stream, __VA_ARGS__);                         \
    } while (0)

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

#define LDS_PTR(p) ((__attribute__((address_space(3))) void *)(p))

constexpr double kU32 = 0x1p-24;  // unit roundoff of binary32; [G] uses a 4 u32 margin

// ---------------------------------------------------------------------------
// Step 1: squared norms with an exact power-of-two rescale
// ---------------------------------------------------------------------------
// A running pair (s, g) stands for s * 4^g: the sum of squares of the entries
// scaled by 2^-g, where 2^g is the smallest power of two above the largest
// |entry| seen so far. Rescaling by powers of two is exact, so the result is
// the sum of (a * 2^-G)^2 for the final G whatever the order of the maxima,
// it cannot overflow or underflow, and a row scaled by 2^s gives the same s
// bit for bit with G shifted by s (the scale invariance of [G] Methodik 2).
__device__ __forceinline__ void ssq_add(double &s, int &g, double a) {
    if (a == 0.0) return;
    int ga;
    (void)frexp(a, &ga);
    if (ga > g) {
        s = ldexp(s, 2 * (g - ga));
        g = ga;
    }
    double t = ldexp(a, -g);
    s = s + t * t;
}

__device__ __forceinline__ void ssq_merge(double &s, int &g, double s2, int g2) {
    if (g2 > g) {
        s = ldexp(s, 2 * (g - g2));
        g = g2;
    }
    s = s + ldexp(s2, 2 * (g2 - g));
}

// floor(P' - 0.5 * (log2(s) + 4 u32)) for s > 0 ([G] Methodik 1), with
// s = f * 2^E, f in [1,2), E = 2h + q: the argument is
// (P' - q/2) - (log2 f + 4 u32)/2 - h, so no rounding depends on E.
__device__ __forceinline__ int exponent_from_bound(double s, double Pp) {
    int E1;
    double mnt = frexp(s, &E1);
    double f = 2.0 * mnt;
    int E = E1 - 1;
    int q = E & 1;
    int h = (E - q) >> 1;
    double z = (Pp - 0.5 * (double)q) - 0.5 * (log2(f) + 4.0 * kU32);
    return (int)floor(z) - h;
}

// The stand-in for the original fast-mode rule that [G] (Problemstellung)
// shows is not scale invariant (OZAKI2_FAST_ORIGINAL; the pages do not print
// it): the squares of the binary32-rounded entries are summed in binary32,
// and e = floor(P' - 0.5 log2f(s)) with no margin and no exponent split.
// An overflowed sum makes mu = 0 (kExpCollapse: every integer becomes 0); a
// sum that underflows to zero on a nonzero line makes mu unbounded
// (kExpFlood: the integers overflow the CRT range). Both are the failure
// directions [G] describes; the result is not checked against anything.
constexpr int kExpCollapse = -2000, kExpFlood = 2000;
__device__ __forceinline__ int exponent_original(float s, bool nonzero, double Pp) {
    if (!nonzero) return 0;
    if (s == 0.0f) return kExpFlood;
    if (!(s <= FLT_MAX)) return kExpCollapse;
    return (int)floorf((float)Pp - 0.5f * log2f(s));
}

// Rows of column-major A. Block = 64 rows x 4 k-lanes over one k-chunk: a
// wavefront reads 64 consecutive rows of one column (512 contiguous bytes),
// each thread accumulates every 4th column of its chunk, and the 4 lanes of a
// row are merged in a fixed order through LDS. Output: one partial
// (s, g, nonfinite) per (chunk, row).
// ORIG: the stand-in's binary32 sum; the partial holds that float (as a
// double) and pg holds 1 if the chunk has a nonzero entry.
template <class T, int W, bool ORIG = false>
__device__ __forceinline__ void row_norms_block(const T *__restrict__ A, int64_t m, int64_t k, int64_t lda,
                                                int64_t kchunk, double *__restrict__ ps, int *__restrict__ pg,
                                                int *__restrict__ pbad, int64_t rowblock, int64_t chunk) {
    __shared__ double sh_s[4][64];
    __shared__ int sh_g[4][64];
    __shared__ int sh_b[4][64];
    const int r = threadIdx.x & 63, kl = threadIdx.x >> 6;
    const int64_t i = rowblock * 64 + r;
    const int64_t h0 = chunk * kchunk;
    const int64_t h1 = h0 + kchunk < k ? h0 + kchunk : k;
    double s = 0.0;
    int g = kExpEmpty;
    int bad = 0;
    float s32 = 0.0f;
    auto add = [&](double x) {  // x = |entry|
        if (!(x <= DBL_MAX)) {
            bad = 1;
        } else if (ORIG) {
            const float a = (float)x;
            s32 = s32 + a * a;
            g |= x != 0.0 ? 1 : 0;
        } else {
            ssq_add(s, g, x);
        }
    };
    if (ORIG) g = 0;
    if (i < m) {
        // element (i, h) part c at A[(i + h*lda)*W + c]
        const T *a = A + i * W;
        const int64_t cs = lda * W;
        int64_t h = h0 + kl;
        for (; h + 28 < h1; h += 32) {
            double v[8][W];
#pragma unroll
            for (int u = 0; u < 8; ++u)
#pragma unroll
                for (int c = 0; c < W; ++c) v[u][c] = (double)a[(h + 4 * u) * cs + c];
#pragma unroll
            for (int u = 0; u < 8; ++u)
#pragma unroll
                for (int c = 0; c < W; ++c) add(fabs(v[u][c]));
        }
        for (; h < h1; h += 4)
#pragma unroll
            for (int c = 0; c < W; ++c) add(fabs((double)a[h * cs + c]));
    }
    if (ORIG) s = (double)s32;
    sh_s[kl][r] = s;
    sh_g[kl][r] = g;
    sh_b[kl][r] = bad;
    __syncthreads();
    if (kl == 0 && i < m) {
#pragma unroll
        for (int q = 1; q < 4; ++q) {
            if (ORIG) {
                s32 = s32 + (float)sh_s[q][r];
                g |= sh_g[q][r];
            } else {
                ssq_merge(s, g, sh_s[q][r], sh_g[q][r]);
            }
            bad |= sh_b[q][r];
        }
        if (ORIG) s = (double)s32;
        const int64_t o = chunk * m + i;
        ps[o] = s;
        pg[o] = g;
        pbad[o] = bad;
    }
}

// Exponent of row i from its chunk partials, merged in ascending chunk order:
// e = fast exponent, g = max exponent (the r_i of accurate mode).
template <bool ORIG = false>
__device__ __forceinline__ void row_exponent_from_partials(const double *__restrict__ ps,
                                                           const int *__restrict__ pg,
                                                           const int *__restrict__ pbad, int64_t m, int64_t i,
                                                           int nchunks, double Pp, int &e, int &g_out) {
    double s = 0.0;
    int g = kExpEmpty;
    int bad = 0;
    float s32 = 0.0f;
    int nonzero = 0;
    // loads in batches of 8 (all issued before the merges), merges in
    // ascending chunk order
    for (int c0 = 0; c0 < nchunks; c0 += 8) {
        double vs[8];
        int vg[8], vb[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int64_t o = (int64_t)(c0 + u < nchunks ? c0 + u : c0) * m + i;
            vs[u] = ps[o];
            vg[u] = pg[o];
            vb[u] = pbad[o];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (c0 + u < nchunks) {
                bad |= vb[u];
                if (ORIG) {
                    s32 = s32 + (float)vs[u];
                    nonzero |= vg[u];
                } else {
                    ssq_merge(s, g, vs[u], vg[u]);
                }
            }
        }
    }
    if (ORIG) {
        e = bad ? kExpNonfinite : exponent_original(s32, nonzero != 0, Pp);
        g_out = 0;
        return;
    }
    if (bad) {
        e = kExpNonfinite;
        g_out = kExpNonfinite;
    } else if (s == 0.0) {
        e = 0;
        g_out = 0;
    } else {
        e = exponent_from_bound(s, Pp) - g;
        g_out = g;
    }
}

// Row exponents of every row from the chunk partials (accurate mode, which
// needs them before the bound product). Rows in [m, m_pad) get 0. The same
// threads clear the row and column maxima the bound product accumulates.
__global__ __launch_bounds__(256) void k_row_exponents(const double *__restrict__ ps, const int *__restrict__ pg,
                                                       const int *__restrict__ pbad, int64_t m, int64_t m_pad,
                                                       int nchunks, double Pp, int32_t *__restrict__ e,
                                                       int32_t *__restrict__ ga, int32_t *__restrict__ rowmax,
                                                       int32_t *__restrict__ colmax, int64_t n_pad) {
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n_pad) colmax[i] = 0;
    if (i >= m_pad) return;
    rowmax[i] = 0;
    int ev = 0, gv = 0;
    if (i < m) row_exponent_from_partials(ps, pg, pbad, m, i, nchunks, Pp, ev, gv);
    e[i] = ev;
    ga[i] = gv;
}

// Columns of column-major B (contiguous): one wavefront per column, lanes
// stride the column, then a fixed xor-butterfly merge (every lane ends with
// the same bits).
template <class T, bool ORIG = false>
__device__ __forceinline__ void col_exponents_block(const T *__restrict__ B, int64_t k, int64_t n,
                                                    int64_t n_pad, int64_t ldb, double Pp, int32_t *__restrict__ f,
                                                    int32_t *__restrict__ gb, int64_t blk) {
    const int lane = threadIdx.x & 63;
    int64_t j = blk * 4 + (threadIdx.x >> 6);
    if (j >= n_pad) return;
    if (j >= n) {
        if (lane == 0) {
            f[j] = 0;
            gb[j] = 0;
        }
        return;
    }
    const T *col = B + j * ldb;
    double s = 0.0;
    int g = kExpEmpty;
    int bad = 0;
    float s32 = 0.0f;
    if (ORIG) g = 0;
    auto add = [&](double x) {  // x = |entry|
        if (!(x <= DBL_MAX)) {
            bad = 1;
        } else if (ORIG) {
            const float a = (float)x;
            s32 = s32 + a * a;
            g |= x != 0.0 ? 1 : 0;
        } else {
            ssq_add(s, g, x);
        }
    };
    int64_t h = lane;
    for (; h + 7 * 64 < k; h += 8 * 64) {
        double v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = (double)col[h + 64 * u];
#pragma unroll
        for (int u = 0; u < 8; ++u) add(fabs(v[u]));
    }
    for (; h < k; h += 64) add(fabs((double)col[h]));
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        bad |= __shfl_xor(bad, off, 64);
        if (ORIG) {
            s32 = s32 + __shfl_xor(s32, off, 64);  // a + b == b + a: both lanes agree
            g |= __shfl_xor(g, off, 64);
        } else {
            double s2 = __shfl_xor(s, off, 64);
            int g2 = __shfl_xor(g, off, 64);
            // the merge is symmetric in its two operands, so both lanes of a
            // pair end with the same bits
            ssq_merge(s, g, s2, g2);
        }
    }
    if (ORIG) {
        if (lane == 0) {
            f[j] = bad ? kExpNonfinite : exponent_original(s32, g != 0, Pp);
            gb[j] = 0;
        }
        return;
    }
    if (lane == 0) {
        if (bad) {
            f[j] = kExpNonfinite;
            gb[j] = kExpNonfinite;
        } else if (s == 0.0) {
            f[j] = 0;
            gb[j] = 0;
        } else {
            f[j] = exponent_from_bound(s, Pp) - g;
            gb[j] = g;
        }
    }
}

// Step 1 for both operands in one launch: blocks [0, nA) are row-norm blocks
// of A (row block fastest, then k-chunk), the rest column blocks of B. W = 2:
// complex operands with interleaved parts; a row's (column's) squared norm is
// the sum over both parts, and a column of B is then 2k contiguous values.
template <class T, int W, bool ORIG>
__global__ __launch_bounds__(256) void k_scale(const T *__restrict__ A, int64_t m, int64_t k, int64_t lda,
                                               int64_t kchunk, int64_t rowblocks, int64_t nA,
                                               double *__restrict__ ps, int *__restrict__ pg,
                                               int *__restrict__ pbad, const T *__restrict__ B, int64_t n,
                                               int64_t n_pad, int64_t ldb, double Pp, int32_t *__restrict__ f,
                                               int32_t *__restrict__ gb) {
    const int64_t bid = blockIdx.x;
    if (bid < nA)
        row_norms_block<T, W, ORIG>(A, m, k, lda, kchunk, ps, pg, pbad, bid % rowblocks, bid / rowblocks);
    else
        col_exponents_block<T, ORIG>(B, k * W, n, n_pad, ldb * W, Pp, f, gb, bid - nA);
}

// Accurate mode: e_i = floor(P' + 6 - r_i - 0.5 (log2 R_i + 4 u32)) with R_i
// the largest entry of row i of the bound product (0 -> e_i = 0).
__global__ __launch_bounds__(256) void k_accurate_exponents(const int32_t *__restrict__ rowmax,
                                                            const int32_t *__restrict__ colmax,
                                                            const int32_t *__restrict__ ga,
                                                            const int32_t *__restrict__ gb, int64_t m,
                                                            int64_t m_pad, int64_t n, int64_t n_pad, double Pp,
                                                            int32_t *__restrict__ e, int32_t *__restrict__ f) {
    int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t < m_pad) {
        int64_t i = t;
        int v = 0;
        if (i < m) {
            if (ga[i] == kExpNonfinite) v = kExpNonfinite;
            else if (rowmax[i] > 0) v = exponent_from_bound((double)rowmax[i], Pp) + 6 - ga[i];
        }
        e[i] = v;
    } else if (t < m_pad + n_pad) {
        int64_t j = t - m_pad;
        int v = 0;
        if (j < n) {
            if (gb[j] == kExpNonfinite) v = kExpNonfinite;
            else if (colmax[j] > 0) v = exponent_from_bound((double)colmax[j], Pp) + 6 - gb[j];
        }
        f[j] = v;
    }
}

// ---------------------------------------------------------------------------
// Steps 1 + 2: integerize and split into int8 residues (packed MFMA order)
// ---------------------------------------------------------------------------
// Block: 32 rows x 128 columns of K, staged through LDS as doubles so that the
// global reads are coalesced whichever way the source is laid out. The block
// covers four fragment blocks of 16 rows x 64 K; wavefront w = t / 64 fills
// block (row half w % 2, K half w / 2), and lane L owns row L % 16 and the 16
// consecutive K of quarter L / 16, exactly the 16 bytes it holds in the
// packed layout.
constexpr int kSplitRows = 32, kSplitCols = 128, kSplitLd = kSplitCols + 2;

// W parts per element (1 real, 2 complex interleaved); X points at the part.
template <bool KCONTIG, class T, int W = 1>
__device__ __forceinline__ void split_load_tile(double (*tile)[kSplitLd], const T *__restrict__ X,
                                                int64_t rows, int64_t kdim, int64_t ld, int64_t r0,
                                                int64_t h0) {
    // All 16 loads of a thread are issued before any LDS write; out-of-range
    // elements read a valid address and are replaced by zero.
    const int t = threadIdx.x;
    double v[16];
    if (!KCONTIG) {  // element (r, h) at X[r + h*ld]: rows contiguous
        const int rr = t & 31, hh = t >> 5;
        const int64_t r = r0 + rr;
        const bool rok = r < rows;
        const int64_t rc = rok ? r : 0;
#pragma unroll
        for (int it = 0; it < 16; ++it) {
            const int64_t h = h0 + hh + 8 * it;
            const bool ok = rok && h < kdim;
            const double x = (double)X[(rc + (ok ? h : 0) * ld) * W];
            v[it] = ok ? x : 0.0;
        }
#pragma unroll
        for (int it = 0; it < 16; ++it) tile[rr][hh + 8 * it] = v[it];
    } else {  // element (r, h) at X[h + r*ld]: K contiguous
        const int hh = (t & 63) * 2, rq = t >> 6;
        const int64_t h = h0 + hh;
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const int64_t r = r0 + rq + 4 * it;
            const bool rok = r < rows;
            const bool ok0 = rok && h < kdim, ok1 = rok && h + 1 < kdim;
            const T *row = X + (rok ? r : 0) * ld * W;
            const double x0 = (double)row[(ok0 ? h : 0) * W], x1 = (double)row[(ok1 ? h + 1 : 0) * W];
            v[2 * it] = ok0 ? x0 : 0.0;
            v[2 * it + 1] = ok1 ? x1 : 0.0;
        }
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const int rr = rq + 4 * it;
            tile[rr][hh] = v[2 * it];
            tile[rr][hh + 1] = v[2 * it + 1];
        }
    }
}

// Low bytes of a, b, c, d packed little-endian into one word (v_perm_b32:
// selector bytes 0-3 pick from the second source, 4-7 from the first, 0x0c
// gives zero).
__device__ __forceinline__ uint32_t pack4(int a, int b, int c, int d) {
    const uint32_t lo = __builtin_amdgcn_perm((uint32_t)b, (uint32_t)a, 0x0c0c0400u);  // a0 b0 0 0
    const uint32_t hi = __builtin_amdgcn_perm((uint32_t)d, (uint32_t)c, 0x04000c0cu);  // 0 0 c0 d0
    return lo | hi;
}

// Streaming (non-temporal) stores for data this library writes once and does
// not read back soon: the residue planes of the split (read by the GEMM only
// after all of them are written) and C. On MI355X they skip allocation in the
// caches, so operands read shortly before (A and B, read by the norm pass and
// again by the split) stay cached: the split ran 13-16% faster at 4096^3.
// Only whole 16-byte stores are streamed: partial-line streaming stores were
// several times slower.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store16_nt(int8_t *dst, uint4 w) {
    __builtin_nontemporal_store((u32x4){w.x, w.y, w.z, w.w}, (u32x4 *)dst);
}

// cnt consecutive values v[0..cnt) to cp[0..cnt): streamed in 16-byte pieces
// when all NV are present and cp is 16-byte aligned, else plain stores.
template <class OutT, int NV>
__device__ __forceinline__ void store_run_nt(OutT *cp, const OutT (&v)[NV], int64_t cnt) {
    constexpr int per = 16 / (int)sizeof(OutT);
    static_assert(NV % per == 0, "whole 16-byte pieces");
    if (cnt >= NV && ((uintptr_t)cp & 15) == 0) {
        typedef OutT vec __attribute__((ext_vector_type(per)));
#pragma unroll
        for (int q = 0; q < NV / per; ++q) {
            vec x;
#pragma unroll
            for (int z = 0; z < per; ++z) x[z] = v[q * per + z];
            __builtin_nontemporal_store(x, (vec *)cp + q);
        }
    } else {
#pragma unroll
        for (int u = 0; u < NV; ++u)
            if (u < cnt) cp[u] = v[u];
    }
}

// One split block: rows [bx*32, +32) x K [by*128, +128) of X (KCONTIG: K
// runs along memory). ex_row(rr) gives the exponent of row bx*32 + rr.
template <bool KCONTIG, class T, class ExpOf>
__device__ __forceinline__ void split_block(double (*tile)[kSplitLd], const T *__restrict__ X, int64_t rows,
                                            int64_t kdim, int64_t ld, ExpOf ex_row, const SplitConsts &sc,
                                            int8_t *__restrict__ out, int64_t plane_bytes, int64_t kb, int64_t bx,
                                            int64_t by) {
    const int64_t r0 = bx * kSplitRows, h0 = by * kSplitCols;
    split_load_tile<KCONTIG, T>(tile, X, rows, kdim, ld, r0, h0);
    __syncthreads();

    const int t = threadIdx.x, fb = t >> 6, lane = t & 63, rr = (fb & 1) * 16 + (lane & 15);
    const int kk0 = (fb >> 1) * 64 + 16 * (lane >> 4);
    const int64_t r = r0 + rr;
    int e = r < rows ? ex_row(rr) : 0;
    const bool zero = (e == kExpNonfinite);
    if (zero) e = 0;

    // x = trunc(a * 2^e) is an integer with |x| < 2^84; split x = d1*2^42 + d0
    // exactly (|d0| < 2^42). Then x = d1*(2^42 mod p) + d0 (mod p) with that
    // sum below 2^49.2 in magnitude, so every fma below is exact and
    // rint(y / p) picks the symmetric residue without ties for odd p.
    double d0[16], d1[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
        double a = zero ? 0.0 : tile[rr][kk0 + u];
        double x = trunc(ldexp(a, e));
        double hi = trunc(x * 0x1p-42);
        d1[u] = hi;
        d0[u] = fma(-hi, 0x1p42, x);
    }

    const int64_t nkq = kb / 2;  // fragment blocks along K
    int8_t *dst = out + ((bx * 2 + (fb & 1)) * nkq + by * 2 + (fb >> 1)) * 1024 + lane * 16;
    // Only the low byte of a residue is stored, and the symmetric residue r of
    // an integer y has the low byte of y - k p for k = round(y / p): the low
    // word of y + 1.5 * 2^52 holds y mod 2^32 (|y| < 2^51, exact), that of
    // RN(y * RN(1/p) + 1.5 * 2^52) holds k mod 2^32 (y / p is never within
    // 2^-9 of a half-integer and the product is off by less than 2^-11), and
    // the 24-bit multiplier keeps k p mod 2^24.
    // modulus 256: x = d0 (mod 256), the low byte of d0
    {
        int v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) v[u] = __double2loint(d0[u] + 0x1.8p52);
        uint4 w;
        w.x = pack4(v[0], v[1], v[2], v[3]);
        w.y = pack4(v[4], v[5], v[6], v[7]);
        w.z = pack4(v[8], v[9], v[10], v[11]);
        w.w = pack4(v[12], v[13], v[14], v[15]);
        store16_nt(dst, w);
    }
    for (int l = 1; l < sc.n; ++l) {
        const double pinv = sc.pinv[l], c = sc.c42[l];
        const int mp = -(int)sc.p[l];
        int v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const double y = fma(d1[u], c, d0[u]);
            v[u] = __mul24(__double2loint(fma(y, pinv, 0x1.8p52)), mp) + __double2loint(y + 0x1.8p52);
        }
        uint4 w;
        w.x = pack4(v[0], v[1], v[2], v[3]);
        w.y = pack4(v[4], v[5], v[6], v[7]);
        w.z = pack4(v[8], v[9], v[10], v[11]);
        w.w = pack4(v[12], v[13], v[14], v[15]);
        store16_nt(dst + l * plane_bytes, w);
    }
}

// The complex form of split_block, over rows [bx*32, +32) x K [by*64, +64).
// Each modulus l gets three planes, 3l + 0: residues of trunc(2^e re),
// 3l + 1: of trunc(2^e im), 3l + 2: of their sum, the operands of the three
// products of Gauss' trick. The sum's residue comes from the exact splits:
// (d1r + d1i) 2^42 + (d0r + d0i) is the sum with |d0r + d0i| < 2^43, so
// y = (d1r + d1i)(2^42 mod p) + (d0r + d0i) stays below 2^50.2 and exact.
// The block covers two fragment blocks (rows 0-15 and 16-31); thread pairs
// share a lane's 16 bytes (8 K each), so every store of a wavefront covers 512
// contiguous bytes. Elements are loaded straight from memory (for A, 16 lanes
// read 16 consecutive complex rows at one k; for B each thread reads 8
// consecutive complex k): no LDS tile.
constexpr int kSplitColsC = 64;
template <bool KCONTIG, class T, class ExpOf>
__device__ __forceinline__ void split_block_c(const T *__restrict__ X, int64_t rows, int64_t kdim, int64_t ld,
                                              ExpOf ex_row, const SplitConsts &sc, int8_t *__restrict__ out,
                                              int64_t plane_bytes, int64_t kb, int64_t bx, int64_t by) {
    const int t = threadIdx.x, fb = t >> 7, q = t & 127, lane = q >> 1, half = q & 1, rr = fb * 16 + (lane & 15);
    const int64_t r = bx * kSplitRows + rr;
    const int64_t k0 = by * kSplitColsC + 16 * (lane >> 4) + 8 * half;
    const bool rok = r < rows;
    const int64_t rc = rok ? r : 0;
    double x[2][8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int64_t h = k0 + u;
        const bool ok = rok && h < kdim;
        const int64_t idx = KCONTIG ? (ok ? h : 0) + rc * ld : rc + (ok ? h : 0) * ld;
        const T re = X[2 * idx], im = X[2 * idx + 1];
        x[0][u] = ok ? (double)re : 0.0;
        x[1][u] = ok ? (double)im : 0.0;
    }
    // row exponents may come from LDS written before this call
    __syncthreads();
    int e = rok ? ex_row(rr) : 0;
    const bool zero = (e == kExpNonfinite);
    if (zero) e = 0;
    double d1[3][8], d0[3][8];  // exact splits of re, im and of their sum
#pragma unroll
    for (int u = 0; u < 8; ++u) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const double xs = zero ? 0.0 : trunc(ldexp(x[c][u], e));
            d1[c][u] = trunc(xs * 0x1p-42);
            d0[c][u] = fma(-d1[c][u], 0x1p42, xs);
        }
        d1[2][u] = d1[0][u] + d1[1][u];
        d0[2][u] = d0[0][u] + d0[1][u];
    }
    int8_t *dst = out + ((bx * 2 + fb) * (kb / 2) + by) * 1024 + lane * 16 + 8 * half;
    for (int l = 0; l < sc.n; ++l) {
        const double pinv = sc.pinv[l], c42 = sc.c42[l];
        const int mp = -(int)sc.p[l];
#pragma unroll
        for (int c = 0; c < 3; ++c) {
            int v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                // the low byte of y - p round(y / p), as in split_block
                // (|y| < 2^51; p = 256: c42 = 0 and 1/p is exact)
                const double y = fma(d1[c][u], c42, d0[c][u]);
                v[u] = __mul24(__double2loint(fma(y, pinv, 0x1.8p52)), mp) + __double2loint(y + 0x1.8p52);
            }
            uint2 w;
            w.x = pack4(v[0], v[1], v[2], v[3]);
            w.y = pack4(v[4], v[5], v[6], v[7]);
            *(uint2 *)(dst + (3 * l + c) * plane_bytes) = w;
        }
    }
}

// Steps 1 + 2 for both operands in one launch: blocks [0, nA) split A (row
// tile fastest, then K tile), the rest split B. FOLD: fast mode, where the
// exponents of A's rows are merged here from the row-norm partials (the first
// K tile of each row tile also stores them for the reconstruction); otherwise
// they are read from e.
template <bool FOLD, class T, int W, bool ORIG>
__global__ __launch_bounds__(256) void k_split(const T *__restrict__ A, int64_t m, int64_t lda,
                                               const T *__restrict__ B, int64_t n, int64_t ldb, int64_t kdim,
                                               int64_t tilesA, int64_t tilesB, int64_t nA,
                                               const double *__restrict__ ps,
                                               const int *__restrict__ pg, const int *__restrict__ pbad,
                                               int nchunks, double Pp, int32_t *__restrict__ e,
                                               const int32_t *__restrict__ f, SplitConsts sc,
                                               int8_t *__restrict__ RA, int64_t planeA, int8_t *__restrict__ RB,
                                               int64_t planeB, int64_t kb) {
    __shared__ double tile[W == 1 ? 1 : 0 + 1][W == 1 ? kSplitRows : 1][W == 1 ? kSplitLd : 1];
    __shared__ int sh_e[kSplitRows];
    const int64_t bid = blockIdx.x;
    auto split_tile = [&](auto kcontig, const T *X, int64_t rows, int64_t ld, auto ex_row, int8_t *out,
                          int64_t plane, int64_t bx, int64_t by) {
        constexpr bool KC = decltype(kcontig)::value;
        if constexpr (W == 2)
            split_block_c<KC, T>(X, rows, kdim, ld, ex_row, sc, out, plane, kb, bx, by);
        else
            split_block<KC, T>(tile[0], X, rows, kdim, ld, ex_row, sc, out, plane, kb, bx, by);
    };
    if (bid < nA) {
        const int64_t bx = bid % tilesA, by = bid / tilesA;
        if (FOLD) {
            if (threadIdx.x < kSplitRows) {
                const int64_t i = bx * kSplitRows + threadIdx.x;
                int ev = 0, gv = 0;
                if (i < m) row_exponent_from_partials<ORIG>(ps, pg, pbad, m, i, nchunks, Pp, ev, gv);
                sh_e[threadIdx.x] = ev;
                if (by == 0) e[i] = ev;  // i < m_pad: the workspace holds m_pad entries
            }
            // the barrier after the tile load orders these LDS writes
            split_tile(std::false_type{}, A, m, lda, [&](int rr) { return sh_e[rr]; }, RA, planeA, bx, by);
        } else {
            const int32_t *er = e + bx * kSplitRows;
            split_tile(std::false_type{}, A, m, lda, [&](int rr) { return (int)er[rr]; }, RA, planeA, bx, by);
        }
    } else {
        const int64_t b = bid - nA;
        const int64_t bx = b % tilesB, by = b / tilesB;
        const int32_t *fr = f + bx * kSplitRows;
        split_tile(std::true_type{}, B, n, ldb, [&](int rr) { return (int)fr[rr]; }, RB, planeB, bx, by);
    }
}

// Accurate mode: Abar_ih = ceil(|a_ih| * 2^(6 - r_i)) in [0, 64], same packing.
template <bool KCONTIG, class T>
__device__ __forceinline__ void quantize_block(double (*tile)[kSplitLd], const T *__restrict__ X, int64_t rows,
                                               int64_t kdim, int64_t ld, const int32_t *__restrict__ gx,
                                               int8_t *__restrict__ out, int64_t kb, int64_t bx, int64_t by) {
    const int64_t r0 = bx * kSplitRows, h0 = by * kSplitCols;
    split_load_tile<KCONTIG, T>(tile, X, rows, kdim, ld, r0, h0);
    __syncthreads();
    const int t = threadIdx.x, fb = t >> 6, lane = t & 63, rr = (fb & 1) * 16 + (lane & 15);
    const int kk0 = (fb >> 1) * 64 + 16 * (lane >> 4);
    const int64_t r = r0 + rr;
    int g = r < rows ? gx[r] : 0;
    const bool zero = (g == kExpNonfinite);
    if (zero) g = 0;
    int v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
        double a = zero ? 0.0 : fabs(tile[rr][kk0 + u]);
        v[u] = (int)ceil(ldexp(a, 6 - g));
    }
    uint4 w;
    w.x = pack4(v[0], v[1], v[2], v[3]);
    w.y = pack4(v[4], v[5], v[6], v[7]);
    w.z = pack4(v[8], v[9], v[10], v[11]);
    w.w = pack4(v[12], v[13], v[14], v[15]);
    *(uint4 *)(out + ((bx * 2 + (fb & 1)) * (kb / 2) + by * 2 + (fb >> 1)) * 1024 + lane * 16) = w;
}

// Both bound operands in one launch: blocks [0, nA) quantize A (row tile
// fastest, then K tile), the rest B.
template <class T>
__global__ __launch_bounds__(256) void k_quantize(const T *__restrict__ A, int64_t m, int64_t lda,
                                                  const T *__restrict__ B, int64_t n, int64_t ldb, int64_t kdim,
                                                  int64_t tilesA, int64_t tilesB, int64_t nA,
                                                  const int32_t *__restrict__ ga, const int32_t *__restrict__ gb,
                                                  int8_t *__restrict__ abar, int8_t *__restrict__ bbar, int64_t kb) {
    __shared__ double tile[kSplitRows][kSplitLd];
    const int64_t bid = blockIdx.x;
    if (bid < nA) {
        quantize_block<false, T>(tile, A, m, kdim, lda, ga, abar, kb, bid % tilesA, bid / tilesA);
    } else {
        const int64_t b = bid - nA;
        quantize_block<true, T>(tile, B, n, kdim, ldb, gb, bbar, kb, b % tilesB, b / tilesB);
    }
}

// ---------------------------------------------------------------------------
// Step 3: INT8 GEMM per modulus on v_mfma_i32_16x16x64_i8
// ---------------------------------------------------------------------------
// Block tile 256 x 256, eight wavefronts in 2 x 4 (two per SIMD), each owning
// 128 x 64 (8 x 4 MFMA tiles of 16 x 16, 128 int32 accumulators per lane);
// for products too small to give every CU two such tiles, a 128 x 128 tile of
// four wavefronts (64 x 64 each, two blocks per CU) with the same schedule.
// K advances 64 bytes per LDS stage, one MFMA k-step. Stages are copied
// global -> LDS with global_load_lds_dwordx4 (no VGPR staging) into a ring of
// kNST = 5 buffers (all 160 KiB of LDS; 80 KiB for the small shape): while the
// 32 MFMAs of a stage run on fragments already in registers (16 in the small
// shape), the wave reads the next stage's 12 fragments (8) and issues its 4
// copies for the stage kNST - 1 ahead, and the
// block barrier at the end of the stage leaves two stages in flight. The
// 16 x 16 x 64 form is used rather than 32 x 32 x 32 because on random
// residues MI355X sustains more INT8 throughput with it under its power
// limit (it moves less accumulator data per operation). The grid runs over
// (modulus, tile row, tile column); block ids are remapped so each XCD works
// through a compact group of tiles of one modulus and its L2 serves the shared
// A and B panels. With more 256 x 256 tiles than compute units (and four or
// more stages per launch) they run on the persistent one-wave-per-SIMD kernel
// further below (k_gemm_persistent), which keeps this kernel's ring, tile order
// and epilogue.
constexpr int kBK = 64;                    // K bytes per stage (one MFMA k-step)
constexpr int kNST = 5;                    // LDS stages in the ring
constexpr int kLoadsPerWave = 4;           // 1 KiB copies per wave per stage of k_gemm (both of its shapes)
constexpr int kGroupM = 4;                 // tile rows per raster group
constexpr int kReduceStages = 1024;        // stages per launch: 1024 * 64 * 2^14 = 2^30, the range of smod
// copies a wave may leave in flight at a stage barrier: the kNST - 3 stages
// after the one the next stage reads
#define OZ2_GEMM_VMCNT "8"
static_assert((kNST - 3) * kLoadsPerWave == 8, "OZ2_GEMM_VMCNT must equal (kNST - 3) * kLoadsPerWave");

// A block shape: WM x WN wavefronts, each owning RT x CT MFMA tiles of 16 x 16
// and issuing LPW 1 KiB copies per stage.
template <int WM_, int WN_, int RT_, int CT_, int LPW_ = kLoadsPerWave>
struct GemmShape {
    static constexpr int WM = WM_, WN = WN_, RT = RT_, CT = CT_, LPW = LPW_;
    static constexpr int W = WM * WN;                        // wavefronts per block
    static constexpr int TM = WM * RT * 16, TN = WN * CT * 16;  // block tile
    static constexpr int FA = TM / 16, FB = TN / 16;         // fragment blocks per stage
    static constexpr int STAGE = (FA + FB) * 1024;           // bytes per LDS stage
    static constexpr int NF = RT + CT;                       // fragments a wave reads per stage
    static constexpr int NQ = RT * CT;                       // MFMAs per wave per stage
    static_assert(FA == FB && FA == (W / 2) * LPW, "half the waves copy A, half B");
    static_assert(kNST * STAGE <= 160 * 1024, "the ring must fit in LDS");
    static_assert(NQ % LPW == 0 && NF % LPW == 0, "copies and reads spread evenly");
    static_assert(RT % 4 == 0, "the epilogue transposes groups of four row tiles");
};
using ShapeL = GemmShape<2, 4, 8, 4>;     // 256 x 256, 8 waves of 128 x 64
using ShapeS = GemmShape<2, 2, 4, 4>;     // 128 x 128, 4 waves of 64 x 64
using ShapeP = GemmShape<2, 2, 8, 8, 8>;  // 256 x 256, 4 waves of 128 x 128 (persistent kernel)
static_assert(ShapeP::TM == ShapeL::TM && ShapeP::TN == ShapeL::TN, "both large kernels cover one tile grid");

enum { EPI_MOD = 0, EPI_RAW = 1, EPI_BOUND = 2 };

struct GemmArgs {
    const int8_t *RA;
    const int8_t *RB;
    int64_t planeA, planeB;  // bytes per modulus of RA, RB
    int64_t kb;              // K / 32
    int64_t ks0;             // first stage (64 K) of this launch
    int nks;                 // stages of this launch (even)
    int accumulate;          // EPI_MOD: add the residues already in the planes
    int tiles_m, tiles_n, nmod;  // nmod: operand/output planes (moduli x group)
    int group;                   // planes per modulus: 1 (real) or 3 (complex)
    int64_t m_pad;
    // epilogues
    int8_t *planes;          // EPI_MOD: [nmod][n_pad][m_pad], symmetric residues
    int32_t *raw;            // EPI_RAW: [nmod][n_pad][m_pad]
    int32_t *rowmax;         // EPI_BOUND
    int32_t *colmax;
    int64_t plane_elems;     // n_pad * m_pad
};

__device__ __forceinline__ void decode_block(int bid, int total, int tiles_m, int tiles_n, int &l, int &tm,
                                             int &tn) {
    // XCD-aware remap: hardware deals consecutive block ids round-robin over
    // the 8 XCDs; give each XCD one contiguous range of the logical order.
    int lid = bid;
    if ((total & 7) == 0) lid = (bid & 7) * (total >> 3) + (bid >> 3);
    const int per = tiles_m * tiles_n;
    l = lid / per;
    int rem = lid - l * per;
    const int group = kGroupM * tiles_n;
    const int gid = rem / group;
    const int first = gid * kGroupM;
    const int gsz = min(tiles_m - first, kGroupM);
    const int in = rem - gid * group;
    tm = first + in % gsz;
    tn = in / gsz;
}

// Symmetric residue r = q - p * round(q / p) of an int32 sum with
// |q| <= 2^30 + 128. One FMA, t = RN(q * RN(1/p) + 1.5 * 2^52), leaves
// round(q / p) in the low word of t: the product is off from q / p by less
// than 2^-30, while for odd p >= 173 q / p is never closer than 1/(2p) to a
// half-integer; for p = 256 the product is exact and the FMA rounds ties to
// even. |round(q / p)| < 2^23, so q - k p is exact with the 24-bit multiplier.
// r lies in [-(p-1)/2, (p-1)/2] (or [-128, 128] for p = 256, stored as a
// byte, where 128 and -128 are the same residue).
__device__ __forceinline__ int smod(int q, double pinv, int p) {
    const double t = fma((double)q, pinv, 0x1.8p52);
    return __mul24(__double2loint(t), -p) + q;  // one v_mad_i32_i24
}

// Step 3 output of one wavefront: its 8 x 4 accumulator tiles reduced mod p
// and stored with 16-byte stores. In a 16 x 16 tile lane L holds rows
// 4 (L/16) .. 4 (L/16) + 3 of column L % 16, one packed word; for four tiles
// stacked in rows, the four lanes L % 16 + 16 q trade words in a 4 x 4
// transpose (two exchange rounds, across lanes L ^ 32 and L ^ 16) so that
// each ends with the 16 consecutive rows of one tile.
// LANE32: the lane's part of the address, (L % 16) m_pad + 16 (L / 16), fits
// 32 bits (m_pad < 2^27) and is added to a wave-uniform tile address, which
// keeps the address arithmetic in scalar registers and one VGPR.
template <int RT, int CT, bool LANE32 = false>
__device__ __forceinline__ void store_mod_tiles(const v4i (&acc)[RT][CT], int p, double pinv, int8_t *plane,
                                                int64_t m_pad, int row0, int col0, int lane, bool accumulate) {
    // LANE32 re-derives the lane index here (v_mbcnt, opaque to the optimiser) so
    // that neither it nor an address built from it stays live across a caller's
    // loop, where every VGPR is taken
    int ln = lane;
    if constexpr (LANE32)
        asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
    const uint32_t lane_elem = (uint32_t)(ln & 15) * (uint32_t)m_pad + 16u * (uint32_t)(ln >> 4);
#pragma unroll
    for (int j = 0; j < CT; ++j)
#pragma unroll
        for (int g = 0; g < RT / 4; ++g) {
            uint32_t w[4];  // w[c]: rows 4 (L/16) + 0..3 of tile 4g + c
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const v4i a = acc[4 * g + c][j];
                w[c] = pack4(smod(a[0], pinv, p), smod(a[1], pinv, p), smod(a[2], pinv, p), smod(a[3], pinv, p));
            }
            // exchange across the wavefront halves, then across the odd and even
            // rows of 16 lanes: permlane32_swap(x, y) trades x of lanes 32..63
            // with y of lanes 0..31, permlane16_swap(x, y) x of the odd rows
            // with y of the even rows
            const auto h0 = __builtin_amdgcn_permlane32_swap(w[0], w[2], false, false);
            const auto h1 = __builtin_amdgcn_permlane32_swap(w[1], w[3], false, false);
            const auto q0 = __builtin_amdgcn_permlane16_swap(h0[0], h1[0], false, false);
            const auto q1 = __builtin_amdgcn_permlane16_swap(h0[1], h1[1], false, false);
            w[0] = q0[0];
            w[1] = q0[1];
            w[2] = q1[0];
            w[3] = q1[1];
            // now w[c] = rows 4c .. 4c + 3 of tile 4g + L/16
            uint4 *dst;
            if constexpr (LANE32)
                dst = (uint4 *)(plane + (int64_t)(col0 + 16 * j) * m_pad + (row0 + 64 * g) + lane_elem);
            else
                dst = (uint4 *)(plane + (int64_t)(col0 + 16 * j + (lane & 15)) * m_pad + row0 +
                                16 * (4 * g + (lane >> 4)));
            if (accumulate) {
                // a later block of the inner dimension: add the residues of the
                // earlier blocks (|sum| <= 256) and reduce again
                const uint4 o = *dst;
                const uint32_t ow[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    int r[4];
#pragma unroll
                    for (int b = 0; b < 4; ++b)
                        r[b] = smod(__builtin_amdgcn_sbfe((int)w[c], 8 * b, 8) + __builtin_amdgcn_sbfe((int)ow[c], 8 * b, 8),
                                    pinv, p);
                    w[c] = pack4(r[0], r[1], r[2], r[3]);
                }
            }
            *dst = make_uint4(w[0], w[1], w[2], w[3]);
            // one group of four tiles at a time: keeps the accumulator reads
            // from being hoisted into one register-hungry block
            if constexpr (LANE32) __builtin_amdgcn_sched_barrier(0);
        }
}

// One launch covers stages [ks0, ks0 + nks) of the inner dimension. Longer
// inner dimensions run in several launches of at most kReduceStages stages
// (the blocks of [Q] step 3), each adding its residues to those already in the
// planes, so every int32 sum stays within smod's range.
template <int EPI, class SH>
__global__ __launch_bounds__(64 * SH::W) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_gemm(GemmArgs ga,
                                                                                                ModConsts mc) {
    constexpr int RT = SH::RT, CT = SH::CT, NF = SH::NF, NQ = SH::NQ, FA = SH::FA, STAGE = SH::STAGE;
    __shared__ __attribute__((aligned(1024))) int8_t lds[kNST * STAGE];

    int l, tm, tn;
    decode_block(blockIdx.x, gridDim.x, ga.tiles_m, ga.tiles_n, l, tm, tn);
    // wave index made explicitly wave-uniform so that all copy addressing
    // below stays in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int wm = wave / SH::WN, wn = wave % SH::WN;

    v4i acc[RT][CT];
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int j = 0; j < CT; ++j) acc[i][j] = (v4i){0, 0, 0, 0};

    const int nk = ga.nks;                              // even
    const int64_t row_bytes = (ga.kb / 2) * 1024;       // one 16-row block over all of K

    // Copy q of a stage (q = 0..3): the first half of the waves copy A
    // fragment blocks (row blocks 4w .. 4w + 3 of the tile), the rest B blocks. Source =
    // wave-uniform row block address + stage * 1 KiB + lane * 16; destination =
    // uniform LDS address (M0). Past the last stage the copy is still issued
    // (from the last stage, into a ring slot that is never read again) so the
    // main loop has no branch and the counter waits stay constant.
    const bool copies_a = wave < SH::W / 2;
    const int wq = wave % (SH::W / 2);
    const int8_t *dma_base = (copies_a ? ga.RA + (int64_t)l * ga.planeA + ((int64_t)tm * FA + wq * 4) * row_bytes
                                       : ga.RB + (int64_t)l * ga.planeB + ((int64_t)tn * SH::FB + wq * 4) * row_bytes) +
                             lane * 16;
    __attribute__((address_space(3))) int8_t *lds3 = (__attribute__((address_space(3))) int8_t *)lds;
    auto dma = [&](int ks_slot, int q) {
        const int ks = ks_slot < nk ? ks_slot : nk - 1;
        __builtin_amdgcn_global_load_lds(dma_base + q * row_bytes + (ga.ks0 + ks) * 1024,
                                         lds3 + (ks_slot % kNST) * STAGE + (wave * kLoadsPerWave + q) * 1024,
                                         16, 0, 0);
    };
    // fragment r of a stage: r < RT -> A tile r of this wave, else B tile r - RT
    auto frag = [&](const int8_t *stage, int r) {
        return *(const v4i *)(stage + (r < RT ? wm * RT + r : FA + wn * CT + (r - RT)) * 1024 + lane * 16);
    };

    // The block barriers below are plain s_barrier with explicit counter waits:
    // __syncthreads() would also drain every in-flight copy.
#pragma unroll
    for (int st = 0; st < kNST - 1; ++st)
#pragma unroll
        for (int q = 0; q < kLoadsPerWave; ++q) dma(st, q);
    asm volatile("s_waitcnt vmcnt(" OZ2_GEMM_VMCNT ")\n\ts_barrier" ::: "memory");  // stages 0 and 1 landed

    v4i f0[NF], f1[NF];  // fragments of the current / next stage: A tiles, then B tiles
#pragma unroll
    for (int r = 0; r < NF; ++r) f0[r] = frag(lds, r);

    // One stage: NQ MFMA slots in 4 groups of SG; the first RG slots of group
    // u also read fragments RG u .. RG u + RG - 1 of the next stage, slot
    // SG / 2 of group u issues copy u (256 x 256: 8 slots, 3 reads).
    // sched_barrier keeps this exact order. At the end: the stage after next
    // must have landed (it is read during the next stage) and every read of the
    // next stage's buffer must be done before a later copy can refill it.
    constexpr int SG = NQ / kLoadsPerWave, RG = NF / kLoadsPerWave;
    auto stage = [&](int ks, v4i(&fc)[NF], v4i(&fn)[NF]) {
        const int8_t *nxt = lds + ((ks + 1) % kNST) * STAGE;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            acc[q / CT][q % CT] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fc[q / CT], fc[RT + q % CT], acc[q / CT][q % CT], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            if ((q % SG) < RG) fn[(q / SG) * RG + (q % SG)] = frag(nxt, (q / SG) * RG + (q % SG));
            if ((q % SG) == SG / 2) dma(ks + kNST - 1, q / SG);
            __builtin_amdgcn_sched_barrier(0);
        }
        asm volatile("s_waitcnt vmcnt(" OZ2_GEMM_VMCNT ") lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };

    for (int ks = 0; ks < nk; ks += 2) {  // nk is even
        stage(ks, f0, f1);
        stage(ks + 1, f1, f0);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // drain the trailing copies before the block ends

    // Accumulator layout of a 16 x 16 MFMA tile: lane L, register v holds row
    // 4 * (L/16) + v, column L % 16.
    const int row0 = tm * SH::TM + wm * RT * 16, col0 = tn * SH::TN + wn * CT * 16;
    if (EPI == EPI_MOD) {
        store_mod_tiles(acc, (int)mc.p[l / ga.group], mc.pinv[l / ga.group], ga.planes + (int64_t)l * ga.plane_elems,
                        ga.m_pad, row0, col0, lane, ga.accumulate != 0);
    } else if (EPI == EPI_RAW) {
        int32_t *plane = ga.raw + (int64_t)l * ga.plane_elems;
#pragma unroll
        for (int i = 0; i < RT; ++i)
#pragma unroll
            for (int j = 0; j < CT; ++j) {
                const int64_t col = col0 + 16 * j + (lane & 15);
                const int row = row0 + 16 * i + 4 * (lane >> 4);
                *(int4 *)(plane + col * ga.m_pad + row) =
                    make_int4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
            }
    } else {  // EPI_BOUND: row and column maxima of the (non-negative) bound product
#pragma unroll
        for (int i = 0; i < RT; ++i) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                int mx = acc[i][0][v];
#pragma unroll
                for (int j = 1; j < CT; ++j) mx = max(mx, acc[i][j][v]);
                // reduce over the 16 lanes that share this row (same L / 16)
#pragma unroll
                for (int off = 8; off >= 1; off >>= 1) mx = max(mx, __shfl_xor(mx, off, 64));
                if ((lane & 15) == 0) atomicMax(&ga.rowmax[row0 + 16 * i + 4 * (lane >> 4) + v], mx);
            }
        }
#pragma unroll
        for (int j = 0; j < CT; ++j) {
            int mx = 0;
#pragma unroll
            for (int i = 0; i < RT; ++i)
#pragma unroll
                for (int v = 0; v < 4; ++v) mx = max(mx, acc[i][j][v]);
            // reduce over the 4 lanes that share this column (same L % 16)
            mx = max(mx, __shfl_xor(mx, 16, 64));
            mx = max(mx, __shfl_xor(mx, 32, 64));
            if (lane < 16) atomicMax(&ga.colmax[col0 + 16 * j + lane], mx);
        }
    }
}

// ---------------------------------------------------------------------------
// Step 3, persistent form of the 256 x 256 tile: one block per compute unit
// walks the tiles bid = blockIdx.x + i * gridDim.x (the same XCD-aware order
// as k_gemm's grid). Four wavefronts, one per SIMD, each own a 128 x 128
// quarter (8 x 8 MFMA tiles, 256 accumulators per lane), so every fragment
// read from LDS feeds eight MFMAs instead of six (a third fewer LDS bytes per
// operation than k_gemm's 128 x 64). The five-slot copy ring runs on across
// tile boundaries: the first four stages of the next tile are copied during the
// last four stages of the current one and land while its epilogue runs.
//
// With one wavefront per SIMD nothing else issues while this one is busy with
// anything but an MFMA, and a wavefront issues at most one instruction per
// four cycles against 16 cycles per MFMA, so the stage schedule keeps at most a
// few instructions between consecutive MFMAs: the block barrier after the 4th
// MFMA of every second stage, one fragment read every 3rd MFMA from the 5th,
// one copy every 6th MFMA from the 6th. A copy is two instructions: an M0
// write (the LDS address) after one MFMA, and after the next a
// buffer_load_dwordx4 ... lds whose resource holds the stage's source address
// and whose scalar offset selects the 16-row block, with the lane offset in one
// VGPR; the MFMA between them provides the wait state an M0 write needs before
// an LDS-DMA load.
//
// Counter waits: vector-memory operations of a wavefront complete in issue
// order, so waiting for some copies means allowing only the operations issued
// after them. The barrier in stage ks (even) waits for the copies of stages
// ks + 1 and ks + 2, read in stages ks and ks + 1, allowing those of ks + 3 (8);
// in a tile's first stage the 16 stores of the previous tile's epilogue sit
// after them too (24). Before the first tile the prologue issues 16 extra
// copies (the same bytes as the first stage's own copies, into the same slot)
// so that the first tile sees the same counts. Requires nks >= kNST - 1 (and
// even), so the copies never reach beyond the next tile.
// ---------------------------------------------------------------------------
template <int N>
__device__ __forceinline__ void vm_wait_barrier() {
    static_assert(N == 8 || N == 16 || N == 24 || N == 32 || N == 40, "add the count");
    if constexpr (N == 8)
        asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");
    else if constexpr (N == 16)
        asm volatile("s_waitcnt vmcnt(16)\n\ts_barrier" ::: "memory");
    else if constexpr (N == 24)
        asm volatile("s_waitcnt vmcnt(24)\n\ts_barrier" ::: "memory");
    else if constexpr (N == 32)
        asm volatile("s_waitcnt vmcnt(32)\n\ts_barrier" ::: "memory");
    else
        asm volatile("s_waitcnt vmcnt(40)\n\ts_barrier" ::: "memory");
}

// Buffer resource for the copies of one stage (raw, stride 0): base = the
// stage's first byte in the wave's copy rows (a device address below 2^47,
// so its high word leaves the stride field zero), nrec bytes from it.
__device__ __forceinline__ v4i copy_rsrc(uint64_t base, uint32_t nrec) {
    return (v4i){(int)(uint32_t)base, (int)((uint32_t)(base >> 32) & 0xffffu), (int)nrec, 0x00020000};
}

// M0 = base + c KiB (one SALU instruction; c a constant after unrolling). The
// copy that uses it is a separate statement one MFMA later; this relies on the
// compiler not touching M0 in between, which holds in k_gemm_persistent (it
// has no LDS-DMA builtins, messages or indexed register moves that would make
// the compiler write M0; the compiled code shows no other M0 writes).
__device__ __forceinline__ void set_m0_kib(uint32_t base, int c) {
    switch (c) {
    case 0: asm volatile("s_mov_b32 m0, %0" :: "s"(base) : "memory"); break;
    case 1: asm volatile("s_add_i32 m0, %0, 0x400" :: "s"(base) : "memory"); break;
    case 2: asm volatile("s_add_i32 m0, %0, 0x800" :: "s"(base) : "memory"); break;
    case 3: asm volatile("s_add_i32 m0, %0, 0xc00" :: "s"(base) : "memory"); break;
    case 4: asm volatile("s_add_i32 m0, %0, 0x1000" :: "s"(base) : "memory"); break;
    case 5: asm volatile("s_add_i32 m0, %0, 0x1400" :: "s"(base) : "memory"); break;
    case 6: asm volatile("s_add_i32 m0, %0, 0x1800" :: "s"(base) : "memory"); break;
    default: asm volatile("s_add_i32 m0, %0, 0x1c00" :: "s"(base) : "memory"); break;
    }
}

__global__ __launch_bounds__(64 * ShapeP::W) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_gemm_persistent(
        GemmArgs ga, ModConsts mc) {
    constexpr int RT = ShapeP::RT, CT = ShapeP::CT, NF = ShapeP::NF, NQ = ShapeP::NQ, FA = ShapeP::FA;
    constexpr int FB = ShapeP::FB, STAGE = ShapeP::STAGE, LPW = ShapeP::LPW, W = ShapeP::W, WN = ShapeP::WN;
    constexpr int TM = ShapeP::TM, TN = ShapeP::TN;
    constexpr int NSTORE = RT * CT / 4;  // 16-byte stores of one epilogue
    constexpr int PRE = 4, RSTEP = 3, CSTEP = 6;
    static_assert(NSTORE == 2 * LPW, "the prologue's extra copies stand in for one epilogue's stores");
    static_assert(PRE + RSTEP * (NF - 1) < NQ && PRE + 1 + CSTEP * (LPW - 1) < NQ, "schedule fits a stage");
    __shared__ __attribute__((aligned(1024))) int8_t lds[kNST * STAGE];

    const int total = ga.tiles_m * ga.tiles_n * ga.nmod;
    const int G = gridDim.x;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int wm = wave / WN, wn = wave % WN;
    const int nk = ga.nks;
    const int64_t row_bytes = (ga.kb / 2) * 1024;
    const bool copies_a = wave < W / 2;
    const int wq = wave % (W / 2);
    // q * row_bytes < 2^32 (the launcher checks it)
    const uint32_t rb32 = (uint32_t)row_bytes;
    const uint32_t nrec = (uint32_t)(LPW - 1) * rb32 + 1024u;
    auto source = [&](int b, int &l, int &tm, int &tn) -> uint64_t {
        decode_block(b, total, ga.tiles_m, ga.tiles_n, l, tm, tn);
        return (uint64_t)(uintptr_t)((copies_a ? ga.RA + (int64_t)l * ga.planeA + ((int64_t)tm * FA + wq * LPW) * row_bytes
                                               : ga.RB + (int64_t)l * ga.planeB + ((int64_t)tn * FB + wq * LPW) * row_bytes) +
                                     ga.ks0 * 1024);
    };
    const uint32_t lane_off = (uint32_t)lane * 16u;
    // LDS byte address of this wave's first copy slot; taken from the array's
    // address so the compiler sees the copies (inline asm) may write it
    const uint32_t wave_lds = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) int8_t *)lds) +
                              (uint32_t)(wave * LPW * 1024);
    auto frag = [&](const int8_t *st, int r) {
        return *(const v4i *)(st + (r < RT ? wm * RT + r : FA + wn * CT + (r - RT)) * 1024 + lane * 16);
    };

    int bid = blockIdx.x;
    int l, tm, tn, nl = 0, ntm = 0, ntn = 0;
    uint64_t cur = source(bid, l, tm, tn);
    int nbid = bid + G;
    uint64_t nxt = nbid < total ? source(nbid, nl, ntm, ntn) : cur;
    // copies issued in stage ks read stage t = ks + kNST - 1 of this tile, or
    // stage t - nk of the next one (tail = the next tile, or this one again
    // after the last tile: an in-bounds copy into a slot that is never read)
    uint64_t tail = nxt;
    uint64_t src = kNST - 1 < nk ? cur + (kNST - 1) * 1024 : tail;

    v4i acc[RT][CT];
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int j = 0; j < CT; ++j) acc[i][j] = (v4i){0, 0, 0, 0};
#pragma unroll
    for (int st = 0; st < kNST - 1; ++st) {
        const v4i rs = copy_rsrc(cur + st * 1024, nrec);
#pragma unroll
        for (int q = 0; q < LPW; ++q)
            asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %3 offen lds"
                         :: "v"(lane_off), "s"(rs), "s"((uint32_t)(st * STAGE) + wave_lds + q * 1024u),
                            "s"(q * rb32) : "memory");
    }
    {
        const v4i rs = copy_rsrc(src, nrec);  // the first stage's own copies, issued twice more
#pragma unroll
        for (int q = 0; q < NSTORE; ++q)
            asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %3 offen lds"
                         :: "v"(lane_off), "s"(rs), "s"((uint32_t)((kNST - 1) * STAGE) + wave_lds + (q % LPW) * 1024u),
                            "s"((q % LPW) * rb32) : "memory");
    }
    vm_wait_barrier<3 * LPW + NSTORE>();  // stage 0 landed
    v4i f0[NF], f1[NF];
#pragma unroll
    for (int r = 0; r < NF; ++r) f0[r] = frag(lds, r);

    uint32_t rd_off = STAGE;                  // slot read during this stage (that of stage ks + 1)
    uint32_t cp_off = (kNST - 1) * STAGE;     // slot the copies of this stage fill
    // stage ks: MFMAs on fc, reads of the next stage into fn (B fragments
    // first), copies for stage ks + kNST - 1; WAIT: the counter value of the
    // stage's barrier, 0 for a stage without one
    auto stage = [&](auto wait, int ks, v4i(&fc)[NF], v4i(&fn)[NF]) {
        const int8_t *next = lds + rd_off;
        const v4i rs = copy_rsrc(src, nrec);
        const uint32_t cbase = cp_off + wave_lds;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            acc[q / CT][q % CT] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fc[q / CT], fc[RT + q % CT],
                                                                       acc[q / CT][q % CT], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            if (q == PRE - 1) {
                if constexpr (decltype(wait)::value > 0) vm_wait_barrier<decltype(wait)::value>();
            }
            if (q >= PRE && (q - PRE) % RSTEP == 0 && (q - PRE) / RSTEP < NF) {
                const int i = (q - PRE) / RSTEP;
                const int r = i < CT ? RT + i : i - CT;
                fn[r] = frag(next, r);
            }
            // copy c: M0 set after MFMA PRE + CSTEP c, the load one MFMA later
            // (the MFMA between provides the wait state the M0 write needs)
            if (q >= PRE && (q - PRE) % CSTEP == 0 && (q - PRE) / CSTEP < LPW) set_m0_kib(cbase, (q - PRE) / CSTEP);
            if (q == PRE + 1)
                asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" :: "v"(lane_off), "s"(rs) : "memory");
            else if (q > PRE + 1 && (q - PRE - 1) % CSTEP == 0 && (q - PRE - 1) / CSTEP < LPW)
                asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds"
                             :: "v"(lane_off), "s"(rs), "s"((uint32_t)((q - PRE - 1) / CSTEP) * rb32) : "memory");
            __builtin_amdgcn_sched_barrier(0);
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        // the next stage's slots and copy source
        rd_off = rd_off == (kNST - 1) * STAGE ? 0u : rd_off + STAGE;
        cp_off = cp_off == (kNST - 1) * STAGE ? 0u : cp_off + STAGE;
        src = ks + kNST == nk ? tail : src + 1024;
    };

    // a block barrier every second stage: the one in stage ks (even) waits for
    // stages ks + 1 and ks + 2 (read in stages ks and ks + 1), and orders every
    // read of the slots the copies of stages ks and ks + 1 refill before them
    const std::integral_constant<int, LPW + NSTORE> first;  // stage 3's copies and NSTORE more after stage 2's
    const std::integral_constant<int, LPW> even;
    const std::integral_constant<int, 0> odd;
    while (true) {
        stage(first, 0, f0, f1);
        stage(odd, 1, f1, f0);
        for (int ks = 2; ks < nk; ks += 2) {
            stage(even, ks, f0, f1);
            stage(odd, ks + 1, f1, f0);
        }
        const int row0 = tm * TM + wm * RT * 16, col0 = tn * TN + wn * CT * 16;
        store_mod_tiles<RT, CT, true>(acc, (int)mc.p[l / ga.group], mc.pinv[l / ga.group],
                                      ga.planes + (int64_t)l * ga.plane_elems, ga.m_pad, row0, col0, lane,
                                      ga.accumulate != 0);
#pragma unroll
        for (int i = 0; i < RT; ++i)
#pragma unroll
            for (int j = 0; j < CT; ++j) acc[i][j] = (v4i){0, 0, 0, 0};
        bid = nbid;
        if (bid >= total) break;
        cur = nxt;
        l = nl;
        tm = ntm;
        tn = ntn;
        nbid = bid + G;
        if (nbid < total) nxt = source(nbid, nl, ntm, ntn);
        tail = nxt;
        src = kNST - 1 < nk ? cur + (kNST - 1) * 1024 : tail;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// ---------------------------------------------------------------------------
// Steps 4 + 5: CRT in exact 40-bit pieces, symmetric lift, round, unscale
// ---------------------------------------------------------------------------
// S = sum_l c_l W_l (c_l the symmetric residues, |c_l| <= 128) is kept as four
// doubles S_t (S = sum_t S_t 2^(40 t)); every term |c_l W_l,t| < 2^47 and the
// sums stay below 2^51.4 in magnitude, so they are exact in any order. q = round(S / P) comes from a double estimate; X_t = S_t - q P_t
// is again exact, carries are propagated, and the rare estimate that lands a
// hair outside (-P/2, P/2] is corrected on the exact pieces. The integer X is
// finally rounded to nearest-even from its 160-bit image, so C equals
// RN(X) * 2^-(e_i + f_j) exactly.
// Pieces of BITS bits: x = sum_t x[t] 2^(BITS t), each x[t] an integer held
// exactly in a double. normalize brings x[0..2] into [0, 2^BITS) and leaves the
// signed remainder in x[3].
template <int BITS, int NP = 4>
__device__ __forceinline__ void normalize4(double x[NP]) {
    constexpr double base = (double)(1ull << BITS), inv = 1.0 / base;
#pragma unroll
    for (int t = 0; t < NP - 1; ++t) {
        double c = floor(x[t] * inv);
        x[t] = fma(-c, base, x[t]);
        x[t + 1] += c;
    }
}

// sign of a normalized piece vector: -1, 0, +1
template <int NP = 4>
__device__ __forceinline__ int sign4(const double x[NP]) {
    if (x[NP - 1] != 0.0) return x[NP - 1] > 0.0 ? 1 : -1;
    bool nz = false;
#pragma unroll
    for (int t = 0; t < NP - 1; ++t) nz = nz || x[t] != 0.0;
    return nz ? 1 : 0;
}

// Exact repair of an estimated quotient: bring X into (-P/2, P/2], with P and
// H = P/2 in the same pieces as x.
template <int BITS, int NP = 4>
__device__ __forceinline__ void crt_range_fix(double x[NP], const double P[], const double H[]) {
    double z[NP];
#pragma unroll
    for (int t = 0; t < NP; ++t) z[t] = x[t] - H[t];
    normalize4<BITS, NP>(z);
    if (sign4<NP>(z) > 0) {  // X > P/2
#pragma unroll
        for (int t = 0; t < NP; ++t) x[t] -= P[t];
        normalize4<BITS, NP>(x);
        return;
    }
#pragma unroll
    for (int t = 0; t < NP; ++t) z[t] = x[t] + H[t];
    normalize4<BITS, NP>(z);
    if (sign4<NP>(z) <= 0) {  // X <= -P/2
#pragma unroll
        for (int t = 0; t < NP; ++t) x[t] += P[t];
        normalize4<BITS, NP>(x);
    }
}

// X = S - q P with q = round(S / P) from a double estimate; X keeps the sign
// the estimate predicts (sg) and its magnitude goes to x. The estimate of S / P
// is good to ~2^-37 absolute, so only |S/P - q| within 2^-30 of 1/2 needs the
// exact wrap check, which valid scalings never reach; the second check catches
// |X| below ~2^-37 P, where the predicted sign can be wrong.
// ZERO_POS: S may be a nonzero multiple of P (the complex form's unreduced
// residues), so X = 0 can come with either predicted sign; it gets +1, the
// sign of RN(0) in the oracle.
template <int BITS, int NP = 4, bool ZERO_POS = false>
__device__ __forceinline__ void crt_lift(const double S[NP], double x[NP], double &sg, double s_over_base3,
                                         const double P[], const double H[], double pinv_base3) {
    const double quo = s_over_base3 * pinv_base3;
    const double q = rint(quo);
    const double d = quo - q;  // ~ X / P
    sg = d < 0.0 ? -1.0 : 1.0;
#pragma unroll
    for (int t = 0; t < NP; ++t) x[t] = sg * fma(-q, P[t], S[t]);
    normalize4<BITS, NP>(x);
    if (fabs(d) > 0.5 - 0x1p-30) {  // near +-P/2: settle the wrap exactly
#pragma unroll
        for (int t = 0; t < NP; ++t) x[t] *= sg;
        crt_range_fix<BITS, NP>(x, P, H);
        sg = sign4<NP>(x) < 0 ? -1.0 : 1.0;
#pragma unroll
        for (int t = 0; t < NP; ++t) x[t] *= sg;
        normalize4<BITS, NP>(x);
    }
    if (x[NP - 1] < 0.0) {  // sign predicted wrongly (|X| tiny)
#pragma unroll
        for (int t = 0; t < NP; ++t) x[t] = -x[t];
        normalize4<BITS, NP>(x);
        sg = -sg;
    }
    if constexpr (ZERO_POS) {
        if (sign4<NP>(x) == 0) sg = 1.0;
    }
}

// Integer value of a double holding an integer in [0, 2^52): adding 2^52
// puts it in the significand field.
__device__ __forceinline__ uint64_t small_int_bits(double x) {
    return (uint64_t)__double_as_longlong(x + 0x1p52) & ((1ull << 52) - 1);
}

// |X| * 2^-scale_down for a normalized non-negative 40-bit piece vector
// (x[0..2] in [0, 2^40), x[3] in [0, 2^36)), from the exact 160-bit integer:
// rounded to nearest-even (ODD = false), or to 53 bits with the bits below
// OR-ed into the last place (round to odd, ODD = true), which a later rounding
// to binary32 turns into the single rounding of the whole integer.
template <bool ODD>
__device__ __forceinline__ double limbs_to_double(const double x[4], int scale_down) {
    const uint64_t L0 = small_int_bits(x[0]), L1 = small_int_bits(x[1]), L2 = small_int_bits(x[2]),
                   L3 = small_int_bits(x[3]);
    const uint64_t w0 = L0 | (L1 << 40);
    const uint64_t w1 = (L1 >> 24) | (L2 << 16) | (L3 << 56);
    const uint64_t w2 = L3 >> 8;
    // value = hi * 2^scale + rest, hi normalized to bit 63, sticky = (rest != 0)
    uint64_t top, nxt, low;
    int scale;
    if (w2) {
        top = w2; nxt = w1; low = w0; scale = 128;
    } else if (w1) {
        top = w1; nxt = w0; low = 0; scale = 64;
    } else {
        top = w0; nxt = 0; low = 0; scale = 0;
    }
    if (top == 0) return 0.0;
    const int lz = __clzll(top);
    const uint64_t hi = lz ? (top << lz) | (nxt >> (64 - lz)) : top;
    const bool sticky = ((lz ? (nxt << lz) : nxt) | low) != 0;
    uint64_t mant = hi >> 11;
    const uint64_t rb = hi & 0x7ff;
    if (ODD)
        mant |= (rb != 0 || sticky) ? 1 : 0;
    else
        mant += (rb > 0x400 || (rb == 0x400 && (sticky || (mant & 1)))) ? 1 : 0;
    return ldexp((double)mant, scale - lz + 11 - scale_down);
}

// The same for a normalized non-negative vector of NP (2..5) 32-bit pieces
// (x[t] in [0, 2^32)): the top 64 bits of the integer with the bits below
// OR-ed into the last place (round to odd) convert to double with a single
// rounding, which then equals the rounding of the whole integer (64 >= 53 + 2
// bits); with ODD the 64 bits are rounded to odd at 53 bits instead.
template <bool ODD, int NP = 4>
__device__ __forceinline__ double limbs32_to_double(const double x[NP], int scale_down) {
    const uint64_t w0 = ((uint64_t)(uint32_t)x[1] << 32) | (uint32_t)x[0];
    const uint64_t w1 = NP < 3 ? 0 : ((NP > 3 ? (uint64_t)(uint32_t)x[NP > 3 ? 3 : 0] << 32 : 0) |
                                      (uint32_t)x[NP > 2 ? 2 : 0]);
    const uint64_t w2 = NP > 4 ? (uint64_t)(uint32_t)x[NP > 4 ? 4 : 0] : 0;
    uint64_t top;
    int scale;
    bool odd;
    if (w2 != 0) {
        const int lz = __clzll(w2);
        top = (w2 << lz) | ((w1 >> 1) >> (63 - lz));
        odd = ((w1 << lz) | w0) != 0;
        scale = 128 - lz;
    } else if (w1 != 0) {
        const int lz = __clzll(w1);
        top = (w1 << lz) | ((w0 >> 1) >> (63 - lz));
        odd = (w0 << lz) != 0;
        scale = 64 - lz;
    } else {
        if (!ODD) return ldexp((double)w0, -scale_down);
        if (w0 == 0) return 0.0;
        const int lz = __clzll(w0);
        top = w0 << lz;
        odd = false;
        scale = -lz;
    }
    if (!ODD) return ldexp((double)(top | (odd ? 1 : 0)), scale - scale_down);
    const uint64_t mant = (top >> 11) | (((top & 0x7ff) != 0 || odd) ? 1 : 0);
    return ldexp((double)mant, scale + 11 - scale_down);
}

// C value of type OutT: RN(X) * 2^-(e + f) for double, the single binary32
// rounding of X * 2^-(e + f) for float (round to odd at 53 bits, an exact
// power-of-two scaling, then one rounding to binary32); NaN for a non-finite
// row or column.
template <class OutT>
__device__ __forceinline__ OutT crt_finish(const double S[4], int ei, int fj, const CrtConsts &cc) {
    // S / 2^120 (|S/P| < 2^12)
    const double s120 = fma(S[0], 0x1p-120, fma(S[1], 0x1p-80, fma(S[2], 0x1p-40, S[3])));
    double x[4], sg;
    crt_lift<40>(S, x, sg, s120, cc.P, cc.H, cc.pinv120);
    const double mag = limbs_to_double<sizeof(OutT) == 4>(x, ei + fj);
    return (ei == kExpNonfinite || fj == kExpNonfinite) ? (OutT)__builtin_nan("") : (OutT)(sg * mag);
}

// As crt_finish for S in NP (2..5) 32-bit pieces, enough for the digit sums
// and for P (P < 2^(32 NP)). The quotient estimate uses S / 2^(32 (NP - 1))
// and RN(2^(32 (NP - 1)) / P).
template <class OutT, int NP = 4, bool ZERO_POS = false>
__device__ __forceinline__ OutT crt_finish32(const double S[NP], int ei, int fj, const CrtConsts &cc) {
    double top = S[NP - 1];
    double sc = 1.0;
#pragma unroll
    for (int t = NP - 2; t >= 0; --t) {
        sc *= 0x1p-32;
        top = fma(S[t], sc, top);
    }
    const double pinv = NP == 5 ? cc.pinv128 : NP == 4 ? cc.pinv96 : NP == 3 ? cc.pinv64 : cc.pinv32;
    double x[NP], sg;
    crt_lift<32, NP, ZERO_POS>(S, x, sg, top, cc.P32, cc.H32, pinv);
    const double mag = limbs32_to_double<sizeof(OutT) == 4, NP>(x, ei + fj);
    return (ei == kExpNonfinite || fj == kExpNonfinite) ? (OutT)__builtin_nan("") : (OutT)(sg * mag);
}

// One thread per 4 consecutive rows of one column. The loop over the moduli is
// kept rolled (one plane load per trip): on MI355X this overlaps the plane
// traffic with the arithmetic better than hoisting all loads.
constexpr int kCrtRows = 4;
template <class OutT>
__global__ __launch_bounds__(256) void k_crt(const int8_t *__restrict__ planes, int64_t plane_elems,
                                             int64_t m_pad, int64_t m, int64_t n, const int32_t *__restrict__ e,
                                             const int32_t *__restrict__ f, CrtConsts cc, OutT *__restrict__ C,
                                             int64_t ldc) {
    const int64_t i0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * kCrtRows;
    if (i0 >= m) return;
    for (int64_t j = blockIdx.y; j < n; j += gridDim.y) {
        const int8_t *src = planes + j * m_pad + i0;
        double S[kCrtRows][4];
#pragma unroll
        for (int u = 0; u < kCrtRows; ++u)
#pragma unroll
            for (int t = 0; t < 4; ++t) S[u][t] = 0.0;
#pragma unroll 1
        for (int l = 0; l < cc.n; ++l) {
            const int32_t w = *(const int32_t *)(src + (int64_t)l * plane_elems);
            const double w0 = cc.w[l][0], w1 = cc.w[l][1], w2 = cc.w[l][2], w3 = cc.w[l][3];
#pragma unroll
            for (int u = 0; u < kCrtRows; ++u) {
                const double c = (double)((w << (24 - 8 * u)) >> 24);  // signed byte u
                S[u][0] = fma(c, w0, S[u][0]);
                S[u][1] = fma(c, w1, S[u][1]);
                S[u][2] = fma(c, w2, S[u][2]);
                S[u][3] = fma(c, w3, S[u][3]);
            }
        }
        const int fj = f[j];
        OutT out[kCrtRows];
#pragma unroll
        for (int u = 0; u < kCrtRows; ++u) {
            const int64_t i = i0 + u;
            out[u] = i < m ? crt_finish<OutT>(S[u], e[i], fj, cc) : (OutT)0;
        }
        store_run_nt(C + i0 + j * ldc, out, m - i0);
    }
}

// The weighted sum S = sum_l c_l W_l on the matrix cores (up to 16 moduli).
// Each weight is written in signed base-256 digits, W_l = sum_v d_lv 256^v
// with |d_lv| <= 128 (16 digits suffice below 2^127), so the digit sums
// D_v = sum_l c_l d_lv are products of int8 matrices, exact in int32
// (|D_v| <= 16 * 128 * 128 = 2^18). One v_mfma_i32_32x32x32_i8 forms them for
// 64 entries at once: lane L supplies the 16 residues of its own entry as the
// B operand (column L % 32, k-half L / 32), and the A operand holds the digits
// only in the rows whose half of the accumulator layout ((row / 4) odd or
// even) matches that k-half, so lane L gets back exactly the 16 digit sums of
// its own entry, digit v in register v. S is then assembled from the D_v into
// NP exact 32-bit pieces (|piece| < 2^42.1) for crt_finish32; NP = 2 or 3
// when the weights and P are short (few moduli), which shortens the lift.
// The row exponents are loaded once, ahead of the column loop. The occupancy
// hint of 7 gives the scalar registers that needs without a vector spill, and
// the 64 VGPRs still allow 8 waves per SIMD.
template <class OutT, int NP = 4>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(7))) void k_crt_mma(
    const int8_t *__restrict__ planes, int64_t plane_elems, int64_t m_pad, int64_t m, int64_t n,
    const int32_t *__restrict__ e, const int32_t *__restrict__ f, CrtConsts cc, OutT *__restrict__ C, int64_t ldc) {
    __shared__ __attribute__((aligned(16))) int8_t digit[16][16];
    if (threadIdx.x < 64) {
        const int v = threadIdx.x >> 2, b4 = (threadIdx.x & 3) * 4;
        *(uint32_t *)&digit[v][b4] = *(const uint32_t *)&cc.digit[v][b4];
    }
    __syncthreads();
    const int lane = threadIdx.x & 63, r = lane & 31;
    const bool mine = ((r >> 2) & 1) == (lane >> 5);
    const v4i aop = mine ? *(const v4i *)&digit[4 * (r >> 3) + (r & 3)][0] : (v4i){0, 0, 0, 0};

    // four consecutive rows per lane; a wavefront covers 256 rows, which lie
    // either all inside or all outside the padded plane (m_pad % 256 == 0), so
    // the MFMAs always run on full wavefronts
    const int64_t i0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (((int64_t)blockIdx.x * 256 + (threadIdx.x & ~63)) * 4 >= m_pad) return;
    int ei[4];  // the row exponents, the same for every column
#pragma unroll
    for (int u = 0; u < 4; ++u) ei[u] = i0 + u < m ? e[i0 + u] : 0;
    for (int64_t j = blockIdx.y; j < n; j += gridDim.y) {
        const int8_t *src = planes + j * m_pad + i0;
        uint32_t w[16];
#pragma unroll
        for (int l = 0; l < 16; ++l) w[l] = l < cc.n ? *(const uint32_t *)(src + (int64_t)l * plane_elems) : 0u;
        // 4 x 4 byte transposes: R[u] = residues of row i0 + u, moduli 0..15
        v4i R[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const uint32_t a0 = w[4 * g], a1 = w[4 * g + 1], a2 = w[4 * g + 2], a3 = w[4 * g + 3];
            const uint32_t t01l = __builtin_amdgcn_perm(a1, a0, 0x05010400u);  // a0.0 a1.0 a0.1 a1.1
            const uint32_t t01h = __builtin_amdgcn_perm(a1, a0, 0x07030602u);  // a0.2 a1.2 a0.3 a1.3
            const uint32_t t23l = __builtin_amdgcn_perm(a3, a2, 0x05010400u);
            const uint32_t t23h = __builtin_amdgcn_perm(a3, a2, 0x07030602u);
            R[0][g] = (int)__builtin_amdgcn_perm(t23l, t01l, 0x05040100u);
            R[1][g] = (int)__builtin_amdgcn_perm(t23l, t01l, 0x07060302u);
            R[2][g] = (int)__builtin_amdgcn_perm(t23h, t01h, 0x05040100u);
            R[3][g] = (int)__builtin_amdgcn_perm(t23h, t01h, 0x07060302u);
        }
        const int fj = f[j];
        OutT out[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const v16i D = __builtin_amdgcn_mfma_i32_32x32x32_i8(aop, R[u], (v16i){0}, 0, 0, 0);
            // 32-bit pieces S_t = D_4t + D_4t+1 2^8 + D_4t+2 2^16 + D_4t+3 2^24:
            // digit pairs in int32 (|.| < 2^26.1), then one exact fma
            double S[NP];
#pragma unroll
            for (int t = 0; t < NP; ++t) {
                const int lo = D[4 * t] + D[4 * t + 1] * 256, hi = D[4 * t + 2] + D[4 * t + 3] * 256;
                S[t] = fma((double)hi, 65536.0, (double)lo);
            }
            const int64_t i = i0 + u;
            out[u] = i < m ? crt_finish32<OutT, NP>(S, ei[u], fj, cc) : (OutT)0;
        }
        store_run_nt(C + i0 + j * ldc, out, m - i0);
    }
}

// 17..20 moduli on the matrix cores: the weights have up to 20 signed
// base-256 digits and P < 2^160 (five 32-bit pieces). The layout is
// k_crt_mma's, extended by a second B operand per entry holding moduli 16..19
// in its first four bytes (zeros after) and a second digit block whose rows
// hold digit 16 + v in register v (v < 4): per group of 64 entries, four
// MFMAs accumulate D0 (digits 0..15) and D1 (digits 16..19) over all the
// moduli. |D_v| <= 20 * 128 * 128 < 2^18.4, so the five 32-bit pieces stay
// exact (|piece| < 2^42.5) for crt_finish32.
template <class OutT, int NM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void k_crt_mma20(
    const int8_t *__restrict__ planes, int64_t plane_elems, int64_t m_pad, int64_t m, int64_t n,
    const int32_t *__restrict__ e, const int32_t *__restrict__ f, CrtConsts cc, OutT *__restrict__ C, int64_t ldc) {
    constexpr int NP = 5;
    __shared__ __attribute__((aligned(16))) int8_t digit[kMaxDigits][32];
    if (threadIdx.x < kMaxDigits * 8) {
        const int v = threadIdx.x >> 3, b4 = (threadIdx.x & 7) * 4;
        *(uint32_t *)&digit[v][b4] = *(const uint32_t *)&cc.digit[v][b4];
    }
    __syncthreads();
    const int lane = threadIdx.x & 63, r = lane & 31;
    const bool mine = ((r >> 2) & 1) == (lane >> 5);
    const int dv = 4 * (r >> 3) + (r & 3);  // the digit this lane's accumulator row carries
    const v4i zero = {0, 0, 0, 0};
    const v4i a_lo0 = mine ? *(const v4i *)&digit[dv][0] : zero;
    const v4i a_hi0 = mine ? (v4i){*(const int *)&digit[dv][16], 0, 0, 0} : zero;
    const v4i a_lo1 = mine && dv < 4 ? *(const v4i *)&digit[16 + (dv & 3)][0] : zero;
    const v4i a_hi1 = mine && dv < 4 ? (v4i){*(const int *)&digit[16 + (dv & 3)][16], 0, 0, 0} : zero;

    const int64_t i0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (((int64_t)blockIdx.x * 256 + (threadIdx.x & ~63)) * 4 >= m_pad) return;
    int ei[4];  // the row exponents, the same for every column
#pragma unroll
    for (int u = 0; u < 4; ++u) ei[u] = i0 + u < m ? e[i0 + u] : 0;
    for (int64_t j = blockIdx.y; j < n; j += gridDim.y) {
        const int8_t *src = planes + j * m_pad + i0;
        uint32_t w[20];
#pragma unroll
        for (int l = 0; l < 20; ++l) w[l] = l < NM ? *(const uint32_t *)(src + (int64_t)l * plane_elems) : 0u;
        // 4 x 4 byte transposes: R[u] = residues of row i0 + u, moduli 0..15;
        // H[u] = moduli 16..19
        v4i R[4];
        uint32_t H[4];
#pragma unroll
        for (int g = 0; g < 5; ++g) {
            const uint32_t a0 = w[4 * g], a1 = w[4 * g + 1], a2 = w[4 * g + 2], a3 = w[4 * g + 3];
            const uint32_t t01l = __builtin_amdgcn_perm(a1, a0, 0x05010400u);  // a0.0 a1.0 a0.1 a1.1
            const uint32_t t01h = __builtin_amdgcn_perm(a1, a0, 0x07030602u);  // a0.2 a1.2 a0.3 a1.3
            const uint32_t t23l = __builtin_amdgcn_perm(a3, a2, 0x05010400u);
            const uint32_t t23h = __builtin_amdgcn_perm(a3, a2, 0x07030602u);
            const uint32_t q0 = __builtin_amdgcn_perm(t23l, t01l, 0x05040100u);
            const uint32_t q1 = __builtin_amdgcn_perm(t23l, t01l, 0x07060302u);
            const uint32_t q2 = __builtin_amdgcn_perm(t23h, t01h, 0x05040100u);
            const uint32_t q3 = __builtin_amdgcn_perm(t23h, t01h, 0x07060302u);
            if (g < 4) {
                R[0][g] = (int)q0;
                R[1][g] = (int)q1;
                R[2][g] = (int)q2;
                R[3][g] = (int)q3;
            } else {
                H[0] = q0;
                H[1] = q1;
                H[2] = q2;
                H[3] = q3;
            }
        }
        const int fj = f[j];
        OutT out[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const v4i Bh = {(int)H[u], 0, 0, 0};
            v16i D0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a_lo0, R[u], (v16i){0}, 0, 0, 0);
            D0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a_hi0, Bh, D0, 0, 0, 0);
            v16i D1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a_lo1, R[u], (v16i){0}, 0, 0, 0);
            D1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a_hi1, Bh, D1, 0, 0, 0);
            double S[NP];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int lo = D0[4 * t] + D0[4 * t + 1] * 256, hi = D0[4 * t + 2] + D0[4 * t + 3] * 256;
                S[t] = fma((double)hi, 65536.0, (double)lo);
            }
            {
                const int lo = D1[0] + D1[1] * 256, hi = D1[2] + D1[3] * 256;
                S[4] = fma((double)hi, 65536.0, (double)lo);
            }
            const int64_t i = i0 + u;
            out[u] = i < m ? crt_finish32<OutT, NP>(S, ei[u], fj, cc) : (OutT)0;
        }
        store_run_nt(C + i0 + j * ldc, out, m - i0);
    }
}

// Complex products: per modulus the planes 3l, 3l+1, 3l+2 hold T1 = re*re,
// T2 = im*im and T3 = (re+im)*(re+im) mod p; the real part is T1 - T2 and the
// imaginary part T3 - T1 - T2 (Gauss' trick, exact in residues). Each is
// brought back to the symmetric range and both sums are accumulated in the
// 40-bit pieces of k_crt (|c| <= 128 keeps every bound of that kernel), then
// lifted and rounded like a real entry. C holds interleaved (re, im) pairs.
template <class OutT>
__global__ __launch_bounds__(256) void k_crt_c(const int8_t *__restrict__ planes, int64_t plane_elems,
                                               int64_t m_pad, int64_t m, int64_t n, const int32_t *__restrict__ e,
                                               const int32_t *__restrict__ f, CrtConsts cc, ModConsts mc,
                                               OutT *__restrict__ C, int64_t ldc) {
    const int64_t i0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * kCrtRows;
    if (i0 >= m) return;
    for (int64_t j = blockIdx.y; j < n; j += gridDim.y) {
        const int8_t *src = planes + j * m_pad + i0;
        double Sr[kCrtRows][4], Si[kCrtRows][4];
#pragma unroll
        for (int u = 0; u < kCrtRows; ++u)
#pragma unroll
            for (int t = 0; t < 4; ++t) Sr[u][t] = Si[u][t] = 0.0;
#pragma unroll 1
        for (int l = 0; l < cc.n; ++l) {
            const int32_t w1 = *(const int32_t *)(src + (int64_t)(3 * l) * plane_elems);
            const int32_t w2 = *(const int32_t *)(src + (int64_t)(3 * l + 1) * plane_elems);
            const int32_t w3 = *(const int32_t *)(src + (int64_t)(3 * l + 2) * plane_elems);
            const double p = mc.p[l], pinv = mc.pinv[l];
            const double W0 = cc.w[l][0], W1 = cc.w[l][1], W2 = cc.w[l][2], W3 = cc.w[l][3];
#pragma unroll
            for (int u = 0; u < kCrtRows; ++u) {
                const int t1 = (w1 << (24 - 8 * u)) >> 24, t2 = (w2 << (24 - 8 * u)) >> 24,
                          t3 = (w3 << (24 - 8 * u)) >> 24;
                const double yr = (double)(t1 - t2), yi = (double)(t3 - t1 - t2);
                const double cr = fma(-p, rint(yr * pinv), yr), ci = fma(-p, rint(yi * pinv), yi);
                Sr[u][0] = fma(cr, W0, Sr[u][0]);
                Sr[u][1] = fma(cr, W1, Sr[u][1]);
                Sr[u][2] = fma(cr, W2, Sr[u][2]);
                Sr[u][3] = fma(cr, W3, Sr[u][3]);
                Si[u][0] = fma(ci, W0, Si[u][0]);
                Si[u][1] = fma(ci, W1, Si[u][1]);
                Si[u][2] = fma(ci, W2, Si[u][2]);
                Si[u][3] = fma(ci, W3, Si[u][3]);
            }
        }
        const int fj = f[j];
        OutT out[2 * kCrtRows];  // interleaved (re, im) of rows i0 .. i0 + 3
#pragma unroll
        for (int u = 0; u < kCrtRows; ++u) {
            const int64_t i = i0 + u;
            const int ei = i < m ? e[i] : 0;
            out[2 * u] = i < m ? crt_finish<OutT>(Sr[u], ei, fj, cc) : (OutT)0;
            out[2 * u + 1] = i < m ? crt_finish<OutT>(Si[u], ei, fj, cc) : (OutT)0;
        }
        store_run_nt(C + 2 * (i0 + j * ldc), out, 2 * (m - i0));
    }
}

// Complex products on the matrix cores (up to 16 moduli). By Gauss' trick the
// real part's weighted sum is sum_l (T1_l - T2_l) W_l and the imaginary part's
// sum_l (T3_l - T1_l - T2_l) W_l. Both only matter mod P, so a negative weight
// -W_l can be replaced by P - W_l, and the residues enter unreduced. The digit
// sums are then int8 products, like those of k_crt_mma: two MFMAs for the real
// part (T1 against the digits of W, T2 against those of P - W) and three for
// the imaginary part (T3 against W, T1 and T2 against P - W), accumulated in
// one 32 x 32 x 32 block each. |D_v| <= 3 * 16 * 128 * 128 < 2^19.6, so the
// 32-bit pieces stay exact (|piece| < 2^43.6) and |S| <= 2^12 P; the lift
// and rounding are those of a real entry, except that S can now be a nonzero
// multiple of P, whose X = 0 must still come out as +0.
template <class OutT, int NP = 4>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void k_crt_c_mma(
    const int8_t *__restrict__ planes, int64_t plane_elems, int64_t m_pad, int64_t m, int64_t n,
    const int32_t *__restrict__ e, const int32_t *__restrict__ f, CrtConsts cc, OutT *__restrict__ C, int64_t ldc) {
    __shared__ __attribute__((aligned(16))) int8_t digit[2][16][16];
    if (threadIdx.x < 128) {
        const int s = threadIdx.x >> 6, v = (threadIdx.x >> 2) & 15, b4 = (threadIdx.x & 3) * 4;
        *(uint32_t *)&digit[s][v][b4] = s ? *(const uint32_t *)&cc.ndigit[v][b4] : *(const uint32_t *)&cc.digit[v][b4];
    }
    __syncthreads();
    const int lane = threadIdx.x & 63, r = lane & 31;
    const bool mine = ((r >> 2) & 1) == (lane >> 5);
    const int dv = 4 * (r >> 3) + (r & 3);
    const v4i aop = mine ? *(const v4i *)&digit[0][dv][0] : (v4i){0, 0, 0, 0};   // digits of W
    const v4i aopn = mine ? *(const v4i *)&digit[1][dv][0] : (v4i){0, 0, 0, 0};  // digits of P - W

    // four consecutive rows per lane, full wavefronts as in k_crt_mma
    const int64_t i0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (((int64_t)blockIdx.x * 256 + (threadIdx.x & ~63)) * 4 >= m_pad) return;
    int ei[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) ei[u] = i0 + u < m ? e[i0 + u] : 0;
    for (int64_t j = blockIdx.y; j < n; j += gridDim.y) {
        const int8_t *src = planes + j * m_pad + i0;
        uint32_t w[3][16];  // w[c][l]: rows i0 .. i0 + 3 of plane 3 l + c
#pragma unroll
        for (int l = 0; l < 16; ++l)
#pragma unroll
            for (int c = 0; c < 3; ++c)
                w[c][l] = l < cc.n ? *(const uint32_t *)(src + (int64_t)(3 * l + c) * plane_elems) : 0u;
        const int fj = f[j];
        OutT out[8];  // interleaved (re, im) of rows i0 .. i0 + 3
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            // B operands of row i0 + u: byte u of the words of each plane group
            v4i R[3];
#pragma unroll
            for (int c = 0; c < 3; ++c)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const uint32_t s01 = __builtin_amdgcn_perm(w[c][4 * g + 1], w[c][4 * g], 0x0c0c0400u + u * 0x0101u);
                    const uint32_t s23 = __builtin_amdgcn_perm(w[c][4 * g + 3], w[c][4 * g + 2], 0x0c0c0400u + u * 0x0101u);
                    R[c][g] = (int)__builtin_amdgcn_perm(s23, s01, 0x05040100u);
                }
            const int64_t i = i0 + u;
#pragma unroll
            for (int part = 0; part < 2; ++part) {
                v16i D;
                if (part == 0) {
                    D = __builtin_amdgcn_mfma_i32_32x32x32_i8(aop, R[0], (v16i){0}, 0, 0, 0);
                    D = __builtin_amdgcn_mfma_i32_32x32x32_i8(aopn, R[1], D, 0, 0, 0);
                } else {
                    D = __builtin_amdgcn_mfma_i32_32x32x32_i8(aop, R[2], (v16i){0}, 0, 0, 0);
                    D = __builtin_amdgcn_mfma_i32_32x32x32_i8(aopn, R[0], D, 0, 0, 0);
                    D = __builtin_amdgcn_mfma_i32_32x32x32_i8(aopn, R[1], D, 0, 0, 0);
                }
                double S[NP];
#pragma unroll
                for (int t = 0; t < NP; ++t) {
                    const int lo = D[4 * t] + D[4 * t + 1] * 256, hi = D[4 * t + 2] + D[4 * t + 3] * 256;
                    S[t] = fma((double)hi, 65536.0, (double)lo);
                }
                out[2 * u + part] = i < m ? crt_finish32<OutT, NP, true>(S, ei[u], fj, cc) : (OutT)0;
            }
        }
        store_run_nt(C + 2 * (i0 + j * ldc), out, 2 * (m - i0));
    }
}

// 17..20 moduli: k_crt_c_mma's digit sums in k_crt_mma20's layout. Each plane
// group gives two B operands (moduli 0..15, and 16..19 in the first four bytes
// of a second). W and P - W have two digit blocks each: digits 0..15, and
// digits 16..19 in registers 0..3 of a second result. One term (a plane group
// against a weight table) is four MFMAs into the part's two blocks: 8 for Re,
// 12 for Im, per 64 entries. |D_v| <= 3 * 20 * 128 * 128 < 2^20, the five
// 32-bit pieces stay below 2^44, and |S| <= 2^12.6 P.
template <class OutT, int NM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_crt_c_mma20(
    const int8_t *__restrict__ planes, int64_t plane_elems, int64_t m_pad, int64_t m, int64_t n,
    const int32_t *__restrict__ e, const int32_t *__restrict__ f, CrtConsts cc, OutT *__restrict__ C, int64_t ldc) {
    constexpr int NP = 5;
    __shared__ __attribute__((aligned(16))) int8_t digit[2][kMaxDigits][32];
    for (int t = threadIdx.x; t < 2 * kMaxDigits * 8; t += blockDim.x) {
        const int sgn = t / (kMaxDigits * 8), v = (t / 8) % kMaxDigits, b4 = (t & 7) * 4;
        *(uint32_t *)&digit[sgn][v][b4] =
            sgn ? *(const uint32_t *)&cc.ndigit[v][b4] : *(const uint32_t *)&cc.digit[v][b4];
    }
    __syncthreads();
    const int lane = threadIdx.x & 63, r = lane & 31;
    const bool mine = ((r >> 2) & 1) == (lane >> 5);
    const int dv = 4 * (r >> 3) + (r & 3);  // the digit this lane's accumulator row carries
    const v4i zero = {0, 0, 0, 0};
    // [0]: digits of W, [1]: digits of P - W
    v4i a_lo0[2], a_hi0[2], a_lo1[2], a_hi1[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        a_lo0[t] = mine ? *(const v4i *)&digit[t][dv][0] : zero;
        a_hi0[t] = mine ? (v4i){*(const int *)&digit[t][dv][16], 0, 0, 0} : zero;
        a_lo1[t] = mine && dv < 4 ? *(const v4i *)&digit[t][16 + (dv & 3)][0] : zero;
        a_hi1[t] = mine && dv < 4 ? (v4i){*(const int *)&digit[t][16 + (dv & 3)][16], 0, 0, 0} : zero;
    }

    const int64_t i0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (((int64_t)blockIdx.x * 256 + (threadIdx.x & ~63)) * 4 >= m_pad) return;
    int ei[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) ei[u] = i0 + u < m ? e[i0 + u] : 0;
    for (int64_t j = blockIdx.y; j < n; j += gridDim.y) {
        const int8_t *src = planes + j * m_pad + i0;
        uint32_t w[3][20];  // w[c][l]: rows i0 .. i0 + 3 of plane 3 l + c
#pragma unroll
        for (int l = 0; l < 20; ++l)
#pragma unroll
            for (int c = 0; c < 3; ++c)
                w[c][l] = l < NM ? *(const uint32_t *)(src + (int64_t)(3 * l + c) * plane_elems) : 0u;
        const int fj = f[j];
        OutT out[8];  // interleaved (re, im) of rows i0 .. i0 + 3
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            // B operands of row i0 + u: byte u of the words of each plane group
            v4i R[3];
            v4i Bh[3];
#pragma unroll
            for (int c = 0; c < 3; ++c) {
#pragma unroll
                for (int g = 0; g < 5; ++g) {
                    const uint32_t s01 = __builtin_amdgcn_perm(w[c][4 * g + 1], w[c][4 * g], 0x0c0c0400u + u * 0x0101u);
                    const uint32_t s23 = __builtin_amdgcn_perm(w[c][4 * g + 3], w[c][4 * g + 2], 0x0c0c0400u + u * 0x0101u);
                    const int q = (int)__builtin_amdgcn_perm(s23, s01, 0x05040100u);
                    if (g < 4)
                        R[c][g] = q;
                    else
                        Bh[c] = (v4i){q, 0, 0, 0};
                }
            }
            const int64_t i = i0 + u;
#pragma unroll
            for (int part = 0; part < 2; ++part) {
                // (plane group, weight table) terms of this part
                constexpr int kRe[2][2] = {{0, 0}, {1, 1}};
                constexpr int kIm[3][2] = {{2, 0}, {0, 1}, {1, 1}};
                v16i D0 = (v16i){0}, D1 = (v16i){0};
#pragma unroll
                for (int t = 0; t < (part == 0 ? 2 : 3); ++t) {
                    const int c = part == 0 ? kRe[t][0] : kIm[t][0], wt = part == 0 ? kRe[t][1] : kIm[t][1];
                    D0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a_lo0[wt], R[c], D0, 0, 0, 0);
                    D0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a_hi0[wt], Bh[c], D0, 0, 0, 0);
                    D1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a_lo1[wt], R[c], D1, 0, 0, 0);
                    D1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a_hi1[wt], Bh[c], D1, 0, 0, 0);
                }
                double S[NP];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int lo = D0[4 * t] + D0[4 * t + 1] * 256, hi = D0[4 * t + 2] + D0[4 * t + 3] * 256;
                    S[t] = fma((double)hi, 65536.0, (double)lo);
                }
                {
                    const int lo = D1[0] + D1[1] * 256, hi = D1[2] + D1[3] * 256;
                    S[4] = fma((double)hi, 65536.0, (double)lo);
                }
                out[2 * u + part] = i < m ? crt_finish32<OutT, NP, true>(S, ei[u], fj, cc) : (OutT)0;
            }
        }
        store_run_nt(C + 2 * (i0 + j * ldc), out, 2 * (m - i0));
    }
}

// CRT-range check against one redundant modulus (debug entry points): the
// integer X the reconstruction returns from the first ck.n residues must agree
// with the residue product of the check modulus pc ([Q] section
// 時計の針で見る定理の中身: outside (-P/2, P/2] the clocks show another number;
// [G] Problemstellung: too large a scaling breaks the reconstruction). X =
// S - q P with q = round(S / P) and S / P = sum_l c_l K_l / p_l, whose FP64 sum
// is good to ~2^-44, so q is the reconstruction's own quotient unless |X| lies
// within 2^-30 P of P / 2 (flag 2). X mod pc follows exactly in int32 from
// W_l mod pc and P mod pc. A wrapped X = Y - j P (0 < |j| < pc) always
// disagrees, since pc does not divide j P.
__global__ __launch_bounds__(256) void k_crt_check(const int8_t *__restrict__ planes, int64_t plane_elems,
                                                   int64_t m_pad, int64_t m, int64_t n, CheckConsts ck,
                                                   uint8_t *__restrict__ flags) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= m) return;
    for (int64_t j = blockIdx.y; j < n; j += gridDim.y) {
        const int8_t *src = planes + j * m_pad + i;
        double sp = 0.0;
        int xm = 0;
        for (int l = 0; l < ck.n; ++l) {
            const int c = src[(int64_t)l * plane_elems];
            sp = fma((double)c, ck.kp[l], sp);
            xm += c * ck.wm[l];
        }
        const double q = rint(sp);
        const int cc = src[(int64_t)ck.n * plane_elems];
        int r = (xm - (int)q * ck.pm - cc) % ck.pc;
        uint8_t flag = r == 0 ? 0 : 1;
        if (fabs(sp - q) > 0.5 - 0x1p-30) flag = 2;
        flags[j * m + i] = flag;
    }
}

// ---------------------------------------------------------------------------
// Steps 3 + 4 + 5 fused: all moduli of one output tile in one block
// ---------------------------------------------------------------------------
// The per-modulus products are independent and carry nothing from one clock
// to another ([Q] section 誤差のないINT8行列積(手順3)), so one block may run them
// back to back for its tile: after the inner dimension of modulus l it reduces
// the int32 products mod p_l in registers and adds c_l W_l into the tile's
// exact 40-bit pieces S (as k_crt does from the planes); after the last
// modulus it lifts, unscales and writes C ([Q] sections 高い精度での復元(手順4)
// and 2の累乗による整数化(手順1と5)). No residue plane leaves the chip and the
// reconstruction needs no launch of its own. The price is a small tile: the N
// residues or the pieces S of a 256 x 256 tile fit neither the registers nor
// LDS, while a 64 x 64 tile keeps S in 128 VGPRs per lane; so each MFMA needs
// 1 KiB of LDS fragments (0.375 KiB in the 256 x 256 GEMM), the L2 serves four
// times the operand bytes per operation, and the block count no longer grows
// with the number of moduli.
//
// Block: 4 waves (2 x 2) of 32 x 32 (2 x 2 MFMA tiles of 16 x 16 x 64); LDS
// ring of kFNST stages of 8 KiB (4 A and 4 B fragment blocks of 64 k), one
// continuous sequence of stages over (modulus, k) so the copies of the next
// modulus start during the last stages of the current one. Each wave copies 2
// fragment blocks per stage (waves 0, 1: A; waves 2, 3: B).
constexpr int kFTile = 64;
constexpr int kFNST = 4;
constexpr int kFStage = 8 * 1024;

template <class OutT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_gemm_crt(
    const int8_t *__restrict__ RA, const int8_t *__restrict__ RB, int64_t planeA, int64_t planeB, int nk,
    int tiles_m, const int32_t *__restrict__ e, const int32_t *__restrict__ f, CrtConsts cc, ModConsts mc,
    OutT *__restrict__ C, int64_t m, int64_t n, int64_t ldc) {
    __shared__ __attribute__((aligned(1024))) int8_t lds[kFNST * kFStage];
    const int tm = blockIdx.x % tiles_m, tn = blockIdx.x / tiles_m;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t row_bytes = (int64_t)nk * 1024;  // one 16-row block over all of K
    const bool copies_a = wave < 2;
    const int cq = (wave & 1) * 2;
    const int8_t *base = (copies_a ? RA + ((int64_t)tm * 4 + cq) * row_bytes : RB + ((int64_t)tn * 4 + cq) * row_bytes) +
                         lane * 16;
    const int64_t plane = copies_a ? planeA : planeB;
    const int total = cc.n * nk;  // stages over all moduli (even: nk is even)
    __attribute__((address_space(3))) int8_t *lds3 = (__attribute__((address_space(3))) int8_t *)lds;
    // copies of global stage g = l * nk + ks (clamped past the end: into a slot never read)
    int cl = 0, cks = 0;  // (modulus, k-stage) of the next stage to copy
    auto copy_next = [&](int g) {
        const int8_t *src = base + cl * plane + cks * 1024;
#pragma unroll
        for (int q = 0; q < 2; ++q)
            __builtin_amdgcn_global_load_lds(src + q * row_bytes, lds3 + (g % kFNST) * kFStage + (wave * 2 + q) * 1024,
                                             16, 0, 0);
        if (g + 1 < total) {
            if (++cks == nk) {
                cks = 0;
                ++cl;
            }
        }
    };
    // fragment r of a stage: r < 2 -> A tile r of this wave, else B tile r - 2
    auto frag = [&](const int8_t *stage, int r) {
        return *(const v4i *)(stage + (r < 2 ? 2 * wm + r : 4 + 2 * wn + (r - 2)) * 1024 + lane * 16);
    };

    v4i acc[2][2];
    double S[2][2][4][4];  // [row tile][col tile][register][piece]
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            acc[i][j] = (v4i){0, 0, 0, 0};
#pragma unroll
            for (int v = 0; v < 4; ++v)
#pragma unroll
                for (int t = 0; t < 4; ++t) S[i][j][v][t] = 0.0;
        }

#pragma unroll
    for (int g = 0; g < kFNST - 1; ++g) copy_next(g);
    asm volatile("s_waitcnt vmcnt(2)\n\ts_barrier" ::: "memory");  // stages 0 and 1 landed
    v4i f0[4], f1[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) f0[r] = frag(lds, r);

    int l = 0, ks = 0;  // modulus and k-stage of the stage being multiplied
    // stage g: MFMAs on fc, reads of stage g + 1 into fn, copies of stage g + 3;
    // at the end stage g + 2 has landed and every read of stage g + 1's slot is
    // done before the copies of a later stage refill it
    auto stage = [&](int g, v4i(&fc)[4], v4i(&fn)[4]) {
        const int8_t *nxt = lds + ((g + 1) % kFNST) * kFStage;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            acc[q >> 1][q & 1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fc[q >> 1], fc[2 + (q & 1)], acc[q >> 1][q & 1], 0, 0, 0);
            fn[q] = frag(nxt, q);
        }
        copy_next(g + kFNST - 1);
        asm volatile("s_waitcnt vmcnt(2) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        if (++ks == nk) {
            // modulus l done: its residues, weighted, into the pieces S
            const double p = mc.p[l], pinv = mc.pinv[l];
            const double w0 = cc.w[l][0], w1 = cc.w[l][1], w2 = cc.w[l][2], w3 = cc.w[l][3];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const double c = (double)smod(acc[i][j][v], pinv, (int)p);
                        S[i][j][v][0] = fma(c, w0, S[i][j][v][0]);
                        S[i][j][v][1] = fma(c, w1, S[i][j][v][1]);
                        S[i][j][v][2] = fma(c, w2, S[i][j][v][2]);
                        S[i][j][v][3] = fma(c, w3, S[i][j][v][3]);
                    }
                    acc[i][j] = (v4i){0, 0, 0, 0};
                }
            ks = 0;
            ++l;
        }
    };
    for (int g = 0; g < total; g += 2) {
        stage(g, f0, f1);
        stage(g + 1, f1, f0);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // drain the trailing copies before the block ends

    // accumulator layout of a 16 x 16 tile: lane L, register v holds row
    // 4 (L / 16) + v, column L % 16
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int64_t col = (int64_t)tn * kFTile + wn * 32 + 16 * j + (lane & 15);
        if (col >= n) continue;
        const int fj = f[col];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int64_t row0 = (int64_t)tm * kFTile + wm * 32 + 16 * i + 4 * (lane >> 4);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int64_t row = row0 + v;
                if (row < m) C[row + col * ldc] = crt_finish<OutT>(S[i][j][v], e[row], fj, cc);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Small helpers
// ---------------------------------------------------------------------------
template <class T>
__global__ void k_zero_c(T *C, int64_t m, int64_t n, int64_t ldc) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= m) return;
    for (int64_t j = blockIdx.y; j < n; j += gridDim.y) C[i + j * ldc] = (T)0;
}

// packed [l][rows_pad/32][kb][64][16] -> logical [l][rows][k]
__global__ void k_unpack(const int8_t *packed, int64_t rows, int64_t k, int64_t plane_bytes, int64_t kb,
                         int8_t *out) {
    const int64_t h = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t l = blockIdx.z;
    if (h >= k) return;
    for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
        const int64_t lane = (r & 15) + 16 * ((h & 63) >> 4);
        const int64_t off = (((r >> 4) * (kb / 2) + (h >> 6)) * 64 + lane) * 16 + (h & 15);
        out[(l * rows + r) * k + h] = packed[l * plane_bytes + off];
    }
}

__global__ void k_copy_planes_i32(const int32_t *planes, int64_t m, int64_t m_pad, int64_t plane_elems, int64_t n,
                                  int32_t *out) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t l = blockIdx.z;
    if (i >= m) return;
    for (int64_t j = blockIdx.y; j < n; j += gridDim.y) out[(l * n + j) * m + i] = planes[l * plane_elems + j * m_pad + i];
}

// symmetric residues -> [0, p)
__global__ void k_copy_planes_red(const int8_t *planes, int64_t m, int64_t m_pad, int64_t plane_elems, int64_t n,
                                  ModConsts mc, int group, uint8_t *out) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t l = blockIdx.z;
    if (i >= m) return;
    const int p = (int)mc.p[l / group];
    for (int64_t j = blockIdx.y; j < n; j += gridDim.y) {
        int v = planes[l * plane_elems + j * m_pad + i];
        if (p == 256) v &= 0xff;
        else if (v < 0) v += p;
        out[(l * n + j) * m + i] = (uint8_t)v;
    }
}

// [0, p) -> symmetric residues in the padded plane layout (padding zeroed)
__global__ void k_pack_planes(const uint8_t *res, int64_t m, int64_t n, int64_t m_pad, int64_t plane_elems,
                              ModConsts mc, int group, int8_t *planes) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t l = blockIdx.z;
    if (i >= m_pad) return;
    const int p = (int)mc.p[l / group];
    for (int64_t j = blockIdx.y; j < n; j += gridDim.y) {
        int v = i < m ? res[(l * n + j) * m + i] : 0;
        if (v > (p - 1) / 2) v -= p;
        planes[l * plane_elems + j * m_pad + i] = (int8_t)v;
    }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
static inline unsigned nblk(int64_t count, int per) { return (unsigned)((count + per - 1) / per); }
static inline unsigned ydim(int64_t count) { return (unsigned)(count < 65535 ? (count > 0 ? count : 1) : 65535); }

template <class T, int W, bool ORIG = false>
static hipError_t launch_scale_t(const T *A, int64_t m, int64_t k, int64_t lda, const T *B, int64_t n, int64_t ldb,
                                 double Pp, const Layout &L, char *ws, hipStream_t s, Ev ev) {
    const int64_t rowblocks = (m + 63) / 64;
    const int64_t nA = rowblocks * L.nchunks, nB = L.n_pad / 4;
    auto kern = k_scale<T, W, ORIG>;
    OZ2_LAUNCH(ev, kern, dim3((unsigned)(nA + nB)), dim3(256), 0, s, A, m, k, lda, L.kchunk, rowblocks, nA,
               (double *)(ws + L.part_s), (int *)(ws + L.part_g), (int *)(ws + L.part_bad), B, n, L.n_pad, ldb, Pp,
               (int32_t *)(ws + L.f), (int32_t *)(ws + L.gb));
    return hipGetLastError();
}

hipError_t launch_scale(Elem el, bool cplx, bool original, const void *A, int64_t m, int64_t k, int64_t lda,
                        const void *B, int64_t n, int64_t ldb, double Pp, const Layout &L, char *ws, hipStream_t s,
                        Ev ev) {
    if (el == Elem::f32) {
        const float *a = (const float *)A, *b = (const float *)B;
        if (original) return launch_scale_t<float, 1, true>(a, m, k, lda, b, n, ldb, Pp, L, ws, s, ev);
        return cplx ? launch_scale_t<float, 2>(a, m, k, lda, b, n, ldb, Pp, L, ws, s, ev)
                    : launch_scale_t<float, 1>(a, m, k, lda, b, n, ldb, Pp, L, ws, s, ev);
    }
    const double *a = (const double *)A, *b = (const double *)B;
    if (original) return launch_scale_t<double, 1, true>(a, m, k, lda, b, n, ldb, Pp, L, ws, s, ev);
    return cplx ? launch_scale_t<double, 2>(a, m, k, lda, b, n, ldb, Pp, L, ws, s, ev)
                : launch_scale_t<double, 1>(a, m, k, lda, b, n, ldb, Pp, L, ws, s, ev);
}

hipError_t launch_row_exponents(int64_t m, double Pp, const Layout &L, char *ws, hipStream_t s, Ev ev) {
    const int64_t span = L.m_pad > L.n_pad ? L.m_pad : L.n_pad;
    OZ2_LAUNCH(ev, k_row_exponents, dim3(nblk(span, 256)), dim3(256), 0, s, (const double *)(ws + L.part_s),
               (const int *)(ws + L.part_g), (const int *)(ws + L.part_bad), m, L.m_pad, L.nchunks, Pp,
               (int32_t *)(ws + L.e), (int32_t *)(ws + L.ga), (int32_t *)(ws + L.rowmax),
               (int32_t *)(ws + L.colmax), L.n_pad);
    return hipGetLastError();
}

template <bool FOLD, class T, int W, bool ORIG = false>
static hipError_t launch_split_t(const T *A, int64_t m, int64_t lda, const T *B, int64_t n, int64_t ldb, int64_t k,
                                 double Pp, const SplitConsts &sc, const Layout &L, char *ws, hipStream_t s, Ev ev) {
    const int64_t tilesA = L.m_pad / kSplitRows, tilesB = L.n_pad / kSplitRows;
    const int64_t tilesK = L.k_pad / (W == 2 ? kSplitColsC : kSplitCols);
    const int64_t nA = tilesA * tilesK, nB = tilesB * tilesK;
    auto kern = k_split<FOLD, T, W, ORIG>;
    OZ2_LAUNCH(ev, kern, dim3((unsigned)(nA + nB)), dim3(256), 0, s, A, m, lda, B, n, ldb, k, tilesA, tilesB, nA,
               (const double *)(ws + L.part_s), (const int *)(ws + L.part_g), (const int *)(ws + L.part_bad),
               L.nchunks, Pp, (int32_t *)(ws + L.e), (const int32_t *)(ws + L.f), sc, (int8_t *)(ws + L.ra),
               L.m_pad * L.k_pad, (int8_t *)(ws + L.rb), L.n_pad * L.k_pad, L.kb);
    return hipGetLastError();
}

hipError_t launch_split(Elem el, bool cplx, bool original, const void *A, int64_t m, int64_t lda, const void *B,
                        int64_t n, int64_t ldb, int64_t k, bool fold_row_exponents, double Pp,
                        const SplitConsts &sc, const Layout &L, char *ws, hipStream_t s, Ev ev) {
    if (el == Elem::f32) {
        const float *a = (const float *)A, *b = (const float *)B;
        if (original) return launch_split_t<true, float, 1, true>(a, m, lda, b, n, ldb, k, Pp, sc, L, ws, s, ev);
        if (cplx) return launch_split_t<true, float, 2>(a, m, lda, b, n, ldb, k, Pp, sc, L, ws, s, ev);
        return fold_row_exponents ? launch_split_t<true, float, 1>(a, m, lda, b, n, ldb, k, Pp, sc, L, ws, s, ev)
                                  : launch_split_t<false, float, 1>(a, m, lda, b, n, ldb, k, Pp, sc, L, ws, s, ev);
    }
    const double *a = (const double *)A, *b = (const double *)B;
    if (original) return launch_split_t<true, double, 1, true>(a, m, lda, b, n, ldb, k, Pp, sc, L, ws, s, ev);
    if (cplx) return launch_split_t<true, double, 2>(a, m, lda, b, n, ldb, k, Pp, sc, L, ws, s, ev);
    return fold_row_exponents ? launch_split_t<true, double, 1>(a, m, lda, b, n, ldb, k, Pp, sc, L, ws, s, ev)
                              : launch_split_t<false, double, 1>(a, m, lda, b, n, ldb, k, Pp, sc, L, ws, s, ev);
}

template <class T>
static hipError_t launch_quantize_t(const T *A, int64_t m, int64_t lda, const T *B, int64_t n, int64_t ldb,
                                    int64_t k, const Layout &L, char *ws, hipStream_t s) {
    const int64_t tilesA = L.m_pad / kSplitRows, tilesB = L.n_pad / kSplitRows, tilesK = L.k_pad / kSplitCols;
    const int64_t nA = tilesA * tilesK, nB = tilesB * tilesK;
    hipLaunchKernelGGL(k_quantize<T>, dim3((unsigned)(nA + nB)), dim3(256), 0, s, A, m, lda, B, n, ldb, k, tilesA,
                       tilesB, nA, (const int32_t *)(ws + L.ga), (const int32_t *)(ws + L.gb), (int8_t *)(ws + L.abar),
                       (int8_t *)(ws + L.bbar), L.kb);
    return hipGetLastError();
}

hipError_t launch_quantize(Elem el, const void *A, int64_t m, int64_t lda, const void *B, int64_t n, int64_t ldb,
                           int64_t k, const Layout &L, char *ws, hipStream_t s) {
    if (el == Elem::f32)
        return launch_quantize_t((const float *)A, m, lda, (const float *)B, n, ldb, k, L, ws, s);
    return launch_quantize_t((const double *)A, m, lda, (const double *)B, n, ldb, k, L, ws, s);
}

// Tile shape of a product: 256 x 256 unless that gives at most one block per
// two compute units, then 128 x 128 (four times the blocks; on MI355X it was
// 1.2-1.9x faster up to that point and slower beyond it, where its larger LDS
// traffic per MFMA costs more than the fuller chip gains). OZ2_GEMM_TILE=128
// or 256 in the environment forces a shape; the results do not depend on it
// (the tests run both shapes at every size).
// Compute units of the current device (cached per device).
static int compute_units() {
    static std::atomic<int> cu_count[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    int cus = cu_count[dev].load(std::memory_order_relaxed);
    if (cus <= 0) {
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        cu_count[dev].store(cus, std::memory_order_relaxed);
    }
    return cus;
}

static bool use_small_tiles(const Layout &L, int planes) {
    if (const char *force = getenv("OZ2_GEMM_TILE")) {
        if (strcmp(force, "128") == 0) return true;
        if (strcmp(force, "256") == 0) return false;
    }
    const int64_t blocks = (L.m_pad / ShapeL::TM) * (L.n_pad / ShapeL::TN) * (int64_t)planes;
    return 2 * blocks <= (int64_t)compute_units();
}

// The 256 x 256 tile runs on the persistent kernel when there are more tiles
// than compute units (with at most one tile per block it only adds the
// one-wave kernel's exposed prologue and epilogue) and the launch has at least
// kNST - 1 stages, m_pad < 2^27 (its 32-bit store offsets) and k_pad < 2^25
// (its 32-bit copy offsets, 7 x 16 k_pad). OZ2_GEMM_KERNEL=blocks or
// =persistent forces either kernel (the latter within those limits).
static bool use_persistent(int nks, const Layout &L, int blocks) {
    if (nks < kNST - 1 || L.m_pad >= ((int64_t)1 << 27) || L.k_pad >= ((int64_t)1 << 25)) return false;
    if (const char *force = getenv("OZ2_GEMM_KERNEL")) {
        if (strcmp(force, "blocks") == 0) return false;
        if (strcmp(force, "persistent") == 0) return true;
    }
    return blocks > compute_units();
}

static GemmArgs gemm_args(const int8_t *RA, const int8_t *RB, int nmod, int group, const Layout &L, bool small) {
    GemmArgs g{};
    g.RA = RA;
    g.RB = RB;
    g.planeA = L.m_pad * L.k_pad;
    g.planeB = L.n_pad * L.k_pad;
    g.kb = L.kb;
    g.ks0 = 0;
    g.nks = (int)(L.kb / 2);
    g.accumulate = 0;
    g.tiles_m = (int)(L.m_pad / (small ? ShapeS::TM : ShapeL::TM));
    g.tiles_n = (int)(L.n_pad / (small ? ShapeS::TN : ShapeL::TN));
    g.nmod = nmod * group;
    g.group = group;
    g.m_pad = L.m_pad;
    g.plane_elems = L.m_pad * L.n_pad;
    return g;
}

hipError_t launch_gemm_mod(const int8_t *RA, const int8_t *RB, int nmod, int group, const ModConsts &mc,
                           int8_t *planes, const Layout &L, hipStream_t s, Ev ev) {
    const bool small = use_small_tiles(L, nmod * group);
    GemmArgs g = gemm_args(RA, RB, nmod, group, L, small);
    g.planes = planes;
    const int blocks = g.tiles_m * g.tiles_n * g.nmod;
    const int64_t nk = L.kb / 2;  // stages of 64 K
    // blocks of at most kReduceStages stages, the later ones accumulating
    for (int64_t ks0 = 0; ks0 < nk; ks0 += kReduceStages) {
        g.ks0 = ks0;
        g.nks = (int)(nk - ks0 < kReduceStages ? nk - ks0 : kReduceStages);
        g.accumulate = ks0 > 0;
        Ev e;
        if (ks0 == 0) e.start = ev.start;
        if (ks0 + kReduceStages >= nk) e.stop = ev.stop;
        if (small) {
            auto kern = k_gemm<EPI_MOD, ShapeS>;
            OZ2_LAUNCH(e, kern, dim3(blocks), dim3(64 * ShapeS::W), 0, s, g, mc);
        } else if (use_persistent(g.nks, L, blocks)) {
            // one block per compute unit (the kernel's 160 KiB of LDS admits no second)
            const int grid = blocks < compute_units() ? blocks : compute_units();
            OZ2_LAUNCH(e, k_gemm_persistent, dim3(grid), dim3(64 * ShapeP::W), 0, s, g, mc);
        } else {
            auto kern = k_gemm<EPI_MOD, ShapeL>;
            OZ2_LAUNCH(e, kern, dim3(blocks), dim3(64 * ShapeL::W), 0, s, g, mc);
        }
    }
    return hipGetLastError();
}

hipError_t launch_gemm_raw(const int8_t *RA, const int8_t *RB, int nmod, int group, int32_t *raw, const Layout &L,
                           hipStream_t s) {
    const bool small = use_small_tiles(L, nmod * group);
    GemmArgs g = gemm_args(RA, RB, nmod, group, L, small);
    g.raw = raw;
    ModConsts mc{};
    const int blocks = g.tiles_m * g.tiles_n * g.nmod;
    if (small)
        hipLaunchKernelGGL((k_gemm<EPI_RAW, ShapeS>), dim3(blocks), dim3(64 * ShapeS::W), 0, s, g, mc);
    else
        hipLaunchKernelGGL((k_gemm<EPI_RAW, ShapeL>), dim3(blocks), dim3(64 * ShapeL::W), 0, s, g, mc);
    return hipGetLastError();
}

hipError_t launch_gemm_bound(const int8_t *Abar, const int8_t *Bbar, int32_t *rowmax, int32_t *colmax,
                             const Layout &L, hipStream_t s) {
    const bool small = use_small_tiles(L, 1);
    GemmArgs g = gemm_args(Abar, Bbar, 1, 1, L, small);
    g.rowmax = rowmax;
    g.colmax = colmax;
    ModConsts mc{};
    const int blocks = g.tiles_m * g.tiles_n;
    if (small)
        hipLaunchKernelGGL((k_gemm<EPI_BOUND, ShapeS>), dim3(blocks), dim3(64 * ShapeS::W), 0, s, g, mc);
    else
        hipLaunchKernelGGL((k_gemm<EPI_BOUND, ShapeL>), dim3(blocks), dim3(64 * ShapeL::W), 0, s, g, mc);
    return hipGetLastError();
}

hipError_t launch_accurate_exponents(int64_t m, int64_t n, double Pp, const Layout &L, char *ws, hipStream_t s,
                                     Ev ev) {
    OZ2_LAUNCH(ev, k_accurate_exponents, dim3(nblk(L.m_pad + L.n_pad, 256)), dim3(256), 0, s,
                       (const int32_t *)(ws + L.rowmax), (const int32_t *)(ws + L.colmax),
                       (const int32_t *)(ws + L.ga), (const int32_t *)(ws + L.gb), m, L.m_pad, n, L.n_pad, Pp,
                       (int32_t *)(ws + L.e), (int32_t *)(ws + L.f));
    return hipGetLastError();
}

template <class OutT>
static hipError_t launch_crt_t(const int8_t *planes, int64_t m, int64_t n, const int32_t *e, const int32_t *f,
                               const CrtConsts &cc, OutT *C, int64_t ldc, const Layout &L, hipStream_t s, Ev ev) {
    dim3 grid(nblk((m + kCrtRows - 1) / kCrtRows, 256), ydim(n));
    if (cc.n <= 16 && cc.nd <= 16 && cc.np32 <= 4) {
        auto kern = cc.np32 == 2 ? k_crt_mma<OutT, 2> : cc.np32 == 3 ? k_crt_mma<OutT, 3> : k_crt_mma<OutT, 4>;
        // two columns per block: half the blocks, each loading the digit
        // table once for both (4096^2, 16 moduli: 0.090 -> 0.086 ms)
        const dim3 g2(grid.x, ydim((n + 1) / 2));
        OZ2_LAUNCH(ev, kern, g2, dim3(256), 0, s, planes, L.m_pad * L.n_pad, L.m_pad, m, n, e, f, cc, C, ldc);
    } else if (cc.n >= 17 && cc.n <= 20 && cc.nd <= 20 && cc.np32 <= 5 &&
               !(getenv("OZ2_CRT") && strcmp(getenv("OZ2_CRT"), "fma") == 0)) {
        auto kern = cc.n == 17 ? k_crt_mma20<OutT, 17> : cc.n == 18 ? k_crt_mma20<OutT, 18>
                  : cc.n == 19 ? k_crt_mma20<OutT, 19> : k_crt_mma20<OutT, 20>;
        OZ2_LAUNCH(ev, kern, grid, dim3(256), 0, s, planes, L.m_pad * L.n_pad, L.m_pad, m, n, e, f, cc, C, ldc);
    } else {
        // FP64-FMA form on 40-bit pieces (OZ2_CRT=fma)
        auto kern = k_crt<OutT>;
        OZ2_LAUNCH(ev, kern, grid, dim3(256), 0, s, planes, L.m_pad * L.n_pad, L.m_pad, m, n, e, f, cc, C, ldc);
    }
    return hipGetLastError();
}

template <class OutT>
static hipError_t launch_gemm_crt_t(const int8_t *RA, const int8_t *RB, int64_t m, int64_t n, const int32_t *e,
                                   const int32_t *f, const CrtConsts &cc, const ModConsts &mc, OutT *C, int64_t ldc,
                                   const Layout &L, hipStream_t s, Ev ev) {
    const int tiles_m = (int)((m + kFTile - 1) / kFTile), tiles_n = (int)((n + kFTile - 1) / kFTile);
    auto kern = k_gemm_crt<OutT>;
    OZ2_LAUNCH(ev, kern, dim3((unsigned)tiles_m * (unsigned)tiles_n), dim3(256), 0, s, RA, RB, L.m_pad * L.k_pad,
               L.n_pad * L.k_pad, (int)(L.kb / 2), tiles_m, e, f, cc, mc, C, m, n, ldc);
    return hipGetLastError();
}

bool gemm_crt_applies(const Layout &L, int64_t m, int64_t n) {
    // the int32 sums of one modulus stay within smod's range for at most
    // kReduceStages stages, and the grid is one block per 64 x 64 tile
    return L.kb / 2 <= kReduceStages && ((m + kFTile - 1) / kFTile) * ((n + kFTile - 1) / kFTile) < (1ll << 31);
}

hipError_t launch_gemm_crt(Elem el, const int8_t *RA, const int8_t *RB, int64_t m, int64_t n, const int32_t *e,
                           const int32_t *f, const CrtConsts &cc, const ModConsts &mc, void *C, int64_t ldc,
                           const Layout &L, hipStream_t s, Ev ev) {
    if (el == Elem::f32) return launch_gemm_crt_t(RA, RB, m, n, e, f, cc, mc, (float *)C, ldc, L, s, ev);
    return launch_gemm_crt_t(RA, RB, m, n, e, f, cc, mc, (double *)C, ldc, L, s, ev);
}

hipError_t launch_crt(Elem el, const int8_t *planes, int64_t m, int64_t n, const int32_t *e, const int32_t *f,
                      const CrtConsts &cc, void *C, int64_t ldc, const Layout &L, hipStream_t s, Ev ev) {
    if (el == Elem::f32) return launch_crt_t(planes, m, n, e, f, cc, (float *)C, ldc, L, s, ev);
    return launch_crt_t(planes, m, n, e, f, cc, (double *)C, ldc, L, s, ev);
}

hipError_t launch_crt_complex(Elem el, const int8_t *planes, int64_t m, int64_t n, const int32_t *e,
                              const int32_t *f, const CrtConsts &cc, const ModConsts &mc, void *C, int64_t ldc,
                              const Layout &L, hipStream_t s, Ev ev) {
    dim3 grid(nblk((m + kCrtRows - 1) / kCrtRows, 256), ydim(n));
    if (cc.n <= 16 && cc.nd <= 16 && cc.nnd <= 16 && cc.np32 <= 4 &&
        !(getenv("OZ2_CRT") && strcmp(getenv("OZ2_CRT"), "fma") == 0)) {
        if (el == Elem::f32) {
            auto kern = cc.np32 == 2 ? k_crt_c_mma<float, 2> : cc.np32 == 3 ? k_crt_c_mma<float, 3> : k_crt_c_mma<float, 4>;
            OZ2_LAUNCH(ev, kern, grid, dim3(256), 0, s, planes, L.m_pad * L.n_pad, L.m_pad, m, n, e, f, cc, (float *)C,
                       ldc);
        } else {
            auto kern = cc.np32 == 2 ? k_crt_c_mma<double, 2> : cc.np32 == 3 ? k_crt_c_mma<double, 3>
                                                                              : k_crt_c_mma<double, 4>;
            OZ2_LAUNCH(ev, kern, grid, dim3(256), 0, s, planes, L.m_pad * L.n_pad, L.m_pad, m, n, e, f, cc, (double *)C,
                       ldc);
        }
    } else if (cc.n >= 17 && cc.n <= 20 && cc.nd <= 20 && cc.nnd <= 20 && cc.np32 <= 5 &&
               !(getenv("OZ2_CRT") && strcmp(getenv("OZ2_CRT"), "fma") == 0)) {
        if (el == Elem::f32) {
            auto kern = cc.n == 17 ? k_crt_c_mma20<float, 17> : cc.n == 18 ? k_crt_c_mma20<float, 18>
                      : cc.n == 19 ? k_crt_c_mma20<float, 19> : k_crt_c_mma20<float, 20>;
            OZ2_LAUNCH(ev, kern, grid, dim3(256), 0, s, planes, L.m_pad * L.n_pad, L.m_pad, m, n, e, f, cc, (float *)C,
                       ldc);
        } else {
            auto kern = cc.n == 17 ? k_crt_c_mma20<double, 17> : cc.n == 18 ? k_crt_c_mma20<double, 18>
                      : cc.n == 19 ? k_crt_c_mma20<double, 19> : k_crt_c_mma20<double, 20>;
            OZ2_LAUNCH(ev, kern, grid, dim3(256), 0, s, planes, L.m_pad * L.n_pad, L.m_pad, m, n, e, f, cc, (double *)C,
                       ldc);
        }
    } else if (el == Elem::f32) {
        auto kern = k_crt_c<float>;
        OZ2_LAUNCH(ev, kern, grid, dim3(256), 0, s, planes, L.m_pad * L.n_pad, L.m_pad, m, n, e, f, cc, mc,
                   (float *)C, ldc);
    } else {
        auto kern = k_crt_c<double>;
        OZ2_LAUNCH(ev, kern, grid, dim3(256), 0, s, planes, L.m_pad * L.n_pad, L.m_pad, m, n, e, f, cc, mc,
                   (double *)C, ldc);
    }
    return hipGetLastError();
}

hipError_t launch_pack_planes(const uint8_t *residues, int nplanes, int group, const ModConsts &mc, int64_t m,
                              int64_t n, const Layout &L, int8_t *planes, hipStream_t s) {
    dim3 grid(nblk(L.m_pad, 256), ydim(n), (unsigned)nplanes);
    hipLaunchKernelGGL(k_pack_planes, grid, dim3(256), 0, s, residues, m, n, L.m_pad, L.m_pad * L.n_pad, mc, group,
                       planes);
    return hipGetLastError();
}

hipError_t launch_crt_check(const int8_t *planes, int64_t m, int64_t n, const CheckConsts &ck, const Layout &L,
                            uint8_t *flags, hipStream_t s) {
    hipLaunchKernelGGL(k_crt_check, dim3(nblk(m, 256), ydim(n)), dim3(256), 0, s, planes, L.m_pad * L.n_pad, L.m_pad,
                       m, n, ck, flags);
    return hipGetLastError();
}

hipError_t launch_zero_fill(Elem el, void *C, int64_t m, int64_t n, int64_t ldc, hipStream_t s) {
    if (el == Elem::f32)
        hipLaunchKernelGGL(k_zero_c<float>, dim3(nblk(m, 256), ydim(n)), dim3(256), 0, s, (float *)C, m, n, ldc);
    else
        hipLaunchKernelGGL(k_zero_c<double>, dim3(nblk(m, 256), ydim(n)), dim3(256), 0, s, (double *)C, m, n, ldc);
    return hipGetLastError();
}

hipError_t launch_unpack_residues(const int8_t *packed, int nmod, int64_t rows, int64_t k, int64_t rows_pad,
                                  const Layout &L, int8_t *out, hipStream_t s) {
    dim3 grid(nblk(k, 256), ydim(rows), (unsigned)nmod);
    hipLaunchKernelGGL(k_unpack, grid, dim3(256), 0, s, packed, rows, k, rows_pad * L.k_pad, L.kb, out);
    return hipGetLastError();
}

hipError_t launch_copy_planes_u8(const int8_t *planes, int nmod, int group, const ModConsts &mc, int64_t m,
                                 int64_t n, const Layout &L, uint8_t *out, hipStream_t s) {
    dim3 grid(nblk(m, 256), ydim(n), (unsigned)(nmod * group));
    hipLaunchKernelGGL(k_copy_planes_red, grid, dim3(256), 0, s, planes, m, L.m_pad, L.m_pad * L.n_pad, n, mc, group,
                       out);
    return hipGetLastError();
}

hipError_t launch_copy_planes_i32(const int32_t *raw, int nmod, int64_t m, int64_t n, const Layout &L,
                                  int32_t *out, hipStream_t s) {
    dim3 grid(nblk(m, 256), ydim(n), (unsigned)nmod);
    hipLaunchKernelGGL(k_copy_planes_i32, grid, dim3(256), 0, s, raw, m, L.m_pad, L.m_pad * L.n_pad, n, out);
    return hipGetLastError();
}

}  // namespace oz2
