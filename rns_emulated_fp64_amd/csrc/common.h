// common.h -- declarations shared by the host API (api.cpp, noalloc.hip) and
// the HIP kernels (kernels.hip) of libozaki2.
//
// Ozaki Scheme II steps follow the Qiita article "8ビットの整数で53ビットの倍精度
// を組み立てる。中国剰余定理をGPUに載せたOzaki Scheme II" ([Q]) and the summary
// "Improved Scaling for Fast Mode of Ozaki Scheme II" ([G]).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace oz2 {

constexpr int kMaxModuli = 20;
constexpr int kChunks = 4;          // CRT weights and P in 40-bit pieces (4 x 40 >= 156 bits)
constexpr int kChunks32 = 5;        // P in 32-bit pieces (5 x 32 >= 156 bits)
constexpr int kChunkBits = 40;
constexpr int kMaxDigits = 20;      // W_l < P < 2^156 has at most 20 signed base-256 digits
constexpr int kExpNonfinite = INT32_MIN;  // exponent marker: row/column holds Inf or NaN
constexpr int kExpEmpty = -4000;          // max-exponent marker of an all-zero row/column

// Tiling of the packed int8 operands and of the GEMM. A packed operand of R
// rows and K columns (K a multiple of kKPad) is stored per modulus as
// [R/16][K/64] fragment blocks of 1 KiB; inside a block, lane L (0..63) owns
// 16 bytes at L*16 holding row (L % 16) and columns 16*(L / 16) .. +15. This is
// the operand order of v_mfma_i32_16x16x64_i8, so every global->LDS and
// LDS->register move is a contiguous 1 KiB per wavefront.
constexpr int kTileM = 256;   // row padding of A (the GEMM's largest block tile; 128 divides it)
constexpr int kTileN = 256;   // column padding of B
constexpr int kKPad = 128;    // K padding granule (split kernel tile width)

// Host-computed constants for the residue split ([Q] steps 1 and 2).
struct SplitConsts {
    int n;                      // number of moduli; moduli[0] is 256
    double p[kMaxModuli];       // moduli as doubles
    double pinv[kMaxModuli];    // RN(1 / p)
    double c42[kMaxModuli];     // 2^42 mod p, symmetric range
};

// Host-computed constants for the CRT reconstruction ([Q] step 4).
struct CrtConsts {
    int n;
    double w[kMaxModuli][kChunks];  // weight W_l = (P/p_l)((P/p_l)^-1 mod p_l), 40-bit pieces
    double P[kChunks];              // P, 40-bit pieces
    double H[kChunks];              // P / 2, 40-bit pieces
    double pinv120;                 // RN(2^120 / P)
    double P32[kChunks32];          // P in 32-bit pieces
    double H32[kChunks32];          // P / 2 in 32-bit pieces
    double pinv128;                 // RN(2^128 / P)
    double pinv96;                  // RN(2^96 / P)
    double pinv64;                  // RN(2^64 / P)
    double pinv32;                  // RN(2^32 / P)
    int np32;                       // 32-bit pieces for the digit sums and for P (2..5)
    int nd;                         // signed base-256 digits of the weights (<= kMaxDigits)
    int8_t digit[kMaxDigits][32];   // digit[v][l] = v-th digit of W_l, |digit| <= 128; 0 for l >= n
    int nnd;                        // signed base-256 digits of P - W_l (<= kMaxDigits)
    int8_t ndigit[kMaxDigits][32];  // ndigit[v][l] = v-th digit of P - W_l; 0 for l >= n
};

// Constants of the CRT-range check against one redundant modulus pc (the
// (n+1)-th of the table): X = S - q P with S / P = sum_l c_l K_l / p_l, so
// X mod pc = sum_l c_l (W_l mod pc) - q (P mod pc) (mod pc).
struct CheckConsts {
    int n;                   // moduli of the reconstruction
    int pc;                  // check modulus
    double kp[kMaxModuli];   // RN(K_l / p_l), K_l = (P / p_l)^-1 mod p_l
    int wm[kMaxModuli];      // W_l mod pc
    int pm;                  // P mod pc
};

// Constants for the GEMM epilogue (reduction mod p_l).
struct ModConsts {
    double p[kMaxModuli];
    double pinv[kMaxModuli];
};

// Byte offsets of the workspace regions (all 256-byte aligned).
struct Layout {
    int64_t m_pad, n_pad, k_pad, kb;  // kb = k_pad / 32
    int nchunks;                      // k-chunks of the row-norm pass over A
    int64_t kchunk;
    size_t e, f, ga, gb;              // int32 [m_pad], [n_pad], [m_pad], [n_pad]
    size_t part_s, part_g, part_bad;  // row-norm partials [nchunks][m]
    size_t rowmax, colmax;            // int32 [m_pad], [n_pad] (accurate mode)
    size_t abar, bbar;                // int8 packed bound operands (accurate mode)
    size_t ra, rb;                    // int8 packed residues [N][m_pad][k_pad], [N][n_pad][k_pad]
    size_t planes;                    // int8 [N][n_pad][m_pad]: products mod p, symmetric range
    size_t raw;                       // int32 [N][n_pad][m_pad] (debug only)
    size_t total;
};

enum Phase { kPhaseScale = 0, kPhaseSplit = 1, kPhaseGemm = 2, kPhaseCrt = 3, kNumPhases = 4 };

// Optional timing events of one kernel launch: start takes the kernel's start
// time, stop its end time.
struct Ev {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};

// Element type of A, B and C: FP64 (ozaki2_dgemm) or binary32 (ozaki2_sgemm).
enum class Elem { f64, f32 };

// A real product on a caller-provided workspace: the checks and phases of
// ozaki2_dgemm_ws / ozaki2_sgemm_ws (api.cpp), for the library's other entry
// points. Returns an ozaki2 status.
int product_ws(Elem el, int64_t m, int64_t n, int64_t k, const void *A, int64_t lda, const void *B, int64_t ldb,
               void *C, int64_t ldc, int nmod, int mode, void *workspace, size_t wbytes, void *stream);

// ---- kernel launchers (kernels.hip). Each returns hipGetLastError(). ----
// cplx: interleaved complex operands (A, B, C hold (re, im) pairs; leading
// dimensions count complex elements).
// original: the stand-in exponents of OZAKI2_FAST_ORIGINAL (real operands only).
hipError_t launch_scale(Elem el, bool cplx, bool original, const void *A, int64_t m, int64_t k, int64_t lda,
                        const void *B, int64_t n, int64_t ldb, double Pp, const Layout &L, char *ws, hipStream_t s,
                        Ev ev = {});
hipError_t launch_row_exponents(int64_t m, double Pp, const Layout &L, char *ws, hipStream_t s, Ev ev = {});
hipError_t launch_split(Elem el, bool cplx, bool original, const void *A, int64_t m, int64_t lda, const void *B,
                        int64_t n, int64_t ldb, int64_t k, bool fold_row_exponents, double Pp,
                        const SplitConsts &sc, const Layout &L, char *ws, hipStream_t s, Ev ev = {});
hipError_t launch_quantize(Elem el, const void *A, int64_t m, int64_t lda, const void *B, int64_t n, int64_t ldb,
                           int64_t k, const Layout &L, char *ws, hipStream_t s);
hipError_t launch_gemm_mod(const int8_t *RA, const int8_t *RB, int nmod, int group, const ModConsts &mc,
                           int8_t *planes, const Layout &L, hipStream_t s, Ev ev = {});
hipError_t launch_gemm_raw(const int8_t *RA, const int8_t *RB, int nmod, int group, int32_t *raw,
                           const Layout &L, hipStream_t s);
hipError_t launch_gemm_bound(const int8_t *Abar, const int8_t *Bbar, int32_t *rowmax, int32_t *colmax,
                             const Layout &L, hipStream_t s);
hipError_t launch_accurate_exponents(int64_t m, int64_t n, double Pp, const Layout &L, char *ws,
                                     hipStream_t s, Ev ev = {});
hipError_t launch_crt(Elem el, const int8_t *planes, int64_t m, int64_t n, const int32_t *e, const int32_t *f,
                      const CrtConsts &cc, void *C, int64_t ldc, const Layout &L, hipStream_t s, Ev ev = {});
// Steps 3-5 in one launch (real products): all moduli of a 64 x 64 tile of C
// per block, reconstructed in registers; applies when gemm_crt_applies.
bool gemm_crt_applies(const Layout &L, int64_t m, int64_t n);
hipError_t launch_gemm_crt(Elem el, const int8_t *RA, const int8_t *RB, int64_t m, int64_t n, const int32_t *e,
                           const int32_t *f, const CrtConsts &cc, const ModConsts &mc, void *C, int64_t ldc,
                           const Layout &L, hipStream_t s, Ev ev = {});
hipError_t launch_crt_complex(Elem el, const int8_t *planes, int64_t m, int64_t n, const int32_t *e,
                              const int32_t *f, const CrtConsts &cc, const ModConsts &mc, void *C, int64_t ldc,
                              const Layout &L, hipStream_t s, Ev ev = {});
// flags[j*m + i]: 0 the reconstruction of entry (i, j) from the first ck.n
// planes agrees with plane ck.n (the check modulus), 1 it does not (the
// integer left (-P/2, P/2]), 2 undecided (|X| at P/2 within 2^-30 P).
hipError_t launch_crt_check(const int8_t *planes, int64_t m, int64_t n, const CheckConsts &ck, const Layout &L,
                            uint8_t *flags, hipStream_t s);
hipError_t launch_zero_fill(Elem el, void *C, int64_t m, int64_t n, int64_t ldc, hipStream_t s);
hipError_t launch_unpack_residues(const int8_t *packed, int nmod, int64_t rows, int64_t k,
                                  int64_t rows_pad, const Layout &L, int8_t *out, hipStream_t s);
hipError_t launch_copy_planes_u8(const int8_t *planes, int nmod, int group, const ModConsts &mc, int64_t m,
                                 int64_t n, const Layout &L, uint8_t *out, hipStream_t s);
// residues [nplanes][n][m] in [0, p) -> symmetric int8 planes; plane q is
// reduced mod p[q / group]
hipError_t launch_pack_planes(const uint8_t *residues, int nplanes, int group, const ModConsts &mc, int64_t m,
                              int64_t n, const Layout &L, int8_t *planes, hipStream_t s);
hipError_t launch_copy_planes_i32(const int32_t *raw, int nmod, int64_t m, int64_t n, const Layout &L,
                                  int32_t *out, hipStream_t s);

}  // namespace oz2
