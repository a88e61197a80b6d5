/*
 * ozaki2.h -- C ABI of libozaki2.so: FP64 matrix products emulated with
 * Ozaki Scheme II on INT8 matrix cores of AMD Instinct MI355X (gfx950).
 *
 * Pages this interface follows:
 *   [Q] "8ビットの整数で53ビットの倍精度を組み立てる。中国剰余定理をGPUに載せた
 *       Ozaki Scheme II" (Qiita article), section "Ozaki Scheme IIのGPU実装"
 *       and its subsections for steps 1-5;
 *   [G] "Improved Scaling for Fast Mode of Ozaki Scheme II" (technical
 *       summary), section Methodik (the proposed fast-mode scaling) and
 *       section Problemstellung (fast and accurate modes).
 *
 * The pages give no programming interface; this one follows BLAS DGEMM
 * conventions: C := A * B (alpha = 1, beta = 0), column-major storage, no
 * transposes.
 *
 * Arguments common to the product entry points
 *   m, n, k   sizes: A is m x k, B is k x n, C is m x n; each >= 0.
 *   A, lda    DEVICE pointer to A, column-major, element (i, h) at
 *             A[i + h*lda]; lda >= max(1, m).
 *   B, ldb    DEVICE pointer to B, element (h, j) at B[h + j*ldb];
 *             ldb >= max(1, k).
 *   C, ldc    DEVICE pointer to C, element (i, j) at C[i + j*ldc];
 *             ldc >= max(1, m). C must not overlap A, B or the workspace.
 *   num_moduli N in [2, 20]: the first N moduli of the implementation's
 *             table (256, 255, 253, 251, 247, 241, 239, 233, 229, 227, 223,
 *             217, 211, 199, 197, 193, 191, 181, 179, 173), the largest
 *             pairwise-coprime integers <= 256 ([Q] section
 *             256以下の法の選び方(手順2) and its footnote). N >= 14 reaches
 *             the accuracy of native FP64 on typical inputs
 *             ([Q] section 行列積の回数と性能).
 *   mode      OZAKI2_FAST: the scale-invariant Cauchy-Schwarz scaling of [G]
 *             section Methodik; OZAKI2_ACCURATE: one extra INT8 GEMM bounds
 *             the products before scaling ([Q] section
 *             2の累乗による整数化(手順1と5), [G] section Problemstellung);
 *             OZAKI2_FAST_ORIGINAL: comparison stand-in, see enum ozaki2_mode.
 *   stream    hipStream_t to enqueue on (NULL = default stream). All device
 *             work is asynchronous; no call synchronises the stream.
 *
 * Environment: OZ2_GEMM_TILE=128 or 256 forces the INT8 GEMM's block shape
 * (by default 256 x 256, or 128 x 128 for products too small to give every
 * two compute units a 256 x 256 block); OZ2_FUSED=1 runs steps 3-5 of real
 * products as one launch (every modulus of a 64 x 64 tile of C in one block,
 * reconstructed in registers; [Q] section 誤差のないINT8行列積(手順3): the
 * per-modulus products are independent), OZ2_FUSED=0 as two (a 256 x 256
 * GEMM writing residue planes and a reconstruction reading them); by default
 * one launch only for tiny products (N times the stages of 64 of k at most
 * 16, at most 64 tiles of 64 x 64), two otherwise; the debug entry points
 * always use two. The 256 x 256 tile runs on a persistent kernel (one block of
 * four wavefronts per compute unit walking its tiles) when there are more
 * tiles than compute units, else one tile per block (eight wavefronts);
 * OZ2_GEMM_KERNEL=blocks or =persistent forces either. Results do not depend
 * on any of these settings. OZ2_CRT=fma reconstructs real products
 * with 17 to 20 moduli, and complex products with any number, with FP64 FMAs
 * on 40-bit pieces instead of digit sums on the matrix cores (the same
 * results).
 *
 * Memory ownership: A, B, C and any workspace belong to the caller. The
 * library keeps one cached workspace per device for ozaki2_dgemm (freed by
 * ozaki2_finalize) and small per-device constant tables.
 *
 * Status codes: 0 success; -i the i-th argument (1-based, in signature order)
 * is invalid, as in BLAS xerbla; positive codes are the OZAKI2_ERR_* values.
 * All argument checks happen before any HIP call, so a negative status
 * never touches the device.
 *
 * Values: inputs should be finite. A row of A (or column of B) holding Inf
 * or NaN turns the matching row (column) of C into NaN. Zero rows and
 * columns give exact zeros. Results are bitwise reproducible from run to run
 * and equal, for every input whose rows and columns are finite,
 * RN(sum_h trunc(2^e_i a_ih) trunc(2^f_j b_hj)) * 2^-(e_i + f_j) with the
 * exponents e, f the chosen mode computes.
 */
#ifndef OZAKI2_H
#define OZAKI2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum ozaki2_mode {
    OZAKI2_FAST = 0,          /* proposed scale-invariant fast-mode scaling ([G] Methodik) */
    OZAKI2_ACCURATE = 1,      /* extra INT8 bound GEMM ([G] Problemstellung, mode 1) */
    OZAKI2_FAST_ORIGINAL = 2  /* for comparisons only: a stand-in for the original fast-mode rule that
                                 [G] Problemstellung shows is not scale invariant (the pages do not
                                 print it): squares of the binary32-rounded entries summed in binary32,
                                 e = floor(P' - 0.5 log2f(sum)), no margin; an overflowed sum gives
                                 mu = 0 and one that underflows to zero leaves mu unbounded, the two
                                 failure directions [G] describes. Results are not guaranteed to
                                 reconstruct; real operands only. */
};

enum ozaki2_status {
    OZAKI2_SUCCESS = 0,
    OZAKI2_ERR_HIP = 1,         /* a HIP runtime call or kernel launch failed */
    OZAKI2_ERR_WORKSPACE = 2,   /* workspace too small, or its allocation failed */
    OZAKI2_ERR_UNSUPPORTED = 3, /* size outside the supported range: k > OZAKI2_MAX_K,
                                   accurate mode with k > OZAKI2_MAX_K_ACCURATE, m or
                                   n >= 2^31, or prod_out requested with k >= 2^17 */
    OZAKI2_ERR_NOALLOC_LIMIT = 4 /* ozaki2_dgemm_noalloc: the product needs more than
                                    OZAKI2_NOALLOC_MAX_WORKSPACE bytes of workspace */
};

#define OZAKI2_MAX_MODULI 20
/* Inner dimension limits. int32 sums of int8 x int8 products are exact only
 * below 2^17 terms ([Q] section 誤差のないINT8行列積(手順3)); longer inner
 * dimensions are handled in blocks (the GEMM reduces each block of at most
 * 1024 * 64 terms mod p and adds the residues of the blocks). The
 * accurate-mode bound product (entries <= 64 * 64
 * per term) stays exact below 2^19 terms. */
#define OZAKI2_MAX_K ((1 << 22) - 1)
#define OZAKI2_MAX_K_ACCURATE ((1 << 19) - 1)

/*
 * C := A * B emulated by Ozaki Scheme II ([Q] steps 1-5). Uses a workspace
 * cached per device, grown on first use of a larger problem (that growth is
 * the only blocking action: hipMalloc after synchronising the device).
 * Every cached-workspace call on a device (ozaki2_dgemm, _sgemm, _zgemm,
 * _cgemm) shares that one workspace: each call's kernels are made to wait
 * (hipStreamWaitEvent) for those of the previous such call, whatever stream
 * it used, so calls on different streams give correct results but run one
 * after another on the GPU. For products that should overlap, use
 * ozaki2_dgemm_ws with a workspace per stream. Not capturable into a HIP
 * graph (it records and waits on a library event); the _ws form is.
 * Returns 0, -1..-11 for an invalid argument (m, n, k, A, lda, B, ldb, C,
 * ldc, num_moduli, mode), OZAKI2_ERR_UNSUPPORTED, OZAKI2_ERR_WORKSPACE or
 * OZAKI2_ERR_HIP. m == 0 or n == 0 returns at once; k == 0 fills C with zeros.
 */
int ozaki2_dgemm(int64_t m, int64_t n, int64_t k,
                 const double *A, int64_t lda, const double *B, int64_t ldb,
                 double *C, int64_t ldc, int num_moduli, int mode, void *stream);

/*
 * Bytes of device workspace ozaki2_dgemm_ws needs for this problem
 * (0 for invalid arguments or empty products). Host-only; no HIP call.
 * The workspace ([Q] section エミュレーションで足りるかを判断する観点: the
 * emulation keeps its intermediates in a workspace of its own) holds, for N
 * moduli, N int8 residue planes of A and of B and N int8 product planes:
 * about N * (m k + n k + m n) bytes, plus small exponent and norm arrays
 * (and the bound operands in accurate mode).
 */
size_t ozaki2_workspace_size(int64_t m, int64_t n, int64_t k, int num_moduli, int mode);

/*
 * As ozaki2_dgemm, with a caller-provided DEVICE workspace of at least
 * ozaki2_workspace_size(...) bytes, 256-byte aligned (the kernels' 16-byte
 * vector and 1 KiB LDS-copy accesses rely on it). The workspace holds the
 * residue planes and products between the steps; [Q] section
 * エミュレーションで足りるかを判断する観点 notes that such emulation needs a
 * workspace of its own (gigabytes for large products), which is why the
 * caller may provide it. Never allocates and is re-entrant; calls that share
 * one workspace must be ordered on one stream.
 * It only enqueues kernels on the stream (no memset, copy or host
 * synchronisation), so it can be captured into a HIP graph and replayed;
 * timing (ozaki2_timing_enable) must be off while capturing.
 * Returns as ozaki2_dgemm; -12 if workspace is NULL (while needed) or not
 * 256-byte aligned, OZAKI2_ERR_WORKSPACE if workspace_bytes is too small.
 */
int ozaki2_dgemm_ws(int64_t m, int64_t n, int64_t k,
                    const double *A, int64_t lda, const double *B, int64_t ldb,
                    double *C, int64_t ldc, int num_moduli, int mode,
                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): exactly
 * ozaki2_dgemm_ws, with the workspace taken from a static device array of
 * OZAKI2_NOALLOC_MAX_WORKSPACE bytes inside the library instead of an
 * argument. Each GPU the library is loaded on holds its own copy of that
 * array until the process ends. The call allocates nothing (no hipMalloc,
 * hipFree or allocating library routine); on its first call on a device it
 * looks up the array's device address (hipGetSymbolAddress) and keeps it.
 * Products whose ozaki2_workspace_size exceeds the array are refused with
 * OZAKI2_ERR_NOALLOC_LIMIT (about 1024^3 at 20 moduli, 1400^3 at 16 fit).
 * Every call on one GPU uses that GPU's one array, so calls that overlap on
 * one GPU (on different streams, or from several threads without ordering
 * their streams) race and corrupt each other's results: order them on one
 * stream. The array keeps the last call's contents; nothing in it needs to
 * start at zero (every call writes all it reads).
 * Returns as ozaki2_dgemm_ws, with OZAKI2_ERR_NOALLOC_LIMIT in place of the
 * workspace errors.
 */
#define OZAKI2_NOALLOC_MAX_WORKSPACE (128u << 20)
int ozaki2_dgemm_noalloc(int64_t m, int64_t n, int64_t k,
                         const double *A, int64_t lda, const double *B, int64_t ldb,
                         double *C, int64_t ldc, int num_moduli, int mode, void *stream);

/*
 * Test entry point (layout of the copies is stable, timing is not): runs
 * ozaki2_dgemm_ws and also copies intermediates into caller DEVICE buffers,
 * each of which may be NULL to skip it:
 *   e_out    int32 [m]: exponent of each row of A (mu_i = 2^e_i), step 1;
 *   f_out    int32 [n]: exponent of each column of B;
 *            INT32_MIN marks a row/column holding Inf or NaN;
 *   resA_out int8 [N][m][k]: residues of trunc(2^e_i a_ih) mod p_l in the
 *            symmetric range (-(p-1)/2..(p-1)/2, -128..127 for 256), step 2;
 *   resB_out int8 [N][n][k]: residues of trunc(2^f_j b_hj), element
 *            (l, j, h) at resB_out[(l*n + j)*k + h];
 *   prod_out int32 [N][n][m]: exact residue products
 *            Q_l(i, j) = sum_h resA(l,i,h) resB(l,j,h) at prod_out[(l*n + j)*m + i], step 3
 *            (only for k < 2^17, where they fit int32);
 *   red_out  uint8 [N][n][m]: Q_l mod p_l in [0, p_l), same indexing.
 * Argument errors as ozaki2_dgemm_ws (workspace_bytes must also cover
 * ozaki2_debug_workspace_size); -13..-18 for a NULL-but-needed debug buffer
 * is never returned (NULL means skip).
 */
int ozaki2_dgemm_debug(int64_t m, int64_t n, int64_t k,
                       const double *A, int64_t lda, const double *B, int64_t ldb,
                       double *C, int64_t ldc, int num_moduli, int mode,
                       void *workspace, size_t workspace_bytes,
                       int32_t *e_out, int32_t *f_out, int8_t *resA_out, int8_t *resB_out,
                       int32_t *prod_out, uint8_t *red_out, void *stream);

/*
 * Test entry point for steps 4 + 5 alone ([Q] sections 秦九韶の大衍求一術 and
 * 2の累乗による整数化(手順1と5)): C = RN(X) * 2^-(e_i + f_j), X the integer in
 * (-P/2, P/2] with X = c_l (mod p_l) for every modulus, reconstructed by the
 * same kernels ozaki2_dgemm uses.
 *   residues DEVICE uint8 [N][n][m]: c_l of entry (i, j) at
 *            residues[(l*n + j)*m + i], each in [0, p_l) (not checked);
 *   e, f     DEVICE int32 [m], [n]: exponents; INT32_MIN makes the row
 *            (column) NaN;
 *   C, ldc   DEVICE output, column-major;
 *   workspace DEVICE, at least ozaki2_workspace_size(m, n, 1, N, OZAKI2_FAST)
 *            bytes.
 * Returns 0; -1 m < 0, -2 n < 0, -3 num_moduli outside [2, 20], -4 residues,
 * -5 e, -6 f or -7 C NULL while needed, -8 ldc < max(1, m), -9 workspace
 * NULL or not 256-byte aligned; OZAKI2_ERR_WORKSPACE if workspace_bytes is too small,
 * OZAKI2_ERR_UNSUPPORTED for m or n >= 2^31, OZAKI2_ERR_HIP.
 */
int ozaki2_crt_debug(int64_t m, int64_t n, int num_moduli, const uint8_t *residues, const int32_t *e,
                     const int32_t *f, double *C, int64_t ldc, void *workspace, size_t workspace_bytes,
                     void *stream);

/*
 * Test entry point: the CRT-range failure flag. An integer outside (-P/2, P/2]
 * is silently reconstructed as another one ([Q] section
 * 時計の針で見る定理の中身; [G] section Problemstellung: too large a scaling
 * breaks the reconstruction). This runs ozaki2_dgemm_ws with num_moduli
 * moduli and, beside them, the residue product for one redundant check
 * modulus, the next one of the table (so num_moduli <= 19): the integer X the
 * reconstruction returns for each entry must agree with that product modulo
 * the check modulus, and cannot when X was wrapped by j*P, 0 < |j| < p_check.
 * C is written exactly as ozaki2_dgemm_ws writes it.
 *   flags_out DEVICE uint8 [n][m], entry (i, j) at flags_out[j*m + i]:
 *             0 consistent, 1 the CRT range was exceeded (C is wrong there),
 *             2 undecided (|X| within 2^-30 P of P/2, where the check's own
 *             quotient may round either way; the fast and accurate scalings
 *             keep |X| below (P-1)/2 * (1 - 2^-22), far from it).
 *   workspace DEVICE, 256-byte aligned, ozaki2_check_workspace_size(...) bytes.
 * Returns as ozaki2_dgemm_ws; -10 also for num_moduli = 20; -14 flags_out NULL
 * while needed.
 */
int ozaki2_dgemm_check(int64_t m, int64_t n, int64_t k,
                       const double *A, int64_t lda, const double *B, int64_t ldb,
                       double *C, int64_t ldc, int num_moduli, int mode,
                       void *workspace, size_t workspace_bytes, uint8_t *flags_out, void *stream);
/* Bytes of workspace ozaki2_dgemm_check needs (0 for invalid arguments,
 * num_moduli = 20 or empty products). Host-only. */
size_t ozaki2_check_workspace_size(int64_t m, int64_t n, int64_t k, int num_moduli, int mode);

/*
 * Test entry point for the range check alone, on caller residues: as
 * ozaki2_crt_debug with num_moduli + 1 residue planes, the last one for the
 * check modulus (the (num_moduli+1)-th of the table), residues[(l*n + j)*m + i]
 * in [0, p_l). C is reconstructed from the first num_moduli planes; flags_out
 * as for ozaki2_dgemm_check.
 * Returns 0; -1 m < 0, -2 n < 0, -3 num_moduli outside [2, 19], -4 residues,
 * -5 e, -6 f, -7 C or -9 flags_out NULL while needed, -8 ldc < max(1, m),
 * -10 workspace NULL or not 256-byte aligned; OZAKI2_ERR_WORKSPACE if
 * workspace_bytes < ozaki2_check_workspace_size(m, n, 1, num_moduli,
 * OZAKI2_FAST); OZAKI2_ERR_UNSUPPORTED; OZAKI2_ERR_HIP.
 */
int ozaki2_crt_check_debug(int64_t m, int64_t n, int num_moduli, const uint8_t *residues, const int32_t *e,
                           const int32_t *f, double *C, int64_t ldc, uint8_t *flags_out, void *workspace,
                           size_t workspace_bytes, void *stream);

/*
 * Single precision: C := A * B for binary32 A, B, C, emulated by the same
 * steps ([G] section Zentrale Beiträge: the scheme is evaluated for SGEMM as
 * well as DGEMM). The binary32 inputs are widened exactly to doubles, so the
 * exponents, residues and integer products are those ozaki2_dgemm computes
 * for the widened operands; each entry of C is X * 2^-(e_i + f_j) rounded
 * once to binary32 (to nearest, ties to even, subnormals included). 8 moduli
 * give about the accuracy of native binary32 on typical data.
 * Arguments, layouts, status codes and workspace sizes are exactly those of
 * ozaki2_dgemm / ozaki2_dgemm_ws / ozaki2_dgemm_debug (ozaki2_workspace_size
 * and ozaki2_debug_workspace_size apply unchanged), with float in place of
 * double for A, B and C.
 */
int ozaki2_sgemm(int64_t m, int64_t n, int64_t k,
                 const float *A, int64_t lda, const float *B, int64_t ldb,
                 float *C, int64_t ldc, int num_moduli, int mode, void *stream);
int ozaki2_sgemm_ws(int64_t m, int64_t n, int64_t k,
                    const float *A, int64_t lda, const float *B, int64_t ldb,
                    float *C, int64_t ldc, int num_moduli, int mode,
                    void *workspace, size_t workspace_bytes, void *stream);
int ozaki2_sgemm_debug(int64_t m, int64_t n, int64_t k,
                       const float *A, int64_t lda, const float *B, int64_t ldb,
                       float *C, int64_t ldc, int num_moduli, int mode,
                       void *workspace, size_t workspace_bytes,
                       int32_t *e_out, int32_t *f_out, int8_t *resA_out, int8_t *resB_out,
                       int32_t *prod_out, uint8_t *red_out, void *stream);

/*
 * Complex products: C := A * B for double complex (ozaki2_zgemm*) or float
 * complex (ozaki2_cgemm*) matrices, the extension to complex products that
 * [G] names in its closing remark (ZGEMM/CGEMM, future work there).
 * A, B, C hold interleaved (re, im) pairs, column-major, and lda, ldb, ldc
 * count complex elements (element (i, h) of A at A[2*(i + h*lda)] and the next
 * value); other arguments, checks and status codes as ozaki2_dgemm.
 * Row i of A (column j of B) gets one fast-mode exponent from its complex
 * 2-norm sum_h (re^2 + im^2); the parts are truncated separately, and per
 * modulus three INT8 products give T1 = re*re, T2 = im*im and
 * T3 = (re+im)*(re+im), so that Re = T1 - T2 and Im = T3 - T1 - T2 hold
 * exactly in residues (Gauss' three-multiplication form, with no rounding).
 * Each part of C is then the exact integer rounded once, as for real products
 * (binary32 parts for cgemm). Only OZAKI2_FAST is supported: mode
 * OZAKI2_ACCURATE returns OZAKI2_ERR_UNSUPPORTED.
 * Debug copies (zgemm/cgemm _debug) use 3N planes in place of N, plane 3l + g
 * for modulus l and product g (g = 0: re*re, 1: im*im, 2: sums), e.g.
 * resA_out int8 [3N][m][k], red_out uint8 [3N][n][m].
 */
int ozaki2_zgemm(int64_t m, int64_t n, int64_t k,
                 const double *A, int64_t lda, const double *B, int64_t ldb,
                 double *C, int64_t ldc, int num_moduli, int mode, void *stream);
int ozaki2_zgemm_ws(int64_t m, int64_t n, int64_t k,
                    const double *A, int64_t lda, const double *B, int64_t ldb,
                    double *C, int64_t ldc, int num_moduli, int mode,
                    void *workspace, size_t workspace_bytes, void *stream);
int ozaki2_zgemm_debug(int64_t m, int64_t n, int64_t k,
                       const double *A, int64_t lda, const double *B, int64_t ldb,
                       double *C, int64_t ldc, int num_moduli, int mode,
                       void *workspace, size_t workspace_bytes,
                       int32_t *e_out, int32_t *f_out, int8_t *resA_out, int8_t *resB_out,
                       int32_t *prod_out, uint8_t *red_out, void *stream);
int ozaki2_cgemm(int64_t m, int64_t n, int64_t k,
                 const float *A, int64_t lda, const float *B, int64_t ldb,
                 float *C, int64_t ldc, int num_moduli, int mode, void *stream);
int ozaki2_cgemm_ws(int64_t m, int64_t n, int64_t k,
                    const float *A, int64_t lda, const float *B, int64_t ldb,
                    float *C, int64_t ldc, int num_moduli, int mode,
                    void *workspace, size_t workspace_bytes, void *stream);
int ozaki2_cgemm_debug(int64_t m, int64_t n, int64_t k,
                       const float *A, int64_t lda, const float *B, int64_t ldb,
                       float *C, int64_t ldc, int num_moduli, int mode,
                       void *workspace, size_t workspace_bytes,
                       int32_t *e_out, int32_t *f_out, int8_t *resA_out, int8_t *resB_out,
                       int32_t *prod_out, uint8_t *red_out, void *stream);

/*
 * Bytes of device workspace the complex _ws entry points need (debug != 0:
 * the _debug ones); 0 for invalid arguments or empty products. Host-only.
 */
size_t ozaki2_zgemm_workspace_size(int64_t m, int64_t n, int64_t k, int num_moduli, int debug);

/*
 * Test entry point: the complex reconstruction alone, from given residues of
 * the three products per modulus ([Q] step 4 for each part: Re = T1 - T2 and
 * Im = T3 - T1 - T2 in residues, each lifted into (-P/2, P/2], rounded once
 * and scaled by 2^-(e_i + f_j)), on the kernels ozaki2_zgemm uses.
 *   residues DEVICE uint8 [3N][n][m]: T_g mod p_l of entry (i, j) at
 *            residues[((3l + g)*n + j)*m + i], g = 0, 1, 2 for T1, T2, T3,
 *            each in [0, p_l) (not checked);
 *   e, f     DEVICE int32 [m], [n] as for ozaki2_crt_debug;
 *   C, ldc   DEVICE double complex output (interleaved), column-major, ldc in
 *            complex elements;
 *   workspace DEVICE, at least ozaki2_zgemm_workspace_size(m, n, 1, N, 0)
 *            bytes, 256-byte aligned.
 * Returns as ozaki2_crt_debug.
 */
int ozaki2_zcrt_debug(int64_t m, int64_t n, int num_moduli, const uint8_t *residues, const int32_t *e,
                      const int32_t *f, double *C, int64_t ldc, void *workspace, size_t workspace_bytes,
                      void *stream);

/* Workspace bytes for ozaki2_dgemm_debug (larger: raw int32 products). */
size_t ozaki2_debug_workspace_size(int64_t m, int64_t n, int64_t k, int num_moduli, int mode);

/* Largest supported number of moduli (20). */
int ozaki2_max_moduli(void);

/*
 * Writes the first num_moduli moduli into the HOST array out[num_moduli].
 * Returns 0, or -1 if num_moduli is outside [1, 20], -2 if out is NULL.
 */
int ozaki2_moduli(int num_moduli, int32_t *out);

/*
 * Writes to HOST *out the constant P'_prop of [G] section Methodik for N
 * moduli: 0.5 * log2((P - 1) / 2) rounded down to a double, P the product of
 * the moduli. Returns 0, -1 for N outside [2, 20], -2 for out NULL.
 */
int ozaki2_scaling_constant(int num_moduli, double *out);

/*
 * Writes the CRT weight W_l = (P/p_l) * ((P/p_l)^-1 mod p_l) ([Q] section
 * 秦九韶の大衍求一術, the 用数) of modulus l for N moduli into the HOST array
 * out_le32 as little-endian 32-bit limbs (out_limbs entries). Returns the
 * number of limbs used, or a negative argument index.
 */
int ozaki2_crt_weight(int num_moduli, int l, uint32_t *out_le32, int out_limbs);

/* Static text for a status code. */
const char *ozaki2_status_string(int status);

/*
 * Per-phase timing with HIP events on the caller's stream (phases: 0
 * scaling/exponents, 1 residue split, 2 INT8 GEMMs, 3 CRT + unscale). The
 * events are attached to the kernel launches themselves
 * (hipExtLaunchKernelGGL): a phase's start event takes the start time of its
 * first kernel and its stop event the end time of its last one, so timing
 * adds no marker packets between kernels.
 * ozaki2_timing_enable(max_calls, all_phases) creates events for up to
 * max_calls product calls (max_calls <= 0 turns timing off); with
 * all_phases == 0 only phase 2 is timed. ozaki2_timing_read synchronises the
 * events, writes the summed milliseconds per phase to HOST ms_out[4] (0 for
 * untimed phases) and the number of timed calls to *calls, and clears the
 * record.
 * Returns 0 or OZAKI2_ERR_HIP.
 */
int ozaki2_timing_enable(int max_calls, int all_phases);
int ozaki2_timing_read(double *ms_out, int *calls);
/*
 * As ozaki2_timing_read, per call: writes the milliseconds of phase p of
 * timed call c to HOST ms_out[c * 4 + p] (ms_out may be NULL to discard) and
 * clears the record. Returns 0, -2 if max_calls is below the number of timed
 * calls (nothing cleared), or OZAKI2_ERR_HIP.
 */
int ozaki2_timing_read_calls(double *ms_out, int max_calls, int *calls);

/* Frees the cached workspaces, timing events and tables. */
void ozaki2_finalize(void);

#ifdef __cplusplus
}
#endif

#endif /* OZAKI2_H */
