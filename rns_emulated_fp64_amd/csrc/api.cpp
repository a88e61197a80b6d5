// api.cpp -- the C ABI of libozaki2 (declared in include/ozaki2.h): argument
// checks, workspace layout, the order of the phases, per-phase timing.
//
// [Q] = Qiita article "8ビットの整数で53ビットの倍精度を組み立てる。中国剰余定理を
// GPUに載せたOzaki Scheme II"; [G] = "Improved Scaling for Fast Mode of Ozaki
// Scheme II". The phases run in the article's order: powers of two (step 1),
// residues (step 2), one INT8 product per modulus (step 3), reconstruction
// and unscaling (steps 4 and 5); [G] section Methodik gives the fast-mode
// exponents and section Problemstellung the two modes.
#include <hip/hip_runtime.h>

#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "common.h"
#include "ozaki2.h"
#include "tables.h"

namespace oz2 {
namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
int64_t round_up(int64_t v, int64_t g) { return (v + g - 1) / g * g; }

// Checks in signature order; returns 0 or -(index of the first bad argument).
int validate(int64_t m, int64_t n, int64_t k, const void *A, int64_t lda, const void *B, int64_t ldb,
             const void *C, int64_t ldc, int nmod, int mode) {
    if (m < 0) return -1;
    if (n < 0) return -2;
    if (k < 0) return -3;
    if (A == nullptr && m > 0 && k > 0) return -4;
    if (lda < (m > 1 ? m : 1)) return -5;
    if (B == nullptr && k > 0 && n > 0) return -6;
    if (ldb < (k > 1 ? k : 1)) return -7;
    if (C == nullptr && m > 0 && n > 0) return -8;
    if (ldc < (m > 1 ? m : 1)) return -9;
    if (nmod < 2 || nmod > kMaxModuli) return -10;
    if (mode != OZAKI2_FAST && mode != OZAKI2_ACCURATE && mode != OZAKI2_FAST_ORIGINAL) return -11;
    return 0;
}

// Supported sizes: every offset below fits comfortably in 63 bits, the grids
// fit their dimensions, and the integer products stay exact.
bool layout_fits(int64_t m, int64_t n, int64_t k, int mode) {
    const int64_t lim = (int64_t)1 << 31;
    return m < lim && n < lim && k <= (mode == OZAKI2_ACCURATE ? OZAKI2_MAX_K_ACCURATE : OZAKI2_MAX_K);
}

// group: residue planes per modulus, 1 for real products, 3 for complex ones
// (real parts, imaginary parts, their sums).
Layout make_layout(int64_t m, int64_t n, int64_t k, int nmod, int mode, bool debug, int group = 1) {
    Layout L{};
    L.m_pad = round_up(m > 0 ? m : 1, kTileM);
    L.n_pad = round_up(n > 0 ? n : 1, kTileN);
    L.k_pad = round_up(k > 0 ? k : 1, kKPad);
    L.kb = L.k_pad / 32;
    // k-chunks of the row-norm pass (blocks of 64 rows): about 1024 blocks,
    // each thread still streaming at least 32 columns
    const int64_t rowblocks = (m + 63) / 64 > 0 ? (m + 63) / 64 : 1;
    int64_t want = (1024 + rowblocks - 1) / rowblocks;
    int64_t maxc = (k + 127) / 128 > 0 ? (k + 127) / 128 : 1;
    if (want > maxc) want = maxc;
    if (want > 65535) want = 65535;
    if (want < 1) want = 1;
    L.kchunk = (k + want - 1) / want > 0 ? (k + want - 1) / want : 1;
    L.nchunks = (int)((k + L.kchunk - 1) / L.kchunk > 0 ? (k + L.kchunk - 1) / L.kchunk : 1);

    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off = align_up(off + bytes);
        return at;
    };
    const size_t mp = (size_t)L.m_pad, np = (size_t)L.n_pad, kp = (size_t)L.k_pad, mm = (size_t)(m > 0 ? m : 1);
    L.e = take(4 * mp);
    L.f = take(4 * np);
    L.ga = take(4 * mp);
    L.gb = take(4 * np);
    L.part_s = take(8 * (size_t)L.nchunks * mm);
    L.part_g = take(4 * (size_t)L.nchunks * mm);
    L.part_bad = take(4 * (size_t)L.nchunks * mm);
    if (mode == OZAKI2_ACCURATE) {
        L.rowmax = take(4 * mp);
        L.colmax = take(4 * np);
        L.abar = take(mp * kp);
        L.bbar = take(np * kp);
    }
    const size_t planes = (size_t)nmod * group;
    L.ra = take(planes * mp * kp);
    L.rb = take(planes * np * kp);
    L.planes = take(planes * np * mp);
    if (debug) L.raw = take(4 * planes * np * mp);
    L.total = off;
    return L;
}

// ---- timing ---------------------------------------------------------------
// Each call records up to kMaxIntervals intervals (a start and a stop event
// around one or more consecutive launches of one phase); the phase of each
// interval is kept in tag (-1 = unused).
constexpr int kMaxIntervals = 8;
struct Timing {
    std::mutex mu;
    std::vector<hipEvent_t> ev;  // 2 * kMaxIntervals per call
    std::vector<int> tag;        // kMaxIntervals per call
    int max_calls = 0;
    int used = 0;
    bool all_phases = false;  // false: only the GEMM phase is timed
};
Timing g_timing;

void timing_free_locked() {
    for (hipEvent_t e : g_timing.ev) (void)hipEventDestroy(e);
    g_timing.ev.clear();
    g_timing.tag.clear();
    g_timing.max_calls = 0;
    g_timing.used = 0;
}

// Event and tag slots for one call, or nullptrs when timing is off or full;
// all_phases is read under the same lock.
void timing_slots(hipEvent_t **ev, int **tag, bool *all_phases) {
    std::lock_guard<std::mutex> lk(g_timing.mu);
    *ev = nullptr;
    *tag = nullptr;
    *all_phases = g_timing.all_phases;
    if (g_timing.used >= g_timing.max_calls) return;
    const size_t c = (size_t)(g_timing.used++);
    *ev = &g_timing.ev[c * (2 * kMaxIntervals)];
    *tag = &g_timing.tag[c * kMaxIntervals];
}

// ---- cached workspace per device ------------------------------------------
// One workspace per device serves every ozaki2_dgemm/_sgemm/_zgemm/_cgemm call
// on it, whatever the stream. The mutex orders the host side; on the device,
// `done` is recorded on the caller's stream after each product's kernels and
// the next call's stream waits on it first, so products on different streams
// take the workspace one after another instead of overwriting each other.
struct Cache {
    std::mutex mu;
    std::vector<void *> ptr;
    std::vector<size_t> bytes;
    std::vector<hipEvent_t> done;
};
Cache g_cache;

#define HIP_TRY(x)                               \
    do {                                         \
        if ((x) != hipSuccess) return OZAKI2_ERR_HIP; \
    } while (0)

// Steps 3-5 as one launch (k_gemm_crt: all moduli of a 64 x 64 tile per
// block, reconstructed in registers) instead of the 256 x 256 GEMM writing
// residue planes and a reconstruction launch reading them. A fused block runs
// its N moduli one after another, so it wins only where the whole product is
// a few stages long and the saved launch dominates: on MI355X 29 against
// 34 us per product at 64^3 with 8 moduli (16 stages of 64 per block), but
// 47 against 28 us at 256^3 and 14 moduli, and slower at every larger size
// measured. Default: fused for N * (k stages) <= 16 and at most 64 tiles.
// OZ2_FUSED=1 or 0 in the environment forces either form.
bool use_fused(const Layout &L, int64_t m, int64_t n, int nmod) {
    if (const char *force = getenv("OZ2_FUSED")) return strcmp(force, "1") == 0;
    const int64_t tiles = ((m + 63) / 64) * ((n + 63) / 64);
    return (int64_t)nmod * (L.kb / 2) <= 16 && tiles <= 64;
}

struct DebugOut {
    int32_t *e, *f;
    int8_t *ra, *rb;
    int32_t *prod;
    uint8_t *red;
    uint8_t *check;  // CRT-range flags against one redundant modulus (ozaki2_dgemm_check)
};

int run(Elem el, bool cplx, int64_t m, int64_t n, int64_t k, const void *A, int64_t lda, const void *B, int64_t ldb,
        void *C, int64_t ldc, int nmod, int mode, char *ws, const Layout &L, const DebugOut *dbg, hipStream_t s) {
    const Tables *T = get_tables(nmod);
    // with the range check, the residues, products and reduced planes carry one
    // more modulus (the next of the table) than the reconstruction uses
    const bool check = dbg != nullptr && dbg->check != nullptr;
    const Tables *TS = check ? get_tables(nmod + 1) : T;
    const int nsplit = check ? nmod + 1 : nmod;
    // Timing events (start/stop per phase) ride on the first and the last
    // kernel launch of a phase; unless all phases were asked for, only the
    // GEMM phase is timed.
    hipEvent_t *ev = nullptr;
    int *tag = nullptr;
    bool all_phases = false;
    timing_slots(&ev, &tag, &all_phases);
    int nint = 0, open = -1;
    auto ev_of = [&](int phase, bool first, bool last) {
        Ev e;
        if (!ev || !(all_phases || phase == kPhaseGemm)) return e;
        if (first && nint < kMaxIntervals) {
            open = nint++;
            tag[open] = phase;
            e.start = ev[2 * open];
        }
        if (last && open >= 0) {
            e.stop = ev[2 * open + 1];
            open = -1;
        }
        return e;
    };
    const bool accurate = mode == OZAKI2_ACCURATE;

    // Step 1: squared norms of the rows of A and exponents of the columns of
    // B ([G] Methodik), one launch.
    const int group = cplx ? 3 : 1;
    const bool original = mode == OZAKI2_FAST_ORIGINAL;
    HIP_TRY(launch_scale(el, cplx, original, A, m, k, lda, B, n, ldb, T->Pp, L, ws, s,
                         ev_of(kPhaseScale, true, !accurate)));
    if (accurate) {
        // Accurate mode bounds the products with one extra INT8 GEMM first
        // ([G] Problemstellung).
        HIP_TRY(launch_row_exponents(m, T->Pp, L, ws, s));  // also clears the row/column maxima
        HIP_TRY(launch_quantize(el, A, m, lda, B, n, ldb, k, L, ws, s));
        HIP_TRY(launch_gemm_bound((const int8_t *)(ws + L.abar), (const int8_t *)(ws + L.bbar),
                                  (int32_t *)(ws + L.rowmax), (int32_t *)(ws + L.colmax), L, s));
        HIP_TRY(launch_accurate_exponents(m, n, T->Pp, L, ws, s, ev_of(kPhaseScale, false, true)));
    }

    // Steps 1 + 2: integerize and split both operands into residues, one
    // launch (in fast mode it also finishes the row exponents of A).
    HIP_TRY(launch_split(el, cplx, original, A, m, lda, B, n, ldb, k, !accurate, T->Pp, TS->split, L, ws, s,
                         ev_of(kPhaseSplit, true, true)));
    const int32_t *e = (const int32_t *)(ws + L.e), *f = (const int32_t *)(ws + L.f);

    if (!cplx && dbg == nullptr && use_fused(L, m, n, nmod) && gemm_crt_applies(L, m, n)) {
        // Steps 3-5 in one launch: every modulus of a tile, reconstructed in registers.
        HIP_TRY(launch_gemm_crt(el, (const int8_t *)(ws + L.ra), (const int8_t *)(ws + L.rb), m, n, e, f, T->crt,
                                T->mod, C, ldc, L, s, ev_of(kPhaseGemm, true, true)));
        return OZAKI2_SUCCESS;
    }

    // Step 3: one exact INT8 product per modulus, reduced mod p_l.
    HIP_TRY(launch_gemm_mod((const int8_t *)(ws + L.ra), (const int8_t *)(ws + L.rb), nsplit, group, TS->mod,
                            (int8_t *)(ws + L.planes), L, s, ev_of(kPhaseGemm, true, true)));

    // Steps 4 + 5: reconstruction and unscaling.
    if (cplx)
        HIP_TRY(launch_crt_complex(el, (const int8_t *)(ws + L.planes), m, n, e, f, T->crt, T->mod, C, ldc, L, s,
                                   ev_of(kPhaseCrt, true, true)));
    else
        HIP_TRY(launch_crt(el, (const int8_t *)(ws + L.planes), m, n, e, f, T->crt, C, ldc, L, s,
                           ev_of(kPhaseCrt, true, true)));

    if (check) HIP_TRY(launch_crt_check((const int8_t *)(ws + L.planes), m, n, T->check, L, dbg->check, s));

    if (dbg) {
        if (dbg->e) HIP_TRY(hipMemcpyAsync(dbg->e, e, 4 * (size_t)m, hipMemcpyDeviceToDevice, s));
        if (dbg->f) HIP_TRY(hipMemcpyAsync(dbg->f, f, 4 * (size_t)n, hipMemcpyDeviceToDevice, s));
        if (dbg->ra)
            HIP_TRY(launch_unpack_residues((const int8_t *)(ws + L.ra), nmod * group, m, k, L.m_pad, L, dbg->ra, s));
        if (dbg->rb)
            HIP_TRY(launch_unpack_residues((const int8_t *)(ws + L.rb), nmod * group, n, k, L.n_pad, L, dbg->rb, s));
        if (dbg->red)
            HIP_TRY(launch_copy_planes_u8((const int8_t *)(ws + L.planes), nmod, group, T->mod, m, n, L, dbg->red,
                                          s));
        if (dbg->prod) {
            HIP_TRY(launch_gemm_raw((const int8_t *)(ws + L.ra), (const int8_t *)(ws + L.rb), nmod, group,
                                    (int32_t *)(ws + L.raw), L, s));
            HIP_TRY(launch_copy_planes_i32((const int32_t *)(ws + L.raw), nmod * group, m, n, L, dbg->prod, s));
        }
    }
    return OZAKI2_SUCCESS;
}

// Common front end of the product entry points.
int front(Elem el, bool cplx, int64_t m, int64_t n, int64_t k, const void *A, int64_t lda, const void *B,
          int64_t ldb, void *C, int64_t ldc, int nmod, int mode, void *workspace, size_t wbytes, bool use_cache,
          const DebugOut *dbg, void *stream) {
    int st = validate(m, n, k, A, lda, B, ldb, C, ldc, nmod, mode);
    if (st) return st;
    if (!layout_fits(m, n, k, mode)) return OZAKI2_ERR_UNSUPPORTED;
    if (cplx && mode != OZAKI2_FAST) return OZAKI2_ERR_UNSUPPORTED;
    if (dbg && dbg->prod && k >= (1 << 17)) return OZAKI2_ERR_UNSUPPORTED;
    hipStream_t s = (hipStream_t)stream;
    if (m == 0 || n == 0) return OZAKI2_SUCCESS;
    if (k == 0) {
        // a complex column is 2m values with stride 2*ldc
        HIP_TRY(launch_zero_fill(el, C, cplx ? 2 * m : m, n, cplx ? 2 * ldc : ldc, s));
        return OZAKI2_SUCCESS;
    }
    const bool check = dbg != nullptr && dbg->check != nullptr;
    const Layout L = make_layout(m, n, k, check ? nmod + 1 : nmod, mode, dbg != nullptr && !check, cplx ? 3 : 1);
    if (!use_cache) {
        if (workspace == nullptr || ((uintptr_t)workspace & (kAlign - 1)) != 0) return -12;
        if (wbytes < L.total) return OZAKI2_ERR_WORKSPACE;
        return run(el, cplx, m, n, k, A, lda, B, ldb, C, ldc, nmod, mode, (char *)workspace, L, dbg, s);
    }
    int dev = 0;
    HIP_TRY(hipGetDevice(&dev));
    std::lock_guard<std::mutex> lk(g_cache.mu);
    if ((int)g_cache.ptr.size() <= dev) {
        g_cache.ptr.resize(dev + 1, nullptr);
        g_cache.bytes.resize(dev + 1, 0);
        g_cache.done.resize(dev + 1, nullptr);
    }
    if (g_cache.done[dev] == nullptr) {
        HIP_TRY(hipEventCreateWithFlags(&g_cache.done[dev], hipEventDisableTiming));
    } else {
        // the previous cached product, on whatever stream, is done with the workspace
        HIP_TRY(hipStreamWaitEvent(s, g_cache.done[dev], 0));
    }
    if (g_cache.bytes[dev] < L.total) {
        if (g_cache.ptr[dev]) {
            HIP_TRY(hipDeviceSynchronize());
            (void)hipFree(g_cache.ptr[dev]);
            g_cache.ptr[dev] = nullptr;
            g_cache.bytes[dev] = 0;
        }
        void *p = nullptr;
        if (hipMalloc(&p, L.total) != hipSuccess) return OZAKI2_ERR_WORKSPACE;
        g_cache.ptr[dev] = p;
        g_cache.bytes[dev] = L.total;
    }
    const int rc = run(el, cplx, m, n, k, A, lda, B, ldb, C, ldc, nmod, mode, (char *)g_cache.ptr[dev], L, dbg, s);
    HIP_TRY(hipEventRecord(g_cache.done[dev], s));
    return rc;
}

}  // namespace

int product_ws(Elem el, int64_t m, int64_t n, int64_t k, const void *A, int64_t lda, const void *B, int64_t ldb,
               void *C, int64_t ldc, int nmod, int mode, void *workspace, size_t wbytes, void *stream) {
    return front(el, false, m, n, k, A, lda, B, ldb, C, ldc, nmod, mode, workspace, wbytes, false, nullptr, stream);
}

}  // namespace oz2

using namespace oz2;

extern "C" {

int ozaki2_dgemm(int64_t m, int64_t n, int64_t k, const double *A, int64_t lda, const double *B, int64_t ldb,
                 double *C, int64_t ldc, int num_moduli, int mode, void *stream) {
    return front(Elem::f64, false, m, n, k, A, lda, B, ldb, C, ldc, num_moduli, mode, nullptr, 0, true, nullptr,
                 stream);
}

size_t ozaki2_workspace_size(int64_t m, int64_t n, int64_t k, int num_moduli, int mode) {
    if (validate(m, n, k, (const double *)1, m > 1 ? m : 1, (const double *)1, k > 1 ? k : 1, (const double *)1,
                 m > 1 ? m : 1, num_moduli, mode))
        return 0;
    if (!layout_fits(m, n, k, mode) || m == 0 || n == 0 || k == 0) return 0;
    return make_layout(m, n, k, num_moduli, mode, false).total;
}

size_t ozaki2_debug_workspace_size(int64_t m, int64_t n, int64_t k, int num_moduli, int mode) {
    if (validate(m, n, k, (const double *)1, m > 1 ? m : 1, (const double *)1, k > 1 ? k : 1, (const double *)1,
                 m > 1 ? m : 1, num_moduli, mode))
        return 0;
    if (!layout_fits(m, n, k, mode) || m == 0 || n == 0 || k == 0) return 0;
    return make_layout(m, n, k, num_moduli, mode, true).total;
}

int ozaki2_dgemm_ws(int64_t m, int64_t n, int64_t k, const double *A, int64_t lda, const double *B, int64_t ldb,
                    double *C, int64_t ldc, int num_moduli, int mode, void *workspace, size_t workspace_bytes,
                    void *stream) {
    return front(Elem::f64, false, m, n, k, A, lda, B, ldb, C, ldc, num_moduli, mode, workspace, workspace_bytes,
                 false, nullptr, stream);
}

int ozaki2_dgemm_debug(int64_t m, int64_t n, int64_t k, const double *A, int64_t lda, const double *B, int64_t ldb,
                       double *C, int64_t ldc, int num_moduli, int mode, void *workspace, size_t workspace_bytes,
                       int32_t *e_out, int32_t *f_out, int8_t *resA_out, int8_t *resB_out, int32_t *prod_out,
                       uint8_t *red_out, void *stream) {
    DebugOut d{e_out, f_out, resA_out, resB_out, prod_out, red_out, nullptr};
    return front(Elem::f64, false, m, n, k, A, lda, B, ldb, C, ldc, num_moduli, mode, workspace, workspace_bytes,
                 false, &d, stream);
}

int ozaki2_sgemm(int64_t m, int64_t n, int64_t k, const float *A, int64_t lda, const float *B, int64_t ldb,
                 float *C, int64_t ldc, int num_moduli, int mode, void *stream) {
    return front(Elem::f32, false, m, n, k, A, lda, B, ldb, C, ldc, num_moduli, mode, nullptr, 0, true, nullptr,
                 stream);
}

int ozaki2_sgemm_ws(int64_t m, int64_t n, int64_t k, const float *A, int64_t lda, const float *B, int64_t ldb,
                    float *C, int64_t ldc, int num_moduli, int mode, void *workspace, size_t workspace_bytes,
                    void *stream) {
    return front(Elem::f32, false, m, n, k, A, lda, B, ldb, C, ldc, num_moduli, mode, workspace, workspace_bytes,
                 false, nullptr, stream);
}

int ozaki2_sgemm_debug(int64_t m, int64_t n, int64_t k, const float *A, int64_t lda, const float *B, int64_t ldb,
                       float *C, int64_t ldc, int num_moduli, int mode, void *workspace, size_t workspace_bytes,
                       int32_t *e_out, int32_t *f_out, int8_t *resA_out, int8_t *resB_out, int32_t *prod_out,
                       uint8_t *red_out, void *stream) {
    DebugOut d{e_out, f_out, resA_out, resB_out, prod_out, red_out, nullptr};
    return front(Elem::f32, false, m, n, k, A, lda, B, ldb, C, ldc, num_moduli, mode, workspace, workspace_bytes,
                 false, &d, stream);
}

int ozaki2_crt_debug(int64_t m, int64_t n, int num_moduli, const uint8_t *residues, const int32_t *e,
                     const int32_t *f, double *C, int64_t ldc, void *workspace, size_t workspace_bytes,
                     void *stream) {
    if (m < 0) return -1;
    if (n < 0) return -2;
    if (num_moduli < 2 || num_moduli > kMaxModuli) return -3;
    const bool any = m > 0 && n > 0;
    if (residues == nullptr && any) return -4;
    if (e == nullptr && any) return -5;
    if (f == nullptr && any) return -6;
    if (C == nullptr && any) return -7;
    if (ldc < (m > 1 ? m : 1)) return -8;
    if (!any) return OZAKI2_SUCCESS;
    if (workspace == nullptr || ((uintptr_t)workspace & (kAlign - 1)) != 0) return -9;
    if (!layout_fits(m, n, 1, OZAKI2_FAST)) return OZAKI2_ERR_UNSUPPORTED;
    const Layout L = make_layout(m, n, 1, num_moduli, OZAKI2_FAST, false);
    if (workspace_bytes < L.total) return OZAKI2_ERR_WORKSPACE;
    const Tables *T = get_tables(num_moduli);
    hipStream_t s = (hipStream_t)stream;
    int8_t *planes = (int8_t *)((char *)workspace + L.planes);
    HIP_TRY(launch_pack_planes(residues, num_moduli, 1, T->mod, m, n, L, planes, s));
    HIP_TRY(launch_crt(Elem::f64, planes, m, n, e, f, T->crt, C, ldc, L, s));
    return OZAKI2_SUCCESS;
}

size_t ozaki2_check_workspace_size(int64_t m, int64_t n, int64_t k, int num_moduli, int mode) {
    if (num_moduli >= kMaxModuli) return 0;
    if (validate(m, n, k, (const double *)1, m > 1 ? m : 1, (const double *)1, k > 1 ? k : 1, (const double *)1,
                 m > 1 ? m : 1, num_moduli, mode))
        return 0;
    if (!layout_fits(m, n, k, mode) || m == 0 || n == 0 || k == 0) return 0;
    return make_layout(m, n, k, num_moduli + 1, mode, false).total;
}

int ozaki2_dgemm_check(int64_t m, int64_t n, int64_t k, const double *A, int64_t lda, const double *B, int64_t ldb,
                       double *C, int64_t ldc, int num_moduli, int mode, void *workspace, size_t workspace_bytes,
                       uint8_t *flags_out, void *stream) {
    int st = validate(m, n, k, A, lda, B, ldb, C, ldc, num_moduli, mode);
    if (st) return st;
    if (num_moduli >= kMaxModuli) return -10;  // the check modulus is the next one of the table
    if (flags_out == nullptr && m > 0 && n > 0) return -14;
    if (k == 0 && m > 0 && n > 0) {
        // C = 0 exactly: nothing to reconstruct, every entry consistent
        HIP_TRY(launch_zero_fill(Elem::f64, C, m, n, ldc, (hipStream_t)stream));
        HIP_TRY(hipMemsetAsync(flags_out, 0, (size_t)m * (size_t)n, (hipStream_t)stream));
        return OZAKI2_SUCCESS;
    }
    DebugOut d{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, flags_out};
    return front(Elem::f64, false, m, n, k, A, lda, B, ldb, C, ldc, num_moduli, mode, workspace, workspace_bytes,
                 false, &d, stream);
}

int ozaki2_crt_check_debug(int64_t m, int64_t n, int num_moduli, const uint8_t *residues, const int32_t *e,
                           const int32_t *f, double *C, int64_t ldc, uint8_t *flags_out, void *workspace,
                           size_t workspace_bytes, void *stream) {
    if (m < 0) return -1;
    if (n < 0) return -2;
    if (num_moduli < 2 || num_moduli >= kMaxModuli) return -3;
    const bool any = m > 0 && n > 0;
    if (residues == nullptr && any) return -4;
    if (e == nullptr && any) return -5;
    if (f == nullptr && any) return -6;
    if (C == nullptr && any) return -7;
    if (ldc < (m > 1 ? m : 1)) return -8;
    if (flags_out == nullptr && any) return -9;
    if (!any) return OZAKI2_SUCCESS;
    if (workspace == nullptr || ((uintptr_t)workspace & (kAlign - 1)) != 0) return -10;
    if (!layout_fits(m, n, 1, OZAKI2_FAST)) return OZAKI2_ERR_UNSUPPORTED;
    const Layout L = make_layout(m, n, 1, num_moduli + 1, OZAKI2_FAST, false);
    if (workspace_bytes < L.total) return OZAKI2_ERR_WORKSPACE;
    const Tables *T = get_tables(num_moduli);
    const Tables *TS = get_tables(num_moduli + 1);
    hipStream_t s = (hipStream_t)stream;
    int8_t *planes = (int8_t *)((char *)workspace + L.planes);
    HIP_TRY(launch_pack_planes(residues, num_moduli + 1, 1, TS->mod, m, n, L, planes, s));
    HIP_TRY(launch_crt(Elem::f64, planes, m, n, e, f, T->crt, C, ldc, L, s));
    HIP_TRY(launch_crt_check(planes, m, n, T->check, L, flags_out, s));
    return OZAKI2_SUCCESS;
}

int ozaki2_zgemm(int64_t m, int64_t n, int64_t k, const double *A, int64_t lda, const double *B, int64_t ldb,
                 double *C, int64_t ldc, int num_moduli, int mode, void *stream) {
    return front(Elem::f64, true, m, n, k, A, lda, B, ldb, C, ldc, num_moduli, mode, nullptr, 0, true, nullptr,
                 stream);
}

int ozaki2_zgemm_ws(int64_t m, int64_t n, int64_t k, const double *A, int64_t lda, const double *B, int64_t ldb,
                    double *C, int64_t ldc, int num_moduli, int mode, void *workspace, size_t workspace_bytes,
                    void *stream) {
    return front(Elem::f64, true, m, n, k, A, lda, B, ldb, C, ldc, num_moduli, mode, workspace, workspace_bytes,
                 false, nullptr, stream);
}

int ozaki2_zgemm_debug(int64_t m, int64_t n, int64_t k, const double *A, int64_t lda, const double *B, int64_t ldb,
                       double *C, int64_t ldc, int num_moduli, int mode, void *workspace, size_t workspace_bytes,
                       int32_t *e_out, int32_t *f_out, int8_t *resA_out, int8_t *resB_out, int32_t *prod_out,
                       uint8_t *red_out, void *stream) {
    DebugOut d{e_out, f_out, resA_out, resB_out, prod_out, red_out, nullptr};
    return front(Elem::f64, true, m, n, k, A, lda, B, ldb, C, ldc, num_moduli, mode, workspace, workspace_bytes,
                 false, &d, stream);
}

int ozaki2_cgemm(int64_t m, int64_t n, int64_t k, const float *A, int64_t lda, const float *B, int64_t ldb,
                 float *C, int64_t ldc, int num_moduli, int mode, void *stream) {
    return front(Elem::f32, true, m, n, k, A, lda, B, ldb, C, ldc, num_moduli, mode, nullptr, 0, true, nullptr,
                 stream);
}

int ozaki2_cgemm_ws(int64_t m, int64_t n, int64_t k, const float *A, int64_t lda, const float *B, int64_t ldb,
                    float *C, int64_t ldc, int num_moduli, int mode, void *workspace, size_t workspace_bytes,
                    void *stream) {
    return front(Elem::f32, true, m, n, k, A, lda, B, ldb, C, ldc, num_moduli, mode, workspace, workspace_bytes,
                 false, nullptr, stream);
}

int ozaki2_cgemm_debug(int64_t m, int64_t n, int64_t k, const float *A, int64_t lda, const float *B, int64_t ldb,
                       float *C, int64_t ldc, int num_moduli, int mode, void *workspace, size_t workspace_bytes,
                       int32_t *e_out, int32_t *f_out, int8_t *resA_out, int8_t *resB_out, int32_t *prod_out,
                       uint8_t *red_out, void *stream) {
    DebugOut d{e_out, f_out, resA_out, resB_out, prod_out, red_out, nullptr};
    return front(Elem::f32, true, m, n, k, A, lda, B, ldb, C, ldc, num_moduli, mode, workspace, workspace_bytes,
                 false, &d, stream);
}

size_t ozaki2_zgemm_workspace_size(int64_t m, int64_t n, int64_t k, int num_moduli, int debug) {
    if (validate(m, n, k, (const double *)1, m > 1 ? m : 1, (const double *)1, k > 1 ? k : 1, (const double *)1,
                 m > 1 ? m : 1, num_moduli, OZAKI2_FAST))
        return 0;
    if (!layout_fits(m, n, k, OZAKI2_FAST) || m == 0 || n == 0 || k == 0) return 0;
    return make_layout(m, n, k, num_moduli, OZAKI2_FAST, debug != 0, 3).total;
}

int ozaki2_zcrt_debug(int64_t m, int64_t n, int num_moduli, const uint8_t *residues, const int32_t *e,
                      const int32_t *f, double *C, int64_t ldc, void *workspace, size_t workspace_bytes,
                      void *stream) {
    if (m < 0) return -1;
    if (n < 0) return -2;
    if (num_moduli < 2 || num_moduli > kMaxModuli) return -3;
    const bool any = m > 0 && n > 0;
    if (residues == nullptr && any) return -4;
    if (e == nullptr && any) return -5;
    if (f == nullptr && any) return -6;
    if (C == nullptr && any) return -7;
    if (ldc < (m > 1 ? m : 1)) return -8;
    if (!any) return OZAKI2_SUCCESS;
    if (workspace == nullptr || ((uintptr_t)workspace & (kAlign - 1)) != 0) return -9;
    if (!layout_fits(m, n, 1, OZAKI2_FAST)) return OZAKI2_ERR_UNSUPPORTED;
    const Layout L = make_layout(m, n, 1, num_moduli, OZAKI2_FAST, false, 3);
    if (workspace_bytes < L.total) return OZAKI2_ERR_WORKSPACE;
    const Tables *T = get_tables(num_moduli);
    hipStream_t s = (hipStream_t)stream;
    int8_t *planes = (int8_t *)((char *)workspace + L.planes);
    HIP_TRY(launch_pack_planes(residues, 3 * num_moduli, 3, T->mod, m, n, L, planes, s));
    HIP_TRY(launch_crt_complex(Elem::f64, planes, m, n, e, f, T->crt, T->mod, C, ldc, L, s, Ev{}));
    return OZAKI2_SUCCESS;
}

int ozaki2_max_moduli(void) { return kMaxModuli; }

int ozaki2_moduli(int num_moduli, int32_t *out) {
    if (num_moduli < 1 || num_moduli > kMaxModuli) return -1;
    if (out == nullptr) return -2;
    greedy_moduli(num_moduli, out);
    return 0;
}

int ozaki2_scaling_constant(int num_moduli, double *out) {
    if (num_moduli < 2 || num_moduli > kMaxModuli) return -1;
    if (out == nullptr) return -2;
    *out = get_tables(num_moduli)->Pp;
    return 0;
}

int ozaki2_crt_weight(int num_moduli, int l, uint32_t *out_le32, int out_limbs) {
    if (num_moduli < 2 || num_moduli > kMaxModuli) return -1;
    if (l < 0 || l >= num_moduli) return -2;
    if (out_le32 == nullptr) return -3;
    const Tables *T = get_tables(num_moduli);
    if (out_limbs < T->weight_limbs) return -4;
    for (int i = 0; i < out_limbs; ++i) out_le32[i] = i < 8 ? T->weight[l][i] : 0u;
    return T->weight_limbs;
}

const char *ozaki2_status_string(int status) {
    switch (status) {
    case OZAKI2_SUCCESS: return "success";
    case OZAKI2_ERR_HIP: return "HIP runtime or kernel launch error";
    case OZAKI2_ERR_WORKSPACE: return "workspace too small or allocation failed";
    case OZAKI2_ERR_NOALLOC_LIMIT:
        return "product needs more workspace than the static scratch of ozaki2_dgemm_noalloc "
               "(OZAKI2_NOALLOC_MAX_WORKSPACE bytes); use ozaki2_dgemm_ws";
    case OZAKI2_ERR_UNSUPPORTED:
        return "unsupported size (k <= 2^22 - 1, or 2^19 - 1 in accurate mode; m, n < 2^31; raw products need k < 2^17)";
    default: break;
    }
    if (status < 0) return "invalid argument (status is minus its 1-based position)";
    return "unknown status";
}

int ozaki2_timing_enable(int max_calls, int all_phases) {
    std::lock_guard<std::mutex> lk(g_timing.mu);
    timing_free_locked();
    g_timing.all_phases = all_phases != 0;
    if (max_calls <= 0) return OZAKI2_SUCCESS;
    g_timing.ev.resize((size_t)max_calls * (2 * kMaxIntervals), nullptr);
    g_timing.tag.assign((size_t)max_calls * kMaxIntervals, -1);
    // The events only measure time (nothing waits on them to read memory), so
    // they skip the system-scope fence that would flush the caches around the
    // timed kernels.
    for (hipEvent_t &e : g_timing.ev) {
        if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) {
            e = nullptr;
            timing_free_locked();
            return OZAKI2_ERR_HIP;
        }
    }
    g_timing.max_calls = max_calls;
    g_timing.used = 0;
    return OZAKI2_SUCCESS;
}

int ozaki2_timing_read_calls(double *ms_out, int max_calls, int *calls) {
    std::lock_guard<std::mutex> lk(g_timing.mu);
    const int used = g_timing.used;
    if (ms_out && max_calls < used) return -2;
    for (int c = 0; c < used; ++c) {
        hipEvent_t *ev = &g_timing.ev[(size_t)c * (2 * kMaxIntervals)];
        int *tag = &g_timing.tag[(size_t)c * kMaxIntervals];
        double acc[kNumPhases] = {0, 0, 0, 0};
        for (int t = 0; t < kMaxIntervals; ++t) {
            if (tag[t] < 0) continue;
            if (hipEventSynchronize(ev[2 * t + 1]) != hipSuccess) return OZAKI2_ERR_HIP;
            float ms = 0.f;
            if (hipEventElapsedTime(&ms, ev[2 * t], ev[2 * t + 1]) != hipSuccess) return OZAKI2_ERR_HIP;
            acc[tag[t]] += ms;
            tag[t] = -1;
        }
        if (ms_out)
            for (int p = 0; p < kNumPhases; ++p) ms_out[(size_t)c * kNumPhases + p] = acc[p];
    }
    if (calls) *calls = used;
    g_timing.used = 0;
    return OZAKI2_SUCCESS;
}

int ozaki2_timing_read(double *ms_out, int *calls) {
    int used = 0;
    {
        std::lock_guard<std::mutex> lk(g_timing.mu);
        used = g_timing.used;
    }
    std::vector<double> per((size_t)(used > 0 ? used : 1) * kNumPhases, 0.0);
    const int st = ozaki2_timing_read_calls(per.data(), used, &used);
    if (st != OZAKI2_SUCCESS) return st;
    if (ms_out) {
        for (int p = 0; p < kNumPhases; ++p) {
            double sum = 0.0;
            for (int c = 0; c < used; ++c) sum += per[(size_t)c * kNumPhases + p];
            ms_out[p] = sum;
        }
    }
    if (calls) *calls = used;
    return OZAKI2_SUCCESS;
}

void ozaki2_finalize(void) {
    {
        std::lock_guard<std::mutex> lk(g_cache.mu);
        int cur = 0;
        (void)hipGetDevice(&cur);
        for (size_t d = 0; d < g_cache.ptr.size(); ++d) {
            if (g_cache.ptr[d] || g_cache.done[d]) {
                (void)hipSetDevice((int)d);
                (void)hipDeviceSynchronize();
                if (g_cache.ptr[d]) (void)hipFree(g_cache.ptr[d]);
                if (g_cache.done[d]) (void)hipEventDestroy(g_cache.done[d]);
            }
        }
        (void)hipSetDevice(cur);
        g_cache.ptr.clear();
        g_cache.bytes.clear();
        g_cache.done.clear();
    }
    std::lock_guard<std::mutex> lk(g_timing.mu);
    timing_free_locked();
}

}  // extern "C"
