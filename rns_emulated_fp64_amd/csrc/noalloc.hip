// noalloc.hip -- ozaki2_dgemm_noalloc: the FP64 product of ozaki2_dgemm_ws
// with its workspace in a static device array instead of a caller or library
// allocation, for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The array lives in this file as a file-scope __device__ variable: every GPU
// the library runs on holds its own copy, kNoallocScratchBytes long, from the
// moment the library's code object is loaded on it until the process ends.
// In host code the name `scratch` is a host-side stand-in, not a device
// address, so host code never passes it anywhere: the device address is
// looked up once per device with hipGetSymbolAddress (with that device
// current) and kept, and only that address reaches the kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "common.h"
#include "ozaki2.h"

namespace oz2 {
namespace {

constexpr size_t kNoallocScratchBytes = (size_t)OZAKI2_NOALLOC_MAX_WORKSPACE;
static_assert(kNoallocScratchBytes % 256 == 0, "whole 256-byte granules");

__device__ __align__(256) char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch[kMaxDevices] = {};  // device address of `scratch` on each device

// Device address of this device's `scratch`, looked up on the first call on
// the device. Returns 0 or OZAKI2_ERR_HIP.
int scratch_address(void **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return OZAKI2_ERR_HIP;
    std::lock_guard<std::mutex> lk(g_mu);
    if (g_scratch[dev] == nullptr) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return OZAKI2_ERR_HIP;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return OZAKI2_SUCCESS;
}

}  // namespace
}  // namespace oz2

extern "C" int ozaki2_dgemm_noalloc(int64_t m, int64_t n, int64_t k, const double *A, int64_t lda, const double *B,
                                    int64_t ldb, double *C, int64_t ldc, int num_moduli, int mode, void *stream) {
    // invalid arguments, unsupported sizes and empty products need no
    // workspace: the common entry reports or handles them before any use of it
    const size_t need = ozaki2_workspace_size(m, n, k, num_moduli, mode);
    if (need == 0)
        return oz2::product_ws(oz2::Elem::f64, m, n, k, A, lda, B, ldb, C, ldc, num_moduli, mode, nullptr, 0, stream);
    if (need > oz2::kNoallocScratchBytes) return OZAKI2_ERR_NOALLOC_LIMIT;
    void *ws = nullptr;
    const int rc = oz2::scratch_address(&ws);
    if (rc != OZAKI2_SUCCESS) return rc;
    return oz2::product_ws(oz2::Elem::f64, m, n, k, A, lda, B, ldb, C, ldc, num_moduli, mode, ws,
                           oz2::kNoallocScratchBytes, stream);
}
