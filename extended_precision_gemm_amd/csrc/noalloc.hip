// The double-double product for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc): dd_gemm_ws run on a workspace that the library holds itself, a
// file-scope device array of DDGEMM_NOALLOC_SCRATCH_BYTES bytes.  Every GPU the
// library runs on has its own copy at its own address, kept until the process
// ends; all calls on that GPU share it (see include/ddgemm.h).
#include <mutex>

#include "common.hpp"

using namespace ddg;

namespace {

// In host code `scratch` names a host-side stand-in, not device memory: every
// host use goes through the device address looked up below.
__device__ __align__(256) unsigned char scratch[DDGEMM_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device (guarded)

// The current device's copy of `scratch`: looked up once per device, with that
// device current, and kept.
ddgemm_status_t current_scratch(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DDGEMM_ERROR_DEVICE;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return DDGEMM_ERROR_LAUNCH;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return DDGEMM_SUCCESS;
}

}  // namespace

extern "C" ddgemm_status_t dd_gemm_noalloc(int64_t m, int64_t n, int64_t k, const double* A_hi, const double* A_lo,
                                           int64_t lda, const double* B_hi, const double* B_lo, int64_t ldb,
                                           double* C_hi, double* C_lo, int64_t ldc, void* stream) {
    if (k < 0) return DDGEMM_ERROR_INVALID_VALUE;
    const ProductCheck chk = check_dd_product(m, n, k, kSlices, default_kblock(k, kSlices), A_hi, A_lo, lda, B_hi,
                                              B_lo, ldb, C_hi, C_lo, ldc);
    if (chk.status != DDGEMM_SUCCESS || chk.empty) return chk.status;
    if (chk.need > DDGEMM_NOALLOC_SCRATCH_BYTES) return DDGEMM_ERROR_WORKSPACE;
    ddgemm_status_t st = check_current_device();
    if (st != DDGEMM_SUCCESS) return st;
    void* ws = nullptr;
    if ((st = current_scratch(&ws)) != DDGEMM_SUCCESS) return st;
    return dd_gemm_ws(m, n, k, A_hi, A_lo, lda, B_hi, B_lo, ldb, C_hi, C_lo, ldc, ws, DDGEMM_NOALLOC_SCRATCH_BYTES,
                      stream);
}
