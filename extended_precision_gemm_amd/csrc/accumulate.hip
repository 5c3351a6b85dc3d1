// Sum of k-block products: C += T in double-double arithmetic, elementwise.
//
// §2 eq. (5) of "Multiple Double Arithmetic on NVIDIA Tensor Cores" bounds how
// many slice products one level sum may hold exactly, so a longer inner
// dimension is cut into blocks, each a separate sliced product; the block
// results are added here with the accurate double-word addition.  HBM-bound:
// 32 B read + 16 B written per output.
#include "common.hpp"
#include "eft.hpp"

namespace ddg {
namespace {

__global__ void __launch_bounds__(256) dd_accumulate_kernel(int64_t m, int64_t n, double* __restrict__ C_hi,
                                                            double* __restrict__ C_lo, int64_t ldc,
                                                            const double* __restrict__ T_hi,
                                                            const double* __restrict__ T_lo, int64_t ldt) {
    const int64_t col = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (col >= n) return;
    for (int64_t row = blockIdx.y; row < m; row += gridDim.y) {
        double zh, zl;
        dd_add(C_hi[row * ldc + col], C_lo[row * ldc + col], T_hi[row * ldt + col], T_lo[row * ldt + col], zh, zl);
        C_hi[row * ldc + col] = zh;
        C_lo[row * ldc + col] = zl;
    }
}

}  // namespace

hipError_t launch_dd_accumulate(int64_t m, int64_t n, double* C_hi, double* C_lo, int64_t ldc, const double* T_hi,
                                const double* T_lo, int64_t ldt, hipStream_t stream) {
    if (m == 0 || n == 0) return hipSuccess;
    const int64_t gy = m < 65535 ? m : 65535;
    dim3 grid(static_cast<unsigned>((n + 255) / 256), static_cast<unsigned>(gy));
    dd_accumulate_kernel<<<grid, 256, 0, stream>>>(m, n, C_hi, C_lo, ldc, T_hi, T_lo, ldt);
    return hipGetLastError();
}

}  // namespace ddg
