// Level planes -> results, and the helpers of a product split over k: the
// double-double cascade of NS level sums ("Multiple Double Arithmetic on NVIDIA
// Tensor Cores", §2 fifth step; Problem 1.1), the exact four-double rounding of
// sixteen, zeroing the planes a split product adds into, and moving a split
// k-block's level sums into the int64 planes of a blocked quad-double product.
#include "common.hpp"
#include "dispatch_ns.hpp"
#include "eft.hpp"
#include "pair_levels.hpp"
#include "qd_levels.hpp"

namespace ddg {
namespace {

// Cascade the NS level sums of each output entry into (hi, lo), one column
// per thread, the rows blockIdx.y, blockIdx.y + gridDim.y, ...; TWO: two rows
// per step, their loads issued together.  The level planes are read once and
// the results not read again here, so both go past the caches (non-temporal).
template <int NS, bool TWO>
__global__ void __launch_bounds__(256) renorm_kernel(int64_t m, int64_t n, const double* __restrict__ levels,
                                                     int64_t ldl, int64_t plane, const int32_t* __restrict__ E,
                                                     const int32_t* __restrict__ F, double* __restrict__ C_hi,
                                                     double* __restrict__ C_lo, int64_t ldc) {
    const int64_t col = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (col >= n) return;
    const int f = F[col];
    auto finish = [&](const double (&S)[NS], int64_t row) {
        double hi, lo;
        renorm_levels<NS>(S, E[row] + f, hi, lo);
        __builtin_nontemporal_store(hi, C_hi + row * ldc + col);
        __builtin_nontemporal_store(lo, C_lo + row * ldc + col);
    };
    int64_t row = blockIdx.y;
    if constexpr (TWO) {
        for (; row + gridDim.y < m; row += 2 * static_cast<int64_t>(gridDim.y)) {
            const int64_t r1 = row + gridDim.y;
            double S[NS], T[NS];
#pragma unroll
            for (int l = 0; l < NS; ++l) {
                S[l] = __builtin_nontemporal_load(levels + l * plane + row * ldl + col);
                T[l] = __builtin_nontemporal_load(levels + l * plane + r1 * ldl + col);
            }
            finish(S, row);
            finish(T, r1);
        }
    }
    for (; row < m; row += gridDim.y) {
        double S[NS];
#pragma unroll
        for (int l = 0; l < NS; ++l) S[l] = __builtin_nontemporal_load(levels + l * plane + row * ldl + col);
        finish(S, row);
    }
}

// Up to this many outputs the renormalisation runs a quarter as many row
// workgroups, two rows per step (1024^2: 15.8 against 18.2 us); above it one
// row per workgroup (4096^2: 0.208 against 0.243 ms).
constexpr int64_t kRenormFewOutputs = int64_t(1) << 21;

template <int NS>
void launch_renorm_ns(int64_t m, int64_t n, const double* levels, int64_t ldl, int64_t plane, const int32_t* E,
                      const int32_t* F, double* C_hi, double* C_lo, int64_t ldc, hipStream_t stream) {
    const unsigned gx = static_cast<unsigned>((n + 255) / 256);
    if (m * n <= kRenormFewOutputs) {
        const int64_t gy = (m + 3) / 4 < 65535 ? (m + 3) / 4 : 65535;
        renorm_kernel<NS, true><<<dim3(gx, static_cast<unsigned>(gy)), 256, 0, stream>>>(m, n, levels, ldl, plane, E, F,
                                                                                        C_hi, C_lo, ldc);
    } else {
        const int64_t gy = m < 65535 ? m : 65535;
        renorm_kernel<NS, false><<<dim3(gx, static_cast<unsigned>(gy)), 256, 0, stream>>>(m, n, levels, ldl, plane, E,
                                                                                         F, C_hi, C_lo, ldc);
    }
}

// One thread per output entry: the exact total of its 16 level sums, rounded to
// the nearest four doubles.
__global__ void __launch_bounds__(256) qd_levels_kernel(int64_t m, int64_t n, const double* __restrict__ levels,
                                                        int64_t ldl, int64_t plane, const int32_t* __restrict__ E,
                                                        const int32_t* __restrict__ F, OutPlanes out, int64_t ldc) {
    const int64_t col = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (col >= n) return;
    const int f = F[col];
    for (int64_t row = blockIdx.y; row < m; row += gridDim.y) {
        double S[kQdSlices];
#pragma unroll
        for (int l = 0; l < kQdSlices; ++l) S[l] = levels[l * plane + row * ldl + col];
        double c[4];
        qd_from_levels<kQdSlices>(S, E[row] + f, c);
#pragma unroll
        for (int q = 0; q < 4; ++q) out.c[q][row * ldc + col] = c[q];
    }
}

// One k-block of a blocked quad-double product that was split over k: its 16
// double level planes (exact integers in units 2^(-13(l+2))) go into the int64
// level planes as kEpiUnitsSet / kEpiUnitsAdd / kEpiUnitsQD would put them.
template <int STEP>  // 0: store, 1: add, 2: add and round the total to four doubles
__global__ void __launch_bounds__(256) qd_units_from_levels_kernel(int64_t m, int64_t n,
                                                                   const double* __restrict__ levels,
                                                                   int64_t* __restrict__ units, int64_t plane,
                                                                   const int32_t* __restrict__ E,
                                                                   const int32_t* __restrict__ F, OutPlanes out,
                                                                   int64_t ldc) {
    const int64_t col = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (col >= n) return;
    for (int64_t row = blockIdx.y; row < m; row += gridDim.y) {
        int64_t N[kQdSlices];
#pragma unroll
        for (int l = 0; l < kQdSlices; ++l) {
            const int64_t i = l * plane + row * n + col;
            N[l] = static_cast<int64_t>(ldexp(levels[i], kSliceBits * (l + 2)));
            if (STEP != 0) N[l] += units[i];
            if (STEP != 2) units[i] = N[l];
        }
        if constexpr (STEP == 2) {
            double c[4];
            qd_from_level_units<kQdSlices>(N, E[row] + F[col], c);
#pragma unroll
            for (int q = 0; q < 4; ++q) out.c[q][row * ldc + col] = c[q];
        }
    }
}

// Zero the NS level planes of an m x n product (row stride ldl) with vector
// stores: workgroup rows y take the planes' rows (plane l, row r) in turn,
// threads run along each row.
__global__ void __launch_bounds__(256) zero_levels_kernel(int64_t m, int64_t n, int ns, double* __restrict__ levels,
                                                          int64_t ldl, int64_t plane) {
    const int64_t rows = ns * m;
    for (int64_t lr = blockIdx.y; lr < rows; lr += gridDim.y) {
        const int64_t l = lr / m, r = lr - l * m;
        double* row = levels + l * plane + r * ldl;
        for (int64_t c = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; c < n;
             c += static_cast<int64_t>(gridDim.x) * blockDim.x)
            row[c] = 0.0;
    }
}

// One thread per output entry of a pair-packed product split over k: the
// parts' int64 group sums are added (exact: the whole k stays within the int64
// bound) and the exact total is rounded to W words.
template <int NS, int W>
__global__ void __launch_bounds__(256) pair_parts_kernel(int64_t m, int64_t n, const int64_t* __restrict__ units,
                                                         int64_t ldu, int64_t plane, int64_t part_stride,
                                                         int64_t parts, const int32_t* __restrict__ E,
                                                         const int32_t* __restrict__ F, OutPlanes out, int64_t ldc) {
    const int64_t col = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (col >= n) return;
    const int f = F[col];
    for (int64_t row = blockIdx.y; row < m; row += gridDim.y) {
        int64_t N[NS - 1];
#pragma unroll
        for (int g = 0; g < NS - 1; ++g) N[g] = 0;
        const int64_t* cell = units + row * ldu + col;
        for (int64_t p = 0; p < parts; ++p) {
#pragma unroll
            for (int g = 0; g < NS - 1; ++g) N[g] += cell[p * part_stride + g * plane];
        }
        double c[W];
        pair_units_round<NS, W>(N, E[row] + f, c);
#pragma unroll
        for (int q = 0; q < W; ++q) out.c[q][row * ldc + col] = c[q];
    }
}

// The double-double exit's rounding on given group sums (diagnostics): entry i
// has NS - 1 int64 group sums units[i (NS - 1) + g], group g counting units
// 2^(sc[i] - 13(g + 3)), and gets the nearest double-double of their exact
// total, as the pair-packed products' exit computes it.
template <int NS>
__global__ void __launch_bounds__(256) pair_round_probe_kernel(int64_t count, const int64_t* __restrict__ units,
                                                               const int32_t* __restrict__ sc,
                                                               double* __restrict__ out) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= count) return;
    int64_t N[NS - 1];
#pragma unroll
    for (int g = 0; g < NS - 1; ++g) N[g] = units[i * (NS - 1) + g];
    double c[2];
    pair_units_round<NS, 2>(N, sc[i], c);
    out[2 * i] = c[0];
    out[2 * i + 1] = c[1];
}

}  // namespace

hipError_t launch_pair_parts(int64_t rows, int64_t cols, int ns, int words, const int64_t* units, int64_t ldu,
                             int64_t plane, int64_t part_stride, int64_t parts, const int32_t* E, const int32_t* F,
                             const OutPlanes& C, int64_t ldc, hipStream_t stream) {
    if (rows == 0 || cols == 0) return hipSuccess;
    if (ns < kMinSlices || ns > kMaxSlices || parts < 1 || (words != 2 && words != 4)) return hipErrorInvalidValue;
    const int64_t gy = rows < 65535 ? rows : 65535;
    const dim3 grid(static_cast<unsigned>((cols + 255) / 256), static_cast<unsigned>(gy));
    return dispatch_ns(ns, [&](auto c) {
        constexpr int NS = decltype(c)::value;
        if (words == 2)
            pair_parts_kernel<NS, 2><<<grid, 256, 0, stream>>>(rows, cols, units, ldu, plane, part_stride, parts, E,
                                                               F, C, ldc);
        else if constexpr (NS == kQdSlices)
            pair_parts_kernel<NS, 4><<<grid, 256, 0, stream>>>(rows, cols, units, ldu, plane, part_stride, parts, E,
                                                               F, C, ldc);
        else
            return hipErrorInvalidValue;  // four words: the quad-double product only
        return hipGetLastError();
    });
}

hipError_t launch_zero_levels(int64_t m, int64_t n, int ns, double* levels, int64_t ldl, hipStream_t stream) {
    if (m == 0 || n == 0) return hipSuccess;
    const int64_t gx = (n + 255) / 256 < 64 ? (n + 255) / 256 : 64;
    const int64_t gy = ns * m < 65535 ? ns * m : 65535;
    const dim3 grid(static_cast<unsigned>(gx), static_cast<unsigned>(gy));
    zero_levels_kernel<<<grid, 256, 0, stream>>>(m, n, ns, levels, ldl, m * ldl);
    return hipGetLastError();
}

hipError_t launch_renorm(int64_t m, int64_t n, const double* levels, int64_t ldl, const int32_t* E,
                         const int32_t* F, double* C_hi, double* C_lo, int64_t ldc, hipStream_t stream) {
    if (m == 0 || n == 0) return hipSuccess;
    launch_renorm_ns<kLevels>(m, n, levels, ldl, m * ldl, E, F, C_hi, C_lo, ldc, stream);
    return hipGetLastError();
}

hipError_t launch_levels_to_qd(int64_t m, int64_t n, const double* levels, int64_t ldl, const int32_t* E,
                               const int32_t* F, const OutPlanes& C, int64_t ldc, hipStream_t stream,
                               int64_t plane) {
    if (m == 0 || n == 0) return hipSuccess;
    if (plane < 0) plane = m * ldl;
    const int64_t gy = m < 65535 ? m : 65535;
    const dim3 grid(static_cast<unsigned>((n + 255) / 256), static_cast<unsigned>(gy));
    qd_levels_kernel<<<grid, 256, 0, stream>>>(m, n, levels, ldl, plane, E, F, C, ldc);
    return hipGetLastError();
}

hipError_t launch_qd_levels_to_units(int64_t m, int64_t n, const double* levels, int64_t* units, QdBlockStep step,
                                     const int32_t* E, const int32_t* F, const OutPlanes& C, int64_t ldc,
                                     hipStream_t stream) {
    if (m == 0 || n == 0) return hipSuccess;
    const int64_t gy = m < 65535 ? m : 65535;
    const dim3 grid(static_cast<unsigned>((n + 255) / 256), static_cast<unsigned>(gy));
    const int64_t plane = m * n;
    if (step == kQdFirstBlock)
        qd_units_from_levels_kernel<0><<<grid, 256, 0, stream>>>(m, n, levels, units, plane, E, F, C, ldc);
    else if (step == kQdMiddleBlock)
        qd_units_from_levels_kernel<1><<<grid, 256, 0, stream>>>(m, n, levels, units, plane, E, F, C, ldc);
    else
        qd_units_from_levels_kernel<2><<<grid, 256, 0, stream>>>(m, n, levels, units, plane, E, F, C, ldc);
    return hipGetLastError();
}

}  // namespace ddg

extern "C" ddgemm_status_t ddgemm_probe_pair_round(int64_t count, int nslices, const int64_t* units,
                                                   const int32_t* scale, double* out, void* stream) {
    using namespace ddg;
    if (count < 0 || count > (int64_t(1) << 38) || nslices < kMinSlices || nslices > kMaxSlices)
        return DDGEMM_ERROR_INVALID_VALUE;
    if (count == 0) return DDGEMM_SUCCESS;
    if (!units || !scale || !out) return DDGEMM_ERROR_INVALID_VALUE;
    const ddgemm_status_t st = check_current_device();
    if (st != DDGEMM_SUCCESS) return st;
    const unsigned grid = static_cast<unsigned>((count + 255) / 256);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t e = dispatch_ns(nslices, [&](auto c) {
        pair_round_probe_kernel<decltype(c)::value><<<grid, 256, 0, s>>>(count, units, scale, out);
        return hipGetLastError();
    });
    return e == hipSuccess ? DDGEMM_SUCCESS : DDGEMM_ERROR_LAUNCH;
}
