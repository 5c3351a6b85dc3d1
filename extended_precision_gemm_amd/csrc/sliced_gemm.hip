// Sliced GEMM on gfx950 FP64 matrix cores ("Multiple Double Arithmetic on NVIDIA
// Tensor Cores", §2 eqs. (1)-(4); exactness from §2 eq. (5)).
//
// Level l = s + t of output entry (i, j) is S_l = sum_{s+t=l} sum_p A_s[i][p] B_t[p][j]
// for l = 0..7: the 36 slice pairs inside the double-double window.  Instead of
// the pages' single product with a block-Toeplitz right operand (28 of whose 64
// blocks are zero), each k step issues exactly the 36 nonzero pair products, one
// v_mfma_f64_16x16x4_f64 per pair and 16x16 output block, into one accumulator
// per level.  Slices are 13-bit integers times powers of two, so every product
// is exact and every partial sum is an integer multiple of 2^(-13(l+2)) below
// 2^53 units: the matrix-core accumulation is exact in any order.
//
// Work split: a workgroup of 4 waves owns a (2*WM*16) x (2*WN*16) output tile,
// each wave a WM x WN grid of 16x16 blocks with 8 level accumulators per block.
// Operand fragments are read straight from the packed slice planes, where every
// (16x4 or 4x16) fragment of one slice is 64 consecutive doubles in the
// instruction's lane order, so each load is one coalesced 512-byte access; the
// next k step's fragments are loaded while the current step's 36*WM*WN matrix
// instructions issue.
#include "common.hpp"
#include "eft.hpp"

namespace ddg {
namespace {

// Result layout of the FP64 16x16x4 instruction, as measured with the probe
// entry point on gfx950: lane L holds rows L/16 + 4v, v = 0..3, of column L % 16.
__device__ __forceinline__ int frag_row(int lane, int v) { return (lane >> 4) + 4 * v; }
__device__ __forceinline__ int frag_col(int lane) { return lane & 15; }

template <int WM, int WN>
__device__ __forceinline__ void load_frags(const double* const (&pa)[WM], const double* const (&pb)[WN],
                                           int64_t kb, double (&a)[kSlices][WM], double (&b)[kSlices][WN]) {
#pragma unroll
    for (int s = 0; s < kSlices; ++s) {
#pragma unroll
        for (int r = 0; r < WM; ++r) a[s][r] = pa[r][kb * kFragSetDoubles + s * kFragDoubles];
#pragma unroll
        for (int c = 0; c < WN; ++c) b[s][c] = pb[c][kb * kFragSetDoubles + s * kFragDoubles];
    }
}

template <int WM, int WN, bool FUSED>
__global__ void __launch_bounds__(256, 1)
sliced_gemm_kernel(int64_t m, int64_t n, int64_t KB, int64_t tiles_n,
                   const double* __restrict__ Ap, const double* __restrict__ Bp,
                   double* __restrict__ levels, int64_t ldl, int64_t plane,
                   const int32_t* __restrict__ E, const int32_t* __restrict__ F,
                   double* __restrict__ C_hi, double* __restrict__ C_lo, int64_t ldc) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t tm = static_cast<int64_t>(blockIdx.x) / tiles_n;
    const int64_t tn = static_cast<int64_t>(blockIdx.x) % tiles_n;
    const int64_t rb0 = tm * (2 * WM) + (wave >> 1) * WM;  // first 16-row block of this wave
    const int64_t cb0 = tn * (2 * WN) + (wave & 1) * WN;   // first 16-column block

    const double* pa[WM];
    const double* pb[WN];
#pragma unroll
    for (int r = 0; r < WM; ++r) pa[r] = Ap + (rb0 + r) * KB * kFragSetDoubles + lane;
#pragma unroll
    for (int c = 0; c < WN; ++c) pb[c] = Bp + (cb0 + c) * KB * kFragSetDoubles + lane;

    double4_t acc[kLevels][WM][WN];
#pragma unroll
    for (int l = 0; l < kLevels; ++l)
#pragma unroll
        for (int r = 0; r < WM; ++r)
#pragma unroll
            for (int c = 0; c < WN; ++c) acc[l][r][c] = double4_t{0.0, 0.0, 0.0, 0.0};

    double a[kSlices][WM], b[kSlices][WN];
    if (KB > 0) load_frags<WM, WN>(pa, pb, 0, a, b);
    for (int64_t kb = 0; kb < KB; ++kb) {
        double an[kSlices][WM], bn[kSlices][WN];
        load_frags<WM, WN>(pa, pb, kb + 1 < KB ? kb + 1 : kb, an, bn);
        // Triangular schedule: pair (s, t) feeds level s + t; the r/c loops put
        // WM*WN independent accumulators between two updates of the same one.
#pragma unroll
        for (int s = 0; s < kSlices; ++s)
#pragma unroll
            for (int t = 0; s + t < kLevels; ++t)
#pragma unroll
                for (int r = 0; r < WM; ++r)
#pragma unroll
                    for (int c = 0; c < WN; ++c)
                        acc[s + t][r][c] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[s][r], b[t][c], acc[s + t][r][c], 0, 0, 0);
#pragma unroll
        for (int s = 0; s < kSlices; ++s) {
#pragma unroll
            for (int r = 0; r < WM; ++r) a[s][r] = an[s][r];
#pragma unroll
            for (int c = 0; c < WN; ++c) b[s][c] = bn[s][c];
        }
    }

#pragma unroll
    for (int r = 0; r < WM; ++r) {
#pragma unroll
        for (int c = 0; c < WN; ++c) {
            const int64_t col = (cb0 + c) * 16 + frag_col(lane);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int64_t row = (rb0 + r) * 16 + frag_row(lane, v);
                if (row < m && col < n) {
                    if constexpr (FUSED) {
                        double S[kLevels];
#pragma unroll
                        for (int l = 0; l < kLevels; ++l) S[l] = acc[l][r][c][v];
                        double hi, lo;
                        renorm_levels(S, E[row] + F[col], hi, lo);
                        C_hi[row * ldc + col] = hi;
                        C_lo[row * ldc + col] = lo;
                    } else {
#pragma unroll
                        for (int l = 0; l < kLevels; ++l) levels[l * plane + row * ldl + col] = acc[l][r][c][v];
                    }
                }
            }
        }
    }
}

// One thread per output entry: cascade its 8 level sums into (hi, lo).
__global__ void __launch_bounds__(256) renorm_kernel(int64_t m, int64_t n, const double* __restrict__ levels,
                                                     int64_t ldl, int64_t plane, const int32_t* __restrict__ E,
                                                     const int32_t* __restrict__ F, double* __restrict__ C_hi,
                                                     double* __restrict__ C_lo, int64_t ldc) {
    const int64_t col = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (col >= n) return;
    const int f = F[col];
    for (int64_t row = blockIdx.y; row < m; row += gridDim.y) {
        double S[kLevels];
#pragma unroll
        for (int l = 0; l < kLevels; ++l) S[l] = levels[l * plane + row * ldl + col];
        double hi, lo;
        renorm_levels(S, E[row] + f, hi, lo);
        C_hi[row * ldc + col] = hi;
        C_lo[row * ldc + col] = lo;
    }
}

__global__ void __launch_bounds__(64) probe_mfma_kernel(double* __restrict__ out) {
    const int lane = threadIdx.x;
    const double a = static_cast<double>(lane + 1);
    const double b = 100.0 * static_cast<double>(lane + 1);
    double4_t c = {0.0, 0.0, 0.0, 0.0};
    c = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
#pragma unroll
    for (int v = 0; v < 4; ++v) out[lane * 4 + v] = c[v];
}

constexpr int kWM = 2, kWN = 2;  // wave tile 32x32, workgroup tile 64x64

}  // namespace

hipError_t launch_sliced_gemm(int64_t m, int64_t n, int64_t k, const double* A_slices,
                              const double* B_slices, double* levels, int64_t ldl,
                              const int32_t* E, const int32_t* F, double* C_hi, double* C_lo,
                              int64_t ldc, bool fused, hipStream_t stream) {
    if (m == 0 || n == 0) return hipSuccess;
    const PackGeom ga(m, k);
    constexpr int BM = 2 * kWM * 16, BN = 2 * kWN * 16;
    static_assert(kPackOuter % BM == 0 && kPackOuter % BN == 0, "tile must divide the packing");
    const int64_t tiles_m = (m + BM - 1) / BM, tiles_n = (n + BN - 1) / BN;
    const int64_t tiles = tiles_m * tiles_n;
    if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
    const int64_t plane = m * ldl;
    if (fused)
        sliced_gemm_kernel<kWM, kWN, true><<<static_cast<unsigned>(tiles), 256, 0, stream>>>(
            m, n, ga.KB, tiles_n, A_slices, B_slices, nullptr, 0, 0, E, F, C_hi, C_lo, ldc);
    else
        sliced_gemm_kernel<kWM, kWN, false><<<static_cast<unsigned>(tiles), 256, 0, stream>>>(
            m, n, ga.KB, tiles_n, A_slices, B_slices, levels, ldl, plane, nullptr, nullptr, nullptr, nullptr, 0);
    return hipGetLastError();
}

hipError_t launch_renorm(int64_t m, int64_t n, const double* levels, int64_t ldl, const int32_t* E,
                         const int32_t* F, double* C_hi, double* C_lo, int64_t ldc, hipStream_t stream) {
    if (m == 0 || n == 0) return hipSuccess;
    const int64_t gy = m < 65535 ? m : 65535;
    dim3 grid(static_cast<unsigned>((n + 255) / 256), static_cast<unsigned>(gy));
    renorm_kernel<<<grid, 256, 0, stream>>>(m, n, levels, ldl, m * ldl, E, F, C_hi, C_lo, ldc);
    return hipGetLastError();
}

hipError_t launch_probe_mfma(double* out, hipStream_t stream) {
    probe_mfma_kernel<<<1, 64, 0, stream>>>(out);
    return hipGetLastError();
}

}  // namespace ddg
