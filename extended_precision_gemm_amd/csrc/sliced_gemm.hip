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
// Work split: a workgroup of 8 waves (two per SIMD) owns a 64x64 output tile;
// wave w computes the 32x16 strip at block row 2*(w/4), block column w%4, with
// eight level accumulators per 16x16 block.  The operand panels move through
// LDS in stages of one k-block (4 values of k): every (16x4 or 4x16) fragment of
// one slice is 64 consecutive doubles in the packed planes, so a stage of the
// tile is 8 contiguous 4 KB runs, copied with 16-byte direct-to-LDS loads and
// read back by the waves as conflict-free 8-byte-per-lane fragment reads.
// NBUF stages are in flight; one barrier per stage.  Two waves per SIMD keep the
// matrix pipe fed while the other waits on LDS or the barrier.
#include "common.hpp"
#include "eft.hpp"

namespace ddg {
namespace {

// Result layout of the FP64 16x16x4 instruction, as measured with the probe
// entry point on gfx950: lane L holds rows L/16 + 4v, v = 0..3, of column L % 16.
__device__ __forceinline__ int frag_row(int lane, int v) { return (lane >> 4) + 4 * v; }
__device__ __forceinline__ int frag_col(int lane) { return lane & 15; }

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void global_void_t;

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kTileBlocks = 4;                                  // 64x64 tile = 4x4 blocks
constexpr int kStageDoubles = 2 * kTileBlocks * kFragSetDoubles;  // 4096 doubles = 32 KB
constexpr int kPiecesPerWave = kStageDoubles / (kWaves * 128);  // 1 KB pieces per wave per stage

// Order the compiler's memory operations around a hardware barrier or wait
// without adding any instruction.
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

template <int NBUF, bool FUSED>
__global__ void __launch_bounds__(kThreads, 1)
sliced_gemm_kernel(int64_t m, int64_t n, int64_t KB, int64_t tiles_n,
                   const double* __restrict__ Ap, const double* __restrict__ Bp,
                   double* __restrict__ levels, int64_t ldl, int64_t plane,
                   const int32_t* __restrict__ E, const int32_t* __restrict__ F,
                   double* __restrict__ C_hi, double* __restrict__ C_lo, int64_t ldc) {
    static_assert(NBUF >= 2 && NBUF <= 4, "stages in flight");
    __shared__ __attribute__((aligned(1024))) double lds[NBUF * kStageDoubles];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wr = wave >> 2;  // block rows 2*wr, 2*wr+1 of the tile
    const int wc = wave & 3;   // block column wc of the tile
    const int64_t tm = static_cast<int64_t>(blockIdx.x) / tiles_n;
    const int64_t tn = static_cast<int64_t>(blockIdx.x) % tiles_n;
    const int64_t rb0 = tm * kTileBlocks, cb0 = tn * kTileBlocks;

    // A stage is 32 pieces of 1 KB: pieces 0-15 are the A panel (block b = q/4,
    // quarter q%4 of its 4 KB fragment set), 16-31 the B panel.  Wave w copies
    // pieces w, w+8, w+16, w+24; lane L moves bytes [16L, 16L+16) of a piece.
    const double* src[kPiecesPerWave];
    int dst[kPiecesPerWave];
#pragma unroll
    for (int i = 0; i < kPiecesPerWave; ++i) {
        const int q = i * kWaves + wave;
        const int op = q >> 4, blk = (q >> 2) & 3, quarter = q & 3;
        const double* base = op == 0 ? Ap + (rb0 + blk) * KB * kFragSetDoubles
                                      : Bp + (cb0 + blk) * KB * kFragSetDoubles;
        src[i] = base + quarter * 128 + lane * 2;
        dst[i] = op * (kTileBlocks * kFragSetDoubles) + blk * kFragSetDoubles + quarter * 128;
    }
    auto issue = [&](int64_t kb, int buf) {
#pragma unroll
        for (int i = 0; i < kPiecesPerWave; ++i)
            __builtin_amdgcn_global_load_lds(
                (global_void_t*)(src[i] + kb * kFragSetDoubles),
                (lds_void_t*)(lds + buf * kStageDoubles + dst[i]), 16, 0, 0);
    };

    double4_t acc[kLevels][2];
#pragma unroll
    for (int l = 0; l < kLevels; ++l) acc[l][0] = acc[l][1] = double4_t{0.0, 0.0, 0.0, 0.0};

    if (KB > 0) {
#pragma unroll
        for (int j = 0; j < NBUF - 1; ++j) issue(j < KB ? j : KB - 1, j);
        for (int64_t kb = 0; kb < KB; ++kb) {
            // Stage kb has landed once at most NBUF-2 younger stages are pending.
            if constexpr (NBUF == 4) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
            else if constexpr (NBUF == 3) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
            else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            compiler_fence();
            __builtin_amdgcn_s_barrier();  // every wave's copy of stage kb is in LDS, and
            compiler_fence();               // every wave is done reading stage kb-1
            const int64_t nxt = kb + NBUF - 1;
            issue(nxt < KB ? nxt : KB - 1, static_cast<int>(nxt % NBUF));

            const double* sa = lds + (kb % NBUF) * kStageDoubles + (2 * wr) * kFragSetDoubles + lane;
            const double* sb = lds + (kb % NBUF) * kStageDoubles + (kTileBlocks + wc) * kFragSetDoubles + lane;
            double a[kSlices][2], b[kSlices];
#pragma unroll
            for (int s = 0; s < kSlices; ++s) {
                a[s][0] = sa[s * kFragDoubles];
                a[s][1] = sa[kFragSetDoubles + s * kFragDoubles];
                b[s] = sb[s * kFragDoubles];
            }
            // Triangular schedule: pair (s, t) feeds level s + t.
#pragma unroll
            for (int s = 0; s < kSlices; ++s)
#pragma unroll
                for (int t = 0; s + t < kLevels; ++t)
#pragma unroll
                    for (int r = 0; r < 2; ++r)
                        acc[s + t][r] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[s][r], b[t], acc[s + t][r], 0, 0, 0);
        }
        // No direct-to-LDS copy may still be in flight when the workgroup ends.
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }

    const int64_t col = (cb0 + wc) * 16 + frag_col(lane);
#pragma unroll
    for (int r = 0; r < 2; ++r) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int64_t row = (rb0 + 2 * wr + r) * 16 + frag_row(lane, v);
            if (row < m && col < n) {
                if constexpr (FUSED) {
                    double S[kLevels];
#pragma unroll
                    for (int l = 0; l < kLevels; ++l) S[l] = acc[l][r][v];
                    double hi, lo;
                    renorm_levels(S, E[row] + F[col], hi, lo);
                    C_hi[row * ldc + col] = hi;
                    C_lo[row * ldc + col] = lo;
                } else {
#pragma unroll
                    for (int l = 0; l < kLevels; ++l) levels[l * plane + row * ldl + col] = acc[l][r][v];
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

constexpr int kNBuf = 4;  // stages in flight

}  // namespace

hipError_t launch_sliced_gemm(int64_t m, int64_t n, int64_t k, const double* A_slices,
                              const double* B_slices, double* levels, int64_t ldl,
                              const int32_t* E, const int32_t* F, double* C_hi, double* C_lo,
                              int64_t ldc, bool fused, hipStream_t stream) {
    if (m == 0 || n == 0) return hipSuccess;
    const PackGeom ga(m, k);
    constexpr int BM = kTileBlocks * 16, BN = kTileBlocks * 16;
    static_assert(kPackOuter % BM == 0 && kPackOuter % BN == 0, "tile must divide the packing");
    const int64_t tiles_m = (m + BM - 1) / BM, tiles_n = (n + BN - 1) / BN;
    const int64_t tiles = tiles_m * tiles_n;
    if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
    const int64_t plane = m * ldl;
    if (fused)
        sliced_gemm_kernel<kNBuf, true><<<static_cast<unsigned>(tiles), kThreads, 0, stream>>>(
            m, n, ga.KB, tiles_n, A_slices, B_slices, nullptr, 0, 0, E, F, C_hi, C_lo, ldc);
    else
        sliced_gemm_kernel<kNBuf, false><<<static_cast<unsigned>(tiles), kThreads, 0, stream>>>(
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
