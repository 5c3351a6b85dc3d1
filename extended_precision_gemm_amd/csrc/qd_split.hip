// Balancing exponents and 13-bit slicing of one quad-double operand
// ("Multiple Double Arithmetic on NVIDIA Tensor Cores": §2 quartering, and its
// remark that a quartered quad-double matrix is sixteen times the size of a
// matrix of doubles; §3 balancing).
//
// An entry x = x0 + x1 + x2 + x3 is normalised: every component is at most half
// an ulp of the one before it (the convention of the quad-double library the
// pages build on).  It is cut as the 208-bit fixed-point window below the
// balancing exponent E of its row (A) or column (B): N = floor(|x| 2^(208-E)),
// slice s = sign(x) * ((N >> 13(15-s)) & 8191) * 2^(-13(s+1)), s = 0..15.  N is
// formed exactly in 256-bit register integers from the components' integer
// mantissas; E is the largest frexp exponent of RN(x) over the row or column.
#include "common.hpp"
#include "split_common.hpp"
#include "window.hpp"

namespace ddg {
namespace {

constexpr int kQdWindowBits = kSliceBits * kQdSlices;  // 208

__device__ __forceinline__ void load_qd(const QdPlanes& X, int64_t idx, double (&x)[4]) {
#pragma unroll
    for (int c = 0; c < 4; ++c) x[c] = X.x[c] ? X.x[c][idx] : 0.0;
}

// Encoded frexp exponent of RN(x), kNoExp for zero.  With e = frexp exponent of
// x0, |x| < 2^e, and M = floor(|x| 2^(55-e)) < 2^55 decides the rounding:
// RN(x) = 2^e from M >= 2^55 - 2 (|x| >= 2^e - 2^(e-54), ties to even), RN(x)
// >= 2^(e-1) from M >= 2^54 - 1, and RN(x) < 2^(e-1) below that.
__device__ __forceinline__ int qd_entry_code(const double (&x)[4]) {
    if (x[0] == 0.0) return kNoExp;
    const int e = frexp_exponent(x[0]);
    const uint64_t M = floor_abs_window<1>(x, e - 55).w[0];
    const int ex = M >= (1ull << 55) - 2 ? e + 1 : (M >= (1ull << 54) - 1 ? e : e - 1);
    return ex + kExpBias;
}

__device__ __forceinline__ void qd_slice_entry(const double (&x)[4], int E, double (&out)[kQdSlices]) {
    if (x[0] == 0.0) {
#pragma unroll
        for (int s = 0; s < kQdSlices; ++s) out[s] = 0.0;
        return;
    }
    const bool neg = x[0] < 0.0;
    const WideInt<4> N = floor_abs_window<4>(x, E - kQdWindowBits);
#pragma unroll
    for (int s = 0; s < kQdSlices; ++s) {
        const int d = static_cast<int>(wide_bits64(N, kSliceBits * (kQdSlices - 1 - s)) & 0x1FFF);
        out[s] = ldexp(static_cast<double>(neg ? -d : d), -kSliceBits * (s + 1));
    }
}

// One wave per row: E[row] = max exponent over the row (axis 0, the A operand).
__global__ void __launch_bounds__(256) qd_exp_rows_kernel(int64_t rows, int64_t cols, QdPlanes X, int64_t ld,
                                                          int32_t* __restrict__ exps) {
    const int lane = threadIdx.x & 63;
    const int64_t parts = gridDim.y;  // k-parts, as in the double-double row kernel
    const int64_t p0 = cols * blockIdx.y / parts, p1 = cols * (blockIdx.y + 1) / parts;
    const int64_t nwaves = static_cast<int64_t>(gridDim.x) * (blockDim.x >> 6);
    for (int64_t row = static_cast<int64_t>(blockIdx.x) * (blockDim.x >> 6) + (threadIdx.x >> 6);
         row < rows; row += nwaves) {
        int code = kNoExp;
        for (int64_t p = p0 + lane; p < p1; p += 64) {
            double x[4];
            load_qd(X, row * ld + p, x);
            code = max(code, qd_entry_code(x));
        }
        code = wave_max(code);
        if (lane == 0) {
            if (parts == 1)
                exps[row] = decode_exp(code);
            else if (code != kNoExp)
                atomicMax(exps + row, code);
        }
    }
}

// Column exponents (axis 1, the B operand): workgroup (b, c) reduces columns
// 16b .. 16b+15 over row part c of gridDim.y; thread t takes column 16b + t % 16
// and rows t / 16, t / 16 + NT / 16, ..., two rows in flight.  With one part
// the decoded exponents are stored; with several the encoded maxima are folded
// into `out` (cleared to kNoExp) with atomicMax and decoded after.
template <int NT>
__global__ void __launch_bounds__(NT) qd_exp_cols_block_kernel(int64_t rows, int64_t cols, QdPlanes X, int64_t ld,
                                                               int32_t* __restrict__ out) {
    constexpr int kRowGroups = NT / 16;
    __shared__ int codes[NT];
    const int t = threadIdx.x;
    const int64_t parts = gridDim.y;
    const int64_t r0 = rows * blockIdx.y / parts, r1 = rows * (blockIdx.y + 1) / parts;
    const int64_t nblocks = (cols + 15) / 16;
    for (int64_t b = blockIdx.x; b < nblocks; b += gridDim.x) {  // uniform per workgroup
        const int64_t o = b * 16 + (t & 15);
        int code = kNoExp;
        if (o < cols) {
            int64_t p = r0 + (t >> 4);
            for (; p + kRowGroups < r1; p += 2 * kRowGroups) {
                double x0[4], x1[4];
                load_qd(X, p * ld + o, x0);
                load_qd(X, (p + kRowGroups) * ld + o, x1);
                code = max(code, max(qd_entry_code(x0), qd_entry_code(x1)));
            }
            for (; p < r1; p += kRowGroups) {
                double x[4];
                load_qd(X, p * ld + o, x);
                code = max(code, qd_entry_code(x));
            }
        }
        codes[t] = code;
        __syncthreads();
        if (t < 16 && o < cols) {
            int c = kNoExp;
            for (int g = 0; g < kRowGroups; ++g) c = max(c, codes[g * 16 + t]);
            if (parts == 1)
                out[o] = decode_exp(c);
            else if (c != kNoExp)
                atomicMax(out + o, c);
        }
        __syncthreads();  // codes[] is rewritten by the next column block
    }
}

// One thread per packed (fragment, lane) position; writes the 16 slices of its
// entry.  AXIS 0: entry (o, p) is X[o][p]; AXIS 1: it is X[p][o].  PK: the
// pair-packed layout of an A operand that the product's pair-packed GEMM reads
// -- plane 2u holds slices 2u and 2u+1 added (one exact 26-bit value, as the
// two share the entry's sign and sit 13 bits apart), plane 2u+1 slice 2u alone.
template <int AXIS, bool PK = false>
__global__ void __launch_bounds__(256) qd_slice_kernel(int64_t outer, int64_t k, int64_t KB, int64_t total,
                                                       QdPlanes X, int64_t ld, const int32_t* __restrict__ exps,
                                                       double* __restrict__ slices) {
    for (int64_t g = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; g < total;
         g += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const int lane = static_cast<int>(g & 63);
        const int64_t frag = g >> 6;
        const int64_t o = (frag / KB) * 16 + (lane & 15);
        const int64_t p = (frag % KB) * 4 + (lane >> 4);
        double x[4] = {0.0, 0.0, 0.0, 0.0};
        int E = 0;
        if (o < outer && p < k) {
            load_qd(X, AXIS == 0 ? o * ld + p : p * ld + o, x);
            E = exps[o];
        }
        double sl[kQdSlices];
        qd_slice_entry(x, E, sl);
        if constexpr (PK) {
#pragma unroll
            for (int u = 0; u < kQdSlices / 2; ++u) {
                const double single = sl[2 * u];
                sl[2 * u] = sl[2 * u] + sl[2 * u + 1];
                sl[2 * u + 1] = single;
            }
        }
        double* dst = slices + frag * (kQdSlices * kFragDoubles) + lane;
#pragma unroll
        for (int s = 0; s < kQdSlices; ++s) dst[s * kFragDoubles] = sl[s];
    }
}

// One pass over a small B operand (column exponents otherwise take four
// launches): workgroup (b, c) finds the exponents of 16-column block b -- every
// part c re-reads the block, from cache at the sizes this is used for -- and
// slices the part's share of the block's k-blocks; part 0 stores the exponents.
template <int NT>
__global__ void __launch_bounds__(NT) qd_split_cols_block_kernel(int64_t outer, int64_t k, int64_t KB, QdPlanes X,
                                                                 int64_t ld, int32_t* __restrict__ exps,
                                                                 double* __restrict__ slices) {
    constexpr int kRowGroups = NT / 16;
    __shared__ int codes[NT];
    __shared__ int block_exp[16];
    const int t = threadIdx.x;
    const int64_t blk = blockIdx.x;
    const int64_t o0 = blk * 16;
    const int64_t kparts = gridDim.y;
    const int64_t kb_begin = KB * blockIdx.y / kparts, kb_end = KB * (blockIdx.y + 1) / kparts;

    // thread t takes column o0 + t % 16 over rows t / 16, t / 16 + kRowGroups, ...
    int code = kNoExp;
    const int64_t oc = o0 + (t & 15);
    if (oc < outer) {
        for (int64_t p = t >> 4; p < k; p += kRowGroups) {
            double x[4];
            load_qd(X, p * ld + oc, x);
            code = max(code, qd_entry_code(x));
        }
    }
    codes[t] = code;
    __syncthreads();
    if (t < 16) {
        int c = kNoExp;
        for (int g = 0; g < kRowGroups; ++g) c = max(c, codes[g * 16 + t]);
        block_exp[t] = decode_exp(c);
    }
    __syncthreads();
    if (blockIdx.y == 0 && t < 16 && o0 + t < outer) exps[o0 + t] = block_exp[t];

    // one thread per packed (fragment, lane) position of the part's k-blocks
    const int64_t total = (kb_end - kb_begin) * kFragDoubles;
    for (int64_t q = t; q < total; q += NT) {
        const int64_t kb = kb_begin + q / kFragDoubles;
        const int lane = static_cast<int>(q % kFragDoubles);
        const int64_t o = o0 + (lane & 15);
        const int64_t p = kb * 4 + (lane >> 4);
        double x[4] = {0.0, 0.0, 0.0, 0.0};
        if (o < outer && p < k) load_qd(X, p * ld + o, x);
        double sl[kQdSlices];
        qd_slice_entry(x, block_exp[lane & 15], sl);
        double* dst = slices + (blk * KB + kb) * (kQdSlices * kFragDoubles) + lane;
#pragma unroll
        for (int s = 0; s < kQdSlices; ++s) dst[s * kFragDoubles] = sl[s];
    }
}

// Limits of the one-pass path: operand bytes (four planes) and the parts'
// exponent re-reads (measured on gfx950, B operand: 256^2 45 -> 18 us, 512^2
// 62 -> 32 us, 1024^2 76 -> 65 us; from 1536^2 up the two passes are as fast).
constexpr int64_t kQdSmallColsBytes = 32ll << 20;
constexpr int64_t kQdSmallColsReread = 512ll << 20;

}  // namespace

hipError_t launch_qd_exps(int64_t rows, int64_t cols, const QdPlanes& X, int64_t ldx, int axis, int32_t* exps,
                          hipStream_t stream) {
    if ((axis == 0 ? rows : cols) == 0) return hipSuccess;
    if (axis == 0) {
        const int64_t parts = exp_row_parts(rows, cols);
        const dim3 grid(grid_for(rows, 4, 1 << 20), static_cast<unsigned>(parts));
        if (parts > 1) fill_int_kernel<<<grid_for(rows, 256, 4096), 256, 0, stream>>>(exps, rows, kNoExp);
        qd_exp_rows_kernel<<<grid, 256, 0, stream>>>(rows, cols, X, ldx, exps);
        if (parts > 1) decode_exps_kernel<<<grid_for(rows, 256, 4096), 256, 0, stream>>>(exps, rows);
    } else {
        const int64_t parts = exp_col_parts(rows, cols);
        const dim3 grid(grid_for(cols, 16, 1 << 20), static_cast<unsigned>(parts));
        if (parts > 1) fill_int_kernel<<<grid_for(cols, 256, 4096), 256, 0, stream>>>(exps, cols, kNoExp);
        qd_exp_cols_block_kernel<1024><<<grid, 1024, 0, stream>>>(rows, cols, X, ldx, exps);
        if (parts > 1) decode_exps_kernel<<<grid_for(cols, 256, 4096), 256, 0, stream>>>(exps, cols);
    }
    return hipGetLastError();
}

hipError_t launch_qd_slices(int64_t rows, int64_t cols, const QdPlanes& X, int64_t ldx, int axis,
                            const int32_t* exps, double* slices, hipStream_t stream, bool pairs) {
    const int64_t outer = axis == 0 ? rows : cols;
    const int64_t k = axis == 0 ? cols : rows;
    const PackGeom g(outer, k);
    if (outer == 0 || g.doubles(kQdSlices) == 0) return hipSuccess;
    const int64_t total = g.RB * g.KB * kFragDoubles;
    const unsigned grid = grid_for(total, 256, 1 << 20);
    if (axis == 0 && pairs)
        qd_slice_kernel<0, true><<<grid, 256, 0, stream>>>(outer, k, g.KB, total, X, ldx, exps, slices);
    else if (axis == 0)
        qd_slice_kernel<0><<<grid, 256, 0, stream>>>(outer, k, g.KB, total, X, ldx, exps, slices);
    else
        qd_slice_kernel<1><<<grid, 256, 0, stream>>>(outer, k, g.KB, total, X, ldx, exps, slices);
    return hipGetLastError();
}

hipError_t launch_qd_split(int64_t rows, int64_t cols, const QdPlanes& X, int64_t ldx, int axis, int32_t* exps,
                           double* slices, hipStream_t stream, int phases, bool pairs) {
    const int64_t outer = axis == 0 ? rows : cols;
    const int64_t k = axis == 0 ? cols : rows;
    if (outer == 0) return hipSuccess;
    if (axis == 1 && rows > 0) {
        const PackGeom gb(outer, k);
        // k-parts for about 256 workgroups: every part re-reads its block for the
        // exponents, so fewer parts read less (qd1024 slicing 0.147 -> 0.110 ms,
        // 512^2 0.065 -> 0.042 ms against 1024 workgroups; bit-identical)
        constexpr int64_t kOnePassWorkgroups = 256;
        int64_t kparts = (kOnePassWorkgroups + gb.RB - 1) / gb.RB;
        if (kparts > gb.KB) kparts = gb.KB;
        const int64_t bytes = rows * cols * 32;
        if (bytes <= kQdSmallColsBytes && bytes * kparts <= kQdSmallColsReread) {
            if (!(phases & kSplitSlices)) return hipSuccess;  // one pass: all of it in the slice phase
            const dim3 grid(static_cast<unsigned>(gb.RB), static_cast<unsigned>(kparts));
            qd_split_cols_block_kernel<1024><<<grid, 1024, 0, stream>>>(outer, k, gb.KB, X, ldx, exps, slices);
            return hipGetLastError();
        }
    }
    if (phases & kSplitExps) {
        hipError_t err = launch_qd_exps(rows, cols, X, ldx, axis, exps, stream);
        if (err != hipSuccess) return err;
    }
    if (!(phases & kSplitSlices)) return hipSuccess;
    return launch_qd_slices(rows, cols, X, ldx, axis, exps, slices, stream, pairs);
}

}  // namespace ddg
