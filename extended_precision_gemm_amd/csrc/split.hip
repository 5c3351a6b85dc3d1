// Balancing exponents and 13-bit slicing of one double-double operand
// ("Multiple Double Arithmetic on NVIDIA Tensor Cores", §2 quartering and its
// worked example; §3 balancing, Problems 3.3 and 3.4).
//
// Every entry x = hi + lo is cut as the 104-bit fixed-point window below the
// balancing exponent E of its row (A) or column (B): N = floor(|x| 2^(104-E)),
// slice s = sign(x) * ((N >> 13(7-s)) & 8191) * 2^(-13(s+1)).  N is formed in
// integer arithmetic from the exact error-free sum of (hi, lo), so opposite
// signs (the pages' Problem 3.3), leading-zero slices (Problem 3.4), unnormalised
// pairs and subnormals need no special borrow steps, and no 2^(104-E) factor
// (which overflows for E < -919) is ever formed in floating point.
#include "common.hpp"
#include "eft.hpp"
#include "split_common.hpp"
#include "window.hpp"

namespace ddg {
namespace {

// Encoded exponent of RN(hi + lo), kNoExp for zero.
__device__ __forceinline__ int entry_exp_code(double hi, double lo) {
    const double s = hi + lo;
    return s == 0.0 ? kNoExp : frexp_exponent(s) + kExpBias;
}

// floor(y * 2^sh) for y = +-mant (mant < 2^53, y's sign given by neg); the
// result is known to fit in int64 when sh >= 0.
__device__ __forceinline__ int64_t floor_scaled(uint64_t mant, bool neg, int sh) {
    if (sh >= 0) {
        const int64_t v = static_cast<int64_t>(mant << sh);
        return neg ? -v : v;
    }
    const int r = -sh;
    if (r >= 60) return (neg && mant != 0) ? -1 : 0;
    const uint64_t q = mant >> r;
    const bool frac = (mant & ((1ull << r) - 1)) != 0;
    return neg ? -static_cast<int64_t>(q + (frac ? 1 : 0)) : static_cast<int64_t>(q);
}

// The NS unit-scaled slices of x = hi + lo in the 13 NS-bit window below
// exponent E (|x| < 2^E).
template <int NS>
__device__ __forceinline__ void slice_entry(double hi, double lo, int E, double (&out)[NS]) {
    double s, e;
    two_sum(hi, lo, s, e);  // x = s + e exactly, |e| <= ulp(s)/2
    if (s == 0.0) {
#pragma unroll
        for (int q = 0; q < NS; ++q) out[q] = 0.0;
        return;
    }
    const bool neg = s < 0.0;
    if constexpr (NS > kSlices) {
        // Windows wider than 128 bits: (s, e) is a normalised pair, so the exact
        // floor comes from the 256-bit window of (s, e, 0, 0).
        const double x[4] = {s, e, 0.0, 0.0};
        const WideInt<4> N = floor_abs_window<4>(x, E - kSliceBits * NS);
#pragma unroll
        for (int q = 0; q < NS; ++q) {
            const int d = static_cast<int>(wide_bits64(N, kSliceBits * (NS - 1 - q)) & 0x1FFF);
            out[q] = ldexp(static_cast<double>(neg ? -d : d), -kSliceBits * (q + 1));
        }
    } else {
        const double ep = neg ? -e : e;  // |x| = |s| + ep
        uint64_t ms;
        int es;
        decompose(s, ms, es);
        const int W = E - kSliceBits * NS;  // exponent of the window's last unit
        unsigned __int128 N;
        if (es >= W) {
            // |s| 2^-W = ms << (es - W) is an integer below 2^(13 NS); add floor(ep 2^-W),
            // which is below 2^51 in magnitude because |ep| <= ulp(s)/2.
            N = static_cast<unsigned __int128>(ms) << (es - W);
            if (ep != 0.0) {
                uint64_t me;
                int ee;
                decompose(ep, me, ee);
                const int64_t f = floor_scaled(me, ep < 0.0, ee - W);
                N = static_cast<unsigned __int128>(static_cast<__int128>(N) + f);
            }
        } else {
            // |s| has bits below the window: floor((ms + ep/2^es) / 2^d) with
            // |ep/2^es| <= 1/2 is floor(ms / 2^d), minus one exactly when ms is a
            // multiple of 2^d and ep < 0.
            const int d = W - es;
            uint64_t q = 0, r = ms;
            if (d < 64) {
                q = ms >> d;
                r = ms & ((1ull << d) - 1);
            }
            if (r == 0 && ep < 0.0) q -= 1;
            N = q;
        }
        constexpr double kScale[kSlices] = {0x1p-13, 0x1p-26, 0x1p-39, 0x1p-52,
                                            0x1p-65, 0x1p-78, 0x1p-91, 0x1p-104};
#pragma unroll
        for (int q = 0; q < NS; ++q) {
            const int d = static_cast<int>(static_cast<uint64_t>(N >> (kSliceBits * (NS - 1 - q))) & 0x1FFF);
            out[q] = static_cast<double>(neg ? -d : d) * kScale[q];
        }
    }
}

// The pair-packed layout of an A operand, read by the product's pair-packed
// GEMM: plane 2u holds slices 2u and 2u+1 added -- one exact 26-bit value, as
// the two share the entry's sign and sit 13 bits apart -- and plane 2u+1 holds
// slice 2u alone; with an odd count the last plane keeps the last slice.
template <int NS>
__device__ __forceinline__ void pair_pack(double (&sl)[NS]) {
#pragma unroll
    for (int u = 0; 2 * u + 1 < NS; ++u) {
        const double single = sl[2 * u];
        sl[2 * u] = sl[2 * u] + sl[2 * u + 1];
        sl[2 * u + 1] = single;
    }
}

// One wave per row and k-part: E[row] = max frexp exponent over the row (axis
// 0, the A operand).  Part y of gridDim.y covers columns [cols y / parts,
// cols (y + 1) / parts).  With one part the decoded exponent is stored; with
// several the encoded maxima are folded into `exps` (cleared to kNoExp) with
// atomicMax and decoded after.
__global__ void __launch_bounds__(256) exp_rows_kernel(int64_t rows, int64_t cols,
                                                       const double* __restrict__ hi,
                                                       const double* __restrict__ lo, int64_t ld,
                                                       int32_t* __restrict__ exps) {
    const int lane = threadIdx.x & 63;
    const int64_t parts = gridDim.y;
    const int64_t p0 = cols * blockIdx.y / parts, p1 = cols * (blockIdx.y + 1) / parts;
    const int64_t nwaves = static_cast<int64_t>(gridDim.x) * (blockDim.x >> 6);
    for (int64_t row = static_cast<int64_t>(blockIdx.x) * (blockDim.x >> 6) + (threadIdx.x >> 6);
         row < rows; row += nwaves) {
        const double* h = hi + row * ld;
        const double* l = lo ? lo + row * ld : nullptr;
        int code = kNoExp;
        for (int64_t p = p0 + lane; p < p1; p += 64) code = max(code, entry_exp_code(h[p], l ? l[p] : 0.0));
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
// and rows t / 16, t / 16 + NT / 16, ..., four rows in flight per plane.  With
// one part the decoded exponents are stored; with several the encoded maxima
// are folded into `out` (cleared to kNoExp) with atomicMax and decoded after.
template <int NT>
__global__ void __launch_bounds__(NT) exp_cols_block_kernel(int64_t rows, int64_t cols,
                                                            const double* __restrict__ hi,
                                                            const double* __restrict__ lo, int64_t ld,
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
            for (; p + 3 * kRowGroups < r1; p += 4 * kRowGroups) {
                double xh[4], xl[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    xh[u] = hi[(p + kRowGroups * u) * ld + o];
                    xl[u] = lo ? lo[(p + kRowGroups * u) * ld + o] : 0.0;
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) code = max(code, entry_exp_code(xh[u], xl[u]));
            }
            for (; p < r1; p += kRowGroups) code = max(code, entry_exp_code(hi[p * ld + o], lo ? lo[p * ld + o] : 0.0));
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

// One thread per packed (fragment, lane) position; writes the NS slices of
// its entry.  AXIS 0: entry (o, p) is X[o][p]; AXIS 1: it is X[p][o].
template <int AXIS, int NS, bool PK = false>
__global__ void __launch_bounds__(256) slice_kernel(int64_t outer, int64_t k, int64_t KB,
                                                    int64_t total, const double* __restrict__ hi,
                                                    const double* __restrict__ lo, int64_t ld,
                                                    const int32_t* __restrict__ exps,
                                                    double* __restrict__ slices) {
    for (int64_t g = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; g < total;
         g += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const int lane = static_cast<int>(g & 63);
        const int64_t frag = g >> 6;  // (o / 16) * KB + p / 4
        const int64_t o = (frag / KB) * 16 + (lane & 15);
        const int64_t p = (frag % KB) * 4 + (lane >> 4);
        double x_hi = 0.0, x_lo = 0.0;
        int E = 0;
        if (o < outer && p < k) {
            const int64_t idx = AXIS == 0 ? o * ld + p : p * ld + o;
            x_hi = hi[idx];
            x_lo = lo ? lo[idx] : 0.0;
            E = exps[o];
        }
        double sl[NS];
        slice_entry<NS>(x_hi, x_lo, E, sl);
        if constexpr (PK) pair_pack<NS>(sl);
        double* dst = slices + frag * (NS * kFragDoubles) + lane;
#pragma unroll
        for (int q = 0; q < NS; ++q) dst[q * kFragDoubles] = sl[q];
    }
}

// Workgroups (b, c) for 16-row (AXIS 0) or 16-column (AXIS 1) block b and part c
// of its k-blocks: first the block's balancing exponents, then the slices of
// the part's k-blocks, so the second read of the block's (hi, lo) comes from
// cache rather than HBM and no atomics are needed.  With several parts every
// part computes the block's exponents (its re-reads hit the cache while the
// operand fits there) and part 0 stores them.
template <int AXIS, int NT, int NS, bool PK = false>
__global__ void __launch_bounds__(NT) split_block_kernel(int64_t outer, int64_t k, int64_t KB,
                                                         const double* __restrict__ hi,
                                                         const double* __restrict__ lo, int64_t ld,
                                                         int32_t* __restrict__ exps,
                                                         double* __restrict__ slices) {
    constexpr int kWavesPerBlock = NT / 64;
    constexpr int kRowsPerWave = 16 / kWavesPerBlock;  // AXIS 0
    constexpr int kRowGroups = NT / 16;                // AXIS 1
    __shared__ int codes[NT];
    __shared__ int block_exp[16];
    const int t = threadIdx.x;
    const int64_t blk = blockIdx.x;
    const int64_t o0 = blk * 16;
    const int64_t kparts = gridDim.y;
    const int64_t kb_begin = KB * blockIdx.y / kparts, kb_end = KB * (blockIdx.y + 1) / kparts;

    // Phase 1: exponents of the block's 16 rows/columns.
    if (AXIS == 0) {
        // each wave scans kRowsPerWave rows; lane L takes k indices L, L+64, ...
        const int lane = t & 63, w = t >> 6;
#pragma unroll 1
        for (int i = 0; i < kRowsPerWave; ++i) {
            const int64_t o = o0 + kRowsPerWave * w + i;
            int c = kNoExp;
            if (o < outer) {
                const double* h = hi + o * ld;
                const double* l = lo ? lo + o * ld : nullptr;
                int64_t p = lane;
                for (; p + 192 < k; p += 256) {
                    double xh[4], xl[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        xh[u] = h[p + 64 * u];
                        xl[u] = l ? l[p + 64 * u] : 0.0;
                    }
#pragma unroll
                    for (int u = 0; u < 4; ++u) c = max(c, entry_exp_code(xh[u], xl[u]));
                }
                for (; p < k; p += 64) c = max(c, entry_exp_code(h[p], l ? l[p] : 0.0));
            }
            c = wave_max(c);
            if (lane == 0) block_exp[kRowsPerWave * w + i] = decode_exp(c);
        }
    } else {
        // thread t takes column o0 + t % 16 over rows t / 16, t / 16 + kRowGroups, ...
        const int j = t & 15;
        const int64_t o = o0 + j;
        int code = kNoExp;
        if (o < outer) {
            int64_t p = t >> 4;
            for (; p + 3 * kRowGroups < k; p += 4 * kRowGroups) {
                double xh[4], xl[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    xh[u] = hi[(p + kRowGroups * u) * ld + o];
                    xl[u] = lo ? lo[(p + kRowGroups * u) * ld + o] : 0.0;
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) code = max(code, entry_exp_code(xh[u], xl[u]));
            }
            for (; p < k; p += kRowGroups) code = max(code, entry_exp_code(hi[p * ld + o], lo ? lo[p * ld + o] : 0.0));
        }
        codes[t] = code;
        __syncthreads();
        if (t < 16) {
            int c = kNoExp;
            for (int g = 0; g < kRowGroups; ++g) c = max(c, codes[g * 16 + t]);
            block_exp[t] = decode_exp(c);
        }
    }
    __syncthreads();
    if (blockIdx.y == 0 && t < 16 && o0 + t < outer) exps[o0 + t] = block_exp[t];

    // Phase 2: slices, two neighbouring packed lanes (entries o, o+1 at one p) per
    // thread and one 16-byte store per slice.
    const int64_t pairs = (kb_end - kb_begin) * 32;
    for (int64_t q = t; q < pairs; q += NT) {
        const int64_t kb = kb_begin + (q >> 5);
        const int lane = static_cast<int>(q & 31) * 2;
        const int oi = lane & 15;
        const int64_t p = kb * 4 + (lane >> 4);
        double sl0[NS], sl1[NS];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int64_t o = o0 + oi + e;
            double x_hi = 0.0, x_lo = 0.0;
            if (o < outer && p < k) {
                const int64_t idx = AXIS == 0 ? o * ld + p : p * ld + o;
                x_hi = hi[idx];
                x_lo = lo ? lo[idx] : 0.0;
            }
            slice_entry<NS>(x_hi, x_lo, block_exp[oi + e], e == 0 ? sl0 : sl1);
        }
        if constexpr (PK) {
            pair_pack<NS>(sl0);
            pair_pack<NS>(sl1);
        }
        double2* dst = reinterpret_cast<double2*>(slices + (blk * KB + kb) * (NS * kFragDoubles) + lane);
#pragma unroll
        for (int s = 0; s < NS; ++s) dst[s * (kFragDoubles / 2)] = make_double2(sl0[s], sl1[s]);
    }
}

// One pass per 16-row (AXIS 0) or 16-column (AXIS 1) block whose (hi, lo) fits
// the workgroup's registers (KB * 32 <= NT * PPT pairs of entries): every
// thread loads, in packed order, the PPT pairs of entries it will slice, the
// block's 16 exponents are reduced from those registers, and the slices are
// cut from them, so the operand is read from HBM exactly once.  Pair q covers
// packed lanes 2(q % 32), 2(q % 32) + 1 of k-block q / 32; as NT is a multiple
// of 32, thread t's pairs all lie on outer indices oi, oi + 1 with
// oi = 2(t % 8).
template <int AXIS, int NT, int NS, int PPT, bool PK = false>
__global__ void __launch_bounds__(NT) split_block_regs_kernel(int64_t outer, int64_t k, int64_t KB,
                                                              const double* __restrict__ hi,
                                                              const double* __restrict__ lo, int64_t ld,
                                                              int32_t* __restrict__ exps,
                                                              double* __restrict__ slices) {
    static_assert(NT % 64 == 0, "whole waves");
    __shared__ int block_code[16];
    const int t = threadIdx.x;
    const int64_t blk = blockIdx.x;
    const int64_t o0 = blk * 16;
    const int64_t pairs = KB * 32;
    const int oi = (t & 7) * 2;
    if (t < 16) block_code[t] = kNoExp;

    double xh[PPT][2], xl[PPT][2];
    int c0 = kNoExp, c1 = kNoExp;
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
        const int64_t q = t + static_cast<int64_t>(i) * NT;
        const int64_t p = (q >> 5) * 4 + (((q & 31) * 2) >> 4);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int64_t o = o0 + oi + e;
            xh[i][e] = 0.0;
            xl[i][e] = 0.0;
            if (q < pairs && o < outer && p < k) {
                const int64_t idx = AXIS == 0 ? o * ld + p : p * ld + o;
                xh[i][e] = hi[idx];
                xl[i][e] = lo ? lo[idx] : 0.0;
            }
        }
        c0 = max(c0, entry_exp_code(xh[i][0], xl[i][0]));
        c1 = max(c1, entry_exp_code(xh[i][1], xl[i][1]));
    }
    // lanes l, l ^ 8, l ^ 16, l ^ 32 of a wave share oi; then one LDS max per wave
#pragma unroll
    for (int off = 8; off <= 32; off <<= 1) {
        c0 = max(c0, __shfl_xor(c0, off, 64));
        c1 = max(c1, __shfl_xor(c1, off, 64));
    }
    __syncthreads();  // block_code initialised
    if ((t & 63) < 8) {
        atomicMax(&block_code[oi], c0);
        atomicMax(&block_code[oi + 1], c1);
    }
    __syncthreads();
    if (t < 16 && o0 + t < outer) exps[o0 + t] = decode_exp(block_code[t]);
    const int e0 = decode_exp(block_code[oi]), e1 = decode_exp(block_code[oi + 1]);

#pragma unroll
    for (int i = 0; i < PPT; ++i) {
        const int64_t q = t + static_cast<int64_t>(i) * NT;
        if (q >= pairs) break;
        double sl0[NS], sl1[NS];
        slice_entry<NS>(xh[i][0], xl[i][0], e0, sl0);
        slice_entry<NS>(xh[i][1], xl[i][1], e1, sl1);
        if constexpr (PK) {
            pair_pack<NS>(sl0);
            pair_pack<NS>(sl1);
        }
        const int lane = static_cast<int>(q & 31) * 2;
        double2* dst = reinterpret_cast<double2*>(slices + (blk * KB + (q >> 5)) * (NS * kFragDoubles) + lane);
#pragma unroll
        for (int s = 0; s < NS; ++s) dst[s * (kFragDoubles / 2)] = make_double2(sl0[s], sl1[s]);
    }
}

// Blocks needed before the one-pass block kernel beats two streaming passes
// (measured: 4096 blocks of k = 512 win, 256 blocks of k = 4096 lose).
constexpr int64_t kFusedMinBlocks = 1024;
// A B operand (column exponents: two passes take four launches) of at most
// kSmallColsBytes of (hi, lo) is sliced in one pass with its k-blocks shared
// among enough workgroups, as long as the parts' exponent re-reads (every part
// re-reads its block) stay within kSmallColsReread bytes and so hit the cache
// (measured on gfx950: 1024^2 29 vs 44 us with 256 MB re-read, 1536^2 61 vs
// 59 us with 396 MB, 4096^2 483 vs 339 us).
constexpr int64_t kSmallColsBytes = 24ll << 20;
// Pairs of entries per thread of the register-resident block kernel: 16 rows
// (columns) of up to 512 values of k with 1024 threads.
constexpr int kRegPairs = 4;
constexpr int64_t kSmallColsReread = 320ll << 20;

template <int NS>
hipError_t launch_split_ns(int64_t rows, int64_t cols, const double* X_hi, const double* X_lo,
                           int64_t ldx, int axis, int32_t* exps, double* slices, hipStream_t stream,
                           int phases, bool pairs) {
    const int64_t outer = axis == 0 ? rows : cols;
    const int64_t k = axis == 0 ? cols : rows;
    if (outer == 0) return hipSuccess;
    const PackGeom g(outer, k);
    constexpr int kBlockThreads = 1024;
    int64_t kparts = (kFusedMinBlocks + g.RB - 1) / g.RB;
    if (kparts > g.KB) kparts = g.KB;
    const int64_t bytes = rows * cols * 16;
    const bool small_cols = axis == 1 && bytes <= kSmallColsBytes && bytes * kparts <= kSmallColsReread;
    if (g.doubles(NS) > 0 && (g.RB >= kFusedMinBlocks || small_cols)) {
        // One pass per block; k-blocks shared among parts when blocks are few.
        // All of it belongs to the slice phase.
        if (!(phases & kSplitSlices)) return hipSuccess;
        if (kparts == 1 && g.KB * 32 <= kBlockThreads * kRegPairs) {
            // the whole block in registers: one read of the operand
            const unsigned blocks = static_cast<unsigned>(g.RB);
            if (axis == 0 && pairs)
                split_block_regs_kernel<0, kBlockThreads, NS, kRegPairs, true><<<blocks, kBlockThreads, 0, stream>>>(
                    outer, k, g.KB, X_hi, X_lo, ldx, exps, slices);
            else if (axis == 0)
                split_block_regs_kernel<0, kBlockThreads, NS, kRegPairs><<<blocks, kBlockThreads, 0, stream>>>(
                    outer, k, g.KB, X_hi, X_lo, ldx, exps, slices);
            else
                split_block_regs_kernel<1, kBlockThreads, NS, kRegPairs><<<blocks, kBlockThreads, 0, stream>>>(
                    outer, k, g.KB, X_hi, X_lo, ldx, exps, slices);
            return hipGetLastError();
        }
        const dim3 grid(static_cast<unsigned>(g.RB), static_cast<unsigned>(kparts));
        if (axis == 0 && pairs)
            split_block_kernel<0, kBlockThreads, NS, true><<<grid, kBlockThreads, 0, stream>>>(
                outer, k, g.KB, X_hi, X_lo, ldx, exps, slices);
        else if (axis == 0)
            split_block_kernel<0, kBlockThreads, NS><<<grid, kBlockThreads, 0, stream>>>(
                outer, k, g.KB, X_hi, X_lo, ldx, exps, slices);
        else
            split_block_kernel<1, kBlockThreads, NS><<<grid, kBlockThreads, 0, stream>>>(
                outer, k, g.KB, X_hi, X_lo, ldx, exps, slices);
        return hipGetLastError();
    }
    // Otherwise two passes over the operand: exponents, then slices.
    if ((phases & kSplitExps) && axis == 0) {
        const int64_t parts = exp_row_parts(rows, cols);
        const dim3 grid(grid_for(rows, 4, 1 << 20), static_cast<unsigned>(parts));
        if (parts > 1) fill_int_kernel<<<grid_for(rows, 256, 4096), 256, 0, stream>>>(exps, rows, kNoExp);
        exp_rows_kernel<<<grid, 256, 0, stream>>>(rows, cols, X_hi, X_lo, ldx, exps);
        if (parts > 1) decode_exps_kernel<<<grid_for(rows, 256, 4096), 256, 0, stream>>>(exps, rows);
    } else if (phases & kSplitExps) {
        const int64_t parts = exp_col_parts(rows, cols);
        const dim3 grid(grid_for(cols, 16, 1 << 20), static_cast<unsigned>(parts));
        if (parts > 1) fill_int_kernel<<<grid_for(cols, 256, 4096), 256, 0, stream>>>(exps, cols, kNoExp);
        exp_cols_block_kernel<1024><<<grid, 1024, 0, stream>>>(rows, cols, X_hi, X_lo, ldx, exps);
        if (parts > 1) decode_exps_kernel<<<grid_for(cols, 256, 4096), 256, 0, stream>>>(exps, cols);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (!(phases & kSplitSlices) || g.doubles(NS) == 0) return hipSuccess;
    const int64_t total = g.RB * g.KB * kFragDoubles;
    const unsigned grid = grid_for(total, 256, 1 << 20);
    if (axis == 0 && pairs)
        slice_kernel<0, NS, true><<<grid, 256, 0, stream>>>(outer, k, g.KB, total, X_hi, X_lo, ldx, exps, slices);
    else if (axis == 0)
        slice_kernel<0, NS><<<grid, 256, 0, stream>>>(outer, k, g.KB, total, X_hi, X_lo, ldx, exps, slices);
    else
        slice_kernel<1, NS><<<grid, 256, 0, stream>>>(outer, k, g.KB, total, X_hi, X_lo, ldx, exps, slices);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_split(int64_t rows, int64_t cols, const double* X_hi, const double* X_lo,
                        int64_t ldx, int axis, int ns, int32_t* exps, double* slices, hipStream_t stream,
                        int phases, bool pairs) {
    switch (ns) {
        case 4: return launch_split_ns<4>(rows, cols, X_hi, X_lo, ldx, axis, exps, slices, stream, phases, pairs);
        case 5: return launch_split_ns<5>(rows, cols, X_hi, X_lo, ldx, axis, exps, slices, stream, phases, pairs);
        case 6: return launch_split_ns<6>(rows, cols, X_hi, X_lo, ldx, axis, exps, slices, stream, phases, pairs);
        case 7: return launch_split_ns<7>(rows, cols, X_hi, X_lo, ldx, axis, exps, slices, stream, phases, pairs);
        case 8: return launch_split_ns<8>(rows, cols, X_hi, X_lo, ldx, axis, exps, slices, stream, phases, pairs);
        case 9: return launch_split_ns<9>(rows, cols, X_hi, X_lo, ldx, axis, exps, slices, stream, phases, pairs);
        case 10: return launch_split_ns<10>(rows, cols, X_hi, X_lo, ldx, axis, exps, slices, stream, phases, pairs);
        case 11: return launch_split_ns<11>(rows, cols, X_hi, X_lo, ldx, axis, exps, slices, stream, phases, pairs);
        case 12: return launch_split_ns<12>(rows, cols, X_hi, X_lo, ldx, axis, exps, slices, stream, phases, pairs);
        case 13: return launch_split_ns<13>(rows, cols, X_hi, X_lo, ldx, axis, exps, slices, stream, phases, pairs);
        case 14: return launch_split_ns<14>(rows, cols, X_hi, X_lo, ldx, axis, exps, slices, stream, phases, pairs);
        case 15: return launch_split_ns<15>(rows, cols, X_hi, X_lo, ldx, axis, exps, slices, stream, phases, pairs);
        case 16: return launch_split_ns<16>(rows, cols, X_hi, X_lo, ldx, axis, exps, slices, stream, phases, pairs);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace ddg
