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

// The NS slices of x = hi + lo below E (|x| < 2^E), in the pair-packed layout
// when PK, as slice_entry then pair_pack compute them.  For NS <= 8 the window
// integer N = floor(|x| 2^(13 NS - E)) < 2^104 is formed as two 52-bit halves
// (N = H 2^52 + L), so that slice q -- bits [13 j, 13 j + 13) of N with
// j = NS - 1 - q -- is one shift and mask of one half, and a packed plane the
// integer 2^13 d_2u + d_2u+1, converted once.
template <int NS, bool PK>
__device__ __forceinline__ void slice_entry_fast(double hi, double lo, int E, double (&out)[NS]) {
    if constexpr (NS > kSlices) {
        slice_entry<NS>(hi, lo, E, out);
        if constexpr (PK) pair_pack<NS>(out);
    } else {
        constexpr uint64_t kMask52 = (1ull << 52) - 1;
        double s, e;
        two_sum(hi, lo, s, e);  // x = s + e exactly, |e| <= ulp(s)/2
        if (s == 0.0) {
#pragma unroll
            for (int q = 0; q < NS; ++q) out[q] = 0.0;
            return;
        }
        const bool neg = s < 0.0;
        const double ep = neg ? -e : e;  // |x| = |s| + ep
        uint64_t ms;
        int es;
        decompose(s, ms, es);
        const int W = E - kSliceBits * NS;  // exponent of the window's last unit
        uint64_t H, L;
        if (es >= W) {
            // |s| 2^-W = ms 2^sh with sh <= 13 NS - 52 <= 52 (|s| <= 2^E, as
            // RN(x) may reach 2^E); |floor(ep 2^-W)| <= 2^(sh-1) <= 2^51, so
            // adding it to L moves at most one unit between the halves
            const int sh = es - W;
            int64_t l = static_cast<int64_t>((ms << sh) & kMask52);
            int64_t h = static_cast<int64_t>(ms >> (52 - sh));
            if (ep != 0.0) {
                uint64_t me;
                int ee;
                decompose(ep, me, ee);
                l += floor_scaled(me, ep < 0.0, ee - W);
                if (l < 0) {
                    l += int64_t{1} << 52;
                    h -= 1;
                } else if (l >= (int64_t{1} << 52)) {
                    l -= int64_t{1} << 52;
                    h += 1;
                }
            }
            H = static_cast<uint64_t>(h);
            L = static_cast<uint64_t>(l);
        } else {
            // bits below the window: floor((ms + ep/2^es) / 2^d), |ep/2^es| <= 1/2
            const int d = W - es;
            uint64_t q = 0, r = ms;
            if (d < 64) {
                q = ms >> d;
                r = ms & ((1ull << d) - 1);
            }
            if (r == 0 && ep < 0.0) q -= 1;
            H = q >> 52;
            L = q & kMask52;
        }
        auto digit = [&](int j) -> uint32_t {  // bits [13 j, 13 j + 13) of N
            return static_cast<uint32_t>(j >= 4 ? H >> (kSliceBits * (j - 4)) : L >> (kSliceBits * j)) & 0x1FFFu;
        };
        auto scaled = [&](uint32_t v, int unit) -> double {  // sign(x) v 2^-unit; +0.0 for v = 0
            const int sv = neg ? -static_cast<int>(v) : static_cast<int>(v);
            return static_cast<double>(sv) * __longlong_as_double(static_cast<long long>(1023 - unit) << 52);
        };
#pragma unroll
        for (int q = 0; q < NS; ++q) {
            const int j = NS - 1 - q;
            if (PK && (q % 2 == 0) && q + 1 < NS)
                out[q] = scaled((digit(j) << kSliceBits) | digit(j - 1), kSliceBits * (q + 2));
            else if (PK && (q % 2 == 1))
                out[q] = scaled(digit(j + 1), kSliceBits * q);  // slice q - 1 alone
            else
                out[q] = scaled(digit(j), kSliceBits * (q + 1));
        }
    }
}

// One wave per row and k-part: E[row] = max frexp exponent over the row (axis
// 0, the A operand).  Part y of gridDim.y covers columns [cols y / parts,
// cols (y + 1) / parts).  With one part the decoded exponent is stored; with
// several the encoded maxima are folded into `exps` (cleared to kNoExp) with
// atomicMax and decoded after.  `pairs_aligned` (X_hi, X_lo and ld allow
// 16-byte loads) with one part: lane L reads the pairs L, L + 64, ... of its
// row, eight pairs in flight.
template <int kWgThreads>
__device__ __forceinline__ void exp_rows_part(int64_t wg, int64_t nwg, int64_t part, int64_t parts, int64_t rows,
                                              int64_t cols, const double* __restrict__ hi,
                                              const double* __restrict__ lo, int64_t ld, bool pairs_aligned,
                                              int32_t* __restrict__ exps) {
    constexpr int kInFlight = 8;
    const int lane = threadIdx.x & 63;
    const int64_t p0 = cols * part / parts, p1 = cols * (part + 1) / parts;
    const int64_t nwaves = nwg * (kWgThreads >> 6);
    const bool vec = pairs_aligned && parts == 1;
    for (int64_t row = wg * (kWgThreads >> 6) + (threadIdx.x >> 6); row < rows; row += nwaves) {
        const double* h = hi + row * ld;
        const double* l = lo ? lo + row * ld : nullptr;
        int code = kNoExp;
        int64_t p = p0 + lane;
        if (vec) {
            const double2* h2 = reinterpret_cast<const double2*>(h);
            const double2* l2 = reinterpret_cast<const double2*>(l);
            const int64_t npairs = cols / 2;
            int64_t j = lane;
            for (; j + 64 * (kInFlight - 1) < npairs; j += 64 * kInFlight) {
                double2 xh[kInFlight], xl[kInFlight];
#pragma unroll
                for (int u = 0; u < kInFlight; ++u) {
                    xh[u] = h2[j + 64 * u];
                    xl[u] = l2 ? l2[j + 64 * u] : make_double2(0.0, 0.0);
                }
#pragma unroll
                for (int u = 0; u < kInFlight; ++u)
                    code = max(code, max(entry_exp_code(xh[u].x, xl[u].x), entry_exp_code(xh[u].y, xl[u].y)));
            }
            for (; j < npairs; j += 64) {
                const double2 xh = h2[j], xl = l2 ? l2[j] : make_double2(0.0, 0.0);
                code = max(code, max(entry_exp_code(xh.x, xl.x), entry_exp_code(xh.y, xl.y)));
            }
            p = 2 * npairs + lane;  // an odd last value
        }
        for (; p < p1; p += 64) code = max(code, entry_exp_code(h[p], l ? l[p] : 0.0));
        code = wave_max(code);
        if (lane == 0) {
            if (parts == 1)
                exps[row] = decode_exp(code);
            else if (code != kNoExp)
                atomicMax(exps + row, code);
        }
    }
}

__global__ void __launch_bounds__(256) exp_rows_kernel(int64_t rows, int64_t cols,
                                                       const double* __restrict__ hi,
                                                       const double* __restrict__ lo, int64_t ld,
                                                       bool pairs_aligned, int32_t* __restrict__ exps) {
    exp_rows_part<256>(blockIdx.x, gridDim.x, blockIdx.y, gridDim.y, rows, cols, hi, lo, ld, pairs_aligned, exps);
}

// Column exponents (axis 1) by streaming whole rows: thread t of workgroup
// (b, c) takes columns o = 2(b NT + t), o + 1 over row part c of `parts`,
// reading each row of the part as consecutive 16-byte pairs (`pairs_aligned`:
// X_hi, X_lo and ld allow them; otherwise one double at a time).  With one part
// the decoded exponents go to `out`; with several each part stores its encoded
// maxima to partial[c][o] and fold_exps_kernel reduces them.  (A last-part
// fold inside the launch costs more than that launch: its device-scope fences
// write back the L2.)
template <int NT>
__device__ __forceinline__ void exp_cols_part(int64_t chunk, int64_t part, int64_t parts, int64_t rows,
                                              int64_t cols, const double* __restrict__ hi,
                                              const double* __restrict__ lo, int64_t ld, bool pairs_aligned,
                                              int32_t* __restrict__ out, int32_t* __restrict__ partial) {
    constexpr int kRowsInFlight = 8;
    const int64_t r0 = rows * part / parts, r1 = rows * (part + 1) / parts;
    const int64_t o = (chunk * NT + threadIdx.x) * 2;
    int c0 = kNoExp, c1 = kNoExp;
    if (o < cols && pairs_aligned && o + 1 < cols) {
        int64_t p = r0;
        for (; p + kRowsInFlight <= r1; p += kRowsInFlight) {
            double2 xh[kRowsInFlight], xl[kRowsInFlight];
#pragma unroll
            for (int u = 0; u < kRowsInFlight; ++u) {
                xh[u] = *reinterpret_cast<const double2*>(hi + (p + u) * ld + o);
                xl[u] = lo ? *reinterpret_cast<const double2*>(lo + (p + u) * ld + o) : make_double2(0.0, 0.0);
            }
#pragma unroll
            for (int u = 0; u < kRowsInFlight; ++u) {
                c0 = max(c0, entry_exp_code(xh[u].x, xl[u].x));
                c1 = max(c1, entry_exp_code(xh[u].y, xl[u].y));
            }
        }
        for (; p < r1; ++p) {
            c0 = max(c0, entry_exp_code(hi[p * ld + o], lo ? lo[p * ld + o] : 0.0));
            c1 = max(c1, entry_exp_code(hi[p * ld + o + 1], lo ? lo[p * ld + o + 1] : 0.0));
        }
    } else if (o < cols) {
        const bool two = o + 1 < cols;
        for (int64_t p = r0; p < r1; ++p) {
            c0 = max(c0, entry_exp_code(hi[p * ld + o], lo ? lo[p * ld + o] : 0.0));
            if (two) c1 = max(c1, entry_exp_code(hi[p * ld + o + 1], lo ? lo[p * ld + o + 1] : 0.0));
        }
    }
    if (parts == 1) {
        if (o < cols) out[o] = decode_exp(c0);
        if (o + 1 < cols) out[o + 1] = decode_exp(c1);
        return;
    }
    if (o < cols) partial[part * cols + o] = c0;
    if (o + 1 < cols) partial[part * cols + o + 1] = c1;
}

template <int NT>
__global__ void __launch_bounds__(NT) exp_cols_stream_kernel(int64_t rows, int64_t cols,
                                                             const double* __restrict__ hi,
                                                             const double* __restrict__ lo, int64_t ld,
                                                             bool pairs_aligned, int32_t* __restrict__ out,
                                                             int32_t* __restrict__ partial) {
    exp_cols_part<NT>(blockIdx.x, blockIdx.y, gridDim.y, rows, cols, hi, lo, ld, pairs_aligned, out, partial);
}

// The decoded maximum of partial[c][o] over the parts c.
__device__ __forceinline__ int32_t fold_column(int64_t parts, int64_t cols, const int32_t* __restrict__ partial,
                                               int64_t o) {
    int c = kNoExp;
    int64_t q = 0;
    for (; q + 8 <= parts; q += 8) {  // eight independent loads in flight
        int v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = partial[(q + u) * cols + o];
#pragma unroll
        for (int u = 0; u < 8; ++u) c = max(c, v[u]);
    }
    for (; q < parts; ++q) c = max(c, partial[q * cols + o]);
    return decode_exp(c);
}

// out[o] = the decoded maximum of partial[c][o] over the parts c.
__global__ void __launch_bounds__(256) fold_exps_kernel(int64_t parts, int64_t cols,
                                                        const int32_t* __restrict__ partial,
                                                        int32_t* __restrict__ out) {
    for (int64_t o = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; o < cols;
         o += static_cast<int64_t>(gridDim.x) * blockDim.x)
        out[o] = fold_column(parts, cols, partial, o);
}

// The B operand's (axis 1) slices after leading-word exponents, one thread
// per packed (fragment, lane) position: workgroup (x, y) takes column block x
// (columns 16x .. 16x+15) and k-blocks 4y .. 4y+3 (KB is a multiple of 4), so
// the workgroups in flight, neighbours in x, read whole row segments of B; no
// index needs a division.  The entry of lane L of k-block kb is B[4 kb +
// L / 16][16 x + L % 16].  CHECK: the exponents came from the leading words
// alone, which is exact when every pair of the column has hi = RN(hi + lo); a
// pair that does not replaces its column's exponent by kUnnormalised, and the
// entries of such a column are written as zeros here; the exact pass
// (split_block_kernel with FIXUP) recomputes the column's exponent from
// (hi, lo) and re-slices it.
template <int NS, bool CHECK>
__global__ void __launch_bounds__(256) slice_cols_kernel(int64_t outer, int64_t k, int64_t KB,
                                                         const double* __restrict__ hi,
                                                         const double* __restrict__ lo, int64_t ld, int32_t* exps,
                                                         double* __restrict__ slices) {
    const int lane = threadIdx.x & 63;
    const int64_t ob = blockIdx.x;
    const int64_t o = ob * 16 + (lane & 15);
    const bool in_o = o < outer;
    for (int64_t kb = static_cast<int64_t>(blockIdx.y) * 4 + (threadIdx.x >> 6); kb < KB;
         kb += static_cast<int64_t>(gridDim.y) * 4) {
        const int64_t p = kb * 4 + (lane >> 4);
        double x_hi = 0.0, x_lo = 0.0;
        int E = 0;
        if (in_o && p < k) {
            x_hi = hi[p * ld + o];
            x_lo = lo ? lo[p * ld + o] : 0.0;
            E = exps[o];
            if constexpr (CHECK) {
                if (x_hi + x_lo != x_hi) {
                    exps[o] = kUnnormalised;
                    E = kUnnormalised;
                }
            }
        }
        double sl[NS];
        if (CHECK && E == kUnnormalised) {
#pragma unroll
            for (int q = 0; q < NS; ++q) sl[q] = 0.0;
        } else {
            slice_entry_fast<NS, false>(x_hi, x_lo, E, sl);
        }
        // the slices are read back only by the GEMM: stream them past the caches
        double* dst = slices + (ob * KB + kb) * (NS * kFragDoubles) + lane;
#pragma unroll
        for (int q = 0; q < NS; ++q) __builtin_nontemporal_store(sl[q], dst + q * kFragDoubles);
    }
}

// The B operand's (axis 1) slices through LDS: workgroup (x, y) takes the tile
// of 64 columns (column blocks 4x .. 4x+3) and 16 rows (k-blocks 4y .. 4y+3),
// reads each row's part as one run of 64 doubles, and writes the tile's 16
// fragments, every slice plane as one 512-byte run.  Neighbouring workgroups
// take neighbouring columns of the same rows.  RB and KB (the padded layout's
// column and k-blocks) are multiples of 4.  CHECK as in slice_cols_kernel.
// STREAM: non-temporal stores, which leave no dirty lines for the next kernel
// to write back (plain stores are faster when a long kernel follows, such as
// the GEMM).
template <int NS, bool CHECK, bool STREAM>
__global__ void __launch_bounds__(256) slice_cols_lds_kernel(int64_t outer, int64_t k, int64_t KB,
                                                             const double* __restrict__ hi,
                                                             const double* __restrict__ lo, int64_t ld,
                                                             bool pairs_aligned, int32_t* exps,
                                                             double* __restrict__ slices) {
    constexpr int kPad = 64 + 1;  // rows kPad doubles apart
    __shared__ double th[16 * kPad], tl[16 * kPad];
    const int t = threadIdx.x;
    const int r = t >> 4, c = (t & 15) * 4;  // load: row r of the tile, columns c .. c+3
    const int64_t o0 = static_cast<int64_t>(blockIdx.x) * 64;
    for (int64_t kg = blockIdx.y; kg * 4 < KB; kg += gridDim.y) {  // uniform per workgroup
        const int64_t p0 = kg * 16;
        const int64_t p = p0 + r, o = o0 + c;
        double vh[4] = {0.0, 0.0, 0.0, 0.0}, vl[4] = {0.0, 0.0, 0.0, 0.0};
        if (p < k) {
            const double* h = hi + p * ld + o;
            const double* l = lo ? lo + p * ld + o : nullptr;
            if (pairs_aligned && o + 3 < outer) {
                const double2 h0 = reinterpret_cast<const double2*>(h)[0], h1 = reinterpret_cast<const double2*>(h)[1];
                vh[0] = h0.x, vh[1] = h0.y, vh[2] = h1.x, vh[3] = h1.y;
                if (l) {
                    const double2 l0 = reinterpret_cast<const double2*>(l)[0];
                    const double2 l1 = reinterpret_cast<const double2*>(l)[1];
                    vl[0] = l0.x, vl[1] = l0.y, vl[2] = l1.x, vl[3] = l1.y;
                }
            } else {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    if (o + u < outer) {
                        vh[u] = h[u];
                        vl[u] = l ? l[u] : 0.0;
                    }
                }
            }
        }
        __syncthreads();  // the previous tile's reads of th, tl are done
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            th[r * kPad + c + u] = vh[u];
            tl[r * kPad + c + u] = vl[u];
        }
        __syncthreads();
        // four entries per thread in packed order: fragment f (column block
        // f / 4, k-block f % 4 of the tile), lane L
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int gi = t + 256 * e;
            const int f = gi >> 6, lane = gi & 63;
            const int ci = (f >> 2) * 16 + (lane & 15), ri = (f & 3) * 4 + (lane >> 4);
            const double x_hi = th[ri * kPad + ci], x_lo = tl[ri * kPad + ci];
            const int64_t col = o0 + ci;
            int E = 0;
            if (col < outer) {
                E = exps[col];
                if constexpr (CHECK) {
                    if (x_hi + x_lo != x_hi) {
                        exps[col] = kUnnormalised;
                        E = kUnnormalised;
                    }
                }
            }
            double sl[NS];
            if (CHECK && E == kUnnormalised) {
#pragma unroll
                for (int q = 0; q < NS; ++q) sl[q] = 0.0;
            } else {
                slice_entry_fast<NS, false>(x_hi, x_lo, E, sl);
            }
            double* dst = slices + ((o0 / 16 + (f >> 2)) * KB + kg * 4 + (f & 3)) * (NS * kFragDoubles) + lane;
#pragma unroll
            for (int q = 0; q < NS; ++q) {
                if constexpr (STREAM)
                    __builtin_nontemporal_store(sl[q], dst + q * kFragDoubles);
                else
                    dst[q * kFragDoubles] = sl[q];
            }
        }
    }
}

// The A operand's (axis 0) slices through LDS: a workgroup takes a tile of 16
// rows and kTileK values of k (kTileK / 4 fragments), reads each row's part as
// one run of kTileK doubles, and writes every slice plane of a fragment as one
// 512-byte run.  The tiles cover the padded layout (RB row blocks of 16, KB
// k-blocks of 4), whose entries beyond the operand get zero slices.  CHECK as
// in slice_cols_kernel.  `pairs_aligned`: X_hi, X_lo and ld allow 16-byte loads.
template <int NS, bool PK, bool CHECK, bool STREAM>
__device__ __forceinline__ void slice_rows_tiles(int64_t first, int64_t stride, int64_t outer, int64_t k, int64_t RB,
                                                 int64_t KB, const double* __restrict__ hi,
                                                 const double* __restrict__ lo, int64_t ld, bool pairs_aligned,
                                                 int32_t* exps, double* __restrict__ slices) {
    constexpr int kTileK = 64;
    constexpr int kPad = kTileK + 1;  // rows kPad doubles apart: the fragment-order reads hit distinct banks
    __shared__ double th[16 * kPad], tl[16 * kPad];
    const int t = threadIdx.x;
    const int64_t tiles_k = (KB + kTileK / 4 - 1) / (kTileK / 4);
    const int64_t tiles = RB * tiles_k;
    const int r = t >> 4, c = (t & 15) * 4;  // load: row r, k values c .. c+3 of the tile
    for (int64_t tile = first; tile < tiles; tile += stride) {  // uniform per workgroup
        const int64_t rb = tile / tiles_k, p0 = (tile % tiles_k) * kTileK;
        const int64_t o = rb * 16 + r, p = p0 + c;
        double vh[4] = {0.0, 0.0, 0.0, 0.0}, vl[4] = {0.0, 0.0, 0.0, 0.0};
        if (o < outer) {
            const double* h = hi + o * ld + p;
            const double* l = lo ? lo + o * ld + p : nullptr;
            if (pairs_aligned && p + 3 < k) {
                const double2 h0 = reinterpret_cast<const double2*>(h)[0], h1 = reinterpret_cast<const double2*>(h)[1];
                vh[0] = h0.x, vh[1] = h0.y, vh[2] = h1.x, vh[3] = h1.y;
                if (l) {
                    const double2 l0 = reinterpret_cast<const double2*>(l)[0];
                    const double2 l1 = reinterpret_cast<const double2*>(l)[1];
                    vl[0] = l0.x, vl[1] = l0.y, vl[2] = l1.x, vl[3] = l1.y;
                }
            } else {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    if (p + u < k) {
                        vh[u] = h[u];
                        vl[u] = l ? l[u] : 0.0;
                    }
                }
            }
        }
        __syncthreads();  // the previous tile's reads of th, tl are done
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            th[r * kPad + c + u] = vh[u];
            tl[r * kPad + c + u] = vl[u];
        }
        __syncthreads();
        // four entries per thread in packed order: fragment f, lane L
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int gi = t + 256 * e;
            const int f = gi >> 6, lane = gi & 63;
            const int oi = lane & 15, pi = 4 * f + (lane >> 4);
            const int64_t kb = p0 / 4 + f;
            if (kb >= KB) continue;
            const double x_hi = th[oi * kPad + pi], x_lo = tl[oi * kPad + pi];
            const int64_t row = rb * 16 + oi;
            int E = 0;
            if (row < outer) {
                E = exps[row];
                if constexpr (CHECK) {
                    if (x_hi + x_lo != x_hi) {
                        exps[row] = kUnnormalised;
                        E = kUnnormalised;
                    }
                }
            }
            double sl[NS];
            if (CHECK && E == kUnnormalised) {
#pragma unroll
                for (int q = 0; q < NS; ++q) sl[q] = 0.0;
            } else {
                slice_entry_fast<NS, PK>(x_hi, x_lo, E, sl);
            }
            double* dst = slices + (rb * KB + kb) * (NS * kFragDoubles) + lane;
#pragma unroll
            for (int q = 0; q < NS; ++q) {
                if constexpr (STREAM)
                    __builtin_nontemporal_store(sl[q], dst + q * kFragDoubles);
                else
                    dst[q * kFragDoubles] = sl[q];
            }
        }
    }
}

template <int NS, bool PK, bool CHECK, bool STREAM>
__global__ void __launch_bounds__(256) slice_rows_lds_kernel(int64_t outer, int64_t k, int64_t RB, int64_t KB,
                                                             const double* __restrict__ hi,
                                                             const double* __restrict__ lo, int64_t ld,
                                                             bool pairs_aligned, int32_t* exps,
                                                             double* __restrict__ slices) {
    slice_rows_tiles<NS, PK, CHECK, STREAM>(blockIdx.x, gridDim.x, outer, k, RB, KB, hi, lo, ld, pairs_aligned, exps,
                                            slices);
}

// Workgroups (b, c) for 16-row (AXIS 0) or 16-column (AXIS 1) block b and part c
// of its k-blocks: first the block's balancing exponents, then the slices of
// the part's k-blocks, so the second read of the block's (hi, lo) comes from
// cache rather than HBM and no atomics are needed.  With several parts every
// part computes the block's exponents (its re-reads hit the cache while the
// operand fits there) and part 0 stores them.
//
// FIXUP (one part): the exact pass after the slice kernels' CHECK -- a block none of
// whose 16 rows (columns) is marked kUnnormalised returns at once; otherwise its
// exponents and slices are recomputed from (hi, lo).
template <int AXIS, int NT, int NS, bool PK, bool FIXUP>
__device__ __forceinline__ void split_block(int64_t blk, int64_t kpart, int64_t kparts, int64_t outer, int64_t k,
                                            int64_t KB, const double* __restrict__ hi,
                                            const double* __restrict__ lo, int64_t ld, int32_t* __restrict__ exps,
                                            double* __restrict__ slices) {
    constexpr int kWavesPerBlock = NT / 64;
    constexpr int kRowsPerWave = 16 / kWavesPerBlock;  // AXIS 0
    constexpr int kRowGroups = NT / 16;                // AXIS 1
    __shared__ int codes[NT];
    __shared__ int block_exp[16];
    const int t = threadIdx.x;
    const int64_t o0 = blk * 16;
    const int64_t kb_begin = KB * kpart / kparts, kb_end = KB * (kpart + 1) / kparts;
    if constexpr (FIXUP) {
        const bool marked = t < 16 && o0 + t < outer && exps[o0 + t] == kUnnormalised;
        if (!__syncthreads_or(marked)) return;  // uniform over the workgroup
    }

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
    if (kpart == 0 && t < 16 && o0 + t < outer) exps[o0 + t] = block_exp[t];

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
            slice_entry_fast<NS, PK>(x_hi, x_lo, block_exp[oi + e], e == 0 ? sl0 : sl1);
        }
        double2* dst = reinterpret_cast<double2*>(slices + (blk * KB + kb) * (NS * kFragDoubles) + lane);
#pragma unroll
        for (int s = 0; s < NS; ++s) dst[s * (kFragDoubles / 2)] = make_double2(sl0[s], sl1[s]);
    }
}

template <int AXIS, int NT, int NS, bool PK = false, bool FIXUP = false>
__global__ void __launch_bounds__(NT) split_block_kernel(int64_t outer, int64_t k, int64_t KB,
                                                         const double* __restrict__ hi,
                                                         const double* __restrict__ lo, int64_t ld,
                                                         int32_t* __restrict__ exps,
                                                         double* __restrict__ slices) {
    split_block<AXIS, NT, NS, PK, FIXUP>(blockIdx.x, blockIdx.y, gridDim.y, outer, k, KB, hi, lo, ld, exps, slices);
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
        slice_entry_fast<NS, PK>(xh[i][0], xl[i][0], e0, sl0);
        slice_entry_fast<NS, PK>(xh[i][1], xl[i][1], e1, sl1);
        const int lane = static_cast<int>(q & 31) * 2;
        double2* dst = reinterpret_cast<double2*>(slices + (blk * KB + (q >> 5)) * (NS * kFragDoubles) + lane);
#pragma unroll
        for (int s = 0; s < NS; ++s) dst[s * (kFragDoubles / 2)] = make_double2(sl0[s], sl1[s]);
    }
}

// One launch for A's row exponents (the first `row_wgs` workgroups, one wave
// per row, leading words) and B's exact pass (one workgroup per 16-column
// block of B).
template <int NS>
__global__ void __launch_bounds__(256) exp_rows_fix_kernel(int64_t m, int64_t ka, const double* __restrict__ a_hi,
                                                           int64_t lda, bool a_aligned, int32_t* __restrict__ E,
                                                           int64_t row_wgs, int64_t n, int64_t KBb,
                                                           const double* __restrict__ b_hi,
                                                           const double* __restrict__ b_lo, int64_t ldb,
                                                           int32_t* __restrict__ F, double* __restrict__ B_sl) {
    const int64_t b = blockIdx.x;
    if (b < row_wgs)
        exp_rows_part<256>(b, row_wgs, 0, 1, m, ka, a_hi, nullptr, lda, a_aligned, E);
    else
        split_block<1, 256, NS, false, true>(b - row_wgs, 0, 1, n, ka, KBb, b_hi, b_lo, ldb, F, B_sl);
}

// Both operands of a small product in one launch of the one-pass block
// kernel: workgroups [0, na) take A's 16-row blocks (pair-packed) in ka_parts
// k-parts each, the rest B's 16-column blocks in kb_parts k-parts.
template <int NS>
__global__ void __launch_bounds__(1024) split_both_block_kernel(
    int64_t m, int64_t k, int64_t KB, const double* __restrict__ a_hi, const double* __restrict__ a_lo, int64_t lda,
    int32_t* __restrict__ E, double* __restrict__ A_sl, int64_t ka_parts, int64_t na, int64_t n,
    const double* __restrict__ b_hi, const double* __restrict__ b_lo, int64_t ldb, int32_t* __restrict__ F,
    double* __restrict__ B_sl, int64_t kb_parts) {
    const int64_t b = blockIdx.x;
    if (b < na)
        split_block<0, 1024, NS, true, false>(b / ka_parts, b % ka_parts, ka_parts, m, k, KB, a_hi, a_lo, lda, E, A_sl);
    else
        split_block<1, 1024, NS, false, false>((b - na) / kb_parts, (b - na) % kb_parts, kb_parts, n, k, KB, b_hi, b_lo,
                                              ldb, F, B_sl);
}

// Blocks needed before the one-pass block kernel beats two streaming passes
// (measured: 4096 blocks of k = 512 win, 256 blocks of k = 4096 lose).
constexpr int64_t kFusedMinBlocks = 1024;
// Workgroups a one-pass launch of fewer blocks shares their k-blocks among
// (every part re-reads its whole block for the exponents, so fewer parts read
// less: B of 1024^2 27.5 -> about 19 us, the 1024^3 slicing 50.4 -> 42.2 us, 512^3
// 30.6 -> 23.8 us against 1024 workgroups; results bit-identical).
constexpr int64_t kOnePassWorkgroups = 256;
// A B operand (column exponents: two passes take four launches) of at most
// kSmallColsBytes of (hi, lo) is sliced in one pass with its k-blocks shared
// among enough workgroups, as long as the parts' exponent re-reads (every part
// re-reads its block) stay within kSmallColsReread bytes and so hit the cache
// (measured on gfx950 with parts for 1024 workgroups: 1024^2 29 vs 44 us
// with 256 MB re-read, 1536^2 61 vs 59 us with 396 MB, 4096^2 483 vs 339 us).
constexpr int64_t kSmallColsBytes = 24ll << 20;
// Pairs of entries per thread of the register-resident block kernel: 16 rows
// (columns) of up to 512 values of k with 1024 threads.
constexpr int kRegPairs = 4;
constexpr int64_t kSmallColsReread = 320ll << 20;
// An A operand of at most this many bytes of (hi, lo) also takes the one-pass
// block kernels.
constexpr int64_t kSmallRowsBytes = 2ll << 20;
// Streaming column-exponent pass: row parts enough for this many workgroups of
// 512 columns, each part at least kMinRowsPerStreamPart rows (which also keeps
// the parts' partial maxima, 4 bytes per column and part, within the slice
// buffer they borrow).
constexpr int64_t kExpColStreamWorkgroups = 256;
constexpr int64_t kMinRowsPerStreamPart = 32;

// Whether an operand is sliced by the one-pass block kernels (true) or in two
// passes; kparts: the k-parts a one-pass launch shares a block among.
inline bool one_pass(const PackGeom& g, int64_t rows, int64_t cols, int axis, int ns, int64_t& kparts) {
    kparts = (kOnePassWorkgroups + g.RB - 1) / g.RB;
    if (kparts > g.KB) kparts = g.KB;
    const int64_t bytes = rows * cols * 16;
    const bool small_cols = axis == 1 && bytes <= kSmallColsBytes && bytes * kparts <= kSmallColsReread;
    // a small A operand: one launch rather than three of a few microseconds each
    const bool small_rows = axis == 0 && bytes <= kSmallRowsBytes && bytes * kparts <= kSmallColsReread;
    return g.doubles(ns) > 0 && (g.RB >= kFusedMinBlocks || small_cols || small_rows);
}

// Row parts of the streaming column-exponent pass over a rows x cols operand.
inline int64_t stream_col_parts(int64_t rows, int64_t cols) {
    const int64_t chunks = exp_col_chunks(cols);
    int64_t parts = (kExpColStreamWorkgroups + chunks - 1) / chunks;
    const int64_t most = rows / kMinRowsPerStreamPart > 1 ? rows / kMinRowsPerStreamPart : 1;
    if (parts > most) parts = most;
    if (parts > 65535) parts = 65535;
    return parts;
}

inline bool pairs_aligned(const double* hi, const double* lo, int64_t ld) {
    return ld % 2 == 0 && reinterpret_cast<uintptr_t>(hi) % 16 == 0 && reinterpret_cast<uintptr_t>(lo) % 16 == 0;
}

constexpr int kBlockThreads = 1024;
constexpr int kFixThreads = 256;
constexpr int kColThreads = static_cast<int>(kExpColChunk / 2);

template <int NS>
void launch_one_pass(const PackGeom& g, int64_t kparts, int64_t outer, int64_t k, const double* X_hi,
                     const double* X_lo, int64_t ldx, int axis, int32_t* exps, double* slices, hipStream_t stream,
                     bool pairs) {
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
        return;
    }
    const dim3 grid(static_cast<unsigned>(g.RB), static_cast<unsigned>(kparts));
    if (axis == 0 && pairs)
        split_block_kernel<0, kBlockThreads, NS, true><<<grid, kBlockThreads, 0, stream>>>(outer, k, g.KB, X_hi, X_lo,
                                                                                          ldx, exps, slices);
    else if (axis == 0)
        split_block_kernel<0, kBlockThreads, NS><<<grid, kBlockThreads, 0, stream>>>(outer, k, g.KB, X_hi, X_lo, ldx,
                                                                                    exps, slices);
    else
        split_block_kernel<1, kBlockThreads, NS><<<grid, kBlockThreads, 0, stream>>>(outer, k, g.KB, X_hi, X_lo, ldx,
                                                                                    exps, slices);
}

// Two-pass exponents of the leading words of A's rows (axis 0).
void launch_exps_rows(int64_t rows, int64_t cols, const double* X_hi, int64_t ldx, int32_t* exps, hipStream_t stream) {
    const int64_t parts = exp_row_parts(rows, cols);
    const dim3 grid(grid_for(rows, 4, 1 << 20), static_cast<unsigned>(parts));
    if (parts > 1) fill_int_kernel<<<grid_for(rows, 256, 4096), 256, 0, stream>>>(exps, rows, kNoExp);
    exp_rows_kernel<<<grid, 256, 0, stream>>>(rows, cols, X_hi, nullptr, ldx, pairs_aligned(X_hi, nullptr, ldx), exps);
    if (parts > 1) decode_exps_kernel<<<grid_for(rows, 256, 4096), 256, 0, stream>>>(exps, rows);
}

// Slices after leading-word exponents, marking rows (columns) for the exact
// pass; with_fix: the exact pass too; streamed: non-temporal stores.
template <int NS, bool STREAM>
void launch_slices_checked(const PackGeom& g, int64_t outer, int64_t k, const double* X_hi, const double* X_lo,
                           int64_t ldx, int axis, int32_t* exps, double* slices, hipStream_t stream, bool pairs,
                           bool with_fix) {
    const unsigned fix = static_cast<unsigned>((outer + 15) / 16);
    if (axis == 0) {
        const bool aligned = pairs_aligned(X_hi, X_lo, ldx);
        const unsigned grid = grid_for(g.RB * ((g.KB + 15) / 16), 1, 1 << 20);
        if (pairs)
            slice_rows_lds_kernel<NS, true, true, STREAM><<<grid, 256, 0, stream>>>(outer, k, g.RB, g.KB, X_hi, X_lo,
                                                                                    ldx, aligned, exps, slices);
        else
            slice_rows_lds_kernel<NS, false, true, STREAM><<<grid, 256, 0, stream>>>(outer, k, g.RB, g.KB, X_hi, X_lo,
                                                                                     ldx, aligned, exps, slices);
        if (with_fix && pairs)
            split_block_kernel<0, kFixThreads, NS, true, true><<<fix, kFixThreads, 0, stream>>>(
                outer, k, g.KB, X_hi, X_lo, ldx, exps, slices);
        else if (with_fix)
            split_block_kernel<0, kFixThreads, NS, false, true><<<fix, kFixThreads, 0, stream>>>(
                outer, k, g.KB, X_hi, X_lo, ldx, exps, slices);
    } else {
        const dim3 grid(static_cast<unsigned>(g.RB / 4), static_cast<unsigned>(g.KB / 4 < 65535 ? g.KB / 4 : 65535));
        slice_cols_lds_kernel<NS, true, STREAM><<<grid, 256, 0, stream>>>(outer, k, g.KB, X_hi, X_lo, ldx,
                                                                          pairs_aligned(X_hi, X_lo, ldx), exps, slices);
        if (with_fix)
            split_block_kernel<1, kFixThreads, NS, false, true><<<fix, kFixThreads, 0, stream>>>(
                outer, k, g.KB, X_hi, X_lo, ldx, exps, slices);
    }
}

// B's column exponents: partial maxima of the row parts go to the slice
// buffer, which the slice pass overwrites only after the fold.
void launch_exps_cols(int64_t rows, int64_t cols, const double* X_hi, int64_t ldx, int32_t* exps, double* slices,
                      hipStream_t stream) {
    const int64_t chunks = exp_col_chunks(cols), parts = stream_col_parts(rows, cols);
    int32_t* partial = reinterpret_cast<int32_t*>(slices);
    exp_cols_stream_kernel<kColThreads>
        <<<dim3(static_cast<unsigned>(chunks), static_cast<unsigned>(parts)), kColThreads, 0, stream>>>(
            rows, cols, X_hi, nullptr, ldx, pairs_aligned(X_hi, nullptr, ldx), exps, partial);
    if (parts > 1) fold_exps_kernel<<<grid_for(cols, 256, 4096), 256, 0, stream>>>(parts, cols, partial, exps);
}

template <int NS>
hipError_t launch_split_ns(int64_t rows, int64_t cols, const double* X_hi, const double* X_lo,
                           int64_t ldx, int axis, int32_t* exps, double* slices, hipStream_t stream,
                           int phases, bool pairs) {
    const int64_t outer = axis == 0 ? rows : cols;
    const int64_t k = axis == 0 ? cols : rows;
    if (outer == 0) return hipSuccess;
    const PackGeom g(outer, k);
    int64_t kparts;
    if (one_pass(g, rows, cols, axis, NS, kparts)) {
        // One pass per block; k-blocks shared among parts when blocks are few.
        // All of it belongs to the slice phase.
        if (phases & kSplitSlices) launch_one_pass<NS>(g, kparts, outer, k, X_hi, X_lo, ldx, axis, exps, slices, stream, pairs);
        return hipGetLastError();
    }
    // Otherwise two passes over the operand.  The exponent pass reads the
    // leading words alone (8 bytes per entry); the slice pass reads (hi, lo),
    // marks every row (column) holding a pair whose leading word is not
    // RN(hi + lo) -- for which that exponent may be wrong -- and a last launch
    // recomputes the exponents and slices of the marked blocks from (hi, lo).
    if ((phases & kSplitExps) && axis == 0) {
        launch_exps_rows(rows, cols, X_hi, ldx, exps, stream);
    } else if (phases & kSplitExps) {
        launch_exps_cols(rows, cols, X_hi, ldx, exps, slices, stream);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (!(phases & kSplitSlices) || g.doubles(NS) == 0) return hipSuccess;
    launch_slices_checked<NS, true>(g, outer, k, X_hi, X_lo, ldx, axis, exps, slices, stream, pairs, true);
    return hipGetLastError();
}

// Both operands of a product (A in the pair-packed layout).  Each operand's
// slice pass runs right after its exponent pass, while the leading words it
// has just read are still in the memory-side cache (measured at 4096^3: 17 us
// less than both exponent passes first; B's exponents overlapped with A's
// slices lose that and take 25 us more).  When both take two passes: B's
// exponents and their fold; B's slices (non-temporal stores, which leave the
// next pass no dirty lines to write back); A's exponents with B's exact pass
// in the same launch; A's slices (plain stores: the GEMM that follows absorbs
// their write-back); A's exact pass.
template <int NS>
hipError_t launch_operands_ns(int64_t m, int64_t n, int64_t k, const double* A_hi, const double* A_lo, int64_t lda,
                              const double* B_hi, const double* B_lo, int64_t ldb, int32_t* E, double* A_sl,
                              int32_t* F, double* B_sl, hipStream_t stream) {
    const PackGeom ga(m, k), gb(n, k);
    int64_t ka_parts, kb_parts;
    const bool a1 = m > 0 && k > 0 && one_pass(ga, m, k, 0, NS, ka_parts);
    const bool b1 = n > 0 && k > 0 && one_pass(gb, k, n, 1, NS, kb_parts);
    if (a1 && b1 && !(ka_parts == 1 && ga.KB * 32 <= kBlockThreads * kRegPairs)) {
        // both small: one launch (A's blocks are not held in registers here)
        const int64_t na = ga.RB * ka_parts, grid = na + gb.RB * kb_parts;
        if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
        split_both_block_kernel<NS><<<static_cast<unsigned>(grid), 1024, 0, stream>>>(
            m, k, ga.KB, A_hi, A_lo, lda, E, A_sl, ka_parts, na, n, B_hi, B_lo, ldb, F, B_sl, kb_parts);
        return hipGetLastError();
    }
    if (m == 0 || n == 0 || k == 0 || a1 || b1 || exp_row_parts(m, k) > 1) {
        hipError_t e = launch_split_ns<NS>(k, n, B_hi, B_lo, ldb, 1, F, B_sl, stream, kSplitAll, false);
        if (e == hipSuccess) e = launch_split_ns<NS>(m, k, A_hi, A_lo, lda, 0, E, A_sl, stream, kSplitAll, true);
        return e;
    }
    launch_exps_cols(k, n, B_hi, ldb, F, B_sl, stream);
    launch_slices_checked<NS, true>(gb, n, k, B_hi, B_lo, ldb, 1, F, B_sl, stream, false, false);
    const int64_t row_wgs = grid_for(m, 4, 1 << 20), grid = row_wgs + (n + 15) / 16;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
    exp_rows_fix_kernel<NS><<<static_cast<unsigned>(grid), 256, 0, stream>>>(
        m, k, A_hi, lda, pairs_aligned(A_hi, nullptr, lda), E, row_wgs, n, gb.KB, B_hi, B_lo, ldb, F, B_sl);
    launch_slices_checked<NS, false>(ga, m, k, A_hi, A_lo, lda, 0, E, A_sl, stream, true, true);
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

hipError_t launch_split_operands(int64_t m, int64_t n, int64_t k, const double* A_hi, const double* A_lo,
                                 int64_t lda, const double* B_hi, const double* B_lo, int64_t ldb, int ns, int32_t* E,
                                 double* A_slices, int32_t* F, double* B_slices, hipStream_t stream) {
    switch (ns) {
#define DDG_OPERANDS(N)                                                                                           \
    case N:                                                                                                       \
        return launch_operands_ns<N>(m, n, k, A_hi, A_lo, lda, B_hi, B_lo, ldb, E, A_slices, F, B_slices, stream);
        DDG_OPERANDS(4) DDG_OPERANDS(5) DDG_OPERANDS(6) DDG_OPERANDS(7) DDG_OPERANDS(8) DDG_OPERANDS(9)
        DDG_OPERANDS(10) DDG_OPERANDS(11) DDG_OPERANDS(12) DDG_OPERANDS(13) DDG_OPERANDS(14) DDG_OPERANDS(15)
        DDG_OPERANDS(16)
#undef DDG_OPERANDS
        default: return hipErrorInvalidValue;
    }
}

}  // namespace ddg
