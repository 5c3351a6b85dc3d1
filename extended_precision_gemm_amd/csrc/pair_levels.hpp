// Epilogue of the pair-packed schedule, device side.
//
// The schedule multiplies slices 2u and 2u+1 of an A entry, packed into one
// exact 26-bit operand, by a 13-bit B slice: one FP64 matrix product covers
// the window pairs (2u, t) and (2u+1, t) at once (where 2u + t = NS - 1 only
// (2u, t) lies in the window, and it runs alone).  The products of one output
// entry fall into NS - 1 groups; group g counts units 2^(-13(g+3)) ("Multiple
// Double Arithmetic on NVIDIA Tensor Cores", §2 eqs. (1)-(4) with two slices of
// A in one operand; exactness as in §2 eq. (5), for 39-bit products).
//
// The group sums, int64 integers, add exactly into a wide integer T of units
// 2^(-13(NS+1)), and the result is the nearest W-word multiple double of
// T 2^(E_i + F_j): W = 2 the nearest double-double, W = 4 the nearest quad
// double (the pages add the parts of an entry in multiple-double arithmetic
// without fixing an order; the exact total rounded once is the most accurate
// order, and the same whatever the grouping of the products).
#pragma once

#include "common.hpp"
#include "qd_levels.hpp"
#include "wide_int.hpp"

namespace ddg {

// Limbs of T: NS - 1 int64 group sums, group g shifted left by 13(NS - 2 - g).
template <int NS>
constexpr int pair_total_limbs() {
    return (63 + kSliceBits * (NS - 2) + 2 + 63) / 64;
}

// The nearest double-double of T = sum_g N_g 2^(13(NS - 2 - g)) units of
// 2^base, for NS <= 8, in a few floating-point operations: the same words as
// the wide-integer rounding below.  The group sums are carried into one
// integer M and 13-bit digits d_g >= 0 (T = M 2^L + D, L = 13(NS - 2),
// 0 <= D < 2^L).  Up to six slices (L <= 52) T = A + B with A = M 2^L and
// B = D exact doubles, so RN(T) is one addition and T - RN(T) its exact error.
// With seven or eight, D is cut into Dh 2^K + Dl (K = L - 39) and, for
// 2^20 <= |M| < 2^53, the doubles A, B = Dh 2^K and C = Dl are exact, and the
// doubles near T are at least 2^(K + 6) apart with the midpoints between them
// multiples of 2^K: C < 2^K moves T across no rounding boundary, except where
// A + B lies exactly on a midpoint, and then RN(T) is the upper neighbour.
// The trailing word is RN(T - hi): one more addition of exact doubles.
// Returns false, leaving c untouched, outside those conditions and where a
// word could need gradual underflow or overflow.
template <int NS>
__device__ __forceinline__ bool pair_dd_round_fast(const int64_t (&N)[NS - 1], int base, double (&c)[2]) {
    static_assert(NS <= 8, "the digits below the leading group fit 78 bits");
    constexpr int L = kSliceBits * (NS - 2);
    constexpr int K = L > 52 ? L - 39 : 0;  // D = Dh 2^K + Dl (K a multiple of 13)
    // |T| < 2^(L + 54) when |M| < 2^53: no word overflows; every nonzero word
    // is an integer times 2^base >= 2^-1022 (normal, no gradual underflow)
    bool ok = base >= -1022 && base <= 1023 - (L + 54);
#pragma unroll
    for (int g = 0; g < NS - 1; ++g)
        ok = ok && static_cast<uint64_t>(N[g]) + (uint64_t(1) << 62) < (uint64_t(1) << 63);
    // carries: d_g = (N_g + carry) mod 2^13 for g = NS-2 .. 1, the rest into group 0
    uint64_t Dh = 0, Dl = 0;
    int64_t carry = 0;
#pragma unroll
    for (int g = NS - 2; g >= 1; --g) {
        const int64_t x = N[g] + carry;
        const uint64_t d = static_cast<uint64_t>(x) & ((uint64_t(1) << kSliceBits) - 1);
        carry = x >> kSliceBits;  // arithmetic: floor division
        const int pos = kSliceBits * (NS - 2 - g);  // d_g's weight in D
        if (pos >= K) Dh |= d << (pos - K);
        else Dl |= d << pos;
    }
    const int64_t M = N[0] + carry;
    const uint64_t am = static_cast<uint64_t>(M < 0 ? -M : M);
    ok = ok && am < (uint64_t(1) << 53) && (K == 0 || am >= (uint64_t(1) << 20));
    if (!ok) return false;
    const double A = ldexp(static_cast<double>(M), L);
    const double B = ldexp(static_cast<double>(Dh), K);
    double s = A + B, e;
    if constexpr (K == 0) {  // TwoSum: |A| may be below B
        const double bb = s - A;
        e = (A - (s - bb)) + (B - bb);
    } else {  // Fast2Sum: |A| >= 2^(L + 20) > B
        e = B - (s - A);
    }
    if constexpr (K > 0) {
        const double C = static_cast<double>(Dl);
        if (C > 0.0 && e > 0.0) {
            // A + B above s; on the midpoint to the next double, C tips it there
            const int64_t sb = __builtin_bit_cast(int64_t, s);
            const double up = __builtin_bit_cast(double, s > 0.0 ? sb + 1 : sb - 1);
            if (up - s == 2.0 * e) {
                s = up;
                e = -e;
            }
        }
        e += C;  // T - hi exactly, rounded once
    }
    c[0] = ldexp(s, base);
    c[1] = ldexp(e, base);  // an exact zero is +0
    return true;
}

template <int NS, int W>
__device__ __forceinline__ void pair_units_round(const int64_t (&N)[NS - 1], int sc, double (&c)[W]) {
    if constexpr (W == 2 && NS <= 8) {
        if (pair_dd_round_fast<NS>(N, sc - kSliceBits * (NS + 1), c)) return;
    }
    WideInt<pair_total_limbs<NS>()> T;
    wide_zero(T);
#pragma unroll
    for (int g = 0; g < NS - 1; ++g) wide_add_shifted(T, N[g], kSliceBits * (NS - 2 - g));
    round_words<W>(T, sc - kSliceBits * (NS + 1), c);  // one unit of T is 2^(sc - 13(NS+1))
}

// Group sum g as an int64 number of its units: the double is an exact integer
// multiple of 2^(-13(g+3)) below 2^53 such units.
__device__ __forceinline__ int64_t pair_group_units(double S, int g) {
    return static_cast<int64_t>(ldexp(S, kSliceBits * (g + 3)));
}

}  // namespace ddg
