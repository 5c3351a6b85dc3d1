// Quad-double epilogue, device side: the NL level sums of one output entry are
// added exactly and the total is rounded greedily to four doubles.
//
// "Multiple Double Arithmetic on NVIDIA Tensor Cores", §2 (fifth step: the parts
// of each product entry are added in multiple-double arithmetic).  Level l is an
// integer number of units 2^(-13(l+2)) below 2^53 (the exact-sum bound of §2
// eq. (5)), so the total is an integer T of units 2^(-13(NL+1)) below 2^252:
// it fits a 256-bit register integer, and the four outputs
//     c0 = RN(T), c1 = RN(T - c0), c2 = RN(T - c0 - c1), c3 = RN(T - c0 - c1 - c2)
// (each times 2^sc, round to nearest even, gradual underflow honoured) are the
// nearest quad double of the exact total.  Results beyond the double range
// overflow to infinity as ldexp does.
#pragma once

#include "common.hpp"
#include "wide_int.hpp"

namespace ddg {

// c[0..W-1] = the nearest W-word multiple double of T * 2^base, T an L-limb
// two's-complement integer (greedy: each word the nearest double of what is
// left); W = 2 is the nearest double-double, W = 4 the nearest quad double.
template <int W, int L>
__device__ __forceinline__ void round_words(WideInt<L> T, int base, double (&c)[W]) {
    bool neg = wide_is_neg(T);
    if (neg) wide_negate(T);
#pragma unroll
    for (int i = 0; i < W; ++i) {
        const int b = wide_bit_length(T);
        double v = 0.0;
        bool up = false;
        if (b > 0) {
            const int top = b - 1 + base;              // T 2^base lies in [2^top, 2^(top+1))
            const int lsb = max(top - 52, -1074);      // exponent of the last bit a double keeps
            const int j = lsb - base;                  // its position in T
            if (j <= 0) {
                v = ldexp(static_cast<double>(T.w[0]), base);  // T < 2^53: exact
                wide_zero(T);
            } else {
                uint64_t q = wide_bits64(T, j);        // at most 53 bits
                const bool half = wide_bit(T, j - 1);
                up = half && (wide_any_below(T, j - 1) || (q & 1));
                wide_keep_low(T, j);                   // remainder below the kept bits
                if (up) {                              // rounded up: 2^j - remainder is left, sign flips
                    q += 1;
                    wide_negate(T);
                    wide_add_shifted(T, 1, j);
                }
                v = ldexp(static_cast<double>(q), lsb);
            }
        }
        c[i] = (b > 0 && neg) ? -v : v;  // an exact zero remainder gives +0
        if (up) neg = !neg;
    }
}

template <int L>
__device__ __forceinline__ void qd_round_total(WideInt<L> T, int base, double (&c)[4]) {
    round_words<4, L>(T, base, c);
}

template <int NL>
__device__ __forceinline__ void qd_from_levels(const double (&S)[NL], int sc, double (&c)[4]) {
    WideInt<4> T;
    wide_zero(T);
#pragma unroll
    for (int l = 0; l < NL; ++l) {
        const int64_t units = static_cast<int64_t>(ldexp(S[l], kSliceBits * (l + 2)));  // exact integer
        wide_add_shifted(T, units, kSliceBits * (NL - 1 - l));
    }
    qd_round_total(T, sc - kSliceBits * (NL + 1), c);  // one unit of T is 2^(sc - 13(NL+1))
}

// The same from level sums already in integer units (summed over k-blocks that
// share their exponents): |N_l| < 2^63, so the total needs five limbs.
template <int NL>
__device__ __forceinline__ void qd_from_level_units(const int64_t (&N)[NL], int sc, double (&c)[4]) {
    WideInt<5> T;
    wide_zero(T);
#pragma unroll
    for (int l = 0; l < NL; ++l) wide_add_shifted(T, N[l], kSliceBits * (NL - 1 - l));
    qd_round_total(T, sc - kSliceBits * (NL + 1), c);
}

}  // namespace ddg
