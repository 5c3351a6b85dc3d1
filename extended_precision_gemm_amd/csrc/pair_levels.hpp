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

template <int NS, int W>
__device__ __forceinline__ void pair_units_round(const int64_t (&N)[NS - 1], int sc, double (&c)[W]) {
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
