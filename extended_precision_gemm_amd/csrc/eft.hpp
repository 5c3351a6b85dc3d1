// Error-free transformations and the level renormalisation, device side.
//
// Everything here is addition only (no products), so fused multiply-add
// contraction cannot change it; the library is still built with
// -ffp-contract=off and never with fast-math, which would license the
// compiler to reassociate the bookkeeping away.
#pragma once

#include "common.hpp"

namespace ddg {

// Knuth's TwoSum: s = RN(a + b) and e = (a + b) - s exactly, any ordering of |a|, |b|.
__device__ __forceinline__ void two_sum(double a, double b, double& s, double& e) {
    s = a + b;
    const double bv = s - a;
    const double av = s - bv;
    e = (a - av) + (b - bv);
}

// Dekker's FastTwoSum: s = RN(a + b), e = (a + b) - s exactly when |a| >= |b|
// (or a = 0).
__device__ __forceinline__ void fast_two_sum(double a, double b, double& s, double& e) {
    s = a + b;
    e = b - (s - a);
}

// Accurate double-word addition (Joldes, Muller and Popescu, "Tight and rigorous
// error bounds for basic building blocks of double-word arithmetic", ACM TOMS
// 2017): relative error below 3u^2 for u = 2^-53.
__device__ __forceinline__ void dd_add(double ah, double al, double bh, double bl, double& zh, double& zl) {
    double sh, sl, th, tl, vh, vl;
    two_sum(ah, bh, sh, sl);
    two_sum(al, bl, th, tl);
    sl = sl + th;
    fast_two_sum(sh, sl, vh, vl);
    vl = vl + tl;
    fast_two_sum(vh, vl, zh, zl);
}

// Level renormalisation ("Multiple Double Arithmetic on NVIDIA Tensor Cores",
// §2, fifth step): add the NL exact level sums of one output entry into a
// double-double, smallest level first, then apply the entry's scale 2^sc.
// TwoSum is used for the renormalising step too (FastTwoSum gives the same bits
// whenever its precondition holds, and TwoSum needs no branch when it does not).
template <int NL>
__device__ __forceinline__ void renorm_levels(const double (&S)[NL], int sc, double& c_hi, double& c_lo) {
    double h = S[NL - 1];
    double t = 0.0;
#pragma unroll
    for (int l = NL - 2; l >= 0; --l) {
        double s, e;
        two_sum(h, S[l], s, e);
        t = t + e;
        two_sum(s, t, h, t);
    }
    c_hi = ldexp(h, sc);
    c_lo = ldexp(t, sc);
}

}  // namespace ddg
