// Exact fixed-point windows of multiple-double values, device side: the
// integer N = floor(|x| 2^-u) for x = x0 + x1 + x2 + x3 normalised (each
// component at most half an ulp of the one before it), formed from the
// components' integer mantissas in L-limb register integers.  Used by the
// quad-double slicer and by the double-double slicer for windows wider than
// 128 bits (more than nine slices), after one TwoSum has normalised the pair.
#pragma once

#include "common.hpp"
#include "split_common.hpp"
#include "wide_int.hpp"

namespace ddg {
namespace {

// floor(|x| 2^-u) for a normalised quad double x, as an L-limb integer (the
// caller picks u so the result fits).  The components' integer parts are summed
// with their signs; the part below the unit is, by the normalisation, smaller in
// magnitude than one unit and has the sign of the first component that reaches
// below the unit, so it lowers the floor by one exactly when that sign is
// negative.
template <int L>
__device__ __forceinline__ WideInt<L> floor_abs_window(const double (&x)[4], int u) {
    WideInt<L> acc;
    wide_zero(acc);
    const bool neg = x[0] < 0.0;
    bool decided = false, borrow = false;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const double y = neg ? -x[c] : x[c];
        if (y != 0.0) {
            uint64_t mant;
            int e;
            decompose(y, mant, e);  // |y| = mant 2^e
            const bool yneg = y < 0.0;
            const int sh = e - u;
            if (sh >= 0) {
                const int64_t v = static_cast<int64_t>(mant);
                wide_add_shifted(acc, yneg ? -v : v, sh);
            } else {
                const int d = -sh;
                const uint64_t t = d < 64 ? mant >> d : 0;
                const bool frac = d < 64 ? (mant & ((1ull << d) - 1)) != 0 : true;
                if (t != 0) wide_add_shifted(acc, yneg ? -static_cast<int64_t>(t) : static_cast<int64_t>(t), 0);
                if (!decided && frac) {
                    decided = true;
                    borrow = yneg;
                }
            }
        }
    }
    if (borrow) wide_add_shifted(acc, -1, 0);
    return acc;
}

}  // namespace
}  // namespace ddg
