// Fixed-width two's-complement integers of L 64-bit limbs, device side.
//
// The quad-double path needs exact integers wider than 128 bits: the 208-bit
// slicing window of an entry and the exact total of sixteen level sums.  Every
// limb index below is a compile-time constant (loops are unrolled and run-time
// shift amounts are resolved with selects), so a value lives in 2 L registers
// and never in scratch memory.
#pragma once

#include "common.hpp"

namespace ddg {

template <int L>
struct WideInt {
    uint64_t w[L];  // little-endian limbs
};

template <int L>
__device__ __forceinline__ void wide_zero(WideInt<L>& a) {
#pragma unroll
    for (int j = 0; j < L; ++j) a.w[j] = 0;
}

template <int L>
__device__ __forceinline__ bool wide_is_zero(const WideInt<L>& a) {
    uint64_t x = 0;
#pragma unroll
    for (int j = 0; j < L; ++j) x |= a.w[j];
    return x == 0;
}

template <int L>
__device__ __forceinline__ bool wide_is_neg(const WideInt<L>& a) { return (a.w[L - 1] >> 63) != 0; }

// a += v * 2^sh, v sign-extended; 0 <= sh < 64 L.
template <int L>
__device__ __forceinline__ void wide_add_shifted(WideInt<L>& a, int64_t v, int sh) {
    const int q = sh >> 6, r = sh & 63;
    const uint64_t lo = static_cast<uint64_t>(v) << r;
    const uint64_t hi = r ? static_cast<uint64_t>(v >> (64 - r)) : static_cast<uint64_t>(v >> 63);
    const uint64_t fill = static_cast<uint64_t>(v >> 63);
    uint64_t carry = 0;
#pragma unroll
    for (int j = 0; j < L; ++j) {
        const uint64_t b = j < q ? 0 : (j == q ? lo : (j == q + 1 ? hi : fill));
        const uint64_t s = a.w[j] + b;
        const uint64_t c1 = s < b;
        const uint64_t s2 = s + carry;
        const uint64_t c2 = s2 < carry;
        a.w[j] = s2;
        carry = c1 | c2;
    }
}

template <int L>
__device__ __forceinline__ void wide_negate(WideInt<L>& a) {
    uint64_t carry = 1;
#pragma unroll
    for (int j = 0; j < L; ++j) {
        const uint64_t x = ~a.w[j] + carry;
        carry = (carry != 0 && x == 0) ? 1 : 0;
        a.w[j] = x;
    }
}

// Significant bits of a nonnegative value (0 for zero).
template <int L>
__device__ __forceinline__ int wide_bit_length(const WideInt<L>& a) {
    int b = 0;
#pragma unroll
    for (int j = 0; j < L; ++j)
        if (a.w[j] != 0) b = 64 * j + 64 - __clzll(static_cast<long long>(a.w[j]));
    return b;
}

// Limb j for a run-time j (0 outside [0, L)).
template <int L>
__device__ __forceinline__ uint64_t wide_limb(const WideInt<L>& a, int j) {
    uint64_t r = 0;
#pragma unroll
    for (int i = 0; i < L; ++i) r = (i == j) ? a.w[i] : r;
    return r;
}

// The 64 bits of a starting at bit s >= 0.
template <int L>
__device__ __forceinline__ uint64_t wide_bits64(const WideInt<L>& a, int s) {
    const int q = s >> 6, r = s & 63;
    const uint64_t lo = wide_limb(a, q), hi = wide_limb(a, q + 1);
    return r ? (lo >> r) | (hi << (64 - r)) : lo;
}

template <int L>
__device__ __forceinline__ bool wide_bit(const WideInt<L>& a, int s) {
    return ((wide_limb(a, s >> 6) >> (s & 63)) & 1) != 0;
}

// Clear every bit at position >= s (s >= 0).
template <int L>
__device__ __forceinline__ void wide_keep_low(WideInt<L>& a, int s) {
#pragma unroll
    for (int j = 0; j < L; ++j) {
        const int b0 = 64 * j;
        const uint64_t m = s >= b0 + 64 ? ~0ull : (s <= b0 ? 0ull : (1ull << (s - b0)) - 1);
        a.w[j] &= m;
    }
}

template <int L>
__device__ __forceinline__ bool wide_any_below(const WideInt<L>& a, int s) {
    WideInt<L> t = a;
    wide_keep_low(t, s);
    return !wide_is_zero(t);
}

}  // namespace ddg
