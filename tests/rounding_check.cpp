// Host build of the double-double exit's rounding (csrc/pair_levels.hpp): the
// fast path pair_dd_round_fast<NS> must give the words of the wide-integer
// rounding (round_words over the exact total) bit for bit, signs of zero
// included, wherever it accepts its input.  Inputs: seeded group sums of every
// magnitude up to 2^63, sparse and tiny ones, carry chains, and totals built
// bit by bit so that the leading or the trailing word sits exactly on, just
// below or just above a tie; exponents across the whole double range.
// Prints one line per slice count and exits nonzero on a mismatch.
#include <hip/hip_runtime.h>
// the device functions, compiled for the host
#undef __device__
#define __device__ __host__ __attribute__((device))
#define __clzll(x) __builtin_clzll(x)
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>

#include "pair_levels.hpp"

using namespace ddg;

namespace {

template <int NS>
void wide_round(const int64_t (&N)[NS - 1], int base, double (&c)[2]) {
    WideInt<pair_total_limbs<NS>()> T;
    wide_zero(T);
    for (int g = 0; g < NS - 1; ++g) wide_add_shifted(T, N[g], kSliceBits * (NS - 2 - g));
    round_words<2>(T, base, c);
}

uint64_t bits(double x) {
    uint64_t u;
    memcpy(&u, &x, 8);
    return u;
}

std::mt19937_64 rng(20261202);

int64_t signed_bits(int maxbits) {
    const int b = static_cast<int>(rng() % (maxbits + 1));
    const int64_t x = b == 0 ? 0 : static_cast<int64_t>(rng() >> (64 - b));
    return (rng() & 1) ? -x : x;
}

template <int NS>
void draw(int64_t (&N)[NS - 1]) {
    constexpr int L = kSliceBits * (NS - 2);
    const int mode = static_cast<int>(rng() % 10);
    if (mode >= 8) {
        // T = M 2^L + R, R a bit pattern with a tie (or a near tie) at a random position
        unsigned __int128 R = 0;
        const int top = static_cast<int>(rng() % (L + 1));
        for (int t = 0; t < top; ++t)
            if (rng() & 1) R |= static_cast<unsigned __int128>(1) << (L - 1 - t);
        const int p = static_cast<int>(rng() % (L + 1));
        if (p > 0) {
            R &= ~((static_cast<unsigned __int128>(1) << p) - 1);
            R |= static_cast<unsigned __int128>(1) << (p - 1);
            const int q = static_cast<int>(rng() % p);
            if (mode == 9 && q > 0) R |= (static_cast<unsigned __int128>(1) << q) - 1;  // just above
            else if (mode == 9 && (rng() & 1)) R -= 1;                                  // just below
        }
        R &= (static_cast<unsigned __int128>(1) << L) - 1;
        N[0] = signed_bits(rng() % 2 ? 53 : 8);
        for (int g = 1; g < NS - 1; ++g) N[g] = static_cast<int64_t>((R >> (kSliceBits * (NS - 2 - g))) & 8191);
        if (rng() & 1)  // negative digits with compensating carries: the same total
            for (int g = NS - 2; g >= 1; --g)
                if (rng() & 1) {
                    N[g] -= 8192;
                    N[g - 1] += 1;
                }
        return;
    }
    for (int g = 0; g < NS - 1; ++g) {
        switch (mode) {
            case 0: N[g] = signed_bits(62); break;
            case 1: N[g] = signed_bits(53); break;
            case 2: N[g] = rng() % 3 == 0 ? signed_bits(53) : 0; break;
            case 3: N[g] = rng() % 2 ? (int64_t(1) << (rng() % 60)) * ((rng() & 1) ? 1 : -1) : 0; break;
            case 4: N[g] = static_cast<int64_t>(rng() % 5) - 2; break;
            case 5: N[g] = (rng() & 1) ? 8191 : ((rng() & 1) ? -1 : 8192); break;
            case 6: N[g] = signed_bits(20) << (rng() % 40); break;
            default: N[g] = signed_bits(63); break;  // 2^62 and beyond: the fast path declines
        }
    }
}

int draw_base() {
    const int m = static_cast<int>(rng() % 10);
    if (m < 6) return -157 + static_cast<int>(rng() % 81);
    if (m == 6) return -1094 + static_cast<int>(rng() % 200);  // the underflow edge
    if (m == 7) return 700 + static_cast<int>(rng() % 400);    // the overflow edge
    return -1300 + static_cast<int>(rng() % 2400);
}

template <int NS>
long check(long cases) {
    long bad = 0, fast = 0;
    for (long i = 0; i < cases; ++i) {
        int64_t N[NS - 1];
        draw<NS>(N);
        const int base = draw_base();
        double a[2] = {0.0, 0.0}, b[2];
        const bool took = pair_dd_round_fast<NS>(N, base, a);
        wide_round<NS>(N, base, b);
        if (!took) continue;
        ++fast;
        if (bits(a[0]) != bits(b[0]) || bits(a[1]) != bits(b[1])) {
            if (bad++ < 5) {
                printf("mismatch NS=%d base=%d N=", NS, base);
                for (int g = 0; g < NS - 1; ++g) printf("%lld ", static_cast<long long>(N[g]));
                printf(": fast %a %a, wide %a %a\n", a[0], a[1], b[0], b[1]);
            }
        }
    }
    printf("NS=%d cases=%ld fast=%ld mismatches=%ld\n", NS, cases, fast, bad);
    return bad;
}

}  // namespace

int main(int argc, char** argv) {
    const long n = argc > 1 ? atol(argv[1]) : 200000;
    const long bad = check<4>(n) + check<5>(n) + check<6>(n) + check<7>(n) + check<8>(n);
    return bad ? 1 : 0;
}
