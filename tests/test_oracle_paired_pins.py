"""Pins for the oracle's pair-packed schedule and its nearest double-double
epilogue (the product entry points' chain), tied to things other than the
oracle itself: a colouring bound on the number of products, the level sums of
the pages' eq. (3) structure, brute-force loops, closed-form roundings and
exact rational arithmetic.  No GPU needed."""
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import exact
import workloads


def _window_pairs(n):
    return {(s, t) for s in range(n) for t in range(n) if s + t <= n - 1}


@pytest.mark.parametrize("n", range(4, 17))
def test_pair_schedule_covers_every_window_pair_once(n):
    covered = []
    for s0, s1, t, g in exact.pair_schedule(n):
        covered.append((s0, t))
        if s1 >= 0:
            assert s1 == s0 + 1 and s0 % 2 == 0
            covered.append((s1, t))
            assert g == s0 + t                      # units of the lower pair's level
        else:
            assert g == n - 2 and s0 + t == n - 1   # a single pair sits on the deepest level
        assert 0 <= g <= n - 2
    assert sorted(covered) == sorted(_window_pairs(n))
    assert len(covered) == len(set(covered))


@pytest.mark.parametrize("n", range(4, 17))
def test_pair_schedule_meets_the_colouring_bound(n):
    """A product covers at most two pairs, and two pairs (s, t), (s+1, t) always
    differ in the parity of s + t; so no schedule of products covering one or
    two vertically adjacent window pairs has fewer products than the window has
    pairs of the more frequent parity.  The schedule reaches that bound."""
    cells = _window_pairs(n)
    odd = sum(1 for s, t in cells if (s + t) % 2 == 1)
    even = len(cells) - odd
    assert len(exact.pair_schedule(n)) == max(odd, even)
    assert len(exact.pair_schedule(8)) == 20 and len(exact.pair_schedule(16)) == 72


def _digits(rng, n, shape, full=False):
    if full:
        return np.full((n,) + shape, 8191, dtype=np.int64)
    D = rng.integers(0, 8192, size=(n,) + shape).astype(np.int64)
    sign = np.where(rng.random(shape) < 0.5, -1, 1)
    return D * sign  # every digit of an entry carries the entry's sign


@pytest.mark.parametrize("n", [4, 5, 8, 11, 16])
def test_group_sums_regroup_the_level_sums_exactly(n):
    """sum_g G_g 2^(13(n-2-g)) == sum_l S_l 2^(13(n-1-l)) (both in the units of
    the deepest group), and group g holds 2^13 times level g's pairs with even s
    plus level g+1's pairs with odd s (the deepest group: all of level n-1)."""
    rng = np.random.default_rng(n)
    DA = _digits(rng, n, (5, 7))
    DB = _digits(rng, n, (7, 6)).transpose(0, 1, 2)
    G = exact.paired_group_units(DA, DB)
    S = exact.level_sums_units(DA, DB)
    for i in range(5):
        for j in range(6):
            lhs = sum(int(G[g, i, j]) << (13 * (n - 2 - g)) for g in range(n - 1))
            rhs = sum(int(S[l, i, j]) << (13 * (n - 1 - l)) for l in range(n))
            assert lhs == rhs
    # the parity split, with plain loops over the digits
    k = DA.shape[2]
    for i in range(5):
        for j in range(6):
            even = [0] * n
            odd = [0] * n
            for s in range(n):
                for t in range(n - s):
                    v = sum(int(DA[s, i, p]) * int(DB[t, p, j]) for p in range(k))
                    (even if s % 2 == 0 else odd)[s + t] += v
            for g in range(n - 2):
                assert G[g, i, j] == (even[g] << 13) + odd[g + 1]
            assert G[n - 2, i, j] == (even[n - 2] << 13) + odd[n - 1] + even[n - 1]


def test_group_sums_brute_force_on_tiny_inputs():
    """Each product of the schedule written out as a loop over k, against the
    vectorised group sums."""
    rng = np.random.default_rng(3)
    n, m, k, c = 8, 2, 3, 2
    DA = _digits(rng, n, (m, k))
    DB = _digits(rng, n, (k, c))
    G = exact.paired_group_units(DA, DB)
    want = np.zeros_like(G)
    for i in range(m):
        for j in range(c):
            for u in range(4):
                for t in range(8):
                    for p in range(k):
                        a0, a1, b = int(DA[2 * u, i, p]), int(DA[2 * u + 1, i, p]), int(DB[t, p, j])
                        if 2 * u + 1 + t <= 7:
                            want[2 * u + t, i, j] += (a0 * 8192 + a1) * b
                        elif 2 * u + t == 7:
                            want[6, i, j] += a0 * b
    assert np.array_equal(G, want)


def test_group_sums_of_the_largest_digits_stay_within_53_bits_for_4096_terms():
    """With every digit at 8191 the deepest group (four packed products and four
    single pairs per term for 8 slices) reaches 2^53 only past 4096 terms: the
    length of k over which FP64 sums of the packed products stay exact."""
    n = 8
    for k, inside in [(4096, True), (4097, False)]:
        DA = np.full((n, 1, k), 8191, dtype=np.int64)
        DB = np.full((n, k, 1), 8191, dtype=np.int64)
        G = exact.paired_group_units(DA, DB)
        assert (int(np.abs(G).max()) < 2 ** 53) == inside
        assert int(G[n - 2, 0, 0]) == k * (4 * (8191 * 8192 + 8191) * 8191 + 4 * 8191 * 8191)


# ---------------------------------------------------------------------------
# nearest double-double
# ---------------------------------------------------------------------------
def _nearest(levels, sc):
    """nearest_dd of one entry with the given level sums {l: S_l} and scale sc = E + F."""
    S = np.zeros((8, 1, 1), dtype=np.int64)
    for l, v in levels.items():
        S[l, 0, 0] = v
    hi, lo = exact.nearest_dd(S, [sc], [0])
    return float(hi[0, 0]), float(lo[0, 0])


# level 0 counts units 2^(sc - 26), level 7 units 2^(sc - 117); sc = -27 makes
# level 0's unit 2^-53 and level 7's 2^-144
@pytest.mark.parametrize("levels,sc,hi,lo", [
    ({0: 3}, 26, 3.0, 0.0),
    ({0: 2 ** 60 + 1}, -34, 1.0, 2.0 ** -60),
    ({0: 2 ** 53 + 1}, -27, 1.0, 2.0 ** -53),                              # tie: the even neighbour stays
    ({0: 2 ** 53 + 3}, -27, 1.0 + 2.0 ** -51, -(2.0 ** -53)),              # tie: rounds up to even
    ({0: -(2 ** 53 + 3)}, -27, -(1.0 + 2.0 ** -51), 2.0 ** -53),
    ({0: 2 ** 53 + 1, 7: 2 ** 44}, -27, 1.0 + 2.0 ** -52, -(2.0 ** -53) + 2.0 ** -100),  # just above the tie
    ({0: 2 ** 53 + 1, 7: -(2 ** 44)}, -27, 1.0, 2.0 ** -53 - 2.0 ** -100),             # just below it
])
def test_nearest_dd_closed_forms(levels, sc, hi, lo):
    assert _nearest(levels, sc) == (hi, lo)


def test_nearest_dd_at_the_ends_of_the_double_range():
    # halfway between the largest double and 2^1024: ties to even give 2^1024 -> inf,
    # and the low word rounds what is left after 2^1024
    v = Fraction(2 ** 1024) - Fraction(2 ** 970)
    S = np.zeros((8, 1, 1), dtype=np.int64)
    S[0, 0, 0] = (2 ** 54 - 1)  # (2^54 - 1) 2^970 = 2^1024 - 2^970
    hi, lo = exact.nearest_dd(S, [970 + 26], [0])
    assert hi[0, 0] == math.inf and lo[0, 0] == -(2.0 ** 970)
    assert Fraction(2 ** 1024) + Fraction(lo[0, 0]) == v
    # three halves of the smallest subnormal: the high word takes two, the rest rounds to -0
    S[0, 0, 0] = 3
    hi, lo = exact.nearest_dd(S, [-1075 + 26], [0])
    assert hi[0, 0] == 2.0 ** -1073 and lo[0, 0] == 0.0 and math.copysign(1.0, lo[0, 0]) < 0


def test_nearest_dd_is_the_nearest_pair_of_doubles():
    """hi is the double nearest to x (no double is closer), lo the double nearest
    to x - hi, and hi = RN(hi + lo): checked with exact rationals on random
    level sums with cancellation."""
    rng = np.random.default_rng(5)
    S = rng.integers(-(2 ** 52), 2 ** 52, size=(8, 20, 20)).astype(np.int64)
    S[0] = rng.integers(-3, 4, size=(20, 20))        # small leading levels: cancellation
    E = rng.integers(-40, 40, size=20)
    F = rng.integers(-40, 40, size=20)
    hi, lo = exact.nearest_dd(S, E, F)
    for i in range(20):
        for j in range(20):
            x = exact.level_target(S, int(E[i]), int(F[j]), i, j)
            h, l = float(hi[i, j]), float(lo[i, j])
            for cand in (math.nextafter(h, math.inf), math.nextafter(h, -math.inf)):
                assert abs(x - Fraction(h)) <= abs(x - Fraction(cand))
            r = x - Fraction(h)
            for cand in (math.nextafter(l, math.inf), math.nextafter(l, -math.inf)):
                assert abs(r - Fraction(l)) <= abs(r - Fraction(cand))
            assert h + l == h
            assert abs(r - Fraction(l)) <= Fraction(abs(x)) * Fraction(1, 2 ** 106)


def test_nearest_dd_is_never_less_accurate_than_the_cascade():
    """On random level sums (a third of them cancelling level by level) the
    nearest double-double is at least as close to the exact total as the
    stage chain's cascade, and strictly closer where the cascade's low word
    picked up a rounding: two such entries are pinned by their level sums."""
    rng = np.random.default_rng(11)
    S = rng.integers(-(2 ** 52), 2 ** 52, size=(8, 20, 20)).astype(np.int64)
    for l in range(7):
        if rng.random() < 0.5:
            S[l] = -(S[l + 1] >> 13) + rng.integers(-3, 4, size=(20, 20))
    S[:, 0, 0] = [-83975627198, 687928338015056, -390270418258, 548825917746, -4495981918188070,
                  -1177740167570751, 3350882771185066, -3550813160548493]
    S[:, 0, 1] = [297178351072, -148953005329, -349016799381, 2859145620506679, -82079493227, 672395208527219,
                  2941444737024889, 1833683882917783]
    E = np.zeros(20, dtype=np.int32)
    hi, lo = exact.nearest_dd(S, E, E)
    ch, cl = exact.renorm_levels(exact.level_values(S), E, E)
    for i in range(20):
        for j in range(20):
            x = exact.level_target(S, 0, 0, i, j)
            e_near = abs(x - Fraction(float(hi[i, j])) - Fraction(float(lo[i, j])))
            e_casc = abs(x - Fraction(float(ch[i, j])) - Fraction(float(cl[i, j])))
            assert e_near <= e_casc
            if (i, j) in ((0, 0), (0, 1)):
                assert e_near < e_casc


def test_paired_product_of_the_identity_is_the_operand_on_its_grid():
    """I·B for B whose entries lie on their columns' 104-bit grid (small integers
    and binary fractions): the exact total is the entry, rounded to itself."""
    rng = np.random.default_rng(7)
    n = 12
    Bh = rng.integers(-1000, 1000, size=(n, n)).astype(np.float64) * 2.0 ** -7
    Bl = np.zeros_like(Bh)
    I = np.eye(n)
    hi, lo = exact.paired_product(I, None, Bh, Bl)
    assert np.array_equal(hi, Bh) and np.array_equal(lo, np.zeros_like(Bh))


@pytest.mark.parametrize("dist", ["uniform", "signed_exp20"])
def test_paired_product_within_its_error_bound_of_the_exact_product(dist):
    """Against the exact rational product: within the window's error bound,
    and within 1e-28 (|A||B|)_ij where entries sit near their row's (column's)
    largest (uniform entries; with exponents over 41 binades and k = 40 an entry
    far down its row keeps fewer bits, which the bound accounts for)."""
    Ah, Al = workloads.random_dd((9, 40), 11, dist)
    Bh, Bl = workloads.random_dd((40, 7), 12, dist)
    hi, lo = exact.paired_product(Ah, Al, Bh, Bl)
    E = exact.balancing_exponents(Ah, Al, 0)
    F = exact.balancing_exponents(Bh, Bl, 1)
    bound = exact.error_bound(Ah, Bh, E, F, 8)
    absAB = np.abs(Ah) @ np.abs(Bh)
    for i in range(9):
        for j in range(7):
            x = exact.exact_dot(Ah[i], Al[i], Bh[:, j], Bl[:, j])
            err = abs(x - Fraction(float(hi[i, j])) - Fraction(float(lo[i, j])))
            assert err <= Fraction(float(bound[i, j]))
            if dist == "uniform":
                assert err <= Fraction(1e-28) * Fraction(float(absAB[i, j]))
