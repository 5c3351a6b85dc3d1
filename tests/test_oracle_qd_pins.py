"""Pins of the quad-double oracle (oracle/qd.py) against facts that do not come
from the oracle itself: closed forms, round trips from chosen digits, brute
force on tiny inputs, the double-double slicer's pinned digits, and the exact
product within the stated error bound.  CPU only."""
import math
from fractions import Fraction

import numpy as np
import pytest

import workloads
from oracle import exact, qd

P = Fraction(2)


def test_exact_value_closed_form():
    comps = (1.0, 2.0 ** -60, -(2.0 ** -120), 2.0 ** -180)
    assert qd.qd_fraction(comps) == 1 + P ** -60 - P ** -120 + P ** -180
    assert qd.qd_fraction((0.0, 0.0, 0.0, 0.0)) == 0
    assert qd.qd_fraction((5e-324, 5e-324, 0.0, 0.0)) == 2 * P ** -1074


def test_normalisation_predicate():
    assert qd.is_normalized((1.0, 2.0 ** -53, 2.0 ** -106, 2.0 ** -159))
    assert qd.is_normalized((1.0, -(2.0 ** -53), 0.0, 0.0))
    assert not qd.is_normalized((1.0, 2.0 ** -52, 0.0, 0.0))
    assert not qd.is_normalized((0.0, 1e-300, 0.0, 0.0))
    assert not qd.is_normalized((1.0, 0.0, 1e-300, 0.0))
    X = workloads.random_qd((40, 40), 5, "signed_exp20")
    assert all(qd.is_normalized(X[:, i, j]) for i in range(40) for j in range(40))


def test_rn_ties_to_even():
    assert qd.rn(1 + P ** -53) == 1.0                            # tie, even is 1
    assert qd.rn(1 + 3 * P ** -53) == 1.0 + 2.0 ** -51          # tie, even is 1 + 2^-51
    assert qd.rn(1 + P ** -53 + P ** -300) == 1.0 + 2.0 ** -52  # above the tie
    assert qd.rn(3 * P ** -1075) == 2 * 5e-324                  # subnormal tie -> even


@pytest.mark.parametrize("comps,expect", [
    ((1.0, 0.0, 0.0, 0.0), 1),
    ((1.0, -(2.0 ** -54), 0.0, 0.0), 1),                    # RN(1 - 2^-54) = 1 (tie to even)
    ((1.0, -(2.0 ** -54), -(2.0 ** -110), 0.0), 0),         # below the tie: 1 - 2^-53
    ((2.0 - 2.0 ** -52, 2.0 ** -53, 0.0, 0.0), 2),          # tie rounds up to 2
    ((2.0 - 2.0 ** -52, 2.0 ** -53, -(2.0 ** -120), 0.0), 1),
    ((-(2.0 - 2.0 ** -52), -(2.0 ** -53), 0.0, 0.0), 2),
    ((0.75, 2.0 ** -60, 0.0, 0.0), 0),
    ((2.0 ** -40, 0.0, 0.0, 0.0), -39),
    ((5e-324, 0.0, 0.0, 0.0), -1073),
])
def test_entry_exponent(comps, expect):
    assert qd.is_normalized(comps)
    assert qd.entry_exponent(comps) == expect
    assert math.frexp(float(qd.qd_fraction(comps)))[1] in (expect, expect - 1, expect + 1)


def test_entry_exponent_zero_and_balancing_skip_zeros():
    assert qd.entry_exponent((0.0, 0.0, 0.0, 0.0)) is None
    X = np.zeros((4, 3, 4))
    X[0, 0, 1] = 0.75
    X[0, 0, 2] = -3.0
    X[0, 2, 3] = 2.0 ** -40
    assert list(qd.balancing_exponents(X, 0)) == [2, 0, -39]
    assert list(qd.balancing_exponents(X.transpose(0, 2, 1), 1)) == [2, 0, -39]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_digits_round_trip(seed):
    """16 chosen digits -> exact value -> greedy four-double form -> slicer -> same digits."""
    rng = np.random.default_rng(seed)
    for trial in range(20):
        d = [int(rng.integers(4096, 8191))] + [int(x) for x in rng.integers(0, 8192, size=15)]
        sign = 1 if trial % 2 == 0 else -1
        v = sign * sum(Fraction(d[s]) * P ** (-13 * (s + 1)) for s in range(16))
        comps = qd.greedy_qd(v)
        assert qd.qd_fraction(comps) == v              # 208 bits fit four doubles exactly
        assert qd.is_normalized(comps)
        assert qd.entry_exponent(comps) == 0
        assert qd.slice_entry(comps, 0) == [sign * x for x in d]
        # one more exponent: every digit moves one 13-bit place down... except
        # that the window is 208 bits, so the last digit falls out
        got = qd.slice_entry(comps, 13)
        assert got == [0] + [sign * x for x in d[:15]]


def test_slicing_reconstruction_truncates_toward_zero():
    X = workloads.random_qd((30, 30), 11, "signed_exp20")
    for i in range(30):
        E = int(qd.balancing_exponents(X[:, i:i + 1, :], 0)[0])
        for j in range(30):
            comps = X[:, i, j]
            x = qd.qd_fraction(comps)
            digits = qd.slice_entry(comps, E)
            assert all(abs(d) <= 8191 for d in digits)
            r = sum(Fraction(d) * P ** (E - 13 * (s + 1)) for s, d in enumerate(digits))
            assert r == 0 or (r > 0) == (x > 0)
            assert 0 <= abs(x) - abs(r) < P ** (E - 208)


def test_top_eight_digits_agree_with_double_double_slicer():
    hi, lo = workloads.random_dd((12, 40), 21, "signed_exp30")
    Edd = exact.balancing_exponents(hi, lo, 0)
    X = np.stack([hi, lo, np.zeros_like(hi), np.zeros_like(hi)])
    Eqd = qd.balancing_exponents(X, 0)
    assert np.array_equal(Edd, Eqd)
    for i in range(12):
        for j in range(40):
            dq = qd.slice_entry(X[:, i, j], int(Eqd[i]))
            dd = exact.slice_entry(hi[i, j], lo[i, j], int(Edd[i]), 8)
            assert dq[:8] == dd


def test_level_sums_brute_force():
    rng = np.random.default_rng(3)
    DA = rng.integers(-8191, 8192, size=(16, 3, 5))
    DB = rng.integers(-8191, 8192, size=(16, 5, 2))
    S = qd.level_sums(DA, DB)
    for l in range(16):
        for i in range(3):
            for j in range(2):
                want = sum(int(DA[s, i, p]) * int(DB[l - s, p, j]) for s in range(l + 1) for p in range(5))
                assert S[l, i, j] == want
    assert qd.QD_K_MAX == 4194304


def test_level_sums_add_over_k_blocks_under_shared_exponents():
    """Integer level sums are sums over k: with the digits taken below the
    exponents of whole rows / columns, blocks of k add up to the full sums
    exactly, whatever the blocks' own exponents would be."""
    A = workloads.random_qd((6, 30), 12, "uniform")
    B = workloads.random_qd((30, 5), 13, "normal")
    A[:, :, 15:] *= 2.0 ** -50
    E, DA = qd.slice_rows(A)
    F, DB = qd.slice_cols(B)
    S = qd.level_sums(DA, DB)
    parts = sum(qd.level_sums(DA[:, :, p0:p0 + 7], DB[:, p0:p0 + 7, :]) for p0 in range(0, 30, 7))
    assert np.array_equal(parts, S)
    # digits of one entry depend only on it and its row's exponent
    i, p = 2, 20
    assert [int(d) for d in DA[:, i, p]] == qd.slice_entry(A[:, i, p], int(E[i]))
    # the second half's own exponents are smaller: its digits would differ
    E_local, DA_local = qd.slice_rows(A[:, :, 15:])
    assert (E_local < E).all()
    assert not np.array_equal(DA_local, DA[:, :, 15:])


def test_greedy_closed_forms_and_properties():
    assert qd.greedy_qd(1 + P ** -60) == [1.0, 2.0 ** -60, 0.0, 0.0]
    assert qd.greedy_qd(3 * P ** -1074) == [3 * 5e-324, 0.0, 0.0, 0.0]
    # rounds up, so the remainder is negative
    assert qd.greedy_qd(1 + P ** -53 + P ** -200) == [1.0 + 2.0 ** -52, -(2.0 ** -53), 2.0 ** -200, 0.0]
    rng = np.random.default_rng(4)
    for _ in range(200):
        v = Fraction(int(rng.integers(1, 1 << 62))) ** 4 * P ** int(rng.integers(-300, -200))
        v = v if rng.random() < 0.5 else -v
        c = qd.greedy_qd(v)
        assert c[0] == qd.rn(v)
        for a, b in zip(c, c[1:]):
            assert a == 0.0 and b == 0.0 or 2 * abs(Fraction(b)) <= Fraction(math.ulp(a))
        rest = v - sum(Fraction(x) for x in c)
        assert abs(rest) <= Fraction(math.ulp(c[3])) / 2 if c[3] != 0.0 else rest == 0


def test_greedy_beyond_the_double_range():
    """Words past the largest double become infinities of the value's sign; the
    next word rounds the exact remainder after the word's unbounded value."""
    inf = math.inf
    assert qd.greedy_qd(3 * P ** 1100) == [inf, 0.0, 0.0, 0.0]
    assert qd.greedy_qd(P ** 1100 + P ** 1000) == [inf, 2.0 ** 1000, 0.0, 0.0]
    assert qd.greedy_qd(-(P ** 1100) - P ** 1000) == [-inf, -(2.0 ** 1000), 0.0, 0.0]
    # just below 2^1024: rounds up to 2^1024 (overflow), remainder negative
    x = P ** 1024 - P ** 969
    assert qd.greedy_qd(x) == [inf, -(2.0 ** 969), 0.0, 0.0]
    # the largest double itself, and a tie below it that rounds to even (down)
    top = P ** 1024 - P ** 971
    assert qd.greedy_qd(top) == [float(top), 0.0, 0.0, 0.0]
    assert qd.greedy_qd(top + P ** 970)[0] == inf   # halfway above the (odd) largest double: to even, 2^1024
    assert qd.greedy_qd(top + P ** 900)[:2] == [float(top), 2.0 ** 900]
    # unbounded rounding agrees with the float path wherever that is defined
    for v in (Fraction(1, 3), P ** 1023 * 3 / 2, -(P ** -1070) / 3):
        c, w = qd.rn_unbounded(v)
        assert c == qd.rn(v) and w == Fraction(c)


def test_renorm_levels_total_and_scale():
    S = np.zeros((16, 1, 2), dtype=np.int64)
    S[0, 0, 0] = 3              # 3 * 2^-26
    S[15, 0, 0] = -1            # -2^-221
    S[7, 0, 1] = 1 << 40        # 2^40 * 2^-117
    C = qd.renorm_levels(S, np.array([5]), np.array([-2, 7]))
    want0 = (3 * P ** -26 - P ** -221) * P ** 3
    assert [Fraction(c) for c in C[:, 0, 0]] == [Fraction(c) for c in qd.greedy_qd(want0)]
    assert sum(Fraction(c) for c in C[:, 0, 0]) == want0
    assert list(C[:, 0, 1]) == [2.0 ** (40 - 117 + 12), 0.0, 0.0, 0.0]


def test_integer_matrices_give_exact_products():
    rng = np.random.default_rng(6)
    a = rng.integers(-100, 101, size=(5, 7)).astype(np.float64)
    b = rng.integers(-100, 101, size=(7, 4)).astype(np.float64)
    A = np.stack([a] + [np.zeros_like(a)] * 3)
    B = np.stack([b] + [np.zeros_like(b)] * 3)
    _, _, _, C = qd.sliced_product(A, B)
    assert np.array_equal(C[0], a @ b)
    assert not C[1:].any()


def test_identity_returns_truncated_right_operand():
    B = workloads.random_qd((6, 5), 8, "signed_exp20")
    A = np.zeros((4, 6, 6))
    A[0] = np.eye(6)
    E, F, _, C = qd.sliced_product(A, B)
    assert list(E) == [1] * 6
    for i in range(6):
        for j in range(5):
            digits = qd.slice_entry(B[:, i, j], int(F[j]))
            trunc = sum(Fraction(d) * P ** (int(F[j]) - 13 * (s + 1)) for s, d in enumerate(digits))
            assert sum(Fraction(c) for c in C[:, i, j]) == trunc


@pytest.mark.parametrize("shape,dist,seed", [((7, 12, 9), "uniform", 30), ((5, 20, 6), "signed_exp20", 31)])
def test_exact_product_within_bound_and_bound_not_vacuous(shape, dist, seed):
    m, k, n = shape
    A = workloads.random_qd((m, k), seed, dist)
    B = workloads.random_qd((k, n), seed + 100, dist)
    E, F, S, C = qd.sliced_product(A, B)
    rows = [i for i in range(m) for _ in range(n)]
    cols = [j for _ in range(m) for j in range(n)]
    ex = qd.exact_entries(A, B, rows, cols)
    err = np.array([float(abs(sum(Fraction(c) for c in C[:, i, j]) - e)) for i, j, e in zip(rows, cols, ex)])
    bound = qd.error_bound(A[0], B[0], E, F, rows, cols)
    ratio = err / bound
    assert ratio.max() <= 1.0
    assert ratio.max() >= 2.0 ** -14          # the bound is within 2^14 of the observed error
    # a planted mistake in the oracle (level 15 dropped) breaks the bound
    S2 = S.copy()
    S2[15] = 0
    C2 = qd.renorm_levels(S2, E, F)
    err2 = np.array([float(abs(sum(Fraction(c) for c in C2[:, i, j]) - e)) for i, j, e in zip(rows, cols, ex)])
    assert (err2 / bound).max() > 1.0
