"""Pins for the CPU oracle: each check ties the oracle to something other than
itself -- values the pages print, exact rational arithmetic, closed forms,
brute force on tiny inputs and invariants of the method.  No GPU needed."""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import compare, exact, native
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_rows(name):
    rows = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = line.split(":", 1)
            rows[key.strip()] = val.strip()
    return rows


# ---------------------------------------------------------------------------
# scalar error-free transformations of the classical oracle
# ---------------------------------------------------------------------------
def _rand_doubles(rng, n, spread=60):
    return [float(np.ldexp(rng.uniform(-1, 1), int(rng.integers(-spread, spread)))) for _ in range(n)]


def test_two_sum_and_two_prod_are_error_free():
    rng = np.random.default_rng(1)
    xs = _rand_doubles(rng, 400)
    ys = _rand_doubles(rng, 400)
    for a, b in zip(xs, ys):
        s, e = native.two_sum(a, b)
        assert s == a + b
        assert Fraction(s) + Fraction(e) == Fraction(a) + Fraction(b)
        p, q = native.two_prod(a, b)
        assert p == a * b
        assert Fraction(p) + Fraction(q) == Fraction(a) * Fraction(b)


def _dd(rng, spread=20):
    hi = float(np.ldexp(rng.uniform(0.5, 1.0), int(rng.integers(-spread, spread)))) * (1 if rng.random() < 0.5 else -1)
    lo_raw = hi * 2.0 ** -53 * rng.uniform(-1, 1)
    s = hi + lo_raw
    return s, lo_raw - (s - hi)


def test_dd_add_and_mul_error_bounds():
    u = 2.0 ** -53
    rng = np.random.default_rng(2)
    for _ in range(2000):
        xh, xl = _dd(rng)
        yh, yl = _dd(rng)
        X = Fraction(xh) + Fraction(xl)
        Y = Fraction(yh) + Fraction(yl)
        zh, zl = native.dd_mul(xh, xl, yh, yl)
        assert abs(Fraction(zh) + Fraction(zl) - X * Y) <= Fraction(5 * u * u) * abs(X * Y)
        assert zh == zh + zl  # normalised pair
        zh, zl = native.dd_add(xh, xl, yh, yl)
        # relative to |X| + |Y| (cancellation-safe form of the 3u^2 bound)
        assert abs(Fraction(zh) + Fraction(zl) - (X + Y)) <= Fraction(4 * u * u) * (abs(X) + abs(Y))
        assert zh == zh + zl


# ---------------------------------------------------------------------------
# classical dd GEMM oracle vs exact rationals and closed forms
# ---------------------------------------------------------------------------
def _rand_dd_matrix(rng, shape, kind):
    if kind == "uniform":
        hi = rng.uniform(-1, 1, shape)
    elif kind == "wide":
        hi = np.ldexp(rng.uniform(0.5, 1, shape), rng.integers(-30, 31, shape)) * rng.choice([-1.0, 1.0], shape)
    elif kind == "ints":
        return rng.integers(-100, 101, shape).astype(np.float64), np.zeros(shape)
    else:
        raise ValueError(kind)
    lo_raw = hi * 2.0 ** -53 * rng.uniform(-1, 1, shape)
    s = hi + lo_raw
    return s, lo_raw - (s - hi)


@pytest.mark.parametrize("shape", [(1, 1, 1), (3, 5, 7), (16, 9, 13), (7, 16, 16), (5, 4, 0)])
@pytest.mark.parametrize("kind", ["uniform", "wide"])
def test_oracle_gemm_vs_exact_rationals(shape, kind):
    m, n, k = shape
    rng = np.random.default_rng(hash((shape, kind)) & 0xFFFF)
    Ah, Al = _rand_dd_matrix(rng, (m, k), kind)
    Bh, Bl = _rand_dd_matrix(rng, (k, n), kind)
    Ch, Cl, _ = native.dd_gemm(Ah, Al, Bh, Bl)
    rows, cols = np.meshgrid(np.arange(m), np.arange(n), indexing="ij")
    ex = exact.exact_entries(Ah, Al, Bh, Bl, rows.ravel(), cols.ravel())
    absAB = compare.abs_product(Ah, Bh)
    assert compare.exact_error_ratio(Ch, Cl, ex, absAB) <= 1e-30
    if k == 0:
        assert np.all(Ch == 0) and np.all(Cl == 0)


def test_oracle_gemm_identity_is_exact():
    rng = np.random.default_rng(3)
    Bh, Bl = _rand_dd_matrix(rng, (12, 9), "wide")
    I = np.eye(12)
    Ch, Cl, _ = native.dd_gemm(I, np.zeros_like(I), Bh, Bl)
    assert np.array_equal(Ch, Bh) and np.array_equal(Cl, Bl)


def test_oracle_gemm_small_integers_exact():
    rng = np.random.default_rng(4)
    Ah, Al = _rand_dd_matrix(rng, (11, 23), "ints")
    Bh, Bl = _rand_dd_matrix(rng, (23, 6), "ints")
    Ch, Cl, _ = native.dd_gemm(Ah, Al, Bh, Bl)
    ref = Ah.astype(np.int64) @ Bh.astype(np.int64)
    assert np.array_equal(Ch, ref.astype(np.float64))
    assert np.all(Cl == 0)


def test_oracle_gemm_power_of_two_scaling_commutes():
    rng = np.random.default_rng(5)
    Ah, Al = _rand_dd_matrix(rng, (8, 10), "uniform")
    Bh, Bl = _rand_dd_matrix(rng, (10, 7), "uniform")
    Ch, Cl, _ = native.dd_gemm(Ah, Al, Bh, Bl)
    Sh, Sl, _ = native.dd_gemm(Ah * 2.0 ** 7, Al * 2.0 ** 7, Bh * 2.0 ** -12, Bl * 2.0 ** -12)
    assert np.array_equal(Sh, Ch * 2.0 ** -5) and np.array_equal(Sl, Cl * 2.0 ** -5)


def test_oracle_entries_match_full_product_bitwise():
    rng = np.random.default_rng(6)
    Ah, Al = _rand_dd_matrix(rng, (20, 33), "wide")
    Bh, Bl = _rand_dd_matrix(rng, (33, 17), "wide")
    Ch, Cl, _ = native.dd_gemm(Ah, Al, Bh, Bl, nthreads=3)
    rows = rng.integers(0, 20, 50)
    cols = rng.integers(0, 17, 50)
    eh, el = native.dd_gemm_entries(Ah, Al, Bh, Bl, rows, cols)
    assert np.array_equal(eh, Ch[rows, cols]) and np.array_equal(el, Cl[rows, cols])


def test_oracle_transpose_symmetry():
    rng = np.random.default_rng(7)
    Ah, Al = _rand_dd_matrix(rng, (9, 14), "uniform")
    Bh, Bl = _rand_dd_matrix(rng, (14, 5), "uniform")
    Ch, Cl, _ = native.dd_gemm(Ah, Al, Bh, Bl)
    Th, Tl, _ = native.dd_gemm(Bh.T, Bl.T, Ah.T, Al.T)
    # the same products in the same k order; dd_mul's cross terms are fused in the
    # other order, so the two agree to the oracle's own O(u^2) error, not bitwise
    assert np.array_equal(Th.T, Ch)
    assert compare.error_ratio(Th.T, Tl.T, Ch, Cl, compare.abs_product(Ah, Bh)) <= 1e-31


@pytest.mark.parametrize("name,samples", [("dd64", 256), ("dd1024", 256), ("dd4096_exp20", 96),
                                          ("panel65536x512x512", 256), ("dd8192_exp30_cancel", 48)])
def test_oracle_accuracy_on_workloads(workload_operands, name, samples):
    """The oracle itself stays far inside the acceptance tolerance on every workload."""
    Ah, Al, Bh, Bl = workload_operands(name)
    m, k = Ah.shape
    n = Bh.shape[1]
    rng = np.random.default_rng(99)
    rows = rng.integers(0, m, samples)
    cols = rng.integers(0, n, samples)
    if name.endswith("cancel"):
        cols[: samples // 4] = 0  # the cancelling column
    eh, el = native.dd_gemm_entries(Ah, Al, Bh, Bl, rows, cols)
    ex = exact.exact_entries(Ah, Al, Bh, Bl, rows, cols)
    absAB = compare.abs_product(Ah, Bh, rows, cols)
    assert compare.exact_error_ratio(eh, el, ex, absAB) <= 1e-29


def test_cancelling_workload_rows_nearly_cancel(workload_operands):
    """Column 0 of B is minus the rounded sum of the other columns, row by row."""
    Ah, Al, Bh, Bl = workload_operands("dd8192_exp30_cancel")
    for r in (0, 1, 4095, 8191):
        tot = sum((Fraction(float(h)) + Fraction(float(l)) for h, l in zip(Bh[r], Bl[r])), Fraction(0))
        scale = float(np.abs(Bh[r]).sum())
        assert abs(float(tot)) <= 2.0 ** -100 * scale


# ---------------------------------------------------------------------------
# slicing
# ---------------------------------------------------------------------------
def _bits(s):
    return "".join(ch for ch in s if ch in "01")


def test_slicing_reproduces_the_pages_worked_example():
    g = _golden_rows("quartering_example.txt")
    f = _bits(g["f"])
    assert len(f) == 52
    fields = []
    for i in range(4):
        row = _bits(g[f"f{i}"])
        assert len(row) == 52
        window = row[13 * i: 13 * (i + 1)]
        assert row[:13 * i].count("1") + row[13 * (i + 1):].count("1") == 0
        assert window == f[13 * i: 13 * (i + 1)]
        fields.append(int(window, 2))
    # the quarters x0..x3 display the same 13-bit fields at exponents 0, -13, -26, -39
    for i in range(4):
        parts = g[f"x{i}"].split()
        xbits = _bits(" ".join(parts[:-1]))[:13]
        assert int(xbits, 2) == fields[i]
        assert int(parts[-1]) == -13 * i
    x = int(f, 2) * 2.0 ** -52
    assert x.hex() == "0x1.234cc9da46998p-1"
    E = exact.entry_exponent(x, 0.0)
    assert E == 0
    assert exact.slice_entry(x, 0.0, E) == fields + [0, 0, 0, 0]
    assert fields == [4660, 6547, 5777, 5324]


def _edge_pairs(rng):
    """(hi, lo) pairs: normalised, unnormalised, opposite signs, subnormal, zero."""
    out = []
    for _ in range(300):
        hi, lo = _dd(rng, spread=40)
        out.append((hi, lo))
    out += [(1.0, -2.0 ** -60), (1.0, 2.0 ** -60), (-1.0, 2.0 ** -70), (0.75, 0.75), (1.0, -0.75),
            (2.0 ** -1074, 0.0), (3 * 2.0 ** -1070, -2.0 ** -1074), (0.0, 0.0), (-0.0, 0.0),
            (2.0 ** -30, 2.0 ** -150), (1.0 - 2.0 ** -53, 2.0 ** -200), (-(1.0 - 2.0 ** -53), -2.0 ** -107),
            (1e300, -1e283), (float.fromhex("0x1.fffffffffffffp+1023"), 0.0)]
    return out


def test_slicing_reconstructs_the_truncated_window():
    rng = np.random.default_rng(8)
    pairs = _edge_pairs(rng)
    for hi, lo in pairs:
        e0 = exact.entry_exponent(hi, lo)
        for E in ([0, 5] if e0 is None else [e0, e0 + 1, e0 + 20]):
            v = Fraction(hi) + Fraction(lo)
            d = exact.slice_entry(hi, lo, E)
            assert all(abs(x) <= 8191 for x in d)
            assert all((x >= 0) if v >= 0 else (x <= 0) for x in d)
            r = exact.reconstruct_entry(d, E)
            unit = Fraction(2) ** (E - 104)
            assert abs(r) <= abs(v) < abs(r) + unit  # truncation toward zero
            if (v / unit).denominator == 1:
                assert r == v  # on-grid values are represented exactly
            if v == 0:
                assert d == [0] * 8


def test_slicing_matches_digit_by_digit_expansion():
    """Brute force: peel 13-bit digits off |v| / 2^E by repeated scaling (a different algorithm)."""
    rng = np.random.default_rng(9)
    for hi, lo in _edge_pairs(rng)[:120]:
        E = exact.entry_exponent(hi, lo) or 0
        v = Fraction(hi) + Fraction(lo)
        r = abs(v) / Fraction(2) ** E
        assert r < 1
        digits = []
        for _ in range(8):
            r *= 8192
            d = math.floor(r)
            digits.append(d)
            r -= d
        sgn = -1 if v < 0 else 1
        assert exact.slice_entry(hi, lo, E) == [sgn * d for d in digits]


def test_slicing_rejects_too_small_exponent():
    with pytest.raises(ValueError):
        exact.slice_entry(1.0, 0.0, 0)  # |v| = 2^0 is not < 2^0


def test_balancing_exponents_bound_every_entry_tightly():
    rng = np.random.default_rng(10)
    Ah, Al = _rand_dd_matrix(rng, (6, 40), "wide")
    Ah[2, :] = 0.0
    Al[2, :] = 0.0  # all-zero row
    Al[3, 5] = -Ah[3, 5] * 0.75  # unnormalised pair in row 3
    E = exact.balancing_exponents(Ah, Al, axis=0)
    F = exact.balancing_exponents(Ah, Al, axis=1)
    assert E[2] == 0
    for i in range(6):
        vals = [abs(Fraction(h) + Fraction(l)) for h, l in zip(Ah[i], Al[i])]
        assert all(v < Fraction(2) ** int(E[i]) for v in vals)
        if i != 2:
            assert max(vals) >= Fraction(2) ** (int(E[i]) - 1) * (1 - Fraction(1, 2 ** 52))
    for j in range(40):
        vals = [abs(Fraction(h) + Fraction(l)) for h, l in zip(Ah[:, j], Al[:, j])]
        assert all(v < Fraction(2) ** int(F[j]) for v in vals)


def test_balancing_exponents_skip_zero_entries():
    """Zeros take no part in the maximum: a row of small values keeps its own
    (negative) exponent even next to a zero, and only an all-zero row gets 0."""
    hi = np.array([[0.0, 0.25, 2.0 ** -40, 0.0],
                   [0.0, 0.0, 0.0, 0.0],
                   [-3.0 * 2.0 ** -1070, 0.0, 2.0 ** -1074, -0.0],
                   [0.0, 0.75, -0.0, 1.0]])
    lo = np.zeros_like(hi)
    lo[3, 3] = -2.0 ** -60
    assert exact.balancing_exponents(hi, lo, axis=0).tolist() == [-1, 0, -1068, 1]  # RN(1 - 2^-60) = 1
    assert exact.balancing_exponents(hi, lo, axis=1).tolist() == [-1068, 0, -39, 1]
    for i in range(4):
        exps = [math.frexp(h + l)[1] for h, l in zip(hi[i], lo[i]) if h + l != 0.0]
        assert exact.balancing_exponents(hi[i:i + 1], lo[i:i + 1], 0)[0] == (max(exps) if exps else 0)


def test_slice_cols_is_slice_rows_of_transpose_with_column_exponents():
    rng = np.random.default_rng(11)
    Bh, Bl = _rand_dd_matrix(rng, (9, 5), "wide")
    F, D = exact.slice_cols(Bh, Bl)
    assert D.shape == (8, 9, 5)
    for j in range(5):
        col_max = max(exact.entry_exponent(h, l) for h, l in zip(Bh[:, j], Bl[:, j]))
        assert F[j] == col_max
        for p in range(9):
            assert list(D[:, p, j]) == exact.slice_entry(Bh[p, j], Bl[p, j], col_max)


# ---------------------------------------------------------------------------
# level sums and the exact-sum bound
# ---------------------------------------------------------------------------
def test_exact_sum_bound_matches_the_page():
    g = _golden_rows("exact_sum_bound.txt")
    assert 2 ** 52 // (2 ** 26 - 1) == int(g["N_max"])
    # a 13-bit by 13-bit digit product has at most 26 significant bits
    assert 8191 * 8191 < 2 ** 26


def test_level_sums_brute_force_eq3_structure():
    """Quarter-only inputs (lo = 0): levels 0..3 follow the convolution of eq. (3)."""
    rng = np.random.default_rng(12)
    m, k, n = 3, 4, 2
    Ah = rng.uniform(-1, 1, (m, k))
    Bh = rng.uniform(-1, 1, (k, n))
    E, DA = exact.slice_rows(Ah, None)
    F, DB = exact.slice_cols(Bh, None)
    S = exact.level_sums_units(DA, DB)
    for i in range(m):
        for j in range(n):
            for l in range(8):
                ref = 0
                for p in range(k):
                    for s in range(8):
                        t = l - s
                        if 0 <= t < 8:
                            ref += int(DA[s, i, p]) * int(DB[t, p, j])
                assert S[l, i, j] == ref


def test_level_sums_plus_dropped_pairs_equal_exact_windowed_product():
    """Kept levels (s+t <= 7) plus the dropped pairs (s+t >= 8) sum to the exact product
    of the windowed operands; a mis-indexed pair or transposed operand breaks this."""
    rng = np.random.default_rng(13)
    m, k, n = 5, 7, 3
    Ah, Al = _rand_dd_matrix(rng, (m, k), "wide")
    Bh, Bl = _rand_dd_matrix(rng, (k, n), "wide")
    E, DA = exact.slice_rows(Ah, Al)
    F, DB = exact.slice_cols(Bh, Bl)
    S = exact.level_sums_units(DA, DB)
    for i in range(m):
        for j in range(n):
            kept = exact.level_target(S, int(E[i]), int(F[j]), i, j)
            dropped = Fraction(0)
            for s in range(8):
                for t in range(8 - s, 8):
                    dd = sum(int(DA[s, i, p]) * int(DB[t, p, j]) for p in range(k))
                    dropped += Fraction(dd) * Fraction(2) ** (int(E[i]) + int(F[j]) - 13 * (s + t + 2))
            win = sum((exact.reconstruct_entry(DA[:, i, p], int(E[i])) *
                       exact.reconstruct_entry(DB[:, p, j], int(F[j])) for p in range(k)), Fraction(0))
            assert kept + dropped == win


def test_level_values_are_exact_and_bounded():
    rng = np.random.default_rng(14)
    DA = rng.integers(-8191, 8192, (8, 4, 64))
    DB = rng.integers(-8191, 8192, (8, 64, 4))
    S = exact.level_sums_units(DA, DB)
    for l in range(8):
        assert np.abs(S[l]).max() <= (l + 1) * 64 * 8191 ** 2
    V = exact.level_values(S)
    for l in range(8):
        assert np.array_equal((V[l] * 2.0 ** (13 * (l + 2))).astype(np.int64), S[l])


# ---------------------------------------------------------------------------
# renormalisation cascade
# ---------------------------------------------------------------------------
def test_cascade_is_exact_on_grid_values():
    """Levels holding the 13-bit digits of a 104-bit value: the cascade returns it exactly."""
    rng = np.random.default_rng(15)
    for _ in range(2000):
        N = int(rng.integers(1, 2 ** 52)) << 52 | int(rng.integers(0, 2 ** 52))
        sgn = -1 if rng.random() < 0.5 else 1
        digits = [sgn * ((N >> (13 * (7 - l))) & 8191) for l in range(8)]
        S = np.array([[[d * 2.0 ** (-13 * (l + 1))]] for l, d in enumerate(digits)])
        h, t = exact.renorm_levels(S, [0], [0])
        assert Fraction(float(h[0, 0])) + Fraction(float(t[0, 0])) == Fraction(sgn * N, 2 ** 104)
        assert h[0, 0] == h[0, 0] + t[0, 0]


def test_cascade_error_bound_with_cancellation():
    rng = np.random.default_rng(16)
    for trial in range(3000):
        units = [int(rng.integers(-2 ** 45, 2 ** 45)) for _ in range(8)]
        if trial % 3 == 0:  # force heavy cancellation between the two top levels
            units[0] = int(rng.integers(-2 ** 38, 2 ** 38))
            units[1] = -units[0] * 8192 + int(rng.integers(-5, 6))
        S = np.array([[[u * 2.0 ** (-13 * (l + 2))]] for l, u in enumerate(units)])
        E, F = int(rng.integers(-40, 40)), int(rng.integers(-40, 40))
        h, t = exact.renorm_levels(S, [E], [F])
        T = sum((Fraction(u) * Fraction(2) ** (E + F - 13 * (l + 2)) for l, u in enumerate(units)), Fraction(0))
        bound = Fraction(2) ** -104 * sum((abs(Fraction(u)) * Fraction(2) ** (E + F - 13 * (l + 2))
                                           for l, u in enumerate(units)), Fraction(0))
        assert abs(Fraction(float(h[0, 0])) + Fraction(float(t[0, 0])) - T) <= bound
        assert h[0, 0] == h[0, 0] + t[0, 0]


def test_cascade_zero_and_single_level():
    S = np.zeros((8, 2, 2))
    S[3, 1, 1] = 12345.0 * 2.0 ** -65
    h, t = exact.renorm_levels(S, [0, 3], [0, -2])
    assert np.all(t == 0)
    assert h[0, 0] == 0 and h[1, 1] == 12345.0 * 2.0 ** -64


# ---------------------------------------------------------------------------
# the acceptance test itself
# ---------------------------------------------------------------------------
def test_error_ratio_detects_a_planted_error():
    rng = np.random.default_rng(17)
    Ah, Al = _rand_dd_matrix(rng, (6, 8), "uniform")
    Bh, Bl = _rand_dd_matrix(rng, (8, 4), "uniform")
    Ch, Cl, _ = native.dd_gemm(Ah, Al, Bh, Bl)
    absAB = compare.abs_product(Ah, Bh)
    assert compare.error_ratio(Ch, Cl, Ch, Cl, absAB) == 0.0
    bad = Cl.copy()
    bad[2, 3] += 1e-25 * absAB[2, 3]
    assert compare.error_ratio(Ch, bad, Ch, Cl, absAB) > 1e-28


# ---------------------------------------------------------------------------
# fewer slices per operand (n = 4: the pages' quarters of a leading double)
# ---------------------------------------------------------------------------
def test_four_slices_are_the_pages_quarters():
    """With n = 4 the window is the 52-bit fraction of the worked example: the four
    slices are exactly the fields f0..f3 the page prints."""
    g = _golden_rows("quartering_example.txt")
    f = _bits(g["f"])
    x = int(f, 2) * 2.0 ** -52
    fields = [int(f[13 * i: 13 * (i + 1)], 2) for i in range(4)]
    assert exact.slice_entry(x, 0.0, 0, nslices=4) == fields
    # and the product of two such quarters-vectors follows eq. (3) level by level
    y = float.fromhex("0x1.9e0a3c2b5d1f8p-1")
    dy = exact.slice_entry(y, 0.0, 0, nslices=4)
    S = exact.level_sums_units(np.array(fields).reshape(4, 1, 1), np.array(dy).reshape(4, 1, 1))
    for l in range(4):
        assert S[l, 0, 0] == sum(fields[s] * dy[l - s] for s in range(l + 1))


@pytest.mark.parametrize("n", [4, 5, 6, 7, 10, 13, 16])
def test_slicing_with_n_slices_reconstructs_the_window(n):
    rng = np.random.default_rng(100 + n)
    for hi, lo in _edge_pairs(rng)[:150]:
        E = exact.entry_exponent(hi, lo)
        E = 0 if E is None else E + int(rng.integers(0, 3))
        v = Fraction(hi) + Fraction(lo)
        d = exact.slice_entry(hi, lo, E, nslices=n)
        assert len(d) == n and all(abs(x) <= 8191 for x in d)
        r = exact.reconstruct_entry(d, E)
        unit = Fraction(2) ** (E - 13 * n)
        assert abs(r) <= abs(v) < abs(r) + unit
        # the n-slice and the 8-slice digits agree on their common leading part
        d8 = exact.slice_entry(hi, lo, E)
        assert d[:8] == d8[:n]


@pytest.mark.parametrize("n", [4, 5])
def test_n_slice_levels_plus_dropped_pairs_equal_windowed_product(n):
    rng = np.random.default_rng(200 + n)
    m, k, c = 4, 6, 3
    Ah, Al = _rand_dd_matrix(rng, (m, k), "wide")
    Bh, Bl = _rand_dd_matrix(rng, (k, c), "wide")
    E, DA = exact.slice_rows(Ah, Al, nslices=n)
    F, DB = exact.slice_cols(Bh, Bl, nslices=n)
    S = exact.level_sums_units(DA, DB)
    assert S.shape == (n, m, c)
    for i in range(m):
        for j in range(c):
            kept = exact.level_target(S, int(E[i]), int(F[j]), i, j)
            dropped = Fraction(0)
            for s in range(n):
                for t in range(n - s, n):
                    dd = sum(int(DA[s, i, p]) * int(DB[t, p, j]) for p in range(k))
                    dropped += Fraction(dd) * Fraction(2) ** (int(E[i]) + int(F[j]) - 13 * (s + t + 2))
            win = sum((exact.reconstruct_entry(DA[:, i, p], int(E[i])) *
                       exact.reconstruct_entry(DB[:, p, j], int(F[j])) for p in range(k)), Fraction(0))
            assert kept + dropped == win


@pytest.mark.parametrize("n", list(range(4, 17)))
@pytest.mark.parametrize("kind", ["uniform", "wide"])
def test_error_bound_holds_for_the_exact_sliced_chain(n, kind):
    """The per-entry bound of exact.error_bound against exact rational products,
    for both ways of adding an entry's parts: the level cascade of the stage
    calls and the nearest double-double of the exact total (the products)."""
    rng = np.random.default_rng(300 + n + (kind == "wide"))
    m, k, c = 5, 17, 4
    Ah, Al = _rand_dd_matrix(rng, (m, k), kind)
    Bh, Bl = _rand_dd_matrix(rng, (k, c), kind)
    E, DA = exact.slice_rows(Ah, Al, nslices=n)
    F, DB = exact.slice_cols(Bh, Bl, nslices=n)
    S = exact.level_sums_units(DA, DB)
    Ch, Cl = exact.renorm_levels(exact.level_values(S), E, F)
    Nh, Nl = exact.nearest_dd(S, E, F)
    bound = exact.error_bound(Ah, Bh, E, F, n)
    rows, cols = np.meshgrid(np.arange(m), np.arange(c), indexing="ij")
    ex = exact.exact_entries(Ah, Al, Bh, Bl, rows.ravel(), cols.ravel())
    worst = 0.0
    for q, (i, j) in enumerate(zip(rows.ravel(), cols.ravel())):
        for (h, l) in ((Ch, Cl), (Nh, Nl)):
            err = abs(exact.dd_to_fraction(h[i, j], l[i, j]) - ex[q])
            assert err <= Fraction(float(bound[i, j])), (n, kind, i, j)
            worst = max(worst, float(err / Fraction(float(bound[i, j]))))
    # the bound is not vacuous for any n: the error comes within 2^14 of it
    # (beyond eight slices through the rounding term, 2^-104 of |A||B|)
    assert worst > 2.0 ** -14


def _wide_range_operands(k=24, gap=60, seed=17):
    """A row of A holds one entry 2^gap times its others, met by a zero row of B:
    the row's exponent is set by an entry that contributes nothing."""
    rng = np.random.default_rng(seed)
    Ah, Al = _rand_dd_matrix(rng, (3, k), "uniform")
    Bh, Bl = _rand_dd_matrix(rng, (k, 2), "uniform")
    Ah[0, 5], Al[0, 5] = 2.0 ** gap * 0.75, 0.0
    Bh[5, :], Bl[5, :] = 0.0, 0.0
    return Ah, Al, Bh, Bl


def test_more_slices_recover_entries_far_below_the_row_maximum():
    """§3 Problem 3.2's concern: with eight slices the small entries of the first
    row keep only 104 - 60 bits and the product misses the tolerance; with
    13 slices (13 * 5 = 65 more bits of window) they keep their full pair."""
    Ah, Al, Bh, Bl = _wide_range_operands()
    ref = exact.exact_entries(Ah, Al, Bh, Bl, [0, 0, 1], [0, 1, 0])
    absab = compare.abs_product(Ah, Bh)

    def worst(n):
        E, DA = exact.slice_rows(Ah, Al, nslices=n)
        F, DB = exact.slice_cols(Bh, Bl, nslices=n)
        Ch, Cl = exact.renorm_levels(exact.level_values(exact.level_sums_units(DA, DB)), E, F)
        return max(float(abs(exact.dd_to_fraction(Ch[i, j], Cl[i, j]) - r)) / absab[i, j]
                   for (i, j), r in zip([(0, 0), (0, 1), (1, 0)], ref))

    assert worst(8) > compare.TOL
    assert worst(13) <= compare.TOL
    assert worst(16) <= compare.TOL


def test_kblocked_chain_with_one_block_is_the_plain_chain():
    rng = np.random.default_rng(41)
    Ah, Al = _rand_dd_matrix(rng, (6, 23), "wide")
    Bh, Bl = _rand_dd_matrix(rng, (23, 5), "wide")
    Ch, Cl = exact.sliced_product(Ah, Al, Bh, Bl)
    for kb in (23, 24, 1000):
        Kh, Kl = exact.sliced_product_kblocks(Ah, Al, Bh, Bl, kb)
        assert np.array_equal(Kh.view(np.int64), Ch.view(np.int64))
        assert np.array_equal(Kl.view(np.int64), Cl.view(np.int64))


@pytest.mark.parametrize("kblock", [1, 5, 8, 16])
def test_kblocked_chain_within_the_summed_bound(kblock):
    """Each block obeys its own error bound (its own exponents); the accurate
    double-word additions add at most 3u^2 of the running sum each (u = 2^-53)."""
    rng = np.random.default_rng(50 + kblock)
    m, k, c = 4, 37, 3
    Ah, Al = _rand_dd_matrix(rng, (m, k), "wide")
    Bh, Bl = _rand_dd_matrix(rng, (k, c), "wide")
    Ch, Cl = exact.sliced_product_kblocks(Ah, Al, Bh, Bl, kblock)
    bound = np.zeros((m, c))
    for p0 in range(0, k, kblock):
        p1 = min(k, p0 + kblock)
        E = exact.balancing_exponents(Ah[:, p0:p1], Al[:, p0:p1], 0)
        F = exact.balancing_exponents(Bh[p0:p1], Bl[p0:p1], 1)
        bound += exact.error_bound(Ah[:, p0:p1], Bh[p0:p1], E, F, 8)
    nblocks = -(-k // kblock)
    bound += (nblocks - 1) * 3 * 2.0 ** -106 * compare.abs_product(Ah, Bh) * 1.000001
    rows, cols = np.meshgrid(np.arange(m), np.arange(c), indexing="ij")
    ex = exact.exact_entries(Ah, Al, Bh, Bl, rows.ravel(), cols.ravel())
    for q, (i, j) in enumerate(zip(rows.ravel(), cols.ravel())):
        err = abs(exact.dd_to_fraction(Ch[i, j], Cl[i, j]) - ex[q])
        assert err <= Fraction(float(bound[i, j])), (kblock, i, j)
    # blocks really are separate: block-local exponents change the low bits
    Ph, Pl = exact.sliced_product(Ah, Al, Bh, Bl)
    assert not (np.array_equal(Ph.view(np.int64), Ch.view(np.int64))
                and np.array_equal(Pl.view(np.int64), Cl.view(np.int64)))
