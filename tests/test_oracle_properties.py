"""Property tests of the oracle's slicing (CPU; hypothesis, derandomised).

The oracle cuts an entry into digits with integer shifts of its exact scaled
value.  These properties check the digits another way, from the definition of
the window in exact rationals: for any finite entry x (double-double pairs,
normalised or not, subnormal parts included; normalised quad doubles), any
slice count n and any window exponent E at or above the entry's balancing
exponent, the digits are 13-bit, carry the sign of x, and add up to
sign(x) * floor(|x| * 2^(13n - E)) * 2^(E - 13n), the truncation toward zero of
x to the window's grid.  Digit order, shift direction, sign handling and the
window's anchor all enter that identity.
"""
import math
from fractions import Fraction

import pytest

hypothesis = pytest.importorskip("hypothesis")
from hypothesis import given, settings, strategies as st  # noqa: E402

from oracle import exact, qd  # noqa: E402

SETTINGS = settings(max_examples=300, deadline=None, derandomize=True, database=None)

finite = st.floats(min_value=-2.0 ** 900, max_value=2.0 ** 900, allow_nan=False, allow_infinity=False,
                   allow_subnormal=True)
scale = st.integers(min_value=-1100, max_value=0)


def _window_truth(x: Fraction, E: int, n: int) -> Fraction:
    """sign(x) * floor(|x| * 2^(13n - E)) * 2^(E - 13n), in exact rationals."""
    unit = Fraction(2) ** (E - 13 * n)
    t = math.floor(abs(x) / unit) * unit
    return t if x >= 0 else -t


def _check_digits(digits, x: Fraction, E: int, n: int):
    assert len(digits) == n
    assert all(-8191 <= d <= 8191 for d in digits)
    assert all(d == 0 or (d > 0) == (x > 0) for d in digits)
    value = sum(Fraction(d) * Fraction(2) ** (E - 13 * (s + 1)) for s, d in enumerate(digits))
    assert value == _window_truth(x, E, n)


@SETTINGS
@given(hi=finite, lo=finite, lo_shift=scale, n=st.integers(4, 16), extra=st.integers(0, 40))
def test_dd_digits_are_the_truncated_window(hi, lo, lo_shift, n, extra):
    lo = math.ldexp(lo, lo_shift)  # lo anywhere from the size of hi down to subnormal
    x = Fraction(hi) + Fraction(lo)
    E0 = exact.entry_exponent(hi, lo)
    if x == 0:
        assert E0 is None
        assert exact.slice_entry(hi, lo, 0, n) == [0] * n
        return
    # E0 is the smallest exponent with |RN(x)| < 2^E0, hence |x| < 2^E0
    assert abs(x) < Fraction(2) ** E0
    E = E0 + extra
    _check_digits(exact.slice_entry(hi, lo, E, n), x, E, n)


def _qd_from(value: Fraction):
    comps = qd.greedy_qd(value)
    assert qd.is_normalized(comps)
    return comps


qd_values = st.builds(lambda num, e: Fraction(num) * Fraction(2) ** e,
                      st.integers(min_value=-(2 ** 230), max_value=2 ** 230), st.integers(-1250, 600))


@SETTINGS
@given(value=qd_values, n=st.integers(8, 16), extra=st.integers(0, 40))
def test_qd_digits_are_the_truncated_window(value, n, extra):
    comps = _qd_from(value)
    x = sum(Fraction(c) for c in comps)
    E0 = qd.entry_exponent(comps)
    if x == 0:
        assert E0 is None
        return
    assert abs(x) < Fraction(2) ** E0
    E = E0 + extra
    _check_digits(qd.slice_entry(comps, E, n), x, E, n)


@SETTINGS
@given(value=qd_values)
def test_qd_greedy_words_are_nonoverlapping_and_nearest(value):
    comps = qd.greedy_qd(value)
    rest = value
    for c in comps:
        if c != 0.0:
            # c is a nearest double of what is left: the remainder is at most half an ulp of c
            ulp = Fraction(2) ** (math.frexp(c)[1] - 53) if abs(c) >= 2.0 ** -1022 else Fraction(2) ** -1074
            assert abs(rest - Fraction(c)) <= ulp / 2
        rest -= Fraction(c)
    for a, b in zip(comps, comps[1:]):
        if a == 0.0:
            assert b == 0.0
        elif abs(a) >= 2.0 ** -1021:
            assert abs(Fraction(b)) <= Fraction(2) ** (math.frexp(a)[1] - 53) / 2
