"""ORACLE -- test infrastructure only.

Only tests/, the smoke check and the bench's CPU-baseline leg may import this
module.  It shares no code with the HIP path.

Exact references for the sliced quad-double product, the same method as the
double-double one ("Multiple Double Arithmetic on NVIDIA Tensor Cores": §2 says
a quartered quad-double matrix is sixteen times the size of a matrix of
doubles, §1 that the algorithms carry over to general multiple doubles, §4.2
Table 1 reports quad-double runs):

* a quad-double entry x = x0 + x1 + x2 + x3 is cut into sixteen 13-bit slices:
  a 208-bit window below a balancing exponent E with |x| < 2^E,
  N = floor(|x| * 2^(208 - E)), digit s = bits [13(15-s), 13(15-s)+13) of N,
  slice s = sign * digit * 2^(-13(s+1)),
* E for a row of A (column of B) is the largest frexp exponent of RN(x) over
  its nonzero entries (RN of the exact four-term sum), 0 when all are zero --
  the reading the double-double path uses for RN(hi + lo),
* level l collects the l + 1 pairs with s + t = l, l = 0..15 (136 pairs);
  pairs with s + t >= 16 are not formed,
* the sixteen level sums of an output entry are added exactly (each is an
  integer multiple of 2^(-13(l+2)) below 2^53 such units) and the exact total
  is rounded greedily to four doubles: c0 = RN(T), c1 = RN(T - c0),
  c2 = RN(T - c0 - c1), c3 = RN(T - c0 - c1 - c2), each scaled by 2^(E_i + F_j).
  The pages only say the parts are added in multiple-double arithmetic; this
  is the plainest exact reading, and its result is the nearest-rounded
  quad double of the exact level total.
* the product's plain definition, C_ij = sum_p a_ip b_pj exactly, is computed
  with Python integers.

Parity status: pinned (closed forms, brute force on tiny inputs, the exact
product within the stated error bound, agreement of the top eight digits with
the double-double slicer; see tests/test_oracle_qd_pins.py).
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

from .exact import DIGIT_BITS, DIGIT_MASK, double_to_scaled_int, level_sums_units

QD_SLICES = 16
QD_WINDOW_BITS = DIGIT_BITS * QD_SLICES  # 208
# §2 eq. (5): a sum of at most 67,108,865 products of 13-bit digits is exact;
# level 15 holds 16 pairs per k, so k <= 67,108,865 / 16.
QD_K_MAX = 67108865 // QD_SLICES
_SCALE_BITS = 1074


# ---------------------------------------------------------------------------
# exact values
# ---------------------------------------------------------------------------
def qd_scaled_int(comps) -> int:
    """X with x0 + x1 + x2 + x3 == X * 2^-1074 exactly."""
    return sum(double_to_scaled_int(float(c)) for c in comps)


def qd_fraction(comps) -> Fraction:
    return Fraction(qd_scaled_int(comps), 1 << _SCALE_BITS)


def is_normalized(comps) -> bool:
    """Every component is at most half an ulp of the one before it."""
    for c in range(len(comps) - 1):
        a, b = float(comps[c]), float(comps[c + 1])
        if a == 0.0:
            if b != 0.0:
                return False
        elif 2 * Fraction(abs(b)) > Fraction(math.ulp(a)):
            return False
    return True


def rn(value: Fraction) -> float:
    """The double nearest to an exact rational, ties to even (Python's int division)."""
    return value.numerator / value.denominator


# ---------------------------------------------------------------------------
# balancing exponents
# ---------------------------------------------------------------------------
def entry_exponent(comps) -> int | None:
    """frexp exponent of RN(x0 + x1 + x2 + x3); None for a zero entry."""
    V = qd_scaled_int(comps)
    if V == 0:
        return None
    return math.frexp(V / (1 << _SCALE_BITS))[1]


def balancing_exponents(X: np.ndarray, axis: int) -> np.ndarray:
    """One exponent per row (axis 0, operand A: X is (4, rows, k)) or per column
    (axis 1, operand B: X is (4, k, cols))."""
    X = np.asarray(X, dtype=np.float64)
    if axis == 1:
        X = X.transpose(0, 2, 1)
    out = np.zeros(X.shape[1], dtype=np.int32)
    for r in range(X.shape[1]):
        best = None
        for p in range(X.shape[2]):
            e = entry_exponent(X[:, r, p])
            if e is not None and (best is None or e > best):
                best = e
        out[r] = 0 if best is None else best
    return out


# ---------------------------------------------------------------------------
# slicing
# ---------------------------------------------------------------------------
def window_integer(comps, E: int, nslices: int = QD_SLICES) -> tuple[int, int]:
    """(sign, N) with N = floor(|x| * 2^(13 nslices - E))."""
    V = qd_scaled_int(comps)
    sign = (V > 0) - (V < 0)
    shift = DIGIT_BITS * nslices - E - _SCALE_BITS
    a = abs(V)
    return sign, (a << shift if shift >= 0 else a >> (-shift))


def slice_entry(comps, E: int, nslices: int = QD_SLICES) -> list[int]:
    """Signed digits d_0..d_{n-1}; the entry's slice s is d_s * 2^(E - 13(s+1))."""
    sign, N = window_integer(comps, E, nslices)
    if N >= 1 << (DIGIT_BITS * nslices):
        raise ValueError("balancing exponent too small for this entry")
    return [sign * ((N >> (DIGIT_BITS * (nslices - 1 - s))) & DIGIT_MASK) for s in range(nslices)]


def slice_rows(X, rows=None, nslices: int = QD_SLICES):
    """Slice operand A (X is (4, m, k)); returns (E, D) with D[s, r, p] int64."""
    X = np.asarray(X, dtype=np.float64)
    rows = range(X.shape[1]) if rows is None else list(rows)
    sub = X[:, list(rows), :]
    E = balancing_exponents(sub, axis=0)
    D = np.zeros((nslices, len(rows), X.shape[2]), dtype=np.int64)
    for r in range(len(rows)):
        for p in range(X.shape[2]):
            D[:, r, p] = slice_entry(sub[:, r, p], int(E[r]), nslices)
    return E, D


def slice_cols(X, cols=None, nslices: int = QD_SLICES):
    """Slice operand B (X is (4, k, n)); returns (F, D) with D[t, p, c]."""
    X = np.asarray(X, dtype=np.float64)
    F, Dt = slice_rows(X.transpose(0, 2, 1), cols, nslices)
    return F, np.ascontiguousarray(Dt.transpose(0, 2, 1))


def level_sums(DA: np.ndarray, DB: np.ndarray) -> np.ndarray:
    """S[l] = sum_{s+t=l} DA[s] @ DB[t] in units of 2^(-13(l+2)), l = 0..15."""
    if DA.shape[2] > QD_K_MAX:
        raise ValueError("k beyond the exact-sum bound")
    return level_sums_units(DA, DB)


# ---------------------------------------------------------------------------
# epilogue: exact level total, rounded greedily to four doubles
# ---------------------------------------------------------------------------
def level_total(S_units: np.ndarray, i: int, j: int) -> int:
    """T with sum_l S_l[i,j] 2^(-13(l+2)) == T * 2^(-13(n+1)), n levels."""
    nl = S_units.shape[0]
    return sum(int(S_units[l, i, j]) << (DIGIT_BITS * (nl - 1 - l)) for l in range(nl))


def rn_unbounded(value: Fraction) -> tuple[float, Fraction]:
    """(c, v): v is the double-precision number nearest to value with the
    exponent range unbounded above (53 significant bits, ties to even), c is v
    as a float -- equal to v, or +-inf once |v| reaches 2^1024, as IEEE
    round-to-nearest overflows."""
    try:
        c = rn(value)
        return c, Fraction(c)
    except OverflowError:
        pass
    a = abs(value)
    e = a.numerator.bit_length() - a.denominator.bit_length()  # 2^(e-1) < a < 2^(e+1)
    if a >= Fraction(2) ** e:
        e += 1                                                   # now 2^(e-1) <= a < 2^e
    ulp = Fraction(2) ** (e - 53)
    q = math.floor(a / ulp)
    rem = a / ulp - q
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and q % 2 == 1):
        q += 1
    v = q * ulp if value > 0 else -q * ulp
    return (math.inf if value > 0 else -math.inf), v


def greedy_qd(value: Fraction, terms: int = 4) -> list[float]:
    """c_0 = RN(value), c_1 = RN(value - c_0), ... (exact remainders).  Beyond
    the double range a word is +-inf and the next one rounds what is left after
    the word's unbounded value (rn_unbounded)."""
    out = []
    rest = value
    for _ in range(terms):
        c, v = rn_unbounded(rest)
        out.append(c)
        rest -= v
    return out


def renorm_levels(S_units: np.ndarray, E, F) -> np.ndarray:
    """Four (m×n) planes c0..c3 of the product from the integer level sums."""
    nl, m, n = S_units.shape
    out = np.zeros((4, m, n), dtype=np.float64)
    E = np.asarray(E, dtype=np.int64)
    F = np.asarray(F, dtype=np.int64)
    for i in range(m):
        for j in range(n):
            T = level_total(S_units, i, j)
            g = int(E[i]) + int(F[j]) - DIGIT_BITS * (nl + 1)
            val = Fraction(T) * (Fraction(2) ** g)
            out[:, i, j] = greedy_qd(val)
    return out


def sliced_product(A, B, nslices: int = QD_SLICES):
    """The whole chain on small inputs: (E, F, S_units, C planes)."""
    E, DA = slice_rows(A, nslices=nslices)
    F, DB = slice_cols(B, nslices=nslices)
    S = level_sums(DA, DB)
    return E, F, S, renorm_levels(S, E, F)


# ---------------------------------------------------------------------------
# the plain definition and an error bound
# ---------------------------------------------------------------------------
def exact_entries(A, B, rows, cols) -> list[Fraction]:
    """Exact C[rows[q], cols[q]] = sum_p a_ip b_pj (A is (4, m, k), B is (4, k, n))."""
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    out = []
    for i, j in zip(rows, cols):
        tot = 0
        for p in range(A.shape[2]):
            tot += qd_scaled_int(A[:, i, p]) * qd_scaled_int(B[:, p, j])
        out.append(Fraction(tot, 1 << (2 * _SCALE_BITS)))
    return out


def error_bound(A0, B0, E, F, rows, cols, nslices: int = QD_SLICES) -> np.ndarray:
    """Upper bound on |sum_c C_c - (A·B)_ij| per sampled entry.

    Cutting an entry below 2^E_i (2^F_j) loses less than 2^(E_i - 13n)
    (2^(F_j - 13n)); the pairs with s + t >= n that are not formed add less than
    n 2^(E_i + F_j - 13n) per term; rounding the exact level total to four
    doubles adds at most an ulp of c3, below 2^-200 (|A||B|)_ij.  |a| <=
    1.000001 |a0| for normalised quad doubles:
        bound = 2^(-13n) (2^F_j sum_p |a_ip| + 2^E_i sum_p |b_pj| + n k 2^(E_i+F_j))
                + 2^-200 (|A||B|)_ij
    """
    A = np.abs(np.asarray(A0, dtype=np.float64)) * 1.000001
    B = np.abs(np.asarray(B0, dtype=np.float64)) * 1.000001
    k = A.shape[1]
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    Sa = A[rows, :].sum(axis=1)
    Sb = B[:, cols].sum(axis=0)
    w = np.ldexp(1.0, np.asarray(E, dtype=np.int64)[rows])
    v = np.ldexp(1.0, np.asarray(F, dtype=np.int64)[cols])
    absAB = np.einsum("qk,kq->q", A[rows, :], B[:, cols])
    return 2.0 ** (-DIGIT_BITS * nslices) * (Sa * v + w * Sb + nslices * k * w * v) + 2.0 ** -200 * absAB
