"""ORACLE -- test infrastructure only.

Only tests/, the smoke check and the bench's CPU-baseline leg may import this
module.  It shares no code with the HIP path.

Exact references for every intermediate of the sliced double-double product
(the method of "Multiple Double Arithmetic on NVIDIA Tensor Cores"):

* balancing exponents and 13-bit slicing (§2 "quartering" and its worked
  example; §3 balancing, Problems 3.3 and 3.4),
* the level sums of slice-pair products (§2, eqs. (1)-(4)),
* the level-ordered renormalisation of the level sums into (hi, lo) (§2, the
  fifth step: sum the parts of each product entry in double-double arithmetic),
* the exact rational value of a double-double inner product.

Readings of points the pages leave open:

* A double-double x = hi + lo is cut as a 13n-bit fixed-point window below a
  balancing exponent E with |hi + lo| < 2^E: N = floor(|hi + lo| * 2^(13n-E)),
  digit s = bits [13(n-1-s), 13(n-1-s)+13) of N, slice s = sign * digit *
  2^(-13(s+1)), for n slices.  n = 8 (a 104-bit window, §2 eq. (4)) is the
  double-double product; n = 4 is the pages' four quarters of a leading double
  (§2 eqs. (1)-(3)); the number of slices is a parameter (default 8).  Slices sit
  at relative exponents 0, -13, ... (the pages' quarters at 0, -13, -26, -39 for
  hi, continued for lo).  Truncation toward zero, as the pages' bit fields are.
* E for a row of A (column of B) is the largest frexp exponent of RN(hi + lo)
  over its nonzero entries, 0 when all are zero.
* Level l collects the pairs s + t = l for l = 0..n-1 (n(n+1)/2 pairs, 36 for
  n = 8); pairs below the window (s + t >= n) are not formed.
* The cascade starts from the smallest level: (h, t) = (S_{n-1}, 0); for l = n-2..0:
  (s, e) = TwoSum(h, S_l), t = t + e, (h, t) = TwoSum(s, t); then both words are
  scaled by 2^(E_i + F_j).  That is the stage chain's epilogue.  The product
  entry points round each entry's exact level total to the nearest double-double
  instead (nearest_dd): the pages fix no order for adding the parts, and the
  exact sum rounded once is the most accurate order and the same for any
  grouping of the slice products (pair_schedule).

Parity status: pinned (the pages' worked example, reconstruction identities,
brute force on tiny inputs, closed forms; see tests/test_oracle_pins.py, and
for the pair-packed schedule and the nearest double-double,
tests/test_oracle_paired_pins.py).
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

WINDOW_BITS = 104
DIGIT_BITS = 13
N_SLICES = 8
N_LEVELS = 8
DIGIT_MASK = (1 << DIGIT_BITS) - 1

# ---------------------------------------------------------------------------
# exact conversions
# ---------------------------------------------------------------------------
_SCALE_BITS = 1074  # every finite double is an integer multiple of 2^-1074


def double_to_scaled_int(x: float) -> int:
    """Return X with x == X * 2^-1074 exactly (x finite)."""
    p, q = float(x).as_integer_ratio()
    return p << (_SCALE_BITS - (q.bit_length() - 1))


def dd_to_fraction(hi: float, lo: float) -> Fraction:
    return Fraction(float(hi)) + Fraction(float(lo))


# ---------------------------------------------------------------------------
# balancing exponents
# ---------------------------------------------------------------------------
def entry_exponent(hi: float, lo: float) -> int | None:
    """frexp exponent of RN(hi + lo) (smallest e with |RN(hi+lo)| < 2^e); None for zero."""
    s = float(hi) + float(lo)
    if s == 0.0:
        return None
    return math.frexp(s)[1]


def balancing_exponents(hi: np.ndarray, lo: np.ndarray | None, axis: int) -> np.ndarray:
    """One exponent per row (axis=0, the A operand) or per column (axis=1, the B operand)."""
    hi = np.asarray(hi, dtype=np.float64)
    lo = np.zeros_like(hi) if lo is None else np.asarray(lo, dtype=np.float64)
    s = hi + lo
    _, ex = np.frexp(s)
    none = np.int64(np.iinfo(np.int64).min)  # zero entries take no part in the maximum
    ex = np.where(s != 0.0, ex.astype(np.int64), none)
    red = ex.max(axis=1 if axis == 0 else 0) if ex.size else np.full(
        hi.shape[0] if axis == 0 else hi.shape[1], none, dtype=np.int64)
    return np.where(red == none, 0, red).astype(np.int32)


# ---------------------------------------------------------------------------
# slicing
# ---------------------------------------------------------------------------
def window_integer(hi: float, lo: float, E: int, nslices: int = N_SLICES) -> tuple[int, int]:
    """(sign, N) with N = floor(|hi + lo| * 2^(13 nslices - E)), sign in {-1, 0, 1}."""
    H = double_to_scaled_int(hi)
    L = double_to_scaled_int(lo)
    V = H + L  # (hi + lo) * 2^1074, exact
    sign = (V > 0) - (V < 0)
    shift = DIGIT_BITS * nslices - E - _SCALE_BITS  # N = floor(|V| * 2^shift)
    a = abs(V)
    N = a << shift if shift >= 0 else a >> (-shift)
    return sign, N


def slice_entry(hi: float, lo: float, E: int, nslices: int = N_SLICES) -> list[int]:
    """Signed 13-bit digits d_0..d_{n-1} of one entry; slice s = d_s * 2^(E - 13(s+1))."""
    sign, N = window_integer(hi, lo, E, nslices)
    if N >= 1 << (DIGIT_BITS * nslices):
        raise ValueError("balancing exponent too small for this entry")
    return [sign * ((N >> (DIGIT_BITS * (nslices - 1 - s))) & DIGIT_MASK)
            for s in range(nslices)]


def slice_rows(hi, lo, rows=None, nslices: int = N_SLICES):
    """Slice the A operand (per-row exponents).

    Returns (E, D) with E[r] for the selected rows and D[s, r, k] the signed
    digits (int64), r indexing ``rows`` (all rows when None).
    """
    hi = np.asarray(hi, dtype=np.float64)
    lo = np.zeros_like(hi) if lo is None else np.asarray(lo, dtype=np.float64)
    rows = range(hi.shape[0]) if rows is None else list(rows)
    E = balancing_exponents(hi[rows, :], lo[rows, :], axis=0)
    D = np.zeros((nslices, len(rows), hi.shape[1]), dtype=np.int64)
    for r, i in enumerate(rows):
        for p in range(hi.shape[1]):
            D[:, r, p] = slice_entry(hi[i, p], lo[i, p], int(E[r]), nslices)
    return E, D


def slice_cols(hi, lo, cols=None, nslices: int = N_SLICES):
    """Slice the B operand (per-column exponents); D[t, k, c] for the selected columns."""
    hi = np.asarray(hi, dtype=np.float64)
    lo = np.zeros_like(hi) if lo is None else np.asarray(lo, dtype=np.float64)
    F, Dt = slice_rows(hi.T, lo.T, cols, nslices)
    return F, np.ascontiguousarray(Dt.transpose(0, 2, 1))


def slice_values(D: np.ndarray) -> np.ndarray:
    """Unit-scaled slice values d_s * 2^(-13(s+1)) (the scale 2^E is kept apart)."""
    n = D.shape[0]
    scale = np.array([2.0 ** (-DIGIT_BITS * (s + 1)) for s in range(n)])
    return D.astype(np.float64) * scale.reshape((n,) + (1,) * (D.ndim - 1))


def reconstruct_entry(digits, E: int) -> Fraction:
    """sum_s d_s * 2^(E - 13(s+1)) as an exact rational."""
    return sum((Fraction(int(d)) * Fraction(2) ** (E - DIGIT_BITS * (s + 1))
                for s, d in enumerate(digits)), Fraction(0))


# ---------------------------------------------------------------------------
# level sums
# ---------------------------------------------------------------------------
def level_sums_units(DA: np.ndarray, DB: np.ndarray) -> np.ndarray:
    """S[l] = sum_{s+t=l} DA[s] @ DB[t] in integer units, l = 0..n-1 for n slices.

    DA[s] is m×k, DB[t] is k×n (int64 digits).  Level l has weight
    2^(E_i + F_j - 13(l+2)).  Every term fits in int64 for k < 2^21.
    """
    nl = DA.shape[0]
    assert DB.shape[0] == nl
    m, k = DA.shape[1], DA.shape[2]
    n = DB.shape[2]
    S = np.zeros((nl, m, n), dtype=np.int64)
    for l in range(nl):
        for s in range(l + 1):
            S[l] += DA[s] @ DB[l - s]
    return S


def level_values(S_units: np.ndarray) -> np.ndarray:
    """Level sums as unit-scaled doubles, S_l = S_units[l] * 2^(-13(l+2)) (exact when < 2^53)."""
    if np.abs(S_units).max(initial=0) >= 2 ** 53:
        raise ValueError("level sum exceeds 53 bits")
    out = S_units.astype(np.float64)
    for l in range(S_units.shape[0]):
        out[l] *= 2.0 ** (-DIGIT_BITS * (l + 2))
    return out


# ---------------------------------------------------------------------------
# renormalisation cascade
# ---------------------------------------------------------------------------
def two_sum(a, b):
    """Knuth's TwoSum, elementwise: s = RN(a + b), e = a + b - s exactly."""
    s = a + b
    bv = s - a
    av = s - bv
    e = (a - av) + (b - bv)
    return s, e


def renorm_levels(S: np.ndarray, E, F):
    """Cascade the unit-scaled level planes S[l] (m×n), l = 0..n-1, into (C_hi, C_lo).

    E (length m) and F (length n) are the balancing exponents of A's rows and
    B's columns.  Smallest level first, as described in the module docstring.
    """
    S = np.asarray(S, dtype=np.float64)
    nl = S.shape[0]
    h = S[nl - 1].copy()
    t = np.zeros_like(h)
    for l in range(nl - 2, -1, -1):
        s, e = two_sum(h, S[l])
        t = t + e
        h, t = two_sum(s, t)
    sc = np.asarray(E, dtype=np.int64).reshape(-1, 1) + np.asarray(F, dtype=np.int64).reshape(1, -1)
    return np.ldexp(h, sc), np.ldexp(t, sc)


def sliced_product(A_hi, A_lo, B_hi, B_lo, nslices: int = N_SLICES):
    """The whole chain on one block: (C_hi, C_lo) of the sliced product."""
    E, DA = slice_rows(A_hi, A_lo, nslices=nslices)
    F, DB = slice_cols(B_hi, B_lo, nslices=nslices)
    return renorm_levels(level_values(level_sums_units(DA, DB)), E, F)


def sliced_product_kblocks(A_hi, A_lo, B_hi, B_lo, kblock: int, nslices: int = N_SLICES, nearest: bool = False):
    """k split into consecutive blocks of kblock columns of A (rows of B); each
    block is an independent sliced product (its own balancing exponents, so the
    exact-sum bound of §2 eq. (5) holds per block), and the block results are
    added into the running (C_hi, C_lo), first block first, with the oracle's
    accurate double-word addition.  Each block's result is the level cascade,
    or with `nearest` the nearest double-double of its exact total (the
    product entry points' chain)."""
    from . import native
    A_hi = np.asarray(A_hi, dtype=np.float64)
    B_hi = np.asarray(B_hi, dtype=np.float64)
    A_lo = np.zeros_like(A_hi) if A_lo is None else np.asarray(A_lo, dtype=np.float64)
    B_lo = np.zeros_like(B_hi) if B_lo is None else np.asarray(B_lo, dtype=np.float64)
    k = A_hi.shape[1]
    starts = list(range(0, k, kblock)) if k > 0 else [0]
    C_hi = C_lo = None
    for p0 in starts:
        p1 = min(k, p0 + kblock)
        block = paired_product if nearest else sliced_product
        Th, Tl = block(A_hi[:, p0:p1], A_lo[:, p0:p1], B_hi[p0:p1, :], B_lo[p0:p1, :], nslices)
        if C_hi is None:
            C_hi, C_lo = Th, Tl
            continue
        for i in range(C_hi.shape[0]):
            for j in range(C_hi.shape[1]):
                C_hi[i, j], C_lo[i, j] = native.dd_add(C_hi[i, j], C_lo[i, j], Th[i, j], Tl[i, j])
    return C_hi, C_lo


def level_target(S_units: np.ndarray, E: int, F: int, i: int, j: int) -> Fraction:
    """Exact value sum_l S_units[l][i,j] * 2^(E + F - 13(l+2)) of one output entry."""
    return sum((Fraction(int(S_units[l, i, j])) * Fraction(2) ** (E + F - DIGIT_BITS * (l + 2))
                for l in range(S_units.shape[0])), Fraction(0))


# ---------------------------------------------------------------------------
# the pair-packed schedule: two slices of A in one 26-bit operand
# ---------------------------------------------------------------------------
def pair_schedule(nslices: int = N_SLICES) -> list[tuple[int, int, int, int]]:
    """The matrix products of the pair-packed schedule, as (s_hi, s_lo, t, g).

    Slices 2u and 2u + 1 of an A entry have the same sign and sit 13 bits apart,
    so d_2u 2^13 + d_(2u+1) is one exact 26-bit integer; its product with a
    13-bit B digit d_t is a 39-bit integer that covers the two window pairs
    (2u, t) and (2u+1, t) at once.  Where only (2u, t) lies in the window
    (2u + t = n - 1), or A has no slice 2u + 1 (odd n), the product is the
    single pair (2u, t), written with s_lo = -1.  Every pair s + t <= n - 1 is
    covered exactly once.  A product's exact value is an integer number of
    units 2^(-13(g+3)) (g = 2u + t for a packed pair, n - 2 for a single one):
    g indexes the n - 1 group sums G_g of an output entry, so that its exact
    windowed total is sum_g G_g 2^(-13(g+3)) (times 2^(E_i + F_j)).
    """
    n = nslices
    out = []
    for u in range((n + 1) // 2):
        s0, s1 = 2 * u, 2 * u + 1
        for t in range(n):
            if s1 < n and s1 + t <= n - 1:
                out.append((s0, s1, t, s0 + t))
            elif s0 + t <= n - 1:
                out.append((s0, -1, t, n - 2))
    return out


def paired_group_units(DA: np.ndarray, DB: np.ndarray) -> np.ndarray:
    """G[g] = sum of the schedule's products of group g, in integer units
    2^(-13(g+3)), g = 0..n-2, from the int64 digit planes DA[s] (m×k) and
    DB[t] (k×n).  Exact in int64 while k (2^39 + 2^26) n < 2^63."""
    n = DA.shape[0]
    m, k = DA.shape[1], DA.shape[2]
    G = np.zeros((n - 1, m, DB.shape[2]), dtype=np.int64)
    for s0, s1, t, g in pair_schedule(n):
        a = DA[s0] * (1 << DIGIT_BITS) + DA[s1] if s1 >= 0 else DA[s0]
        G[g] += a @ DB[t]
    return G


# ---------------------------------------------------------------------------
# the product's epilogue: the nearest double-double of the exact total
# ---------------------------------------------------------------------------
def nearest_dd(S_units: np.ndarray, E, F):
    """(C_hi, C_lo) of every entry from its exact level total
    x = sum_l S_units[l] 2^(E_i + F_j - 13(l+2)): C_hi = RN(x), C_lo =
    RN(x - C_hi), the double-double nearest to x (ties to even, gradual
    underflow).  Beyond the double range C_hi is +-inf and C_lo rounds what is
    left after C_hi's value with an unbounded exponent range (the reading the
    quad-double words use).  The pages add the parts of an entry in
    double-double arithmetic without fixing the order; the exact total rounded
    once is the most accurate such sum and does not depend on how the slice
    products were grouped."""
    from .qd import greedy_qd
    nl, m, n = S_units.shape
    E = np.asarray(E, dtype=np.int64)
    F = np.asarray(F, dtype=np.int64)
    hi = np.zeros((m, n), dtype=np.float64)
    lo = np.zeros((m, n), dtype=np.float64)
    for i in range(m):
        for j in range(n):
            hi[i, j], lo[i, j] = greedy_qd(level_target(S_units, int(E[i]), int(F[j]), i, j), 2)
    return hi, lo


def paired_product(A_hi, A_lo, B_hi, B_lo, nslices: int = N_SLICES):
    """The product entry points' chain on one block: slices, the exact sum of
    the window pairs, rounded to the nearest double-double."""
    E, DA = slice_rows(A_hi, A_lo, nslices=nslices)
    F, DB = slice_cols(B_hi, B_lo, nslices=nslices)
    return nearest_dd(level_sums_units(DA, DB), E, F)


# ---------------------------------------------------------------------------
# exact double-double inner products
# ---------------------------------------------------------------------------
def exact_dot(a_hi, a_lo, b_hi, b_lo) -> Fraction:
    """sum_k (a_hi[k] + a_lo[k]) * (b_hi[k] + b_lo[k]) exactly."""
    tot = 0
    for ah, al, bh, bl in zip(a_hi, a_lo, b_hi, b_lo):
        tot += (double_to_scaled_int(ah) + double_to_scaled_int(al)) * \
               (double_to_scaled_int(bh) + double_to_scaled_int(bl))
    return Fraction(tot, 1 << (2 * _SCALE_BITS))


def exact_entries(A_hi, A_lo, B_hi, B_lo, rows, cols) -> list[Fraction]:
    """Exact C[rows[q], cols[q]] for every q (A_lo / B_lo may be None)."""
    A_lo = np.zeros_like(A_hi) if A_lo is None else A_lo
    B_lo = np.zeros_like(B_hi) if B_lo is None else B_lo
    return [exact_dot(A_hi[i, :], A_lo[i, :], B_hi[:, j], B_lo[:, j]) for i, j in zip(rows, cols)]


def error_bound(A_hi, B_hi, E, F, nslices: int, rows=None, cols=None):
    """Upper bound on |C - A·B| for the sliced product with n slices, per entry,
    against the exact product.

    Cutting each entry below 2^E_i (2^F_j) loses less than 2^(E_i - 13n)
    (2^(F_j - 13n)), so one product term is off by less than
    2^(-13n) (|a| 2^F_j + |b| 2^E_i); the pairs with s + t >= n that are not formed
    add at most (n-1) 2^(E_i + F_j - 13n) per term.  Adding the parts of an entry
    costs at most 2^-104 of the sum of their magnitudes: the level cascade's
    TwoSum steps, or, for the nearest double-double of the exact total,
    |T - hi - lo| <= 2^-106 |T| (1 + 2^-52).  The digits of one entry share its
    sign, so the level (or group) magnitudes add up to at most (|A||B|)_ij.  With
    the lo words below 2^-52 of hi, |a| and |b| are bounded by 1.000001 |a_hi|,
    |b_hi|:
        bound_ij = 2^(-13n) (2^F_j S_a[i] + 2^E_i S_b[j] + n k 2^(E_i+F_j))
                   + 2^-104 (|A||B|)_ij
    with S_a[i] = sum_p |a_ip|, S_b[j] = sum_p |b_pj| (times 1.000001).
    """
    A = np.abs(np.asarray(A_hi, dtype=np.float64)) * 1.000001
    B = np.abs(np.asarray(B_hi, dtype=np.float64)) * 1.000001
    k = A.shape[1]
    Sa = A.sum(axis=1)
    Sb = B.sum(axis=0)
    w = np.ldexp(1.0, np.asarray(E, dtype=np.int64))
    v = np.ldexp(1.0, np.asarray(F, dtype=np.int64))
    if rows is None:
        absAB = A @ B
        return 2.0 ** (-DIGIT_BITS * nslices) * (np.outer(Sa, v) + np.outer(w, Sb) + nslices * k * np.outer(w, v)) \
            + 2.0 ** -104 * absAB
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    absAB = np.einsum("qk,kq->q", A[rows, :], B[:, cols])
    return 2.0 ** (-DIGIT_BITS * nslices) * (Sa[rows] * v[cols] + w[rows] * Sb[cols]
                                             + nslices * k * w[rows] * v[cols]) + 2.0 ** -104 * absAB
