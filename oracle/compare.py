"""ORACLE -- test infrastructure only: the componentwise acceptance test for a
double-double product against a reference.

A result C is accepted at entry (i, j) when |C_ij - R_ij| <= tol * (|A||B|)_ij,
with (|A||B|)_ij = sum_k |a_hi[i,k]| * |b_hi[k,j]| in float64 (the lo words and
the rounding of this sum change it by a relative 2^-50 at most, irrelevant at
tol = 1e-28).  The difference is formed as (C_hi - R_hi) + (C_lo - R_lo): when
the hi words are within a few ulps the first subtraction is exact (Sterbenz),
and otherwise the difference is far above any tolerance anyway.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

TOL = 1e-28


def abs_product(A_hi, B_hi, rows=None, cols=None):
    A = np.abs(np.asarray(A_hi, dtype=np.float64))
    B = np.abs(np.asarray(B_hi, dtype=np.float64))
    if rows is None:
        return A @ B
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    return np.einsum("qk,kq->q", A[rows, :], B[:, cols])


def error_ratio(C_hi, C_lo, R_hi, R_lo, absAB):
    """max over entries of |C - R| / (|A||B|); entries with |A||B| == 0 must match exactly."""
    d = (np.asarray(C_hi) - np.asarray(R_hi)) + (np.asarray(C_lo) - np.asarray(R_lo))
    absAB = np.asarray(absAB, dtype=np.float64)
    zero = absAB == 0
    if np.any(d[zero] != 0):
        return float("inf")
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(zero, 0.0, np.abs(d) / np.where(zero, 1.0, absAB))
    return float(r.max(initial=0.0))


def exact_error_ratio(C_hi, C_lo, exact, absAB) -> float:
    """max_q |C_q - exact_q| / absAB_q with exact rationals (Fractions)."""
    worst = 0.0
    for ch, cl, ex, ab in zip(np.ravel(C_hi), np.ravel(C_lo), exact, np.ravel(absAB)):
        err = abs(Fraction(float(ch)) + Fraction(float(cl)) - ex)
        if ab == 0:
            if err != 0:
                return float("inf")
            continue
        worst = max(worst, float(err / Fraction(float(ab))))
    return worst


def eps_max(C_hi, C_lo, R_hi, R_lo) -> float:
    """max |C - R| over all entries (the pages' eq. (9), §4.2)."""
    d = (np.asarray(C_hi) - np.asarray(R_hi)) + (np.asarray(C_lo) - np.asarray(R_lo))
    return float(np.abs(d).max(initial=0.0))
