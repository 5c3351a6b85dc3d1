"""Seeded synthetic inputs for the double-double matrix product C = A·B.

This module is the only code shared by the HIP path's tests/bench and the CPU
oracle.  It draws random numbers and lays them out; it holds none of the
product's arithmetic (no slicing, no pair products, no renormalisation).

A double-double matrix is two float64 planes (hi, lo), row-major.  Every entry
is built the same way: draw ``hi`` from the workload's distribution, draw
``u ~ U(-1, 1)``, set ``lo_raw = hi * 2**-53 * u`` and store the pair
normalised, ``hi' = RN(hi + lo_raw)``, ``lo' = lo_raw - (hi' - hi)`` (Dekker's fast
two-sum, exact here because |lo_raw| < |hi|).  Seeds: the A operand of workload
``c`` uses ``numpy.random.default_rng(1000 + 10*c)``, the B operand
``default_rng(1000 + 10*c + 1)``; within one operand the draws are, in order,
the hi distribution's variates (sign, magnitude, exponent where present) and
then ``u``.

The pages ("Multiple Double Arithmetic on NVIDIA Tensor Cores", §4.1) say only
that random numbers were used; the five workloads below fix the shapes and
value distributions.

A quad-double matrix is four float64 planes (x0, x1, x2, x3).  Entry recipe:
draw x0 from the distribution, then for c = 0, 1, 2 draw u_c ~ U(-1/2, 1/2) and
set x_{c+1} = RN(x_c * 2**-53 * u_c), so every component is at most half an
ulp of the one before it (the normalisation of the quad-double library the
pages cite, [3]).  Seeds ``default_rng(2000 + 10*c)`` (A) and ``+ 1`` (B) for
quad-double workload ``c``; draws in order: x0's variates, then u_0, u_1, u_2.
The sizes follow the pages' quad-double runs (§4.2, Table 1: n = 1024, 2048).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

__all__ = ["Workload", "WORKLOADS", "QD_WORKLOADS", "by_name", "make_operands", "dd_pair_from_hi",
           "qd_from_x0", "random_qd", "make_qd_operands"]


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    m: int
    n: int
    k: int
    a_dist: str
    b_dist: str
    cancel_col0: bool = False
    description: str = ""

    @property
    def seeds(self) -> tuple[int, int]:
        return 1000 + 10 * self.index, 1000 + 10 * self.index + 1


WORKLOADS: tuple[Workload, ...] = (
    Workload(0, "dd64", 64, 64, 64, "uniform", "uniform",
             description="m=n=k=64, hi ~ U(-1,1)"),
    Workload(1, "dd1024", 1024, 1024, 1024, "uniform", "uniform",
             description="m=n=k=1024, hi ~ U(-1,1)"),
    Workload(2, "dd4096_exp20", 4096, 4096, 4096, "signed_exp20", "signed_exp20",
             description="m=n=k=4096, hi = sign*U(0.5,1)*2^e, e in [-20,20]"),
    Workload(3, "panel65536x512x512", 65536, 512, 512, "normal", "uniform",
             description="tall-skinny panel update m=65536, k=512, n=512; A hi ~ N(0,1), B hi ~ U(-1,1)"),
    Workload(4, "dd8192_exp30_cancel", 8192, 8192, 8192, "signed_exp30", "signed_exp30",
             cancel_col0=True,
             description="m=n=k=8192, hi = +-2^e*U(1,2), e in [-30,30]; B column 0 makes row sums of A·B cancel"),
)


QD_WORKLOADS: tuple[Workload, ...] = (
    Workload(0, "qd64", 64, 64, 64, "uniform", "uniform",
             description="quad-double m=n=k=64, x0 ~ U(-1,1)"),
    Workload(1, "qd1024", 1024, 1024, 1024, "uniform", "uniform",
             description="quad-double m=n=k=1024, x0 ~ U(-1,1)"),
    Workload(2, "qd2048", 2048, 2048, 2048, "uniform", "uniform",
             description="quad-double m=n=k=2048, x0 ~ U(-1,1)"),
    Workload(3, "qd4096_exp20", 4096, 4096, 4096, "signed_exp20", "signed_exp20",
             description="quad-double m=n=k=4096, x0 = sign*U(0.5,1)*2^e, e in [-20,20]"),
)


def by_name(name: str) -> Workload:
    for w in QD_WORKLOADS:
        if w.name == name:
            return w
    for w in WORKLOADS:
        if w.name == name or str(w.index) == str(name):
            return w
    raise KeyError(name)


def _draw_hi(rng: np.random.Generator, dist: str, shape) -> np.ndarray:
    if dist == "uniform":
        return rng.uniform(-1.0, 1.0, size=shape)
    if dist == "normal":
        return rng.standard_normal(size=shape)
    if dist in ("signed_exp20", "signed_exp30"):
        lo_b, hi_b, lo_e = (0.5, 1.0, 20) if dist == "signed_exp20" else (1.0, 2.0, 30)
        sign = rng.integers(0, 2, size=shape).astype(np.float64) * 2.0 - 1.0
        mag = rng.uniform(lo_b, hi_b, size=shape)
        e = rng.integers(-lo_e, lo_e + 1, size=shape)  # inclusive bounds
        return sign * np.ldexp(mag, e)
    raise ValueError(f"unknown distribution {dist!r}")


def dd_pair_from_hi(rng: np.random.Generator, hi: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Attach a low word at relative scale 2^-53 and store the pair normalised."""
    u = rng.uniform(-1.0, 1.0, size=hi.shape)
    lo_raw = hi * (2.0 ** -53) * u
    s = hi + lo_raw
    lo = lo_raw - (s - hi)
    return np.ascontiguousarray(s), np.ascontiguousarray(lo)


def _cancel_first_column(b_hi: np.ndarray, b_lo: np.ndarray) -> None:
    """Set B[r, 0] = -(sum over j >= 1 of B[r, j]) rounded to a normalised pair.

    math.fsum returns the correctly rounded sum of its (exact) inputs, so
    s_hi = RN(sum) and s_lo = RN(sum - s_hi); each row of B then sums to the
    tiny residue sum - s_hi - s_lo, and the row sums of A·B nearly cancel.
    """
    rows = b_hi.shape[0]
    for r in range(rows):
        terms = b_hi[r, 1:].tolist() + b_lo[r, 1:].tolist()
        s_hi = math.fsum(terms)
        terms.append(-s_hi)
        s_lo = math.fsum(terms)
        b_hi[r, 0] = -s_hi
        b_lo[r, 0] = -s_lo


def make_operands(w: Workload | str | int):
    """Return (A_hi, A_lo, B_hi, B_lo): contiguous float64, A is m×k, B is k×n."""
    if not isinstance(w, Workload):
        w = by_name(str(w))
    sa, sb = w.seeds
    ra = np.random.default_rng(sa)
    a_hi, a_lo = dd_pair_from_hi(ra, _draw_hi(ra, w.a_dist, (w.m, w.k)))
    rb = np.random.default_rng(sb)
    b_hi, b_lo = dd_pair_from_hi(rb, _draw_hi(rb, w.b_dist, (w.k, w.n)))
    if w.cancel_col0:
        _cancel_first_column(b_hi, b_lo)
    return a_hi, a_lo, b_hi, b_lo


def random_dd(shape, seed: int, dist: str = "uniform"):
    """A small seeded (hi, lo) matrix with a workload distribution (edge-case tests)."""
    rng = np.random.default_rng(seed)
    return dd_pair_from_hi(rng, _draw_hi(rng, dist, shape))


def qd_from_x0(rng: np.random.Generator, x0: np.ndarray) -> np.ndarray:
    """Stack (x0, x1, x2, x3) with x_{c+1} = RN(x_c * 2^-53 * u_c), u_c ~ U(-1/2, 1/2)."""
    out = np.empty((4,) + x0.shape, dtype=np.float64)
    out[0] = x0
    for c in range(3):
        u = rng.uniform(-0.5, 0.5, size=x0.shape)
        out[c + 1] = out[c] * (2.0 ** -53) * u
    return out


def random_qd(shape, seed: int, dist: str = "uniform") -> np.ndarray:
    """A small seeded quad-double matrix, shape (4, *shape) (edge-case tests)."""
    rng = np.random.default_rng(seed)
    return qd_from_x0(rng, _draw_hi(rng, dist, shape))


def make_qd_operands(w: Workload | str):
    """Return (A, B): float64 arrays of shape (4, m, k) and (4, k, n)."""
    if not isinstance(w, Workload):
        w = by_name(str(w))
    if w not in QD_WORKLOADS:
        raise KeyError(f"{w.name} is not a quad-double workload")
    ra = np.random.default_rng(2000 + 10 * w.index)
    A = qd_from_x0(ra, _draw_hi(ra, w.a_dist, (w.m, w.k)))
    rb = np.random.default_rng(2000 + 10 * w.index + 1)
    B = qd_from_x0(rb, _draw_hi(rb, w.b_dist, (w.k, w.n)))
    return A, B
