"""ORACLE -- test infrastructure only: ctypes loader for the classical CPU
double-double GEMM in dd_gemm_oracle.c.  Only tests/, the smoke check and the
bench's CPU-baseline leg may import it."""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_lib = None
_dp = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.c_int64


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build(verbose=False)
        L = ctypes.CDLL(_build.LIB)
        L.oracle_dd_gemm.restype = ctypes.c_int
        L.oracle_dd_gemm.argtypes = [_i64, _i64, _i64, _dp, _dp, _i64, _dp, _dp, _i64,
                                     _dp, _dp, _i64, ctypes.c_int]
        L.oracle_dd_gemm_entries.restype = ctypes.c_int
        L.oracle_dd_gemm_entries.argtypes = [_i64, ctypes.POINTER(_i64), ctypes.POINTER(_i64),
                                             _i64, _i64, _i64, _dp, _dp, _i64, _dp, _dp, _i64,
                                             _dp, _dp, ctypes.c_int]
        for name in ("oracle_two_sum", "oracle_two_prod"):
            f = getattr(L, name)
            f.restype = None
            f.argtypes = [ctypes.c_double, ctypes.c_double, _dp, _dp]
        for name in ("oracle_dd_mul", "oracle_dd_add"):
            f = getattr(L, name)
            f.restype = None
            f.argtypes = [ctypes.c_double] * 4 + [_dp, _dp]
        L.oracle_max_threads.restype = ctypes.c_int
        L.oracle_max_threads.argtypes = []
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_dp)


def _c64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def dd_gemm(A_hi, A_lo, B_hi, B_lo, nthreads: int = 0):
    """C = A·B in classical double-double arithmetic. Returns (C_hi, C_lo, threads_used)."""
    A_hi, A_lo, B_hi, B_lo = map(_c64, (A_hi, A_lo, B_hi, B_lo))
    m, k = A_hi.shape
    k2, n = B_hi.shape
    assert k == k2
    C_hi = np.zeros((m, n))
    C_lo = np.zeros((m, n))
    used = lib().oracle_dd_gemm(m, n, k, _ptr(A_hi), _ptr(A_lo), max(k, 1),
                                _ptr(B_hi), _ptr(B_lo), max(n, 1),
                                _ptr(C_hi), _ptr(C_lo), max(n, 1), int(nthreads))
    if used < 0:
        raise ValueError("oracle_dd_gemm rejected its arguments")
    return C_hi, C_lo, used


def dd_gemm_entries(A_hi, A_lo, B_hi, B_lo, rows, cols, nthreads: int = 0):
    """Selected entries C[rows[q], cols[q]] (same arithmetic as dd_gemm)."""
    A_hi, A_lo, B_hi, B_lo = map(_c64, (A_hi, A_lo, B_hi, B_lo))
    m, k = A_hi.shape
    n = B_hi.shape[1]
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    assert rows.shape == cols.shape
    out_hi = np.zeros(rows.shape)
    out_lo = np.zeros(rows.shape)
    p64 = ctypes.POINTER(_i64)
    used = lib().oracle_dd_gemm_entries(rows.size, rows.ctypes.data_as(p64), cols.ctypes.data_as(p64),
                                        m, n, k, _ptr(A_hi), _ptr(A_lo), max(k, 1),
                                        _ptr(B_hi), _ptr(B_lo), max(n, 1),
                                        _ptr(out_hi), _ptr(out_lo), int(nthreads))
    if used < 0:
        raise ValueError("oracle_dd_gemm_entries rejected its arguments")
    return out_hi, out_lo


def _pair(fn, *args):
    a, b = ctypes.c_double(), ctypes.c_double()
    fn(*args, ctypes.byref(a), ctypes.byref(b))
    return a.value, b.value


def two_sum(a, b):
    return _pair(lib().oracle_two_sum, a, b)


def two_prod(a, b):
    return _pair(lib().oracle_two_prod, a, b)


def dd_mul(xh, xl, yh, yl):
    return _pair(lib().oracle_dd_mul, xh, xl, yh, yl)


def dd_add(xh, xl, yh, yl):
    return _pair(lib().oracle_dd_add, xh, xl, yh, yl)


def max_threads() -> int:
    return lib().oracle_max_threads()
