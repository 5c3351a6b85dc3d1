"""Seeded random combinations of the path's parameters (GPU tests).

Each case draws a ragged shape spanning up to a few tiles, a slice count, a
k-block size (or none), which lo planes are present and the entry
distributions; the product is compared bit for bit with the oracle's chain for
the same inputs (oracle.exact.paired_product / sliced_product_kblocks with the
nearest double-double per block for double doubles, oracle.qd.sliced_product
for quad doubles).  The grid tests
elsewhere cover each parameter on its own; these cover their combinations,
with a set of small outputs and long k that take the split-over-k path with
varying part counts.
"""
import sys

import numpy as np
import pytest

import workloads
from oracle import exact, qd

pytestmark = pytest.mark.gpu

DISTS = ["uniform", "normal", "signed_exp20", "signed_exp30"]


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def _host(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _bits_equal(a, b):
    a = np.ascontiguousarray(a, dtype=np.float64)
    b = np.ascontiguousarray(b, dtype=np.float64)
    return a.shape == b.shape and np.array_equal(a.view(np.int64), b.view(np.int64))


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _dd_cases(count, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        m, n, k = (int(x) for x in rng.integers(1, [150, 150, 300]))
        ns = int(rng.integers(4, 17))
        kb = None if rng.random() < 0.4 else int(rng.integers(1, k + 10))
        lo_a, lo_b = bool(rng.random() < 0.75), bool(rng.random() < 0.75)
        da, db = (DISTS[int(x)] for x in rng.integers(0, len(DISTS), 2))
        out.append((i, m, n, k, ns, kb, lo_a, lo_b, da, db))
    return out


def _dd_split_cases(count, seed):
    """Small outputs with k long enough to split over k (parts vary with the
    shape, the slice count and the k-block)."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        m, n = (int(x) for x in rng.integers(1, 70, 2))
        k = int(rng.integers(241, 2000))
        ns = int(rng.integers(4, 17))
        kb = None if rng.random() < 0.6 else int(rng.integers(241, k + 10))
        lo_a, lo_b = bool(rng.random() < 0.8), bool(rng.random() < 0.8)
        da, db = (DISTS[int(x)] for x in rng.integers(0, len(DISTS), 2))
        out.append((i, m, n, k, ns, kb, lo_a, lo_b, da, db))
    return out


def _qd_cases(count, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        m, n, k = (int(x) for x in rng.integers(1, [90, 90, 150]))
        kb = None if rng.random() < 0.4 else int(rng.integers(1, k + 10))
        planes_a, planes_b = (int(x) for x in rng.integers(1, 5, 2))  # components given
        da, db = (DISTS[int(x)] for x in rng.integers(0, len(DISTS), 2))
        out.append((i, m, n, k, kb, planes_a, planes_b, da, db))
    return out


def _qd_split_cases(count, seed):
    """Quad-double products small enough in m, n and long enough in k to split."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        m, n = (int(x) for x in rng.integers(1, 60, 2))
        k = int(rng.integers(241, 1200))
        kb = None if rng.random() < 0.6 else int(rng.integers(241, k + 10))
        planes_a, planes_b = (int(x) for x in rng.integers(1, 5, 2))
        da, db = (DISTS[int(x)] for x in rng.integers(0, len(DISTS), 2))
        out.append((100 + i, m, n, k, kb, planes_a, planes_b, da, db))
    return out


@pytest.mark.parametrize("case", _dd_cases(40, 20261202), ids=lambda c: f"dd{c[0]}")
def test_random_dd_case_bit_exact(gpu, case):
    i, m, n, k, ns, kb, lo_a, lo_b, da, db = case
    _say(f"[random dd {i}] m={m} n={n} k={k} nslices={ns} kblock={kb} lo=({lo_a},{lo_b}) dist=({da},{db})")
    Ah, Al = workloads.random_dd((m, k), 7000 + 2 * i, da)
    Bh, Bl = workloads.random_dd((k, n), 7001 + 2 * i, db)
    if not lo_a:
        Al = np.zeros_like(Ah)
    if not lo_b:
        Bl = np.zeros_like(Bh)
    Ch, Cl = gpu.dd_gemm(_dev(Ah), _dev(Al) if lo_a else None, _dev(Bh), _dev(Bl) if lo_b else None,
                         nslices=ns, kblock=kb)
    if kb is None or kb >= k:
        Rh, Rl = exact.paired_product(Ah, Al, Bh, Bl, ns)
    else:
        Rh, Rl = exact.sliced_product_kblocks(Ah, Al, Bh, Bl, kb, ns, nearest=True)
    assert _bits_equal(_host(Ch), Rh) and _bits_equal(_host(Cl), Rl)


@pytest.mark.parametrize("case", _dd_split_cases(30, 20261204), ids=lambda c: f"ddsplit{c[0]}")
def test_random_split_dd_case_bit_exact(gpu, case):
    i, m, n, k, ns, kb, lo_a, lo_b, da, db = case
    parts = gpu.split_parts(m, n, k if kb is None else min(k, kb), ns)
    _say(f"[random split dd {i}] m={m} n={n} k={k} nslices={ns} kblock={kb} parts={parts}")
    Ah, Al = workloads.random_dd((m, k), 7500 + 2 * i, da)
    Bh, Bl = workloads.random_dd((k, n), 7501 + 2 * i, db)
    if not lo_a:
        Al = np.zeros_like(Ah)
    if not lo_b:
        Bl = np.zeros_like(Bh)
    Ch, Cl = gpu.dd_gemm(_dev(Ah), _dev(Al) if lo_a else None, _dev(Bh), _dev(Bl) if lo_b else None,
                         nslices=ns, kblock=kb)
    if kb is None or kb >= k:
        Rh, Rl = exact.paired_product(Ah, Al, Bh, Bl, ns)
    else:
        Rh, Rl = exact.sliced_product_kblocks(Ah, Al, Bh, Bl, kb, ns, nearest=True)
    assert _bits_equal(_host(Ch), Rh) and _bits_equal(_host(Cl), Rl)


@pytest.mark.parametrize("case", _qd_cases(15, 20261203) + _qd_split_cases(10, 20261205),
                         ids=lambda c: f"qd{c[0]}")
def test_random_qd_case_bit_exact(gpu, case):
    i, m, n, k, kb, planes_a, planes_b, da, db = case
    _say(f"[random qd {i}] m={m} n={n} k={k} kblock={kb} planes=({planes_a},{planes_b}) dist=({da},{db})")
    A = workloads.random_qd((m, k), 8000 + 2 * i, da)
    B = workloads.random_qd((k, n), 8001 + 2 * i, db)
    A[planes_a:] = 0.0
    B[planes_b:] = 0.0
    dA, dB = _dev(A), _dev(B)
    C = gpu.qd_gemm([dA[c] if c < planes_a else None for c in range(4)],
                    [dB[c] if c < planes_b else None for c in range(4)], kblock=kb)
    _, _, _, C_ref = qd.sliced_product(A, B)
    assert _bits_equal(_host(C), C_ref)
