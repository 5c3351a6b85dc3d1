"""Operands whose packed slices pass 2^31 values (GPU tests).

A tall double-double A (65536 x 8192), a wide double-double B (8192 x 65536)
and a tall quad-double A (36864 x 4096): each packed slice buffer holds more
than 2^31 doubles, so a 32-bit index anywhere on the path (slicer, GEMM stage
copies, epilogue) would read or write the wrong place.  The large operand is a
seeded block repeated along its long side on the device, which keeps input
generation cheap; outputs of the last repeat must equal those of the first,
and sampled outputs there are compared bit for bit with the oracle's chain on
the same rows and columns of the seeded block.  A last test takes k to the
exact-sum bound with the largest digits, where the level sums are largest.
"""
import sys

import numpy as np
import pytest

import workloads
from oracle import exact, qd

pytestmark = pytest.mark.gpu


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


def _free():
    import torch
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _dd_chain(ah, al, bh, bl, rows, cols):
    """The product entry points' chain on a block: nearest double-double of the exact level totals."""
    E, DA = exact.slice_rows(ah, al, rows)
    F, DB = exact.slice_cols(bh, bl, cols)
    return exact.nearest_dd(exact.level_sums_units(DA, DB), E, F)


@pytest.mark.timeout(600)
def test_dd_tall_A_past_2_31_slice_values(gpu):
    base, reps, k, n = 1024, 64, 8192, 64
    m = base * reps
    assert gpu.slices_bytes(m, k) // 8 > 2 ** 31
    _say(f"[large] dd tall A {m}x{k} (block of {base} rows x {reps}), n={n}")
    ah, al = workloads.random_dd((base, k), 5151, "signed_exp20")
    bh, bl = workloads.random_dd((k, n), 5152, "normal")
    dAh, dAl = _dev(ah).repeat(reps, 1), _dev(al).repeat(reps, 1)
    Ch, Cl = gpu.dd_gemm(dAh, dAl, _dev(bh), _dev(bl))
    del dAh, dAl
    hCh, hCl = _host(Ch), _host(Cl)
    del Ch, Cl
    _free()
    assert _bits_equal(hCh[-base:], hCh[:base]) and _bits_equal(hCl[-base:], hCl[:base])
    rows, cols = [0, 517, base - 1], [0, 31, n - 1]
    Rh, Rl = _dd_chain(ah, al, bh, bl, rows, cols)
    last = [(reps - 1) * base + r for r in rows]
    assert _bits_equal(hCh[np.ix_(last, cols)], Rh) and _bits_equal(hCl[np.ix_(last, cols)], Rl)


@pytest.mark.timeout(600)
def test_dd_wide_B_past_2_31_slice_values(gpu):
    base, reps, k, m = 1024, 64, 8192, 64
    n = base * reps
    assert gpu.slices_bytes(n, k) // 8 > 2 ** 31
    _say(f"[large] dd wide B {k}x{n} (block of {base} columns x {reps}), m={m}")
    ah, al = workloads.random_dd((m, k), 5161, "uniform")
    bh, bl = workloads.random_dd((k, base), 5162, "signed_exp20")
    dBh, dBl = _dev(bh).repeat(1, reps), _dev(bl).repeat(1, reps)
    Ch, Cl = gpu.dd_gemm(_dev(ah), _dev(al), dBh, dBl)
    del dBh, dBl
    hCh, hCl = _host(Ch), _host(Cl)
    del Ch, Cl
    _free()
    assert _bits_equal(hCh[:, -base:], hCh[:, :base]) and _bits_equal(hCl[:, -base:], hCl[:, :base])
    rows, cols = [0, 40, m - 1], [0, 700, base - 1]
    Rh, Rl = _dd_chain(ah, al, bh, bl, rows, cols)
    last = [(reps - 1) * base + c for c in cols]
    assert _bits_equal(hCh[np.ix_(rows, last)], Rh) and _bits_equal(hCl[np.ix_(rows, last)], Rl)


@pytest.mark.timeout(600)
def test_qd_tall_A_past_2_31_slice_values(gpu):
    base, reps, k, n = 512, 72, 4096, 64
    m = base * reps
    assert gpu.qd_slices_bytes(m, k) // 8 > 2 ** 31
    _say(f"[large] qd tall A {m}x{k} (block of {base} rows x {reps}), n={n}")
    A = workloads.random_qd((base, k), 5171, "signed_exp20")
    B = workloads.random_qd((k, n), 5172, "uniform")
    dA = _dev(A).repeat(1, reps, 1)
    C = gpu.qd_gemm(dA, _dev(B))
    del dA
    hC = _host(C)
    del C
    _free()
    assert _bits_equal(hC[:, -base:], hC[:, :base])
    rows, cols = [0, 300, base - 1], [0, n - 1]
    E, DA = qd.slice_rows(A, rows=rows)
    F, DB = qd.slice_cols(B, cols=cols)
    ref = qd.renorm_levels(qd.level_sums(DA, DB), E, F)
    last = [(reps - 1) * base + r for r in rows]
    assert _bits_equal(hC[:, last][:, :, cols], ref)


# The largest window integer an entry can have: RN(hi + lo) < 2^E forces
# |x| < 2^E (1 - 2^-54), so N <= 2^104 - 2^50 - 1 (E = 0 for this entry).
MAX_HI, MAX_LO = 1.0 - 2.0 ** -53, 2.0 ** -54 - 2.0 ** -104


@pytest.mark.timeout(600)
def test_dd_level_sums_exact_at_the_k_bound(gpu):
    """k at the exact-sum bound (2^23, "Multiple Double Arithmetic on NVIDIA
    Tensor Cores", §2 eq. (5)) with the largest digits in every slice of every
    entry: level 7 reaches k * 503189512 ~ 2^51.9 units, inside the 53 exact
    bits, and A's packed slices hold 2^33 doubles (68.7 GB), so a 32-bit
    offset anywhere would fail.  The level-plane stage call (split over
    k into atomically added parts) must give the closed-form level sums
    exactly, and the unsplit fused call (one workgroup) the oracle's cascade of
    them, bit for bit."""
    import torch
    m, n, k = 100, 2, gpu.K_MAX
    assert gpu.split_parts(m, n, k) > 1
    assert gpu.slices_bytes(m, k) // 8 == 2 ** 33
    digits = exact.slice_entry(MAX_HI, MAX_LO, 0)
    assert digits == [8191, 8191, 8191, 8191, 6143, 8191, 8191, 8191]
    units = [-k * sum(digits[s] * digits[l - s] for s in range(l + 1)) for l in range(8)]
    assert max(abs(u) for u in units) < 2 ** 53 and abs(units[7]) > 2 ** 51
    S_units = np.array([np.full((m, n), u, dtype=np.int64) for u in units])
    S_ref = exact.level_values(S_units)
    Rh, Rl = exact.renorm_levels(S_ref, np.zeros(m, np.int64), np.zeros(n, np.int64))
    _free()
    _say(f"[large] dd k = {k} at the exact-sum bound, m={m} n={n}, largest digits")
    A_hi = torch.full((m, k), MAX_HI, dtype=torch.float64, device="cuda")
    A_lo = torch.full((m, k), MAX_LO, dtype=torch.float64, device="cuda")
    E, As = gpu.split_balanced(A_hi, A_lo, 0)
    del A_hi, A_lo
    B_hi = torch.full((k, n), -MAX_HI, dtype=torch.float64, device="cuda")
    B_lo = torch.full((k, n), -MAX_LO, dtype=torch.float64, device="cuda")
    F, Bs = gpu.split_balanced(B_hi, B_lo, 1)
    del B_hi, B_lo
    assert _host(E).tolist() == [0] * m and _host(F).tolist() == [0] * n
    _say("[large] split stage call")
    levels = _host(gpu.sliced_gemm(m, n, k, As, Bs))
    assert _bits_equal(levels, S_ref)
    _say("[large] unsplit fused call")
    Fh, Fl = gpu.sliced_gemm_renorm(m, n, k, As, E, Bs, F)
    assert _bits_equal(_host(Fh), Rh) and _bits_equal(_host(Fl), Rl)
    del As, Bs
    _free()


@pytest.mark.timeout(600)
def test_dd_pair_group_sums_exact_at_the_product_k_bound(gpu):
    """k at the product's k-block limit (2^22 for 8 slices: the most values of k
    whose int64 group sums of the pair-packed schedule stay below 2^63) with
    the largest digits in every slice of every entry: the deepest group reaches
    ~2^62.9 units after 1024 chunks of exact FP64 sums.  The group-sum stage
    call (one workgroup, every chunk) gives the closed form exactly, and the
    product (split over k into parts) the oracle's nearest double-double of it."""
    import torch
    m, n, k = 64, 3, gpu.kblock_max(8)
    assert k == 1 << 22 and gpu.split_parts(m, n, k) > 1
    digits = exact.slice_entry(MAX_HI, MAX_LO, 0)
    DA = np.array(digits, dtype=np.int64).reshape(8, 1, 1)
    DB = -DA.reshape(8, 1, 1)
    G1 = exact.paired_group_units(DA, DB)[:, 0, 0]                 # one value of k
    G = [int(g) * k for g in G1]
    assert max(abs(g) for g in G) < 2 ** 63 and abs(G[6]) > 2 ** 62
    S_units = np.array([np.full((m, n), -k * sum(digits[s] * digits[l - s] for s in range(l + 1)), dtype=np.int64)
                        for l in range(8)])
    Rh, Rl = exact.nearest_dd(S_units[:, :1, :1], [0], [0])
    _free()
    _say(f"[large] pair group sums at k = {k}, m={m} n={n}, largest digits")
    A_hi = torch.full((m, k), MAX_HI, dtype=torch.float64, device="cuda")
    A_lo = torch.full((m, k), MAX_LO, dtype=torch.float64, device="cuda")
    B_hi = torch.full((k, n), -MAX_HI, dtype=torch.float64, device="cuda")
    B_lo = torch.full((k, n), -MAX_LO, dtype=torch.float64, device="cuda")
    _say("[large] product (split over k)")
    Ch, Cl = gpu.dd_gemm(A_hi, A_lo, B_hi, B_lo)
    assert (_host(Ch) == Rh[0, 0]).all() and (_host(Cl) == Rl[0, 0]).all()
    del Ch, Cl
    E, As = gpu.split_balanced(A_hi, A_lo, 0)
    del A_hi, A_lo
    F, Bs = gpu.split_balanced(B_hi, B_lo, 1)
    del B_hi, B_lo
    _say("[large] group-sum stage call (one workgroup, 1024 chunks)")
    units = _host(gpu.sliced_gemm_pairs(m, n, k, As, Bs))
    for g in range(7):
        assert (units[g] == G[g]).all(), g
    del As, Bs
    _free()


# A normalised quad double just below 1 whose every component is the largest the
# one above it allows: window digits 8191 except 6143, 7679 and 8063 (E = 0).
QD_MAX = [1.0 - 2.0 ** -53, 2.0 ** -54 - 2.0 ** -107, 2.0 ** -108 - 2.0 ** -161, 2.0 ** -162 - 2.0 ** -215]


@pytest.mark.timeout(600)
def test_qd_level_sums_exact_at_the_k_bound(gpu):
    """The quad-double product at its exact-sum bound (k = 2^22; sixteen pairs on
    the deepest levels, "Multiple Double Arithmetic on NVIDIA Tensor Cores", §2
    eq. (5)) with near-largest digits everywhere: the deeper levels reach 2^52
    units.  The unsplit fused call (one workgroup) and the product entry point
    (split over k into atomically added parts) must both give the oracle's
    exact four-double rounding of the closed-form level sums, bit for bit."""
    import torch
    m, n, k = 3, 2, gpu.QD_K_MAX
    assert gpu.split_parts(m, n, k, 16) > 1
    assert qd.is_normalized(QD_MAX) and qd.entry_exponent(QD_MAX) == 0
    digits = qd.slice_entry(QD_MAX, 0)
    units = [-k * sum(digits[s] * digits[l - s] for s in range(l + 1)) for l in range(16)]
    assert max(abs(u) for u in units) < 2 ** 53 and abs(units[15]) > 2 ** 51
    S_units = np.array([np.full((m, n), u, dtype=np.int64) for u in units])
    ref = qd.renorm_levels(S_units, np.zeros(m, np.int64), np.zeros(n, np.int64))
    _free()
    _say(f"[large] qd k = {k} at the exact-sum bound, m={m} n={n}, near-largest digits")
    A = torch.empty((4, m, k), dtype=torch.float64, device="cuda")
    B = torch.empty((4, k, n), dtype=torch.float64, device="cuda")
    for c in range(4):
        A[c].fill_(QD_MAX[c])
        B[c].fill_(-QD_MAX[c])
    E, As = gpu.qd_split_balanced(A, 0)
    F, Bs = gpu.qd_split_balanced(B, 1)
    assert _host(E).tolist() == [0] * m and _host(F).tolist() == [0] * n
    _say("[large] unsplit fused call")
    assert _bits_equal(_host(gpu.qd_sliced_gemm_renorm(m, n, k, As, E, Bs, F)), ref)
    del As, Bs
    _free()
    _say("[large] product entry point, split over k")
    assert _bits_equal(_host(gpu.qd_gemm(A, B)), ref)
    del A, B
    _free()
