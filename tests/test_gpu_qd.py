"""Parity of the quad-double HIP path with the CPU oracle (GPU tests; C ABI).

Bars:
* exponents, every one of the sixteen slices, and the whole chain (slices ->
  level sums -> exact total -> nearest four-double result) are bit-exact
  against oracle/qd.py, on small shapes spanning several tiles with ragged
  edges, on edge-case entries, and on sampled outputs of the full workloads in
  the configuration the bench times;
* the product is within oracle/qd.py's error bound of the exact product
  (Python integers), all entries at 64^3 and sampled entries at full size.
Every expected value comes from oracle/ on the same seeded inputs.
"""
import sys
from fractions import Fraction

import numpy as np
import pytest

import workloads
from oracle import exact, qd

pytestmark = pytest.mark.gpu


def _dev(a):
    import torch
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


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


def _unpack(packed, outer, k, nslices=16):
    from extended_precision_gemm_amd import layout
    return _host(layout.unpack(packed, outer, k, nslices).contiguous())


# Entries whose rounding decides the exponent, or whose lower components reach
# far below the window with either sign (all normalised quad doubles).
_SPECIAL = [
    (1.0, -(2.0 ** -54), 0.0, 0.0),                    # RN = 1 (tie to even)
    (1.0, -(2.0 ** -53), 0.0, 0.0),                    # 1 - 2^-53 exactly
    (1.0, -(2.0 ** -54), -(2.0 ** -110), 0.0),         # just below the tie
    (2.0 - 2.0 ** -52, 2.0 ** -53, 0.0, 0.0),          # tie rounds up to 2
    (2.0 - 2.0 ** -52, 2.0 ** -53, -(2.0 ** -120), 0.0),
    (-(2.0 - 2.0 ** -52), -(2.0 ** -53), 0.0, 0.0),
    (1.0, 2.0 ** -60, -(2.0 ** -300), 0.0),            # negative tail far below: floor borrows
    (-1.0, -(2.0 ** -60), 2.0 ** -300, 0.0),
    (0.75, 2.0 ** -56, -(2.0 ** -112), 2.0 ** -170),
    (5e-324, 0.0, 0.0, 0.0),
    (3 * 5e-324, 0.0, 0.0, 0.0),
    (2.0 ** -1022, 0.0, 0.0, 0.0),
    (2.0 ** 900 * 1.25, 2.0 ** 840, -(2.0 ** 780), 2.0 ** 700),
    (0.0, 0.0, 0.0, 0.0),
]


def _edge_matrix(rows, cols, seed):
    """Random normalised quad doubles with the special entries planted, a zero row."""
    X = workloads.random_qd((rows, cols), seed, "signed_exp30")
    rng = np.random.default_rng(seed)
    for q, e in enumerate(_SPECIAL):
        i, j = int(rng.integers(rows)), int(rng.integers(cols))
        X[:, i, j] = e
        if q % 3 == 0 and rows > 4:
            X[:, (i + 1) % rows, :] *= 2.0 ** -200  # a row far below its neighbours
    if rows > 2:
        X[:, rows // 2, :] = 0.0
    for i in range(rows):
        for j in range(cols):
            assert qd.is_normalized(X[:, i, j])
    return X


def _oracle_slice_values(D):
    return exact.slice_values(D)


# ---------------------------------------------------------------------------
# slicing
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("rows,cols", [(1, 1), (17, 5), (40, 33), (130, 21), (5, 140)])
@pytest.mark.parametrize("axis", [0, 1])
def test_qd_split_bit_exact(gpu, rows, cols, axis):
    _say(f"[qd split] {rows}x{cols} axis={axis}")
    X = _edge_matrix(rows, cols, 100 + rows + cols + axis)
    E, packed = gpu.qd_split_balanced(_dev(X), axis)
    if axis == 0:
        E_ref, D = qd.slice_rows(X)
        outer, k = rows, cols
    else:
        E_ref, D = qd.slice_cols(X)
        D = D.transpose(0, 2, 1)
        outer, k = cols, rows
    assert np.array_equal(_host(E), E_ref)
    assert _bits_equal(_unpack(packed, outer, k), _oracle_slice_values(D))


def test_qd_split_large_B_two_pass_bit_exact(gpu):
    """A quad-double B above the one-pass size (32 MiB) takes the two-pass split
    (column-block exponents, then slices): ragged column blocks, special
    entries, a column decided by its last row."""
    rows, cols = 1100, 1100
    assert rows * cols * 32 > 32 << 20
    X = workloads.random_qd((rows, cols), 4321, "signed_exp30")
    X[:, :, 17] *= 2.0 ** 300
    rng = np.random.default_rng(4321)
    for e in _SPECIAL:
        X[:, int(rng.integers(rows)), int(rng.integers(cols))] = e
    X[:, :, 1050] = 0.0
    X[:, rows - 1, 1050] = (2.0 ** -700, 2.0 ** -760, 0.0, 0.0)
    E, packed = gpu.qd_split_balanced(_dev(X), 1)
    assert np.array_equal(_host(E), qd.balancing_exponents(X, 1))
    cols_s = [0, 17, 1023, 1024, 1050, cols - 1]
    E_s, D = qd.slice_cols(X, cols=cols_s)
    got = _unpack(packed, cols, rows)
    assert _bits_equal(got[:, cols_s, :], _oracle_slice_values(D.transpose(0, 2, 1)))


def test_qd_split_null_components_and_stride(gpu):
    import torch
    X = workloads.random_qd((37, 29), 7, "uniform")
    X[2:] = 0.0
    big = torch.zeros((2, 37, 40), dtype=torch.float64, device="cuda")
    big[0, :, :29] = _dev(X[0])
    big[1, :, :29] = _dev(X[1])
    E, packed = gpu.qd_split_balanced([big[0, :, :29], big[1, :, :29], None, None], 0)
    E_ref, D = qd.slice_rows(X)
    assert np.array_equal(_host(E), E_ref)
    assert _bits_equal(_unpack(packed, 37, 29), _oracle_slice_values(D))


def test_qd_split_of_double_double_matches_dd_slicer(gpu):
    """Top eight of the sixteen slices of (hi, lo, 0, 0) are the double-double slices."""
    hi, lo = workloads.random_dd((70, 45), 12, "signed_exp30")
    for axis in (0, 1):
        Eq, pq = gpu.qd_split_balanced([_dev(hi), _dev(lo)], axis)
        Ed, pd = gpu.split_balanced(_dev(hi), _dev(lo), axis)
        outer, k = (70, 45) if axis == 0 else (45, 70)
        assert np.array_equal(_host(Eq), _host(Ed))
        assert _bits_equal(_unpack(pq, outer, k)[:8], _unpack(pd, outer, k, 8))


# ---------------------------------------------------------------------------
# the chain
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("m,n,k", [(1, 1, 1), (64, 64, 64), (100, 70, 33), (33, 130, 17), (130, 65, 200)])
def test_qd_chain_bit_exact(gpu, m, n, k):
    _say(f"[qd chain] {m}x{n}x{k}")
    A = workloads.random_qd((m, k), 200 + m, "uniform")
    B = workloads.random_qd((k, n), 300 + n, "signed_exp20")
    C = gpu.qd_gemm(_dev(A), _dev(B))
    _, _, _, C_ref = qd.sliced_product(A, B)
    assert _bits_equal(_host(C), C_ref)


def test_qd_chain_edge_entries_bit_exact(gpu):
    A = _edge_matrix(40, 36, 401)
    B = _edge_matrix(36, 23, 402)
    # keep the products finite: scale the huge planted entries down
    A[:, np.abs(A[0]) > 2.0 ** 500] *= 2.0 ** -800
    B[:, np.abs(B[0]) > 2.0 ** 500] *= 2.0 ** -800
    C = gpu.qd_gemm(_dev(A), _dev(B))
    _, _, _, C_ref = qd.sliced_product(A, B)
    assert _bits_equal(_host(C), C_ref)


def test_qd_subnormal_and_zero_outputs_bit_exact(gpu):
    A = workloads.random_qd((20, 30), 501, "uniform") * 2.0 ** -560
    B = workloads.random_qd((30, 25), 502, "uniform") * 2.0 ** -520
    A[:, 3, :] = 0.0
    B[:, :, 4] = 0.0
    C = gpu.qd_gemm(_dev(A), _dev(B))
    _, _, _, C_ref = qd.sliced_product(A, B)
    got = _host(C)
    assert _bits_equal(got, C_ref)
    assert (np.abs(got[0]) < 2.0 ** -1022).any()          # subnormal results occur


def test_qd_results_beyond_the_double_range_overflow_like_ldexp(gpu):
    """Quad-double products near 2^1200 round to infinities of the right sign,
    with finite rows alongside, bit for bit as in the oracle's chain."""
    rng = np.random.default_rng(78)
    m, n, k = 12, 10, 16
    A = np.zeros((4, m, k))
    B = np.zeros((4, k, n))
    A[0] = rng.integers(-9, 10, (m, k)) * 2.0 ** 600
    A[1] = A[0] * 2.0 ** -60 * rng.choice([-1.0, 1.0], (m, k))   # normalised: below half an ulp of A[0]
    B[0] = rng.integers(-9, 10, (k, n)) * 2.0 ** 600
    A[:, :4] *= 2.0 ** -700
    assert all(qd.is_normalized(A[:, i, p]) for i in range(m) for p in range(k))
    C = _host(gpu.qd_gemm(_dev(A), _dev(B)))
    _, _, _, C_ref = qd.sliced_product(A, B)
    assert _bits_equal(C, C_ref)
    over = np.isinf(C[0])
    assert over[4:].any() and np.isfinite(C[:, :4]).all()
    assert (C[1][over] != 0).any()          # a finite second word after an infinite first


def test_qd_identity_returns_truncated_operand(gpu):
    B = workloads.random_qd((48, 37), 601, "signed_exp20")
    A = np.zeros((4, 48, 48))
    A[0] = np.eye(48)
    C = _host(gpu.qd_gemm(_dev(A), _dev(B)))
    _, _, _, C_ref = qd.sliced_product(A, B)
    assert _bits_equal(C, C_ref)


def test_qd_entry_points_agree(gpu):
    import torch
    m, n, k = 90, 77, 51
    A = workloads.random_qd((m, k), 701, "normal")
    B = workloads.random_qd((k, n), 702, "uniform")
    dA, dB = _dev(A), _dev(B)
    C1 = _host(gpu.qd_gemm(dA, dB))
    C2 = _host(gpu.qd_gemm_alloc(dA, dB))
    E, As = gpu.qd_split_balanced(dA, 0)
    F, Bs = gpu.qd_split_balanced(dB, 1)
    C3 = _host(gpu.qd_sliced_gemm_renorm(m, n, k, As, E, Bs, F))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        C4 = gpu.qd_gemm(dA, dB, stream=s)
    s.synchronize()
    # strided output planes
    out = torch.full((4, m, n + 9), 7.0, dtype=torch.float64, device="cuda")
    gpu.qd_gemm(dA, dB, C=[out[c, :, :n] for c in range(4)])
    C5 = _host(out[:, :, :n].contiguous())
    assert (_host(out[:, :, n:]) == 7.0).all()
    for Cx in (C2, C3, _host(C4), C5):
        assert _bits_equal(Cx, C1)


def test_qd_k_zero_and_empty(gpu):
    import torch
    A = torch.zeros((4, 5, 0), dtype=torch.float64, device="cuda")
    B = torch.zeros((4, 0, 6), dtype=torch.float64, device="cuda")
    C = torch.full((4, 5, 6), 3.0, dtype=torch.float64, device="cuda")
    gpu.qd_gemm(A, B, C=C)
    assert _bits_equal(_host(C), np.zeros((4, 5, 6)))
    E = gpu.qd_gemm(torch.zeros((4, 0, 3), dtype=torch.float64, device="cuda"),
                    torch.zeros((4, 3, 4), dtype=torch.float64, device="cuda"))
    assert tuple(E.shape) == (4, 0, 4)


# ---------------------------------------------------------------------------
# k-blocks: every block sliced below the exponents of the whole k, level sums
# added exactly in int64, one rounding -- the unblocked result, bit for bit
# ---------------------------------------------------------------------------
def _two_scale_operands(m, n, k, seed):
    """Operands whose second half of k is far smaller, so a block's own
    exponents would differ from those of the whole row / column."""
    A = workloads.random_qd((m, k), seed, "uniform")
    B = workloads.random_qd((k, n), seed + 1, "signed_exp20")
    A[:, :, k // 2:] *= 2.0 ** -60
    B[:, k // 2:, :] *= 2.0 ** -40
    return A, B


def _local_exponent_blocks(A, B, kblock):
    """Oracle only: the result if each k-block were sliced below its own
    exponents and the blocks' exact totals added (the design not taken)."""
    m, k, n = A.shape[1], A.shape[2], B.shape[2]
    unit = 2 ** (-13 * (qd.QD_SLICES + 1))
    total = [[Fraction(0)] * n for _ in range(m)]
    for p0 in range(0, k, kblock):
        E, F, S, _ = qd.sliced_product(A[:, :, p0:p0 + kblock], B[:, p0:p0 + kblock, :])
        for i in range(m):
            for j in range(n):
                total[i][j] += qd.level_total(S, i, j) * Fraction(2) ** int(E[i] + F[j]) * Fraction(unit)
    out = np.zeros((4, m, n))
    for i in range(m):
        for j in range(n):
            out[:, i, j] = qd.greedy_qd(total[i][j])
    return out


@pytest.mark.parametrize("m,n,k,kblock", [(100, 70, 130, 33), (33, 130, 200, 64), (64, 64, 64, 1),
                                          (40, 50, 97, 96), (17, 18, 45, 45), (130, 65, 200, 7)])
def test_qd_kblocked_chain_equals_unblocked_oracle(gpu, m, n, k, kblock):
    _say(f"[qd k-blocks] {m}x{n}x{k} kblock={kblock}")
    A, B = _two_scale_operands(m, n, k, 1000 + k + kblock)
    C = _host(gpu.qd_gemm(_dev(A), _dev(B), kblock=kblock))
    _, _, _, C_ref = qd.sliced_product(A, B)
    assert _bits_equal(C, C_ref)


def test_qd_kblocked_inputs_distinguish_local_exponents(gpu):
    """The operands above make block-local exponents give another result, so
    the bit-exact comparison checks that the whole k's exponents are used."""
    m, n, k, kblock = 12, 10, 40, 16
    A, B = _two_scale_operands(m, n, k, 77)
    _, _, _, C_ref = qd.sliced_product(A, B)
    assert not _bits_equal(_local_exponent_blocks(A, B, kblock), C_ref)
    assert _bits_equal(_host(gpu.qd_gemm(_dev(A), _dev(B), kblock=kblock)), C_ref)


def test_qd_kblocked_strided_and_null_planes(gpu):
    import torch
    m, n, k = 50, 41, 90
    A, B = _two_scale_operands(m, n, k, 88)
    A[2:] = 0.0                                       # double-double A: two planes given
    bigA = torch.zeros((2, m, k + 5), dtype=torch.float64, device="cuda")
    bigA[:, :, :k] = _dev(A[:2])
    bigB = torch.zeros((4, k, n + 3), dtype=torch.float64, device="cuda")
    bigB[:, :, :n] = _dev(B)
    out = torch.full((4, m, n + 2), 5.0, dtype=torch.float64, device="cuda")
    gpu.qd_gemm([bigA[0, :, :k], bigA[1, :, :k], None, None], [bigB[c, :, :n] for c in range(4)],
                C=[out[c, :, :n] for c in range(4)], kblock=25)
    _, _, _, C_ref = qd.sliced_product(A, B)
    assert _bits_equal(_host(out[:, :, :n].contiguous()), C_ref)
    assert (_host(out[:, :, n:]) == 5.0).all()


def test_qd_kblocked_workload_matches_unblocked(gpu):
    """qd1024 in blocks of 256 (four blocks: first, two middle, last) equals the
    one-block product everywhere and the oracle on sampled entries."""
    import torch
    w = workloads.by_name("qd1024")
    A, B = workloads.make_qd_operands(w)
    dA, dB = _dev(A), _dev(B)
    C1 = gpu.qd_gemm(dA, dB)
    C4 = gpu.qd_gemm(dA, dB, kblock=256)
    assert torch.equal(C1.view(torch.int64), C4.view(torch.int64))
    rng = np.random.default_rng(31)
    for i, j in zip(rng.integers(0, w.m, 6), rng.integers(0, w.n, 6)):
        _, _, ref = _oracle_entry(A, B, int(i), int(j))
        assert _bits_equal(_host(C4[:, int(i), int(j)]), ref)


# ---------------------------------------------------------------------------
# workloads: accuracy against the exact product, bit-exact sampled outputs
# ---------------------------------------------------------------------------
def _oracle_entry(A, B, i, j):
    """The oracle's chain for one output entry: its row of A, its column of B."""
    E, DA = qd.slice_rows(A, rows=[i])
    F, DB = qd.slice_cols(B, cols=[j])
    S = qd.level_sums(DA, DB)
    return int(E[0]), int(F[0]), qd.renorm_levels(S, E, F)[:, 0, 0]


@pytest.mark.parametrize("name,samples", [("qd64", None), ("qd1024", 24), ("qd2048", 12), ("qd4096_exp20", 6)])
def test_qd_workload_parity(gpu, name, samples):
    w = workloads.by_name(name)
    _say(f"[qd workload] {name} m={w.m} n={w.n} k={w.k}")
    A, B = workloads.make_qd_operands(w)
    dA, dB = _dev(A), _dev(B)
    E, As = gpu.qd_split_balanced(dA, 0)
    F, Bs = gpu.qd_split_balanced(dB, 1)
    C = gpu.qd_sliced_gemm_renorm(w.m, w.n, w.k, As, E, Bs, F)
    Eh, Fh = _host(E), _host(F)
    del As, Bs
    if samples is None:
        rows = [i for i in range(w.m) for _ in range(w.n)]
        cols = [j for _ in range(w.m) for j in range(w.n)]
        got = _host(C)
        E_ref, F_ref, _, C_ref = qd.sliced_product(A, B)
        assert np.array_equal(Eh, E_ref) and np.array_equal(Fh, F_ref)
        assert _bits_equal(got, C_ref)
        vals = [got[:, i, j] for i, j in zip(rows, cols)]
    else:
        rng = np.random.default_rng(w.m + samples)
        rows = [int(x) for x in rng.integers(0, w.m, samples)] + [0, w.m - 1]
        cols = [int(x) for x in rng.integers(0, w.n, samples)] + [w.n - 1, 0]
        import torch
        ri = torch.as_tensor(rows, device="cuda")
        ci = torch.as_tensor(cols, device="cuda")
        got = _host(C[:, ri, ci])
        vals = [got[:, q] for q in range(len(rows))]
        for q, (i, j) in enumerate(zip(rows, cols)):
            Ei, Fj, ref = _oracle_entry(A, B, i, j)
            assert Ei == Eh[i] and Fj == Fh[j]
            assert _bits_equal(got[:, q], ref), (i, j)
    exact_vals = qd.exact_entries(A, B, rows, cols)
    err = np.array([float(abs(sum(Fraction(float(c)) for c in v) - e)) for v, e in zip(vals, exact_vals)])
    bound = qd.error_bound(A[0], B[0], Eh, Fh, rows, cols)
    ratio = float((err / bound).max())
    absAB = np.einsum("qk,kq->q", np.abs(A[0])[rows, :], np.abs(B[0])[:, cols])
    rel = float((err / absAB).max())
    _say(f"[qd parity] {name}: max err/bound = {ratio:.3e}, max err/(|A||B|) = {rel:.3e}")
    assert ratio <= 1.0


# ---------------------------------------------------------------------------
# metamorphic relations (exact level sums make these hold bit for bit)
# ---------------------------------------------------------------------------
def test_qd_metamorphic_relations(gpu):
    m, n, k = 70, 45, 90
    A = workloads.random_qd((m, k), 801, "signed_exp20")
    B = workloads.random_qd((k, n), 802, "uniform")
    C = _host(gpu.qd_gemm(_dev(A), _dev(B)))
    # k permutation: the same products summed in another order
    perm = np.random.default_rng(3).permutation(k)
    Cp = _host(gpu.qd_gemm(_dev(A[:, :, perm]), _dev(B[:, perm, :])))
    assert _bits_equal(Cp, C)
    # power-of-two scaling of A's rows and B's columns scales C exactly
    er = np.random.default_rng(4).integers(-40, 41, m)
    ec = np.random.default_rng(5).integers(-40, 41, n)
    As = A * np.ldexp(1.0, er)[None, :, None]
    Bs = B * np.ldexp(1.0, ec)[None, None, :]
    Cs = _host(gpu.qd_gemm(_dev(As), _dev(Bs)))
    assert _bits_equal(Cs, C * np.ldexp(1.0, er[:, None] + ec[None, :])[None])
    # negation of A negates C (compared as values: an exact zero stays +0)
    Cn = _host(gpu.qd_gemm(_dev(-A), _dev(B)))
    assert np.array_equal(Cn, -C)
    # transposition: (A B)^T = B^T A^T, the operands swapping roles
    Ct = _host(gpu.qd_gemm(_dev(B.transpose(0, 2, 1)), _dev(A.transpose(0, 2, 1))))
    assert _bits_equal(Ct, C.transpose(0, 2, 1))
