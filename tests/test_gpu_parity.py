"""Parity of the HIP path with the CPU oracle (GPU tests; call through the C ABI).

Bars:
* slicing (exponents and every slice), level sums, and the whole sliced chain
  (slices -> level sums -> cascade) are bit-exact against the oracle's exact
  big-integer implementation of the same steps;
* the product is within 1e-28 * (|A||B|)_ij of the classical double-double
  oracle on the five workloads (all entries at 64^3 and 1024^3, sampled entries
  at the full sizes of the others), in the launch configuration the bench times.
Every expected value comes from oracle/ on oracle inputs; nothing is read back
from the GPU and fed to the oracle.
"""
import math
import os
import sys

import numpy as np
import pytest

from oracle import compare, exact, native
import workloads

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


def _gpu_split(ddg, hi, lo, axis):
    from extended_precision_gemm_amd import layout
    E, packed = ddg.split_balanced(_dev(hi), _dev(lo), axis)
    outer = hi.shape[0] if axis == 0 else hi.shape[1]
    k = hi.shape[1] if axis == 0 else hi.shape[0]
    return E, packed, outer, k


def _unpacked(packed, outer, k, rows=None):
    """(8, outer, k) host planes (only the selected outer indices when given)."""
    from extended_precision_gemm_amd import layout
    import torch
    planes = layout.unpack(packed, outer, k)
    if rows is not None:
        planes = planes[:, torch.as_tensor(np.asarray(rows), device=packed.device), :]
    return _host(planes.contiguous())


# ---------------------------------------------------------------------------
# device probe
# ---------------------------------------------------------------------------
def test_mfma_f64_lane_layout(gpu):
    """a-operand lane L holds A[L%16][L//16], b-operand lane L holds B[L//16][L%16],
    result lane L holds D[L//16 + 4v][L%16]: the layout the packing and the
    result stores assume (measured on gfx950)."""
    out = _host(gpu.probe_mfma_f64())
    lanes = np.arange(64)
    A = np.zeros((16, 4))
    B = np.zeros((4, 16))
    A[lanes % 16, lanes // 16] = lanes + 1
    B[lanes // 16, lanes % 16] = 100.0 * (lanes + 1)
    D = A @ B
    expect = np.array([[D[L // 16 + 4 * v, L % 16] for v in range(4)] for L in range(64)])
    assert np.array_equal(out, expect), out


# ---------------------------------------------------------------------------
# slicing
# ---------------------------------------------------------------------------
def test_split_reproduces_the_pages_worked_example(gpu):
    x = float.fromhex("0x1.234cc9da46998p-1")  # the fraction bits of §2's example, exponent 0
    hi = np.full((1, 1), x)
    for axis in (0, 1):
        E, packed, outer, k = _gpu_split(gpu, hi, np.zeros_like(hi), axis)
        assert _host(E).tolist() == [0]
        got = _unpacked(packed, outer, k)[:, 0, 0]
        digits = [4660, 6547, 5777, 5324, 0, 0, 0, 0]
        assert got.tolist() == [d * 2.0 ** (-13 * (s + 1)) for s, d in enumerate(digits)]


def _edge_matrix(rng, m, k):
    hi = rng.uniform(-1, 1, (m, k))
    hi *= np.ldexp(1.0, rng.integers(-12, 3, (m, k)))
    lo_raw = hi * 2.0 ** -53 * rng.uniform(-1, 1, (m, k))
    s = hi + lo_raw
    lo = lo_raw - (s - hi)
    hi = s
    if m > 2 and k > 2:
        hi[1, :] = 0.0
        lo[1, :] = 0.0                          # all-zero row
        hi[:, 2] = 0.0
        lo[:, 2] = 0.0                          # all-zero column
        hi[0, 0], lo[0, 0] = 1.0, -0.75         # unnormalised: |hi + lo| < |hi|
        hi[0, 1], lo[0, 1] = 0.5, -2.0 ** -60   # opposite signs (Problem 3.3)
        hi[2, 0], lo[2, 0] = -0.0, 0.0          # negative zero
        hi[-1, -1], lo[-1, -1] = 2.0 ** -1074, 0.0  # subnormal
        hi[-1, 0], lo[-1, 0] = 3 * 2.0 ** -1060, -2.0 ** -1074
    return hi, lo


SMALL_SHAPES = [(1, 1, 1), (3, 5, 7), (16, 16, 4), (17, 33, 5), (64, 64, 64), (130, 65, 33), (1, 300, 200), (200, 1, 300)]


@pytest.mark.parametrize("m,n,k", SMALL_SHAPES)
def test_split_bit_exact_small(gpu, m, n, k):
    rng = np.random.default_rng(m * 1000 + n * 10 + k)
    Ah, Al = _edge_matrix(rng, m, k)
    Bh, Bl = _edge_matrix(rng, k, n)
    for (hi, lo, axis) in ((Ah, Al, 0), (Bh, Bl, 1)):
        E, packed, outer, k_ = _gpu_split(gpu, hi, lo, axis)
        if axis == 0:
            E_ref, D = exact.slice_rows(hi, lo)
        else:
            E_ref, D = exact.slice_cols(hi, lo)
            D = D.transpose(0, 2, 1)  # (8, outer=n, k)
        assert np.array_equal(_host(E), E_ref)
        assert _bits_equal(_unpacked(packed, outer, k_), exact.slice_values(D))
        # padding holds +0.0
        from extended_precision_gemm_amd import layout
        Op, Kp = layout.padded(outer, k_)
        full = _host(packed).reshape(-1)
        mask = np.ones(Op * Kp * 8, dtype=bool)
        mask[layout.pack(np.ones((8, outer, k_)), outer, k_) != 0] = False
        assert np.all(full[mask].view(np.int64) == 0)


@pytest.mark.parametrize("axis", [0, 1])
@pytest.mark.parametrize("k", [37, 300, 512, 513])
def test_split_block_path_bit_exact(gpu, axis, k):
    """Operands with >= 1024 blocks of 16 rows (columns) take a one-pass block
    kernel: up to k = 512 the block's entries stay in registers and are read
    once, above that they are read twice, the second time from cache.  Ragged
    outer size, the edge values of the small tests, an all-zero block and an
    entry far above the rest.  The leading 1040 rows (columns) sliced on their
    own (65 blocks: the two-pass path) give the same exponents and slices bit
    for bit; sampled rows (columns), and at k = 37 all of them, equal the
    oracle's."""
    rng = np.random.default_rng(55 + axis + 7 * k)
    outer, lead = 16500, 1040
    hi, lo = _edge_matrix(rng, outer, k)
    hi[200:216, :] = 0.0
    lo[200:216, :] = 0.0                      # a whole all-zero 16-row block
    hi[16400, 5] = 2.0 ** 300                 # one row far above the others
    if axis == 1:
        hi, lo = np.ascontiguousarray(hi.T), np.ascontiguousarray(lo.T)
    _say(f"[split block] axis={axis} outer={outer} k={k}")
    E, packed, outer_, k_ = _gpu_split(gpu, hi, lo, axis)
    assert (outer_, k_) == (outer, k)
    sub = (lambda x: x[:lead]) if axis == 0 else (lambda x: x[:, :lead])
    E2, packed2, _, _ = _gpu_split(gpu, np.ascontiguousarray(sub(hi)), np.ascontiguousarray(sub(lo)), axis)
    hE = _host(E)
    assert np.array_equal(hE[:lead], _host(E2))
    assert _bits_equal(_unpacked(packed, outer, k, range(lead)), _unpacked(packed2, lead, k))
    if k == 37:
        rows = list(range(outer))
    else:
        rows = sorted({0, 1, 2, 3, 15, 16, 205, lead - 1, lead, 8191, 16383, 16384, 16400, outer - 1}
                      | {int(x) for x in rng.integers(0, outer, 6)})
    if axis == 0:
        E_ref, D = exact.slice_rows(hi, lo, rows)
    else:
        E_ref, D = exact.slice_cols(hi, lo, rows)
        D = D.transpose(0, 2, 1)
    assert np.array_equal(hE[rows], E_ref)
    assert _bits_equal(_unpacked(packed, outer, k, rows), exact.slice_values(D))


@pytest.mark.parametrize("rows,cols", [(3000, 2500), (64, 30000), (1500, 4100)])
def test_split_large_B_two_pass_bit_exact(gpu, rows, cols):
    """B operands above the one-pass size (24 MiB) take the two-pass split
    (column-block exponents, then slices): ragged column blocks, the edge values
    of the small tests, a column whose only nonzero entry is in the last row, an
    entry whose RN(hi + lo) rounds up to the next binade; then NULL lo and a
    strided view."""
    import torch
    assert rows * cols * 16 > 24 << 20
    rng = np.random.default_rng(rows + cols)
    hi, lo = _edge_matrix(rng, rows, cols)
    hi[:, cols - 3] = 0.0
    lo[:, cols - 3] = 0.0
    hi[rows - 1, cols - 3] = 2.0 ** 30                      # last row decides the column
    hi[rows // 2, cols - 5], lo[rows // 2, cols - 5] = 2.0 ** 40 - 2.0 ** -13, 2.0 ** -14  # tie: RN -> 2^40
    hi[:, 1030] *= 2.0 ** 200                                # a column far above the others
    E, packed, outer, k = _gpu_split(gpu, hi, lo, 1)
    F_ref = exact.balancing_exponents(hi, lo, 1)
    assert np.array_equal(_host(E), F_ref)
    cols_s = sorted({0, 2, 1023, 1024, 1030, cols - 5, cols - 3, cols - 1})
    _, D = exact.slice_cols(hi, lo, cols_s)
    assert _bits_equal(_unpacked(packed, outer, k, cols_s), exact.slice_values(D.transpose(0, 2, 1)))
    # NULL lo
    E0, _ = gpu.split_balanced(_dev(hi), None, 1)
    assert np.array_equal(_host(E0), exact.balancing_exponents(hi, np.zeros_like(lo), 1))
    # a strided view: columns of a wider matrix
    wide_h = torch.zeros((rows, cols + 40), dtype=torch.float64, device="cuda")
    wide_l = torch.zeros_like(wide_h)
    wide_h[:, 7:7 + cols] = _dev(hi)
    wide_l[:, 7:7 + cols] = _dev(lo)
    Es, Ps = gpu.split_balanced(wide_h[:, 7:7 + cols], wide_l[:, 7:7 + cols], 1)
    assert np.array_equal(_host(Es), F_ref)
    assert torch.equal(Ps.view(torch.int64), packed.view(torch.int64))


# The largest window integer any entry can have: RN(hi + lo) < 2^E forces
# |x| < 2^E (1 - 2^-54), so N <= 2^104 - 2^50 - 1, digits 8191 except 6143 in slice 4.
MAX_HI, MAX_LO = 1.0 - 2.0 ** -53, 2.0 ** -54 - 2.0 ** -104
MAX_DIGITS = [8191, 8191, 8191, 8191, 6143, 8191, 8191, 8191]


def test_split_largest_digits(gpu):
    hi = np.full((3, 40), MAX_HI)
    lo = np.full((3, 40), MAX_LO)
    assert exact.slice_entry(MAX_HI, MAX_LO, 0) == MAX_DIGITS
    E, packed, outer, k = _gpu_split(gpu, hi, lo, 0)
    assert _host(E).tolist() == [0, 0, 0]
    got = _unpacked(packed, outer, k)
    for s in range(8):
        assert np.all(got[s] == MAX_DIGITS[s] * 2.0 ** (-13 * (s + 1)))


# ---------------------------------------------------------------------------
# level sums, cascade, and the whole sliced chain
# ---------------------------------------------------------------------------
def _oracle_chain(Ah, Al, Bh, Bl, rows=None, cols=None):
    """Level sums, the stage chain's cascade and the product's nearest double-double."""
    E, DA = exact.slice_rows(Ah, Al, rows)
    F, DB = exact.slice_cols(Bh, Bl, cols)
    S_units = exact.level_sums_units(DA, DB)
    S = exact.level_values(S_units)
    Ch, Cl = exact.renorm_levels(S, E, F)
    Nh, Nl = exact.nearest_dd(S_units, E, F)
    return S, Ch, Cl, Nh, Nl


def _gpu_chain(gpu, Ah, Al, Bh, Bl):
    m, k = Ah.shape
    n = Bh.shape[1]
    E, As = gpu.split_balanced(_dev(Ah), _dev(Al), 0)
    F, Bs = gpu.split_balanced(_dev(Bh), _dev(Bl), 1)
    levels = gpu.sliced_gemm(m, n, k, As, Bs)
    Ch, Cl = gpu.renorm_levels(levels, E, F)
    Fh, Fl = gpu.sliced_gemm_renorm(m, n, k, As, E, Bs, F)
    return levels, Ch, Cl, Fh, Fl


@pytest.mark.parametrize("m,n,k", SMALL_SHAPES + [(128, 128, 16), (96, 160, 100)])
def test_sliced_chain_bit_exact_small(gpu, m, n, k):
    rng = np.random.default_rng(7 + m + 3 * n + 5 * k)
    Ah, Al = _edge_matrix(rng, m, k)
    Bh, Bl = _edge_matrix(rng, k, n)
    S, Ch_ref, Cl_ref, Nh_ref, Nl_ref = _oracle_chain(Ah, Al, Bh, Bl)
    levels, Ch, Cl, Fh, Fl = _gpu_chain(gpu, Ah, Al, Bh, Bl)
    assert _bits_equal(_host(levels), S), "level sums"
    assert _bits_equal(_host(Ch), Ch_ref) and _bits_equal(_host(Cl), Cl_ref), "cascade"
    assert _bits_equal(_host(Fh), Ch_ref) and _bits_equal(_host(Fl), Cl_ref), "fused epilogue"
    Gh, Gl = gpu.dd_gemm(_dev(Ah), _dev(Al), _dev(Bh), _dev(Bl))
    assert _bits_equal(_host(Gh), Nh_ref) and _bits_equal(_host(Gl), Nl_ref), "dd_gemm_ws"
    Hh, Hl = gpu.dd_gemm_alloc(_dev(Ah), _dev(Al), _dev(Bh), _dev(Bl))
    assert _bits_equal(_host(Hh), Nh_ref) and _bits_equal(_host(Hl), Nl_ref), "dd_gemm"


def test_level_sums_exact_at_the_bound(gpu):
    """Largest digits everywhere and k = 8192: level sums reach ~2^42 units, exactly."""
    m, n, k = 32, 48, 8192
    Ah = np.full((m, k), MAX_HI)
    Al = np.full((m, k), MAX_LO)
    E, As = gpu.split_balanced(_dev(Ah), _dev(Al), 0)
    F, Bs = gpu.split_balanced(_dev(np.full((k, n), -MAX_HI)), _dev(np.full((k, n), -MAX_LO)), 1)
    levels = _host(gpu.sliced_gemm(m, n, k, As, Bs))
    for l in range(8):
        expect = -k * sum(MAX_DIGITS[s] * MAX_DIGITS[l - s] for s in range(l + 1))
        assert np.all(levels[l] * 2.0 ** (13 * (l + 2)) == expect), l


@pytest.mark.parametrize("m,n,k,ns", [(40, 50, 8292, 8), (33, 70, 4096, 8), (20, 30, 4097, 8),
                                      (45, 17, 4133, 16), (21, 40, 12000, 5), (30, 30, 5500, 12)])
def test_pair_group_sums_across_exact_chunks(gpu, m, n, k, ns):
    """The pair-packed schedule's group sums, bit for bit against the oracle,
    for k at, just past and several times past the most values whose FP64 group
    sums stay exact (4096 for 8 slices): the kernel moves them into int64
    planes chunk by chunk."""
    rng = np.random.default_rng(m * n + k + ns)
    Ah, Al = _edge_matrix(rng, m, k)
    Bh, Bl = _edge_matrix(rng, k, n)
    _, DA = exact.slice_rows(Ah, Al, nslices=ns)
    _, DB = exact.slice_cols(Bh, Bl, nslices=ns)
    _, As = gpu.split_balanced(_dev(Ah), _dev(Al), 0, nslices=ns)
    _, Bs = gpu.split_balanced(_dev(Bh), _dev(Bl), 1, nslices=ns)
    G = gpu.sliced_gemm_pairs(m, n, k, As, Bs, nslices=ns)
    assert np.array_equal(_host(G), exact.paired_group_units(DA, DB))


def test_unsplit_product_across_exact_chunks(gpu):
    """A product whose 256 output tiles fill one round (never split) with k past
    one exact FP64 chunk: the int64 chunk planes of the workspace carry the
    group sums; sampled entries equal the oracle's nearest chain bit for bit."""
    m, n, k = 1024, 1024, 4200
    assert gpu.split_parts(m, n, k) == 1
    Ah, Al = workloads.random_dd((m, k), 71, "signed_exp20")
    Bh, Bl = workloads.random_dd((k, n), 72, "normal")
    Ch, Cl = gpu.dd_gemm(_dev(Ah), _dev(Al), _dev(Bh), _dev(Bl))
    rows = [0, 1, 511, 1023]
    cols = [0, 63, 64, 1023]
    _, _, _, Nh, Nl = _oracle_chain(Ah, Al, Bh, Bl, rows, cols)
    assert _bits_equal(_host(Ch)[np.ix_(rows, cols)], Nh) and _bits_equal(_host(Cl)[np.ix_(rows, cols)], Nl)


# ---------------------------------------------------------------------------
# end to end against the classical oracle, edge cases, metamorphic relations
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("m,n,k", [(1, 1, 1), (17, 33, 5), (130, 65, 33), (64, 200, 300)])
def test_dd_gemm_within_tolerance_small(gpu, m, n, k):
    rng = np.random.default_rng(m + n + k)
    Ah, Al = workloads.random_dd((m, k), rng.integers(1 << 30))
    Bh, Bl = workloads.random_dd((k, n), rng.integers(1 << 30))
    Ch, Cl = gpu.dd_gemm(_dev(Ah), _dev(Al), _dev(Bh), _dev(Bl))
    Rh, Rl, _ = native.dd_gemm(Ah, Al, Bh, Bl)
    assert compare.error_ratio(_host(Ch), _host(Cl), Rh, Rl, compare.abs_product(Ah, Bh)) <= compare.TOL


def test_k_zero_writes_zeros_and_empty_is_noop(gpu):
    import torch
    Ch = torch.full((5, 7), 3.0, dtype=torch.float64, device="cuda")
    Cl = torch.full((5, 7), 3.0, dtype=torch.float64, device="cuda")
    A = torch.zeros((5, 0), dtype=torch.float64, device="cuda")
    B = torch.zeros((0, 7), dtype=torch.float64, device="cuda")
    gpu.dd_gemm(A, None, B, None, Ch, Cl)
    assert np.all(_host(Ch) == 0) and np.all(_host(Cl) == 0)
    E = torch.zeros((0, 4), dtype=torch.float64, device="cuda")
    out = gpu.dd_gemm(E, None, torch.zeros((4, 3), dtype=torch.float64, device="cuda"), None)
    assert out[0].shape == (0, 3)


def test_strided_operands_and_null_lo(gpu):
    import torch
    rng = np.random.default_rng(21)
    Ah, Al = workloads.random_dd((40, 70), 5)
    Bh, Bl = workloads.random_dd((70, 90), 6)
    # operands as column windows of wider matrices (lda > k, ldb > n), C likewise
    Abig = torch.zeros((40, 100), dtype=torch.float64, device="cuda")
    Abig[:, 10:80] = _dev(Ah)
    Bbig = torch.zeros((70, 128), dtype=torch.float64, device="cuda")
    Bbig[:, 3:93] = _dev(Bh)
    Cbig = torch.zeros((2, 40, 96), dtype=torch.float64, device="cuda")
    Ch, Cl = gpu.dd_gemm(Abig[:, 10:80], None, Bbig[:, 3:93], None, Cbig[0, :, :90], Cbig[1, :, :90])
    ref = gpu.dd_gemm(_dev(Ah), None, _dev(Bh), None)
    assert _bits_equal(_host(Ch), _host(ref[0])) and _bits_equal(_host(Cl), _host(ref[1]))
    assert np.all(_host(Cbig[:, :, 90:]) == 0)
    Rh, Rl, _ = native.dd_gemm(Ah, None, Bh, None)
    assert compare.error_ratio(_host(Ch), _host(Cl), Rh, Rl, compare.abs_product(Ah, Bh)) <= compare.TOL


def test_identity_returns_the_windowed_operand(gpu):
    rng = np.random.default_rng(22)
    Bh, Bl = workloads.random_dd((50, 37), 9)
    I = np.eye(50)
    Ch, Cl = gpu.dd_gemm(_dev(I), None, _dev(Bh), _dev(Bl))
    # each column of B is cut at 104 bits below its own exponent: exact when on the grid
    F, DB = exact.slice_cols(Bh, Bl)
    for j in (0, 7, 36):
        for p in (0, 13, 49):
            got = exact.dd_to_fraction(_host(Ch)[p, j], _host(Cl)[p, j])
            assert got == exact.reconstruct_entry(DB[:, p, j], int(F[j]))


def test_metamorphic_relations_bitwise(gpu):
    """Exact level sums make these hold bit for bit: power-of-two scaling of A's
    rows and B's columns, permutation of k, transposition, negation, repetition."""
    import torch
    rng = np.random.default_rng(23)
    m, n, k = 70, 90, 130
    Ah, Al = workloads.random_dd((m, k), 11)
    Bh, Bl = workloads.random_dd((k, n), 12)
    C = [_host(t) for t in gpu.dd_gemm(_dev(Ah), _dev(Al), _dev(Bh), _dev(Bl))]
    ra = np.ldexp(1.0, rng.integers(-40, 40, m)).reshape(-1, 1)
    cb = np.ldexp(1.0, rng.integers(-40, 40, n)).reshape(1, -1)
    S = [_host(t) for t in gpu.dd_gemm(_dev(Ah * ra), _dev(Al * ra), _dev(Bh * cb), _dev(Bl * cb))]
    assert _bits_equal(S[0], C[0] * ra * cb) and _bits_equal(S[1], C[1] * ra * cb)
    perm = rng.permutation(k)
    P = [_host(t) for t in gpu.dd_gemm(_dev(Ah[:, perm]), _dev(Al[:, perm]), _dev(Bh[perm]), _dev(Bl[perm]))]
    assert _bits_equal(P[0], C[0]) and _bits_equal(P[1], C[1])
    T = [_host(t) for t in gpu.dd_gemm(_dev(Bh.T), _dev(Bl.T), _dev(Ah.T), _dev(Al.T))]
    assert _bits_equal(T[0].T, C[0]) and _bits_equal(T[1].T, C[1])
    N = [_host(t) for t in gpu.dd_gemm(_dev(-Ah), _dev(-Al), _dev(Bh), _dev(Bl))]
    assert _bits_equal(N[0], -C[0]) and _bits_equal(N[1], -C[1])
    R = [_host(t) for t in gpu.dd_gemm(_dev(Ah), _dev(Al), _dev(Bh), _dev(Bl))]
    assert _bits_equal(R[0], C[0]) and _bits_equal(R[1], C[1])


def test_results_beyond_the_double_range_overflow_like_ldexp(gpu):
    """Entries near 2^600 in both operands: products near 2^1200 become
    infinities of the right sign (the scaling 2^(E_i + F_j) overflows as ldexp
    does), rows scaled back into range stay finite, all bit for bit as in the
    oracle's chain."""
    rng = np.random.default_rng(77)
    m, n, k = 20, 18, 24
    Ah = rng.integers(-9, 10, (m, k)).astype(np.float64) * 2.0 ** 600
    Bh = rng.integers(-9, 10, (k, n)).astype(np.float64) * 2.0 ** 600
    Ah[:5] *= 2.0 ** -700                       # these rows' products stay finite
    Al, Bl = np.zeros_like(Ah), np.zeros_like(Bh)
    Ch, Cl = gpu.dd_gemm(_dev(Ah), None, _dev(Bh), None)
    _, Sh, Sl, Rh, Rl = _oracle_chain(Ah, Al, Bh, Bl)
    hCh, hCl = _host(Ch), _host(Cl)
    assert _bits_equal(hCh, Rh) and _bits_equal(hCl, Rl)
    E, As = gpu.split_balanced(_dev(Ah), None, 0)
    F, Bs = gpu.split_balanced(_dev(Bh), None, 1)
    Fh, Fl = gpu.sliced_gemm_renorm(m, n, k, As, E, Bs, F)  # the stage chain's cascade
    assert _bits_equal(_host(Fh), Sh) and _bits_equal(_host(Fl), Sl)
    assert np.isinf(hCh[5:]).any() and np.isfinite(hCh[:5]).all()
    exact_sign = np.sign((Ah[5:] * 2.0 ** -600) @ (Bh * 2.0 ** -600))   # small integers: exact
    inf_rows = np.isinf(hCh[5:])
    assert np.array_equal(np.sign(hCh[5:])[inf_rows], exact_sign[inf_rows])


def test_results_near_the_bottom_of_the_double_range_underflow_gradually(gpu):
    """Entries near 2^-500 with rows scaled down by up to 2^-47: the products'
    leading words run from normal doubles near 2^-1000 into subnormals, and
    the trailing words of the normal ones are subnormal.  The nearest
    double-double honours gradual underflow (each word rounded at 2^-1074
    where it reaches that far), as in the oracle's pair-packed chain, bit for
    bit."""
    rng = np.random.default_rng(79)
    m, n, k = 24, 20, 30
    sign = lambda shape: np.where(rng.integers(0, 2, shape) == 1, 1.0, -1.0)
    Ah = rng.uniform(1, 2, (m, k)) * sign((m, k)) * 2.0 ** -500
    Bh = rng.uniform(1, 2, (k, n)) * sign((k, n)) * 2.0 ** -505
    Ah *= np.ldexp(1.0, -rng.integers(0, 48, (m, 1)))
    Al = Ah * 2.0 ** -53 * rng.uniform(-1, 1, (m, k))
    t = Ah + Al
    Al, Ah = Al - (t - Ah), t
    Bl = Bh * 2.0 ** -53 * rng.uniform(-1, 1, (k, n))
    t = Bh + Bl
    Bl, Bh = Bl - (t - Bh), t
    Rh, Rl = exact.paired_product(Ah, Al, Bh, Bl, 8)
    tiny = 2.0 ** -1022
    assert (np.abs(Rh) >= tiny).sum() > 50 and ((np.abs(Rh) < tiny) & (Rh != 0)).sum() > 50
    assert ((Rl != 0) & (np.abs(Rl) < tiny)).sum() > 50
    Ch, Cl = gpu.dd_gemm(_dev(Ah), _dev(Al), _dev(Bh), _dev(Bl))
    assert _bits_equal(_host(Ch), Rh) and _bits_equal(_host(Cl), Rl)


def test_level_planes_with_a_wider_stride(gpu):
    """dd_sliced_gemm / dd_renorm_levels with ldl > n and ldc > n, through the C
    ABI: the level sums and the cascade match the packed-stride calls, and the
    padding columns are left untouched."""
    import torch
    m, n, k, pad = 70, 45, 33, 7
    Ah, Al = workloads.random_dd((m, k), 61, "signed_exp20")
    Bh, Bl = workloads.random_dd((k, n), 62, "uniform")
    E, As = gpu.split_balanced(_dev(Ah), _dev(Al), 0)
    F, Bs = gpu.split_balanced(_dev(Bh), _dev(Bl), 1)
    ref = gpu.sliced_gemm(m, n, k, As, Bs)
    Rh, Rl = gpu.renorm_levels(ref, E, F)
    ldl = n + pad
    wide = torch.full((8, m, ldl), 3.0, dtype=torch.float64, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    L = gpu.lib
    assert L.dd_sliced_gemm(m, n, k, As.data_ptr(), Bs.data_ptr(), wide.data_ptr(), ldl, s) == 0
    assert _bits_equal(_host(wide[:, :, :n].contiguous()), _host(ref))
    assert (_host(wide[:, :, n:]) == 3.0).all()
    Ch = torch.full((m, ldl + 2), 5.0, dtype=torch.float64, device="cuda")
    Cl = torch.full((m, ldl + 2), 5.0, dtype=torch.float64, device="cuda")
    assert L.dd_renorm_levels(m, n, wide.data_ptr(), ldl, E.data_ptr(), F.data_ptr(), Ch.data_ptr(),
                              Cl.data_ptr(), ldl + 2, s) == 0
    assert _bits_equal(_host(Ch[:, :n].contiguous()), _host(Rh))
    assert _bits_equal(_host(Cl[:, :n].contiguous()), _host(Rl))
    assert (_host(Ch[:, n:]) == 5.0).all() and (_host(Cl[:, n:]) == 5.0).all()


def test_nondefault_stream(gpu):
    import torch
    Ah, Al = workloads.random_dd((64, 64), 31)
    Bh, Bl = workloads.random_dd((64, 64), 32)
    ref = [_host(t) for t in gpu.dd_gemm(_dev(Ah), _dev(Al), _dev(Bh), _dev(Bl))]
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out = gpu.dd_gemm(_dev(Ah), _dev(Al), _dev(Bh), _dev(Bl))
    s.synchronize()
    assert _bits_equal(_host(out[0]), ref[0]) and _bits_equal(_host(out[1]), ref[1])


def test_workspace_of_a_call_on_a_stream_that_is_not_current(gpu):
    """dd_gemm / qd_gemm given a stream that is not the current one take their
    workspace from the allocator on the current stream; it must stay reserved
    until the kernels on the given stream are done.  Memory taken and written
    on the current stream right after the call must not corrupt the result."""
    import torch
    m, n, k = 512, 384, 1024
    Ah, Al = (_dev(x) for x in workloads.random_dd((m, k), 41, "signed_exp20"))
    Bh, Bl = (_dev(x) for x in workloads.random_dd((k, n), 42, "signed_exp20"))
    ref = [_host(t) for t in gpu.dd_gemm(Ah, Al, Bh, Bl)]
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    out = gpu.dd_gemm(Ah, Al, Bh, Bl, stream=s)
    junk = torch.empty(gpu.workspace_size(m, n, k), dtype=torch.uint8, device=Ah.device)
    junk.fill_(0x7F)
    s.synchronize()
    torch.cuda.synchronize()
    assert _bits_equal(_host(out[0]), ref[0]) and _bits_equal(_host(out[1]), ref[1])
    A = _dev(workloads.random_qd((m, k), 43, "uniform"))
    B = _dev(workloads.random_qd((k, n), 44, "uniform"))
    qref = _host(gpu.qd_gemm(A, B))
    torch.cuda.synchronize()
    s.wait_stream(torch.cuda.current_stream())
    qout = gpu.qd_gemm(A, B, stream=s)
    junk = torch.empty(gpu.qd_workspace_size(m, n, k), dtype=torch.uint8, device=A.device)
    junk.fill_(0x7F)
    s.synchronize()
    torch.cuda.synchronize()
    assert _bits_equal(_host(qout), qref)


# ---------------------------------------------------------------------------
# the five workloads at full size
# ---------------------------------------------------------------------------
def _sample_indices(rng, size, count):
    idx = set([0, size - 1]) | set(rng.integers(0, size, count).tolist())
    return np.array(sorted(idx))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", [w.name for w in workloads.WORKLOADS])
def test_workload_parity(gpu, workload_operands, name):
    import torch
    w = workloads.by_name(name)
    _say(f"[parity] {name}: generating operands m={w.m} n={w.n} k={w.k}")
    Ah, Al, Bh, Bl = workload_operands(name)
    m, n, k = w.m, w.n, w.k
    rng = np.random.default_rng(2024 + w.index)
    dA, dAl, dB, dBl = _dev(Ah), _dev(Al), _dev(Bh), _dev(Bl)

    _say(f"[parity] {name}: slicing")
    E, As = gpu.split_balanced(dA, dAl, 0)
    F, Bs = gpu.split_balanced(dB, dBl, 1)
    assert np.array_equal(_host(E), exact.balancing_exponents(Ah, Al, 0)), "row exponents"
    assert np.array_equal(_host(F), exact.balancing_exponents(Bh, Bl, 1)), "column exponents"
    rows = _sample_indices(rng, m, 6)
    cols = _sample_indices(rng, n, 6)
    if w.cancel_col0:
        cols = np.union1d(cols, [0])
    _, DA = exact.slice_rows(Ah, Al, rows)
    _, DB = exact.slice_cols(Bh, Bl, cols)
    from extended_precision_gemm_amd import layout
    gotA = _unpacked(As, m, k, rows)
    assert _bits_equal(gotA, exact.slice_values(DA)), "A slices"
    gotB = _unpacked(Bs, n, k, cols)
    assert _bits_equal(gotB, exact.slice_values(DB.transpose(0, 2, 1))), "B slices"

    _say(f"[parity] {name}: level sums and cascade (sampled {len(rows)}x{len(cols)} block)")
    levels = gpu.sliced_gemm(m, n, k, As, Bs)
    S_ref = exact.level_values(exact.level_sums_units(DA, DB))
    ri = torch.as_tensor(rows, device="cuda")
    ci = torch.as_tensor(cols, device="cuda")
    got_levels = _host(levels[:, ri][:, :, ci].contiguous())
    assert _bits_equal(got_levels, S_ref), "level sums"
    E_s = exact.balancing_exponents(Ah[rows], Al[rows], 0)
    F_s = exact.balancing_exponents(Bh[:, cols], Bl[:, cols], 1)
    Ch_ref, Cl_ref = exact.renorm_levels(S_ref, E_s, F_s)
    Rh, Rl = gpu.renorm_levels(levels, E, F)
    del levels
    Fh, Fl = gpu.sliced_gemm_renorm(m, n, k, As, E, Bs, F)
    assert _bits_equal(_host(Fh), _host(Rh)) and _bits_equal(_host(Fl), _host(Rl)), "fused == two-step"
    assert _bits_equal(_host(Fh[ri][:, ci]), Ch_ref) and _bits_equal(_host(Fl[ri][:, ci]), Cl_ref), "cascade"
    del Rh, Rl, Fh, Fl

    _say(f"[parity] {name}: pair-packed group sums (sampled {len(rows)}x{len(cols)} block)")
    G = gpu.sliced_gemm_pairs(m, n, k, As, Bs)
    assert np.array_equal(_host(G[:, ri][:, :, ci].contiguous()), exact.paired_group_units(DA, DB)), "group sums"
    del G, As, Bs
    torch.cuda.empty_cache()

    _say(f"[parity] {name}: dd_gemm end to end")
    Ch, Cl = gpu.dd_gemm(dA, dAl, dB, dBl)
    hCh, hCl = _host(Ch), _host(Cl)
    Nh_ref, Nl_ref = exact.nearest_dd(exact.level_sums_units(DA, DB), E_s, F_s)
    sub_h = hCh[np.ix_(rows, cols)]
    sub_l = hCl[np.ix_(rows, cols)]
    assert _bits_equal(sub_h, Nh_ref) and _bits_equal(sub_l, Nl_ref), "product vs oracle's nearest chain"

    if m * n * k <= 1024 ** 3:
        _say(f"[parity] {name}: classical oracle, all {m * n} entries")
        Rh, Rl, threads = native.dd_gemm(Ah, Al, Bh, Bl)
        absAB = compare.abs_product(Ah, Bh)
        ratio = compare.error_ratio(hCh, hCl, Rh, Rl, absAB)
        eps = compare.eps_max(hCh, hCl, Rh, Rl)
    else:
        cnt = 2048
        qr = rng.integers(0, m, cnt)
        qc = rng.integers(0, n, cnt)
        if w.cancel_col0:
            qc[: cnt // 8] = 0
        _say(f"[parity] {name}: classical oracle, {cnt} sampled entries")
        Rh, Rl = native.dd_gemm_entries(Ah, Al, Bh, Bl, qr, qc)
        absAB = compare.abs_product(Ah, Bh, qr, qc)
        ratio = compare.error_ratio(hCh[qr, qc], hCl[qr, qc], Rh, Rl, absAB)
        eps = compare.eps_max(hCh[qr, qc], hCl[qr, qc], Rh, Rl)
    _say(f"[parity] {name}: max |C-C_ref|/(|A||B|) = {ratio:.3e} (log2 {math.log2(ratio) if ratio > 0 else -math.inf:.1f}), "
         f"eps_max = {eps:.3e}")
    assert ratio <= compare.TOL
    if w.cancel_col0:
        # row sums of C cancel down to sum_p a_ip * rho_p, rho_p the rounding
        # residue of row p of B (math.fsum: correctly rounded sums of exact inputs)
        rho = np.array([math.fsum(Bh[p].tolist() + Bl[p].tolist()) for p in range(k)])
        for i in rows[:3]:
            tot = math.fsum(hCh[i].tolist() + hCl[i].tolist())
            expect = math.fsum((Ah[i] * rho).tolist() + (Al[i] * rho).tolist())
            bound = compare.TOL * float(compare.abs_product(Ah[i:i + 1], Bh).sum())
            _say(f"[parity] {name}: row {i}: sum_j C_ij = {tot:.3e}, expected {expect:.3e}, bound {bound:.3e}")
            assert abs(tot - expect) <= bound


@pytest.mark.parametrize("name", ["dd1024", "dd4096_exp20"])
def test_timed_entry_point_equals_the_product(gpu, workload_operands, name):
    """dd_gemm_ws_timed, the call the benchmark times (preallocated workspace,
    an event recorded after the slicing), writes the product of dd_gemm_ws bit
    for bit, with and without the event."""
    import torch
    w = workloads.by_name(name)
    _say(f"[parity] {name}: dd_gemm_ws_timed against dd_gemm_ws")
    Ah, Al, Bh, Bl = workload_operands(name)
    dA, dAl, dB, dBl = _dev(Ah), _dev(Al), _dev(Bh), _dev(Bl)
    Ch, Cl = gpu.dd_gemm(dA, dAl, dB, dBl)
    ws = torch.empty(gpu.workspace_size(w.m, w.n, w.k), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    start, after_split, end = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    after_split.record(stream)  # creates the event the library records
    for event in (after_split, None):
        Th = torch.full_like(Ch, float("nan"))
        Tl = torch.full_like(Cl, float("nan"))
        start.record(stream)
        gpu.dd_gemm_timed(dA, dAl, dB, dBl, Th, Tl, ws, event.cuda_event if event else None, stream)
        end.record(stream)
        torch.cuda.synchronize()
        assert _bits_equal(_host(Th), _host(Ch)) and _bits_equal(_host(Tl), _host(Cl))
        if event:
            t_split, t_all = start.elapsed_time(after_split), start.elapsed_time(end)
            _say(f"[parity] {name}: slicing {t_split:.3f} of {t_all:.3f} ms")
            assert 0.0 <= t_split <= t_all


def test_timed_qd_entry_point_equals_the_product(gpu):
    """qd_gemm_ws_timed on the 1024^3 quad-double workload writes qd_gemm_ws's
    product bit for bit, with and without its event."""
    import torch
    w = workloads.by_name("qd1024")
    A, B = workloads.make_qd_operands(w)
    dA, dB = _dev(A), _dev(B)
    C = gpu.qd_gemm(dA, dB)
    ws = torch.empty(gpu.qd_workspace_size(w.m, w.n, w.k), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    after_split = torch.cuda.Event(enable_timing=True)
    after_split.record(stream)
    for event in (after_split, None):
        T = torch.full_like(C, float("nan"))
        gpu.qd_gemm_timed(dA, dB, T, ws, event.cuda_event if event else None, stream)
        torch.cuda.synchronize()
        assert _bits_equal(_host(T), _host(C))


# ---------------------------------------------------------------------------
# fewer slices per entry (n = 4: the pages' quarters of a leading double)
# ---------------------------------------------------------------------------
def test_four_slices_split_is_the_pages_quarters(gpu):
    x = float.fromhex("0x1.234cc9da46998p-1")
    hi = np.full((1, 1), x)
    E, packed = gpu.split_balanced(_dev(hi), None, 0, nslices=4)
    from extended_precision_gemm_amd import layout
    got = _host(layout.unpack(packed, 1, 1, nslices=4).contiguous())[:, 0, 0]
    assert _host(E).tolist() == [0]
    assert got.tolist() == [d * 2.0 ** (-13 * (s + 1)) for s, d in enumerate([4660, 6547, 5777, 5324])]


@pytest.mark.parametrize("nslices", [4, 5, 6, 7, 9, 10, 11, 12, 13, 14, 15, 16])
@pytest.mark.parametrize("m,n,k", [(17, 33, 5), (130, 65, 33), (96, 160, 100)])
def test_n_slice_chain_bit_exact(gpu, nslices, m, n, k):
    rng = np.random.default_rng(nslices * 1000 + m + n + k)
    Ah, Al = _edge_matrix(rng, m, k)
    Bh, Bl = _edge_matrix(rng, k, n)
    E, DA = exact.slice_rows(Ah, Al, nslices=nslices)
    F, DB = exact.slice_cols(Bh, Bl, nslices=nslices)
    S = exact.level_values(exact.level_sums_units(DA, DB))
    Ch_ref, Cl_ref = exact.renorm_levels(S, E, F)
    from extended_precision_gemm_amd import layout
    gE, gA = gpu.split_balanced(_dev(Ah), _dev(Al), 0, nslices=nslices)
    gF, gB = gpu.split_balanced(_dev(Bh), _dev(Bl), 1, nslices=nslices)
    assert np.array_equal(_host(gE), E) and np.array_equal(_host(gF), F)
    assert _bits_equal(_host(layout.unpack(gA, m, k, nslices).contiguous()), exact.slice_values(DA))
    assert _bits_equal(_host(layout.unpack(gB, n, k, nslices).contiguous()),
                       exact.slice_values(DB).transpose(0, 2, 1))
    Fh, Fl = gpu.sliced_gemm_renorm(m, n, k, gA, gE, gB, gF, nslices=nslices)
    assert _bits_equal(_host(Fh), Ch_ref) and _bits_equal(_host(Fl), Cl_ref)
    G = gpu.sliced_gemm_pairs(m, n, k, gA, gB, nslices=nslices)
    assert np.array_equal(_host(G), exact.paired_group_units(DA, DB))
    Nh_ref, Nl_ref = exact.nearest_dd(exact.level_sums_units(DA, DB), E, F)
    Gh, Gl = gpu.dd_gemm(_dev(Ah), _dev(Al), _dev(Bh), _dev(Bl), nslices=nslices)
    assert _bits_equal(_host(Gh), Nh_ref) and _bits_equal(_host(Gl), Nl_ref)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["dd1024", "dd4096_exp20"])
def test_n_slice_products_within_their_error_bound(gpu, workload_operands, name):
    """Against the classical oracle: every n = 4..16 stays inside the per-entry
    bound of window truncation, pairs not formed and the final rounding
    (oracle.exact.error_bound, against the exact product) widened by 2^-96
    (|A||B|)_ij for the classical reference's own error; from eight slices on
    every entry also meets the tolerance 1e-28 (|A||B|)_ij."""
    Ah, Al, Bh, Bl = workload_operands(name)
    m, k = Ah.shape
    n = Bh.shape[1]
    rng = np.random.default_rng(7)
    qr = rng.integers(0, m, 1024)
    qc = rng.integers(0, n, 1024)
    Rh, Rl = native.dd_gemm_entries(Ah, Al, Bh, Bl, qr, qc)
    E = exact.balancing_exponents(Ah, Al, 0)
    F = exact.balancing_exponents(Bh, Bl, 1)
    dA, dAl, dB, dBl = _dev(Ah), _dev(Al), _dev(Bh), _dev(Bl)
    absAB = compare.abs_product(Ah, Bh, qr, qc)
    for nslices in range(4, 17):
        Ch, Cl = gpu.dd_gemm(dA, dAl, dB, dBl, nslices=nslices)
        hCh, hCl = _host(Ch), _host(Cl)
        err = np.abs((hCh[qr, qc] - Rh) + (hCl[qr, qc] - Rl))
        bound = exact.error_bound(Ah, Bh, E, F, nslices, qr, qc) + 2.0 ** -96 * absAB
        ratio = float((err / bound).max())
        tol = float((err / absAB).max())
        _say(f"[parity] {name} n={nslices}: max |C-C_ref| / bound = {ratio:.3e}, / (|A||B|) = {tol:.3e}")
        assert ratio <= 1.0
        if nslices >= 8:
            assert tol <= compare.TOL
        del Ch, Cl


def test_more_slices_recover_entries_far_below_the_row_maximum(gpu):
    """A row whose exponent is set by an entry 2^60 above its others, met by a
    zero row of B: eight slices miss the tolerance there, thirteen meet it
    (§3 Problem 3.2's concern), and both match the oracle's chain bit for bit."""
    rng = np.random.default_rng(61)
    Ah, Al = workloads.random_dd((70, 200), 62, "uniform")
    Bh, Bl = workloads.random_dd((200, 50), 63, "uniform")
    for i in range(0, 70, 7):
        p = int(rng.integers(200))
        Ah[i, p], Al[i, p] = 0.75 * 2.0 ** 60, 0.0
        Bh[p, :], Bl[p, :] = 0.0, 0.0
    rows = np.repeat(np.arange(0, 70, 7), 50)
    cols = np.tile(np.arange(50), 10)
    Rh, Rl = native.dd_gemm_entries(Ah, Al, Bh, Bl, rows, cols)
    absab = compare.abs_product(Ah, Bh)[rows, cols]
    worst = {}
    for nslices in (8, 13):
        Ch, Cl = gpu.dd_gemm(_dev(Ah), _dev(Al), _dev(Bh), _dev(Bl), nslices=nslices)
        hCh, hCl = _host(Ch), _host(Cl)
        E, DA = exact.slice_rows(Ah, Al, nslices=nslices)
        F, DB = exact.slice_cols(Bh, Bl, nslices=nslices)
        Sh, Sl = exact.nearest_dd(exact.level_sums_units(DA, DB), E, F)
        assert _bits_equal(hCh, Sh) and _bits_equal(hCl, Sl)
        worst[nslices] = float((np.abs((hCh[rows, cols] - Rh) + (hCl[rows, cols] - Rl)) / absab).max())
    _say(f"[parity] wide-range rows: n=8 {worst[8]:.3e}, n=13 {worst[13]:.3e} (tolerance {compare.TOL})")
    assert worst[8] > compare.TOL
    assert worst[13] <= compare.TOL


# ---------------------------------------------------------------------------
# k-blocked products (block results added in double-double arithmetic)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("nslices", [8, 12])
@pytest.mark.parametrize("m,n,k", [(40, 30, 250), (130, 65, 97)])
def test_kblocked_chain_bit_exact(gpu, nslices, m, n, k):
    rng = np.random.default_rng(k + m + nslices)
    Ah, Al = _edge_matrix(rng, m, k)
    Bh, Bl = _edge_matrix(rng, k, n)
    dA, dAl, dB, dBl = _dev(Ah), _dev(Al), _dev(Bh), _dev(Bl)
    for kblock in (16, 33, 100, k, k + 5):
        Rh, Rl = exact.sliced_product_kblocks(Ah, Al, Bh, Bl, kblock, nslices, nearest=True)
        Ch, Cl = gpu.dd_gemm(dA, dAl, dB, dBl, nslices=nslices, kblock=kblock)
        assert _bits_equal(_host(Ch), Rh) and _bits_equal(_host(Cl), Rl), kblock


def test_kblocked_strided_operands_and_null_lo(gpu):
    """k-blocks step through strided operands (lda > k, ldb > n) by pointer
    offsets; the result equals the oracle's blocked chain bit for bit, with and
    without lo planes, and the output's padding stays untouched."""
    import torch
    rng = np.random.default_rng(808)
    m, n, k, kblock = 50, 41, 97, 30
    Ah, Al = _edge_matrix(rng, m, k)
    Bh, Bl = _edge_matrix(rng, k, n)
    wideA = torch.zeros((2, m, k + 9), dtype=torch.float64, device="cuda")
    wideB = torch.zeros((2, k, n + 4), dtype=torch.float64, device="cuda")
    wideA[0, :, 3:3 + k], wideA[1, :, 3:3 + k] = _dev(Ah), _dev(Al)
    wideB[0, :, 1:1 + n], wideB[1, :, 1:1 + n] = _dev(Bh), _dev(Bl)
    vA = [wideA[c, :, 3:3 + k] for c in range(2)]
    vB = [wideB[c, :, 1:1 + n] for c in range(2)]
    out = torch.full((2, m, n + 6), 9.0, dtype=torch.float64, device="cuda")
    Ch, Cl = out[0, :, :n], out[1, :, :n]
    gpu.dd_gemm(vA[0], vA[1], vB[0], vB[1], C_hi=Ch, C_lo=Cl, kblock=kblock)
    Rh, Rl = exact.sliced_product_kblocks(Ah, Al, Bh, Bl, kblock, 8, nearest=True)
    assert _bits_equal(_host(Ch.contiguous()), Rh) and _bits_equal(_host(Cl.contiguous()), Rl)
    assert (_host(out[:, :, n:]) == 9.0).all()
    gpu.dd_gemm(vA[0], None, vB[0], None, C_hi=Ch, C_lo=Cl, kblock=kblock)
    Zh, Zl = exact.sliced_product_kblocks(Ah, np.zeros_like(Al), Bh, np.zeros_like(Bl), kblock, 8, nearest=True)
    assert _bits_equal(_host(Ch.contiguous()), Zh) and _bits_equal(_host(Cl.contiguous()), Zl)


def test_kblocked_workload_within_tolerance(gpu, workload_operands):
    """dd4096_exp20 cut into four k-blocks of 1024: within the dd tolerance of the
    classical oracle on sampled entries."""
    Ah, Al, Bh, Bl = workload_operands("dd4096_exp20")
    rng = np.random.default_rng(11)
    qr = rng.integers(0, Ah.shape[0], 512)
    qc = rng.integers(0, Bh.shape[1], 512)
    Rh, Rl = native.dd_gemm_entries(Ah, Al, Bh, Bl, qr, qc)
    Ch, Cl = gpu.dd_gemm(_dev(Ah), _dev(Al), _dev(Bh), _dev(Bl), kblock=1024)
    hCh, hCl = _host(Ch), _host(Cl)
    err = np.abs((hCh[qr, qc] - Rh) + (hCl[qr, qc] - Rl))
    ratio = float((err / np.einsum("qk,kq->q", np.abs(Ah[qr]), np.abs(Bh[:, qc]))).max())
    _say(f"[parity] dd4096_exp20 in 4 k-blocks: max |C-C_ref|/(|A||B|) = {ratio:.3e}")
    assert ratio <= compare.TOL


def test_binding_rejects_a_host_or_mistyped_workspace(gpu):
    """A caller's workspace must be uint8 device memory on the operands' device;
    the binding raises before any library call."""
    import torch
    A = torch.ones((8, 8), dtype=torch.float64, device="cuda")
    need = gpu.workspace_size(8, 8, 8)
    with pytest.raises(ValueError, match="device tensor"):
        gpu.dd_gemm(A, None, A, None, workspace=torch.empty(need, dtype=torch.uint8))
    with pytest.raises(TypeError, match="uint8"):
        gpu.dd_gemm(A, None, A, None, workspace=torch.empty(need, dtype=torch.float64, device="cuda"))
    with pytest.raises(ValueError, match="device tensor"):
        gpu.qd_gemm([A], [A], workspace=torch.empty(gpu.qd_workspace_size(8, 8, 8), dtype=torch.uint8))
    with pytest.raises(ValueError, match="one device"):
        gpu.dd_gemm(A, None, A, None, C_hi=torch.empty((8, 8), dtype=torch.float64, device="meta"))
    C_hi, C_lo = gpu.dd_gemm(A, None, A, None, workspace=torch.empty(need, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(C_hi.cpu(), torch.full((8, 8), 8.0, dtype=torch.float64)) and not C_lo.any()



@pytest.mark.parametrize("with_lo", [True, False])
def test_one_pass_B_beside_two_pass_A(gpu, with_lo):
    """A product whose B is sliced in one pass and whose A takes two passes
    (600 x 160 x 1000): A's exponents from the leading words, its rows holding
    an unnormalised pair recomputed by the exact pass.  A is an unaligned
    window of a wider matrix (odd offset and leading dimension: no 16-byte
    loads), with unnormalised pairs planted in its rows, or with no trailing
    words.  The product equals the oracle's nearest chain bit for bit on
    sampled rows and columns (planted ones included) and the call on
    contiguous operands."""
    import torch
    m, n, k = 600, 160, 1000
    rng = np.random.default_rng(600 + with_lo)
    Ah, Al = _edge_matrix(rng, m, k)
    Bh, Bl = _edge_matrix(rng, k, n)
    planted = [0, 37, 300, m - 1]
    Ah[37] *= 2.0 ** -8
    Al[37] *= 2.0 ** -8
    Ah[37, 5], Al[37, 5] = 1.0, -0.75        # exponent down
    Ah[300, 999], Al[300, 999] = 0.0, 3.0     # exponent up
    Ah[m - 1, 0], Al[m - 1, 0] = 2.0 ** -30, 2.0 ** 20
    if not with_lo:
        Al = np.zeros_like(Ah)
    assert Bh.nbytes + Bl.nbytes <= 24 << 20 and Ah.nbytes + Al.nbytes > 2 << 20  # B one pass, A two
    Abig = torch.zeros((2, m, k + 3), dtype=torch.float64, device="cuda")
    Abig[0, :, 1:k + 1] = _dev(Ah)
    Abig[1, :, 1:k + 1] = _dev(Al)
    a_lo = Abig[1, :, 1:k + 1] if with_lo else None
    rows = np.union1d(planted, _sample_indices(rng, m, 6))
    cols = _sample_indices(rng, n, 6)
    E_s, DA = exact.slice_rows(Ah, Al, rows)
    F_s, DB = exact.slice_cols(Bh, Bl, cols)
    if with_lo:
        Eh = exact.balancing_exponents(Ah[rows], np.zeros_like(Ah[rows]), 0)
        assert np.any(Eh != E_s), "some planted pair moves its row's exponent"
    _say(f"[parity] one-pass B beside two-pass A: {m}x{n}x{k}, lo {with_lo}")
    Ch, Cl = gpu.dd_gemm(Abig[0, :, 1:k + 1], a_lo, _dev(Bh), _dev(Bl))
    Nh_ref, Nl_ref = exact.nearest_dd(exact.level_sums_units(DA, DB), E_s, F_s)
    hCh, hCl = _host(Ch), _host(Cl)
    assert _bits_equal(hCh[np.ix_(rows, cols)], Nh_ref) and _bits_equal(hCl[np.ix_(rows, cols)], Nl_ref)
    Rh, Rl = gpu.dd_gemm(_dev(Ah), _dev(Al) if with_lo else None, _dev(Bh), _dev(Bl))
    assert _bits_equal(hCh, _host(Rh)) and _bits_equal(hCl, _host(Rl))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("size", [1280, 1024])
def test_product_recomputes_rows_and_columns_with_unnormalised_pairs(gpu, size):
    """The product entry points take a row's (column's) balancing exponent from
    the leading words when both operands are sliced in two passes; a row or
    column holding a pair whose leading word is not RN(hi + lo) is recomputed
    from (hi, lo) ("Multiple Double Arithmetic on NVIDIA Tensor Cores", §3,
    balancing; Problems 3.3 and 3.4 for opposite signs and leading zeros).
    1280^3 takes that path for both operands, 1024^3 for A beside a B
    sliced in one pass.
    Pairs planted in some rows of A and columns of B move the exact exponent
    up or down from the leading words' one, or leave it.  The product equals
    the oracle's nearest chain bit for bit on those rows and columns and on
    sampled others, and the stage call's exponents equal the oracle's."""
    import torch
    m = n = k = size
    rng = np.random.default_rng(size)
    Ah, Al = _edge_matrix(rng, m, k)
    Bh, Bl = _edge_matrix(rng, k, n)
    # A rows: r0 exponent down (1 - 0.75 = 0.25 the largest), r1 a zero leading
    # word with a large trailing one (exponent up), r2 |lo| >> |hi| on a 16-row
    # block boundary, r3 an unnormalised pair that leaves the exponent
    r0, r1, r2, r3 = 37, 600, 1023, m - 1
    Ah[r0] *= 2.0 ** -8
    Al[r0] *= 2.0 ** -8
    Ah[r0, 5], Al[r0, 5] = 1.0, -0.75
    Ah[r1, 700], Al[r1, 700] = 0.0, 3.0
    Ah[r2, 0], Al[r2, 0] = 2.0 ** -30, 2.0 ** 20
    Ah[r3, 9], Al[r3, 9] = 2.0 ** -40, -2.0 ** -45
    # B columns the same way
    c0, c1, c2, c3 = 16, 400, n - 180, n - 1
    Bh[:, c0] *= 2.0 ** -8
    Bl[:, c0] *= 2.0 ** -8
    Bh[3, c0], Bl[3, c0] = -1.0, 0.75
    Bh[k - 1, c1], Bl[k - 1, c1] = 0.0, -5.0
    Bh[640, c2], Bl[640, c2] = -2.0 ** -30, 2.0 ** 25
    Bh[11, c3], Bl[11, c3] = 2.0 ** -40, 2.0 ** -46 * 3
    # B sliced in two passes at 1280^3, in one pass at 1024^3
    assert (Bh.nbytes + Bl.nbytes > 24 << 20) == (size == 1280)
    rows = np.union1d([r0, r1, r2, r3], _sample_indices(rng, m, 6))
    cols = np.union1d([c0, c1, c2, c3], _sample_indices(rng, n, 6))
    E_s, DA = exact.slice_rows(Ah, Al, rows)
    F_s, DB = exact.slice_cols(Bh, Bl, cols)
    Eh = exact.balancing_exponents(Ah[rows], np.zeros_like(Ah[rows]), 0)
    assert np.any(Eh != E_s), "some planted pair moves its row's exponent"
    _say(f"[parity] unnormalised pairs: product {m}x{n}x{k}")
    Ch, Cl = gpu.dd_gemm(_dev(Ah), _dev(Al), _dev(Bh), _dev(Bl))
    Nh_ref, Nl_ref = exact.nearest_dd(exact.level_sums_units(DA, DB), E_s, F_s)
    hCh, hCl = _host(Ch), _host(Cl)
    assert _bits_equal(hCh[np.ix_(rows, cols)], Nh_ref) and _bits_equal(hCl[np.ix_(rows, cols)], Nl_ref)
    E, _ = gpu.split_balanced(_dev(Ah), _dev(Al), 0)
    F, _ = gpu.split_balanced(_dev(Bh), _dev(Bl), 1)
    assert np.array_equal(_host(E), exact.balancing_exponents(Ah, Al, 0))
    assert np.array_equal(_host(F), exact.balancing_exponents(Bh, Bl, 1))
