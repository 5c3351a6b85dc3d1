"""Products split over k (GPU tests).

Outputs whose tiles leave the chip partly idle (a few output tiles and a long
k, or a last round of workgroups far from full) are computed in k-parts.  The
double-double product runs the pair-packed schedule: each part stores the
exact int64 group sums of its outputs in planes of its own, and one more
launch adds the parts and rounds each entry's exact total to the nearest
double-double -- no atomics.  Exact integer sums make the split result equal,
bit for bit, the oracle's chain on the same inputs, the nearest rounding of the
unsplit group sums (dd_sliced_gemm_pairs), and itself on every repetition; the
path must also replay in a HIP graph.  The level stage call (dd_sliced_gemm)
and the quad-double product split into level planes with exact atomic adds.
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


def _nearest_of_groups(G, E, F):
    """(hi, lo) = (RN(x), RN(x - hi)) for x = 2^(E_i + F_j) sum_g G_g 2^(-13(g+3)), from
    int64 group sums, with Python's correctly rounded int -> float conversion;
    for results in the normal range (the inputs here keep them there)."""
    import math
    ng, m, n = G.shape
    hi = np.empty((m, n))
    lo = np.empty((m, n))
    for i in range(m):
        for j in range(n):
            T = 0
            for g in range(ng):
                T += int(G[g, i, j]) << (13 * (ng - 1 - g))
            h = float(T)
            r = T - int(h)
            sc = int(E[i]) + int(F[j]) - 13 * (ng + 2)
            hi[i, j] = math.ldexp(h, sc)
            lo[i, j] = math.ldexp(float(r), sc)
    return hi, lo


def _unsplit_reference(gpu, dAh, dAl, dBh, dBl, ns):
    """The nearest double-double of the unsplit group sums (one launch, no parts)."""
    m, k = dAh.shape
    n = dBh.shape[1]
    E, As = gpu.split_balanced(dAh, dAl, 0, nslices=ns)
    F, Bs = gpu.split_balanced(dBh, dBl, 1, nslices=ns)
    G = _host(gpu.sliced_gemm_pairs(m, n, k, As, Bs, nslices=ns))
    return _nearest_of_groups(G, _host(E), _host(F))


@pytest.mark.parametrize("m,n,k,ns", [(64, 64, 8192, 8), (40, 70, 3000, 8), (3, 5, 100000, 8),
                                      (100, 80, 5000, 16), (64, 64, 2048, 6), (33, 130, 4100, 12)])
def test_split_dd_product_equals_the_unsplit_chain(gpu, m, n, k, ns):
    assert gpu.split_parts(m, n, k, ns) > 1
    _say(f"[split-k dd] {m}x{n}x{k} nslices={ns} parts={gpu.split_parts(m, n, k, ns)}")
    Ah, Al = workloads.random_dd((m, k), 9100 + k, "signed_exp20")
    Bh, Bl = workloads.random_dd((k, n), 9101 + k, "uniform")
    dAh, dAl, dBh, dBl = _dev(Ah), _dev(Al), _dev(Bh), _dev(Bl)
    Ch, Cl = gpu.dd_gemm(dAh, dAl, dBh, dBl, nslices=ns)
    Rh, Rl = exact.paired_product(Ah, Al, Bh, Bl, ns)
    assert _bits_equal(_host(Ch), Rh) and _bits_equal(_host(Cl), Rl)
    # the unsplit group sums round to the same bits
    Uh, Ul = _unsplit_reference(gpu, dAh, dAl, dBh, dBl, ns)
    assert _bits_equal(Uh, Rh) and _bits_equal(Ul, Rl)
    # and the split is deterministic
    for _ in range(2):
        Dh, Dl = gpu.dd_gemm(dAh, dAl, dBh, dBl, nslices=ns)
        assert _bits_equal(_host(Dh), Rh) and _bits_equal(_host(Dl), Rl)


@pytest.mark.parametrize("m,n,k,ns", [(512, 512, 32768, 8), (512, 512, 20000, 16)])
def test_split_parts_longer_than_an_exact_chunk(gpu, m, n, k, ns):
    """k-parts longer than the exact FP64 range of the group sums (4096 values
    of k with 8 slices, 2048 with 16): each part moves its group sums to int64
    inside the part, after the products a stage defers past the next barrier.
    The product equals the unsplit stage call's group sums rounded, bit for
    bit, and the oracle's nearest chain on sampled rows and columns."""
    chunk = {8: 4096, 16: 2048}[ns]
    parts = gpu.split_parts(m, n, k, ns)
    assert parts > 1 and k // parts > chunk
    _say(f"[split-k dd] {m}x{n}x{k} nslices={ns} parts={parts}: {k // parts} values of k a part")
    Ah, Al = workloads.random_dd((m, k), 9300 + ns, "signed_exp20")
    Bh, Bl = workloads.random_dd((k, n), 9301 + ns, "uniform")
    dAh, dAl, dBh, dBl = _dev(Ah), _dev(Al), _dev(Bh), _dev(Bl)
    Ch, Cl = gpu.dd_gemm(dAh, dAl, dBh, dBl, nslices=ns)
    hCh, hCl = _host(Ch), _host(Cl)
    Uh, Ul = _unsplit_reference(gpu, dAh, dAl, dBh, dBl, ns)
    assert _bits_equal(hCh, Uh) and _bits_equal(hCl, Ul)
    rng = np.random.default_rng(ns)
    rows = np.unique(np.concatenate([[0, m - 1], rng.integers(0, m, 5)]))
    cols = np.unique(np.concatenate([[0, n - 1], rng.integers(0, n, 5)]))
    E_s, DA = exact.slice_rows(Ah, Al, rows, nslices=ns)
    F_s, DB = exact.slice_cols(Bh, Bl, cols, nslices=ns)
    Nh, Nl = exact.nearest_dd(exact.level_sums_units(DA, DB), E_s, F_s)
    assert _bits_equal(hCh[np.ix_(rows, cols)], Nh) and _bits_equal(hCl[np.ix_(rows, cols)], Nl)


def test_split_level_planes_of_the_stage_call(gpu):
    """dd_sliced_gemm splits into the caller's level planes (zeroed first, so
    stale contents do not leak), with a row stride wider than n."""
    import torch
    m, n, k = 50, 60, 2500
    assert gpu.split_parts(m, n, k, 8) > 1
    Ah, Al = workloads.random_dd((m, k), 9201, "normal")
    Bh, Bl = workloads.random_dd((k, n), 9202, "signed_exp20")
    E, As = gpu.split_balanced(_dev(Ah), _dev(Al), 0)
    F, Bs = gpu.split_balanced(_dev(Bh), _dev(Bl), 1)
    ldl = n + 3
    levels = torch.full((8, m, ldl), 7.0, dtype=torch.float64, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    assert gpu.lib.dd_sliced_gemm(m, n, k, As.data_ptr(), Bs.data_ptr(), levels.data_ptr(), ldl, s) == 0
    _, DA = exact.slice_rows(Ah, Al)
    _, DB = exact.slice_cols(Bh, Bl)
    S_ref = exact.level_values(exact.level_sums_units(DA, DB))
    assert _bits_equal(_host(levels[:, :, :n].contiguous()), S_ref)
    assert (_host(levels[:, :, n:]) == 7.0).all()


@pytest.mark.parametrize("m,n,k", [(40, 33, 3000), (70, 64, 1500)])
def test_split_qd_product_equals_the_unsplit_chain(gpu, m, n, k):
    assert gpu.split_parts(m, n, k, 16) > 1
    _say(f"[split-k qd] {m}x{n}x{k} parts={gpu.split_parts(m, n, k, 16)}")
    A = workloads.random_qd((m, k), 9300 + k, "signed_exp20")
    B = workloads.random_qd((k, n), 9301 + k, "uniform")
    dA, dB = _dev(A), _dev(B)
    C = _host(gpu.qd_gemm(dA, dB))
    _, _, _, C_ref = qd.sliced_product(A, B)
    assert _bits_equal(C, C_ref)
    E, As = gpu.qd_split_balanced(dA, 0)
    F, Bs = gpu.qd_split_balanced(dB, 1)
    assert _bits_equal(_host(gpu.qd_sliced_gemm_renorm(m, n, k, As, E, Bs, F)), C_ref)
    assert _bits_equal(_host(gpu.qd_gemm(dA, dB)), C_ref)


@pytest.mark.parametrize("m,n,k,kblock", [(40, 33, 3000, 1000), (20, 20, 2500, 700), (50, 40, 1030, 1000)])
def test_blocked_qd_product_with_split_blocks_equals_the_unblocked_chain(gpu, m, n, k, kblock):
    """k-blocks of a quad-double product that are themselves split over k: each
    block's double level planes go into the int64 level planes; the short last
    block of the third case is too small to split and takes the unsplit path."""
    _say(f"[split-k qd blocks] {m}x{n}x{k} kblock={kblock}")
    A = workloads.random_qd((m, k), 9400 + k, "signed_exp20")
    B = workloads.random_qd((k, n), 9401 + k, "uniform")
    A[:, :, k // 2:] *= 2.0 ** -40            # blocks whose own exponents would differ
    C = _host(gpu.qd_gemm(_dev(A), _dev(B), kblock=kblock))
    _, _, _, C_ref = qd.sliced_product(A, B)
    assert _bits_equal(C, C_ref)


def test_split_products_replay_in_a_graph(gpu):
    """The split path zeroes its level planes with a kernel (no memset), so a
    captured product replays correctly over a workspace full of garbage."""
    import torch
    m, n, k = 64, 64, 2048
    assert gpu.split_parts(m, n, k, 8) > 1 and gpu.split_parts(m, n, k, 16) > 1
    dAh = torch.empty((m, k), dtype=torch.float64, device="cuda")
    dAl = torch.empty_like(dAh)
    dBh = torch.empty((k, n), dtype=torch.float64, device="cuda")
    dBl = torch.empty_like(dBh)
    qA = torch.empty((4, m, k), dtype=torch.float64, device="cuda")
    qB = torch.empty((4, k, n), dtype=torch.float64, device="cuda")
    Ch = torch.empty((m, n), dtype=torch.float64, device="cuda")
    Cl = torch.empty_like(Ch)
    Cq = torch.empty((4, m, n), dtype=torch.float64, device="cuda")
    ws = torch.empty(gpu.workspace_size(m, n, k), dtype=torch.uint8, device="cuda")
    wq = torch.empty(gpu.qd_workspace_size(m, n, k), dtype=torch.uint8, device="cuda")

    def load(seed):
        ah, al = workloads.random_dd((m, k), seed, "signed_exp20")
        bh, bl = workloads.random_dd((k, n), seed + 1, "normal")
        for dst, src in ((dAh, ah), (dAl, al), (dBh, bh), (dBl, bl)):
            dst.copy_(_dev(src))
        qA.copy_(_dev(workloads.random_qd((m, k), seed + 2, "uniform")))
        qB.copy_(_dev(workloads.random_qd((k, n), seed + 3, "signed_exp20")))

    def product():
        gpu.dd_gemm(dAh, dAl, dBh, dBl, C_hi=Ch, C_lo=Cl, workspace=ws)
        gpu.qd_gemm(qA, qB, C=Cq, workspace=wq)

    load(500)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        product()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        product()
    for rep, seed in enumerate((500, 510, 510, 520)):
        load(seed)
        for t in (Ch, Cl, Cq):
            t.fill_(float("nan"))
        ws.fill_(0x3C)
        wq.fill_(0x3C)
        graph.replay()
        Rh, Rl = gpu.dd_gemm(dAh, dAl, dBh, dBl)
        Rq = gpu.qd_gemm(qA, qB)
        assert _bits_equal(_host(Ch), _host(Rh)) and _bits_equal(_host(Cl), _host(Rl)), rep
        assert _bits_equal(_host(Cq), _host(Rq)), rep


@pytest.mark.parametrize("m,n,k,ns", [(700, 900, 4096, 8), (520, 1030, 900, 12), (1000, 1100, 700, 16),
                                      (1536, 1024, 2048, 8)])
def test_split_of_partly_idle_rounds(gpu, m, n, k, ns):
    """Outputs of 128 tiles and more whose last round of workgroups is partly
    idle: the split product equals the unsplit fused stage call on every entry
    and the oracle's chain on sampled rows and columns, bit for bit."""
    parts = gpu.split_parts(m, n, k, ns)
    assert parts > 1
    _say(f"[split-k rounds] {m}x{n}x{k} nslices={ns} parts={parts}")
    Ah, Al = workloads.random_dd((m, k), 9500 + m, "signed_exp20")
    Bh, Bl = workloads.random_dd((k, n), 9501 + n, "normal")
    dAh, dAl, dBh, dBl = _dev(Ah), _dev(Al), _dev(Bh), _dev(Bl)
    Ch, Cl = gpu.dd_gemm(dAh, dAl, dBh, dBl, nslices=ns)
    hCh, hCl = _host(Ch), _host(Cl)
    Uh, Ul = _unsplit_reference(gpu, dAh, dAl, dBh, dBl, ns)
    assert _bits_equal(hCh, Uh) and _bits_equal(hCl, Ul)
    rng = np.random.default_rng(m * n + k)
    rows = sorted({0, m - 1, *(int(x) for x in rng.integers(0, m, 5))})
    cols = sorted({0, n - 1, *(int(x) for x in rng.integers(0, n, 5))})
    E_ref, DA = exact.slice_rows(Ah, Al, rows, ns)
    F_ref, DB = exact.slice_cols(Bh, Bl, cols, ns)
    Rh, Rl = exact.nearest_dd(exact.level_sums_units(DA, DB), E_ref, F_ref)
    assert _bits_equal(hCh[np.ix_(rows, cols)], Rh) and _bits_equal(hCl[np.ix_(rows, cols)], Rl)


def test_qd_split_of_partly_idle_rounds(gpu):
    """A quad-double output of 192 tiles (32x64) split over k: bit-identical to
    the unsplit fused stage call everywhere and to the oracle on sampled entries."""
    import torch
    m, n, k = 768, 512, 2048
    parts = gpu.split_parts(m, n, k, 16)
    assert parts > 1
    _say(f"[split-k rounds qd] {m}x{n}x{k} parts={parts}")
    A = workloads.random_qd((m, k), 9601, "signed_exp20")
    B = workloads.random_qd((k, n), 9602, "uniform")
    dA, dB = _dev(A), _dev(B)
    C = _host(gpu.qd_gemm(dA, dB))
    E, As = gpu.qd_split_balanced(dA, 0)
    F, Bs = gpu.qd_split_balanced(dB, 1)
    assert _bits_equal(C, _host(gpu.qd_sliced_gemm_renorm(m, n, k, As, E, Bs, F)))
    del As, Bs
    torch.cuda.empty_cache()
    for i, j in [(0, 0), (m - 1, n - 1), (381, 17), (5, 500)]:
        Ei, DA = qd.slice_rows(A, rows=[i])
        Fj, DB = qd.slice_cols(B, cols=[j])
        ref = qd.renorm_levels(qd.level_sums(DA, DB), Ei, Fj)[:, 0, 0]
        assert _bits_equal(C[:, i, j], ref), (i, j)


def _sample(rng, size, must):
    return sorted({x for x in must if 0 <= x < size} | {int(x) for x in rng.integers(0, size, 4)})


@pytest.mark.parametrize("m,n,k,ns", [(1150, 1160, 1152, 8), (1536, 1024, 2048, 8), (1280, 1280, 1280, 6),
                                      (1300, 1300, 1300, 12), (2500, 2600, 900, 8), (1800, 1700, 1500, 8),
                                      (1300, 1700, 1100, 12)])
def test_split_of_the_last_rows_only(gpu, m, n, k, ns):
    """Plans that run whole rounds of leading tiles unsplit and split only the
    tiles from the plan's first split tile on -- from the start of a tile row,
    or from inside one (the rest of that row, then the rows below it, including
    a last tile row of only 8 rows): the product equals the unsplit fused stage
    call on every entry and the oracle's chain on sampled rows and columns on
    both sides of the first split tile, bit for bit."""
    r0, parts = gpu.split_first_row(m, n, k, ns), gpu.split_parts(m, n, k, ns)
    t0 = gpu.split_first_tile(m, n, k, ns)
    c0 = t0 % -(-n // 64) * 64
    assert 0 < r0 < m and parts > 1
    _say(f"[split tail] {m}x{n}x{k} nslices={ns} first split tile={t0} row={r0} col={c0} parts={parts}")
    Ah, Al = workloads.random_dd((m, k), 9700 + m, "signed_exp20")
    Bh, Bl = workloads.random_dd((k, n), 9701 + n, "normal")
    dAh, dAl, dBh, dBl = _dev(Ah), _dev(Al), _dev(Bh), _dev(Bl)
    Ch, Cl = gpu.dd_gemm(dAh, dAl, dBh, dBl, nslices=ns)
    hCh, hCl = _host(Ch), _host(Cl)
    Uh, Ul = _unsplit_reference(gpu, dAh, dAl, dBh, dBl, ns)
    assert _bits_equal(hCh, Uh) and _bits_equal(hCl, Ul)
    rng = np.random.default_rng(m + n + k + ns)
    rows = _sample(rng, m, [0, r0 - 1, r0, r0 + 1, m - 1])
    cols = _sample(rng, n, [0, c0 - 1, c0, n - 1])
    E_ref, DA = exact.slice_rows(Ah, Al, rows, ns)
    F_ref, DB = exact.slice_cols(Bh, Bl, cols, ns)
    Rh, Rl = exact.nearest_dd(exact.level_sums_units(DA, DB), E_ref, F_ref)
    assert _bits_equal(hCh[np.ix_(rows, cols)], Rh) and _bits_equal(hCl[np.ix_(rows, cols)], Rl)


@pytest.mark.parametrize("kblock", [1152, 1000])
def test_blocked_product_whose_blocks_split_their_last_rows(gpu, kblock):
    """A k-blocked product whose blocks split their last rows over k (the last,
    shorter block may plan differently or not split): sampled entries equal the
    oracle's blocked chain on the same rows and columns, bit for bit."""
    m, n, k = 1152, 1152, 2300
    assert 0 < gpu.split_first_row(m, n, kblock, 8) < m
    _say(f"[split tail blocks] {m}x{n}x{k} kblock={kblock}")
    Ah, Al = workloads.random_dd((m, k), 9801 + kblock, "uniform")
    Bh, Bl = workloads.random_dd((k, n), 9802 + kblock, "signed_exp20")
    Ch, Cl = gpu.dd_gemm(_dev(Ah), _dev(Al), _dev(Bh), _dev(Bl), kblock=kblock)
    hCh, hCl = _host(Ch), _host(Cl)
    rng = np.random.default_rng(kblock)
    r0 = gpu.split_first_row(m, n, kblock, 8)
    rows = _sample(rng, m, [0, r0 - 1, r0, m - 1])
    cols = _sample(rng, n, [0, n - 1])
    Rh, Rl = exact.sliced_product_kblocks(Ah[rows], Al[rows], Bh[:, cols], Bl[:, cols], kblock, 8, nearest=True)
    assert _bits_equal(hCh[np.ix_(rows, cols)], Rh) and _bits_equal(hCl[np.ix_(rows, cols)], Rl)


@pytest.mark.parametrize("m,n,k", [(800, 900, 700), (768, 768, 768), (1000, 1800, 700), (900, 1700, 1000)])
def test_qd_split_of_the_last_rows_only(gpu, m, n, k):
    """The quad-double product with only its last rows split over k: equal to
    the unsplit fused call everywhere and to the oracle on sampled entries."""
    import torch
    r0, parts = gpu.split_first_row(m, n, k, 16), gpu.split_parts(m, n, k, 16)
    assert 0 < r0 < m and parts > 1
    _say(f"[split tail qd] {m}x{n}x{k} first split row={r0} parts={parts}")
    A = workloads.random_qd((m, k), 9901 + m, "signed_exp20")
    B = workloads.random_qd((k, n), 9902 + n, "uniform")
    dA, dB = _dev(A), _dev(B)
    C = _host(gpu.qd_gemm(dA, dB))
    E, As = gpu.qd_split_balanced(dA, 0)
    F, Bs = gpu.qd_split_balanced(dB, 1)
    assert _bits_equal(C, _host(gpu.qd_sliced_gemm_renorm(m, n, k, As, E, Bs, F)))
    del As, Bs
    torch.cuda.empty_cache()
    c0 = gpu.split_first_tile(m, n, k, 16) % -(-n // 64) * 64
    for i, j in [(0, 0), (r0 - 1, n - 1), (r0, 3), (m - 1, n // 2), (r0, max(c0 - 1, 0)), (r0, c0), (m - 1, n - 1)]:
        Ei, DA = qd.slice_rows(A, rows=[i])
        Fj, DB = qd.slice_cols(B, cols=[j])
        ref = qd.renorm_levels(qd.level_sums(DA, DB), Ei, Fj)[:, 0, 0]
        assert _bits_equal(C[:, i, j], ref), (i, j)


def test_last_row_splits_and_row_exponent_parts_replay_in_a_graph(gpu):
    """Plans that run some rows unsplit and split the rest (head launch, plane
    zeroing, k-parts, renormalisation), and A operands with few long rows
    (row exponents in k-parts: fill, atomic maxima, decode), captured once and
    replayed over a garbage workspace with new inputs: every replay equals the
    eager product bit for bit."""
    import torch
    shapes = [(1150, 1160, 1152), (64, 64, 65536)]
    assert 0 < gpu.split_first_row(1150, 1160, 1152, 8) < 1150
    qm, qn, qk = 800, 900, 700
    assert 0 < gpu.split_first_row(qm, qn, qk, 16) < qm
    bufs = []
    for (m, n, k) in shapes:
        A = [torch.empty((m, k), dtype=torch.float64, device="cuda") for _ in range(2)]
        B = [torch.empty((k, n), dtype=torch.float64, device="cuda") for _ in range(2)]
        C = [torch.empty((m, n), dtype=torch.float64, device="cuda") for _ in range(2)]
        ws = torch.empty(gpu.workspace_size(m, n, k), dtype=torch.uint8, device="cuda")
        bufs.append((m, n, k, A, B, C, ws))
    qA = torch.empty((4, qm, qk), dtype=torch.float64, device="cuda")
    qB = torch.empty((4, qk, qn), dtype=torch.float64, device="cuda")
    qC = torch.empty((4, qm, qn), dtype=torch.float64, device="cuda")
    qws = torch.empty(gpu.qd_workspace_size(qm, qn, qk), dtype=torch.uint8, device="cuda")

    def load(seed):
        for i, (m, n, k, A, B, C, ws) in enumerate(bufs):
            ah, al = workloads.random_dd((m, k), seed + 10 * i, "signed_exp20")
            bh, bl = workloads.random_dd((k, n), seed + 10 * i + 1, "normal")
            for dst, src in ((A[0], ah), (A[1], al), (B[0], bh), (B[1], bl)):
                dst.copy_(_dev(src))
        qA.copy_(_dev(workloads.random_qd((qm, qk), seed + 7, "uniform")))
        qB.copy_(_dev(workloads.random_qd((qk, qn), seed + 8, "signed_exp20")))

    def product():
        for (m, n, k, A, B, C, ws) in bufs:
            gpu.dd_gemm(A[0], A[1], B[0], B[1], C_hi=C[0], C_lo=C[1], workspace=ws)
        gpu.qd_gemm(qA, qB, C=qC, workspace=qws)

    load(700)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        product()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        product()
    for rep, seed in enumerate((700, 720, 720, 740)):
        load(seed)
        for (m, n, k, A, B, C, ws) in bufs:
            C[0].fill_(float("nan"))
            C[1].fill_(float("nan"))
            ws.fill_(0x3C)
        qC.fill_(float("nan"))
        qws.fill_(0x3C)
        graph.replay()
        for (m, n, k, A, B, C, ws) in bufs:
            Rh, Rl = gpu.dd_gemm(A[0], A[1], B[0], B[1])
            assert _bits_equal(_host(C[0]), _host(Rh)) and _bits_equal(_host(C[1]), _host(Rl)), (rep, m, n, k)
        assert _bits_equal(_host(qC), _host(gpu.qd_gemm(qA, qB))), rep


@pytest.mark.parametrize("m,n,k,ns", [(64, 64, 64, 8), (1, 1, 1, 8), (17, 33, 5, 8), (100, 100, 100, 8),
                                      (250, 7, 100, 5), (16, 16, 16, 4), (48, 80, 60, 16), (200, 200, 64, 7),
                                      (130, 65, 33, 8), (256, 256, 256, 8)])
def test_small_products_equal_the_oracle(gpu, m, n, k, ns):
    """Products of a few outputs and a short k run as one 4-wave workgroup per
    16x16 output block whose waves split k and add their exact group sums
    through LDS: the nearest double-double of the exact total, as everywhere."""
    assert gpu.small_product(m, n, k, ns) and gpu.split_parts(m, n, k, ns) == 1
    _say(f"[small] {m}x{n}x{k} nslices={ns}")
    Ah, Al = workloads.random_dd((m, k), 9400 + k + m, "signed_exp20")
    Bh, Bl = workloads.random_dd((k, n), 9401 + k + n, "uniform")
    Ch, Cl = gpu.dd_gemm(_dev(Ah), _dev(Al), _dev(Bh), _dev(Bl), nslices=ns)
    Rh, Rl = exact.paired_product(Ah, Al, Bh, Bl, ns)
    assert _bits_equal(_host(Ch), Rh) and _bits_equal(_host(Cl), Rl)


def _edge_dd(rng, rows, cols):
    """A seeded (hi, lo) matrix with the slicer's edge entries: an all-zero row
    and column, an unnormalised pair, opposite signs, a negative zero,
    subnormals, and entries 2^-12 .. 2^2 apart."""
    hi = rng.uniform(-1, 1, (rows, cols)) * np.ldexp(1.0, rng.integers(-12, 3, (rows, cols)))
    lo_raw = hi * 2.0 ** -53 * rng.uniform(-1, 1, (rows, cols))
    s = hi + lo_raw
    lo = lo_raw - (s - hi)
    hi = s
    if rows > 2 and cols > 2:
        hi[1, :] = 0.0
        lo[1, :] = 0.0
        hi[:, 2] = 0.0
        lo[:, 2] = 0.0
        hi[0, 0], lo[0, 0] = 1.0, -0.75
        hi[0, 1], lo[0, 1] = 0.5, -2.0 ** -60
        hi[2, 0], lo[2, 0] = -0.0, 0.0
        hi[-1, -1], lo[-1, -1] = 2.0 ** -1074, 0.0
        hi[-1, 0], lo[-1, 0] = 3 * 2.0 ** -1060, -2.0 ** -1074
    return hi, lo


@pytest.mark.parametrize("m,n,k,ns", [(64, 64, 64, 8), (33, 17, 50, 8), (3, 40, 7, 8), (20, 20, 128, 6),
                                      (40, 24, 30, 12), (16, 48, 64, 16)])
def test_small_products_on_edge_entries(gpu, m, n, k, ns):
    """The small-output path (both operands sliced in one launch, then one
    4-wave workgroup per 16x16 block) with zero rows and columns, unnormalised
    pairs, opposite signs, negative zeros and subnormals in both operands: the
    product equals the oracle's pair-packed chain bit for bit."""
    assert gpu.small_product(m, n, k, ns)
    _say(f"[small edge] {m}x{n}x{k} nslices={ns}")
    rng = np.random.default_rng(7100 + m + n + k + ns)
    Ah, Al = _edge_dd(rng, m, k)
    Bh, Bl = _edge_dd(rng, k, n)
    Ch, Cl = gpu.dd_gemm(_dev(Ah), _dev(Al), _dev(Bh), _dev(Bl), nslices=ns)
    Rh, Rl = exact.paired_product(Ah, Al, Bh, Bl, ns)
    assert _bits_equal(_host(Ch), Rh) and _bits_equal(_host(Cl), Rl)


@pytest.mark.parametrize("m,n,k", [(64, 64, 64), (48, 80, 100), (16, 100, 40)])
def test_small_qd_products_equal_the_oracle(gpu, m, n, k):
    assert gpu.small_product(m, n, k, 16)
    _say(f"[small qd] {m}x{n}x{k}")
    A = workloads.random_qd((m, k), 9500 + k, "signed_exp20")
    B = workloads.random_qd((k, n), 9501 + k, "uniform")
    C = _host(gpu.qd_gemm(_dev(A), _dev(B)))
    _, _, _, C_ref = qd.sliced_product(A, B)
    assert _bits_equal(C, C_ref)
