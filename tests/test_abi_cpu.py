"""Host-side checks of the C ABI: the library loads, exports every symbol the
header declares, sizes its buffers as documented and rejects bad arguments
before touching a device.  No GPU needed (no compute call is made)."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]


@pytest.fixture(scope="module")
def ddg():
    import extended_precision_gemm_amd as m
    return m


def _declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b((?:dd|qd)\w+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_boundary():
    names = _declared_functions()
    for required in ("dd_gemm", "dd_gemm_ws", "dd_gemm_workspace_size", "dd_split_balanced",
                     "dd_sliced_gemm", "dd_renorm_levels", "dd_sliced_gemm_renorm",
                     "ddgemm_status_string", "dd_split_slices_bytes", "qd_gemm", "qd_gemm_ws",
                     "qd_split_balanced", "qd_sliced_gemm_renorm", "qd_split_slices_bytes",
                     "qd_gemm_workspace_size", "qd_gemm_workspace_size_kb", "qd_gemm_ws_kb"):
        assert required in names


def test_library_exports_every_declared_symbol(ddg):
    raw = ctypes.CDLL(ddg.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(raw, name), name
    assert set(_declared_functions()) == set(ddg._SIGNATURES)


def test_library_links_no_oracle_code(ddg):
    raw = ctypes.CDLL(ddg.LIB_PATH)
    for name in ("oracle_dd_gemm", "oracle_two_sum", "oracle_dd_add"):
        assert not hasattr(raw, name)


def test_packed_sizes(ddg):
    assert ddg.slices_bytes(0, 10) == 0
    assert ddg.slices_bytes(10, 0) == 0
    assert ddg.slices_bytes(1, 1) == 64 * 16 * 8 * 8
    assert ddg.slices_bytes(129, 17) == 192 * 32 * 8 * 8
    assert ddg.slices_bytes(128, 17) == 128 * 32 * 8 * 8
    assert ddg.slices_bytes(4096, 4096) == 4096 * 4096 * 64
    assert ddg.slices_bytes(-1, 5) == 0
    m, n, k = 1000, 70, 33
    ws = ddg.workspace_size(m, n, k)
    r = lambda x: (x + 255) // 256 * 256
    assert ws == r(ddg.slices_bytes(m, k)) + r(ddg.slices_bytes(n, k)) + r(4 * m) + r(4 * n)
    assert ddg.workspace_size(-1, 2, 3) == 0
    # beyond the product's k-block limit (the int64 bound of the pair-packed
    # group sums, 2^22 for 8 slices) k is cut into the fewest equal blocks:
    # slices for one block, two m×n planes for the block results, seven int64
    # group-sum planes between k-chunks of 4096 and -- one 64x64 tile cannot
    # fill the chip -- seven int64 planes for each k-part of the split
    kmax = ddg.kblock_max(8)
    assert kmax == 1 << 22
    k2 = ddg.K_MAX + 1
    kb = -(-k2 // 3)
    parts = ddg.split_parts(3, 5, kb)
    assert parts > 1 and ddg.split_first_row(3, 5, kb) == 0
    assert ddg.workspace_size(3, 5, k2) == (r(ddg.slices_bytes(3, kb)) + r(ddg.slices_bytes(5, kb)) + r(12) + r(20)
                                            + 2 * r(3 * 5 * 8) + r(7 * 3 * 5 * 8) + r(parts * 7 * 3 * 5 * 8))
    assert ddg.workspace_size(3, 5, 100, kblock=100) == ddg.workspace_size(3, 5, 100)
    assert ddg.workspace_size(3, 5, 100, kblock=30) == (r(ddg.slices_bytes(3, 30)) + r(ddg.slices_bytes(5, 30))
                                                        + r(12) + r(20) + 2 * r(3 * 5 * 8))
    assert ddg.workspace_size(3, 5, 100, kblock=0) == 0
    assert ddg.workspace_size(3, 5, 100, kblock=kmax + 1) == 0
    assert ddg.workspace_size(3, 5, 100, kblock=kmax) == ddg.workspace_size(3, 5, 100)
    assert ddg.workspace_size(3, 5, 0, kblock=0) > 0


def test_split_parts_query(ddg):
    """The k-part count the product entry points use (host-only query): outputs
    whose 64x64 (32x64 for 6 and 9..16 slices) tiles fill whole rounds of 256
    workgroups never split; every part keeps at least one stage (a stage is 8
    values of k, 4 for 14..16 slices); at most 256 parts; invalid sizes give 0."""
    sp = ddg.split_parts
    for k in (64, 4096, 100000, ddg.K_MAX):
        assert sp(1024, 1024, k, 8) == 1 and sp(4096, 4096, k, 8) == 1 and sp(2048, 1024, k, 8) == 1
        assert sp(512, 1024, k, 16) == 1 and sp(256, 2048, k, 12) == 1
        assert sp(1024, 1024, k, 4) == 1 and sp(2048, 2048, k, 6) == 1 and sp(4096, 1024, k, 5) == 1
    for (m, n, k, ns) in [(1, 1, 10 ** 6, 8), (3, 5, 100000, 8), (64, 64, 2 ** 20, 16), (100, 80, 5000, 16),
                          (700, 900, 4096, 8), (1024, 512, 4096, 8), (40, 33, 3000, 16), (520, 1030, 900, 12)]:
        p = sp(m, n, k, ns)
        ks = 1 if ns >= 14 else 2
        stages = -(-k // 16) * 16 // 4 // ks
        assert 2 <= p <= min(256, stages), (m, n, k, ns, p)
    # one tile and a short k: the small-output kernel, not a split
    assert sp(64, 64, 240, 8) == 1 and ddg.small_product(64, 64, 240, 8)
    # one tile and a k beyond one exact chunk: one part per workgroup slot, one stage or more each
    assert sp(64, 64, 8192, 8) > 100
    assert sp(1024, 512, 4096, 8) == 2      # 128 tiles: one half-empty round becomes one full one
    assert sp(1, 1, 10 ** 6, 8) == 256
    assert sp(0, 5, 100, 8) == 1 and sp(5, 5, 0, 8) == 1
    assert sp(-1, 5, 100, 8) == 0 and sp(5, 5, 100, 3) == 0 and sp(5, 5, 100, 17) == 0
    # the split part starts at a whole tile row; the rows before it run unsplit
    fr = ddg.split_first_row
    for (m, n, k, ns) in [(1152, 1152, 1152, 8), (1536, 1024, 4096, 8), (2560, 1024, 4096, 8), (896, 896, 896, 16),
                          (960, 1280, 4096, 8), (700, 900, 4096, 8), (3, 5, 100000, 8), (1024, 1024, 4096, 8),
                          (1000, 1100, 700, 16), (520, 1030, 900, 12), (1280, 1280, 1024, 6)]:
        p, r = sp(m, n, k, ns), fr(m, n, k, ns)
        tm = 32 if ns == 6 or ns >= 9 else 64
        assert (r == m) == (p == 1), (m, n, k, ns)
        assert 0 <= r <= m and (r == m or r % tm == 0), (m, n, k, ns, r)
    assert fr(1024, 1024, 4096, 8) == 1024 and fr(4096, 4096, 4096, 8) == 4096
    assert fr(1536, 1024, 4096, 8) == 1024 and sp(1536, 1024, 4096, 8) == 2   # one full round, then 128 tiles in 2
    assert fr(3, 5, 100000, 8) == 0                                           # one tile: all of it split
    assert fr(-1, 5, 100, 8) == -1 and fr(5, 5, 100, 3) == -1


# the most values of k whose FP64 group sums of the pair-packed schedule stay exact
PAIR_CHUNK = {4: 8192, 5: 8176, 6: 5456, 7: 5456, 8: 4096, 9: 4080, 10: 3264, 11: 3264, 12: 2720, 13: 2720,
              14: 2336, 15: 2336, 16: 2048}


def test_workspace_holds_group_sum_planes_for_chunks_and_split_parts(ddg):
    """The double-double product's workspace: slices and exponents, plus n - 1
    int64 group-sum planes of m×n when k needs more than one exact FP64 chunk,
    plus n - 1 int64 planes of the split rows for every k-part of a split."""
    L = ddg.lib
    r = lambda x: (x + 255) // 256 * 256
    for (m, n, k, ns) in [(64, 64, 512, 8), (64, 64, 511, 8), (64, 64, 240, 8), (3, 5, 100000, 8),
                          (1000, 1000, 100000, 8), (700, 900, 4096, 8), (256, 256, 65536, 12),
                          (100, 80, 5000, 16), (64, 64, 1024, 6), (1024, 1024, 4096, 8),
                          (1536, 1024, 4096, 8), (1152, 1152, 1152, 8), (2048, 2048, 8192, 8)]:
        base = (r(L.dd_split_slices_bytes_ns(m, k, ns)) + r(L.dd_split_slices_bytes_ns(n, k, ns))
                + r(4 * m) + r(4 * n))
        chunks = r((ns - 1) * m * n * 8) if k > PAIR_CHUNK[ns] else 0
        parts = ddg.split_parts(m, n, k, ns)
        rows = m - ddg.split_first_row(m, n, k, ns)
        split = r(parts * (ns - 1) * rows * n * 8) if parts > 1 else 0
        assert L.dd_gemm_workspace_size_ns(m, n, k, ns) == base + chunks + split, (m, n, k, ns)
        if ns == 8:
            assert L.dd_gemm_workspace_size(m, n, k) == L.dd_gemm_workspace_size_ns(m, n, k, ns)
    assert ddg.split_parts(64, 64, 8192, 8) > 1 and ddg.split_parts(64, 64, 240, 8) == 1
    assert ddg.split_parts(1024, 1024, 4096, 8) == 1
    # quad double, one block within the pair-packed int64 bound (k <= 2^21): the
    # same group-sum planes with 16 slices -- 15 chunk planes beyond k = 2048,
    # 15 part planes per k-part of a split
    for (m, n, k) in [(64, 64, 300), (64, 64, 100000), (2048, 2048, 4096), (50, 40, 30), (896, 896, 896)]:
        base = r(L.qd_split_slices_bytes(m, k)) + r(L.qd_split_slices_bytes(n, k)) + r(4 * m) + r(4 * n)
        chunks = r(15 * m * n * 8) if k > PAIR_CHUNK[16] else 0
        parts = ddg.split_parts(m, n, k, 16)
        rows = m - ddg.split_first_row(m, n, k, 16)
        split = r(parts * 15 * rows * n * 8) if parts > 1 else 0
        assert L.qd_gemm_workspace_size(m, n, k) == base + chunks + split, (m, n, k)
        assert parts == ddg.split_parts(m, n, k, 12 + 4)  # the dd product with 16 slices plans alike
    assert ddg.split_parts(64, 64, 300, 16) > 1 and ddg.split_parts(2048, 2048, 4096, 16) == 1
    # beyond it, sixteen double level planes for a split (32x64 tiles, 4 values of k per stage)
    m, n, k = 64, 64, (1 << 21) + 4
    base = r(L.qd_split_slices_bytes(m, k)) + r(L.qd_split_slices_bytes(n, k)) + r(4 * m) + r(4 * n)
    parts = ddg.split_parts(m, n, k, 16)
    assert parts > 1 and L.qd_gemm_workspace_size(m, n, k) == base + r(16 * m * n * 8)
    # a blocked quad-double product whose blocks split: int64 planes and double planes
    m, n, k, kb = 40, 33, 3000, 1000
    assert ddg.split_parts(m, n, kb, 16) > 1
    base = r(L.qd_split_slices_bytes(m, kb)) + r(L.qd_split_slices_bytes(n, kb)) + r(4 * m) + r(4 * n)
    assert L.qd_gemm_workspace_size_kb(m, n, k, kb) == base + 2 * r(16 * m * n * 8)


def test_small_product_query(ddg):
    """Small outputs with a short k take the small-output kernel and never
    split; a k beyond one exact chunk, many output blocks or bad sizes do not."""
    for (m, n, k, ns) in [(64, 64, 64, 8), (1, 1, 1, 8), (100, 100, 100, 8), (16, 16, 16, 4), (48, 80, 60, 16)]:
        assert ddg.small_product(m, n, k, ns) and ddg.split_parts(m, n, k, ns) == 1
    assert not ddg.small_product(64, 64, PAIR_CHUNK[8] + 1, 8)        # beyond one exact FP64 chunk
    assert not ddg.small_product(48, 80, PAIR_CHUNK[16] + 1, 16)
    assert not ddg.small_product(272, 272, 64, 8)                      # 289 blocks of 16x16
    assert not ddg.small_product(4096, 4096, 4096, 8)
    assert not ddg.small_product(128, 128, 1024, 8)  # 64 k-blocks a wave: the split is modelled faster
    assert not ddg.small_product(-1, 4, 4, 8) and not ddg.small_product(4, 4, 4, 3)
    assert not ddg.small_product(0, 4, 4, 8) and not ddg.small_product(4, 4, 0, 8)


def test_status_strings(ddg):
    for code in range(5):
        s = ddg.status_string(code)
        assert s.startswith("DDGEMM_")
    assert "unknown" in ddg.status_string(99)


# Fake device addresses: never dereferenced, since every call below fails validation.
P = [0x10000000 * (i + 1) for i in range(8)]


def test_gemm_argument_validation(ddg):
    L = ddg.lib
    INV, WS = ddg.ERROR_INVALID_VALUE, ddg.ERROR_WORKSPACE
    ok = dict(m=4, n=5, k=6, A_hi=P[0], A_lo=P[1], lda=6, B_hi=P[2], B_lo=P[3], ldb=5,
              C_hi=P[4], C_lo=P[5], ldc=5)

    def call(**kw):
        a = dict(ok, **kw)
        return L.dd_gemm_ws(a["m"], a["n"], a["k"], a["A_hi"], a["A_lo"], a["lda"], a["B_hi"], a["B_lo"],
                            a["ldb"], a["C_hi"], a["C_lo"], a["ldc"], kw.get("ws", P[6]),
                            kw.get("ws_bytes", 0), None)

    assert call(m=-1) == INV
    assert call(n=-1) == INV
    assert call(k=-1) == INV
    far = [(1 << 40) * (i + 1) for i in range(7)]             # extents of gigabytes must not overlap
    assert call(k=ddg.K_MAX + 1, lda=ddg.K_MAX + 1, A_hi=far[0], A_lo=far[1], B_hi=far[2], B_lo=far[3],
                C_hi=far[4], C_lo=far[5], ws=far[6]) == WS         # blocked: needs its workspace
    assert call(lda=5) == INV
    assert call(ldb=4) == INV
    assert call(ldc=4) == INV
    assert call(A_hi=None) == INV
    assert call(B_hi=None) == INV
    assert call(C_hi=None) == INV
    assert call(C_lo=None) == INV
    assert call(C_hi=P[0]) == INV            # C aliases A
    assert call(C_lo=P[2] + 8) == INV        # C overlaps B
    assert call(C_lo=P[4] + 16) == INV       # C_hi and C_lo overlap
    assert call(ws_bytes=10) == WS           # too small
    need = ddg.workspace_size(4, 5, 6)
    assert call(ws=P[6] + 8, ws_bytes=need) == WS   # misaligned
    # m = 0 or n = 0 is a successful no-op that needs no pointers at all
    assert L.dd_gemm_ws(0, 5, 6, None, None, 6, None, None, 5, None, None, 5, None, 0, None) == 0
    assert L.dd_gemm_ws(4, 0, 6, None, None, 6, None, None, 1, None, None, 1, None, 0, None) == 0
    assert L.dd_gemm(0, 0, 0, None, None, 1, None, None, 1, None, None, 1, None) == 0
    assert L.dd_gemm(3, 3, 3, P[0], None, 2, P[1], None, 3, P[2], P[3], 3, None) == INV


def test_stage_argument_validation(ddg):
    L = ddg.lib
    INV = ddg.ERROR_INVALID_VALUE
    assert L.dd_split_balanced(4, 4, P[0], None, 4, 2, P[1], P[2], None) == INV   # bad axis
    assert L.dd_split_balanced(4, 4, P[0], None, 3, 0, P[1], P[2], None) == INV   # ld < cols
    assert L.dd_split_balanced(4, 4, None, None, 4, 0, P[1], P[2], None) == INV   # NULL X
    assert L.dd_split_balanced(4, 4, P[0], None, 4, 1, None, P[2], None) == INV   # NULL exps
    assert L.dd_split_balanced(4, 4, P[0], None, 4, 1, P[1], None, None) == INV   # NULL slices
    assert L.dd_split_balanced(ddg.K_MAX + 1, 1, P[0], None, 1, 1, P[1], P[2], None) == INV
    assert L.dd_split_balanced(0, 4, None, None, 4, 0, None, None, None) == 0      # empty
    assert L.dd_sliced_gemm(4, 4, 4, P[0], P[1], P[2], 3, None) == INV            # ldl < n
    assert L.dd_sliced_gemm(4, 4, 4, None, P[1], P[2], 4, None) == INV
    assert L.dd_sliced_gemm(4, 4, 4, P[0], P[1], None, 4, None) == INV
    assert L.dd_renorm_levels(4, 4, P[0], 4, P[1], P[2], P[3], P[3], 4, None) == INV  # C_hi == C_lo
    assert L.dd_renorm_levels(4, 4, P[0], 4, None, P[2], P[3], P[4], 4, None) == INV
    assert L.dd_sliced_gemm_renorm(4, 4, 4, P[0], P[1], P[2], P[3], P[4], P[5], 3, None) == INV
    assert L.ddgemm_probe_mfma_f64(None, None) == INV
    assert L.ddgemm_probe_pair_round(-1, 8, P[0], P[1], P[2], None) == INV          # count < 0
    assert L.ddgemm_probe_pair_round(2 ** 38 + 1, 8, P[0], P[1], P[2], None) == INV
    assert L.ddgemm_probe_pair_round(4, 3, P[0], P[1], P[2], None) == INV           # slice count
    assert L.ddgemm_probe_pair_round(4, 17, P[0], P[1], P[2], None) == INV
    assert L.ddgemm_probe_pair_round(4, 8, None, P[1], P[2], None) == INV
    assert L.ddgemm_probe_pair_round(4, 8, P[0], P[1], None, None) == INV
    assert L.ddgemm_probe_pair_round(0, 8, None, None, None, None) == 0               # empty


def test_valid_call_without_gpu_reports_device_error(ddg):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    L = ddg.lib
    assert L.dd_split_balanced(4, 4, P[0], None, 4, 0, P[1], P[2], None) == ddg.ERROR_DEVICE


def test_leading_dimensions_whose_extent_would_overflow_are_rejected(ddg):
    """rows x ld must stay within the 2^58-element size bound, so the extent and
    byte arithmetic behind the overlap checks cannot overflow."""
    L = ddg.lib
    INV = ddg.ERROR_INVALID_VALUE
    huge = 1 << 62
    assert L.dd_gemm_ws(3, 4, 5, P[0], None, huge, P[1], None, 4, P[2], P[3], 4, P[4], 1 << 30, None) == INV
    assert L.dd_gemm_ws(3, 4, 5, P[0], None, 5, P[1], None, huge, P[2], P[3], 4, P[4], 1 << 30, None) == INV
    assert L.dd_gemm_ws(3, 4, 5, P[0], None, 5, P[1], None, 4, P[2], P[3], huge, P[4], 1 << 30, None) == INV
    assert L.dd_gemm(3, 4, 5, P[0], None, huge, P[1], None, 4, P[2], P[3], 4, None) == INV
    assert L.dd_split_balanced(3, 4, P[0], None, huge, 0, P[1], P[2], None) == INV
    assert L.dd_sliced_gemm(3, 4, 5, P[0], P[1], P[2], huge, None) == INV
    assert L.dd_renorm_levels(3, 4, P[0], huge, P[1], P[2], P[3], P[4], 4, None) == INV
    assert L.dd_renorm_levels(3, 4, P[0], 4, P[1], P[2], P[3], P[4], huge, None) == INV
    assert L.dd_sliced_gemm_renorm(3, 4, 5, P[0], P[1], P[2], P[3], P[4], P[5], huge, None) == INV
    A, B = _arr(P[0]), _arr(P[1])
    C = _arr(P[2], P[2] + 4096, P[2] + 8192, P[2] + 12288)
    assert L.qd_gemm_ws(3, 4, 5, A, 5, B, huge, C, 4, P[4], 1 << 30, None) == INV
    assert L.qd_gemm_ws_kb(3, 4, 5, 2, A, huge, B, 4, C, 4, P[4], 1 << 30, None) == INV
    assert L.qd_split_balanced(3, 4, A, huge, 0, P[1], P[2], None) == INV
    # the bound is rows x ld <= 2^58, whatever the row count
    assert L.dd_split_balanced(1, 4, P[0], None, huge, 0, P[1], P[2], None) == INV
    assert L.dd_split_balanced(1, 4, P[0], None, 1 << 58, 0, P[1], P[2], None) in (ddg.ERROR_DEVICE, 0)


def test_workspaces_past_2_62_bytes_are_rejected(ddg):
    """Sizes within the 2^58-element bound whose workspace would not fit 64-bit
    byte counts (sixteen m x n level planes of 8 bytes at m n = 2^58: 2^65
    bytes) have no workspace size (0), and the products reject them before any
    device call instead of accepting a wrapped-around size."""
    L = ddg.lib
    INV = ddg.ERROR_INVALID_VALUE
    m = n = 1 << 29
    assert L.qd_gemm_workspace_size(m, n, ddg.QD_K_MAX + 1) == 0
    assert L.dd_gemm_workspace_size(m, n, ddg.K_MAX + 1) == 0
    assert L.dd_gemm_workspace_size(m >> 4, n, ddg.K_MAX + 1) > 1 << 58
    # disjoint operands: A, B at 2^56, 2^57 (2^55 bytes each), output planes of 2^61 bytes from 2^61 on
    k = ddg.K_MAX + 1
    A, B, Ch, Cl = 1 << 56, 1 << 57, 1 << 61, 1 << 62
    assert L.dd_gemm_ws(m, n, k, A, None, k, B, None, n, Ch, Cl, n, P[0], 1 << 30, None) == INV
    assert L.dd_gemm(m, n, k, A, None, k, B, None, n, Ch, Cl, n, None) == INV
    kq = ddg.QD_K_MAX + 1
    C = _arr(1 << 61, 1 << 62, 3 << 61, 1 << 63)
    assert L.qd_gemm_ws(m, n, kq, _arr(A), kq, _arr(B), n, C, n, P[0], 1 << 30, None) == INV
    assert L.qd_gemm(m, n, kq, _arr(A), kq, _arr(B), n, C, n, None) == INV


def test_layout_pack_unpack_roundtrip(ddg):
    from extended_precision_gemm_amd import layout
    rng = np.random.default_rng(0)
    for outer, k in [(1, 1), (17, 5), (130, 33), (128, 16)]:
        planes = rng.standard_normal((8, outer, k))
        packed = layout.pack(planes, outer, k)
        assert packed.size * 8 == ddg.slices_bytes(outer, k)
        assert np.array_equal(layout.unpack(packed, outer, k), planes)
        # spot-check the documented index formula
        KB = layout.padded(outer, k)[1] // 4
        for (s, o, p) in [(0, 0, 0), (7, outer - 1, k - 1), (3, outer // 2, k // 2)]:
            idx = (((o // 16) * KB + p // 4) * 8 + s) * 64 + (p % 4) * 16 + (o % 16)
            assert packed[idx] == planes[s, o, p]


def _pair_term_max(n):
    """The largest group sum one value of k adds in the pair-packed schedule
    (digits 8191): packed products (2u, 2u+1) x t into group 2u + t, singles
    (2u + t = n - 1) into group n - 2."""
    d = 8191
    groups = [0] * (n - 1)
    for u in range((n + 1) // 2):
        for t in range(n):
            if 2 * u + 1 < n and 2 * u + 1 + t <= n - 1:
                groups[2 * u + t] += (d * 8192 + d) * d
            elif 2 * u + t == n - 1:
                groups[n - 2] += d * d
    return max(groups)


def test_n_slice_sizes_and_validation(ddg):
    L = ddg.lib
    INV = ddg.ERROR_INVALID_VALUE
    for n in range(ddg.MIN_SLICES, ddg.MAX_SLICES + 1):
        assert L.dd_split_slices_bytes_ns(130, 33, n) == 192 * 48 * n * 8
        kmax = ddg.k_max(n)
        assert kmax == (8388608 if n <= 8 else 67108865 // n)
        # the product's k-blocks: the smaller of the slicer's limit and the int64 bound of the group sums
        kbm = ddg.kblock_max(n)
        assert kbm == min(kmax, (2 ** 63 - 1) // _pair_term_max(n))
        assert L.dd_gemm_workspace_size_ns(4, 4, kbm, n) > 0
        assert L.dd_gemm_workspace_size_ns(4, 4, kbm + 1, n) == L.dd_gemm_workspace_size_kb(4, 4, kbm + 1, n,
                                                                                            (kbm + 2) // 2)
        assert L.dd_gemm_workspace_size_kb(4, 4, 10, n, kbm + 1) == 0
        assert L.dd_gemm_ws_kb(4, 4, 10, n, kbm + 1, P[0], None, 10, P[1], None, 4, P[2], P[3], 4, P[4], 1 << 30,
                               None) == INV
        assert L.dd_gemm_ws_kb(4, 4, 10, n, 0, P[0], None, 10, P[1], None, 4, P[2], P[3], 4, P[4], 1 << 30,
                               None) == INV
        assert L.dd_split_balanced_ns(4, kmax + 1, P[0], None, kmax + 1, 0, n, P[1], P[2], None) == INV
        assert L.dd_sliced_gemm_renorm_ns(4, 4, kmax + 1, n, P[0], P[1], P[2], P[3], P[4], P[5], 4, None) == INV
    assert L.dd_split_slices_bytes_ns(130, 33, 8) == ddg.slices_bytes(130, 33)
    assert L.dd_gemm_workspace_size_ns(100, 70, 33, 8) == ddg.workspace_size(100, 70, 33)
    assert L.dd_gemm_workspace_size_ns(100, 70, 33, 4) < ddg.workspace_size(100, 70, 33)
    assert L.dd_gemm_workspace_size_ns(100, 70, 33, 16) > ddg.workspace_size(100, 70, 33)
    for bad in (0, 3, 17, -1):
        assert L.dd_split_slices_bytes_ns(10, 10, bad) == 0
        assert L.dd_gemm_workspace_size_ns(10, 10, 10, bad) == 0
        assert L.dd_split_balanced_ns(4, 4, P[0], None, 4, 0, bad, P[1], P[2], None) == INV
        assert L.dd_sliced_gemm_renorm_ns(4, 4, 4, bad, P[0], P[1], P[2], P[3], P[4], P[5], 4, None) == INV
        assert L.dd_gemm_ws_ns(4, 5, 6, bad, P[0], P[1], 6, P[2], P[3], 5, P[4], P[5], 5, P[6], 1 << 20,
                               None) == INV
    # the suffixed entry points validate like their counterparts
    assert L.dd_gemm_ws_ns(4, 5, 6, 4, P[0], P[1], 5, P[2], P[3], 5, P[4], P[5], 5, P[6], 1 << 20, None) == INV
    assert L.dd_gemm_ws_ns(4, 5, 6, 4, P[0], P[1], 6, P[2], P[3], 5, P[4], P[5], 5, P[6], 10, None) == \
        ddg.ERROR_WORKSPACE
    assert L.dd_gemm_ws_ns(0, 5, 6, 4, None, None, 6, None, None, 5, None, None, 5, None, 0, None) == 0


def _arr(*ptrs):
    return (ctypes.c_void_p * 4)(*(list(ptrs) + [None] * (4 - len(ptrs))))


def test_qd_sizes(ddg):
    L = ddg.lib
    assert L.qd_split_slices_bytes(130, 33) == 192 * 48 * 16 * 8
    assert L.qd_split_slices_bytes(0, 33) == 0
    assert L.qd_split_slices_bytes(-1, 33) == 0
    r = lambda x: (x + 255) // 256 * 256
    m, n, k = 100, 70, 33
    assert L.qd_gemm_workspace_size(m, n, k) == (r(L.qd_split_slices_bytes(m, k)) + r(L.qd_split_slices_bytes(n, k))
                                                  + r(4 * m) + r(4 * n))
    assert L.qd_gemm_workspace_size(4, 4, ddg.QD_K_MAX) > 0
    assert ddg.QD_K_MAX == 67108865 // 16
    # k-blocks: slices of one block, and sixteen int64 m x n level planes when k needs two or more
    for kb in (1, 7, 32, 33):
        blocked = 16 * 8 * m * n if kb < k else 0
        assert L.qd_gemm_workspace_size_kb(m, n, k, kb) == (r(L.qd_split_slices_bytes(m, min(k, kb)))
                                                            + r(L.qd_split_slices_bytes(n, min(k, kb)))
                                                            + r(4 * m) + r(4 * n) + r(blocked))
    assert L.qd_gemm_workspace_size_kb(m, n, k, k) == L.qd_gemm_workspace_size(m, n, k)
    # beyond QD_K_MAX the default is the fewest equal blocks within it
    big = ddg.QD_K_MAX + 1
    assert L.qd_gemm_workspace_size(4, 4, big) == L.qd_gemm_workspace_size_kb(4, 4, big, (big + 1) // 2)
    assert L.qd_gemm_workspace_size(4, 4, 3 * ddg.QD_K_MAX) == \
        L.qd_gemm_workspace_size_kb(4, 4, 3 * ddg.QD_K_MAX, ddg.QD_K_MAX)
    assert L.qd_gemm_workspace_size(1, 1, ddg.QD_K_MAX_BLOCKED) > 0
    assert L.qd_gemm_workspace_size(1, 1, ddg.QD_K_MAX_BLOCKED + 1) == 0
    assert ddg.QD_K_MAX_BLOCKED == 1 << 32
    # the int64 level sums cannot overflow: |S_l| <= 16 k (2^13 - 1)^2 < 2^62 for k <= 2^32
    assert 16 * ddg.QD_K_MAX_BLOCKED * (2 ** 13 - 1) ** 2 < 2 ** 62
    for bad in (0, -1, ddg.QD_K_MAX + 1):
        assert L.qd_gemm_workspace_size_kb(m, n, k, bad) == 0
    assert L.qd_gemm_workspace_size_kb(m, n, 0, 0) > 0            # k = 0 takes no block size


def test_qd_argument_validation(ddg):
    L = ddg.lib
    INV, WS = ddg.ERROR_INVALID_VALUE, ddg.ERROR_WORKSPACE
    A, B, C = _arr(P[0], P[1]), _arr(P[2]), _arr(P[3], P[3] + 4096, P[3] + 8192, P[3] + 12288)
    need = L.qd_gemm_workspace_size(4, 5, 6)

    def gemm(m=4, n=5, k=6, A=A, lda=6, B=B, ldb=5, C=C, ldc=5, ws=P[6], ws_bytes=need):
        return L.qd_gemm_ws(m, n, k, A, lda, B, ldb, C, ldc, ws, ws_bytes, None)

    assert gemm(m=-1) == INV
    assert gemm(k=ddg.QD_K_MAX_BLOCKED + 1, lda=ddg.QD_K_MAX_BLOCKED + 1) == INV
    assert gemm(k=ddg.QD_K_MAX + 1, lda=ddg.QD_K_MAX + 1) == WS           # blocked: a bigger workspace
    assert gemm(lda=5) == INV
    assert gemm(ldb=4) == INV
    assert gemm(ldc=4) == INV
    assert gemm(A=None) == INV
    assert gemm(A=_arr(None, P[1])) == INV                                 # first component missing
    assert gemm(C=_arr(P[3], P[3] + 4096, None, P[3] + 12288)) == INV       # an output plane missing
    assert gemm(C=_arr(P[3], P[3] + 64, P[3] + 8192, P[3] + 12288)) == INV  # output planes overlap
    assert gemm(C=_arr(P[0], P[3] + 4096, P[3] + 8192, P[3] + 12288)) == INV  # C aliases A
    assert gemm(C=_arr(P[3], P[3] + 4096, P[3] + 8192, P[1] + 8)) == INV     # C overlaps A's x1
    assert gemm(ws_bytes=10) == WS
    assert gemm(ws=P[6] + 8) == WS
    assert gemm(m=0, A=None, B=None, C=None) == 0                           # empty: no-op
    assert L.qd_gemm(0, 5, 6, None, 6, None, 5, None, 5, None) == 0
    # the timed form checks the same arguments and the same workspace
    timed = lambda **kw: L.qd_gemm_ws_timed(kw.get("m", 4), 5, kw.get("k", 6), A, 6, B, 5, kw.get("C", C), 5,
                                            P[6], kw.get("ws_bytes", need), None, None)
    assert timed(m=-1) == INV and timed(k=-1) == INV and timed(ws_bytes=need - 1) == WS
    assert timed(C=_arr(P[0], P[3] + 4096, P[3] + 8192, P[3] + 12288)) == INV
    assert timed(m=0) == 0

    def gemm_kb(kb, m=4, n=5, k=6, ws_bytes=1 << 30):
        return L.qd_gemm_ws_kb(m, n, k, kb, A, max(k, 1), B, n, C, n, P[6], ws_bytes, None)

    assert gemm_kb(0) == INV
    assert gemm_kb(-3) == INV
    assert gemm_kb(ddg.QD_K_MAX + 1) == INV
    assert gemm_kb(2, ws_bytes=L.qd_gemm_workspace_size_kb(4, 5, 6, 2) - 1) == WS
    assert gemm_kb(0, m=0) == INV                                        # kblock is checked first
    assert gemm_kb(0, k=0, ws_bytes=0) == WS                             # k = 0: no block size needed
    assert L.qd_gemm(3, 3, 3, A, 3, B, 3, None, 3, None) == INV
    # stage calls
    assert L.qd_split_balanced(4, 4, A, 4, 2, P[4], P[5], None) == INV          # bad axis
    assert L.qd_split_balanced(4, 4, A, 3, 0, P[4], P[5], None) == INV          # ld < cols
    assert L.qd_split_balanced(4, 4, _arr(None), 4, 0, P[4], P[5], None) == INV
    assert L.qd_split_balanced(4, 4, A, 4, 0, None, P[5], None) == INV
    assert L.qd_split_balanced(4, 4, A, 4, 0, P[4], None, None) == INV
    assert L.qd_split_balanced(ddg.QD_K_MAX + 1, 1, A, 1, 1, P[4], P[5], None) == INV
    assert L.qd_split_balanced(0, 4, None, 4, 0, None, None, None) == 0
    assert L.qd_sliced_gemm_renorm(4, 4, 4, P[0], P[1], P[2], P[3], C, 3, None) == INV   # ldc < n
    assert L.qd_sliced_gemm_renorm(4, 4, 4, P[0], None, P[2], P[3], C, 4, None) == INV
    assert L.qd_sliced_gemm_renorm(4, 4, 4, P[0], P[1], P[2], P[3], None, 4, None) == INV


def test_qd_valid_call_without_gpu_reports_device_error(ddg):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert ddg.lib.qd_split_balanced(4, 4, _arr(P[0]), 4, 0, P[1], P[2], None) == ddg.ERROR_DEVICE
    L = ddg.lib
    C = _arr(P[3], P[3] + 4096, P[3] + 8192, P[3] + 12288)
    assert L.qd_gemm_ws_kb(4, 5, 6, 2, _arr(P[0]), 6, _arr(P[2]), 5, C, 5, P[6],
                           L.qd_gemm_workspace_size_kb(4, 5, 6, 2), None) == ddg.ERROR_DEVICE
    assert L.qd_gemm_ws_timed(4, 5, 6, _arr(P[0]), 6, _arr(P[2]), 5, C, 5, P[6], L.qd_gemm_workspace_size(4, 5, 6),
                              None, None) == ddg.ERROR_DEVICE


def test_binding_rejects_host_and_wrong_dtype_tensors(ddg):
    """The Python binding checks its tensors before any call into the library:
    float64 only, device memory only, 2-D planes, one to four qd components."""
    import torch
    a32 = torch.zeros((4, 4), dtype=torch.float32)
    a64 = torch.zeros((4, 4), dtype=torch.float64)
    with pytest.raises(TypeError, match="float64"):
        ddg.dd_gemm(a32, None, a64, None)
    with pytest.raises(ValueError, match="device tensor"):
        ddg.dd_gemm(a64, None, a64, None)
    with pytest.raises(ValueError, match="device tensor"):
        ddg.split_balanced(a64, None, 0)
    with pytest.raises(ValueError, match="one to four"):
        ddg.qd_gemm([a64] * 5, [a64])
    with pytest.raises(ValueError, match="one to four"):
        ddg.qd_gemm([None, a64], [a64])
    with pytest.raises(ValueError, match="device tensor"):
        ddg.qd_gemm(torch.zeros((4, 3, 3), dtype=torch.float64), [a64])


def test_binding_checks_devices_and_the_callers_workspace(ddg):
    """Operands and results of a product share one device, on which the call
    runs; a caller's workspace is a contiguous uint8 tensor on that device (a
    host buffer would hand the kernels a host pointer)."""
    import torch
    cpu = torch.device("cpu")
    with pytest.raises(ValueError, match="one device"):
        ddg._device(torch.zeros(1), None, torch.zeros(1, device="meta"))
    assert ddg._device(torch.zeros(1), None, torch.zeros(2)) == cpu
    with pytest.raises(TypeError, match="uint8"):
        ddg._workspace(torch.zeros(4, dtype=torch.float64), 8, cpu)
    with pytest.raises(ValueError, match="device tensor"):
        ddg._workspace(torch.zeros(8, dtype=torch.uint8), 8, torch.device("meta"))
    with pytest.raises(ValueError, match="contiguous"):
        ddg._workspace(torch.zeros(16, dtype=torch.uint8)[::2], 8, cpu)
    assert ddg._workspace(None, 0, torch.device("meta")).numel() == 1



def test_no_alloc_product_validation(ddg):
    """dd_gemm_noalloc checks its arguments like dd_gemm_ws and rejects products
    whose workspace exceeds its fixed device array before any device call."""
    L = ddg.lib
    INV, WS = ddg.ERROR_INVALID_VALUE, ddg.ERROR_WORKSPACE
    assert ddg.NOALLOC_SCRATCH_BYTES == 256 << 20
    assert L.dd_gemm_workspace_size(1024, 1024, 1024) <= ddg.NOALLOC_SCRATCH_BYTES
    far = [(1 << 40) * (i + 1) for i in range(6)]
    n = 2048
    assert L.dd_gemm_workspace_size(n, n, n) > ddg.NOALLOC_SCRATCH_BYTES
    assert L.dd_gemm_noalloc(n, n, n, far[0], far[1], n, far[2], far[3], n, far[4], far[5], n, None) == WS
    assert L.dd_gemm_noalloc(-1, 4, 4, P[0], None, 4, P[1], None, 4, P[2], P[3], 4, None) == INV
    assert L.dd_gemm_noalloc(4, 4, -1, P[0], None, 4, P[1], None, 4, P[2], P[3], 4, None) == INV
    assert L.dd_gemm_noalloc(4, 4, 4, P[0], None, 3, P[1], None, 4, P[2], P[3], 4, None) == INV   # lda < k
    assert L.dd_gemm_noalloc(4, 4, 4, None, None, 4, P[1], None, 4, P[2], P[3], 4, None) == INV
    assert L.dd_gemm_noalloc(4, 4, 4, P[0], None, 4, P[1], None, 4, P[0], P[3], 4, None) == INV   # C aliases A
    assert L.dd_gemm_noalloc(0, 4, 4, None, None, 4, None, None, 4, None, None, 4, None) == 0      # no-op
    import torch
    if not torch.cuda.is_available():
        assert L.dd_gemm_noalloc(4, 4, 4, P[0], None, 4, P[1], None, 4, P[2], P[3], 4, None) == ddg.ERROR_DEVICE


def test_workspace_sizes_of_operands_too_large_to_slice_are_rejected(ddg):
    """An operand whose packed slices cannot be sized (outer·k·n past the
    2^58-element bound) has no workspace: the size queries give 0 and the
    products reject the sizes, rather than leaving its slices out."""
    L = ddg.lib
    m, k = 1 << 35, 1 << 23
    assert L.dd_split_slices_bytes(m, k) == 0
    assert L.dd_gemm_workspace_size(m, 1, k) == 0
    assert L.qd_gemm_workspace_size(m, 1, 1 << 22) == 0
    far = [(1 << 62) + (i << 59) for i in range(4)]
    assert L.dd_gemm_ws(m, 1, k, 1 << 40, None, k, 1 << 41, None, 1, far[0], far[1], 1, P[0], 1 << 40,
                        None) == ddg.ERROR_INVALID_VALUE
    C = _arr(far[0], far[1], far[2], far[3])
    assert L.qd_gemm_ws(m, 1, 1 << 22, _arr(1 << 40), 1 << 22, _arr(1 << 41), 1, C, 1, P[0], 1 << 40,
                        None) == ddg.ERROR_INVALID_VALUE


def test_binding_checks_stage_call_buffers(ddg):
    """The stage calls check the slices, exponents and level planes they pass on:
    dtype, contiguity, device memory and length (a short or host buffer would
    reach the kernels as an out-of-bounds pointer)."""
    import torch
    m, n, k = 4, 5, 6
    f64 = lambda c: torch.zeros(c, dtype=torch.float64)
    i32 = lambda c: torch.zeros(c, dtype=torch.int32)
    As, Bs = f64(ddg.slices_bytes(m, k) // 8), f64(ddg.slices_bytes(n, k) // 8)
    with pytest.raises(ValueError, match="device tensor"):
        ddg.sliced_gemm(m, n, k, As, Bs)
    with pytest.raises(ValueError, match="device tensor"):
        ddg.sliced_gemm_renorm(m, n, k, As, i32(m), Bs, i32(n))
    with pytest.raises(TypeError, match="float64"):
        ddg.sliced_gemm(m, n, k, i32(10), Bs)
    with pytest.raises(ValueError, match=r"\(8, m, n\)"):
        ddg.renorm_levels(f64((7, m, n)), i32(m), i32(n))
    with pytest.raises(ValueError, match="device tensor"):
        ddg.renorm_levels(f64((8, m, n)), i32(m), i32(n))
    with pytest.raises(ValueError, match="device tensor"):
        ddg.qd_sliced_gemm_renorm(m, n, k, f64(ddg.qd_slices_bytes(m, k) // 8), i32(m),
                                  f64(ddg.qd_slices_bytes(n, k) // 8), i32(n))
    # the checks themselves, on host tensors standing for device ones
    with pytest.raises(ValueError, match="needs at least"):
        _buffer_on_host(ddg, f64(3), torch.float64, 4)
    with pytest.raises(ValueError, match="contiguous"):
        _buffer_on_host(ddg, f64(8)[::2], torch.float64, 4)
    with pytest.raises(TypeError, match="int32"):
        _buffer_on_host(ddg, f64(8), torch.int32, 4)
    assert _buffer_on_host(ddg, i32(8), torch.int32, 8).numel() == 8


def _buffer_on_host(ddg, t, dtype, numel):
    """ddg._buffer with the device-memory check lifted (host tensors stand in)."""
    import unittest.mock
    with unittest.mock.patch.object(type(t), "is_cuda", new=property(lambda self: True)):
        return ddg._buffer(t, "buf", dtype, numel, t.device)
