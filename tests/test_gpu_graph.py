"""The workspace entry points inside a captured HIP graph, and concurrent calls
from several host threads (GPU tests).

dd_gemm_ws and qd_gemm_ws allocate nothing and clear memory with a kernel, not
a memset, so a caller can capture them once and replay them with new operands
copied into the same buffers.  Every replay is checked bit for bit against an
eager call on the same inputs, with eager work and synchronisations between
the replays.
"""
import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def _bits(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy().view(np.int64)


def test_dd_gemm_ws_replays_in_a_graph(gpu):
    import torch
    m, n, k = 200, 150, 130
    dAh = torch.empty((m, k), dtype=torch.float64, device="cuda")
    dAl = torch.empty_like(dAh)
    dBh = torch.empty((k, n), dtype=torch.float64, device="cuda")
    dBl = torch.empty_like(dBh)
    Ch = torch.empty((m, n), dtype=torch.float64, device="cuda")
    Cl = torch.empty_like(Ch)
    ws = torch.empty(gpu.workspace_size(m, n, k), dtype=torch.uint8, device="cuda")

    def load(seed):
        ah, al = workloads.random_dd((m, k), seed, "signed_exp20")
        bh, bl = workloads.random_dd((k, n), seed + 1, "normal")
        for dst, src in ((dAh, ah), (dAl, al), (dBh, bh), (dBl, bl)):
            dst.copy_(_dev(src))

    load(10)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture (device check cached)
        gpu.dd_gemm(dAh, dAl, dBh, dBl, C_hi=Ch, C_lo=Cl, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gpu.dd_gemm(dAh, dAl, dBh, dBl, C_hi=Ch, C_lo=Cl, workspace=ws)
    for rep, seed in enumerate((10, 20, 20, 30, 10)):
        load(seed)
        Ch.fill_(float("nan"))
        Cl.fill_(float("nan"))
        graph.replay()
        Rh, Rl = gpu.dd_gemm(dAh, dAl, dBh, dBl)  # eager, its own outputs and workspace
        assert np.array_equal(_bits(Ch), _bits(Rh)), rep
        assert np.array_equal(_bits(Cl), _bits(Rl)), rep


def test_qd_gemm_ws_replays_in_a_graph(gpu):
    import torch
    m, n, k = 97, 130, 64
    dA = torch.empty((4, m, k), dtype=torch.float64, device="cuda")
    dB = torch.empty((4, k, n), dtype=torch.float64, device="cuda")
    C = torch.empty((4, m, n), dtype=torch.float64, device="cuda")
    ws = torch.empty(gpu.qd_workspace_size(m, n, k), dtype=torch.uint8, device="cuda")

    def load(seed):
        dA.copy_(_dev(workloads.random_qd((m, k), seed, "uniform")))
        dB.copy_(_dev(workloads.random_qd((k, n), seed + 1, "signed_exp20")))

    load(40)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        gpu.qd_gemm(dA, dB, C=C, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gpu.qd_gemm(dA, dB, C=C, workspace=ws)
    for rep, seed in enumerate((40, 50, 50, 60)):
        load(seed)
        C.fill_(float("nan"))
        graph.replay()
        R = gpu.qd_gemm(dA, dB)
        assert np.array_equal(_bits(C), _bits(R)), rep


def test_dd_gemm_ws_kb_replays_in_a_graph(gpu):
    """The k-blocked double-double product: the first block writes C, later
    blocks go to the workspace's block planes and are added by a kernel, so a
    replay over a workspace full of garbage still gives the eager result."""
    import torch
    m, n, k, kb = 90, 70, 130, 40
    dAh = torch.empty((m, k), dtype=torch.float64, device="cuda")
    dAl = torch.empty_like(dAh)
    dBh = torch.empty((k, n), dtype=torch.float64, device="cuda")
    dBl = torch.empty_like(dBh)
    Ch = torch.empty((m, n), dtype=torch.float64, device="cuda")
    Cl = torch.empty_like(Ch)
    ws = torch.empty(gpu.workspace_size(m, n, k, kblock=kb), dtype=torch.uint8, device="cuda")

    def load(seed):
        ah, al = workloads.random_dd((m, k), seed, "signed_exp20")
        bh, bl = workloads.random_dd((k, n), seed + 1, "normal")
        for dst, src in ((dAh, ah), (dAl, al), (dBh, bh), (dBl, bl)):
            dst.copy_(_dev(src))

    load(110)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        gpu.dd_gemm(dAh, dAl, dBh, dBl, C_hi=Ch, C_lo=Cl, workspace=ws, kblock=kb)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gpu.dd_gemm(dAh, dAl, dBh, dBl, C_hi=Ch, C_lo=Cl, workspace=ws, kblock=kb)
    for rep, seed in enumerate((110, 120, 120, 130)):
        load(seed)
        Ch.fill_(float("nan"))
        Cl.fill_(float("nan"))
        ws.fill_(0x5A)
        graph.replay()
        Rh, Rl = gpu.dd_gemm(dAh, dAl, dBh, dBl, kblock=kb)  # eager
        assert np.array_equal(_bits(Ch), _bits(Rh)), rep
        assert np.array_equal(_bits(Cl), _bits(Rl)), rep


def test_qd_gemm_ws_kb_replays_in_a_graph(gpu):
    """The k-blocked product: its int64 level planes are written by the first
    block's kernel (no clearing pass), so replays start from a clean state."""
    import torch
    m, n, k, kb = 70, 90, 100, 30
    dA = torch.empty((4, m, k), dtype=torch.float64, device="cuda")
    dB = torch.empty((4, k, n), dtype=torch.float64, device="cuda")
    C = torch.empty((4, m, n), dtype=torch.float64, device="cuda")
    ws = torch.empty(gpu.qd_workspace_size(m, n, k, kblock=kb), dtype=torch.uint8, device="cuda")

    def load(seed):
        dA.copy_(_dev(workloads.random_qd((m, k), seed, "signed_exp20")))
        dB.copy_(_dev(workloads.random_qd((k, n), seed + 1, "uniform")))

    load(70)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        gpu.qd_gemm(dA, dB, C=C, workspace=ws, kblock=kb)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gpu.qd_gemm(dA, dB, C=C, workspace=ws, kblock=kb)
    for rep, seed in enumerate((70, 80, 80, 90)):
        load(seed)
        C.fill_(float("nan"))
        ws.fill_(0xA5)                     # stale level planes must not leak into a replay
        graph.replay()
        R = gpu.qd_gemm(dA, dB)            # eager, one block
        assert np.array_equal(_bits(C), _bits(R)), rep


def test_concurrent_calls_from_threads_on_their_own_streams(gpu):
    """The entry points keep no per-call state in the library: products issued
    at the same time from several host threads, each on its own stream, equal
    the same products issued one after another."""
    import threading
    import torch
    jobs = []
    for t in range(4):
        m, n, k = 60 + 17 * t, 50 + 9 * t, 40 + 23 * t
        ah, al = workloads.random_dd((m, k), 900 + t, "signed_exp20")
        bh, bl = workloads.random_dd((k, n), 950 + t, "uniform")
        jobs.append(tuple(_dev(x) for x in (ah, al, bh, bl)))
    qa = _dev(workloads.random_qd((33, 70), 990, "uniform"))
    qb = _dev(workloads.random_qd((70, 41), 991, "uniform"))
    serial = [gpu.dd_gemm(*j) for j in jobs]
    serial_q = gpu.qd_gemm(qa, qb)
    torch.cuda.synchronize()
    results = [None] * (len(jobs) + 1)
    errors = []

    def run(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for _ in range(3):
                    out = gpu.dd_gemm(*jobs[i], stream=s) if i < len(jobs) else gpu.qd_gemm(qa, qb, stream=s)
            s.synchronize()
            results[i] = out
        except Exception as exc:  # reported below
            errors.append(exc)

    threads = [threading.Thread(target=run, args=(i,)) for i in range(len(jobs) + 1)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors
    for i, (Sh, Sl) in enumerate(serial):
        Ch, Cl = results[i]
        assert np.array_equal(_bits(Ch), _bits(Sh)) and np.array_equal(_bits(Cl), _bits(Sl)), i
    assert np.array_equal(_bits(results[-1]), _bits(serial_q))
