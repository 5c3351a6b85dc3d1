"""dd_gemm_noalloc: the product entry point that allocates nothing, its
workspace being the library's own per-GPU device array.  Called through the C
ABI and compared bit for bit with dd_gemm_ws (the same kernels on a caller's
workspace), on consecutive calls whose later ones are smaller, so that they
run on what the earlier calls left in the array."""
import ctypes

import numpy as np
import pytest

import workloads


def _dd(shape, seed, dist):
    return workloads.random_dd(shape, seed, dist)


def _ws_product(ddg, dev, Ah, Al, Bh, Bl):
    import torch
    m, k = Ah.shape
    n = Bh.shape[1]
    ws = torch.empty(max(ddg.workspace_size(m, n, k), 1), dtype=torch.uint8, device=dev)
    return ddg.dd_gemm(Ah, Al, Bh, Bl, workspace=ws)


def _noalloc_product(ddg, Ah, Al, Bh, Bl, Ch, Cl):
    """One call straight through the C ABI (ctypes), outputs preallocated."""
    import torch
    m, k = Ah.shape
    n = Bh.shape[1]
    st = ddg.lib.dd_gemm_noalloc(m, n, k, Ah.data_ptr(), Al.data_ptr(), k, Bh.data_ptr(), Bl.data_ptr(), n,
                                 Ch.data_ptr(), Cl.data_ptr(), n,
                                 ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == ddg.SUCCESS, ddg.status_string(st)


@pytest.mark.gpu
def test_no_alloc_product_equals_the_workspace_product(gpu):
    import torch
    ddg = gpu
    dev = torch.device("cuda:0")
    # largest first, then smaller: a whole-tile shape, a product split over k
    # (level planes in the array), a ragged small one and a single tile
    cases = [((1024, 1024, 1024), "signed_exp20", 1), ((96, 80, 3000), "uniform", 2),
             ((333, 257, 190), "signed_exp20", 3), ((70, 45, 33), "uniform", 4)]
    for (m, n, k), dist, seed in cases:
        print(f"[no-alloc] m={m} n={n} k={k} {dist} seed={seed} parts={ddg.split_parts(m, n, k)}", flush=True)
        assert ddg.lib.dd_gemm_workspace_size(m, n, k) <= ddg.NOALLOC_SCRATCH_BYTES
        Ah, Al = (torch.from_numpy(x).to(dev) for x in _dd((m, k), 10 * seed, dist))
        Bh, Bl = (torch.from_numpy(x).to(dev) for x in _dd((k, n), 10 * seed + 1, dist))
        Rh, Rl = _ws_product(ddg, dev, Ah, Al, Bh, Bl)
        Ch = torch.full((m, n), float("nan"), dtype=torch.float64, device=dev)
        Cl = torch.full((m, n), float("nan"), dtype=torch.float64, device=dev)
        _noalloc_product(ddg, Ah, Al, Bh, Bl, Ch, Cl)
        torch.cuda.synchronize()
        assert torch.equal(Ch.view(torch.int64), Rh.view(torch.int64))
        assert torch.equal(Cl.view(torch.int64), Rl.view(torch.int64))
        # the binding's wrapper of the same entry point, on a stream that is not the current one
        s = torch.cuda.Stream(device=dev)
        s.wait_stream(torch.cuda.current_stream())
        Dh, Dl = ddg.dd_gemm_noalloc(Ah, Al, Bh, Bl, stream=s)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        assert torch.equal(Dh.view(torch.int64), Rh.view(torch.int64))
        assert torch.equal(Dl.view(torch.int64), Rl.view(torch.int64))


@pytest.mark.gpu
def test_no_alloc_rejects_products_beyond_its_array(gpu):
    import torch
    ddg = gpu
    dev = torch.device("cuda:0")
    m = n = k = 2048
    assert ddg.workspace_size(m, n, k) > ddg.NOALLOC_SCRATCH_BYTES
    A = torch.zeros((m, k), dtype=torch.float64, device=dev)
    with pytest.raises(ddg.DDGemmError) as e:
        ddg.dd_gemm_noalloc(A, None, A, None)
    assert e.value.status == ddg.ERROR_WORKSPACE
