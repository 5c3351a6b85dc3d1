import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP path")
    config.addinivalue_line("markers", "slow: long-running (large workloads)")


def _gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def gpu():
    """The HIP binding, loaded; fails loudly when a GPU test runs without a GPU."""
    if not _gpu_available():
        pytest.fail("GPU test selected but no GPU is visible")
    import extended_precision_gemm_amd as ddg
    return ddg


_WORKLOAD_CACHE = {}


@pytest.fixture(scope="session")
def workload_operands():
    """Seeded operands per workload name, generated once per session."""
    import workloads

    def get(name):
        if name not in _WORKLOAD_CACHE:
            _WORKLOAD_CACHE.clear()  # keep at most one large workload in memory
            _WORKLOAD_CACHE[name] = workloads.make_operands(workloads.by_name(name))
        return _WORKLOAD_CACHE[name]
    return get
