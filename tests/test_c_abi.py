"""The library used from plain C (tests/c_abi_example.c).

CPU: both headers compile as strict C11 (-pedantic -Werror) and the example
links against libddgemm.so and the HIP runtime.  GPU: the example runs --
double-double, n-slice and quad-double products of small integer matrices,
checked against integer matrix products it computes itself, plus status codes
for bad arguments and a short workspace.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "extended_precision_gemm_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _build(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    assert os.path.exists(os.path.join(PKG, "libddgemm.so")), "libddgemm.so is not built"
    exe = str(tmp_path / "c_abi_example")
    cmd = [gcc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic", "-D__HIP_PLATFORM_AMD__",
           "-isystem", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c_abi_example.c"),
           "-L", PKG, "-lddgemm", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           f"-Wl,-rpath,{PKG}", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    return exe


def test_headers_are_strict_c_and_the_example_links(tmp_path):
    assert os.path.exists(_build(tmp_path))


@pytest.mark.gpu
def test_c_example_runs_on_the_gpu(tmp_path):
    exe = _build(tmp_path)
    print("[c abi] running the C example", flush=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    assert "c abi ok" in r.stdout
