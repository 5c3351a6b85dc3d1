"""Host-side checks of bench.py (no GPU): the one-GPU contract, the error
without a GPU, and that the HBM traffic of the dominant kernel is taken from
the committed counter summary only while that summary was taken on the
current GEMM source."""
import hashlib
import importlib.util
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench_module():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _run(*args):
    env = dict(os.environ, HIP_VISIBLE_DEVICES="")
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, timeout=300, env=env)


def test_more_than_one_gpu_exits_with_a_message():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_without_a_gpu_the_bench_says_so():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    r = _run("--steps", "1", "--warmup", "0")
    assert r.returncode != 0
    assert "GPU" in r.stderr and r.stdout == ""


def _summary_values(path):
    vals = {}
    for line in open(path):
        if ":" in line and not line.lstrip().startswith("#"):
            key, val = line.split(":", 1)
            vals[key.strip()] = val.strip()
    return vals


@pytest.mark.parametrize("workload", ["dd4096_exp20", "qd4096_exp20"])
def test_traffic_is_read_only_for_the_profiled_source(workload, tmp_path):
    bench = _bench_module()
    path = os.path.join(ROOT, "profiles", f"sliced_gemm_renorm_{workload}_hbm_traffic.txt")
    vals = _summary_values(path)
    src = os.path.join(ROOT, "extended_precision_gemm_amd", "csrc", "sliced_gemm.hip")
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    got = bench._traffic_from_profile(workload)
    if vals["kernel_source_sha256_16"] == sha:
        assert got == float(vals["hbm_bytes_per_launch"]) and got > 0
    else:
        assert got is None
    # a copy of the tree whose GEMM source differs by one byte reads no traffic
    fake = tmp_path / "root"
    (fake / "profiles").mkdir(parents=True)
    (fake / "extended_precision_gemm_amd" / "csrc").mkdir(parents=True)
    shutil.copy(path, fake / "profiles")
    (fake / "extended_precision_gemm_amd" / "csrc" / "sliced_gemm.hip").write_bytes(open(src, "rb").read() + b"\n")
    bench.ROOT = str(fake)
    assert bench._traffic_from_profile(workload) is None
    assert bench._traffic_from_profile("no_such_workload") is None


def test_profiles_of_the_gemm_carry_one_source_hash():
    """The traffic and shader-counter summaries of the GEMM were taken on one
    kernel source, recorded in each."""
    hashes = set()
    for name in sorted(os.listdir(os.path.join(ROOT, "profiles"))):
        if name.endswith(("_hbm_traffic.txt", "_sq_counters.txt")):
            hashes.add(_summary_values(os.path.join(ROOT, "profiles", name)).get("kernel_source_sha256_16"))
    assert len(hashes) == 1 and None not in hashes
