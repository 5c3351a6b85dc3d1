"""Host-side checks of bench.py (no GPU): the one-GPU contract, the error
without a GPU, and that the HBM traffic of the dominant kernel is taken from
the committed counter summary only while that summary was taken on the
current GEMM source."""
import importlib.util
import os
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


@pytest.mark.parametrize("workload,product", [("dd4096_exp20", "dd"), ("qd4096_exp20", "qd")])
def test_traffic_is_read_only_for_the_profiled_source(workload, product, monkeypatch):
    bench = _bench_module()
    from extended_precision_gemm_amd import profiling
    path = os.path.join(ROOT, "profiles", f"{product}_product_{workload}_hbm_traffic.txt")
    vals = _summary_values(path)
    got = bench._traffic_from_profile(workload, product)
    if vals["kernel_source_sha256_16"] == profiling.source_hash():
        assert got == float(vals["hbm_bytes_per_launch"]) and got > 0
    else:
        assert got is None
    # a GEMM source that differs from the profiled one reads no traffic
    monkeypatch.setattr(profiling, "source_hash", lambda: "0" * 16)
    assert bench._traffic_from_profile(workload, product) is None
    assert bench._traffic_from_profile("no_such_workload") is None


def test_source_hash_covers_the_gemm_sources(tmp_path, monkeypatch):
    """One byte more in any of the GEMM's sources changes the hash."""
    from extended_precision_gemm_amd import profiling
    base = profiling.source_hash()
    for f in profiling.GEMM_SOURCES:
        pkg = tmp_path / f.replace(".", "_")
        (pkg / "csrc").mkdir(parents=True)
        for g in profiling.GEMM_SOURCES:
            data = open(os.path.join(profiling._PKG, "csrc", g), "rb").read()
            (pkg / "csrc" / g).write_bytes(data + (b"\n" if g == f else b""))
        monkeypatch.setattr(profiling, "_PKG", str(pkg))
        assert profiling.source_hash() != base
        monkeypatch.undo()
    assert profiling.source_hash() == base


def test_profiles_of_the_gemm_carry_one_source_hash():
    """The traffic and shader-counter summaries of the GEMM were taken on one
    kernel source, recorded in each."""
    hashes = set()
    for name in sorted(os.listdir(os.path.join(ROOT, "profiles"))):
        if name.endswith(("_hbm_traffic.txt", "_sq_counters.txt")):
            hashes.add(_summary_values(os.path.join(ROOT, "profiles", name)).get("kernel_source_sha256_16"))
    assert len(hashes) == 1 and None not in hashes
