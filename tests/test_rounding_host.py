"""The double-double exit's fast rounding (csrc/pair_levels.hpp,
pair_dd_round_fast) against the wide-integer rounding it short-cuts, compiled
for the host: the nearest double-double of the exact total of the group sums
("Multiple Double Arithmetic on NVIDIA Tensor Cores", §2, step 5 of the
overview, with the total rounded once) must come out the same, bit for bit, on
200,000 seeded totals per slice count, exact ties and near ties included."""
import os
import re
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    exe = str(tmp_path_factory.mktemp("rounding") / "rounding_check")
    cmd = [HIPCC, "--offload-host-only", "-O2", "-std=c++17", "-w",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "extended_precision_gemm_amd", "csrc"),
           os.path.join(HERE, "rounding_check.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True, timeout=600)
    return exe


def test_fast_rounding_equals_the_wide_integer_rounding(checker):
    out = subprocess.run([checker, "200000"], capture_output=True, text=True, timeout=600)
    assert out.returncode == 0, out.stdout + out.stderr
    lines = re.findall(r"NS=(\d+) cases=(\d+) fast=(\d+) mismatches=(\d+)", out.stdout)
    assert [int(ns) for ns, *_ in lines] == [4, 5, 6, 7, 8]
    for ns, cases, fast, bad in lines:
        assert int(bad) == 0
        assert int(fast) > int(cases) // 4  # the fast path takes a good share of these adversarial totals
