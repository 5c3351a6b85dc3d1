"""The rocprofv3 harness (extended_precision_gemm_amd.profiling) on trimmed
rocprofv3 output of a 4096^3 double-double product: the last two steps of a
kernel trace, and the GEMM, slice and calibration-copy dispatches of the
FETCH_SIZE / WRITE_SIZE runs and of two SQ counter passes
(tests/data/rocprof).  Expected figures are recomputed here from the CSV rows
with the csv module, independently of the harness's parsing."""
import csv
import glob
import os
import statistics

import pytest

from extended_precision_gemm_amd import profiling as P

DATA = os.path.join(os.path.dirname(__file__), "data", "rocprof")
M = N = K = 4096


def _rows(name):
    path = glob.glob(os.path.join(DATA, name, "*.csv"))[0]
    with open(path, newline="") as fh:
        return list(csv.DictReader(fh))


def test_kernel_names_parse():
    name = ("void ddg::(anonymous namespace)::sliced_gemm_kernel<ddg::(anonymous namespace)::GemmConfig<4, 4, 2, 2, "
            "1, 8, 1, 0>, 1, true, true>(long, long, long, long, long, double const*, double const*, double*)")
    short = P.short_name(name)
    assert short == "sliced_gemm_kernel<GemmConfig<4, 4, 2, 2, 1, 8, 1, 0>, 1, true, true>"
    assert P.family(short) == "sliced_gemm_kernel"
    assert P.template_args(short) == ["GemmConfig<4, 4, 2, 2, 1, 8, 1, 0>", "1", "true", "true"]
    assert P.short_name("ddg::(anonymous namespace)::exp_rows_kernel(long, long, double const*)") == "exp_rows_kernel"


def test_pair_products_match_the_schedule_and_the_library():
    # B slice t meets ns - t A slices, two per product
    assert [P.pair_products(n) for n in (4, 8, 16)] == [6, 20, 72]
    import extended_precision_gemm_amd as ddg
    for n in range(4, 17):
        assert P.pair_products(n) == ddg.pair_products(n)


def test_work_model():
    gemm = "sliced_gemm_kernel<GemmConfig<4, 4, 2, 2, 1, 8, 1, 0>, 1, true, true>"
    full = (M // 64) * (N // 64) * 1024  # threads: 16-wave workgroups, one per 64x64 tile
    w = P.kernel_work(gemm, M, N, K, 8, (full, 1, 1))
    assert w.unit == "flop" and w.amount == 20 * 2.0 * M * N * K
    # a launch over part of the tiles, or a k-part of a split product, is not rated
    assert P.kernel_work(gemm, M, N, K, 8, (full // 2, 1, 1)) is None
    assert P.kernel_work("sliced_gemm_kernel<GemmConfig<4, 4, 2, 2, 1, 8, 1, 0>, 7, true, true>", M, N, K, 8) is None
    level = P.kernel_work("sliced_gemm_kernel<GemmConfig<2, 4, 2, 2, 1, 8, 2, 0>, 1, false, false>", M, N, K, 8)
    assert level.amount == 36 * 2.0 * M * N * K
    assert P.kernel_work("slice_rows_lds_kernel<8, true, true, false>", M, N, K, 8).amount == 80.0 * M * K
    assert P.kernel_work("slice_cols_lds_kernel<8, true, true>", M, N, K, 8).amount == 80.0 * K * N
    assert P.kernel_work("exp_rows_fix_kernel<8>", M, N, K, 8).amount == 8.0 * M * K
    assert P.kernel_work("exp_cols_stream_kernel<256>", M, N, K, 8).amount == 8.0 * K * N
    assert P.kernel_work("split_block_kernel<0, 256, 8, true, true>", M, N, K, 8) is None  # the exact pass
    assert P.kernel_work("split_block_regs_kernel<0, 1024, 8, 4, true>", M, N, K, 8).amount == 88.0 * M * K
    assert P.kernel_work("renorm_kernel<8>", M, N, K, 8).amount == 80.0 * M * N


def test_trace_summary_against_the_rows():
    rows = _rows("dd4096_exp20_trace")
    gemm = [r for r in rows if "sliced_gemm_kernel" in r["Kernel_Name"]]
    ms = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-6 for r in gemm]
    tflops = 20 * 2.0 * M * N * K / (statistics.median(ms) * 1e-3) / 1e12
    text = P.trace_summary(os.path.join(DATA, "dd4096_exp20_trace"), M, N, K, 8, "t", ["cmd"])
    line = [l for l in text.splitlines() if l.startswith("sliced_gemm_kernel<") and "flop per launch" in l][0]
    assert f"-> {tflops:.2f} TFLOP/s of 78.6 ({100 * tflops / 78.6:.1f} %)" in line
    table = [l for l in text.splitlines() if l.startswith("sliced_gemm_kernel<") and "flop" not in l][0]
    assert table.split()[-6] == f"{statistics.mean(ms):.4f}" or f"{statistics.mean(ms):.4f}" in table
    # the slicer: 2 x 8 B exponent passes + 2 x 80 B slice passes per entry
    sl = [r for r in rows if any(x in r["Kernel_Name"] for x in ("exp_rows_fix", "exp_cols_stream", "slice_rows_lds",
                                                                    "slice_cols_lds"))]
    by = {}
    for r in sl:
        by.setdefault(P.short_name(r["Kernel_Name"]), []).append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-6)
    t = sum(statistics.median(v) for v in by.values())
    frac = 88.0 * 2 * M * N / (t * 1e-3) / 1e9 / 8000
    assert f"= {100 * frac:.1f} % of 8000 GB/s" in text
    assert "kernel_source_sha256_16: " in text and text.startswith("# t\n")


def test_traffic_summary_calibrates_by_the_copy():
    def kib(name, counter, kernel):
        return statistics.mean(float(r["Counter_Value"]) for r in _rows(name)
                               if kernel in r["Kernel_Name"] and r["Counter_Name"] == counter)
    f_copy = max(float(r["Counter_Value"]) for r in _rows("dd4096_fetch") if "copyBuffer" in r["Kernel_Name"])
    w_copy = max(float(r["Counter_Value"]) for r in _rows("dd4096_write") if "copyBuffer" in r["Kernel_Name"])
    rs, ws = (1 << 30) / (f_copy * 1024), (1 << 30) / (w_copy * 1024)
    assert 1.9 < rs < 2.1 and 0.95 < ws < 1.05  # FETCH_SIZE counts half of a copy's read bytes
    gemm_bytes = (kib("dd4096_fetch", "FETCH_SIZE", "sliced_gemm_kernel") * 1024 * rs
                  + kib("dd4096_write", "WRITE_SIZE", "sliced_gemm_kernel") * 1024 * ws)
    text = P.traffic_summary(os.path.join(DATA, "dd4096_fetch"), os.path.join(DATA, "dd4096_write"), M, N, K, 1024)
    assert float(P.read_summary_value_text(text, "hbm_bytes_per_launch")) == pytest.approx(gemm_bytes, rel=1e-6)
    # the slice pass moves its algorithmic bytes once
    line = [l for l in text.splitlines() if l.startswith("slice_rows_lds_kernel")][0]
    assert abs(float(line.split()[-1]) - 1.0) < 0.01


def test_counters_summary():
    text = P.counters_summary([os.path.join(DATA, "dd4096_sq1"), os.path.join(DATA, "dd4096_sq2")], M, N, K, 8)
    assert "(ratio 1.0000)" in text  # 20 MFMAs per 16x16 block per k-block of 4
    busy = [l for l in text.splitlines() if l.startswith("MFMA busy")][0]
    rows = _rows("dd4096_sq2")
    mb = statistics.mean(float(r["Counter_Value"]) for r in rows if r["Counter_Name"] == "SQ_VALU_MFMA_BUSY_CYCLES")
    ga = statistics.mean(float(r["Counter_Value"]) for r in rows if r["Counter_Name"] == "GRBM_GUI_ACTIVE")
    assert busy.endswith(f"= {100 * mb / (ga / 8 * 1024):.1f} %")


def test_command_line_writes_the_summary(tmp_path):
    out = tmp_path / "s.txt"
    assert P.main(["trace", os.path.join(DATA, "dd4096_exp20_trace"), "--shape", "4096,4096,4096",
                   "--command", "rocprofv3 ...", "-o", str(out)]) == 0
    text = out.read_text()
    assert "#   rocprofv3 ..." in text and P.read_summary_value(str(out), "kernel_source_sha256_16") == P.source_hash()
