"""Benchmark: effective double-double GFLOP/s (2mnk/t) of C = A·B on one MI355X.

One step is one call of the product entry point dd_gemm_ws on resident inputs
and a preallocated workspace: both operands' exponent passes and slice passes,
then the pair-packed sliced GEMM on FP64 matrix cores (20 products per
k-block covering the 36 window slice pairs) with the nearest-double-double
epilogue fused.  `value` comes from the median step; HIP events on the
product's stream bracket each step, and the library records one more event
after the slicing (dd_gemm_ws_timed), so the GEMM's launch duration is
measured live inside the timed region.

With a quad-double workload (``--workload qd1024``, ``qd2048``, ``qd4096_exp20``)
the step is the quad-double product: slice A and B into sixteen slices, then
the fused 136-pair GEMM with the exact four-double epilogue.

Prints ONE JSON line.  Default workload: the 4096^3 product with per-entry
exponents in [-20, 20].
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "effective double-double GFLOP/s (2mnk/t) at 4096³; % of sliced FP64-MFMA roof"
PEAK_FP64_MFMA_TFLOPS = 78.6   # MI355X dense FP64 matrix peak (AMD datasheet)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PAIRS = 36                     # slice pairs with s + t <= 7
# The pages' own full-path time for a 4096^3 double-double product (build the
# sliced operands, tensor-core product, assemble; unstated NVIDIA GPU): 7.93621 s
# ("Multiple Double Arithmetic on NVIDIA Tensor Cores", §4.2, Table 1, t_TC).
PAGES_TTC_4096_S = 7.93621
# The pages' quad-double full-path times (same table): n = 1024 and n = 2048.
PAGES_QD_TTC_S = {1024: 0.752966, 2048: 4.23463}
QD_METRIC = "effective quad-double GFLOP/s (2mnk/t); % of sliced FP64-MFMA roof (peak / 136 pairs)"
QD_PAIRS = 136


def _parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warm-up steps (default: at least 3, and at least half a second of them, so that the clocks have ramped up)")
    ap.add_argument("--workload", default="dd4096_exp20")
    ap.add_argument("--nslices", type=int, default=8,
                    help="13-bit slices per entry: 8 = double-double (the metric); 4..7 keep fewer pairs, "
                         "9..16 a deeper window")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing leg")
    ap.add_argument("--no-epilogue", action="store_true", help="skip the stand-alone renormalisation timing")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU work of the oracle sample")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run one device copy of this many MiB first (HBM counter calibration)")
    ap.add_argument("--shape", default=None,
                    help="M,N,K: time the product entry point (dd_gemm_ws, or qd_gemm_ws with --qd) on that shape "
                         "with its split-over-k plan, beside the unsplit stage calls (not the metric's line)")
    ap.add_argument("--qd", action="store_true", help="with --shape: the quad-double product")
    return ap.parse_args()


def _traffic_from_profile(workload: str, product: str = "dd"):
    """HBM bytes per GEMM launch from the committed counter summary, if it was
    taken on the current kernel sources; None otherwise."""
    from extended_precision_gemm_amd import profiling
    path = os.path.join(ROOT, "profiles", f"{product}_product_{workload}_hbm_traffic.txt")
    if profiling.read_summary_value(path, "kernel_source_sha256_16") != profiling.source_hash():
        return None
    try:
        return float(profiling.read_summary_value(path, "hbm_bytes_per_launch"))
    except (TypeError, ValueError):
        return None


def _host_info(threads_used):
    """CPU model, logical CPUs and the OpenMP thread setting of the host running the oracle."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": os.cpu_count(), "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
            "threads_used": threads_used}


def _calibration_copy(args, dev):
    """One device copy of known size first, so HBM counters can be scaled by it."""
    import torch
    if args.calib_copy_mib > 0:
        x = torch.ones(args.calib_copy_mib * (1 << 20) // 8, dtype=torch.float64, device=dev)
        y = torch.empty_like(x)
        y.copy_(x)
        torch.cuda.synchronize()
        del x, y


def _warm_up(step, steps):
    """Run untimed steps: exactly `steps` if given, else at least 3 and at least
    half a second of them (short steps need that many for the clocks to ramp
    up).  Returns the number run."""
    import torch
    t0 = time.perf_counter()
    i = 0
    while (i < steps) if steps is not None else (i < 3 or time.perf_counter() - t0 < 0.5):
        step()
        torch.cuda.synchronize()
        i += 1
    return i


def main():
    args = _parse()
    if args.gpus != 1:
        print(f"bench.py: the library runs on exactly one GPU (asked for --gpus {args.gpus}); "
              "the product shards by output tiles with no exchange, but runs across GPUs are not implemented.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import extended_precision_gemm_amd as ddg
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.shape:
        return _run_shape(args)
    w = workloads.by_name(args.workload)
    if w in workloads.QD_WORKLOADS:
        return _run_qd(args, w)
    m, n, k = w.m, w.n, w.k
    dev = torch.device("cuda:0")
    print(f"[bench] generating {w.name} (m={m} n={n} k={k})", file=sys.stderr, flush=True)
    Ah, Al, Bh, Bl = workloads.make_operands(w)
    A_hi, A_lo, B_hi, B_lo = (torch.from_numpy(x).to(dev) for x in (Ah, Al, Bh, Bl))
    C_hi = torch.empty((m, n), dtype=torch.float64, device=dev)
    C_lo = torch.empty((m, n), dtype=torch.float64, device=dev)
    ns = args.nslices
    pairs = ns * (ns + 1) // 2
    products = ddg.pair_products(ns)
    ws = torch.empty(max(ddg.workspace_size(m, n, k, ns), 1), dtype=torch.uint8, device=dev)

    _calibration_copy(args, dev)

    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for e in ev:
        e[1].record(stream)  # creates the event the library records after slicing

    def step(events=None):
        if events:
            events[0].record(stream)
        ddg.dd_gemm_timed(A_hi, A_lo, B_hi, B_lo, C_hi, C_lo, ws, events[1].cuda_event if events else None,
                          stream, nslices=ns)
        if events:
            events[2].record(stream)

    args.warmup = _warm_up(step, args.warmup)
    print(f"[bench] timing {args.steps} steps of dd_gemm_ws", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(ev[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    import statistics
    step_ms = [e[0].elapsed_time(e[2]) for e in ev]
    split_ms_l = [e[0].elapsed_time(e[1]) for e in ev]
    gemm_ms_l = [e[1].elapsed_time(e[2]) for e in ev]
    step_med = statistics.median(step_ms)
    split_ms = statistics.median(split_ms_l)
    gemm_ms = statistics.median(gemm_ms_l)
    ms_per_step = elapsed * 1e3 / args.steps
    value = 2.0 * m * n * k / (step_med * 1e-3) / 1e9
    issued_roof_gflops = PEAK_FP64_MFMA_TFLOPS * 1e3 / products
    pair_roof_gflops = PEAK_FP64_MFMA_TFLOPS * 1e3 / pairs
    gemm_flops = products * 2.0 * m * n * k       # the FP64 matrix products the kernel issues
    gemm_tflops = gemm_flops / (gemm_ms * 1e-3) / 1e12
    traffic = _traffic_from_profile(w.name) if ns == 8 else None
    # slicer: 8 B exponent pass + 16 B read + 8 B per slice written per entry
    split_bytes = (8.0 + 16.0 + 8.0 * ns) * (m * k + k * n)

    rec = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "GFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": (round(value / (2.0 * 4096 ** 3 / PAGES_TTC_4096_S / 1e9), 3)
                        if (m, n, k) == (4096,) * 3 and ns == 8 else None),
        "vs_baseline_ref": "pages' t_TC = 7.93621 s at n = 4096 (17.32 GFLOP/s, unstated NVIDIA GPU, random inputs)",
        "dtype": "f64",
        "data": "synthetic",
        "config": {"workload": w.name, "m": m, "n": n, "k": k, "description": w.description,
                   "slices": ns, "slice_bits": 13, "pairs": pairs, "matrix_products": products},
        "timed": "dd_gemm_ws (slicing + pair-packed sliced GEMM with fused nearest-double-double epilogue), "
                 "median of the steps' HIP-event times; workspace preallocated, inputs resident",
        "pct_sliced_roof": round(100.0 * value / issued_roof_gflops, 2),
        "pct_36pair_roof": round(100.0 * value / pair_roof_gflops, 2),
        "roofline": {
            "kernel": "sliced_gemm_kernel, pair-packed schedule (fused nearest double-double epilogue)",
            "bound": "mfma",
            "achieved": round(gemm_tflops, 3),
            "peak": PEAK_FP64_MFMA_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(gemm_tflops / PEAK_FP64_MFMA_TFLOPS, 4),
            "traffic": traffic,
            "flops_per_launch": gemm_flops,
            "launch_ms": round(gemm_ms, 4),
        },
        "stages": {
            "split_ms": round(split_ms, 4),
            "split_bytes_per_entry": 8 + 16 + 8 * ns,
            "split_GBps": round(split_bytes / (split_ms * 1e-3) / 1e9, 1),
            "split_frac_hbm": round(split_bytes / (split_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "gemm_ms": round(gemm_ms, 4),
        },
        "timing": {"step_ms_median": round(step_med, 4), "step_ms_mean": round(statistics.mean(step_ms), 4),
                   "step_ms_min": round(min(step_ms), 4), "gemm_ms_min": round(min(gemm_ms_l), 4),
                   "split_ms_min": round(min(split_ms_l), 4)},
    }

    # The stand-alone renormalisation (dd_renorm_levels, the stage entry point the
    # fused path does not use), timed on its own outside the timed region:
    # 64 B of level sums read + 16 B of (hi, lo) written per output.
    if not args.no_epilogue and ns == 8:
        del ws
        E, As = ddg.split_balanced(A_hi, A_lo, 0, stream=stream)
        F, Bs = ddg.split_balanced(B_hi, B_lo, 1, stream=stream)
        levels = ddg.sliced_gemm(m, n, k, As, Bs)
        del As, Bs
        R_hi = torch.empty_like(C_hi)
        R_lo = torch.empty_like(C_lo)
        ddg.renorm_levels(levels, E, F, R_hi, R_lo, stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 5
        e0.record(stream)
        for _ in range(reps):
            ddg.renorm_levels(levels, E, F, R_hi, R_lo, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        ren_ms = e0.elapsed_time(e1) / reps
        # the stage chain's cascade and the product's nearest rounding of the same exact totals
        differ = int((R_hi != C_hi).sum().item() + (R_lo != C_lo).sum().item())
        rec["stages"]["renorm_standalone_ms"] = round(ren_ms, 4)
        rec["stages"]["renorm_GBps"] = round(80.0 * m * n / (ren_ms * 1e-3) / 1e9, 1)
        rec["stages"]["renorm_frac_hbm"] = round(80.0 * m * n / (ren_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
        rec["stages"]["renorm_words_differing_from_nearest"] = differ
        del levels, R_hi, R_lo

    if not args.no_cpu_baseline:
        from oracle import compare, native
        threads = native.max_threads()
        print(f"[bench] cpu baseline: oracle on {threads} threads", file=sys.stderr, flush=True)
        # calibrate on a few rows per thread (rows are the parallel dimension),
        # then take as many leading rows as fit the time budget
        native.dd_gemm(Ah[:1, :16], Al[:1, :16], Bh[:16], Bl[:16])  # start the thread pool
        cal = min(m, 2 * threads)
        t = time.perf_counter()
        native.dd_gemm(Ah[:cal], Al[:cal], Bh, Bl)
        per_row = max(time.perf_counter() - t, 1e-6) / cal
        rows = int(max(1, min(m, args.cpu_seconds / per_row)))
        rows = max(threads, rows // threads * threads) if rows >= threads else rows
        t = time.perf_counter()
        Rh, Rl, used = native.dd_gemm(Ah[:rows], Al[:rows], Bh, Bl)
        t_cpu = time.perf_counter() - t
        cpu_gflops = 2.0 * rows * n * k / t_cpu / 1e9
        gh, gl = C_hi[:rows].cpu().numpy(), C_lo[:rows].cpu().numpy()
        rec["cpu_baseline"] = {
            "value": round(cpu_gflops, 3), "unit": "GFLOP/s", "cores": used, "kind": "oracle",
            "sample": f"first {rows} rows of C ({rows}x{n}x{k}, classical dd GEMM, {t_cpu:.1f} s)",
            "host": _host_info(used),
        }
        if ns == 8:
            ratio = compare.error_ratio(gh, gl, Rh, Rl, compare.abs_product(Ah[:rows], Bh))
            rec["parity_sample"] = {"rows": rows, "max_err_over_absAB": ratio, "tol": compare.TOL,
                                    "eps_max": compare.eps_max(gh, gl, Rh, Rl),
                                    "ok": bool(ratio <= compare.TOL)}
        else:
            from oracle import exact
            absAB = compare.abs_product(Ah[:rows], Bh)
            # the bound against the exact product, widened for the classical reference's own error
            bound = exact.error_bound(Ah[:rows], Bh, exact.balancing_exponents(Ah[:rows], Al[:rows], 0),
                                      exact.balancing_exponents(Bh, Bl, 1), ns) + 2.0 ** -96 * absAB
            ratio = float((np.abs((gh - Rh) + (gl - Rl)) / bound).max())
            rec["parity_sample"] = {"rows": rows, "max_err_over_bound": ratio, "ok": bool(ratio <= 1.0),
                                    "max_err_over_absAB": compare.error_ratio(gh, gl, Rh, Rl, absAB)}
    print(json.dumps(rec), flush=True)


def _run_shape(args):
    """The product entry point on an arbitrary shape with the split-over-k plan it
    takes (tiles before the first split tile unsplit, the rest in `parts`
    k-parts), timed beside the unsplit 36-pair stage chain (slicing + the fused
    level-cascade call, which never splits) on the same inputs.  The two round
    the same exact totals differently (nearest double-double vs the level
    cascade); the line reports how many words differ."""
    import torch

    import extended_precision_gemm_amd as ddg
    import workloads

    m, n, k = (int(x) for x in args.shape.split(","))
    ns = 16 if args.qd else args.nslices
    dev = torch.device("cuda:0")
    print(f"[bench] shape m={m} n={n} k={k} ({'qd' if args.qd else f'dd, {ns} slices'})", file=sys.stderr, flush=True)
    stream = torch.cuda.current_stream()
    if args.qd:
        A = torch.from_numpy(workloads.random_qd((m, k), 11, "uniform")).to(dev)
        B = torch.from_numpy(workloads.random_qd((k, n), 12, "uniform")).to(dev)
        C = torch.empty((4, m, n), dtype=torch.float64, device=dev)
        U = torch.empty_like(C)
        ws = torch.empty(max(ddg.qd_workspace_size(m, n, k), 1), dtype=torch.uint8, device=dev)
        E, As = ddg.qd_split_balanced(A, 0)
        F, Bs = ddg.qd_split_balanced(B, 1)

        def product():
            ddg.qd_gemm(A, B, C=C, workspace=ws, stream=stream)

        def unsplit():
            ddg.qd_split_balanced(A, 0, E, As, stream)
            ddg.qd_split_balanced(B, 1, F, Bs, stream)
            ddg.qd_sliced_gemm_renorm(m, n, k, As, E, Bs, F, U, stream)
        outs = ((C,), (U,))
    else:
        Ah, Al = (torch.from_numpy(x).to(dev) for x in workloads.random_dd((m, k), 11, "uniform"))
        Bh, Bl = (torch.from_numpy(x).to(dev) for x in workloads.random_dd((k, n), 12, "uniform"))
        C_hi = torch.empty((m, n), dtype=torch.float64, device=dev)
        C_lo = torch.empty_like(C_hi)
        U_hi, U_lo = torch.empty_like(C_hi), torch.empty_like(C_hi)
        ws = torch.empty(max(ddg.workspace_size(m, n, k, ns), 1), dtype=torch.uint8, device=dev)
        E, As = ddg.split_balanced(Ah, Al, 0, nslices=ns)
        F, Bs = ddg.split_balanced(Bh, Bl, 1, nslices=ns)

        def product():
            ddg.dd_gemm(Ah, Al, Bh, Bl, C_hi=C_hi, C_lo=C_lo, workspace=ws, stream=stream, nslices=ns)

        def unsplit():
            ddg.split_balanced(Ah, Al, 0, E, As, stream, nslices=ns)
            ddg.split_balanced(Bh, Bl, 1, F, Bs, stream, nslices=ns)
            ddg.sliced_gemm_renorm(m, n, k, As, E, Bs, F, U_hi, U_lo, stream, nslices=ns)
        outs = ((C_hi, C_lo), (U_hi, U_lo))

    def timed(fn):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / args.steps

    # warm both paths up, for at least half a second so that the clocks have
    # ramped, then time product, stage chain, product: the mean of the two
    # product runs cancels a drift of the clock over the measurement
    def both():
        product()
        unsplit()

    args.warmup = _warm_up(both, args.warmup)
    print(f"[bench] timing {args.steps} steps of each path", file=sys.stderr, flush=True)
    t_prod_a = timed(product)
    t_unsplit = timed(unsplit)
    t_prod = 0.5 * (t_prod_a + timed(product))
    differ = sum(int((a != b).sum().item()) for a, b in zip(*outs))
    gf = lambda t: 2.0 * m * n * k / t / 1e9
    rec = {
        "metric": "product entry point GFLOP/s (2mnk/t) on the given shape; unsplit stage chain beside it",
        "value": round(gf(t_prod), 3),
        "unit": "GFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_prod * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64",
        "data": "synthetic",
        "config": {"workload": f"{'qd' if args.qd else 'dd'} {m}x{n}x{k}", "m": m, "n": n, "k": k, "slices": ns,
                   "description": "entries U(-1,1), lo (further components) at 2^-53 relative scale"},
        "split_plan": {"first_split_row": ddg.split_first_row(m, n, k, ns), "parts": ddg.split_parts(m, n, k, ns)},
        "stage_chain": {"ms_per_step": round(t_unsplit * 1e3, 4), "value": round(gf(t_unsplit), 3)},
        "speedup_vs_stage_chain": round(t_unsplit / t_prod, 3),
        "words_differing_from_stage_chain": differ,
    }
    print(json.dumps(rec), flush=True)


def _run_qd(args, w):
    """The quad-double product qd_gemm_ws (both operands sliced into sixteen
    slices, then the sliced GEMM with the exact four-double epilogue: the
    pair-packed schedule's 72 matrix products per k-block up to k = 2^21, the
    136 level products beyond), timed whole; the library records one more
    event after the slicing."""
    import numpy as np
    import statistics
    import torch

    import extended_precision_gemm_amd as ddg
    import workloads

    m, n, k = w.m, w.n, w.k
    dev = torch.device("cuda:0")
    print(f"[bench] generating {w.name} (m={m} n={n} k={k})", file=sys.stderr, flush=True)
    A, B = workloads.make_qd_operands(w)
    dA = torch.from_numpy(A).to(dev)
    dB = torch.from_numpy(B).to(dev)
    C = torch.empty((4, m, n), dtype=torch.float64, device=dev)
    ws = torch.empty(max(ddg.qd_workspace_size(m, n, k), 1), dtype=torch.uint8, device=dev)
    _calibration_copy(args, dev)
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for e in ev:
        e[1].record(stream)  # creates the event the library records after slicing

    def step(events=None):
        if events:
            events[0].record(stream)
        ddg.qd_gemm_timed(dA, dB, C, ws, events[1].cuda_event if events else None, stream)
        if events:
            events[2].record(stream)

    args.warmup = _warm_up(step, args.warmup)
    print(f"[bench] timing {args.steps} steps of qd_gemm_ws", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(ev[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    step_l = [e[0].elapsed_time(e[2]) for e in ev]
    gemm_l = [e[1].elapsed_time(e[2]) for e in ev]
    split_ms = statistics.median(e[0].elapsed_time(e[1]) for e in ev)
    gemm_ms = statistics.median(gemm_l)
    step_med = statistics.median(step_l)
    value = 2.0 * m * n * k / (step_med * 1e-3) / 1e9
    products = ddg.pair_products(16) if k <= (1 << 21) else QD_PAIRS
    gemm_flops = products * 2.0 * m * n * k
    gemm_tflops = gemm_flops / (gemm_ms * 1e-3) / 1e12
    split_bytes = (32.0 + 128.0) * (m * k + k * n)  # four components read, sixteen slices written
    ttc = PAGES_QD_TTC_S.get(m) if m == n == k else None
    rec = {
        "metric": QD_METRIC,
        "value": round(value, 3),
        "unit": "GFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(value / (2.0 * m ** 3 / ttc / 1e9), 3) if ttc else None,
        "vs_baseline_ref": ("pages' quad-double t_TC = %g s at n = %d (unstated NVIDIA GPU)" % (ttc, m)) if ttc
        else None,
        "dtype": "f64",
        "data": "synthetic",
        "config": {"workload": w.name, "m": m, "n": n, "k": k, "description": w.description,
                   "slices": 16, "slice_bits": 13, "pairs": QD_PAIRS, "matrix_products": products},
        "timed": "qd_gemm_ws (slicing + sliced GEMM with the exact four-double epilogue), median of the steps' "
                 "HIP-event times; workspace preallocated, inputs resident",
        "pct_sliced_roof": round(100.0 * value / (PEAK_FP64_MFMA_TFLOPS * 1e3 / products), 2),
        "pct_136pair_roof": round(100.0 * value / (PEAK_FP64_MFMA_TFLOPS * 1e3 / QD_PAIRS), 2),
        "roofline": {
            "kernel": "sliced_gemm_kernel, 16 slices (fused exact four-double epilogue)",
            "bound": "mfma",
            "achieved": round(gemm_tflops, 3),
            "peak": PEAK_FP64_MFMA_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(gemm_tflops / PEAK_FP64_MFMA_TFLOPS, 4),
            "traffic": _traffic_from_profile(w.name, "qd"),
            "flops_per_launch": gemm_flops,
            "launch_ms": round(gemm_ms, 4),
        },
        "stages": {
            "split_ms": round(split_ms, 4),
            "split_GBps": round(split_bytes / (split_ms * 1e-3) / 1e9, 1),
            "split_frac_hbm": round(split_bytes / (split_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "gemm_ms": round(gemm_ms, 4),
        },
        "timing": {"step_ms_median": round(statistics.median(step_l), 4), "step_ms_min": round(min(step_l), 4),
                   "gemm_ms_median": round(statistics.median(gemm_l), 4), "gemm_ms_min": round(min(gemm_l), 4)},
    }
    if not args.no_cpu_baseline:
        from fractions import Fraction

        from oracle import qd
        # the exact-integer oracle, one entry at a time, for about cpu_seconds
        rng = np.random.default_rng(7)
        rows, cols = [], []
        t = time.perf_counter()
        exact_vals = []
        while time.perf_counter() - t < args.cpu_seconds and len(rows) < m * n:
            i, j = int(rng.integers(m)), int(rng.integers(n))
            exact_vals += qd.exact_entries(A, B, [i], [j])
            rows.append(i)
            cols.append(j)
        t_cpu = time.perf_counter() - t
        rec["cpu_baseline"] = {
            "value": round(2.0 * k * len(rows) / t_cpu / 1e9, 6), "unit": "GFLOP/s", "cores": 1, "kind": "oracle",
            "sample": f"{len(rows)} random entries of C by the exact-integer oracle ({t_cpu:.1f} s, one thread)",
            "host": _host_info(1),
        }
        ri = torch.as_tensor(rows, device=dev)
        ci = torch.as_tensor(cols, device=dev)
        got = C[:, ri, ci].cpu().numpy()
        err = np.array([float(abs(sum(Fraction(float(c)) for c in got[:, q]) - e))
                        for q, e in enumerate(exact_vals)])
        E, _ = ddg.qd_split_balanced(dA, 0)  # the balancing exponents, for the bound
        F, _ = ddg.qd_split_balanced(dB, 1)
        Eh, Fh = E.cpu().numpy(), F.cpu().numpy()
        bound = qd.error_bound(A[0], B[0], Eh, Fh, rows, cols)
        absAB = np.einsum("qk,kq->q", np.abs(A[0])[rows, :], np.abs(B[0])[:, cols])
        ratio = float((err / bound).max())
        rec["parity_sample"] = {"entries": len(rows), "max_err_over_bound": ratio,
                                "max_err_over_absAB": float((err / absAB).max()), "ok": bool(ratio <= 1.0)}
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
