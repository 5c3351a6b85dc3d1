"""rocprofv3 harness: per-kernel time, roofline fractions and HBM traffic of the
products, from the CSV files rocprofv3 writes.

The pages judge their method by the time of each stage of a product (building
the sliced operands, the matrix-core products, the classical reference:
"Multiple Double Arithmetic on NVIDIA Tensor Cores", §4.2, Table 1).  This
module splits a measured step the same way, by kernel, and relates every
kernel to what bounds it on MI355X: the FP64 matrix cores (78.6 TFLOP/s dense)
for the sliced GEMM, HBM (8 TB/s) for the slicer, the renormalisation and the
other streaming kernels.  Algorithmic work is counted per launch: the matrix
products a GEMM issues times 2mnk; for a streaming kernel the bytes it has to
move -- 8 B per entry for an exponent pass over the leading words, 16 B read
and 8 B per slice written for a slice pass, 8 B per level read and 16 B
written per output for a renormalisation.

Three summaries, each written as text with the commands that produced it:

    python -m extended_precision_gemm_amd.profiling trace DIR --shape M,N,K [--nslices n]
        [--bench-json FILE] [--command CMD ...] [--title T] [-o OUT]
    python -m extended_precision_gemm_amd.profiling traffic FETCH_DIR WRITE_DIR --shape M,N,K
        --calib-mib MIB [--nslices n] [--command CMD ...] [-o OUT]
    python -m extended_precision_gemm_amd.profiling counters DIR [DIR ...] --shape M,N,K
        [--nslices n] [--command CMD ...] [-o OUT]

DIR is a rocprofv3 output directory (``-d``) holding ``*_kernel_trace.csv`` (and
``*_kernel_stats.csv``) or ``*_counter_collection.csv``.  ``traffic`` scales
FETCH_SIZE and WRITE_SIZE by what the same counters read for the device copy
of --calib-mib MiB that ``bench.py --calib-copy-mib`` runs first.  Reading
rocprofv3's output is all this module does: it launches nothing on the GPU.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import re
import statistics
import sys
from dataclasses import dataclass, field

PEAK_FP64_MFMA_TFLOPS = 78.6  # MI355X dense FP64 matrix peak
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
SLICE_BITS = 13

_PKG = os.path.dirname(os.path.abspath(__file__))
# the sources whose change makes the GEMM's counter figures stale: the kernels
# and the host code that picks their launches (plans, the small-output path)
GEMM_SOURCES = ("sliced_gemm.hip", "pair_levels.hpp", "qd_levels.hpp", "wide_int.hpp", "common.hpp", "api.cpp",
                "split_k.cpp")


def source_hash(files=GEMM_SOURCES) -> str:
    """First 16 hex digits of the SHA-256 of the named kernel sources, in order."""
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(_PKG, "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def pair_products(ns: int) -> int:
    """FP64 matrix products per k-block of the pair-packed schedule: B slice t
    meets the A slices s < ns - t, two of them per product."""
    return sum((ns - t + 1) // 2 for t in range(ns))


# ---------------------------------------------------------------- CSV input


@dataclass
class Dispatch:
    name: str
    short: str
    start: int
    end: int
    grid: tuple
    workgroup: int
    vgpr: int
    agpr: int
    sgpr: int
    lds: int
    scratch: int
    dispatch_id: int = 0
    counters: dict = field(default_factory=dict)

    @property
    def ms(self) -> float:
        return (self.end - self.start) * 1e-6


def short_name(name: str) -> str:
    """The kernel's name without return type, namespaces and argument list."""
    s = name.replace("void ", "", 1) if name.startswith("void ") else name
    s = s.replace("(anonymous namespace)::", "")
    s = re.sub(r"\b[A-Za-z_]\w*::", "", s)
    depth = 0
    for i, ch in enumerate(s):  # cut the argument list (the first '(' outside template brackets)
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            return s[:i].strip()
    return s.strip()


def family(short: str) -> str:
    return short.split("<", 1)[0]


def template_args(short: str) -> list[str]:
    """Top-level template arguments of a short kernel name."""
    if "<" not in short:
        return []
    inner = short[short.index("<") + 1: short.rindex(">")]
    out, depth, cur = [], 0, ""
    for ch in inner:
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        if ch == "," and depth == 0:
            out.append(cur.strip())
            cur = ""
        else:
            cur += ch
    if cur.strip():
        out.append(cur.strip())
    return out


def _find(directory: str, suffix: str) -> str:
    hits = sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {directory}")
    return hits[0]


def load_trace(directory: str) -> list[Dispatch]:
    """The kernel dispatches of a ``--kernel-trace`` run, in start order."""
    out = []
    with open(_find(directory, "_kernel_trace.csv"), newline="") as fh:
        for r in csv.DictReader(fh):
            out.append(Dispatch(
                name=r["Kernel_Name"], short=short_name(r["Kernel_Name"]),
                start=int(r["Start_Timestamp"]), end=int(r["End_Timestamp"]),
                grid=(int(r["Grid_Size_X"]), int(r["Grid_Size_Y"]), int(r["Grid_Size_Z"])),
                workgroup=int(r["Workgroup_Size_X"]) * int(r["Workgroup_Size_Y"]) * int(r["Workgroup_Size_Z"]),
                vgpr=int(r["VGPR_Count"]), agpr=int(r.get("Accum_VGPR_Count") or 0), sgpr=int(r["SGPR_Count"]),
                lds=int(r["LDS_Block_Size"]), scratch=int(r["Scratch_Size"]),
                dispatch_id=int(r["Dispatch_Id"])))
    out.sort(key=lambda d: d.start)
    return out


def load_counters(directory: str) -> list[Dispatch]:
    """The dispatches of a ``--pmc`` run with their counter values (summed over
    the rows of one counter, which rocprofv3 may split by dimension)."""
    by_id: dict[int, Dispatch] = {}
    with open(_find(directory, "_counter_collection.csv"), newline="") as fh:
        for r in csv.DictReader(fh):
            did = int(r["Dispatch_Id"])
            d = by_id.get(did)
            if d is None:
                d = by_id[did] = Dispatch(
                    name=r["Kernel_Name"], short=short_name(r["Kernel_Name"]),
                    start=int(r["Start_Timestamp"]), end=int(r["End_Timestamp"]), grid=(int(r["Grid_Size"]), 1, 1),
                    workgroup=int(r["Workgroup_Size"]), vgpr=int(r["VGPR_Count"]),
                    agpr=int(r.get("Accum_VGPR_Count") or 0), sgpr=int(r["SGPR_Count"]),
                    lds=int(r["LDS_Block_Size"]), scratch=int(r["Scratch_Size"]), dispatch_id=did)
            name = r["Counter_Name"]
            d.counters[name] = d.counters.get(name, 0.0) + float(r["Counter_Value"])
    return sorted(by_id.values(), key=lambda d: d.start)


# ---------------------------------------------------------------- work model


@dataclass
class Work:
    amount: float  # flop or bytes per launch
    unit: str      # "flop" or "B"
    note: str


def kernel_work(short: str, m: int, n: int, k: int, ns: int, grid: tuple | None = None) -> Work | None:
    """Algorithmic work of one full launch of a kernel of the m×k by k×n product
    with ns slices per entry; None for kernels that carry none of their own
    (exact passes that find nothing to redo, folds, fills) or whose launch
    covers only part of the product (a GEMM launch of a split product: k-parts,
    or the tiles before the first split one -- told apart by `grid`, the
    launch's grid in threads)."""
    fam, args = family(short), template_args(short)
    a_ent, b_ent, outs = m * k, k * n, m * n
    if fam == "sliced_gemm_kernel" and args:
        cfg = template_args(args[0])
        cfg_ns = int(cfg[5]) if len(cfg) > 5 else ns
        epi = int(args[1]) if len(args) > 1 else 0
        paired = len(args) > 2 and args[2] == "true"
        if epi in (6, 7):  # k-parts of a split product: a partial launch
            return None
        if grid is not None and len(cfg) > 6:
            wm, wn, rpw = int(cfg[0]), int(cfg[1]), int(cfg[6])
            bm, bn = 16 * rpw * wm, 16 * wn
            tiles = -(-m // bm) * -(-n // bn)
            if grid[0] // (64 * wm * wn) != tiles or grid[1] != 1:
                return None
        prods = pair_products(cfg_ns) if paired else cfg_ns * (cfg_ns + 1) // 2
        kind = "pair-packed products" if paired else "slice-pair products"
        return Work(prods * 2.0 * m * n * k, "flop", f"{prods} {kind} x 2mnk")
    slice_b = 16 + 8 * ns
    if fam in ("slice_rows_lds_kernel",):
        return Work(slice_b * a_ent, "B", f"A: 16 B read + {8 * ns} B written per entry")
    if fam in ("slice_cols_lds_kernel", "slice_cols_kernel"):
        return Work(slice_b * b_ent, "B", f"B: 16 B read + {8 * ns} B written per entry")
    if fam in ("exp_rows_kernel", "exp_rows_fix_kernel"):
        return Work(8.0 * a_ent, "B", "A: 8 B (leading word) read per entry")
    if fam in ("exp_cols_stream_kernel",):
        return Work(8.0 * b_ent, "B", "B: 8 B (leading word) read per entry")
    if fam in ("split_block_regs_kernel", "split_block_kernel") and args:
        if fam == "split_block_kernel" and len(args) > 4 and args[4] == "true":  # the exact pass
            return None
        ent = a_ent if args[0] == "0" else b_ent
        return Work((8 + slice_b) * ent, "B", f"one pass: 8 + 16 B read + {8 * ns} B written per entry")
    if fam == "renorm_kernel":
        return Work((8.0 * ns + 16) * outs, "B", f"{8 * ns} B of levels read + 16 B written per output")
    if fam == "qd_slice_kernel" and args:
        ent = a_ent if args[0] == "0" else b_ent
        return Work(160.0 * ent, "B", "32 B read + 128 B written per entry")
    if fam in ("qd_exp_rows_kernel",):
        return Work(32.0 * a_ent, "B", "32 B read per entry")
    if fam in ("qd_exp_cols_block_kernel",):
        return Work(32.0 * b_ent, "B", "32 B read per entry")
    return None


def roofline(work: Work, ms: float) -> tuple[float, float, str, float]:
    """(achieved, peak, unit, fraction) for one launch of `ms` milliseconds."""
    if work.unit == "flop":
        a = work.amount / (ms * 1e-3) / 1e12
        return a, PEAK_FP64_MFMA_TFLOPS, "TFLOP/s", a / PEAK_FP64_MFMA_TFLOPS
    a = work.amount / (ms * 1e-3) / 1e9
    return a, PEAK_HBM_GBS, "GB/s", a / PEAK_HBM_GBS


# ---------------------------------------------------------------- summaries


def _group(dispatches: list[Dispatch], skip=("__amd_rocclr", "at::", "elementwise")) -> dict[str, list[Dispatch]]:
    groups: dict[str, list[Dispatch]] = {}
    for d in dispatches:
        if any(s in d.name for s in skip):
            continue
        groups.setdefault(d.short, []).append(d)
    return groups


def _header(title: str, commands: list[str], source: str) -> list[str]:
    out = [f"# {title}", "#", "# commands (repository root as $REPO on the measuring host):"]
    out += [f"#   {c}" for c in commands]
    out.append(f"# source: {source}")
    return out


def trace_summary(directory: str, m: int, n: int, k: int, ns: int = 8, title: str = "",
                  commands: list[str] | None = None, bench: dict | None = None) -> str:
    """Per-kernel times of a --kernel-trace run, with each kernel's roofline
    (achieved rates from the median launch; the first launch of a run warms up)."""
    disp = load_trace(directory)
    groups = _group(disp)
    total = sum(d.ms for g in groups.values() for d in g)
    lines = _header(title or f"rocprofv3 kernel trace, {m}x{n}x{k}, {ns} slices", commands or [],
                    "rocprofv3 kernel_trace.csv (every launch; averages over the launches)")
    lines.append("")
    lines.append(f"{'kernel':58s} {'calls':>5s} {'avg_ms':>10s} {'med_ms':>10s} {'min_ms':>10s} {'max_ms':>10s} "
                 f"{'pct':>6s}  {'achieved':>10s} {'of peak':>8s}")
    rows = sorted(groups.items(), key=lambda kv: -sum(d.ms for d in kv[1]))
    slicer_bytes, slicer_ms = 0.0, 0.0
    for short, g in rows:
        ms = [d.ms for d in g]
        avg = statistics.mean(ms)
        med = statistics.median(ms)
        w = kernel_work(short, m, n, k, ns, g[0].grid)
        ach = ""
        if w is not None:
            a, p, unit, frac = roofline(w, med)
            ach = f"{a:10.1f} {100 * frac:7.1f}%"
            if w.unit == "B" and not short.startswith(("renorm", "qd_")):
                slicer_bytes += w.amount
                slicer_ms += med
        lines.append(f"{short[:58]:58s} {len(g):5d} {avg:10.4f} {statistics.median(ms):10.4f} {min(ms):10.4f} "
                     f"{max(ms):10.4f} {100 * sum(ms) / total:6.2f}  {ach}")
    lines.append("")
    for short, g in rows:
        w = kernel_work(short, m, n, k, ns, g[0].grid)
        if w is None:
            continue
        d = g[0]
        a, p, unit, frac = roofline(w, statistics.median(x.ms for x in g))
        lines.append(f"{short}: {w.note}; {w.amount:.4e} {w.unit} per launch -> {a:.2f} {unit} of {p:g} "
                     f"({100 * frac:.1f} %); grid {d.grid[0]}x{d.grid[1]}x{d.grid[2]} threads, workgroup "
                     f"{d.workgroup}, vgpr {d.vgpr}, agpr {d.agpr}, sgpr {d.sgpr}, lds {d.lds} B, scratch {d.scratch} B")
    if slicer_ms > 0:
        lines.append("")
        lines.append(f"slicer (exponent and slice passes): {slicer_bytes:.4e} B in {slicer_ms:.4f} ms of kernel time "
                     f"= {slicer_bytes / (slicer_ms * 1e-3) / 1e9:.1f} GB/s = "
                     f"{100 * slicer_bytes / (slicer_ms * 1e-3) / 1e9 / PEAK_HBM_GBS:.1f} % of {PEAK_HBM_GBS:g} GB/s")
    gemm = [g for s, g in rows if family(s) == "sliced_gemm_kernel"]
    if gemm:
        g = max(gemm, key=lambda gg: sum(d.ms for d in gg))
        lines.append("")
        lines.append("GEMM per-launch durations (ms): " + ", ".join(f"{d.ms:.3f}" for d in g))
        if bench and "roofline" in bench:
            r = bench["roofline"]
            lines.append(f"bench.py's live HIP-event figure for the GEMM in the same run: {r.get('launch_ms')} ms, "
                         f"{r.get('achieved')} {r.get('unit')}")
    lines.append("")
    lines.append(f"kernel_source_sha256_16: {source_hash()}")
    return "\n".join(lines) + "\n"


CALIB_KERNEL = "__amd_rocclr_copyBuffer"


def traffic_summary(fetch_dir: str, write_dir: str, m: int, n: int, k: int, calib_mib: int, ns: int = 8,
                    title: str = "", commands: list[str] | None = None) -> str:
    """HBM bytes per launch from FETCH_SIZE and WRITE_SIZE runs (KiB per
    dispatch), each scaled by what it reads for the calibration copy."""
    calib = calib_mib * (1 << 20)
    per: dict[str, dict[str, list[float]]] = {}
    scale = {}
    for counter, directory in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        disp = load_counters(directory)
        copies = [d for d in disp if CALIB_KERNEL in d.name and counter in d.counters]
        if not copies:
            raise ValueError(f"no calibration copy ({CALIB_KERNEL}) in {directory}")
        kib = max(d.counters[counter] for d in copies)
        scale[counter] = calib / (kib * 1024.0)
        for d in disp:
            if counter not in d.counters or any(s in d.name for s in ("__amd_rocclr", "at::", "elementwise")):
                continue
            per.setdefault(d.short, {}).setdefault(counter, []).append(d.counters[counter])
    lines = _header(title or f"HBM traffic per launch, {m}x{n}x{k}, {ns} slices", commands or [],
                    "rocprofv3 counter_collection.csv, KiB per dispatch, averaged over the launches")
    lines.append("#")
    lines.append(f"# calibration: a device copy of {calib_mib} MiB in the same runs reads FETCH_SIZE x "
                 f"{scale['FETCH_SIZE']:.4f} and WRITE_SIZE x {scale['WRITE_SIZE']:.4f} bytes per KiB counted")
    lines.append("# bytes = FETCH_SIZE KiB x 1024 x read scale + WRITE_SIZE KiB x 1024 x write scale; FETCH_SIZE "
                 "counts L2 misses served by the fabric (memory-side cache hits included)")
    lines.append("")
    lines.append(f"{'kernel':58s} {'fetch_KiB':>12s} {'write_KiB':>12s} {'bytes':>12s} {'algorithmic':>12s} "
                 f"{'ratio':>6s}")
    gemm_bytes = None
    for short, c in sorted(per.items(), key=lambda kv: -statistics.mean(kv[1].get("FETCH_SIZE", [0]))):
        f = statistics.mean(c.get("FETCH_SIZE", [0.0]))
        w = statistics.mean(c.get("WRITE_SIZE", [0.0]))
        b = f * 1024 * scale["FETCH_SIZE"] + w * 1024 * scale["WRITE_SIZE"]
        work = kernel_work(short, m, n, k, ns)
        alg = _algorithmic_bytes(short, work, m, n, k, ns)
        ratio = f"{b / alg:6.2f}" if alg else "     -"
        lines.append(f"{short[:58]:58s} {f:12.1f} {w:12.1f} {b:12.4e} {alg or 0:12.4e} {ratio}")
        if family(short) == "sliced_gemm_kernel" and work is not None:
            gemm_bytes = b if gemm_bytes is None else max(gemm_bytes, b)
    lines.append("")
    lines.append("algorithmic bytes: a GEMM reads every slice of both operands once and writes its outputs "
                 f"(8 ns B per operand entry + 8 B per output word); the slicer and exponent passes as in the "
                 "trace summary.")
    lines.append("")
    lines.append(f"kernel_source_sha256_16: {source_hash()}")
    if gemm_bytes is not None:
        lines.append(f"hbm_bytes_per_launch: {gemm_bytes:.6e}")
    return "\n".join(lines) + "\n"


def _algorithmic_bytes(short: str, work: Work | None, m: int, n: int, k: int, ns: int) -> float | None:
    if work is None:
        return None
    if work.unit == "B":
        return work.amount
    if family(short) == "sliced_gemm_kernel":
        args = template_args(short)
        words = 4 if len(args) > 1 and args[1] == "2" else 2
        return 8.0 * ns * (m * k + k * n) + 8.0 * words * m * n
    return None


def counters_summary(directories: list[str], m: int, n: int, k: int, ns: int = 8, title: str = "",
                     commands: list[str] | None = None) -> str:
    """SQ/GRBM counters of the sliced GEMM: matrix-core busy fraction, MFMA and
    LDS instruction counts against the schedule's."""
    rows = []
    for i, directory in enumerate(directories):
        disp = [d for d in load_counters(directory) if family(d.short) == "sliced_gemm_kernel"]
        if not disp:
            continue
        g = max(_group(disp).values(), key=len)
        for name in sorted(g[0].counters):
            rows.append((name, statistics.mean(d.counters[name] for d in g), i + 1, g[0].short))
    lines = _header(title or f"SQ / GRBM counters of the sliced GEMM, {m}x{n}x{k}", commands or [],
                    "rocprofv3 counter_collection.csv, summed over the counters' dimensions, averaged over the "
                    "launches")
    lines.append("")
    lines.append(f"{'counter':36s} {'per launch':>14s}")
    vals = {}
    for name, v, run, short in rows:
        lines.append(f"{name:36s} {v:14.4e}   (pass {run})")
        vals.setdefault(name, v)
    lines.append("")
    kernel = rows[0][3] if rows else ""
    args = template_args(kernel)
    paired = len(args) > 2 and args[2] == "true"
    prods = pair_products(ns) if paired else ns * (ns + 1) // 2
    expect = prods * (m // 16) * (n // 16) * (k // 4)
    if "SQ_INSTS_MFMA" in vals:
        lines.append(f"MFMA instructions: {vals['SQ_INSTS_MFMA']:.4e} = {prods} products x (m/16)(n/16)(k/4) "
                     f"= {expect:.4e} (ratio {vals['SQ_INSTS_MFMA'] / expect:.4f})")
    if "SQ_VALU_MFMA_BUSY_CYCLES" in vals and "GRBM_GUI_ACTIVE" in vals:
        cycles = vals["GRBM_GUI_ACTIVE"] / 8  # GRBM_GUI_ACTIVE sums the 8 XCDs
        busy = vals["SQ_VALU_MFMA_BUSY_CYCLES"] / (cycles * 1024)
        lines.append(f"MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE per XCD x 1024 SIMDs) = "
                     f"{100 * busy:.1f} %")
        lines.append(f"GPU cycles per launch (GRBM_GUI_ACTIVE per XCD): {cycles:.4e}")
    if "SQ_LDS_BANK_CONFLICT" in vals and "SQ_LDS_IDX_ACTIVE" in vals:
        lines.append(f"LDS bank conflicts: {vals['SQ_LDS_BANK_CONFLICT']:.4g} of {vals['SQ_LDS_IDX_ACTIVE']:.4e} "
                     "active LDS cycles")
    if "SQ_WAIT_INST_LDS" in vals and "SQ_WAVE_CYCLES" in vals:
        lines.append(f"LDS waits: SQ_WAIT_INST_LDS / SQ_WAVE_CYCLES = "
                     f"{100 * vals['SQ_WAIT_INST_LDS'] / vals['SQ_WAVE_CYCLES']:.2f} % of wave cycles")
    lines.append("")
    lines.append(f"kernel: {kernel}")
    lines.append(f"kernel_source_sha256_16: {source_hash()}")
    return "\n".join(lines) + "\n"


def read_summary_value_text(text: str, key: str) -> str | None:
    """The value of a `key: value` line of a summary, or None."""
    for line in text.splitlines():
        if not line.startswith("#") and line.startswith(key + ":"):
            return line.split(":", 1)[1].strip()
    return None


def read_summary_value(path: str, key: str) -> str | None:
    """The value of a `key: value` line of a summary file, or None."""
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        return read_summary_value_text(fh.read(), key)


# ---------------------------------------------------------------- command line


def _shape(text: str) -> tuple[int, int, int]:
    m, n, k = (int(x) for x in text.split(","))
    return m, n, k


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(prog="python -m extended_precision_gemm_amd.profiling", description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="what", required=True)
    for name in ("trace", "traffic", "counters"):
        p = sub.add_parser(name)
        p.add_argument("dirs", nargs="+")
        p.add_argument("--shape", required=True, type=_shape, help="M,N,K of the product")
        p.add_argument("--nslices", type=int, default=8)
        p.add_argument("--title", default="")
        p.add_argument("--command", action="append", default=[], help="a command that produced the input")
        p.add_argument("-o", "--output", default="-")
        if name == "trace":
            p.add_argument("--bench-json", default=None, help="bench.py's JSON line from the same run")
        if name == "traffic":
            p.add_argument("--calib-mib", type=int, required=True)
    a = ap.parse_args(argv)
    m, n, k = a.shape
    if a.what == "trace":
        bench = None
        if a.bench_json:
            import json
            with open(a.bench_json) as fh:
                for line in fh:
                    if line.lstrip().startswith("{"):
                        bench = json.loads(line)
        text = trace_summary(a.dirs[0], m, n, k, a.nslices, a.title, a.command, bench)
    elif a.what == "traffic":
        if len(a.dirs) != 2:
            ap.error("traffic takes FETCH_DIR WRITE_DIR")
        text = traffic_summary(a.dirs[0], a.dirs[1], m, n, k, a.calib_mib, a.nslices, a.title, a.command)
    else:
        text = counters_summary(a.dirs, m, n, k, a.nslices, a.title, a.command)
    if a.output == "-":
        sys.stdout.write(text)
    else:
        with open(a.output, "w") as fh:
            fh.write(text)
    return 0


if __name__ == "__main__":
    sys.exit(main())
