"""Summaries of rocprofv3 output for the profiles kept with the library.

The measurement contract quotes, next to the event-timed throughput, the
average duration of the dominant kernel from a rocprofv3 kernel trace of the
same command, and the HBM-side bytes per launch from two counter runs
(FETCH_SIZE, then WRITE_SIZE) scaled by what the same counters read for a
plain device copy of known size. This module turns the CSV files rocprofv3
writes into those summaries; it runs no GPU code itself.

    python -m shape_adaptive_matrix_amd.profiling trace KT_DIR WORKLOAD KERNEL OUT --command CMD [--bench-json F]
    python -m shape_adaptive_matrix_amd.profiling traffic FETCH_DIR WRITE_DIR COPY_FETCH_DIR COPY_WRITE_DIR \\
        WORKLOAD KERNEL OUT --digest D --alg-bytes N --copy-bytes N --commands JSON
    python -m shape_adaptive_matrix_amd.profiling counters DIR KERNEL

KERNEL is a substring of the kernel's full name (e.g. "gemm_f32_ring_kernel<").
"""
from __future__ import annotations

import argparse
import csv
import json
import sys
from collections import defaultdict
from pathlib import Path


def _one(d: Path, suffix: str) -> Path:
    hits = sorted(Path(d).rglob(f"*{suffix}"))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    return hits[0]


def kernel_stats(kt_dir) -> tuple[str, list[str]]:
    """Header line and data lines of the kernel_stats.csv of a kernel trace."""
    lines = _one(Path(kt_dir), "kernel_stats.csv").read_text().splitlines()
    return lines[0], lines[1:]


def counter_means(pmc_dir, kernel: str) -> dict:
    """Per counter: its mean value per dispatch of the kernels whose name
    contains `kernel`, and the number of such dispatches."""
    sums, disp = defaultdict(float), defaultdict(set)
    with _one(Path(pmc_dir), "counter_collection.csv").open() as f:
        for row in csv.DictReader(f):
            if kernel in row["Kernel_Name"]:
                sums[row["Counter_Name"]] += float(row["Counter_Value"])
                disp[row["Counter_Name"]].add(row["Dispatch_Id"])
    return {c: {"mean": sums[c] / len(disp[c]), "dispatches": len(disp[c])} for c in sums}


def kernel_full_name(pmc_dir, kernel: str) -> str:
    with _one(Path(pmc_dir), "counter_collection.csv").open() as f:
        for row in csv.DictReader(f):
            if kernel in row["Kernel_Name"]:
                return row["Kernel_Name"]
    raise KeyError(kernel)


def trace_text(kt_dir, workload: str, kernel: str, command: str, bench_json=None) -> str:
    header, rows = kernel_stats(kt_dir)
    cells_of = [next(csv.reader([r])) for r in rows]
    dom = [c for c in cells_of if kernel in c[0]]
    if not dom:
        raise KeyError(f"{kernel} not in the kernel trace")
    cells = dom[0]
    lib = [(r, c) for r, c in zip(rows, cells_of) if "sam::" in c[0]]   # every kernel of the library's plan
    avg_us = float(cells[3]) / 1e3
    per_call_us = sum(float(c[2]) for _, c in lib) / float(cells[1]) / 1e3
    short = kernel.rstrip("<").split("::")[-1]
    out = [f"# {short}, {workload} -- kernel trace", "",
           "Command (run from the repository root on one MI355X, ROCm 7.2):", "", f"    {command}", "",
           "kernel_stats.csv, the rows of the library's kernels:", "", header, *[r for r, _ in lib], "",
           f"Average duration of {short} under the profiler: {avg_us:.1f} us over {cells[1]} dispatches."]
    if len(lib) > 1:
        out.append(f"All of the plan's kernels together: {per_call_us:.1f} us per call.")
    if bench_json:
        d = json.loads(Path(bench_json).read_text().strip().splitlines()[-1])
        ev_us = d["ms_per_step"] * 1e3
        out += [f"The same command without the profiler, HIP events on the launch stream: {ev_us:.1f} us per "
                f"call ({d['value']:.1f} {d['unit']}, plan {d['config'].get('plan', '?')}).",
                f"The two differ by {100 * (per_call_us - ev_us) / ev_us:+.1f}%."]
    return "\n".join(out) + "\n"


def traffic_record(fetch_dir, write_dir, cfetch_dir, cwrite_dir, workload: str, kernel: str, digest: str,
                   alg_bytes: int, copy_bytes: int, commands: dict) -> dict:
    fetch = counter_means(fetch_dir, kernel)["FETCH_SIZE"]["mean"]
    write = counter_means(write_dir, kernel)["WRITE_SIZE"]["mean"]
    # The copy: the largest dispatch of the copy run (the device-to-device
    # copy kernel; the fill that creates the source is smaller in FETCH).
    cf = max(_copy_values(cfetch_dir, "FETCH_SIZE"))
    cw = max(_copy_values(cwrite_dir, "WRITE_SIZE"))
    true_kib = copy_bytes / 1024
    sf, sw = true_kib / cf, true_kib / cw
    hbm = int(round((fetch * sf + write * sw) * 1024))
    return {"workload": workload, "kernel": kernel_full_name(fetch_dir, kernel), "src_digest": digest,
            "commands": commands, "fetch_kib_per_launch": round(fetch, 1), "write_kib_per_launch": round(write, 1),
            "copy": {"bytes": copy_bytes, "fetch_kib": round(cf, 1), "write_kib": round(cw, 1)},
            "scale": {"fetch": round(sf, 4), "write": round(sw, 4)},
            "hbm_bytes_per_launch": hbm, "algorithmic_bytes_per_launch": alg_bytes,
            "ratio_to_algorithmic": round(hbm / alg_bytes, 3),
            "note": "FETCH_SIZE / WRITE_SIZE count L2-to-fabric traffic (Infinity Cache hits included), each "
                    "scaled by the ratio of a plain copy's true bytes to what the same counter reads for it."}


def _copy_values(pmc_dir, counter: str) -> list[float]:
    vals = []
    with _one(Path(pmc_dir), "counter_collection.csv").open() as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] == counter and "copyBuffer" in row["Kernel_Name"]:
                vals.append(float(row["Counter_Value"]))
    if not vals:
        raise KeyError(f"no copy dispatch with {counter}")
    return vals


def mfma_row(pmc_dir, workload: str, kernel: str, event_us=None) -> dict:
    """MFMA utilisation of one kernel from the SQ_VALU_MFMA_BUSY_CYCLES /
    SQ_INSTS_VALU_MFMA_MOPS_* / GRBM_GUI_ACTIVE run: MFMA-busy SIMD-cycles
    over (1024 SIMDs x kernel cycles), kernel cycles = GRBM_GUI_ACTIVE / 8
    XCDs, and the clock those cycles imply at the event-timed duration."""
    m = counter_means(pmc_dir, kernel)
    cyc = m["GRBM_GUI_ACTIVE"]["mean"] / 8
    mops = sum(m[c]["mean"] for c in m if c.startswith("SQ_INSTS_VALU_MFMA_MOPS_"))
    row = {"workload": workload, "kernel": kernel_full_name(pmc_dir, kernel), "kernel_cycles": cyc,
           "mops_x512": mops * 512, "mfma_util": m["SQ_VALU_MFMA_BUSY_CYCLES"]["mean"] / (1024 * cyc)}
    if event_us:
        row["clock_ghz"] = cyc / (event_us * 1e3)
    return row


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("kt_dir"), t.add_argument("workload"), t.add_argument("kernel"), t.add_argument("out")
    t.add_argument("--command", required=True)
    t.add_argument("--bench-json", default=None)
    r = sub.add_parser("traffic")
    for a in ("fetch_dir", "write_dir", "cfetch_dir", "cwrite_dir", "workload", "kernel", "out"):
        r.add_argument(a)
    r.add_argument("--digest", required=True)
    r.add_argument("--alg-bytes", type=int, required=True)
    r.add_argument("--copy-bytes", type=int, required=True)
    r.add_argument("--commands", required=True, help="JSON object of the four commands")
    c = sub.add_parser("counters")
    c.add_argument("dir"), c.add_argument("kernel")
    a = ap.parse_args(argv)
    if a.cmd == "trace":
        Path(a.out).write_text(trace_text(a.kt_dir, a.workload, a.kernel, a.command, a.bench_json))
    elif a.cmd == "traffic":
        rec = traffic_record(a.fetch_dir, a.write_dir, a.cfetch_dir, a.cwrite_dir, a.workload, a.kernel, a.digest,
                             a.alg_bytes, a.copy_bytes, json.loads(a.commands))
        Path(a.out).write_text(json.dumps(rec, indent=1) + "\n")
    else:
        print(json.dumps(counter_means(a.dir, a.kernel), indent=1))
    return 0


if __name__ == "__main__":
    sys.exit(main())
