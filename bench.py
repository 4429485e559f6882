#!/usr/bin/env python3
"""Throughput of C = A·B on one MI355X through the library's C ABI.

One step = one GEMM call (dispatcher, main kernel, and the split-K reduce
when the plan has one) on resident device operands. The headline workload is
FP32 M = N = K = 2048 (uniform [-1, 1) from seed 2); ``--workload`` picks
another from the table in ``sam_inputs``. Before the headline is timed, the
sweep (on unless ``--no-sweep``) times every workload with the batch protocol
of page "Scale coverage exposes a remaining GEMM gap" (section "GEMM: frozen
schedules at larger dimensions": warmup, several rounds of batched launches,
median of round medians), plus a cold-cache single-launch time for the
HBM-bound skinny shapes; each entry carries its own roofline record. Running
it first also lets the clock settle under load, so that a short timed region
measures the kernel and not the clock ramp.

Prints one JSON line (rank 0, N = 1 only: this path runs on one GPU).

The CPU baseline leg times the oracle (test infrastructure, double precision,
as it stands) on a bounded slab of rows of the same workload.
"""
from __future__ import annotations

import argparse
import csv
import ctypes
import hashlib
import json
import math
import os
import statistics
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

PEAK_TFLOPS = {"f32": 157.3, "bf16": 2516.6, "f16": 2516.6, "mxfp8": 5000.0, "mxfp4": 10100.0}   # MI355X dense MFMA
PEAK_HBM_GBS = 8000.0


KERNEL_SOURCES = ["sam_kernels.hip", "sam_kernels_dma.hip", "sam_kernels_dma_t.hip", "sam_ring16.h", "sam_sk.h",
                  "sam_kernels_stream.hip", "sam_kernels_f32ring.hip", "sam_kernels_mx.hip", "sam_kernels_kq.hip",
                  "sam_kernels_kp.hip", "sam_dma.h", "sam_internal.h", "sam_variants.h", "sam_variants_mx.h"]

# Kernel function of a plan, by the leading letters of its variant name.
KERNEL_OF = {"t": "sam::gemm_kernel", "r": "sam::gemm16_dma_kernel", "q": "sam::gemm16_dma_kernel",
             "h": "sam::gemm16_dma_kernel", "s": "sam::stream_m_kernel / sam::stream_n_kernel",
             "f": "sam::gemm_f32_ring_kernel", "x": "sam::gemm_mx8_kernel", "kq": "sam::gemm_f32_kq_kernel",
             "kp": "sam::gemm_f32_kp_kernel"}


def kernel_name(plan) -> str:
    variant = plan["name"].split("_", 1)[1]
    return KERNEL_OF.get(variant[:2], KERNEL_OF.get(variant[0], "?"))


# The sources a kernel family is built from: a stored counter reading of one
# of its kernels stays valid while these are unchanged.
SOURCES_OF_KERNEL = {
    "sam::gemm_f32_ring_kernel": ["sam_kernels_f32ring.hip", "sam_dma.h", "sam_sk.h", "sam_internal.h",
                                  "sam_variants.h"],
    "sam::gemm16_dma_kernel": ["sam_ring16.h", "sam_kernels_dma.hip", "sam_dma.h", "sam_sk.h", "sam_internal.h",
                               "sam_variants.h"],
    "sam::gemm_mx8_kernel": ["sam_kernels_mx.hip", "sam_dma.h", "sam_internal.h", "sam_variants.h",
                             "sam_variants_mx.h"],
}


def src_digest(plan=None) -> str:
    """Hash of the sources of the plan's kernel (of every kernel source
    without a plan): a stored counter reading is only reported while the
    kernel it was taken on is unchanged."""
    names = SOURCES_OF_KERNEL.get(kernel_name(plan), KERNEL_SOURCES) if plan is not None else KERNEL_SOURCES
    h = hashlib.sha256()
    for name in names:
        p = ROOT / "shape_adaptive_matrix_amd" / "csrc" / name
        h.update(name.encode())
        h.update(p.read_bytes())
    return h.hexdigest()[:16]


def prepare_mx(w, torch, sam, si, variant=None, split=0):
    """Block-scaled workload: sam_gemm_mxfp8 / sam_gemm_mxfp4 (or the forced
    variant)."""
    ops = [torch.from_numpy(x).cuda() for x in si.make_mx_operands(w)]
    C = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")
    if variant is None:
        plan = sam.plan(w.M, w.N, w.K, w.dtype)
    else:
        plan = sam.variant_plan(variant, w.M, w.N, w.K, w.dtype, split)
    ws = sam.workspace_for(plan, C.device)
    L = sam.lib()
    stream = torch.cuda.current_stream()
    fp4 = w.dtype == "mxfp4"
    fmts = () if fp4 else (sam.FP8_FORMATS[w.fmt_a], sam.FP8_FORMATS[w.fmt_b])
    args = (*fmts, *(ctypes.c_void_p(t.data_ptr()) for t in ops), ctypes.c_void_p(C.data_ptr()),
            w.M, w.N, w.K, ctypes.c_void_p(ws.data_ptr()) if ws is not None else None,
            ws.numel() * 4 if ws is not None else 0, ctypes.c_void_p(stream.cuda_stream))
    if variant is None:
        fn = L.sam_gemm_mxfp4 if fp4 else L.sam_gemm_mxfp8
    else:
        forced = L.sam_gemm_mxfp4_variant if fp4 else L.sam_gemm_mxfp8_variant

        def fn(*a):
            return forced(variant, plan["split_k"], *a)

    def step():
        rc = fn(*args)
        if rc != 0:
            raise RuntimeError(f"{sam.STATUS.get(rc, rc)}: {sam.last_error()}")

    return {"step": step, "plan": plan, "keep": (ops, C, ws), "stream": stream}


def prepare(w, torch, sam, si, variant=None, split=0):
    if w.dtype in ("mxfp8", "mxfp4"):
        return prepare_mx(w, torch, sam, si, variant, split)
    A, B = si.make_operands(w)
    if w.dtype == "f32":
        dA = torch.from_numpy(A).cuda()
        dB = torch.from_numpy(B).cuda()
    else:
        t = {"bf16": torch.bfloat16, "f16": torch.float16}[w.dtype]
        dA = torch.from_numpy(A.view("int16")).cuda().view(t)
        dB = torch.from_numpy(B.view("int16")).cuda().view(t)
    del A, B
    C = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")
    if variant is None:
        plan = sam.plan(w.M, w.N, w.K, w.dtype)
    else:
        plan = sam.variant_plan(variant, w.M, w.N, w.K, w.dtype, split)
    ws = sam.workspace_for(plan, dA.device)
    L = sam.lib()
    stream = torch.cuda.current_stream()
    args = (ctypes.c_void_p(dA.data_ptr()), ctypes.c_void_p(dB.data_ptr()), ctypes.c_void_p(C.data_ptr()),
            w.M, w.N, w.K, ctypes.c_void_p(ws.data_ptr()) if ws is not None else None,
            ws.numel() * 4 if ws is not None else 0, ctypes.c_void_p(stream.cuda_stream))
    if variant is None:
        fn = {"f32": L.sam_gemm_f32, "bf16": L.sam_gemm_bf16, "f16": L.sam_gemm_f16}[w.dtype]
    else:
        forced = L.sam_gemm_variant
        code = sam.DTYPES[w.dtype]

        def fn(*a):
            return forced(variant, code, plan["split_k"], *a)

    def step():
        rc = fn(*args)
        if rc != 0:
            raise RuntimeError(f"{sam.STATUS.get(rc, rc)}: {sam.last_error()}")

    return {"step": step, "plan": plan, "keep": (dA, dB, C, ws), "stream": stream}


def prepare_ex(w, torch, sam, si, ta: bool, tb: bool, alpha: float, beta: float, pad: int):
    """One call of the general entry point sam_gemm_ex on the workload's
    operands, stored transposed where asked and with `pad` extra elements per
    row (the leading dimensions); C is read when beta != 0."""
    import numpy as np
    A, B = si.make_operands(w)
    if ta:
        A = np.ascontiguousarray(A.T)
    if tb:
        B = np.ascontiguousarray(B.T)

    def dev(x):
        x = np.pad(x, ((0, 0), (0, pad)))
        t = torch.from_numpy(x if w.dtype == "f32" else x.view("int16")).cuda()
        return t if w.dtype == "f32" else t.view({"bf16": torch.bfloat16, "f16": torch.float16}[w.dtype])

    dA, dB = dev(A), dev(B)
    del A, B
    lda, ldb, ldc = dA.shape[1], dB.shape[1], w.N + pad
    C = torch.zeros((w.M, ldc), dtype=torch.float32, device="cuda")
    n = sam.ex_workspace_bytes(w.M, w.N, w.K, ta, tb, lda, ldb, ldc, alpha, beta, w.dtype)
    ws = torch.empty((n + 3) // 4, dtype=torch.float32, device="cuda") if n else None
    L = sam.lib()
    stream = torch.cuda.current_stream()
    args = (sam.DTYPES[w.dtype], int(ta), int(tb), w.M, w.N, w.K, ctypes.c_float(alpha),
            ctypes.c_void_p(dA.data_ptr()), lda, ctypes.c_void_p(dB.data_ptr()), ldb, ctypes.c_float(beta),
            ctypes.c_void_p(C.data_ptr()), ldc, ctypes.c_void_p(ws.data_ptr()) if ws is not None else None,
            n, ctypes.c_void_p(stream.cuda_stream))

    def step():
        rc = L.sam_gemm_ex(*args)
        if rc != 0:
            raise RuntimeError(f"{sam.STATUS.get(rc, rc)}: {sam.last_error()}")

    return {"step": step, "plan": sam.plan(w.M, w.N, w.K, w.dtype), "keep": (dA, dB, C, ws), "stream": stream}


def profile_kernel_avg_us(workload: str, kernel: str):
    """Average duration (us) of `kernel` in the committed rocprofv3
    kernel-trace summary of `workload` (profiles/<kernel>_<workload>.txt,
    the kernel_stats.csv row it quotes), with the file's name; None if there
    is none."""
    short = kernel.split("::")[-1]
    p = ROOT / "profiles" / f"{short}_{workload}.txt"
    if not p.exists():
        return None
    for line in p.read_text().splitlines():
        if line.startswith('"') and short + "<" in line.split(",")[0]:
            cells = next(csv.reader([line]))
            return {"file": str(p.relative_to(ROOT)), "kernel": cells[0], "calls": int(cells[1]),
                    "avg_us": round(float(cells[3]) / 1e3, 3)}
    return None


def pads(w, plan) -> bool:
    """Whether the plan copies an operand into padded rows first (16-bit ring
    plans with K or N not a multiple of 8, FP32 padding forms with K or N not
    a multiple of 4)."""
    form = plan["name"].split("_", 1)[1]
    if w.dtype in ("bf16", "f16") and form[0] in "rqh":
        return w.K % 8 != 0 or w.N % 8 != 0
    return "_pad" in form and (w.K % 4 != 0 or w.N % 4 != 0)


def roofline_of(w, t_ms: float, plan) -> dict:
    """Roofline record of one timed workload: MFMA-bound for the dense
    shapes (2MNK FLOP against the dtype's peak), HBM-bound for the skinny ones
    (algorithmic bytes against 8 TB/s)."""
    skinny = min(w.M, w.N) <= 16
    split = plan["split_k"] > 1
    if skinny:
        achieved = w.alg_bytes / t_ms / 1e6
        rec = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
               "frac": round(achieved / PEAK_HBM_GBS, 4)}
    else:
        achieved = w.flops / t_ms / 1e9
        rec = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_TFLOPS[w.dtype], "unit": "TFLOP/s",
               "frac": round(achieved / PEAK_TFLOPS[w.dtype], 4)}
    rec["traffic"] = None if split else load_traffic(w.name, src_digest(plan))
    rec["kernel"] = kernel_name(plan) + (" + sam::splitk_reduce_kernel" if split else "") + \
        (" + sam::sk_fixup_kernel" if plan["split_k"] == -1 else "") + (" + sam::pad_kernel" if pads(w, plan) else "")
    if plan["split_k"] == 1:
        prof = profile_kernel_avg_us(w.name, kernel_name(plan))
        if prof is not None:
            prof["frac_at_profile_avg"] = round(
                (w.flops / (prof["avg_us"] * 1e-6) / 1e12 / PEAK_TFLOPS[w.dtype]) if not skinny else
                (w.alg_bytes / (prof["avg_us"] * 1e-6) / 1e9 / PEAK_HBM_GBS), 4)
            rec["profile"] = prof
    return rec


def time_steps(torch, step, steps: int) -> float:
    """Milliseconds for `steps` back-to-back calls, HIP events on the stream the
    kernels run on (torch's current stream, which the calls are given)."""
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(steps):
        step()
    e.record()
    e.synchronize()
    return s.elapsed_time(e)


def sweep(torch, sam, si, rounds: int = 5):
    """Every workload: median over rounds of the per-launch time of a batch
    lasting >= 20 ms; cold-cache single launches for the skinny shapes."""
    out = []
    flush = None
    for w in si.WORKLOADS + si.MX_WORKLOADS + si.LLM_WORKLOADS + si.LLM_MX_WORKLOADS:
        g = prepare(w, torch, sam, si)
        step = g["step"]
        for _ in range(3):
            step()
        torch.cuda.synchronize()
        one = time_steps(torch, step, 3) / 3
        n = max(3, math.ceil(20.0 / max(one, 1e-3)))
        meds = []
        for _ in range(rounds):
            samples = [time_steps(torch, step, n) / n for _ in range(5)]
            meds.append(statistics.median(samples))
        t_ms = statistics.median(meds)
        rec = {
            "workload": w.name, "dtype": w.dtype, "M": w.M, "N": w.N, "K": w.K,
            "plan": g["plan"]["name"], "ms": round(t_ms, 5),
            "ms_range": [round(min(meds), 5), round(max(meds), 5)],
            "tflops": round(w.flops / t_ms / 1e9, 2),
            "pct_mfma_peak": round(100 * w.flops / t_ms / 1e9 / PEAK_TFLOPS[w.dtype], 1),
            "alg_gbs": round(w.alg_bytes / t_ms / 1e6, 1),
            "roofline": roofline_of(w, t_ms, g["plan"]),
        }
        if min(w.M, w.N) <= 16:
            # Evict the operands by reading 1 GiB: a read leaves clean lines,
            # whereas a fill would leave dirty ones whose write-back the timed
            # launch would pay for.
            if flush is None:
                flush = torch.ones(1024 * 1024 * 1024 // 4, dtype=torch.float32, device="cuda")
            cold = []
            for _ in range(20):
                flush.sum()
                cold.append(time_steps(torch, step, 1))
            c_ms = statistics.median(cold)
            rec["cold_ms"] = round(c_ms, 5)
            rec["cold_alg_gbs"] = round(w.alg_bytes / c_ms / 1e6, 1)
            rec["cold_pct_hbm"] = round(100 * w.alg_bytes / c_ms / 1e6 / PEAK_HBM_GBS, 1)
        out.append(rec)
        del g
        torch.cuda.empty_cache()
    return out


def cpu_baseline(w, si, seconds: float):
    """The oracle (as it stands) on a bounded sample of the workload: a slab of
    rows sized to take about `seconds` on the host cores, or the whole product
    repeated until that long when the whole product is quicker."""
    import oracle
    o = oracle.get()
    threads = o.max_threads()
    if w.dtype == "mxfp8":
        A, SA, Bt, SB = si.make_mx_operands(w)

        def slab(n):
            o.gemm_mxfp8(w.fmt_a, w.fmt_b, A[:n], SA[:n], Bt, SB)
    elif w.dtype == "mxfp4":
        A, SA, Bt, SB = si.make_mx_operands(w)

        def slab(n):
            o.gemm_mxfp4(A[:n], SA[:n], Bt, SB)
    else:
        A, B = si.make_operands(w)

        def slab(n):
            o.gemm_rows(w.dtype, A, B, 0, n)
    rows = max(1, min(w.M, 16))
    t0 = time.perf_counter()
    slab(rows)
    t = time.perf_counter() - t0
    target = max(1, min(w.M, int(rows * seconds / max(t, 1e-6))))
    reps, elapsed = 0, 0.0
    while elapsed < 0.8 * seconds or reps == 0:
        t0 = time.perf_counter()
        slab(target)
        elapsed += time.perf_counter() - t0
        reps += 1
    flops = 2.0 * target * w.N * w.K * reps
    what = (f"rows 0..{target - 1}" if target < w.M else "all rows") + f" of {w.name}"
    return {"value": round(flops / elapsed / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{what} (N={w.N}, K={w.K}) x{reps}, {elapsed:.1f} s, double-precision i-k-j loop"}


def cpu_model() -> str:
    try:
        for line in Path("/proc/cpuinfo").read_text().splitlines():
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def load_traffic(workload: str, digest: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; else None."""
    p = ROOT / "profiles" / f"traffic_{workload}.json"
    if not p.exists():
        return None
    d = json.loads(p.read_text())
    if d.get("src_digest") != digest:
        return None
    return d.get("hbm_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--workload", default="f32_2048")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--shape", default=None,
                    help="M,N,K[,dtype]: time an ad-hoc shape (uniform / normal inputs) instead of a named workload")
    ap.add_argument("--variant", type=int, default=None,
                    help="force this variant id (calibration); default: the dispatcher's plan")
    ap.add_argument("--split", type=int, default=0, help="split-K for --variant (0: the variant's pick)")
    ap.add_argument("--ex", default=None, metavar="TA,TB,ALPHA,BETA,PAD",
                    help="time the general entry point instead (e.g. T,N,2,1,8: A stored transposed, "
                         "alpha 2, beta 1, rows padded by 8 elements)")
    ap.add_argument("--ceilings", action="store_true",
                    help="also run the MFMA-loop / HBM-copy ceiling probe and report its figures")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run a plain device copy of this many bytes (counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this GEMM path runs on one GPU; --gpus {args.gpus} / WORLD_SIZE {world} "
              "is not supported (the single-GPU kernel is the unit that would be sharded).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import sam_inputs as si
    import shape_adaptive_matrix_amd as sam

    if args.copy_bytes:
        n = args.copy_bytes // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n * 4, "launches": 5}))
        return

    sam.device_check()
    if args.shape:
        parts = args.shape.split(",")
        M, N, K = (int(x) for x in parts[:3])
        dt = parts[3] if len(parts) > 3 else "f32"
        dist = {"f32": "uniform", "mxfp8": "mx_normal", "mxfp4": "mx_normal"}.get(dt, "normal16")
        fmt = "e2m1" if dt == "mxfp4" else "e4m3"
        w = si.Workload(f"{dt}_{M}x{N}x{K}", dt, M, N, K, dist, 99, fmt_a=fmt, fmt_b=fmt)
    else:
        w = si.by_name(args.workload)
    if args.ex:
        ta, tb, alpha, beta, pad = args.ex.split(",")
        g = prepare_ex(w, torch, sam, si, ta == "T", tb == "T", float(alpha), float(beta), int(pad))
    else:
        g = prepare(w, torch, sam, si, args.variant, args.split)
    step = g["step"]
    digest = src_digest(g["plan"])
    # The sweep runs first: after it the clock has settled under load, so a
    # short timed region measures the kernel rather than the clock ramp.
    sweep_rec = None
    if not args.no_sweep:
        sweep_rec = sweep(torch, sam, si)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms = time_steps(torch, step, args.steps)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = ms / args.steps
    tflops = w.flops / ms_step / 1e9

    split = g["plan"]["split_k"] > 1
    prof = None if (args.ex or args.variant is not None or args.shape or split) else \
        profile_kernel_avg_us(w.name, kernel_name(g["plan"]))
    if prof is not None:
        # The committed kernel trace of the same command: the fraction at its
        # average kernel duration, next to the event-timed one above.
        prof["frac_at_profile_avg"] = round(w.flops / (prof["avg_us"] * 1e-6) / 1e12 / PEAK_TFLOPS[w.dtype], 4)
    line = {
        "metric": "GEMM TFLOP/s and % of MFMA peak on 1 MI355X, fp32 and bf16, D=2048-8192",
        "value": round(tflops, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": f"{w.name}: C=A*B, M={w.M} N={w.N} K={w.K}, {w.dtype} operands, "
                               f"FP32 accumulate/output, {w.dist} inputs seed {w.seed}",
                   "M": w.M, "N": w.N, "K": w.K, "plan": g["plan"]["name"],
                   **({"general_entry_point": args.ex} if args.ex else {})},
        "pct_mfma_peak": round(100 * tflops / PEAK_TFLOPS[w.dtype], 2),
        "wall_s": round(wall, 4),
        "roofline": {
            "bound": "mfma", "achieved": round(tflops, 3), "peak": PEAK_TFLOPS[w.dtype],
            "unit": "TFLOP/s", "frac": round(tflops / PEAK_TFLOPS[w.dtype], 4),
            "traffic": None if split else load_traffic(w.name, digest),
            "kernel": kernel_name(g["plan"]) + (" + sam::splitk_reduce_kernel" if split else ""),
            "per_launch_flops": w.flops, "src_digest": digest,
            "timing": f"HIP events on the launch stream around {args.steps} back-to-back calls, "
                      f"after {args.warmup} warm-up calls" + (" and the sweep" if sweep_rec else ""),
            "profile": prof,
        },
        "build": sam.build_info(),
    }
    del g
    torch.cuda.empty_cache()
    if sweep_rec is not None:
        line["sweep"] = sweep_rec
    if args.ceilings:
        import subprocess
        exe = ROOT / "shape_adaptive_matrix_amd" / "microbench" / "sam_ceilings"
        r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
        line["ceilings"] = json.loads(r.stdout) if r.returncode == 0 else {"error": r.stderr[-500:]}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, si, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
