"""Offline tuning: measure every admissible (variant, split-K) pair on a fixed
set of shapes and freeze the fastest into the dispatcher's table.

Two steps, so that selection at run time never times anything (the
measured-tactic shortlist idea of page "fix(fp4_gemm autotune) SM107 kernel
family excluded from autotune candidates and heuristics update - #4856",
section "Reviewer Notes", with the result frozen in source; the same shape
always gets the same plan):

  1. on a gfx950 machine, measure and append JSON lines to a record:
        python -m shape_adaptive_matrix_amd.tune measure shape_adaptive_matrix_amd/tuning/tuning_sweep.jsonl
  2. anywhere, turn the record into the frozen table:
        python -m shape_adaptive_matrix_amd.tune emit shape_adaptive_matrix_amd/tuning/tuning_sweep.jsonl
     which rewrites csrc/sam_tuned.h, and a readable summary with
        python -m shape_adaptive_matrix_amd.tune report shape_adaptive_matrix_amd/tuning/tuning_sweep.jsonl

Timing protocol per candidate: 3 warm-up calls, then the median of 5
batches of back-to-back calls lasting at least 15 ms each, HIP events on the
launch stream; skinny shapes (at most 16 rows or columns of C, HBM-bound)
instead take the median of 15 single launches, each after a 1 GiB read that
evicts the operands. Inputs are the seeded generators of ``sam_inputs``.
"""
from __future__ import annotations

import ctypes
import json
import statistics
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
TUNED_H = PKG / "csrc" / "sam_tuned.h"
DTYPE_CODE = {"f32": 0, "bf16": 1, "f16": 2, "mxfp8": 3, "mxfp4": 4}

# Shapes beyond the named workloads: square sizes between and around them,
# K-heavy and K-light rectangles, skinny-ish panels, and the LLM-like shapes
# of page "Measured data point on fixed-tile vs shape-adaptive GEMM".
EXTRA = {
    "f32": [(512, 512, 512), (1024, 1024, 1024), (1536, 1536, 1536), (3072, 3072, 3072),
            (6144, 6144, 6144), (1000, 1000, 1000), (3000, 3000, 3000), (2048, 2048, 512),
            (2048, 2048, 8192), (4096, 4096, 1024), (64, 4096, 4096), (4096, 64, 4096),
            (32, 8192, 8192), (256, 11008, 4096), (4096, 4096, 11008), (2049, 4097, 1025),
            (5000, 5000, 5000), (7168, 7168, 7168)],
    "bf16": [(1024, 1024, 1024), (2048, 2048, 2048), (3072, 3072, 3072), (6144, 6144, 6144),
             (4096, 4096, 1024), (2048, 8192, 2048), (256, 11008, 4096), (4096, 4096, 11008),
             (2049, 4097, 1025), (5120, 5120, 5120), (8192, 8192, 8190), (1536, 1536, 1536),
             (2560, 2560, 2560), (3584, 3584, 3584), (7168, 7168, 7168)],
    "f16": [(2048, 2048, 2048), (6144, 6144, 6144), (4096, 4096, 11008), (256, 11008, 4096), (2049, 4097, 1025)],
    "mxfp8": [(2048, 2048, 2048), (3072, 3072, 3072), (6144, 6144, 6144), (4096, 4096, 1024),
              (256, 11008, 4096), (4096, 4096, 11008), (2048, 8192, 2048)],
    "mxfp4": [(2048, 2048, 2048), (6144, 6144, 6144), (4096, 4096, 11008), (256, 11008, 4096)],
}

SPLITS = (1, 2, 3, 4, 6, 8, 12, 16)

# Shapes with at most this many rows or columns of C are bound by reading
# the large operand from HBM once; they are timed cold (operands evicted
# before each launch), the condition under which such a product runs when
# its large operand is a weight matrix streamed from memory.
COLD_EDGE = 16


def shapes():
    import sam_inputs as si
    out = [(w.dtype, w.M, w.N, w.K, w.name) for w in si.WORKLOADS + si.MX_WORKLOADS
           if (w.fmt_a, w.fmt_b) in (("e4m3", "e4m3"), ("e2m1", "e2m1"))]
    seen = {(d, m, n, k) for d, m, n, k, _ in out}
    for dt, lst in EXTRA.items():
        for (m, n, k) in lst:
            if (dt, m, n, k) not in seen:
                out.append((dt, m, n, k, f"{dt}_{m}x{n}x{k}"))
                seen.add((dt, m, n, k))
    return out


def candidates(sam, dt, M, N, K):
    """(variant, split, raster) triples: every admissible variant with its
    own split and raster choice and its stream-K form (split -1) where it has
    one; for the four variants the cost model ranks best, the other raster
    order (M-major 0 / N-major 1) too, and, when their tile count leaves CUs
    idle (fewer tiles than CUs, or a last round of tiles less than 90% full),
    the other admissible splits."""
    own = []
    for vid in range(sam.variant_count()):
        try:
            own.append(sam.variant_plan(vid, M, N, K, dt, 0))
        except sam.SamError:
            continue
    out = {(p["variant_id"], p["split_k"], p["raster_n"]) for p in own}
    for p in own:   # stream-K forms (split -1) where the variant has one
        try:
            q = sam.variant_plan(p["variant_id"], M, N, K, dt, -1)
            out.add((p["variant_id"], -1, q["raster_n"]))
        except sam.SamError:
            pass
    mx = dt in ("mxfp8", "mxfp4")   # block-scaled calls take the cost model's raster order
    for p in sorted(own, key=lambda p: (p["est_us"], p["variant_id"]))[:4]:
        if not mx:
            try:
                sam.variant_plan(p["variant_id"], M, N, K, dt, p["split_k"], 1 - p["raster_n"])
                out.add((p["variant_id"], p["split_k"], 1 - p["raster_n"]))
            except sam.SamError:
                pass
        tiles = -(-M // p["tile_m"]) * -(-N // p["tile_n"])
        if tiles >= 256 and tiles / (256 * -(-tiles // 256)) >= 0.9:
            continue
        for s in SPLITS:
            try:
                q = sam.variant_plan(p["variant_id"], M, N, K, dt, s)
                out.add((p["variant_id"], s, q["raster_n"]))
            except sam.SamError:
                pass
    return sorted(out)


def model_plan(sam, dt, M, N, K):
    """The cost model's own pick, ignoring the frozen table."""
    return sam.plan_model(M, N, K, dt)


def measure(record: Path, only=None):
    import torch

    import sam_inputs as si
    import shape_adaptive_matrix_amd as sam

    sam.device_check()
    flush = None
    done = set()
    if record.exists():
        for line in record.read_text().splitlines():
            r = json.loads(line)
            done.add((r["dtype"], r["M"], r["N"], r["K"], r["variant"], r["split"], r.get("raster", 0)))
    with record.open("a") as f:
        for (dt, M, N, K, name) in shapes():
            if only and name not in only:
                continue
            dist = {"f32": "uniform", "mxfp8": "mx_normal", "mxfp4": "mx_normal"}.get(dt, "normal16")
            fmt = "e2m1" if dt == "mxfp4" else "e4m3"
            w = si.Workload(name, dt, M, N, K, dist, 77, fmt_a=fmt, fmt_b=fmt)
            if dt in ("mxfp8", "mxfp4"):
                mx = [torch.from_numpy(x).cuda() for x in si.make_mx_operands(w)]
                dA = mx[0]
            elif dt == "f32":
                A, B = si.make_operands(w)
                dA, dB = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
            else:
                A, B = si.make_operands(w)
                t = {"bf16": torch.bfloat16, "f16": torch.float16}[dt]
                dA = torch.from_numpy(A.view("int16")).cuda().view(t)
                dB = torch.from_numpy(B.view("int16")).cuda().view(t)
            C = torch.empty((M, N), dtype=torch.float32, device="cuda")
            stream = torch.cuda.current_stream()
            auto = model_plan(sam, dt, M, N, K)
            cold = min(M, N) <= COLD_EDGE
            if cold and flush is None:
                flush = torch.ones(1024 * 1024 * 1024 // 4, dtype=torch.float32, device="cuda")
            print(f"[tune] {name}: {len(candidates(sam, dt, M, N, K))} candidates", flush=True)
            for (vid, split, raster) in candidates(sam, dt, M, N, K):
                if (dt, M, N, K, vid, split, raster) in done:
                    continue
                p = sam.variant_plan(vid, M, N, K, dt, split, raster if dt not in ("mxfp8", "mxfp4") else -1)
                ws = sam.workspace_for(p, dA.device)
                tail = (ctypes.c_void_p(C.data_ptr()), M, N, K, ctypes.c_void_p(ws.data_ptr()) if ws is not None else None,
                        ws.numel() * 4 if ws is not None else 0, ctypes.c_void_p(stream.cuda_stream))
                if dt == "mxfp8":   # E4M3 operands, scales as drawn
                    fn = sam.lib().sam_gemm_mxfp8_variant
                    args = (vid, split, 0, 0, *(ctypes.c_void_p(x.data_ptr()) for x in mx), *tail)
                elif dt == "mxfp4":
                    fn = sam.lib().sam_gemm_mxfp4_variant
                    args = (vid, split, *(ctypes.c_void_p(x.data_ptr()) for x in mx), *tail)
                else:
                    fn = sam.lib().sam_gemm_variant_r
                    args = (vid, sam.DTYPES[dt], split, raster, ctypes.c_void_p(dA.data_ptr()),
                            ctypes.c_void_p(dB.data_ptr()), *tail)
                for _ in range(3):
                    rc = fn(*args)
                    if rc != 0:
                        raise RuntimeError(f"{name} variant {vid} split {split}: {sam.last_error()}")
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                if cold:
                    # HBM-bound skinny shape: single launches, each after a
                    # 1 GiB read that evicts the operands (a read leaves clean
                    # lines, so no write-back lands in the timed launch).
                    samples = []
                    for _ in range(15):
                        flush.sum()
                        e0.record()
                        fn(*args)
                        e1.record()
                        e1.synchronize()
                        samples.append(e0.elapsed_time(e1))
                    ms = statistics.median(samples)
                else:
                    e0.record()
                    fn(*args)
                    e1.record()
                    e1.synchronize()
                    n = max(3, int(15.0 / max(e0.elapsed_time(e1), 1e-3)))
                    samples = []
                    for _ in range(5):
                        e0.record()
                        for _ in range(n):
                            fn(*args)
                        e1.record()
                        e1.synchronize()
                        samples.append(e0.elapsed_time(e1) / n)
                    ms = statistics.median(samples)
                f.write(json.dumps({"shape": name, "dtype": dt, "M": M, "N": N, "K": K, "variant": vid,
                                    "split": split, "raster": p["raster_n"], "plan": p["name"], "ms": round(ms, 5),
                                    "timing": "cold" if cold else "batch",
                                    "tflops": round(2.0 * M * N * K / ms / 1e9, 2),
                                    "est_us": round(p["est_us"], 1),
                                    "model_pick": (vid, split, p["raster_n"]) == (auto["variant_id"], auto["split_k"],
                                                                                  auto["raster_n"])}) + "\n")
                f.flush()
                del ws
            del dA, C
            if dt in ("mxfp8", "mxfp4"):
                del mx
            else:
                del dB
            torch.cuda.empty_cache()


def load(record: Path):
    """Per shape: the measured candidates, fastest first (ties: lower id, then
    lower split, then M-major). Records without a raster field were taken
    when every plan was M-major."""
    by = {}
    for line in record.read_text().splitlines():
        r = json.loads(line)
        r.setdefault("raster", 0)
        by.setdefault((r["dtype"], r["M"], r["N"], r["K"]), {})[(r["variant"], r["split"], r["raster"])] = r
    return {k: sorted(v.values(), key=lambda r: (r["ms"], r["variant"], r["split"], r["raster"]))
            for k, v in by.items()}


def emit(record: Path, out: Path = TUNED_H) -> str:
    table = load(record)
    lines = [
        "// Frozen dispatch table: the fastest measured (variant, split-K, raster order) per shape.",
        "// Generated by shape_adaptive_matrix_amd/tune.py from tuning/" + record.name + ";",
        "// regenerate with `python -m shape_adaptive_matrix_amd.tune emit <record>`, do not edit.",
        "//   T(dtype, M, N, K, variant, split, raster_n)   dtype: 0 f32, 1 bf16, 2 f16, 3 mxfp8, 4 mxfp4",
        "#pragma once",
        "",
        "#define SAM_TUNED_PLANS(T) \\",
    ]
    rows = []
    for (dt, M, N, K), rs in sorted(table.items(), key=lambda kv: (DTYPE_CODE[kv[0][0]], kv[0][1:])):
        best = rs[0]
        rows.append(f"    T({DTYPE_CODE[dt]}, {M}, {N}, {K}, {best['variant']}, {best['split']}, {best['raster']})")
    lines += [r + " \\" for r in rows[:-1]] + rows[-1:]
    text = "\n".join(lines) + "\n"
    out.write_text(text)
    return text


def report(record: Path) -> str:
    import shape_adaptive_matrix_amd as sam
    table = load(record)
    out = ["| shape | dtype | best plan | TFLOP/s | cost-model pick | its TFLOP/s | candidates |",
           "|---|---|---|---:|---|---:|---:|"]
    for (dt, M, N, K), rs in sorted(table.items(), key=lambda kv: (DTYPE_CODE[kv[0][0]], kv[0][1:])):
        best = rs[0]
        mp = model_plan(sam, dt, M, N, K)
        model = next((r for r in rs if (r["variant"], r["split"], r["raster"]) ==
                      (mp["variant_id"], mp["split_k"], mp["raster_n"])), None)
        out.append(f"| {M}x{N}x{K} | {dt} | {best['plan']} | {best['tflops']} | "
                   f"{model['plan'] if model else '-'} | {model['tflops'] if model else '-'} | {len(rs)} |")
    return "\n".join(out) + "\n"


def main(argv):
    if len(argv) < 2 or argv[0] not in ("measure", "emit", "report"):
        print(__doc__)
        return 2
    rec = Path(argv[1])
    if argv[0] == "measure":
        measure(rec, set(argv[2:]) or None)
    elif argv[0] == "emit":
        print(emit(rec), end="")
    else:
        print(report(rec), end="")
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
