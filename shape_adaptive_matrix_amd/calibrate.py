"""Offline calibration sweep: time every admissible variant (the
dispatcher's own split choice for each) on the named workloads and print one
JSON line per (workload, variant).

The dispatcher itself never times anything: its variant table carries a
frozen steady-state efficiency per variant and dtype, and this sweep is how
those numbers are measured (the measured-tactic shortlist idea of page
"fix(fp4_gemm autotune) SM107 kernel family excluded from autotune
candidates and heuristics update - #4856", section "Reviewer Notes", with the
result frozen in source so that selection stays deterministic).

Usage (on a gfx950 machine):
    python -m shape_adaptive_matrix_amd.calibrate [workload ...]
"""
from __future__ import annotations

import ctypes
import json
import statistics
import sys


def main(argv):
    import torch

    import sam_inputs as si
    import shape_adaptive_matrix_amd as sam

    sam.device_check()
    names = argv or [w.name for w in si.WORKLOADS]
    for name in names:
        w = si.by_name(name)
        A, B = si.make_operands(w)
        if w.dtype == "f32":
            dA, dB = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
        else:
            t = {"bf16": torch.bfloat16, "f16": torch.float16}[w.dtype]
            dA = torch.from_numpy(A.view("int16")).cuda().view(t)
            dB = torch.from_numpy(B.view("int16")).cuda().view(t)
        C = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")
        auto = sam.plan(w.M, w.N, w.K, w.dtype)
        stream = torch.cuda.current_stream()
        for vid in range(sam.variant_count()):
            try:
                p = sam.variant_plan(vid, w.M, w.N, w.K, w.dtype, 0)
            except sam.SamError:
                continue
            ws = sam.workspace_for(p, dA.device)
            args = (vid, sam.DTYPES[w.dtype], p["split_k"], ctypes.c_void_p(dA.data_ptr()),
                    ctypes.c_void_p(dB.data_ptr()), ctypes.c_void_p(C.data_ptr()), w.M, w.N, w.K,
                    ctypes.c_void_p(ws.data_ptr()) if ws is not None else None,
                    ws.numel() * 4 if ws is not None else 0, ctypes.c_void_p(stream.cuda_stream))
            fn = sam.lib().sam_gemm_variant
            for _ in range(3):
                assert fn(*args) == 0, sam.last_error()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
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
            print(json.dumps({"workload": name, "variant": vid, "plan": p["name"], "ms": round(ms, 5),
                              "tflops": round(w.flops / ms / 1e9, 2), "est_us": round(p["est_us"], 1),
                              "auto": p["variant_id"] == auto["variant_id"] and p["split_k"] == auto["split_k"]}),
                  flush=True)
            del ws
        del dA, dB, C
        torch.cuda.empty_cache()


if __name__ == "__main__":
    main(sys.argv[1:])
