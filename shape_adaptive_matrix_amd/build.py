"""Build ``libsam.so`` (the HIP GEMM library) for gfx950 with hipcc.

The old library is deleted before anything is compiled, so a failed build
can never leave a stale one in place (page "Post-mortem: a GPU stack without
nvcc, cuBLAS, or LLVM", section 8: a failed step that keeps the previous
artifact is worse than a loud failure). The library is stamped with the git
revision, the hipcc version and the target, and ``sam_build_info()`` returns
that stamp.

Usage: ``python -m shape_adaptive_matrix_amd.build`` or ``build()``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import time
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
LIB = PKG / "libsam.so"
BUILD_DIR = ROOT / "_build" / "sam"
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["sam_kernels.hip", "sam_kernels_dma.hip", "sam_kernels_dma_t.hip", "sam_kernels_stream.hip", "sam_kernels_f32ring.hip", "sam_kernels_ex.hip", "sam_kernels_mx.hip", "sam_kernels_kq.hip", "sam_kernels_kp.hip", "sam_plan.cpp", "sam_api.cpp"]

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # Packed FP32 instructions stay off in all device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # The MFMA chunk steps are fully unrolled by pragma; the largest (128
    # MFMAs each) exceed the default size limit and would otherwise stay
    # rolled with their accumulators in scratch.
    "-mllvm", "-pragma-unroll-threshold=1000000",
    "-Wall", "-Wno-unused-function",
]


def _stamp() -> str:
    try:
        rev = subprocess.run(["git", "-C", str(ROOT), "rev-parse", "--short", "HEAD"],
                             capture_output=True, text=True, check=True).stdout.strip()
        dirty = subprocess.run(["git", "-C", str(ROOT), "status", "--porcelain", "--", "shape_adaptive_matrix_amd", "include"],
                               capture_output=True, text=True).stdout.strip()
        rev += "+dirty" if dirty else ""
    except (OSError, subprocess.CalledProcessError):
        rev = "nogit"
    try:
        ver = subprocess.run([HIPCC, "--version"], capture_output=True, text=True).stdout.splitlines()[0]
    except (OSError, IndexError):
        ver = "hipcc ?"
    return f"libsam git={rev} {ver.strip()} target={ARCH} built={time.strftime('%Y-%m-%dT%H:%M:%S')}"


def _compile(src: str, stamp: str, verbose: bool) -> Path:
    obj = BUILD_DIR / (src + ".o")
    if obj.exists():
        obj.unlink()
    cmd = [HIPCC, *HIP_FLAGS, f'-DSAM_BUILD_STAMP="{stamp}"']
    if not src.endswith(".hip"):
        cmd += ["-x", "hip"]
    cmd += ["-c", str(CSRC / src), "-o", str(obj)]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
    if msg.strip() and verbose:
        print(msg, flush=True)
    return obj


CEILINGS_SRC = PKG / "microbench" / "sam_ceilings.hip"
CEILINGS_BIN = PKG / "microbench" / "sam_ceilings"


def _build_ceilings(verbose: bool) -> Path:
    """The MFMA-loop / HBM-copy ceiling probe (a standalone executable)."""
    if CEILINGS_BIN.exists():
        CEILINGS_BIN.unlink()
    # Accumulators in ordinary VGPRs: with AGPRs the compiler shuffles the
    # 16x16x32 accumulators between iterations and serialises the loop.
    cmd = [HIPCC, *HIP_FLAGS, "-mllvm", "-amdgpu-mfma-vgpr-form", str(CEILINGS_SRC), "-o", str(CEILINGS_BIN)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {CEILINGS_SRC.name}:\n{r.stdout}{r.stderr}")
    return CEILINGS_BIN


def build(verbose: bool = False) -> Path:
    if LIB.exists():
        LIB.unlink()
    BUILD_DIR.mkdir(parents=True, exist_ok=True)
    stamp = _stamp()
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, stamp, verbose), SOURCES))
    tmp = LIB.with_suffix(".so.tmp")
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *map(str, objs), "-o", str(tmp)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    _build_ceilings(verbose)
    if verbose:
        print(f"built {LIB} ({stamp})", flush=True)
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
