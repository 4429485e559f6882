"""Seeded synthetic operands for the GEMM workloads.

Shared by the tests, the benchmark and the smoke check. It holds no GEMM
arithmetic: only random draws, the rounding of a draw to a 16- or 8-bit
storage format (part of the input's definition: normal(0,1) values stored as
bfloat16, binary16 or an 8-bit float), and the workload table.

Recipes:
  * ``uniform``: FP32 uniform on [-1, 1). Drawn directly as float32 (24 random
    bits, so multiples of 2^-24 on [0, 1)), then x*2-1, which is exact in FP32
    and never reaches +1.
  * ``ints``: integers uniform on the closed range [lo, hi], stored as FP32.
    Small integers make every FP32 partial sum exact (dyadic inputs).
  * ``normal16``: float32 standard normal, rounded to nearest-even to bfloat16
    or binary16; the 16-bit bit patterns are returned as uint16.
A is always drawn before B from one ``numpy.random.default_rng(seed)``.

Block-scaled 8-bit operands (``mxfp8`` workloads: element codes of the OCP
MX formats E4M3 / E5M2 and E8M0 scale codes, one per 32 values of K; A is M
rows and B is given as N rows of K codes):
  * ``mx_normal``: float32 standard normal stored in the element format
    (round to nearest-even by torch's float8 conversion; no draw comes near
    the largest finite value), scale codes uniform on [123, 131] (block
    scales a few octaves apart).
  * ``mx_dyadic``: codes assembled from random fields: sign uniform, the
    exponent field one of two adjacent values (values in [1, 4)), the
    fraction field uniform, one code in 16 replaced by zero; scale codes
    uniform on [126, 128]. Every value is a multiple of 2^-4 below 8, so for
    K <= 1024 every partial sum is a multiple of 2^-8 below 2^16 and exact in
    FP32, whatever the order.
  * E2M1 (``mxfp4`` workloads): packed bytes uniform over all values, i.e.
    both 4-bit codes uniform over the 16 codes (for either recipe; the
    recipe only sets the scale range). With scales on [126, 128] every value
    is a multiple of 2^-2 of magnitude at most 12, so for K <= 1024 every
    partial sum is a multiple of 2^-4 below 2^18: exact in FP32.
Draw order: A codes, B codes, A scales, B scales.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

__all__ = ["Workload", "WORKLOADS", "MX_WORKLOADS", "LLM_WORKLOADS", "LLM_MX_WORKLOADS", "LLM_SHAPES", "by_name", "uniform_pm1", "small_ints",
           "normal16", "make_operands", "sample_points", "bf16_rne_bits",
           "mx_codes", "mx_scales", "make_mx_operands", "MX_BLOCK"]

MX_BLOCK = 32   # values of K per scale


def uniform_pm1(rng: np.random.Generator, shape) -> np.ndarray:
    x = rng.random(shape, dtype=np.float32)
    return x * np.float32(2.0) - np.float32(1.0)


def small_ints(rng: np.random.Generator, shape, lo: int, hi: int) -> np.ndarray:
    return rng.integers(lo, hi + 1, size=shape).astype(np.float32)


def bf16_rne_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest, ties to even.

    Finite inputs only (normal draws never produce NaN or Inf)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def normal16(rng: np.random.Generator, shape, kind: str) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if kind == "bf16":
        return bf16_rne_bits(x)
    if kind == "f16":
        return x.astype(np.float16).view(np.uint16)  # numpy rounds to nearest-even
    raise ValueError(kind)


def mx_codes(rng: np.random.Generator, shape, fmt: str, dist: str) -> np.ndarray:
    """uint8 element codes of ``fmt`` ("e4m3" | "e5m2") drawn per ``dist``;
    for "e2m1", rows of packed bytes (two codes each, shape[1] // 2 per row)."""
    if fmt == "e2m1":
        return rng.integers(0, 256, size=(shape[0], shape[1] // 2), dtype=np.uint8)
    if dist == "mx_normal":
        import torch
        x = torch.from_numpy(rng.standard_normal(shape, dtype=np.float32))
        t = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}[fmt]
        return x.to(t).view(torch.uint8).numpy().copy()
    if dist == "mx_dyadic":
        sign = rng.integers(0, 2, size=shape, dtype=np.uint8)
        if fmt == "e4m3":   # exponent field 7 or 8 (bias 7), 3 fraction bits
            code = (sign << 7) | (rng.integers(7, 9, size=shape, dtype=np.uint8) << 3) | \
                rng.integers(0, 8, size=shape, dtype=np.uint8)
        else:               # exponent field 15 or 16 (bias 15), 2 fraction bits
            code = (sign << 7) | (rng.integers(15, 17, size=shape, dtype=np.uint8) << 2) | \
                rng.integers(0, 4, size=shape, dtype=np.uint8)
        zero = rng.integers(0, 16, size=shape) == 0
        return np.where(zero, np.uint8(0), code).astype(np.uint8)
    raise ValueError(dist)


def mx_scales(rng: np.random.Generator, rows: int, K: int, dist: str) -> np.ndarray:
    """uint8 E8M0 scale codes, ``rows`` x K/32."""
    lo, hi = (123, 131) if dist == "mx_normal" else (126, 128)
    return rng.integers(lo, hi + 1, size=(rows, K // MX_BLOCK), dtype=np.uint8)


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str          # "f32" | "bf16" | "f16" | "mxfp8" | "mxfp4"
    M: int
    N: int
    K: int
    dist: str           # "uniform" | "ints" | "normal16" | "mx_normal" | "mx_dyadic"
    seed: int
    lo: int = 0         # integer range for "ints"
    hi: int = 0
    check: str = "rel_rms"   # "bitexact" | "rel_rms"
    tol: float = 1e-5
    fmt_a: str = "e4m3"      # mxfp8 element formats
    fmt_b: str = "e4m3"

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    @property
    def in_bytes(self) -> int:
        return {"f32": 4, "bf16": 2, "f16": 2, "mxfp8": 1, "mxfp4": 0.5}[self.dtype]

    @property
    def alg_bytes(self) -> int:
        """Operands (and block scales) read once, C written once (beta = 0, C
        is never read)."""
        b = int(self.in_bytes * (self.M * self.K + self.K * self.N)) + 4 * self.M * self.N
        if self.dtype in ("mxfp8", "mxfp4"):
            b += (self.M + self.N) * (self.K // MX_BLOCK)
        return b


def _u(name, M, N, K, seed):
    return Workload(name, "f32", M, N, K, "uniform", seed)


WORKLOADS = [
    Workload("f32_256_ints", "f32", 256, 256, 256, "ints", 1, -4, 4, "bitexact", 0.0),
    _u("f32_2048", 2048, 2048, 2048, 2),
    Workload("f32_2048_ints", "f32", 2048, 2048, 2048, "ints", 3, -2, 2, "bitexact", 0.0),
    _u("f32_4096", 4096, 4096, 4096, 4),
    _u("f32_8192", 8192, 8192, 8192, 5),
    Workload("bf16_4096", "bf16", 4096, 4096, 4096, "normal16", 6, tol=1e-2),
    Workload("bf16_8192", "bf16", 8192, 8192, 8192, "normal16", 7, tol=1e-2),
    Workload("f16_4096", "f16", 4096, 4096, 4096, "normal16", 8, tol=1e-2),
    Workload("f16_8192", "f16", 8192, 8192, 8192, "normal16", 9, tol=1e-2),
    _u("f32_768", 768, 768, 768, 10),
    _u("f32_4097x3071x8191", 4097, 3071, 8191, 11),
    _u("f32_8191x8193x4096", 8191, 8193, 4096, 12),
    _u("f32_16x8192x8192", 16, 8192, 8192, 13),
    _u("f32_8192x16x8192", 8192, 16, 8192, 14),
    _u("f32_8192x8192x64", 8192, 8192, 64, 15),
]

# Block-scaled 8-bit workloads (the block-scaled low-precision extension),
# kept apart from the FP32 / 16-bit list above.
MX_WORKLOADS = [
    Workload("mxfp8_4096", "mxfp8", 4096, 4096, 4096, "mx_normal", 16, tol=5e-5),
    Workload("mxfp8_8192", "mxfp8", 8192, 8192, 8192, "mx_normal", 17, tol=5e-5),
    Workload("mxfp8_e5m2_4096", "mxfp8", 4096, 4096, 4096, "mx_normal", 18, tol=5e-5,
             fmt_a="e5m2", fmt_b="e5m2"),
    Workload("mxfp4_4096", "mxfp4", 4096, 4096, 4096, "mx_normal", 19, tol=5e-5, fmt_a="e2m1", fmt_b="e2m1"),
    Workload("mxfp4_8192", "mxfp4", 8192, 8192, 8192, "mx_normal", 20, tol=5e-5, fmt_a="e2m1", fmt_b="e2m1"),
]

# A second, LLM-like workload: the projection shapes of page "Scale coverage
# exposes a remaining GEMM gap", section "GEMM: frozen schedules at larger
# dimensions" (256 x 11008 x 4096, 4096 x 4096 x 11008 and the ragged
# 2049 x 4097 x 1025), in FP32, bfloat16 and binary16, plus the two shapes
# that also have block-scaled plans.
LLM_SHAPES = [(256, 11008, 4096), (4096, 4096, 11008), (2049, 4097, 1025)]


def _llm(dtype, seed0):
    out = []
    for i, (M, N, K) in enumerate(LLM_SHAPES):
        name = f"llm_{dtype}_{M}x{N}x{K}"
        if dtype == "f32":
            out.append(Workload(name, "f32", M, N, K, "uniform", seed0 + i))
        else:
            out.append(Workload(name, dtype, M, N, K, "normal16", seed0 + i, tol=1e-2))
    return out


LLM_WORKLOADS = _llm("f32", 21) + _llm("bf16", 24) + _llm("f16", 27)
LLM_MX_WORKLOADS = [
    Workload("llm_mxfp8_256x11008x4096", "mxfp8", 256, 11008, 4096, "mx_normal", 30, tol=5e-5),
    Workload("llm_mxfp8_4096x4096x11008", "mxfp8", 4096, 4096, 11008, "mx_normal", 31, tol=5e-5),
    Workload("llm_mxfp4_256x11008x4096", "mxfp4", 256, 11008, 4096, "mx_normal", 32, tol=5e-5,
             fmt_a="e2m1", fmt_b="e2m1"),
    Workload("llm_mxfp4_4096x4096x11008", "mxfp4", 4096, 4096, 11008, "mx_normal", 33, tol=5e-5,
             fmt_a="e2m1", fmt_b="e2m1"),
]

_BY_NAME = {w.name: w for w in WORKLOADS + MX_WORKLOADS + LLM_WORKLOADS + LLM_MX_WORKLOADS}


def by_name(name: str) -> Workload:
    return _BY_NAME[name]


def make_operands(w: Workload, seed: int | None = None):
    """(A, B) as numpy arrays: float32 for f32, uint16 bit patterns otherwise."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    sa, sb = (w.M, w.K), (w.K, w.N)
    if w.dist == "uniform":
        return uniform_pm1(rng, sa), uniform_pm1(rng, sb)
    if w.dist == "ints":
        return small_ints(rng, sa, w.lo, w.hi), small_ints(rng, sb, w.lo, w.hi)
    if w.dist == "normal16":
        return normal16(rng, sa, w.dtype), normal16(rng, sb, w.dtype)
    raise ValueError(w.dist)


def make_mx_operands(w: Workload, seed: int | None = None):
    """(A, SA, Bt, SB) uint8 arrays for an ``mxfp8`` / ``mxfp4`` workload: A
    [M][K] and Bt [N][K] element codes (E2M1: [M][K/2] and [N][K/2] packed
    bytes), SA [M][K/32] and SB [N][K/32] scale codes."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    A = mx_codes(rng, (w.M, w.K), w.fmt_a, w.dist)
    Bt = mx_codes(rng, (w.N, w.K), w.fmt_b, w.dist)
    return A, mx_scales(rng, w.M, w.K, w.dist), Bt, mx_scales(rng, w.N, w.K, w.dist)


def sample_points(M: int, N: int, count: int, seed: int):
    """Distinct output positions for a spot check: ``count`` seeded random ones
    plus the four corners and samples of the last row and last column (the
    elements next to the M and N tails). Returns (rows, cols) int64 arrays."""
    rng = np.random.default_rng(seed)
    total = M * N
    flat = rng.choice(total, size=min(count, total), replace=False).astype(np.int64)
    extra = [0, N - 1, (M - 1) * N, M * N - 1]
    extra += [(M - 1) * N + j for j in np.linspace(0, N - 1, 16, dtype=np.int64)]
    extra += [i * N + (N - 1) for i in np.linspace(0, M - 1, 16, dtype=np.int64)]
    flat = np.unique(np.concatenate([flat, np.asarray(extra, dtype=np.int64)]))
    return flat // N, flat % N
