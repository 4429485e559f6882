"""Comparison rules of the parity tests.

* bit-exact: the GPU's FP32 output must have exactly the bits of the oracle's
  double result rounded to FP32. Used on dyadic (small-integer) inputs where
  every FP32 partial sum is exact, so any summation order gives the same
  bits (page "Scale coverage exposes a remaining GEMM gap", section
  "Measurement contract and evidence": the dyadic input family gives zero
  error, which says nothing about general FP32 accuracy).
* rel_rms: the pages use the name without defining it (page "Measured data
  point on fixed-tile vs shape-adaptive GEMM", section "What we measured").
  Reading: relative Frobenius error ||C_gpu - C_ref||_F / ||C_ref||_F in
  double, over the compared elements. Non-finite GPU values fail outright.
"""
from __future__ import annotations

import numpy as np


def bitexact_mismatches(gpu: np.ndarray, ref64: np.ndarray) -> int:
    """Number of elements whose FP32 bits differ from round-to-FP32(ref)."""
    g = np.ascontiguousarray(gpu, dtype=np.float32)
    r = np.ascontiguousarray(ref64, dtype=np.float64).astype(np.float32)
    if g.shape != r.shape:
        raise ValueError(f"shape {g.shape} vs {r.shape}")
    return int(np.count_nonzero(g.view(np.uint32) != r.view(np.uint32)))


def rel_rms(gpu: np.ndarray, ref64: np.ndarray) -> float:
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref64, dtype=np.float64)
    if g.shape != r.shape:
        raise ValueError(f"shape {g.shape} vs {r.shape}")
    if not np.all(np.isfinite(g)):
        return float("inf")
    den = np.sqrt(np.sum(r * r))
    num = np.sqrt(np.sum((g - r) ** 2))
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)


# Gate of the block-scaled random-input tests: every element within this
# fraction of sum_k |a_k b_k| of the oracle's exact sum. The scaled matrix
# instruction sums each group of products with fewer bits than FP32, so the
# block-scaled path is not held to the FP32 bound; a wrong scale or a dropped
# 32-value block moves an element by a block's partial sum, far beyond it.
MX_ELEMENT_BOUND = 2.0 ** -12
MX_REL_RMS = 5e-5


def mx_bound_excess(gpu: np.ndarray, ref64: np.ndarray, absum: np.ndarray) -> float:
    """Largest |gpu - ref| - MX_ELEMENT_BOUND * absum over the elements
    (positive: the gate rejects); +inf when any GPU value is not finite."""
    g = np.asarray(gpu, dtype=np.float64)
    if not np.all(np.isfinite(g)):
        return float("inf")
    err = np.abs(g - np.asarray(ref64, dtype=np.float64))
    return float(np.max(err - MX_ELEMENT_BOUND * np.asarray(absum, dtype=np.float64)))
