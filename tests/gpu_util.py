"""Helpers shared by the GPU tests: move seeded numpy operands to the device,
run the library, bring C back."""
from __future__ import annotations

import numpy as np
import torch

import shape_adaptive_matrix_amd as sam

TORCH16 = {"bf16": torch.bfloat16, "f16": torch.float16}


def to_dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "f32":
        assert x.dtype == np.float32
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()
    assert x.dtype == np.uint16
    t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda()
    return t.view(TORCH16[dtype])


def ints_operands(M, N, K, dtype, seed, lo=-3, hi=3):
    """Small integers: exact in FP32, bfloat16 and binary16."""
    rng = np.random.default_rng(seed)
    A = rng.integers(lo, hi + 1, (M, K)).astype(np.float32)
    B = rng.integers(lo, hi + 1, (K, N)).astype(np.float32)
    if dtype == "f32":
        return A, B
    if dtype == "f16":
        return A.astype(np.float16).view(np.uint16), B.astype(np.float16).view(np.uint16)
    return (A.view(np.uint32) >> 16).astype(np.uint16), (B.view(np.uint32) >> 16).astype(np.uint16)


def run(A: np.ndarray, B: np.ndarray, dtype: str, variant=None, split=0) -> np.ndarray:
    dA, dB = to_dev(A, dtype), to_dev(B, dtype)
    C = torch.full((A.shape[0], B.shape[1]), float("nan"), dtype=torch.float32, device="cuda")
    if variant is None:
        sam.gemm(dA, dB, C)
    else:
        sam.gemm_variant(variant, dA, dB, C, split_k=split)
    torch.cuda.synchronize()
    return C.cpu().numpy()
