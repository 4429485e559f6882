"""The allocation-free entry point (sam_gemm_noalloc) against the entry point
it mirrors (sam_gemm_<dtype> with a caller workspace), through the C ABI.

Both run the same plan and kernels; sam_gemm_noalloc keeps the plan's
workspace in the library's per-GPU scratch array. Two calls in a row, the
second on a smaller input, must each give exactly the bits of the ordinary
call (and, on small integers, the oracle's bits); the second call must not
see anything the first left in the array.
"""
import numpy as np
import pytest
import torch

import oracle
import sam_inputs as si
import shape_adaptive_matrix_amd as sam
from tests.compare import bitexact_mismatches
from tests.gpu_util import ints_operands, to_dev

pytestmark = pytest.mark.gpu

# (M, N, K, dtype): split-K and stream-K plans, each pair larger then smaller.
PAIRS = [
    [(8192, 16, 8192, "f32"), (2048, 16, 8192, "f32")],          # split-K partials, 4 MiB then 1.5 MiB
    [(2200, 1900, 4092, "f32"), (1500, 3000, 2047, "f32")],      # stream-K slots (32 MiB), then a smaller problem
                                                                 # whose padded copies sit in front of its slots
    [(512, 512, 8192, "bf16"), (64, 1024, 8192, "bf16")],        # 16-bit split-K
    [(64, 1024, 8192, "f16"), (16, 8192, 8192, "f32")],
]


def _random(M, N, K, dtype, seed):
    rng = np.random.default_rng(seed)
    if dtype == "f32":
        return si.uniform_pm1(rng, (M, K)), si.uniform_pm1(rng, (K, N))
    return si.normal16(rng, (M, K), dtype), si.normal16(rng, (K, N), dtype)


def _both(A, B, dtype):
    dA, dB = to_dev(A, dtype), to_dev(B, dtype)
    M, N = A.shape[0], B.shape[1]
    ref = torch.full((M, N), float("nan"), device="cuda")
    sam.gemm(dA, dB, ref)
    got = torch.full((M, N), float("nan"), device="cuda")
    sam.gemm_noalloc(dA, dB, got)
    torch.cuda.synchronize()
    return got.cpu().numpy(), ref.cpu().numpy()


@pytest.mark.parametrize("pair", PAIRS, ids=lambda p: f"{p[0]}->{p[1]}")
def test_noalloc_equals_workspace_entry_point(pair):
    for i, (M, N, K, dtype) in enumerate(pair):
        p = sam.plan(M, N, K, dtype)
        assert 0 < p["workspace_bytes"] <= sam.SCRATCH_BYTES, p
        print(f"[noalloc] call {i} {dtype} {(M, N, K)} {p['name']}", flush=True)
        got, ref = _both(*_random(M, N, K, dtype, seed=M + N + K + i), dtype)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), (M, N, K, dtype)


def test_noalloc_dyadic_matches_oracle():
    """Small integers, a larger then a smaller split-K shape: bit-exact
    against the oracle as well."""
    o = oracle.get()
    for (M, N, K, dtype) in [(700, 600, 9000, "f32"), (100, 200, 3000, "f32")]:
        A, B = ints_operands(M, N, K, dtype, seed=K)
        got, ref = _both(A, B, dtype)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
        assert bitexact_mismatches(got, o.gemm(dtype, A, B)) == 0


def test_noalloc_refuses_plans_beyond_the_scratch():
    """A plan whose workspace exceeds the array is refused on the host with
    SAM_ERR_WORKSPACE, before any device work."""
    M, N, K = 4097, 3071, 8191
    assert sam.plan(M, N, K, "f32")["workspace_bytes"] > sam.SCRATCH_BYTES
    A = torch.zeros((M, K), device="cuda")
    B = torch.zeros((K, N), device="cuda")
    with pytest.raises(sam.SamError) as e:
        sam.gemm_noalloc(A, B)
    assert e.value.name == "SAM_ERR_WORKSPACE"
