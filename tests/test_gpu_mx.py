"""Parity of the block-scaled 8-bit path (sam_gemm_mxfp8) with the oracle on
an MI355X (gfx950), through the C ABI.

Dyadic inputs (``mx_dyadic``: every partial sum is exact in FP32) must match
the oracle bit for bit. Random inputs (``mx_normal``) are held to the
precision of the scaled matrix instruction, which sums each group of 64
products with fewer bits than FP32 (measured with one-hot and two-term
operands: sums across instructions are exact to 2^-23, and random operands
give rel_rms about 1.3e-5 for E4M3 and 9e-6 for E5M2 already at K = 64, with
|error| at most about 640 u sum_k |a_k b_k|, u = 2^-24). The gates: every
element within 2^-12 sum_k |a_k b_k| of the oracle's exact sum (a wrong
scale or a dropped block moves an element by far more), and rel_rms <= 5e-5.
Repeated runs must give the same bits.
"""
import numpy as np
import pytest
import torch

import oracle
import sam_inputs as si
import shape_adaptive_matrix_amd as sam
from tests.compare import bitexact_mismatches, mx_bound_excess, rel_rms

pytestmark = pytest.mark.gpu

MX_VARIANTS = [v for v in range(sam.variant_count()) if sam.variant_info(v)["name"].startswith("x")]
FORMATS = [("e4m3", "e4m3"), ("e5m2", "e4m3"), ("e4m3", "e5m2"), ("e5m2", "e5m2")]
RAGGED = [(1, 1, 32), (37, 45, 96), (64, 64, 64), (130, 257, 160), (256, 256, 256), (300, 200, 1024),
          (513, 129, 224), (16, 300, 128)]

ORC = None


def orc():
    global ORC
    if ORC is None:
        ORC = oracle.get()
    return ORC


def _dev(*xs):
    return [torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in xs]


def _operands(M, N, K, fa, fb, dist, seed):
    w = si.Workload("t", "mxfp8", M, N, K, dist, seed, fmt_a=fa, fmt_b=fb)
    return si.make_mx_operands(w)


def _run(ops, fa, fb, variant=None, split=0):
    A, SA, Bt, SB = _dev(*ops)
    C = torch.full((A.shape[0], Bt.shape[0]), float("nan"), dtype=torch.float32, device="cuda")
    if variant is None:
        sam.gemm_mxfp8(A, SA, Bt, SB, fa, fb, C)
    else:
        sam.gemm_mxfp8_variant(variant, A, SA, Bt, SB, fa, fb, C, split_k=split)
    torch.cuda.synchronize()
    return C.cpu().numpy()


def _abs_sum(ops, fa, fb):
    """sum_k |a_k b_k| per element: the oracle on codes with the sign bit
    cleared (every term then positive)."""
    A, SA, Bt, SB = ops
    return orc().gemm_mxfp8(fa, fb, A & 0x7F, SA, Bt & 0x7F, SB)


def _check_bound(C, ref, absum, K):
    assert np.isfinite(C).all()
    worst = mx_bound_excess(C, ref, absum)
    assert worst <= 0, f"error exceeds the instruction-precision bound by {worst}"


def _supported(vid, M, N, K, split=0):
    try:
        sam.variant_plan(vid, M, N, K, "mxfp8", split)
        return True
    except sam.SamError:
        return False


def test_variants_present():
    assert len(MX_VARIANTS) >= 3
    for v in MX_VARIANTS:
        assert _supported(v, 256, 256, 256)


@pytest.mark.parametrize("fa,fb", FORMATS)
@pytest.mark.parametrize("vid", MX_VARIANTS)
def test_every_mx_variant_dyadic_ragged(vid, fa, fb):
    """Each block-scaled variant, forced, on ragged shapes with exact sums:
    bit-exact, for splits 1, 2 and 3 where admissible."""
    for (M, N, K) in RAGGED:
        ops = _operands(M, N, K, fa, fb, "mx_dyadic", seed=M * 7 + N * 3 + K)
        ref = orc().gemm_mxfp8(fa, fb, *ops)
        tk = sam.variant_plan(vid, M, N, K, "mxfp8", 1)["tile_k"]
        for s in [0, 1] + [s for s in (2, 3) if s * tk <= K]:
            if not _supported(vid, M, N, K, s):
                continue
            print(f"[mx] variant {vid} {fa}x{fb} {(M, N, K)} split {s}", flush=True)
            C = _run(ops, fa, fb, variant=vid, split=s)
            bad = bitexact_mismatches(C, ref)
            assert bad == 0, f"variant {vid} {fa}x{fb} {(M, N, K)} split {s}: {bad} mismatches"


@pytest.mark.parametrize("vid", MX_VARIANTS)
def test_every_mx_variant_random(vid):
    """Normal data stored in 8-bit formats with scales a few octaves apart:
    within the FP32 accumulation bound of the oracle, element by element."""
    M, N, K = 200, 328, 576
    for fa, fb in FORMATS:
        ops = _operands(M, N, K, fa, fb, "mx_normal", seed=vid + 300)
        ref = orc().gemm_mxfp8(fa, fb, *ops)
        C = _run(ops, fa, fb, variant=vid)
        _check_bound(C, ref, _abs_sum(ops, fa, fb), K)
        assert rel_rms(C, ref) <= 5e-5


def test_mx_auto_plans_random_shapes():
    """The dispatcher's own plans on seeded random shapes (K a multiple of 32)."""
    rng = np.random.default_rng(77)
    for n in range(10):
        M, N = (int(x) for x in rng.integers(1, 700, size=2))
        K = 32 * int(rng.integers(1, 40))
        fa, fb = FORMATS[n % 4]
        ops = _operands(M, N, K, fa, fb, "mx_dyadic", seed=1000 + n)
        ref = orc().gemm_mxfp8(fa, fb, *ops)
        print(f"[mx] auto {fa}x{fb} {(M, N, K)} plan={sam.plan(M, N, K, 'mxfp8')['name']}", flush=True)
        C = _run(ops, fa, fb)
        assert bitexact_mismatches(C, ref) == 0, (M, N, K, fa, fb)


@pytest.mark.parametrize("name", [w.name for w in si.MX_WORKLOADS + si.LLM_MX_WORKLOADS if w.dtype == "mxfp8"])
def test_mx_workload_sampled(name):
    """Full-size workloads in the launch configuration the benchmark times:
    sampled outputs (random points plus the corners and tail rows/columns)
    against the oracle's single-point sums."""
    w = si.by_name(name)
    ops = si.make_mx_operands(w)
    print(f"[mx] {name} plan={sam.plan(w.M, w.N, w.K, 'mxfp8')['name']}", flush=True)
    C = _run(ops, w.fmt_a, w.fmt_b)
    rows, cols = si.sample_points(w.M, w.N, 1500, seed=w.seed)
    ref = orc().gemm_mxfp8_points(w.fmt_a, w.fmt_b, *ops, rows, cols)
    A, SA, Bt, SB = ops
    absum = orc().gemm_mxfp8_points(w.fmt_a, w.fmt_b, A & 0x7F, SA, Bt & 0x7F, SB, rows, cols)
    got = C[rows, cols]
    _check_bound(got, ref, absum, w.K)
    assert rel_rms(got, ref) <= w.tol
    assert np.isfinite(C).all()


def test_mx_run_to_run_bitwise():
    """Five runs give identical bytes; another seed gives different bytes."""
    M, N, K = 1024, 1536, 2048
    ops = _operands(M, N, K, "e4m3", "e4m3", "mx_normal", seed=5)
    first = _run(ops, "e4m3", "e4m3")
    for _ in range(4):
        assert np.array_equal(first.view(np.uint32), _run(ops, "e4m3", "e4m3").view(np.uint32))
    other = _run(_operands(M, N, K, "e4m3", "e4m3", "mx_normal", seed=6), "e4m3", "e4m3")
    assert not np.array_equal(first.view(np.uint32), other.view(np.uint32))


def test_mx_nan_beyond_operands_never_reaches_c():
    """NaN codes stored right after A's and Bt's last rows, and NaN scale
    codes after the scale arrays, must never reach C (tails are masked)."""
    M, N, K = 70, 45, 96
    for fa, fb in FORMATS:
        A, SA, Bt, SB = _operands(M, N, K, fa, fb, "mx_dyadic", seed=11)
        ref = orc().gemm_mxfp8(fa, fb, A, SA, Bt, SB)
        nan = 0x7F   # S.1111.111 in E4M3 and S.11111.11 in E5M2: NaN in both
        pA = np.full((M + 8, K), nan, np.uint8); pA[:M] = A
        pB = np.full((N + 8, K), nan, np.uint8); pB[:N] = Bt
        pSA = np.full((M + 8, K // 32), 0xFF, np.uint8); pSA[:M] = SA
        pSB = np.full((N + 8, K // 32), 0xFF, np.uint8); pSB[:N] = SB
        dA, dB, dSA, dSB = _dev(pA, pB, pSA, pSB)
        C = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        sam.gemm_mxfp8(dA[:M], dSA[:M], dB[:N], dSB[:N], fa, fb, C)
        torch.cuda.synchronize()
        assert bitexact_mismatches(C.cpu().numpy(), ref) == 0, (fa, fb)


def test_mx_degenerate_sizes():
    """K = 0 writes +0; M = 0 or N = 0 leaves C untouched."""
    z = torch.zeros((0,), dtype=torch.uint8, device="cuda")
    C = torch.full((3, 5), float("nan"), dtype=torch.float32, device="cuda")
    sam.gemm_mxfp8(z.view(3, 0), z.view(3, 0), z.view(5, 0), z.view(5, 0), "e4m3", "e4m3", C)
    torch.cuda.synchronize()
    c = C.cpu().numpy()
    assert (c == 0).all() and not np.signbit(c).any()
    C = torch.full((4, 4), 7.0, dtype=torch.float32, device="cuda")
    sam.gemm_mxfp8(z.view(0, 64), z.view(0, 2), torch.zeros((4, 64), dtype=torch.uint8, device="cuda"),
                   torch.zeros((4, 2), dtype=torch.uint8, device="cuda"), "e4m3", "e4m3", C[:0])
    torch.cuda.synchronize()
    assert (C.cpu().numpy() == 7.0).all()


# -- block-scaled 4-bit elements (MXFP4: E2M1 packed two per byte) ----------------
RAGGED4 = [(1, 1, 32), (37, 45, 96), (64, 64, 64), (130, 257, 160), (256, 256, 512), (300, 200, 1024),
           (513, 129, 224), (16, 300, 640)]


def _operands4(M, N, K, dist, seed):
    w = si.Workload("t", "mxfp4", M, N, K, dist, seed, fmt_a="e2m1", fmt_b="e2m1")
    return si.make_mx_operands(w)


def _run4(ops, variant=None, split=0):
    A, SA, Bt, SB = _dev(*ops)
    C = torch.full((A.shape[0], Bt.shape[0]), float("nan"), dtype=torch.float32, device="cuda")
    if variant is None:
        sam.gemm_mxfp4(A, SA, Bt, SB, C)
    else:
        sam.gemm_mxfp4_variant(variant, A, SA, Bt, SB, C, split_k=split)
    torch.cuda.synchronize()
    return C.cpu().numpy()


def _abs_sum4(ops):
    A, SA, Bt, SB = ops
    return orc().gemm_mxfp4(A & 0x77, SA, Bt & 0x77, SB)   # both sign bits cleared


@pytest.mark.parametrize("vid", MX_VARIANTS)
def test_every_mx4_variant_dyadic_ragged(vid):
    """Each block-scaled variant running E2M1 elements, forced, on ragged
    shapes with exact sums (any E2M1 value times scales on [1/2, 2]): bit-exact,
    splits 1, 2 and 3 where admissible, K not a multiple of 128 included
    (the per-lane scale form)."""
    for (M, N, K) in RAGGED4:
        ops = _operands4(M, N, K, "mx_dyadic", seed=M * 5 + N * 11 + K)
        ref = orc().gemm_mxfp4(*ops)
        tk = sam.variant_plan(vid, M, N, K, "mxfp4", 1)["tile_k"]
        for s in [0, 1] + [s for s in (2, 3) if s * tk <= K]:
            try:
                sam.variant_plan(vid, M, N, K, "mxfp4", s)
            except sam.SamError:
                continue
            print(f"[mx4] variant {vid} {(M, N, K)} split {s}", flush=True)
            C = _run4(ops, variant=vid, split=s)
            bad = bitexact_mismatches(C, ref)
            assert bad == 0, f"variant {vid} {(M, N, K)} split {s}: {bad} mismatches"


@pytest.mark.parametrize("vid", MX_VARIANTS)
def test_every_mx4_variant_random(vid):
    """Codes uniform over E2M1 with scales a few octaves apart: within the
    instruction-precision bound of the oracle, element by element."""
    M, N, K = 200, 328, 1152
    ops = _operands4(M, N, K, "mx_normal", seed=vid + 400)
    ref = orc().gemm_mxfp4(*ops)
    C = _run4(ops, variant=vid)
    _check_bound(C, ref, _abs_sum4(ops), K)
    assert rel_rms(C, ref) <= 5e-5


def test_mx4_auto_plans_random_shapes():
    rng = np.random.default_rng(78)
    for n in range(8):
        M, N = (int(x) for x in rng.integers(1, 700, size=2))
        K = 32 * int(rng.integers(1, 60))
        ops = _operands4(M, N, K, "mx_dyadic", seed=2000 + n)
        print(f"[mx4] auto {(M, N, K)} plan={sam.plan(M, N, K, 'mxfp4')['name']}", flush=True)
        assert bitexact_mismatches(_run4(ops), orc().gemm_mxfp4(*ops)) == 0, (M, N, K)


@pytest.mark.parametrize("name", [w.name for w in si.MX_WORKLOADS + si.LLM_MX_WORKLOADS if w.dtype == "mxfp4"])
def test_mx4_workload_sampled(name):
    w = si.by_name(name)
    ops = si.make_mx_operands(w)
    print(f"[mx4] {name} plan={sam.plan(w.M, w.N, w.K, 'mxfp4')['name']}", flush=True)
    C = _run4(ops)
    rows, cols = si.sample_points(w.M, w.N, 1500, seed=w.seed)
    ref = orc().gemm_mxfp4_points(*ops, rows, cols)
    A, SA, Bt, SB = ops
    absum = orc().gemm_mxfp4_points(A & 0x77, SA, Bt & 0x77, SB, rows, cols)
    got = C[rows, cols]
    _check_bound(got, ref, absum, w.K)
    assert rel_rms(got, ref) <= w.tol
    assert np.isfinite(C).all()


def test_mx4_nan_scales_beyond_arrays_never_reach_c():
    """NaN scale codes after the scale arrays, and 0x77 bytes (6, 6) after
    A's and Bt's rows, never reach C; runs are bitwise repeatable."""
    M, N, K = 70, 45, 192
    A, SA, Bt, SB = _operands4(M, N, K, "mx_dyadic", seed=12)
    ref = orc().gemm_mxfp4(A, SA, Bt, SB)
    pA = np.full((M + 8, K // 2), 0x77, np.uint8); pA[:M] = A
    pB = np.full((N + 8, K // 2), 0x77, np.uint8); pB[:N] = Bt
    pSA = np.full((M + 8, K // 32), 0xFF, np.uint8); pSA[:M] = SA
    pSB = np.full((N + 8, K // 32), 0xFF, np.uint8); pSB[:N] = SB
    dA, dB, dSA, dSB = _dev(pA, pB, pSA, pSB)
    outs = []
    for _ in range(3):
        C = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        sam.gemm_mxfp4(dA[:M], dSA[:M], dB[:N], dSB[:N], C)
        torch.cuda.synchronize()
        outs.append(C.cpu().numpy())
    assert bitexact_mismatches(outs[0], ref) == 0
    assert all(np.array_equal(outs[0].view(np.uint32), o.view(np.uint32)) for o in outs[1:])
