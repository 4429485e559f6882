"""The general entry point C = alpha·op(A)·op(B) + beta·C (sam_gemm_ex) on an
MI355X, against the oracle's gemm_ex. Small-integer operands and dyadic
alpha/beta make every step exact, so the bits must match; random operands
use the FP32 rel_rms bound."""
import numpy as np
import pytest
import torch

import oracle
import sam_inputs as si
import shape_adaptive_matrix_amd as sam
from tests.compare import bitexact_mismatches, rel_rms
from tests.gpu_util import TORCH16

pytestmark = pytest.mark.gpu

_ORC = None


def orc():
    global _ORC
    if _ORC is None:
        _ORC = oracle.get()
    return _ORC


def _enc(dtype, x):
    x = np.asarray(x, np.float32)
    if dtype == "f32":
        return x
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def _dev(dtype, bits):
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(bits)).cuda()
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(TORCH16[dtype])


CASES = [((70, 130, 100), 0), ((129, 64, 72), 1), ((33, 257, 40), 2), ((256, 256, 256), 3)]
SCALES = [(1.0, 0.0), (2.0, -1.0), (0.5, 0.25), (0.0, 2.0), (-1.0, 0.0)]


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("ta,tb", [(False, False), (True, False), (False, True), (True, True)])
def test_ex_dyadic(dtype, ta, tb):
    for (M, N, K), pad in CASES:
        rng = np.random.default_rng(M + 3 * N + 5 * K + pad + 17 * ta + 31 * tb)
        ra, ca = (K, M) if ta else (M, K)
        rb, cb = (N, K) if tb else (K, N)
        lda, ldb, ldc = ca + pad, cb + 2 * pad, N + pad
        Av = rng.integers(-3, 4, size=(ra, lda)).astype(np.float32)
        Bv = rng.integers(-3, 4, size=(rb, ldb)).astype(np.float32)
        for alpha, beta in SCALES:
            C0 = rng.integers(-3, 4, size=(M, ldc)).astype(np.float32)
            if beta == 0.0:
                C0[:, :N] = np.nan                       # must never reach the result
            C0[:, N:] = 12345.0                          # padding columns: untouched
            Cd = torch.from_numpy(C0.copy()).cuda()
            sam.gemm_ex(_dev(dtype, _enc(dtype, Av))[:, :ca], _dev(dtype, _enc(dtype, Bv))[:, :cb],
                        Cd[:, :N], trans_a=ta, trans_b=tb, alpha=alpha, beta=beta)
            torch.cuda.synchronize()
            got = Cd.cpu().numpy()
            ref = orc().gemm_ex(dtype, M, N, K, _enc(dtype, Av), lda, _enc(dtype, Bv), ldb, ta, tb, alpha, beta,
                                np.ascontiguousarray(C0[:, :N]))
            bad = bitexact_mismatches(got[:, :N], ref)
            assert bad == 0, (dtype, ta, tb, (M, N, K), pad, alpha, beta, bad)
            assert np.all(got[:, N:] == 12345.0), (dtype, ta, tb, (M, N, K), alpha, beta)


@pytest.mark.parametrize("ta,tb", [(False, False), (True, False), (False, True), (True, True)])
def test_ex_random_f32(ta, tb):
    M, N, K = 300, 250, 520
    rng = np.random.default_rng(7 + ta + 2 * tb)
    A = rng.uniform(-1, 1, size=(K, M) if ta else (M, K)).astype(np.float32)
    B = rng.uniform(-1, 1, size=(N, K) if tb else (K, N)).astype(np.float32)
    C0 = rng.uniform(-1, 1, size=(M, N)).astype(np.float32)
    Cd = torch.from_numpy(C0.copy()).cuda()
    sam.gemm_ex(torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda(), Cd, trans_a=ta, trans_b=tb, alpha=0.7,
                beta=-0.3)
    torch.cuda.synchronize()
    ref = orc().gemm_ex("f32", M, N, K, A, A.shape[1], B, B.shape[1], ta, tb, 0.7, -0.3, C0)
    assert rel_rms(Cd.cpu().numpy(), ref) <= 1e-5


def test_ex_plain_case_is_the_gemm_path():
    rng = np.random.default_rng(3)
    A = torch.from_numpy(rng.uniform(-1, 1, size=(2048, 2048)).astype(np.float32)).cuda()
    B = torch.from_numpy(rng.uniform(-1, 1, size=(2048, 2048)).astype(np.float32)).cuda()
    C1 = sam.gemm(A, B)
    C2 = sam.gemm_ex(A, B)
    torch.cuda.synchronize()
    assert torch.equal(C1.view(torch.int32), C2.view(torch.int32))


def test_ex_k_zero_and_alpha_zero():
    M, N = 40, 70
    C0 = np.arange(M * N, dtype=np.float32).reshape(M, N)
    A = torch.full((M, 0), float("nan"), device="cuda")
    B = torch.full((0, N), float("nan"), device="cuda")
    Cd = torch.from_numpy(C0.copy()).cuda()
    sam.gemm_ex(A, B, Cd, alpha=3.0, beta=-2.0)                      # K = 0: C = beta C
    torch.cuda.synchronize()
    assert np.array_equal(Cd.cpu().numpy(), -2.0 * C0)
    A = torch.full((M, 33), float("nan"), device="cuda")              # alpha = 0: A, B never read
    B = torch.full((33, N), float("nan"), device="cuda")
    Cd = torch.from_numpy(C0.copy()).cuda()
    sam.gemm_ex(A, B, Cd, alpha=0.0, beta=0.5)
    torch.cuda.synchronize()
    assert np.array_equal(Cd.cpu().numpy(), 0.5 * C0)


# Operands with padded rows read in place by the 16-bit ring kernel (no
# packed copy): row strides that keep 16-byte rows, and misaligned ones on a
# shape whose plan copies both operands into zero-padded rows anyway (the
# copy then reads the caller's stride). Every case's plan is a ring plan.
RING16_STRIDED = [((1024, 768, 200), 8, 16), ((1500, 1200, 1032), 64, 8), ((2048, 2048, 2048), 24, 40),
                  ((2049, 4097, 1025), 3, 5)]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("case", RING16_STRIDED, ids=lambda c: "x".join(map(str, c[0])) + f"_p{c[1]}_{c[2]}")
def test_ex_ring16_strided_in_place(dtype, case):
    (M, N, K), pa, pb = case
    plan = sam.plan(M, N, K, dtype)
    assert plan["name"].startswith(dtype + "_r"), plan["name"]
    lda, ldb = K + pa, N + pb
    # no region for a packed copy: the workspace is the plan's own
    assert sam.ex_workspace_bytes(M, N, K, False, False, lda, ldb, N, 1.0, 0.0, dtype) == plan["workspace_bytes"]
    rng = np.random.default_rng(M + 7 * N + 11 * K + pa)
    Av = rng.integers(-3, 4, size=(M, lda)).astype(np.float32)
    Bv = rng.integers(-3, 4, size=(K, ldb)).astype(np.float32)
    Av[:, K:] = np.inf                                                # gaps: never read
    Bv[:, N:] = np.inf
    Cd = torch.full((M, N), float("nan"), device="cuda")
    sam.gemm_ex(_dev(dtype, _enc(dtype, Av))[:, :K], _dev(dtype, _enc(dtype, Bv))[:, :N], Cd)
    torch.cuda.synchronize()
    ref = orc().gemm(dtype, np.ascontiguousarray(_enc(dtype, Av)[:, :K]),
                     np.ascontiguousarray(_enc(dtype, Bv)[:, :N]), nthreads=orc().max_threads())
    assert bitexact_mismatches(Cd.cpu().numpy(), ref) == 0


# Ring plans take strided operands in place and store C themselves: row
# stride ldc and alpha / beta in the kernel that writes C (the data-parallel
# epilogue, the split-K reduce or the stream-K fix-up), with no packed copy
# of a non-transposed operand, no temporary product and no separate pass
# over C. Each case names the plan form its shape takes.
FUSED = [
    ("f32", (1792, 1792, 256), False, False, 4, 8, 8, 0.5, -1.0, "f32_f", "s1"),
    ("f32", (1792, 1792, 256), True, True, 0, 0, 4, 2.0, 0.0, "f32_f", "s1"),
    ("f32", (256, 1536, 3072), False, False, 0, 0, 12, -1.0, 0.25, "f32_f", "s8"),
    ("f32", (2304, 2560, 1536), False, False, 4, 4, 4, 0.5, 2.0, "f32_f", "sk"),
    ("f32", (2049, 4097, 1025), False, False, 3, 1, 3, 1.0, 1.0, "f32_f", "pad_s3"),
    ("bf16", (640, 1792, 256), False, False, 8, 8, 4, 0.5, -1.0, "bf16_r", "s1"),
    ("bf16", (256, 384, 3072), True, False, 0, 0, 8, 1.0, 1.0, "bf16_r", "s12"),
    ("f16", (640, 1792, 256), False, True, 0, 0, 4, -2.0, 0.5, "f16_r", "s1"),
    # beta != 0 on a 16x16x32 plan: its operand-swap form reads and writes C
    ("bf16", (2560, 3072, 256), False, False, 8, 8, 4, 0.5, 1.0, "bf16_r", "b16_s1"),
    ("f16", (2560, 3072, 256), True, True, 0, 0, 4, -1.0, 0.25, "f16_r", "b16_s1"),
]


def _fused_case(dtype, M, N, K, ta, tb, pa, pb, pc, alpha, beta, seed):
    rng = np.random.default_rng(seed)
    ra, ca = (K, M) if ta else (M, K)
    rb, cb = (N, K) if tb else (K, N)
    lda, ldb, ldc = ca + pa, cb + pb, N + pc
    Av = rng.integers(-3, 4, size=(ra, lda)).astype(np.float32)
    Bv = rng.integers(-3, 4, size=(rb, ldb)).astype(np.float32)
    Av[:, ca:] = np.inf
    Bv[:, cb:] = np.inf
    C0 = rng.integers(-3, 4, size=(M, ldc)).astype(np.float32)
    if beta == 0.0:
        C0[:, :N] = np.nan                       # must never reach the result
    C0[:, N:] = 12345.0                          # padding columns: untouched
    return Av, Bv, C0, lda, ldb, ldc


@pytest.mark.parametrize("case", FUSED, ids=lambda c: f"{c[0]}_{'x'.join(map(str, c[1]))}_{'T' if c[2] else 'N'}"
                         f"{'T' if c[3] else 'N'}_{c[10]}")
def test_ex_fused_epilogue_on_ring_plans(case):
    dtype, (M, N, K), ta, tb, pa, pb, pc, alpha, beta, prefix, form = case
    plan = sam.plan(M, N, K, dtype)
    assert plan["name"].startswith(prefix) and f"_{form}" in plan["name"], plan["name"]
    Av, Bv, C0, lda, ldb, ldc = _fused_case(dtype, M, N, K, ta, tb, pa, pb, pc, alpha, beta, M + N + K + pc)
    if not ta and not tb:       # nothing but the plan's own workspace
        assert sam.ex_workspace_bytes(M, N, K, ta, tb, lda, ldb, ldc, alpha, beta, dtype) == plan["workspace_bytes"]
    ca, cb = (M if ta else K), (K if tb else N)
    Cd = torch.from_numpy(C0.copy()).cuda()
    sam.gemm_ex(_dev(dtype, _enc(dtype, Av))[:, :ca], _dev(dtype, _enc(dtype, Bv))[:, :cb], Cd[:, :N],
                trans_a=ta, trans_b=tb, alpha=alpha, beta=beta)
    torch.cuda.synchronize()
    got = Cd.cpu().numpy()
    ref = orc().gemm_ex(dtype, M, N, K, _enc(dtype, Av), lda, _enc(dtype, Bv), ldb, ta, tb, alpha, beta,
                        np.ascontiguousarray(C0[:, :N]), nthreads=orc().max_threads())
    assert bitexact_mismatches(got[:, :N], ref) == 0
    assert np.all(got[:, N:] == 12345.0)


# The FP32 ring's element-load forms (rows that are not 16-byte pieces read
# one value at a time, C stored one value at a time) under the fused
# epilogue, forced: the dispatcher prefers the padding forms at this size.
@pytest.mark.parametrize("split", [1, 3, -1])
def test_ex_fused_epilogue_on_element_forms(split):
    M, N, K = 2049, 4097, 1025
    vid = next(v for v in range(sam.variant_count()) if sam.variant_info(v)["name"] == "f128x128_w4x2_k32n2")
    p = sam.variant_plan(vid, M, N, K, "f32", split)
    assert p["a_vector"] == 0 and p["b_vector"] == 0, p["name"]
    alpha, beta = 1.0, 1.0
    Av, Bv, C0, lda, ldb, ldc = _fused_case("f32", M, N, K, False, False, 3, 1, 3, alpha, beta, 17 + split)
    assert sam.ex_workspace_bytes(M, N, K, False, False, lda, ldb, ldc, alpha, beta, "f32", variant=vid,
                                  split=split) == p["workspace_bytes"]
    Cd = torch.from_numpy(C0.copy()).cuda()
    sam.gemm_ex(_dev("f32", Av)[:, :K], _dev("f32", Bv)[:, :N], Cd[:, :N], alpha=alpha, beta=beta, variant=vid,
                split=split)
    torch.cuda.synchronize()
    got = Cd.cpu().numpy()
    ref = orc().gemm_ex("f32", M, N, K, Av, lda, Bv, ldb, False, False, alpha, beta, np.ascontiguousarray(C0[:, :N]),
                        nthreads=orc().max_threads())
    assert bitexact_mismatches(got[:, :N], ref) == 0
    assert np.all(got[:, N:] == 12345.0)


# The operand-swap forms of the 16-bit ring (the ones a call that reads C
# runs) at full size, in their stream-K form with the fix-up at 6144^3 and
# data-parallel with K = 11008: the product against the oracle's plain GEMM
# of the compact operands, then alpha P + beta C0 (exact here: small
# integers, dyadic alpha / beta).
@pytest.mark.parametrize("dtype,shape,split", [("bf16", (6144, 6144, 6144), -1), ("f16", (4096, 4096, 11008), 1)])
def test_ex_fused_epilogue_16bit_stream_k_and_swap(dtype, shape, split):
    M, N, K = shape
    vid = next(v for v in range(sam.variant_count()) if sam.variant_info(v)["name"] == "r256x256_w2x4_k64n2_b16_sw")
    plan = sam.variant_plan(vid, M, N, K, dtype, split)
    assert plan["operand_swap"] == 1 and (plan["name"].endswith("_sk") if split < 0 else "_s1" in plan["name"])
    alpha, beta = 0.5, -1.0
    Av, Bv, C0, lda, ldb, ldc = _fused_case(dtype, M, N, K, False, False, 8, 16, 4, alpha, beta, 5)
    Cd = torch.from_numpy(C0.copy()).cuda()
    sam.gemm_ex(_dev(dtype, _enc(dtype, Av))[:, :K], _dev(dtype, _enc(dtype, Bv))[:, :N], Cd[:, :N],
                alpha=alpha, beta=beta, variant=vid, split=split)
    torch.cuda.synchronize()
    got = Cd.cpu().numpy()
    P = orc().gemm(dtype, np.ascontiguousarray(_enc(dtype, Av)[:, :K]), np.ascontiguousarray(_enc(dtype, Bv)[:, :N]),
                   nthreads=orc().max_threads())
    ref = alpha * P + beta * C0[:, :N].astype(np.float64)
    assert bitexact_mismatches(got[:, :N], ref) == 0
    assert np.all(got[:, N:] == 12345.0)


# Operands given transposed (B as N rows of K values, A as K rows of M
# values, or both) read straight by every 16x16x32 ring variant, in its
# data-parallel, split-K and stream-K forms (forced plans), with ragged M,
# strided rows, ldc and alpha / beta. No packed copy: the workspace is the
# plan's own (192-row tiles read a transposed B straight and pack A^T).
RING16_B16 = [v for v in range(sam.variant_count())
              if sam.variant_info(v)["name"].startswith("r") and "_b16" in sam.variant_info(v)["name"]]
NT_SHAPES = [(300, 520, 264), (1000, 776, 1032)]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("ta,tb", [(False, True), (True, False), (True, True)], ids=["NT", "TN", "TT"])
@pytest.mark.parametrize("vid", RING16_B16)
def test_ex_transposed_operands_read_straight(dtype, ta, tb, vid):
    ran = 0
    for (M, N, K) in NT_SHAPES:
        for split in (1, 2, -1):
            try:
                p = sam.variant_plan(vid, M, N, K, dtype, split)
            except sam.SamError:
                continue
            alpha, beta = 0.5, -1.0
            pa = (8 - M % 8) if ta else 8          # transposed A: rows of lda % 8 == 0 values
            Av, Bv, C0, lda, ldb, ldc = _fused_case(dtype, M, N, K, ta, tb, pa, 8, 4, alpha, beta,
                                                    M + N + vid + 3 * split + 5 * ta)
            ws = sam.ex_workspace_bytes(M, N, K, ta, tb, lda, ldb, ldc, alpha, beta, dtype, variant=vid, split=split)
            if ta and sam.variant_info(vid)["tile_m"] not in (128, 256):
                assert ws > p["workspace_bytes"]   # no A^T form for this tile: A is packed first
            else:
                assert ws == p["workspace_bytes"]
            print(f"[tr] variant {vid} {dtype} {'T' if ta else 'N'}{'T' if tb else 'N'} {(M, N, K)} split {split}",
                  flush=True)
            ca, cb = (M if ta else K), (K if tb else N)
            Cd = torch.from_numpy(C0.copy()).cuda()
            sam.gemm_ex(_dev(dtype, _enc(dtype, Av))[:, :ca], _dev(dtype, _enc(dtype, Bv))[:, :cb], Cd[:, :N],
                        trans_a=ta, trans_b=tb, alpha=alpha, beta=beta, variant=vid, split=split)
            torch.cuda.synchronize()
            got = Cd.cpu().numpy()
            ref = orc().gemm_ex(dtype, M, N, K, _enc(dtype, Av), lda, _enc(dtype, Bv), ldb, ta, tb, alpha, beta,
                                np.ascontiguousarray(C0[:, :N]), nthreads=orc().max_threads())
            assert bitexact_mismatches(got[:, :N], ref) == 0, (vid, dtype, ta, tb, (M, N, K), split)
            assert np.all(got[:, N:] == 12345.0)
            ran += 1
    assert ran > 0


@pytest.mark.parametrize("ta,tb", [(False, True), (True, False), (True, True)], ids=["NT", "TN", "TT"])
def test_ex_transposed_random_repeatable(ta, tb):
    """Random bf16 operands given transposed through the dispatcher's plan:
    rel_rms within 1e-5 of the oracle (exact products, FP32 sums), and
    bitwise the same twice."""
    M, N, K = 2560, 3072, 256
    assert sam.plan(M, N, K, "bf16")["name"].startswith("bf16_r")
    assert sam.ex_workspace_bytes(M, N, K, ta, tb, M if ta else K, K if tb else N, N, 1.0, 0.0, "bf16") == 0
    rng = np.random.default_rng(11 + 2 * ta + tb)
    A = si.normal16(rng, (M, K), "bf16")
    B = si.normal16(rng, (K, N), "bf16")
    dA = _dev("bf16", np.ascontiguousarray(A.T) if ta else A)
    dB = _dev("bf16", np.ascontiguousarray(B.T) if tb else B)
    C1 = sam.gemm_ex(dA, dB, trans_a=ta, trans_b=tb)
    C2 = sam.gemm_ex(dA, dB, trans_a=ta, trans_b=tb)
    torch.cuda.synchronize()
    assert torch.equal(C1.view(torch.int32), C2.view(torch.int32))
    ref = orc().gemm("bf16", A, B, nthreads=orc().max_threads())
    assert rel_rms(C1.cpu().numpy(), ref) <= 1e-5   # exact products, FP32 accumulation


# FP32 with B given transposed (N rows of K values) read straight by the
# ring variants that have that form (B placed K-contiguous like A, four K
# values of one column per read), data-parallel, split-K and stream-K, with
# strided rows, ldc, alpha / beta, ragged M and N (C rows not 16-byte pieces
# too): no copy, the workspace is the plan's own.
F32_BT = [v for v in range(sam.variant_count())
          if sam.variant_info(v)["name"] in ("f128x128_w2x2s2_k64n2_b16", "f128x128_w4x2_k64n2_b16",
                                             "f128x128_w4x2_k32n2_b16")]
F32_BT_SHAPES = [(300, 518, 264), (1000, 776, 1032), (129, 130, 512)]


@pytest.mark.parametrize("vid", F32_BT)
@pytest.mark.parametrize("alpha,beta", [(1.0, 0.0), (0.5, -1.0)])
def test_ex_f32_transposed_b_read_straight(vid, alpha, beta):
    ran = 0
    for (M, N, K) in F32_BT_SHAPES:
        for split in (1, 2, -1):
            try:
                p = sam.variant_plan(vid, M, N, K, "f32", split)
            except sam.SamError:
                continue
            pc = 4 - N % 4 if N % 4 else 4
            Av, Bv, C0, lda, ldb, ldc = _fused_case("f32", M, N, K, False, True, 4, 4, pc, alpha, beta,
                                                    M + N + vid + 3 * split)
            assert sam.ex_workspace_bytes(M, N, K, False, True, lda, ldb, ldc, alpha, beta, "f32", variant=vid,
                                          split=split) == p["workspace_bytes"]
            print(f"[bt] variant {vid} {(M, N, K)} split {split} alpha {alpha} beta {beta}", flush=True)
            Cd = torch.from_numpy(C0.copy()).cuda()
            sam.gemm_ex(_dev("f32", Av)[:, :K], _dev("f32", Bv)[:, :K], Cd[:, :N], trans_b=True, alpha=alpha,
                        beta=beta, variant=vid, split=split)
            torch.cuda.synchronize()
            got = Cd.cpu().numpy()
            ref = orc().gemm_ex("f32", M, N, K, Av, lda, Bv, ldb, False, True, alpha, beta,
                                np.ascontiguousarray(C0[:, :N]), nthreads=orc().max_threads())
            assert bitexact_mismatches(got[:, :N], ref) == 0, (vid, (M, N, K), split)
            assert np.all(got[:, N:] == 12345.0)
            ran += 1
    assert ran > 0


# FP32 with A given transposed (K rows of M values) read straight: A^T rows
# placed M-contiguous like B's and read two or four rows at a time, the row
# order inside each group of row blocks undone at the store; B's and C's
# rows whole 16-byte pieces (N % 4 == 0), any K, ragged M with Inf in the
# padding of A^T's rows (it reaches only rows of C that are never stored).
F32_AT_SHAPES = [(300, 520, 264), (1000, 776, 1030), (129, 136, 512)]


F32_AT = F32_BT + [v for v in range(sam.variant_count()) if sam.variant_info(v)["name"] == "f256x256_w4x2_k32n2_b16"]


@pytest.mark.parametrize("vid", F32_AT)
@pytest.mark.parametrize("alpha,beta", [(1.0, 0.0), (0.5, -1.0)])
def test_ex_f32_transposed_a_read_straight(vid, alpha, beta):
    ran = 0
    for (M, N, K) in F32_AT_SHAPES:
        for split in (1, 2, -1):
            try:
                p = sam.variant_plan(vid, M, N, K, "f32", split)
            except sam.SamError:
                continue
            pa = 4 - M % 4 if M % 4 else 4
            Av, Bv, C0, lda, ldb, ldc = _fused_case("f32", M, N, K, True, False, pa, 4, 4, alpha, beta,
                                                    M + 2 * N + vid + 3 * split)
            assert sam.ex_workspace_bytes(M, N, K, True, False, lda, ldb, ldc, alpha, beta, "f32", variant=vid,
                                          split=split) == p["workspace_bytes"]
            print(f"[at] variant {vid} {(M, N, K)} split {split} alpha {alpha} beta {beta}", flush=True)
            Cd = torch.from_numpy(C0.copy()).cuda()
            sam.gemm_ex(_dev("f32", Av)[:, :M], _dev("f32", Bv)[:, :N], Cd[:, :N], trans_a=True, alpha=alpha,
                        beta=beta, variant=vid, split=split)
            torch.cuda.synchronize()
            got = Cd.cpu().numpy()
            ref = orc().gemm_ex("f32", M, N, K, Av, lda, Bv, ldb, True, False, alpha, beta,
                                np.ascontiguousarray(C0[:, :N]), nthreads=orc().max_threads())
            assert bitexact_mismatches(got[:, :N], ref) == 0, (vid, (M, N, K), split)
            assert np.all(got[:, N:] == 12345.0)
            ran += 1
    assert ran > 0


def test_ex_f32_transposed_a_random_repeatable():
    """FP32 2048^3 with A given transposed through the dispatcher's plan: no
    copy, rel_rms within 1e-5 of the oracle, bitwise the same twice."""
    M = N = K = 2048
    assert sam.ex_workspace_bytes(M, N, K, True, False, M, N, N, 1.0, 0.0, "f32") == 0
    rng = np.random.default_rng(31)
    A = si.uniform_pm1(rng, (M, K))
    B = si.uniform_pm1(rng, (K, N))
    dAt = torch.from_numpy(np.ascontiguousarray(A.T)).cuda()
    dB = torch.from_numpy(B).cuda()
    C1 = sam.gemm_ex(dAt, dB, trans_a=True)
    C2 = sam.gemm_ex(dAt, dB, trans_a=True)
    torch.cuda.synchronize()
    assert torch.equal(C1.view(torch.int32), C2.view(torch.int32))
    ref = orc().gemm("f32", A, B, nthreads=orc().max_threads())
    assert rel_rms(C1.cpu().numpy(), ref) <= 1e-5


def test_ex_f32_transposed_b_random_repeatable():
    """FP32 2048^3 with B given transposed through the dispatcher's plan: no
    copy, rel_rms within 1e-5 of the oracle, bitwise the same twice."""
    M = N = K = 2048
    assert sam.ex_workspace_bytes(M, N, K, False, True, K, K, N, 1.0, 0.0, "f32") == 0
    rng = np.random.default_rng(29)
    A = si.uniform_pm1(rng, (M, K))
    B = si.uniform_pm1(rng, (K, N))
    dA = torch.from_numpy(A).cuda()
    dBt = torch.from_numpy(np.ascontiguousarray(B.T)).cuda()
    C1 = sam.gemm_ex(dA, dBt, trans_b=True)
    C2 = sam.gemm_ex(dA, dBt, trans_b=True)
    torch.cuda.synchronize()
    assert torch.equal(C1.view(torch.int32), C2.view(torch.int32))
    ref = orc().gemm("f32", A, B, nthreads=orc().max_threads())
    assert rel_rms(C1.cpu().numpy(), ref) <= 1e-5


# FP32 with both operands given transposed: C = A^T B^T computed as the
# plain product B A of the operands as stored, whose ring plan (for N x M x K)
# stores C transposed, in the kernel, the split-K reduce or the stream-K
# fix-up; element forms where rows are not 16-byte pieces, and a tile edge
# inside a group of four rows of the product (N odd).
TT_F32 = [((1792, 1792, 256), "s1"), ((1536, 256, 3072), "s8"), ((2560, 2304, 1536), "sk"),
          ((4097, 2049, 1025), "pad_s3"), ((3000, 3000, 3001), "_ua")]


@pytest.mark.parametrize("case", TT_F32, ids=lambda c: "x".join(map(str, c[0])))
@pytest.mark.parametrize("alpha,beta", [(1.0, 0.0), (0.5, -1.0)])
def test_ex_f32_both_transposed_as_transposed_store(case, alpha, beta):
    (M, N, K), form = case
    q = sam.plan(N, M, K, "f32")
    assert q["name"].startswith("f32_f") and form in q["name"], q["name"]
    pc = 4 - N % 4 if N % 4 else 4
    Av, Bv, C0, lda, ldb, ldc = _fused_case("f32", M, N, K, True, True, 4, 4, pc, alpha, beta, M + 3 * N + K)
    assert sam.ex_workspace_bytes(M, N, K, True, True, lda, ldb, ldc, alpha, beta, "f32") == q["workspace_bytes"]
    print(f"[tt] {(M, N, K)} {q['name']} alpha {alpha} beta {beta}", flush=True)
    Cd = torch.from_numpy(C0.copy()).cuda()
    sam.gemm_ex(_dev("f32", Av)[:, :M], _dev("f32", Bv)[:, :K], Cd[:, :N], trans_a=True, trans_b=True, alpha=alpha,
                beta=beta)
    torch.cuda.synchronize()
    got = Cd.cpu().numpy()
    ref = orc().gemm_ex("f32", M, N, K, Av, lda, Bv, ldb, True, True, alpha, beta, np.ascontiguousarray(C0[:, :N]),
                        nthreads=orc().max_threads())
    assert bitexact_mismatches(got[:, :N], ref) == 0
    assert np.all(got[:, N:] == 12345.0)
