"""Parity of the HIP path with the oracle on an MI355X (gfx950).

Every call goes through the C ABI (the ctypes binding). Dyadic inputs must
match bit for bit; random inputs must meet the rel_rms bound of the
workload; repeated runs must be bitwise identical.
"""
import numpy as np
import pytest
import torch

import oracle
import sam_inputs as si
import shape_adaptive_matrix_amd as sam
from tests.compare import bitexact_mismatches, rel_rms
from tests.gpu_util import ints_operands, run, to_dev

pytestmark = pytest.mark.gpu

ORC = None


def orc():
    global ORC
    if ORC is None:
        ORC = oracle.get()
    return ORC


def test_device_is_gfx950():
    sam.device_check()
    assert "gfx950" in torch.cuda.get_device_properties(0).gcnArchName


RAGGED = [(1, 1, 1), (17, 33, 45), (64, 64, 64), (70, 130, 100), (129, 257, 200), (16, 300, 96),
          (300, 16, 96), (256, 256, 256),
          # K and N multiples of 8 (the LDS-ring variants' domain), ragged M/N/K tiles
          (129, 136, 200), (257, 392, 328), (33, 520, 72), (1000, 264, 40),
          # short K with N % 4 == 0 (the persistent short-K variants' domain too)
          (70, 132, 28)]


def _supported(vid, M, N, K, dtype, split=0):
    try:
        sam.variant_plan(vid, M, N, K, dtype, split)
        return True
    except sam.SamError:
        return False


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("vid", range(sam.variant_count()))
def test_every_variant_dyadic_ragged(vid, dtype):
    """Each variant, forced, on ragged shapes with small integers: the sums
    are exact, so the bits must equal the oracle's."""
    ran = 0
    for (M, N, K) in RAGGED:
        if not _supported(vid, M, N, K, dtype, 1):
            continue
        A, B = ints_operands(M, N, K, dtype, seed=M * 7 + N * 3 + K)
        ref = orc().gemm(dtype, A, B)
        splits = [0, 1] + [s for s in (2, 3) if s * sam.variant_plan(vid, M, N, K, dtype, 1)["tile_k"] <= K]
        for s in splits:
            try:
                sam.variant_plan(vid, M, N, K, dtype, s)
            except sam.SamError:
                continue
            C = run(A, B, dtype, variant=vid, split=s)
            bad = bitexact_mismatches(C, ref)
            assert bad == 0, f"variant {vid} {dtype} {(M, N, K)} split {s}: {bad} mismatches"
            ran += 1
    if ran == 0:
        pytest.skip(f"variant {vid} does not take {dtype}")


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("vid", range(sam.variant_count()))
def test_every_variant_random(vid, dtype):
    M, N, K = 150, 176, 336
    if not _supported(vid, M, N, K, dtype):
        M, N, K = 150, 174, 333   # rows that are not 16-byte pieces (the padding forms' domain)
    if not _supported(vid, M, N, K, dtype):
        pytest.skip(f"variant {vid} does not take {dtype}")
    rng = np.random.default_rng(vid + 40)
    if dtype == "f32":
        A, B = si.uniform_pm1(rng, (M, K)), si.uniform_pm1(rng, (K, N))
        tol = 1e-5
    else:
        A, B = si.normal16(rng, (M, K), dtype), si.normal16(rng, (K, N), dtype)
        tol = 1e-5   # exact products, FP32 accumulation: far below the 1e-2 gate
    ref = orc().gemm(dtype, A, B)
    C = run(A, B, dtype, variant=vid)
    assert rel_rms(C, ref) <= tol


# Skinny shapes (M <= 16 or N <= 16, the streaming variants' domain, also run
# by every other variant that takes them): several K blocks per split, a K
# tail inside a wave, K % 4 != 0 and N % 4 != 0 element paths, rows and
# columns past one tile.
SKINNY = [(16, 1000, 5000), (5, 77, 4100), (13, 4096, 2049), (1, 3, 9001), (16, 64, 2048),
          (1000, 16, 5000), (777, 3, 4099), (2000, 12, 3002), (64, 16, 1024), (3, 5, 70)]
_SKINNY_REF = {}


@pytest.mark.parametrize("vid", range(sam.variant_count()))
def test_every_variant_dyadic_skinny(vid):
    ran = 0
    for (M, N, K) in SKINNY:
        if not _supported(vid, M, N, K, "f32", 1):
            continue
        A, B = ints_operands(M, N, K, "f32", seed=M * 5 + N * 11 + K)
        if (M, N, K) not in _SKINNY_REF:
            _SKINNY_REF[(M, N, K)] = orc().gemm("f32", A, B)
        ref = _SKINNY_REF[(M, N, K)]
        for s in (0, 1, 2, 3, 4, 8):
            if not _supported(vid, M, N, K, "f32", s):
                continue
            print(f"[skinny] variant {vid} {(M, N, K)} split {s}", flush=True)
            C = run(A, B, "f32", variant=vid, split=s)
            bad = bitexact_mismatches(C, ref)
            assert bad == 0, f"variant {vid} {(M, N, K)} split {s}: {bad} mismatches"
            ran += 1
    if ran == 0:
        pytest.skip(f"variant {vid} takes no skinny FP32 shape")


# Stream-K (split -1): shapes where ranges cut tiles into several shares
# (300x300x4096: ~28 shares per tile), ragged and odd-K/N ones, and a range
# that touches three tiles.
SK_SHAPES = [(300, 300, 4096), (768, 768, 768), (129, 257, 2000), (1000, 1000, 1000), (17, 2000, 3000),
             (1536, 1536, 1536), (260, 1030, 2052),
             # K % 4 != 0 (and N % 4 != 0): the element-load forms inside stream-K segments,
             # shapes for which the dispatcher itself picks a stream-K plan
             (1500, 1500, 2047), (260, 1030, 2051), (3000, 3000, 3001), (1500, 3000, 2047)]
_SK_REF = {}


@pytest.mark.parametrize("vid", range(sam.variant_count()))
def test_every_variant_stream_k_dyadic(vid):
    ran = 0
    for (M, N, K) in SK_SHAPES:
        if not _supported(vid, M, N, K, "f32", -1):
            continue
        A, B = ints_operands(M, N, K, "f32", seed=M + 3 * N + 7 * K)
        if (M, N, K) not in _SK_REF:
            _SK_REF[(M, N, K)] = orc().gemm("f32", A, B)
        print(f"[sk] variant {vid} {(M, N, K)}", flush=True)
        C = run(A, B, "f32", variant=vid, split=-1)
        bad = bitexact_mismatches(C, _SK_REF[(M, N, K)])
        assert bad == 0, f"variant {vid} {(M, N, K)} stream-K: {bad} mismatches"
        ran += 1
    if ran == 0:
        pytest.skip(f"variant {vid} has no stream-K form for these shapes")


@pytest.mark.parametrize("shape", [(300, 300, 4096), (1500, 1500, 2047)], ids=str)
def test_stream_k_random_and_repeatable(shape):
    """Random inputs: within the FP32 bound, and bitwise identical on repeats
    (the shares of a tile are always added in the same order); K % 4 != 0
    runs the element-load form inside the segments."""
    M, N, K = shape
    rng = np.random.default_rng(5 + K)
    A, B = si.uniform_pm1(rng, (M, K)), si.uniform_pm1(rng, (K, N))
    ref = orc().gemm("f32", A, B)
    vids = [v for v in range(sam.variant_count()) if _supported(v, M, N, K, "f32", -1)]
    assert vids
    for vid in vids:
        outs = [run(A, B, "f32", variant=vid, split=-1) for _ in range(3)]
        assert rel_rms(outs[0], ref) <= 1e-5
        for o in outs[1:]:
            assert np.array_equal(o.view(np.uint32), outs[0].view(np.uint32)), vid


# 16-bit stream-K (data-parallel waves, then the last wave's tiles shared):
# no data-parallel part (few tiles), ranges crossing tile boundaries, M, N
# and K tails, one or two iterations per range.
SK16_SHAPES = [(300, 264, 2048), (1000, 1000, 1000), (4352, 4352, 512), (2304, 8192, 1024),
               (4400, 4104, 520)]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("vid", range(sam.variant_count()))
def test_every_16bit_variant_stream_k_dyadic(vid, dtype):
    ran = 0
    for (M, N, K) in SK16_SHAPES:
        if not _supported(vid, M, N, K, dtype, -1):
            continue
        p = sam.variant_plan(vid, M, N, K, dtype, -1)
        A, B = ints_operands(M, N, K, dtype, seed=M + 5 * N + 3 * K)
        print(f"[sk16] variant {vid} {dtype} {(M, N, K)} dp={p['sk_dp_tiles']} grid={p['grid_wgs']}", flush=True)
        C = run(A, B, dtype, variant=vid, split=-1)
        bad = bitexact_mismatches(C, orc().gemm(dtype, A, B))
        assert bad == 0, f"variant {vid} {dtype} {(M, N, K)} stream-K: {bad} mismatches"
        ran += 1
    if ran == 0:
        pytest.skip(f"variant {vid} has no 16-bit stream-K form")


def test_16bit_stream_k_random_and_repeatable():
    M, N, K = 2304, 8192, 1024
    rng = np.random.default_rng(17)
    A, B = si.normal16(rng, (M, K), "bf16"), si.normal16(rng, (K, N), "bf16")
    ref = orc().gemm("bf16", A, B)
    vids = [v for v in range(sam.variant_count()) if _supported(v, M, N, K, "bf16", -1)]
    assert vids
    for vid in vids:
        outs = [run(A, B, "bf16", variant=vid, split=-1) for _ in range(3)]
        assert rel_rms(outs[0], ref) <= 1e-5
        for o in outs[1:]:
            assert np.array_equal(o.view(np.uint32), outs[0].view(np.uint32)), vid


# N-major raster (groups of tile columns sweep the rows): every tiled variant
# on shapes with several tile rows and columns, ragged in M, N and K.
RASTER_SHAPES = [(1000, 1096, 200), (520, 2056, 136), (2056, 520, 72)]


@pytest.mark.parametrize("vid", range(sam.variant_count()))
def test_every_variant_n_major_raster_dyadic(vid):
    ran = 0
    for (M, N, K) in RASTER_SHAPES:
        for dtype in ("f32", "bf16"):
            try:
                p = sam.variant_plan(vid, M, N, K, dtype, 0, 1)
            except sam.SamError:
                continue
            assert p["raster_n"] == 1
            A, B = ints_operands(M, N, K, dtype, seed=M + N + 11 * K)
            dA, dB = to_dev(A, dtype), to_dev(B, dtype)
            C = torch.full((M, N), float("nan"), device="cuda")
            print(f"[raster] variant {vid} {dtype} {(M, N, K)} {p['name']}", flush=True)
            sam.gemm_variant(vid, dA, dB, C, raster=1)
            torch.cuda.synchronize()
            bad = bitexact_mismatches(C.cpu().numpy(), orc().gemm(dtype, A, B))
            assert bad == 0, f"variant {vid} {dtype} {(M, N, K)} N-major: {bad} mismatches"
            ran += 1
    if ran == 0:
        pytest.skip(f"variant {vid} takes none of the raster shapes")


def test_dispatcher_picks_stream_k_on_odd_k():
    """The shapes above with K % 4 != 0 are ones the dispatcher itself sends
    to stream-K, so those segments are the automatic path, not only forced."""
    picked = [s for s in [(1500, 1500, 2047), (3000, 3000, 3001), (260, 1030, 2051), (1500, 3000, 2047)]
              if sam.plan(*s, "f32")["split_k"] == -1]
    assert picked, "no odd-K shape goes to stream-K any more; pick new shapes"


def test_persistent_short_k():
    """The persistent short-K variants on grids with more tiles than resident
    workgroups, so that workgroups walk several tiles with the next panels
    loading and the last stores draining; ragged M and N tails, K not a
    multiple of the 16-value step. Small integers: bit-exact. Random inputs:
    within the FP32 bound and bitwise repeatable."""
    kp = [v for v in range(sam.variant_count()) if sam.variant_info(v)["name"].startswith("kp")]
    assert len(kp) == 2
    cases = [(2341, 2324, 60), (3100, 3000, 28), (130, 260, 4)]
    ran = 0
    for (M, N, K) in cases:
        A, B = ints_operands(M, N, K, "f32", seed=M + N + K)
        ref = orc().gemm("f32", A, B)
        for vid in kp:
            if not _supported(vid, M, N, K, "f32"):
                continue
            plan = sam.variant_plan(vid, M, N, K, "f32", 0)
            C = run(A, B, "f32", variant=vid)
            bad = bitexact_mismatches(C, ref)
            assert bad == 0, f"variant {vid} {(M, N, K)} grid {plan['grid_wgs']}: {bad} mismatches"
            ran += 1
    assert ran >= 4
    # More tiles than resident workgroups for both variants.
    assert sam.variant_plan(kp[0], 3100, 3000, 28, "f32", 0)["grid_wgs"] < 25 * 24
    assert sam.variant_plan(kp[1], 2341, 2324, 60, "f32", 0)["grid_wgs"] < 19 * 19
    M, N, K = 1500, 1000, 64
    rng = np.random.default_rng(11)
    A, B = si.uniform_pm1(rng, (M, K)), si.uniform_pm1(rng, (K, N))
    ref = orc().gemm("f32", A, B)
    for vid in kp:
        if not _supported(vid, M, N, K, "f32"):
            continue
        outs = [run(A, B, "f32", variant=vid) for _ in range(3)]
        assert rel_rms(outs[0], ref) <= 1e-5
        for o in outs[1:]:
            assert np.array_equal(o.view(np.uint32), outs[0].view(np.uint32)), vid


def test_c_is_write_only_and_fully_written():
    """NaN-prefilled C: every element written; guard band after C untouched."""
    M, N, K = 99, 77, 55
    A, B = ints_operands(M, N, K, "f32", seed=3)
    ref = orc().gemm("f32", A, B)
    guard = 4096
    buf = torch.full((M * N + guard,), float("nan"), dtype=torch.float32, device="cuda")
    buf[M * N:] = 12345.0
    C = buf[:M * N].view(M, N)
    for vid in range(sam.variant_count()):
        if not _supported(vid, M, N, K, "f32"):
            continue
        buf[:M * N] = float("nan")
        sam.gemm_variant(vid, to_dev(A, "f32"), to_dev(B, "f32"), C)
        torch.cuda.synchronize()
        out = buf.cpu().numpy()
        assert bitexact_mismatches(out[:M * N].reshape(M, N), ref) == 0, vid
        assert np.all(out[M * N:] == 12345.0), vid


def test_k_zero_writes_positive_zero():
    C = torch.full((33, 65), float("nan"), device="cuda")
    A = torch.empty((33, 0), device="cuda")
    B = torch.empty((0, 65), device="cuda")
    sam.gemm(A, B, C)
    torch.cuda.synchronize()
    assert np.all(C.cpu().numpy().view(np.uint32) == 0)


@pytest.mark.parametrize("shape", [(64, 64, 37), (5, 70, 1037), (70, 5, 1037)])
def test_inf_beyond_k_tail_is_not_read(shape):
    """An Inf just past A and just past B in memory must not leak into C: the
    K tail is zero-filled on both operands."""
    M, N, K = shape
    sA = np.full((M * K + 64,), np.inf, np.float32)
    sA[:M * K] = 1.0
    sB = np.full((K * N + 64,), np.inf, np.float32)
    sB[:K * N] = 1.0
    dA = torch.from_numpy(sA).cuda()[:M * K].view(M, K)
    dB = torch.from_numpy(sB).cuda()[:K * N].view(K, N)
    ran = 0
    for vid in range(sam.variant_count()):
        if not _supported(vid, M, N, K, "f32"):
            continue
        C = sam.gemm_variant(vid, dA, dB)
        torch.cuda.synchronize()
        assert np.all(C.cpu().numpy() == K), vid
        ran += 1
    assert ran > 0


@pytest.mark.parametrize("dtype,shape", [("f32", (130, 132, 60)), ("f32", (70, 136, 45)), ("f32", (37, 64, 1037)),
                                         ("bf16", (130, 136, 200)), ("f16", (70, 264, 40)),
                                         # rows that are not whole 16-byte pieces (padded copies)
                                         ("bf16", (130, 133, 201)), ("f16", (70, 261, 45))])
def test_inf_at_start_of_next_row_is_not_read(dtype, shape):
    """A row's K tail is the start of the next row in memory. Inf there (A
    rows 1 and 3 start with Inf) must reach only those rows' outputs: rows 0
    and 2, whose last K stage or chunk ends inside the Inf, must come out
    exactly K. Run on every variant that takes the shape."""
    M, N, K = shape
    A = np.ones((M, K), np.float32)
    A[1, 0] = np.inf
    A[3, 0:4] = np.inf
    B = np.ones((K, N), np.float32)
    if dtype == "f32":
        dA, dB = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    else:
        t = {"bf16": torch.bfloat16, "f16": torch.float16}[dtype]
        dA, dB = torch.from_numpy(A).cuda().to(t), torch.from_numpy(B).cuda().to(t)
    ran = 0
    for vid in range(sam.variant_count()):
        if not _supported(vid, M, N, K, dtype):
            continue
        C = sam.gemm_variant(vid, dA, dB).cpu().numpy()
        torch.cuda.synchronize()
        for r in (0, 2, 4, M - 1):
            assert np.all(C[r] == K), (vid, r)
        for r in (1, 3):
            assert np.all(np.isposinf(C[r])), (vid, r)
        ran += 1
    assert ran > 0


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_inf_beyond_k_tail_16bit(dtype):
    """Same for 16-bit operands, K a multiple of 8 but not of any stage depth:
    the next 'row' past A holds Inf and must never be multiplied."""
    M, N, K = 96, 128, 40
    one, inf = (0x3F80, 0x7F80) if dtype == "bf16" else (0x3C00, 0x7C00)
    store = np.full((M * K + 64,), one, np.uint16)
    store[M * K:] = inf
    B = np.full((K, N), one, np.uint16)
    dstore = to_dev(store, dtype)
    dA = dstore[:M * K].view(M, K)
    for vid in range(sam.variant_count()):
        if not _supported(vid, M, N, K, dtype):
            continue
        C = sam.gemm_variant(vid, dA, to_dev(B, dtype))
        torch.cuda.synchronize()
        assert np.all(C.cpu().numpy() == K), vid


# -- the workloads at their real sizes ------------------------------------------------
def _check_workload(w, C, A=None, B=None):
    """Every element of C against the full oracle (the FP64 product of the
    whole workload, computed on the host's cores in seconds even at 8192^3)."""
    if A is None:
        A, B = si.make_operands(w)
    ref = orc().gemm(w.dtype, A, B)
    if w.check == "bitexact":
        assert bitexact_mismatches(C, ref) == 0
    else:
        e = rel_rms(C, ref)
        assert e <= w.tol, e
        if w.dtype != "f32":
            # FP32 accumulation of exact products: anything near the 1e-2 gate
            # would mean a reduced-precision output or accumulator.
            assert e <= 1e-4, e


@pytest.mark.parametrize("name", [w.name for w in si.WORKLOADS + si.LLM_WORKLOADS])
def test_workload_parity(name):
    """The dispatcher's own plan (the launch configuration the benchmark
    times) at the workload's full size, every element against the oracle."""
    w = si.by_name(name)
    A, B = si.make_operands(w)
    print(f"[parity] {name} plan={sam.plan(w.M, w.N, w.K, w.dtype)['name']}", flush=True)
    C = run(A, B, w.dtype)
    _check_workload(w, C, A, B)


@pytest.mark.parametrize("shape", si.LLM_SHAPES, ids=str)
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_llm_shapes_dyadic(shape, dtype):
    """The LLM-like shapes in their frozen (or modelled) plans on small
    integers: every partial sum is exact, so every element must equal the
    oracle bit for bit."""
    M, N, K = shape
    A, B = ints_operands(M, N, K, dtype, seed=M + N + K, lo=-2, hi=2)
    print(f"[llm] {dtype} {shape} plan={sam.plan(M, N, K, dtype)['name']}", flush=True)
    C = run(A, B, dtype)
    assert bitexact_mismatches(C, orc().gemm(dtype, A, B)) == 0


@pytest.mark.parametrize("name", ["f32_2048", "bf16_4096", "f32_16x8192x8192", "f32_768"])
def test_run_to_run_bitwise(name):
    """Five runs give identical bytes; a different seed gives different bytes
    (so the equality is not vacuous)."""
    w = si.by_name(name)
    A, B = si.make_operands(w)
    dA, dB = to_dev(A, w.dtype), to_dev(B, w.dtype)
    outs = []
    for _ in range(5):
        C = torch.full((w.M, w.N), float("nan"), device="cuda")
        sam.gemm(dA, dB, C)
        torch.cuda.synchronize()
        outs.append(C.cpu().numpy().view(np.uint32).copy())
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])
    A2, B2 = si.make_operands(w, seed=w.seed + 1000)
    C2 = sam.gemm(to_dev(A2, w.dtype), to_dev(B2, w.dtype))
    torch.cuda.synchronize()
    assert not np.array_equal(C2.cpu().numpy().view(np.uint32), outs[0])


# -- the dispatcher's own plans on arbitrary shapes ---------------------------------
def test_auto_plans_random_shapes_dyadic():
    """Seeded random shapes through the automatic path (whatever plan the
    dispatcher picks: tuned or cost model, split-K, stream-K, element forms),
    every dtype, bit-exact on small integers."""
    rng = np.random.default_rng(2024)
    shapes = set()
    while len(shapes) < 24:
        M, N, K = (int(x) for x in rng.integers(1, 700, size=3))
        shapes.add((M, N, K))
    for i, (M, N, K) in enumerate(sorted(shapes)):
        dtype = ("f32", "bf16", "f16")[i % 3]
        A, B = ints_operands(M, N, K, dtype, seed=i)
        p = sam.plan(M, N, K, dtype)
        print(f"[auto] {dtype} {(M, N, K)} {p['name']}", flush=True)
        C = run(A, B, dtype)
        bad = bitexact_mismatches(C, orc().gemm(dtype, A, B))
        assert bad == 0, (dtype, (M, N, K), p["name"], bad)
