"""The C ABI and the dispatcher without a GPU: the library loads, exports
every symbol the header declares, plans are pure and deterministic, the
automatic choice is the audited minimum, and bad calls are rejected before
any device work."""
import ctypes
import subprocess

import pytest

import shape_adaptive_matrix_amd as sam

L = sam.lib()


def test_exports_every_header_symbol():
    names = sam.header_symbols()
    assert len(names) >= 12
    out = subprocess.run(["nm", "-D", "--defined-only", str(sam.LIB_PATH)],
                         capture_output=True, text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        getattr(L, n)


def test_plan_struct_abi():
    p = sam.SamPlan()
    assert L.sam_gemm_plan(64, 64, 64, sam.F32, ctypes.byref(p)) == 0
    assert p.struct_size == ctypes.sizeof(sam.SamPlan)


def test_build_stamp_names_target():
    info = sam.build_info()
    assert "gfx950" in info and "git=" in info


def test_status_strings():
    for code, name in sam.STATUS.items():
        assert L.sam_status_string(code).decode() == name


SHAPES = [(256, 256, 256), (2048, 2048, 2048), (4096, 4096, 4096), (8192, 8192, 8192),
          (768, 768, 768), (4097, 3071, 8191), (8191, 8193, 4096), (16, 8192, 8192),
          (8192, 16, 8192), (8192, 8192, 64), (1, 1, 1), (3, 5, 7)]


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("shape", SHAPES, ids=str)
def test_plan_is_audited_argmin(shape, dtype):
    """The automatic plan is the minimum estimate over every admissible
    variant, ties to the lowest id, and asking twice gives the same plan.
    Shapes in the frozen table of measured plans take the table's entry
    instead (checked against the measurement record in test_tuning)."""
    M, N, K = shape
    p = sam.plan(M, N, K, dtype)
    assert p == sam.plan(M, N, K, dtype)
    if p["tuned"] == 0:
        best = None
        for vid in range(sam.variant_count()):
            try:
                q = sam.variant_plan(vid, M, N, K, dtype, 0)
            except sam.SamError:
                continue
            if best is None or q["est_us"] < best["est_us"]:
                best = q
        assert best is not None
        assert (p["variant_id"], p["split_k"], p["raster_n"]) == \
            (best["variant_id"], best["split_k"], best["raster_n"])
        assert p == sam.plan_model(M, N, K, dtype)
    tiles = -(-M // p["tile_m"]) * -(-N // p["tile_n"])
    if "_kp" in p["name"]:
        # Persistent short-K plans launch the resident workgroups only: one
        # per CU with a 64-value K panel (128 KB of LDS), two with 32.
        assert p["grid_wgs"] == min(tiles, 256 * (1 if p["tile_k"] == 64 else 2))
    elif p["split_k"] == -1:
        # Stream-K: data-parallel tiles (16-bit form) plus the sharing workgroups.
        assert p["sk_dp_tiles"] <= p["grid_wgs"] and p["sk_dp_tiles"] <= tiles
    else:
        assert p["grid_wgs"] == tiles * p["split_k"]
    assert p["workspace_bytes"] == expected_workspace(p, M, N, K, dtype)


def _a256(x):
    return (x + 255) // 256 * 256


def expected_workspace(p, M, N, K, dtype):
    """Padded operand copies (16-bit ring kernels with K or N not a multiple
    of 8, FP32 padding forms with K or N not a multiple of 4), then split-K
    partials or stream-K slots."""
    pad = 0
    q, es = 0, 0
    if dtype in ("bf16", "f16") and p["name"].split("_", 1)[1][0] in "rqh":
        q, es = 8, 2
    elif dtype == "f32" and "_pad" in p["name"]:
        q, es = 4, 4
    if q:
        if K % q:
            pad = _a256(M * ((K + q - 1) // q * q) * es)
        if N % q:
            pad = _a256(pad + K * ((N + q - 1) // q * q) * es)
    if p["split_k"] > 1:
        return pad + p["split_k"] * M * N * 4
    if p["split_k"] == -1:
        G = p["grid_wgs"] - p["sk_dp_tiles"]
        return pad + 2 * G * p["tile_m"] * p["tile_n"] * 4
    return pad


def test_large_d_picks_other_tile_than_2048():
    """Wave quantisation on 256 CUs makes the 2048 and 4096/8192 choices differ."""
    p2 = sam.plan(2048, 2048, 2048, "f32")
    for d in (4096, 8192):
        pd = sam.plan(d, d, d, "f32")
        assert (pd["variant_id"], pd["split_k"]) != (p2["variant_id"], p2["split_k"])


def test_alignment_routes():
    # FP32 ring variants with an element-load form: rows that are not 16-byte
    # pieces are read one value at a time.
    p = sam.variant_plan(39, 4097, 3071, 8191, "f32", 4)
    assert p["a_vector"] == 0 and p["b_vector"] == 0 and p["workspace_bytes"] == 4 * 4097 * 3071 * 4
    p = sam.variant_plan(38, 8191, 8193, 4096, "f32", 1)
    assert p["a_vector"] == 1 and p["b_vector"] == 0 and p["workspace_bytes"] == 0
    # Their padding forms (the measured choice at these sizes) load 16 bytes
    # at a time from copies with rows padded to multiples of 4 values.
    p = sam.plan(4097, 3071, 8191, "f32")
    assert p["name"].startswith("f32_f128x128_w4x2_k32n2_b16_pad_")
    assert p["a_vector"] == 1 and p["b_vector"] == 1
    p = sam.plan(8191, 8193, 4096, "f32")
    assert "_pad_" in p["name"] and p["workspace_bytes"] == _a256(4096 * 8196 * 4)
    p = sam.plan(64, 64, 68, "bf16")
    assert p["a_vector"] == 0 and p["b_vector"] == 1


def test_variant_table():
    n = sam.variant_count()
    assert n >= 5
    seen = set()
    for vid in range(n):
        v = sam.variant_info(vid)
        assert v["variant_id"] == vid and v["name"] not in seen
        seen.add(v["name"])
        assert v["tile_m"] % v["mfma_m"] == 0 and v["tile_n"] % v["mfma_m"] == 0
    with pytest.raises(sam.SamError) as e:
        sam.variant_info(n)
    assert e.value.status == -1


def test_forced_split_admission():
    # K = 64 FP32 is two stages of 32: split 2 is fine, split 3 would leave one empty.
    assert sam.variant_plan(1, 256, 256, 64, "f32", 2)["split_k"] == 2
    with pytest.raises(sam.SamError) as e:
        sam.variant_plan(1, 256, 256, 64, "f32", 3)
    assert e.value.status == -4


@pytest.mark.parametrize("args,code", [
    ((-1, 4, 4), -1), ((4, -1, 4), -1), ((4, 4, -1), -1), ((1 << 31, 4, 4), -1),
])
def test_plan_rejects_bad_sizes(args, code):
    p = sam.SamPlan()
    assert L.sam_gemm_plan(*args, sam.F32, ctypes.byref(p)) == code
    assert L.sam_gemm_plan(4, 4, 4, 7, ctypes.byref(p)) == -1
    assert L.sam_gemm_plan(4, 4, 4, sam.F32, None) == -1


# Fake, never dereferenced device addresses: every call below must be
# rejected by the host checks before any HIP call.
A_, B_, C_, W_ = 0x10000000, 0x20000000, 0x30000000, 0x40000000


def _call(A, B, C, M, N, K, ws=None, wsb=0, fn="sam_gemm_f32"):
    return getattr(L, fn)(A, B, C, M, N, K, ws, wsb, None)


def test_rejects_before_device():
    assert _call(A_, B_, C_, -1, 4, 4) == -1
    assert _call(A_, B_, None, 4, 4, 4) == -1                  # null C
    assert _call(None, B_, C_, 4, 4, 4) == -1                  # null A with K > 0
    assert _call(A_ + 4, B_, C_, 4, 4, 4) == -2                # misaligned A
    assert _call(A_, B_, C_ + 8, 4, 4, 4, fn="sam_gemm_bf16") == -2
    assert _call(A_, B_, A_ + 16, 4, 4, 4) == -1               # C overlaps A
    assert "overlap" in sam.last_error()
    # 16 x 8192 x 8192 plans a split: workspace missing or short
    p = sam.plan(16, 8192, 8192, "f32")
    assert p["workspace_bytes"] > 0
    assert _call(A_, B_, C_, 16, 8192, 8192) == -3
    assert _call(A_, B_, C_, 16, 8192, 8192, W_, p["workspace_bytes"] - 4) == -3


def test_empty_outputs_are_noops():
    # M == 0 or N == 0: nothing to do, nothing touched, even with null pointers.
    assert _call(None, None, None, 0, 5, 5) == 0
    assert _call(None, None, None, 5, 0, 5) == 0


def test_no_gpu_is_reported_not_hidden():
    """Without a usable gfx950 device a well-formed call fails loudly."""
    if L.sam_device_check() == 0:
        pytest.skip("a gfx950 device is present")
    assert _call(A_, B_, C_, 64, 64, 64) == -5
    assert sam.last_error()


def test_stream_k_plans():
    """split_k = -1 asks for a variant's stream-K form: 256 CUs x resident
    workgroups, two BM x BN float slots per workgroup; only the FP32 ring
    variants with tiles up to 128 x 256 have one, and only when there are at
    least as many K iterations as workgroups and at most 2 tiles' worth each."""
    p = sam.variant_plan(35, 300, 300, 4096, "f32", -1)
    assert p["split_k"] == -1 and p["grid_wgs"] == 256
    assert p["workspace_bytes"] == 2 * 256 * 128 * 128 * 4
    assert p["name"].endswith("_sk")
    with pytest.raises(sam.SamError) as e:
        sam.variant_plan(0, 300, 300, 4096, "f32", -1)      # staged variant: no stream-K form
    assert e.value.status == -4
    with pytest.raises(sam.SamError):
        sam.variant_plan(36, 300, 300, 4096, "f32", -1)     # 256 x 256 tiles: none either
    with pytest.raises(sam.SamError):
        sam.variant_plan(35, 64, 64, 64, "f32", -1)         # 1 tile x 1 iteration < 256 workgroups
    with pytest.raises(sam.SamError) as e:
        sam.variant_plan(35, 300, 300, 4096, "f32", -2)
    assert e.value.status == -1


def test_gemm_ex_rejections_before_any_device_call():
    """Bad flags, short leading dimensions and a short workspace are refused on
    the host (no GPU here: the calls must fail before touching one)."""
    f = L.sam_gemm_ex
    A_, B_, C_, W_ = 1 << 20, 2 << 20, 3 << 20, 4 << 20      # aligned, never dereferenced
    vp = ctypes.c_void_p
    assert f(0, 2, 0, 4, 4, 4, 1.0, vp(A_), 4, vp(B_), 4, 0.0, vp(C_), 4, None, 0, None) == -1   # bad trans
    assert f(0, 0, 0, 4, 4, 4, 1.0, vp(A_), 3, vp(B_), 4, 0.0, vp(C_), 4, None, 0, None) == -1   # lda < K
    assert f(0, 1, 0, 8, 4, 4, 1.0, vp(A_), 4, vp(B_), 4, 0.0, vp(C_), 4, None, 0, None) == -1   # lda < M for A^T
    assert f(0, 0, 0, 4, 4, 4, 1.0, vp(A_), 4, vp(B_), 4, 0.0, vp(C_), 3, None, 0, None) == -1   # ldc < N
    need = sam.ex_workspace_bytes(64, 64, 64, True, False, 64, 64, 64, 1.0, 0.0, "f32")
    assert need >= 64 * 64 * 4
    assert f(0, 1, 0, 64, 64, 64, 1.0, vp(A_), 64, vp(B_), 64, 0.0, vp(C_), 64, vp(W_), need - 1, None) == -3
    assert sam.ex_workspace_bytes(64, 64, 64, False, False, 64, 64, 64, 1.0, 0.0, "f32") == 0


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_ex_strided_rows_on_a_16bit_ring_plan_need_no_packed_copy(dtype):
    """A 16-bit ring plan reads padded rows in place when the stride keeps
    16-byte rows, and through its own padded copy when the plan makes one:
    the workspace is then the plan's alone. Other strides, transposes and
    other plan kinds still reserve a packed copy."""
    M, N, K = 1024, 768, 200
    p = sam.plan(M, N, K, dtype)
    assert p["name"].startswith(dtype + "_r")
    ws = lambda ta, tb, lda, ldb: sam.ex_workspace_bytes(M, N, K, ta, tb, lda, ldb, N, 1.0, 0.0, dtype)
    assert ws(False, False, K + 8, N + 16) == p["workspace_bytes"]
    assert ws(False, False, K + 3, N) >= M * K * 2                      # misaligned rows: packed
    if "_b16" in p["name"]:                                             # 16x16x32 ring: A^T read straight
        assert ws(True, False, M, N) == p["workspace_bytes"]
    else:                                                               # 32x32x16 ring: transposed is packed
        assert ws(True, False, M, N) >= M * K * 2
    assert ws(True, False, M + 4, N) >= M * K * 2                       # rows of A^T not 16-byte pieces: packed
    q = sam.plan(2049, 4097, 1025, dtype)                               # plan pads both operands
    assert q["name"].startswith(dtype + "_r") and q["workspace_bytes"] > 0
    assert sam.ex_workspace_bytes(2049, 4097, 1025, False, False, 1028, 4102, 4097, 1.0, 0.0,
                                  dtype) == q["workspace_bytes"]
    r = sam.plan(512, 512, 512, dtype)                                  # staged plan: packed
    assert not r["name"].startswith(dtype + "_r")
    assert sam.ex_workspace_bytes(512, 512, 512, False, False, 520, 520, 512, 1.0, 0.0, dtype) >= 512 * 512 * 4


def test_ex_on_a_ring_plan_writes_c_itself():
    """Ring plans apply ldc and alpha / beta where they store C: no
    temporary product is reserved unless ldc breaks 16-byte stores; other
    plan kinds still take the temporary and the separate pass."""
    M, N, K = 1792, 1792, 256
    p = sam.plan(M, N, K, "f32")
    assert p["name"].startswith("f32_f")
    ws = lambda ldc, a, b: sam.ex_workspace_bytes(M, N, K, False, False, K, N, ldc, a, b, "f32")
    assert ws(N + 8, 0.5, -1.0) == p["workspace_bytes"]
    assert ws(N, 2.0, 0.0) == p["workspace_bytes"]
    assert ws(N + 3, 0.5, -1.0) >= p["workspace_bytes"] + M * N * 4     # ldc % 4 != 0: temporary
    q = sam.plan(256, 256, 256, "f32")
    assert not q["name"].startswith("f32_f")
    assert sam.ex_workspace_bytes(256, 256, 256, False, False, 256, 256, 264, 0.5, -1.0, "f32") >= 256 * 256 * 4


def test_ex_f32_transposed_b_read_straight_where_the_variant_can():
    """FP32 with B given transposed: a ring plan with the transposed-B form
    (tiles up to 128 x 256) reads it in place, K % 4 == 0 and 16-byte rows of
    B^T; the 256 x 256 tile, K % 4 != 0 and misaligned rows still pack B."""
    M = N = K = 2048
    p = sam.plan(M, N, K, "f32")
    assert p["name"].startswith("f32_f128x128")
    ws = lambda M, N, K, ldb: sam.ex_workspace_bytes(M, N, K, False, True, K, ldb, N, 1.0, 0.0, "f32")
    assert ws(M, N, K, K) == p["workspace_bytes"] == 0
    assert ws(M, N, K, K + 4) == 0
    assert ws(M, N, K, K + 2) >= K * N * 4                               # rows of B^T not 16-byte pieces
    q = sam.plan(4096, 4096, 4096, "f32")
    assert q["name"].startswith("f32_f256x256")
    assert ws(4096, 4096, 4096, 4096) >= 4096 * 4096 * 4                 # no transposed-B form: packed
    assert ws(1000, 776, 1030, 1030) >= 1030 * 776 * 4                   # K % 4 != 0: packed


def test_ex_f32_transposed_a_read_straight_where_the_variant_can():
    """FP32 with A given transposed: the same variants read it in place when
    B's and C's rows are 16-byte pieces (any K) and A^T's rows are too."""
    ws = lambda M, N, K, lda: sam.ex_workspace_bytes(M, N, K, True, False, lda, N, N, 1.0, 0.0, "f32")
    assert ws(2048, 2048, 2048, 2048) == 0
    assert ws(2048, 2048, 2048, 2052) == 0
    assert ws(2048, 2048, 2048, 2050) >= 2048 * 2048 * 4                 # rows of A^T not 16-byte pieces
    assert ws(4096, 4096, 4096, 4096) == 0                               # the 256 x 256 tile too
    assert sam.ex_workspace_bytes(2048, 2046, 2048, True, False, 2048, 2046, 2048, 1.0, 0.0, "f32") > 0


def test_mxfp8_plans_and_rejections_before_any_device_call():
    """Block-scaled plans come from the block-scaled variants only; K not a
    multiple of 32, bad formats, a negative split, null scales and the plain
    forced-variant entry point are refused on the host."""
    p = sam.plan(4096, 4096, 4096, "mxfp8")
    assert p["name"].startswith("mxfp8_x") and p["dtype"] == sam.MXFP8
    for shape in [(1, 1, 32), (4096, 4096, 4096), (37, 45, 96), (16, 8192, 8192)]:
        assert sam.plan(*shape, "mxfp8")["name"].startswith("mxfp8_x")
    for vid in range(sam.variant_count()):
        name = sam.variant_info(vid)["name"]
        for dt in ("f32", "bf16", "f16"):
            if name.startswith("x"):
                with pytest.raises(sam.SamError):
                    sam.variant_plan(vid, 256, 256, 256, dt)
        if not name.startswith("x"):
            with pytest.raises(sam.SamError):
                sam.variant_plan(vid, 256, 256, 256, "mxfp8")
    with pytest.raises(sam.SamError):
        sam.plan(64, 64, 48, "mxfp8")
    f = L.sam_gemm_mxfp8
    vp = ctypes.c_void_p
    A_, SA_, B_, SB_, C_ = 1 << 20, 2 << 20, 3 << 20, 4 << 20, 5 << 20   # aligned, never dereferenced
    assert f(0, 0, vp(A_), vp(SA_), vp(B_), vp(SB_), vp(C_), 64, 64, 48, None, 0, None) == -1   # K % 32
    assert f(2, 0, vp(A_), vp(SA_), vp(B_), vp(SB_), vp(C_), 64, 64, 64, None, 0, None) == -1   # format
    assert f(0, 0, vp(A_), None, vp(B_), vp(SB_), vp(C_), 64, 64, 64, None, 0, None) == -1      # null scale
    assert f(0, 0, vp(A_ + 8), vp(SA_), vp(B_), vp(SB_), vp(C_), 64, 64, 64, None, 0, None) == -2  # misaligned
    g = L.sam_gemm_mxfp8_variant
    vid = next(v for v in range(sam.variant_count()) if sam.variant_info(v)["name"].startswith("x"))
    assert g(vid, -1, 0, 0, vp(A_), vp(SA_), vp(B_), vp(SB_), vp(C_), 64, 64, 64, None, 0, None) == -1
    assert g(0, 0, 0, 0, vp(A_), vp(SA_), vp(B_), vp(SB_), vp(C_), 64, 64, 64, None, 0, None) == -4   # not MX
    assert L.sam_gemm_variant(vid, sam.MXFP8, 0, vp(A_), vp(B_), vp(C_), 64, 64, 64, None, 0, None) == -1


def test_mxfp4_plans_and_rejections():
    """E2M1 plans come from the block-scaled variants with twice the values of
    K per stage; K % 32 != 0 and the plain forced-variant entry point are
    refused on the host."""
    p8 = sam.plan(4096, 4096, 4096, "mxfp8")
    p4 = sam.plan(4096, 4096, 4096, "mxfp4")
    assert p4["name"].startswith("mxfp4_x") and p4["dtype"] == sam.MXFP4
    assert sam.variant_plan(p8["variant_id"], 4096, 4096, 4096, "mxfp4", 1)["tile_k"] == 2 * p8["tile_k"]
    with pytest.raises(sam.SamError):
        sam.plan(64, 64, 48, "mxfp4")
    vp = ctypes.c_void_p
    A_, SA_, B_, SB_, C_ = 1 << 20, 2 << 20, 3 << 20, 4 << 20, 5 << 20
    assert L.sam_gemm_mxfp4(vp(A_), vp(SA_), vp(B_), vp(SB_), vp(C_), 64, 64, 48, None, 0, None) == -1
    assert L.sam_gemm_mxfp4(vp(A_), None, vp(B_), vp(SB_), vp(C_), 64, 64, 64, None, 0, None) == -1
    assert L.sam_gemm_mxfp4_variant(0, 0, vp(A_), vp(SA_), vp(B_), vp(SB_), vp(C_), 64, 64, 64, None, 0, None) == -4
    assert L.sam_gemm_variant(p4["variant_id"], sam.MXFP4, 0, vp(A_), vp(B_), vp(C_), 64, 64, 64, None, 0, None) == -1


def test_binding_rejects_host_tensors_and_bad_c():
    """The binding checks C (shape, float32, contiguity) and that every tensor
    is a GPU tensor before it calls into the library: a host pointer or a
    short C must never reach a kernel."""
    import torch
    A = torch.ones(4, 3)
    B = torch.ones(3, 5)
    with pytest.raises(ValueError, match="GPU tensor"):
        sam.gemm(A, B)
    with pytest.raises(ValueError, match="GPU tensor"):
        sam.gemm_variant(0, A, B, torch.empty(4, 5))
    with pytest.raises(ValueError, match="shape"):
        sam.gemm(A, B, torch.empty(4, 4))
    with pytest.raises(ValueError, match="shape"):
        sam.gemm_variant(0, A, B, torch.empty(5, 4))
    with pytest.raises(TypeError, match="float32"):
        sam.gemm(A, B, torch.empty(4, 5, dtype=torch.float64))
    with pytest.raises(ValueError, match="contiguous"):
        sam.gemm(A, B, torch.empty(5, 4).t())
    with pytest.raises(ValueError, match="contiguous"):
        sam.gemm(A, B, torch.empty(4, 5), workspace=torch.empty(8, 2).t())
    with pytest.raises(ValueError, match="GPU tensor"):
        sam.gemm_ex(A, B)
    u8 = torch.zeros(4, 32, dtype=torch.uint8)
    s8 = torch.zeros(4, 1, dtype=torch.uint8)
    with pytest.raises(ValueError, match="shape"):
        sam.gemm_mxfp8(u8, s8, u8, s8, C=torch.empty(3, 4))
    with pytest.raises(ValueError, match="GPU tensor"):
        sam.gemm_mxfp8(u8, s8, u8, s8)
    with pytest.raises(ValueError, match="GPU tensor"):
        sam.gemm_mxfp4(u8[:, :16].contiguous(), s8, u8[:, :16].contiguous(), s8)


def test_noalloc_refusals_before_any_device_call():
    """sam_gemm_noalloc refuses, on the host, a plan whose workspace exceeds
    its scratch array (SAM_ERR_WORKSPACE) and bad dtypes or sizes; without a
    GPU an ordinary call reports the missing device."""
    vp = ctypes.c_void_p
    big = sam.plan(4097, 3071, 8191, "f32")["workspace_bytes"]
    assert big > sam.SCRATCH_BYTES
    assert L.sam_gemm_noalloc(sam.F32, vp(16), vp(1 << 40), vp(1 << 41), 4097, 3071, 8191, None) == -3
    assert "scratch" in sam.last_error()
    assert L.sam_gemm_noalloc(sam.MXFP8, vp(16), vp(32), vp(48), 4, 4, 32, None) == -1
    assert L.sam_gemm_noalloc(sam.F32, vp(16), vp(32), vp(48), -1, 4, 4, None) == -1
    assert L.sam_gemm_noalloc(sam.F32, None, None, None, 0, 4, 4, None) == 0
    rc = L.sam_gemm_noalloc(sam.F32, vp(16), vp(1 << 40), vp(1 << 41), 16, 8192, 8192, None)
    assert rc == -5, rc


def test_no_alloc_pairs_still_need_scratch():
    """The allocation-free entry point's GPU test compares calls whose
    plans use the scratch array (split-K or stream-K workspace within its
    size); planner changes must not turn any of them into a plan without."""
    from tests.test_zz_no_alloc import PAIRS
    for pair in PAIRS:
        for (M, N, K, dtype) in pair:
            p = sam.plan(M, N, K, dtype)
            assert 0 < p["workspace_bytes"] <= sam.SCRATCH_BYTES, (M, N, K, dtype, p["name"])
    firsts = [sam.plan(*pair[0][:3], pair[0][3])["workspace_bytes"] for pair in PAIRS]
    seconds = [sam.plan(*pair[1][:3], pair[1][3])["workspace_bytes"] for pair in PAIRS]
    assert any(b < a for a, b in zip(firsts, seconds))        # a smaller second call is covered
