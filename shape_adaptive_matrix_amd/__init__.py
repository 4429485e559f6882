"""Python binding of the shape-adaptive GEMM library (``libsam.so``).

Argument marshalling only: every step of C = A·B runs in the library's HIP
kernels. PyTorch supplies device memory and the current stream; nothing here
computes a product, and there is no CPU fallback — if the library is missing
or the device is not gfx950 the call raises.

The C ABI is declared in ``include/sam.h``; the names here follow it without
the ``sam_`` prefix.
"""
from __future__ import annotations

import ctypes
import re
from pathlib import Path

import os

PKG = Path(__file__).resolve().parent
# SAM_LIBRARY may point at another build of the same library (A/B timing).
LIB_PATH = Path(os.environ.get("SAM_LIBRARY", PKG / "libsam.so"))
HEADER = PKG.parent / "include" / "sam.h"

F32, BF16, F16, MXFP8, MXFP4 = 0, 1, 2, 3, 4
DTYPES = {"f32": F32, "bf16": BF16, "f16": F16, "mxfp8": MXFP8, "mxfp4": MXFP4}
FP8_FORMATS = {"e4m3": 0, "e5m2": 1}
DTYPE_NAMES = {v: k for k, v in DTYPES.items()}

STATUS = {
    0: "SAM_OK", -1: "SAM_ERR_INVALID_ARG", -2: "SAM_ERR_MISALIGNED",
    -3: "SAM_ERR_WORKSPACE", -4: "SAM_ERR_UNSUPPORTED",
    -5: "SAM_ERR_UNSUPPORTED_DEVICE", -6: "SAM_ERR_LAUNCH", -7: "SAM_ERR_INTERNAL",
}


class SamError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        self.name = STATUS.get(status, str(status))
        super().__init__(f"{self.name}: {detail}")


class SamPlan(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32), ("variant_id", ctypes.c_int32),
        ("name", ctypes.c_char * 64), ("dtype", ctypes.c_int32),
        ("tile_m", ctypes.c_int32), ("tile_n", ctypes.c_int32), ("tile_k", ctypes.c_int32),
        ("waves_m", ctypes.c_int32), ("waves_n", ctypes.c_int32), ("mfma_m", ctypes.c_int32),
        ("split_k", ctypes.c_int32), ("group_m", ctypes.c_int32), ("xcd_remap", ctypes.c_int32),
        ("a_vector", ctypes.c_int32), ("b_vector", ctypes.c_int32),
        ("grid_wgs", ctypes.c_int64), ("workspace_bytes", ctypes.c_uint64),
        ("est_us", ctypes.c_double), ("raster_n", ctypes.c_int32), ("operand_swap", ctypes.c_int32),
        ("sk_dp_tiles", ctypes.c_int64), ("tuned", ctypes.c_int32),
    ]

    def as_dict(self) -> dict:
        d = {f: getattr(self, f) for f, _ in self._fields_}
        d["name"] = self.name.decode()
        return d


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library. Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not LIB_PATH.exists():
        raise ImportError(f"{LIB_PATH} is missing: run `python -m shape_adaptive_matrix_amd.build`")
    # torch ships its own HIP runtime under the same soname as the system one
    # libsam.so links. Whichever is loaded first serves the whole process, and
    # torch cannot initialise the GPU on the other; so when torch is present
    # it is loaded first and the library binds to its runtime.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    L = ctypes.CDLL(str(LIB_PATH))
    i64, u64, vp, i32 = ctypes.c_int64, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int32
    P = ctypes.POINTER(SamPlan)
    sig = {
        "sam_gemm_plan": ([i64, i64, i64, ctypes.c_int, P], ctypes.c_int),
        "sam_gemm_f32": ([vp, vp, vp, i64, i64, i64, vp, u64, vp], ctypes.c_int),
        "sam_gemm_bf16": ([vp, vp, vp, i64, i64, i64, vp, u64, vp], ctypes.c_int),
        "sam_gemm_f16": ([vp, vp, vp, i64, i64, i64, vp, u64, vp], ctypes.c_int),
        "sam_variant_count": ([], i32),
        "sam_variant_info": ([i32, P], ctypes.c_int),
        "sam_variant_plan": ([i32, i64, i64, i64, ctypes.c_int, i32, P], ctypes.c_int),
        "sam_gemm_variant": ([i32, ctypes.c_int, i32, vp, vp, vp, i64, i64, i64, vp, u64, vp], ctypes.c_int),
        "sam_variant_plan_r": ([i32, i64, i64, i64, ctypes.c_int, i32, i32, P], ctypes.c_int),
        "sam_gemm_variant_r": ([i32, ctypes.c_int, i32, i32, vp, vp, vp, i64, i64, i64, vp, u64, vp], ctypes.c_int),
        "sam_gemm_plan_model": ([i64, i64, i64, ctypes.c_int, P], ctypes.c_int),
        "sam_gemm_ex": ([ctypes.c_int, ctypes.c_int, ctypes.c_int, i64, i64, i64, ctypes.c_float, vp, i64, vp, i64,
                         ctypes.c_float, vp, i64, vp, u64, vp], ctypes.c_int),
        "sam_gemm_ex_workspace": ([ctypes.c_int, ctypes.c_int, ctypes.c_int, i64, i64, i64, i64, i64, i64,
                                   ctypes.c_float, ctypes.c_float, ctypes.POINTER(ctypes.c_uint64)], ctypes.c_int),
        "sam_gemm_ex_variant": ([i32, i32, i32, ctypes.c_int, ctypes.c_int, ctypes.c_int, i64, i64, i64,
                                 ctypes.c_float, vp, i64, vp, i64, ctypes.c_float, vp, i64, vp, u64, vp],
                                ctypes.c_int),
        "sam_gemm_ex_variant_workspace": ([i32, i32, i32, ctypes.c_int, ctypes.c_int, ctypes.c_int, i64, i64, i64,
                                           i64, i64, i64, ctypes.c_float, ctypes.c_float,
                                           ctypes.POINTER(ctypes.c_uint64)], ctypes.c_int),
        "sam_gemm_mxfp8": ([ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, vp, i64, i64, i64, vp, u64, vp],
                           ctypes.c_int),
        "sam_gemm_mxfp8_variant": ([i32, i32, ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, vp, i64, i64, i64, vp,
                                    u64, vp], ctypes.c_int),
        "sam_gemm_mxfp4": ([vp, vp, vp, vp, vp, i64, i64, i64, vp, u64, vp], ctypes.c_int),
        "sam_gemm_mxfp4_variant": ([i32, i32, vp, vp, vp, vp, vp, i64, i64, i64, vp, u64, vp], ctypes.c_int),
        "sam_gemm_noalloc": ([ctypes.c_int, vp, vp, vp, i64, i64, i64, vp], ctypes.c_int),
        "sam_device_check": ([], ctypes.c_int),
        "sam_status_string": ([ctypes.c_int], ctypes.c_char_p),
        "sam_last_error": ([], ctypes.c_char_p),
        "sam_build_info": ([], ctypes.c_char_p),
    }
    for name, (args, res) in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = res
    _lib = L
    return L


def header_symbols() -> list[str]:
    """Function names declared in include/sam.h."""
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sam_\w+)\s*\(", text)))


def _check(status: int):
    if status != 0:
        raise SamError(status, lib().sam_last_error().decode())


def _dt(dtype) -> int:
    if isinstance(dtype, int):
        return dtype
    return DTYPES[dtype]


# -- host-only queries ---------------------------------------------------------
def plan(M: int, N: int, K: int, dtype="f32") -> dict:
    p = SamPlan()
    _check(lib().sam_gemm_plan(M, N, K, _dt(dtype), ctypes.byref(p)))
    return p.as_dict()


def variant_count() -> int:
    return lib().sam_variant_count()


def variant_info(vid: int) -> dict:
    p = SamPlan()
    _check(lib().sam_variant_info(vid, ctypes.byref(p)))
    return p.as_dict()


def variant_plan(vid: int, M: int, N: int, K: int, dtype="f32", split_k: int = 0, raster: int = -1) -> dict:
    """Plan of a forced variant and split (0: its own choice, -1: stream-K)
    and raster order (-1: the cost model's choice, 0 M-major, 1 N-major)."""
    p = SamPlan()
    _check(lib().sam_variant_plan_r(vid, M, N, K, _dt(dtype), split_k, raster, ctypes.byref(p)))
    return p.as_dict()


def plan_model(M: int, N: int, K: int, dtype="f32") -> dict:
    """The cost model's own plan, ignoring the frozen table (host only)."""
    p = SamPlan()
    _check(lib().sam_gemm_plan_model(M, N, K, _dt(dtype), ctypes.byref(p)))
    return p.as_dict()


def build_info() -> str:
    return lib().sam_build_info().decode()


def device_check() -> None:
    _check(lib().sam_device_check())


def last_error() -> str:
    return lib().sam_last_error().decode()


# -- device calls (torch tensors for memory and streams) ------------------------
def _torch_dtype_code(t, dtype):
    import torch
    if dtype is not None:
        return _dt(dtype)
    m = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16}
    if t.dtype not in m:
        raise TypeError(f"pass dtype= for operands of type {t.dtype}")
    return m[t.dtype]


def _stream_ptr(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() else None


def _on_device(tensors, names, device=None):
    """Every tensor lives on one GPU (the first one's unless `device` is
    given): the library is handed raw device pointers, and a host pointer or
    another GPU's memory must never reach a kernel."""
    dev = device
    for t, name in zip(tensors, names):
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor (got device {t.device})")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the other operands on {dev}")
    return dev


def _operands(A, B, dtype):
    code = _torch_dtype_code(A, dtype)
    if A.dim() != 2 or B.dim() != 2 or A.shape[1] != B.shape[0]:
        raise ValueError(f"bad shapes {tuple(A.shape)} x {tuple(B.shape)}")
    if not (A.is_contiguous() and B.is_contiguous()):
        raise ValueError("A and B must be contiguous row-major")
    want = 4 if code == F32 else 2
    if A.element_size() != want or B.element_size() != want:
        raise TypeError("operand element size does not match the dtype")
    return code


def _output(C, M, N, others, names, workspace=None):
    """Checks, before anything reaches the library, that the caller's C is a
    compact float32 [M][N] matrix and that C, the workspace and the operands
    (`others`) all live on one GPU; returns C, or a new one on that GPU."""
    import torch
    if C is not None:
        if C.dtype != torch.float32:
            raise TypeError(f"C must be float32 (got {C.dtype})")
        if tuple(C.shape) != (M, N):
            raise ValueError(f"C must have shape ({M}, {N}) (got {tuple(C.shape)})")
        if not C.is_contiguous():
            raise ValueError("C must be contiguous row-major")
    if workspace is not None and not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    dev = _on_device((*others, C, workspace), (*names, "C", "workspace"))
    if C is None:
        C = torch.empty((M, N), dtype=torch.float32, device=dev)
    return C


def _workspace_bytes(workspace) -> int:
    return 0 if workspace is None else workspace.numel() * workspace.element_size()


def workspace_for(plan_dict: dict, device, stream=None):
    """A workspace of the plan's size, allocated on `stream` (torch's current
    stream when None). The caching allocator hands freed memory only to later
    work on the stream it was allocated on, so a workspace that goes out of
    scope when the call returns is not reused while the call's kernels, queued
    on that stream, still use it."""
    import torch
    n = int(plan_dict["workspace_bytes"])
    if n == 0:
        return None
    if stream is None:
        return torch.empty((n + 3) // 4, dtype=torch.float32, device=device)
    with torch.cuda.stream(stream):
        return torch.empty((n + 3) // 4, dtype=torch.float32, device=device)


def gemm(A, B, C=None, dtype=None, workspace=None, stream=None):
    """C = A·B on the tensors' device through the dispatcher; returns C (FP32)."""
    code = _operands(A, B, dtype)
    M, K = A.shape
    N = B.shape[1]
    C = _output(C, M, N, (A, B), ("A", "B"), workspace)
    p = plan(M, N, K, code)
    if workspace is None:
        workspace = workspace_for(p, A.device, stream)
    ws_bytes = _workspace_bytes(workspace)
    fn = {F32: lib().sam_gemm_f32, BF16: lib().sam_gemm_bf16, F16: lib().sam_gemm_f16}[code]
    _check(fn(_ptr(A), _ptr(B), _ptr(C), M, N, K, _ptr(workspace), ws_bytes, _stream_ptr(stream)))
    return C


def gemm_variant(vid: int, A, B, C=None, split_k: int = 0, dtype=None, workspace=None, stream=None,
                 raster: int = -1):
    """C = A·B with a forced variant (and split; 0 = the variant's own pick;
    raster -1 = the cost model's raster order, 0 M-major, 1 N-major)."""
    code = _operands(A, B, dtype)
    M, K = A.shape
    N = B.shape[1]
    C = _output(C, M, N, (A, B), ("A", "B"), workspace)
    p = variant_plan(vid, M, N, K, code, split_k, raster)
    if workspace is None:
        workspace = workspace_for(p, A.device, stream)
    ws_bytes = _workspace_bytes(workspace)
    _check(lib().sam_gemm_variant_r(vid, code, p["split_k"], p["raster_n"], _ptr(A), _ptr(B), _ptr(C), M, N, K,
                                    _ptr(workspace), ws_bytes, _stream_ptr(stream)))
    return C


SCRATCH_BYTES = 64 << 20   # SAM_SCRATCH_BYTES of include/sam.h


def gemm_noalloc(A, B, C=None, dtype=None, stream=None):
    """C = A·B through sam_gemm_noalloc: the plan of gemm(), with its
    workspace in the library's per-GPU scratch array (no allocation in the
    library; C is allocated here only when not given)."""
    code = _operands(A, B, dtype)
    M, K = A.shape
    N = B.shape[1]
    C = _output(C, M, N, (A, B), ("A", "B"))
    _check(lib().sam_gemm_noalloc(code, _ptr(A), _ptr(B), _ptr(C), M, N, K, _stream_ptr(stream)))
    return C


def _rows(t, name):
    """Row stride of a 2-D tensor whose rows are contiguous (a compact matrix
    or a view of one with padded rows)."""
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError(f"{name} must be 2-D with contiguous rows")
    return max(int(t.stride(0)), int(t.shape[1]), 1)


def ex_workspace_bytes(M, N, K, trans_a, trans_b, lda, ldb, ldc, alpha, beta, dtype="f32", variant=None,
                       split=0, raster=-1) -> int:
    n = ctypes.c_uint64()
    if variant is None:
        _check(lib().sam_gemm_ex_workspace(_dt(dtype), int(trans_a), int(trans_b), M, N, K, lda, ldb, ldc,
                                           float(alpha), float(beta), ctypes.byref(n)))
    else:
        _check(lib().sam_gemm_ex_variant_workspace(int(variant), int(split), int(raster), _dt(dtype), int(trans_a),
                                                   int(trans_b), M, N, K, lda, ldb, ldc, float(alpha), float(beta),
                                                   ctypes.byref(n)))
    return int(n.value)


def gemm_ex(A, B, C=None, trans_a=False, trans_b=False, alpha=1.0, beta=0.0, dtype=None, workspace=None,
            stream=None, variant=None, split=0, raster=-1):
    """C = alpha·op(A)·op(B) + beta·C (sam_gemm_ex); returns C. op(A) is A or
    A.T as stored (A is K x M when trans_a), likewise B; A, B and C may be
    views with padded rows (their row stride is the leading dimension).
    variant: a forced plan (sam_gemm_ex_variant, with split and raster)."""
    import torch
    code = _torch_dtype_code(A, dtype)
    want = 4 if code == F32 else 2
    if A.element_size() != want or B.element_size() != want:
        raise TypeError("operand element size does not match the dtype")
    lda, ldb = _rows(A, "A"), _rows(B, "B")
    M, K = (A.shape[1], A.shape[0]) if trans_a else (A.shape[0], A.shape[1])
    Kb, N = (B.shape[1], B.shape[0]) if trans_b else (B.shape[0], B.shape[1])
    if Kb != K:
        raise ValueError(f"op(A) is {M}x{K} but op(B) is {Kb}x{N}")
    if workspace is not None and not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    dev = _on_device((A, B, C, workspace), ("A", "B", "C", "workspace"))
    if C is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs C")
        C = torch.empty((M, N), dtype=torch.float32, device=dev)
    if tuple(C.shape) != (M, N) or C.dtype != torch.float32:
        raise ValueError(f"C must be float32 [{M}, {N}]")
    ldc = _rows(C, "C")
    if workspace is None:
        n = ex_workspace_bytes(M, N, K, trans_a, trans_b, lda, ldb, ldc, alpha, beta, code, variant, split, raster)
        workspace = workspace_for({"workspace_bytes": n}, dev, stream)
    ws_bytes = _workspace_bytes(workspace)
    tail = (M, N, K, float(alpha), _ptr(A), lda, _ptr(B), ldb, float(beta), _ptr(C), ldc, _ptr(workspace), ws_bytes,
            _stream_ptr(stream))
    if variant is None:
        _check(lib().sam_gemm_ex(code, int(trans_a), int(trans_b), *tail))
    else:
        _check(lib().sam_gemm_ex_variant(int(variant), int(split), int(raster), code, int(trans_a), int(trans_b),
                                         *tail))
    return C



def _mx_operands(A, SA, Bt, SB, fmt_a, fmt_b):
    import torch
    for t, name in ((A, "A"), (SA, "scale_a"), (Bt, "Bt"), (SB, "scale_b")):
        if t.dtype != torch.uint8 or t.dim() != 2 or not t.is_contiguous():
            raise TypeError(f"{name} must be a contiguous 2-D uint8 tensor")
    M, K = A.shape
    N = Bt.shape[0]
    if Bt.shape[1] != K or tuple(SA.shape) != (M, K // 32) or tuple(SB.shape) != (N, K // 32):
        raise ValueError(f"bad shapes A{tuple(A.shape)} scale_a{tuple(SA.shape)} Bt{tuple(Bt.shape)} "
                         f"scale_b{tuple(SB.shape)}")
    return M, N, K, FP8_FORMATS[fmt_a], FP8_FORMATS[fmt_b]


def gemm_mxfp8(A, SA, Bt, SB, fmt_a="e4m3", fmt_b="e4m3", C=None, workspace=None, stream=None):
    """Block-scaled 8-bit GEMM (sam_gemm_mxfp8): A [M][K] and Bt [N][K] element
    codes, SA [M][K/32] and SB [N][K/32] E8M0 scale codes, all uint8 on the
    device; returns C [M][N] FP32."""
    import torch
    M, N, K, fa, fb = _mx_operands(A, SA, Bt, SB, fmt_a, fmt_b)
    C = _output(C, M, N, (A, SA, Bt, SB), ("A", "scale_a", "Bt", "scale_b"), workspace)
    if workspace is None:
        workspace = workspace_for(plan(M, N, K, MXFP8), A.device, stream)
    ws_bytes = _workspace_bytes(workspace)
    _check(lib().sam_gemm_mxfp8(fa, fb, _ptr(A), _ptr(SA), _ptr(Bt), _ptr(SB), _ptr(C), M, N, K, _ptr(workspace),
                                ws_bytes, _stream_ptr(stream)))
    return C


def gemm_mxfp8_variant(vid: int, A, SA, Bt, SB, fmt_a="e4m3", fmt_b="e4m3", C=None, split_k: int = 0,
                       workspace=None, stream=None):
    """gemm_mxfp8 with a forced variant and split (0 = the variant's pick)."""
    import torch
    M, N, K, fa, fb = _mx_operands(A, SA, Bt, SB, fmt_a, fmt_b)
    C = _output(C, M, N, (A, SA, Bt, SB), ("A", "scale_a", "Bt", "scale_b"), workspace)
    p = variant_plan(vid, M, N, K, MXFP8, split_k)
    if workspace is None:
        workspace = workspace_for(p, A.device, stream)
    ws_bytes = _workspace_bytes(workspace)
    _check(lib().sam_gemm_mxfp8_variant(vid, p["split_k"], fa, fb, _ptr(A), _ptr(SA), _ptr(Bt), _ptr(SB), _ptr(C),
                                        M, N, K, _ptr(workspace), ws_bytes, _stream_ptr(stream)))
    return C


def _mx4_operands(A, SA, Bt, SB):
    import torch
    for t, name in ((A, "A"), (SA, "scale_a"), (Bt, "Bt"), (SB, "scale_b")):
        if t.dtype != torch.uint8 or t.dim() != 2 or not t.is_contiguous():
            raise TypeError(f"{name} must be a contiguous 2-D uint8 tensor")
    M, K = A.shape[0], 2 * A.shape[1]
    N = Bt.shape[0]
    if Bt.shape[1] != K // 2 or tuple(SA.shape) != (M, K // 32) or tuple(SB.shape) != (N, K // 32):
        raise ValueError(f"bad shapes A{tuple(A.shape)} scale_a{tuple(SA.shape)} Bt{tuple(Bt.shape)} "
                         f"scale_b{tuple(SB.shape)}")
    return M, N, K


def gemm_mxfp4(A, SA, Bt, SB, C=None, workspace=None, stream=None):
    """Block-scaled 4-bit GEMM (sam_gemm_mxfp4): A [M][K/2] and Bt [N][K/2]
    bytes of packed E2M1 codes (low nibble first), SA [M][K/32] and SB
    [N][K/32] E8M0 scale codes, all uint8 on the device; returns C [M][N] FP32."""
    import torch
    M, N, K = _mx4_operands(A, SA, Bt, SB)
    C = _output(C, M, N, (A, SA, Bt, SB), ("A", "scale_a", "Bt", "scale_b"), workspace)
    if workspace is None:
        workspace = workspace_for(plan(M, N, K, MXFP4), A.device, stream)
    ws_bytes = _workspace_bytes(workspace)
    _check(lib().sam_gemm_mxfp4(_ptr(A), _ptr(SA), _ptr(Bt), _ptr(SB), _ptr(C), M, N, K, _ptr(workspace), ws_bytes,
                                _stream_ptr(stream)))
    return C


def gemm_mxfp4_variant(vid: int, A, SA, Bt, SB, C=None, split_k: int = 0, workspace=None, stream=None):
    """gemm_mxfp4 with a forced variant and split (0 = the variant's pick)."""
    import torch
    M, N, K = _mx4_operands(A, SA, Bt, SB)
    C = _output(C, M, N, (A, SA, Bt, SB), ("A", "scale_a", "Bt", "scale_b"), workspace)
    p = variant_plan(vid, M, N, K, MXFP4, split_k)
    if workspace is None:
        workspace = workspace_for(p, A.device, stream)
    ws_bytes = _workspace_bytes(workspace)
    _check(lib().sam_gemm_mxfp4_variant(vid, p["split_k"], _ptr(A), _ptr(SA), _ptr(Bt), _ptr(SB), _ptr(C), M, N, K,
                                        _ptr(workspace), ws_bytes, _stream_ptr(stream)))
    return C
