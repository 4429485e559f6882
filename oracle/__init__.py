"""Reference GEMM in double precision (the oracle).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import this package. The product path (the
HIP library under ``shape_adaptive_matrix_amd``) never imports it, and the two
share no code.

What it computes: C = A·B for compact row-major operands, alpha one and beta
zero (page "Scale coverage exposes a remaining GEMM gap", section "Measurement
contract and evidence"), with FP32 or 16-bit (bfloat16 / binary16) operands as
in page "Measured data point on fixed-tile vs shape-adaptive GEMM", section
"One more result that surprised us". Values are decoded exactly to double and
summed in double in ascending k. Block-scaled 8-bit operands (the OCP MX
formats E4M3 / E5M2 with E8M0 scales per 32 values of K, the reading taken
for the block-scaled FP4 GEMM of page "fix(fp4_gemm autotune) SM107 kernel
family excluded from autotune candidates and heuristics update - #4856")
follow the same rule with each value multiplied by its block's scale. The arithmetic lives in ``oracle.c``; this
module only builds and calls it.

Every function here is pinned by ``tests/test_oracle_pins.py`` (brute force,
closed forms, invariants, the FP64 error bound); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

HERE = Path(__file__).resolve().parent
SRC = HERE / "oracle.c"
LIB = HERE / "liboracle.so"

F32, BF16, F16 = 0, 1, 2
_DTYPES = {"f32": F32, "bf16": BF16, "f16": F16}
FP8 = {"e4m3": 0, "e5m2": 1}

CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
          "-shared", "-fPIC", "-std=c11"]


def build(src: Path = SRC, out: Path = LIB, extra_flags=()) -> Path:
    """Compile ``src`` into the shared library ``out`` with gcc.

    The old library is deleted first, so a failed compile never leaves a
    stale one behind.
    """
    out = Path(out)
    if out.exists():
        out.unlink()
    tmp = out.with_suffix(".so.tmp")
    cmd = ["gcc", *CFLAGS, *extra_flags, str(src), "-o", str(tmp), "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


class Oracle:
    """ctypes view of one compiled oracle library."""

    def __init__(self, path: Path = LIB):
        path = Path(path)
        if not path.exists():
            build(out=path)
        self.path = path
        lib = ctypes.CDLL(str(path))
        i64, vp, dp = ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p
        lib.oracle_gemm.argtypes = [ctypes.c_int, vp, vp, i64, i64, i64, dp,
                                    ctypes.c_int]
        lib.oracle_gemm.restype = ctypes.c_int
        lib.oracle_gemm_rows.argtypes = [ctypes.c_int, vp, vp, i64, i64, i64,
                                         i64, i64, dp, ctypes.c_int]
        lib.oracle_gemm_rows.restype = ctypes.c_int
        lib.oracle_gemm_points.argtypes = [ctypes.c_int, vp, vp, i64, i64,
                                           i64, vp, vp, i64, dp, ctypes.c_int]
        lib.oracle_gemm_points.restype = ctypes.c_int
        lib.oracle_decode_bf16.argtypes = [ctypes.c_uint16]
        lib.oracle_decode_bf16.restype = ctypes.c_double
        lib.oracle_decode_f16.argtypes = [ctypes.c_uint16]
        lib.oracle_decode_f16.restype = ctypes.c_double
        lib.oracle_gemm_ex.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, i64, i64, i64, ctypes.c_double,
                                       vp, i64, vp, i64, ctypes.c_double, vp, dp, ctypes.c_int]
        lib.oracle_gemm_ex.restype = ctypes.c_int
        lib.oracle_decode_fp8.argtypes = [ctypes.c_int, ctypes.c_uint8]
        lib.oracle_decode_fp8.restype = ctypes.c_double
        lib.oracle_decode_e8m0.argtypes = [ctypes.c_uint8]
        lib.oracle_decode_e8m0.restype = ctypes.c_double
        lib.oracle_gemm_mxfp8.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, i64, i64, i64, dp,
                                          ctypes.c_int]
        lib.oracle_gemm_mxfp8.restype = ctypes.c_int
        lib.oracle_gemm_mxfp8_points.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, i64, i64, i64,
                                                 vp, vp, i64, dp, ctypes.c_int]
        lib.oracle_gemm_mxfp8_points.restype = ctypes.c_int
        lib.oracle_decode_fp4.argtypes = [ctypes.c_uint8]
        lib.oracle_decode_fp4.restype = ctypes.c_double
        lib.oracle_gemm_mxfp4.argtypes = [vp, vp, vp, vp, i64, i64, i64, dp, ctypes.c_int]
        lib.oracle_gemm_mxfp4.restype = ctypes.c_int
        lib.oracle_gemm_mxfp4_points.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, vp, i64, dp, ctypes.c_int]
        lib.oracle_gemm_mxfp4_points.restype = ctypes.c_int
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = ctypes.c_int
        self.lib = lib

    # -- helpers -----------------------------------------------------------
    @staticmethod
    def _operands(dtype: str, A, B):
        code = _DTYPES[dtype]
        want = np.float32 if code == F32 else np.uint16
        A = np.ascontiguousarray(A)
        B = np.ascontiguousarray(B)
        if A.dtype != want or B.dtype != want:
            raise TypeError(f"{dtype} operands must be {np.dtype(want).name}")
        if A.ndim != 2 or B.ndim != 2 or A.shape[1] != B.shape[0]:
            raise ValueError(f"bad shapes {A.shape} x {B.shape}")
        return code, A, B

    @staticmethod
    def _ptr(a: np.ndarray):
        return a.ctypes.data_as(ctypes.c_void_p) if a.size else None

    # -- entry points --------------------------------------------------------
    def gemm(self, dtype: str, A, B, nthreads: int = 0) -> np.ndarray:
        """Full C = A·B as float64[M, N]."""
        code, A, B = self._operands(dtype, A, B)
        M, K = A.shape
        N = B.shape[1]
        C = np.empty((M, N), dtype=np.float64)
        rc = self.lib.oracle_gemm(code, self._ptr(A), self._ptr(B), M, N, K,
                                  self._ptr(C), nthreads)
        if rc != 0:
            raise ValueError("oracle_gemm rejected its arguments")
        return C

    def gemm_rows(self, dtype: str, A, B, row0: int, nrows: int,
                  nthreads: int = 0) -> np.ndarray:
        """Rows [row0, row0+nrows) of C as float64[nrows, N]."""
        code, A, B = self._operands(dtype, A, B)
        M, K = A.shape
        N = B.shape[1]
        C = np.empty((nrows, N), dtype=np.float64)
        rc = self.lib.oracle_gemm_rows(code, self._ptr(A), self._ptr(B), M, N,
                                       K, row0, nrows, self._ptr(C), nthreads)
        if rc != 0:
            raise ValueError("oracle_gemm_rows rejected its arguments")
        return C

    def gemm_points(self, dtype: str, A, B, rows, cols,
                    nthreads: int = 0) -> np.ndarray:
        """C[rows[p], cols[p]] for every p, as float64[npts]."""
        code, A, B = self._operands(dtype, A, B)
        M, K = A.shape
        N = B.shape[1]
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        cols = np.ascontiguousarray(cols, dtype=np.int64)
        if rows.shape != cols.shape or rows.ndim != 1:
            raise ValueError("rows and cols must be equal-length vectors")
        out = np.empty(rows.shape[0], dtype=np.float64)
        rc = self.lib.oracle_gemm_points(code, self._ptr(A), self._ptr(B), M,
                                         N, K, self._ptr(rows),
                                         self._ptr(cols), rows.shape[0],
                                         self._ptr(out), nthreads)
        if rc != 0:
            raise ValueError("oracle_gemm_points rejected its arguments")
        return out

    def gemm_ex(self, dtype: str, M: int, N: int, K: int, A, lda: int, B, ldb: int, trans_a: bool,
                       trans_b: bool, alpha: float, beta: float, C0=None, nthreads: int = 0) -> np.ndarray:
        """alpha·op(A)·op(B) + beta·C0 as float64[M, N] (oracle_gemm_ex), with
        A and B given as flat buffers and explicit row strides."""
        code = _DTYPES[dtype]
        want = np.float32 if code == F32 else np.uint16
        A = np.ascontiguousarray(A).ravel()
        B = np.ascontiguousarray(B).ravel()
        if A.dtype != want or B.dtype != want:
            raise TypeError(f"{dtype} operands must be {np.dtype(want).name}")
        C0p = None
        if C0 is not None:   # handed over as given: the C side must not read it when beta is 0
            C0 = np.ascontiguousarray(C0, dtype=np.float32)
            if C0.shape != (M, N):
                raise ValueError("C0 must be [M, N]")
            C0p = self._ptr(C0)
        out = np.empty((M, N), dtype=np.float64)
        rc = self.lib.oracle_gemm_ex(code, int(bool(trans_a)), int(bool(trans_b)), M, N, K, float(alpha),
                                     self._ptr(A), lda, self._ptr(B), ldb, float(beta), C0p, self._ptr(out),
                                     nthreads)
        if rc != 0:
            raise ValueError("oracle_gemm_ex rejected its arguments")
        return out

    def decode(self, dtype: str, bits: int) -> float:
        """Exact value of one 16-bit bit pattern."""
        if dtype == "bf16":
            return self.lib.oracle_decode_bf16(bits)
        if dtype == "f16":
            return self.lib.oracle_decode_f16(bits)
        raise ValueError(dtype)

    # -- block-scaled 8-bit operands (OCP MX formats) ------------------------
    @staticmethod
    def _mx_operands(A, SA, Bt, SB):
        A, SA, Bt, SB = (np.ascontiguousarray(x) for x in (A, SA, Bt, SB))
        for x in (A, SA, Bt, SB):
            if x.dtype != np.uint8 or x.ndim != 2:
                raise TypeError("MX operands and scales are 2-D uint8 arrays")
        M, K = A.shape
        N = Bt.shape[0]
        if Bt.shape[1] != K or SA.shape != (M, K // 32) or SB.shape != (N, K // 32):
            raise ValueError(f"bad MX shapes A{A.shape} SA{SA.shape} Bt{Bt.shape} SB{SB.shape}")
        return A, SA, Bt, SB, M, N, K

    def gemm_mxfp8(self, fmt_a: str, fmt_b: str, A, SA, Bt, SB, nthreads: int = 0) -> np.ndarray:
        """C = (SA-scaled A)·(SB-scaled B) as float64[M, N] (oracle_gemm_mxfp8):
        A [M][K] and Bt [N][K] element codes, SA [M][K/32] and SB [N][K/32]
        scale codes; formats "e4m3" or "e5m2"."""
        A, SA, Bt, SB, M, N, K = self._mx_operands(A, SA, Bt, SB)
        C = np.empty((M, N), dtype=np.float64)
        rc = self.lib.oracle_gemm_mxfp8(FP8[fmt_a], FP8[fmt_b], self._ptr(A), self._ptr(SA), self._ptr(Bt),
                                        self._ptr(SB), M, N, K, self._ptr(C), nthreads)
        if rc != 0:
            raise ValueError("oracle_gemm_mxfp8 rejected its arguments")
        return C

    def gemm_mxfp8_points(self, fmt_a: str, fmt_b: str, A, SA, Bt, SB, rows, cols,
                          nthreads: int = 0) -> np.ndarray:
        """C[rows[p], cols[p]] of gemm_mxfp8, as float64[npts]."""
        A, SA, Bt, SB, M, N, K = self._mx_operands(A, SA, Bt, SB)
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        cols = np.ascontiguousarray(cols, dtype=np.int64)
        if rows.shape != cols.shape or rows.ndim != 1:
            raise ValueError("rows and cols must be equal-length vectors")
        out = np.empty(rows.shape[0], dtype=np.float64)
        rc = self.lib.oracle_gemm_mxfp8_points(FP8[fmt_a], FP8[fmt_b], self._ptr(A), self._ptr(SA),
                                               self._ptr(Bt), self._ptr(SB), M, N, K, self._ptr(rows),
                                               self._ptr(cols), rows.shape[0], self._ptr(out), nthreads)
        if rc != 0:
            raise ValueError("oracle_gemm_mxfp8_points rejected its arguments")
        return out

    @staticmethod
    def _mx4_operands(A, SA, Bt, SB):
        A, SA, Bt, SB = (np.ascontiguousarray(x) for x in (A, SA, Bt, SB))
        for x in (A, SA, Bt, SB):
            if x.dtype != np.uint8 or x.ndim != 2:
                raise TypeError("MXFP4 operands and scales are 2-D uint8 arrays")
        M, K = A.shape[0], 2 * A.shape[1]
        N = Bt.shape[0]
        if Bt.shape[1] != K // 2 or SA.shape != (M, K // 32) or SB.shape != (N, K // 32):
            raise ValueError(f"bad MXFP4 shapes A{A.shape} SA{SA.shape} Bt{Bt.shape} SB{SB.shape}")
        return A, SA, Bt, SB, M, N, K

    def gemm_mxfp4(self, A, SA, Bt, SB, nthreads: int = 0) -> np.ndarray:
        """C for E2M1 operands packed two per byte (low nibble first): A [M][K/2],
        Bt [N][K/2] bytes, SA [M][K/32], SB [N][K/32] scale codes."""
        A, SA, Bt, SB, M, N, K = self._mx4_operands(A, SA, Bt, SB)
        C = np.empty((M, N), dtype=np.float64)
        rc = self.lib.oracle_gemm_mxfp4(self._ptr(A), self._ptr(SA), self._ptr(Bt), self._ptr(SB), M, N, K,
                                        self._ptr(C), nthreads)
        if rc != 0:
            raise ValueError("oracle_gemm_mxfp4 rejected its arguments")
        return C

    def gemm_mxfp4_points(self, A, SA, Bt, SB, rows, cols, nthreads: int = 0) -> np.ndarray:
        A, SA, Bt, SB, M, N, K = self._mx4_operands(A, SA, Bt, SB)
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        cols = np.ascontiguousarray(cols, dtype=np.int64)
        out = np.empty(rows.shape[0], dtype=np.float64)
        rc = self.lib.oracle_gemm_mxfp4_points(self._ptr(A), self._ptr(SA), self._ptr(Bt), self._ptr(SB), M, N, K,
                                               self._ptr(rows), self._ptr(cols), rows.shape[0], self._ptr(out),
                                               nthreads)
        if rc != 0:
            raise ValueError("oracle_gemm_mxfp4_points rejected its arguments")
        return out

    def decode_fp4(self, code: int) -> float:
        """Exact value of one 4-bit E2M1 code."""
        return self.lib.oracle_decode_fp4(code)

    def decode_fp8(self, fmt: str, code: int) -> float:
        """Exact value of one 8-bit element code ("e4m3" or "e5m2")."""
        return self.lib.oracle_decode_fp8(FP8[fmt], code)

    def decode_e8m0(self, code: int) -> float:
        """Exact value of one 8-bit scale code."""
        return self.lib.oracle_decode_e8m0(code)

    def max_threads(self) -> int:
        return self.lib.oracle_max_threads()


_default: Oracle | None = None


def get() -> Oracle:
    """The oracle built from ``oracle.c`` (compiled on first use)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default
