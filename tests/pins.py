"""Checks that tie the oracle to facts outside itself.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises AssertionError when the
oracle disagrees with brute force, a closed form, an invariant, a hand-worked
fixture, a library routine or the FP64 error bound. ``test_oracle_pins.py``
runs them on the real oracle; ``test_oracle_mutants.py`` runs them on copies of
the oracle with planted mistakes and requires that some pin fails for each.
"""
from __future__ import annotations

import math
from fractions import Fraction
from pathlib import Path

import numpy as np

GOLDEN = Path(__file__).resolve().parent / "golden"


# -- fixtures ---------------------------------------------------------------
def _parse_value(tok: str) -> float:
    if tok in ("inf", "-inf"):
        return float(tok)
    neg = tok.startswith("-")
    t = tok[1:] if neg else tok
    if t.startswith("2^"):
        v = 2.0 ** int(t[2:])
    elif "*2^" in t:
        a, e = t.split("*2^")
        v = float(int(a)) * 2.0 ** int(e)
    elif "/" in t:
        v = float(Fraction(t))
    else:
        v = float(t)
    return -v if neg else v


def decode_table():
    rows = []
    for line in (GOLDEN / "decode_16bit.txt").read_text().splitlines():
        if not line.strip() or line.startswith("#"):
            continue
        fmt, bits, val = line.split()[:3]
        rows.append((fmt, int(bits, 16), _parse_value(val)))
    return rows


def small_gemm_cases():
    lines = [l for l in (GOLDEN / "small_gemms.txt").read_text().splitlines()
             if l.strip() and not l.startswith("#")]
    cases, i = [], 0
    while i < len(lines):
        _, name, M, N, K = lines[i].split()
        M, N, K = int(M), int(N), int(K)
        i += 1
        rd = lambda n: [[float(x) for x in lines[i + r].split()] for r in range(n)]
        A = rd(M); i += M
        B = rd(K); i += K
        C = rd(M); i += M
        cases.append((name, np.array(A, np.float32), np.array(B, np.float32),
                      np.array(C, np.float64)))
    return cases


# -- helpers ------------------------------------------------------------------
def _bits(x: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float64).view(np.uint64)


def _bruteforce_int(A, B):
    A = [[int(v) for v in row] for row in A.tolist()]
    B = [[int(v) for v in row] for row in B.tolist()]
    M, K, N = len(A), len(B), len(B[0]) if B else 0
    return [[sum(A[i][k] * B[k][j] for k in range(K)) for j in range(N)]
            for i in range(M)]


# -- pins ---------------------------------------------------------------------
def pin_golden_small(o):
    """Hand-worked products from the definition match exactly."""
    for name, A, B, C in small_gemm_cases():
        got = o.gemm("f32", A, B)
        assert np.array_equal(got, C), (name, got, C)
        assert not np.signbit(got[C == 0]).any(), (name, "negative zero")


def pin_decode_table(o):
    """16-bit decoding matches the hand-worked format table bit for bit."""
    for fmt, bits, val in decode_table():
        got = o.decode(fmt, bits)
        assert got == val and math.copysign(1, got) == math.copysign(1, val), \
            (fmt, hex(bits), got, val)
    for fmt in ("bf16", "f16"):   # NaN patterns
        nan_bits = 0x7FC0 if fmt == "bf16" else 0x7E00
        assert math.isnan(o.decode(fmt, nan_bits))


def pin_decode_library(o):
    """Every finite 16-bit pattern decodes to what numpy's own routines give:
    binary16 through numpy.float16, bfloat16 as the top half of a float32."""
    allbits = np.arange(1 << 16, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        f16 = allbits.astype(np.uint16).view(np.float16).astype(np.float64)
        bf = (allbits << 16).view(np.float32).astype(np.float64)
    step = 97  # a spread subset keeps the ctypes loop short
    for b in range(0, 1 << 16, step):
        for fmt, ref in (("f16", f16[b]), ("bf16", bf[b])):
            got = o.decode(fmt, b)
            if math.isnan(ref):
                assert math.isnan(got), (fmt, hex(b))
            else:
                assert got == ref and math.copysign(1, got) == math.copysign(1, ref), \
                    (fmt, hex(b), got, ref)


def pin_bruteforce_ints(o):
    """Integer operands on tiny shapes equal a pure-Python integer triple sum."""
    rng = np.random.default_rng(101)
    sizes = [1, 2, 3, 4, 5, 7, 13, 17]
    for M in sizes:
        for N in sizes:
            for K in (1, 2, 3, 5, 17):
                A = rng.integers(-9, 10, size=(M, K)).astype(np.float32)
                B = rng.integers(-9, 10, size=(K, N)).astype(np.float32)
                ref = np.array(_bruteforce_int(A, B), dtype=np.float64)
                got = o.gemm("f32", A, B)
                assert np.array_equal(got, ref), (M, N, K)


def pin_bruteforce_16bit(o):
    """16-bit operands: the oracle equals exact rational arithmetic on values
    decoded by numpy (float16, and bfloat16 as the top half of a float32)."""
    rng = np.random.default_rng(102)
    for fmt in ("bf16", "f16"):
        for (M, N, K) in [(3, 5, 7), (4, 4, 16), (1, 9, 33)]:
            x = rng.standard_normal((M * K + K * N,)).astype(np.float32)
            if fmt == "f16":
                bits = x.astype(np.float16).view(np.uint16)
                vals = bits.view(np.float16).astype(np.float64)
            else:
                bits = (x.view(np.uint32) >> 16).astype(np.uint16)  # truncation is fine here
                vals = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            A, B = bits[:M * K].reshape(M, K), bits[M * K:].reshape(K, N)
            Av, Bv = vals[:M * K].reshape(M, K), vals[M * K:].reshape(K, N)
            got = o.gemm(fmt, A, B)
            for i in range(M):
                for j in range(N):
                    exact = sum(Fraction(Av[i, k]) * Fraction(Bv[k, j]) for k in range(K))
                    bound = (K - 1) * 2.0 ** -53 * float(sum(abs(Fraction(Av[i, k]) * Fraction(Bv[k, j])) for k in range(K)))
                    assert abs(Fraction(got[i, j]) - exact) <= Fraction(bound), (fmt, i, j)


def pin_fsum_bound(o):
    """Random FP32: each element is within the recursive-summation bound
    (K-1)*u*sum|a_k b_k| of the exact sum (math.fsum of exact double products)."""
    rng = np.random.default_rng(103)
    for (M, N, K) in [(9, 11, 64), (5, 3, 257), (16, 16, 16)]:
        A = (rng.random((M, K), dtype=np.float32) * 2 - 1).astype(np.float32)
        B = (rng.random((K, N), dtype=np.float32) * 2 - 1).astype(np.float32)
        got = o.gemm("f32", A, B)
        A64, B64 = A.astype(np.float64), B.astype(np.float64)
        for i in range(M):
            for j in range(N):
                prods = A64[i, :] * B64[:, j]
                exact = math.fsum(prods)
                bound = (K - 1) * 2.0 ** -53 * math.fsum(np.abs(prods))
                assert abs(got[i, j] - exact) <= bound, (M, N, K, i, j)


def pin_closed_forms(o):
    """ones*ones = K; A=1, B[k][j]=k gives K(K-1)/2; A[i][k]=i, B[k][j]=j
    gives K*i*j."""
    for (M, N, K) in [(3, 4, 5), (8, 1, 100), (1, 7, 1000), (6, 6, 1)]:
        A = np.ones((M, K), np.float32)
        B = np.ones((K, N), np.float32)
        assert np.array_equal(o.gemm("f32", A, B), np.full((M, N), float(K)))
        Bk = np.repeat(np.arange(K, dtype=np.float32)[:, None], N, axis=1)
        assert np.array_equal(o.gemm("f32", A, Bk), np.full((M, N), K * (K - 1) / 2))
        Ai = np.repeat(np.arange(M, dtype=np.float32)[:, None], K, axis=1)
        Bj = np.repeat(np.arange(N, dtype=np.float32)[None, :], K, axis=0)
        ref = K * np.outer(np.arange(M), np.arange(N)).astype(np.float64)
        assert np.array_equal(o.gemm("f32", Ai, Bj), ref)


def pin_identity_permutation(o):
    """A*I = A and I*B = B bitwise; row/column permutations commute with the
    product bitwise (same dot products in the same order); (A*B)^T = B^T*A^T
    bitwise."""
    rng = np.random.default_rng(104)
    M, N, K = 13, 11, 17
    A = (rng.random((M, K), dtype=np.float32) * 2 - 1).astype(np.float32)
    B = (rng.random((K, N), dtype=np.float32) * 2 - 1).astype(np.float32)
    assert np.array_equal(o.gemm("f32", A, np.eye(K, dtype=np.float32)), A.astype(np.float64))
    assert np.array_equal(o.gemm("f32", np.eye(K, dtype=np.float32), B), B.astype(np.float64))
    C = o.gemm("f32", A, B)
    p = rng.permutation(M)
    q = rng.permutation(N)
    assert np.array_equal(_bits(o.gemm("f32", A[p], B)), _bits(C[p]))
    assert np.array_equal(_bits(o.gemm("f32", A, B[:, q])), _bits(C[:, q]))
    Ct = o.gemm("f32", np.ascontiguousarray(B.T), np.ascontiguousarray(A.T))
    assert np.array_equal(_bits(Ct), _bits(np.ascontiguousarray(C.T)))
    # Permuting the summation index: exact on integers, within the bound otherwise.
    r = rng.permutation(K)
    Ai = rng.integers(-7, 8, (M, K)).astype(np.float32)
    Bi = rng.integers(-7, 8, (K, N)).astype(np.float32)
    assert np.array_equal(o.gemm("f32", Ai[:, r], Bi[r, :]), o.gemm("f32", Ai, Bi))
    Cr = o.gemm("f32", np.ascontiguousarray(A[:, r]), np.ascontiguousarray(B[r, :]))
    assert np.max(np.abs(Cr - C)) <= 2 * K * 2.0 ** -53 * K


def pin_associativity_linearity(o):
    """Small integers keep every intermediate exact: (AB)C = A(BC) and
    A(B1+B2) = AB1 + AB2 exactly."""
    rng = np.random.default_rng(105)
    A = rng.integers(-5, 6, (7, 9)).astype(np.float32)
    B = rng.integers(-5, 6, (9, 6)).astype(np.float32)
    Cm = rng.integers(-5, 6, (6, 8)).astype(np.float32)
    AB = o.gemm("f32", A, B).astype(np.float32)
    BC = o.gemm("f32", B, Cm).astype(np.float32)
    assert np.array_equal(o.gemm("f32", AB, Cm), o.gemm("f32", A, BC))
    B2 = rng.integers(-5, 6, (9, 6)).astype(np.float32)
    lhs = o.gemm("f32", A, (B + B2).astype(np.float32))
    assert np.array_equal(lhs, o.gemm("f32", A, B) + o.gemm("f32", A, B2))


def pin_numpy_matmul(o):
    """numpy's float64 BLAS product agrees within the FP64 error bound."""
    rng = np.random.default_rng(106)
    for (M, N, K) in [(64, 48, 200), (128, 128, 128), (1, 300, 77)]:
        A = (rng.random((M, K), dtype=np.float32) * 2 - 1).astype(np.float32)
        B = (rng.random((K, N), dtype=np.float32) * 2 - 1).astype(np.float32)
        A64, B64 = A.astype(np.float64), B.astype(np.float64)
        ref = A64 @ B64
        bound = 2 * K * 2.0 ** -53 * (np.abs(A64) @ np.abs(B64))
        assert np.all(np.abs(o.gemm("f32", A, B) - ref) <= bound)


def pin_rows_points_consistent(o):
    """Row slabs and single points are the same sums as the full product,
    bit for bit, and independent of the thread count."""
    rng = np.random.default_rng(107)
    M, N, K = 37, 29, 71
    A = (rng.random((M, K), dtype=np.float32) * 2 - 1).astype(np.float32)
    B = (rng.random((K, N), dtype=np.float32) * 2 - 1).astype(np.float32)
    C1 = o.gemm("f32", A, B, nthreads=1)
    C8 = o.gemm("f32", A, B, nthreads=8)
    assert np.array_equal(_bits(C1), _bits(C8))
    assert np.array_equal(_bits(o.gemm_rows("f32", A, B, 5, 20)), _bits(C1[5:25]))
    rows = rng.integers(0, M, 200)
    cols = rng.integers(0, N, 200)
    assert np.array_equal(_bits(o.gemm_points("f32", A, B, rows, cols)), _bits(C1[rows, cols]))


def pin_degenerate(o):
    """K = 0 gives +0 everywhere; M = 0 or N = 0 gives an empty result."""
    z = o.gemm("f32", np.zeros((3, 0), np.float32), np.zeros((0, 4), np.float32))
    assert z.shape == (3, 4) and np.array_equal(_bits(z), np.zeros((3, 4), np.uint64))
    assert o.gemm("f32", np.zeros((0, 5), np.float32), np.ones((5, 4), np.float32)).shape == (0, 4)
    assert o.gemm("f32", np.ones((2, 5), np.float32), np.ones((5, 0), np.float32)).shape == (2, 0)


def _encode_small(fmt, vals):
    """Small integers (exact in every format) as operand arrays of `fmt`."""
    v = np.asarray(vals, dtype=np.float32)
    if fmt == "f32":
        return v
    if fmt == "f16":
        return v.astype(np.float16).view(np.uint16)
    return (v.view(np.uint32) >> 16).astype(np.uint16)


def pin_ex_bruteforce(o):
    """General form alpha·op(A)·op(B) + beta·C0 with transposes and padded row
    strides equals exact rational arithmetic from the definition (small
    integer operands, dyadic alpha and beta: every intermediate is exact).
    C0 holds NaN wherever beta is 0, and A and B hold NaN in the padding and
    everywhere when alpha is 0: neither may reach the result."""
    rng = np.random.default_rng(111)
    alphas = [1.0, 2.0, -0.5, 0.25, 0.0]
    betas = [0.0, 1.0, -2.0, 0.5]
    for case in range(120):
        fmt = ("f32", "bf16", "f16")[case % 3]
        M, N, K = (int(x) for x in rng.integers(1, 6, size=3))
        ta, tb = bool(case & 4), bool(case & 8)
        alpha, beta = alphas[case % 5], betas[(case // 5) % 4]
        ra, ca = (K, M) if ta else (M, K)          # stored A: ra rows of ca values
        rb, cb = (N, K) if tb else (K, N)
        lda, ldb = ca + int(rng.integers(0, 3)), cb + int(rng.integers(0, 3))
        Aval = rng.integers(-4, 5, size=(ra, ca))
        Bval = rng.integers(-4, 5, size=(rb, cb))
        A = np.full((ra, lda), np.nan, np.float32)
        B = np.full((rb, ldb), np.nan, np.float32)
        if alpha != 0.0:
            A[:, :ca] = Aval
            B[:, :cb] = Bval
        C0 = rng.integers(-4, 5, size=(M, N)).astype(np.float32)
        if beta == 0.0:
            C0[:] = np.nan
        Ae, Be = _encode_small(fmt, A), _encode_small(fmt, B)
        got = o.gemm_ex(fmt, M, N, K, Ae, lda, Be, ldb, ta, tb, alpha, beta, C0)
        for i in range(M):
            for j in range(N):
                want = Fraction(0)
                if alpha != 0.0:
                    p = sum(Fraction(int(Aval[k, i] if ta else Aval[i, k])) *
                            Fraction(int(Bval[j, k] if tb else Bval[k, j])) for k in range(K))
                    want += Fraction(alpha) * p
                if beta != 0.0:
                    want += Fraction(beta) * Fraction(float(C0[i, j]))
                assert Fraction(got[i, j]) == want, (case, fmt, ta, tb, alpha, beta, i, j)


def pin_ex_inexact_scales(o):
    """Non-dyadic alpha and beta on random operands: within a few double
    roundings of the exact rational value of the definition."""
    rng = np.random.default_rng(112)
    for (ta, tb) in [(False, False), (True, False), (False, True), (True, True)]:
        M, N, K = 4, 5, 9
        A = rng.uniform(-1, 1, size=(K, M) if ta else (M, K)).astype(np.float32)
        B = rng.uniform(-1, 1, size=(N, K) if tb else (K, N)).astype(np.float32)
        C0 = rng.uniform(-1, 1, size=(M, N)).astype(np.float32)
        alpha, beta = 0.1, -0.3
        got = o.gemm_ex("f32", M, N, K, A, A.shape[1], B, B.shape[1], ta, tb, alpha, beta, C0)
        for i in range(M):
            for j in range(N):
                terms = [Fraction(float(A[k, i] if ta else A[i, k])) * Fraction(float(B[j, k] if tb else B[k, j]))
                         for k in range(K)]
                want = Fraction(alpha) * sum(terms) + Fraction(beta) * Fraction(float(C0[i, j]))
                scale = Fraction(abs(alpha)) * sum(abs(t) for t in terms) + abs(Fraction(beta) * Fraction(float(C0[i, j])))
                assert abs(Fraction(got[i, j]) - want) <= (K + 3) * Fraction(2) ** -52 * scale, (ta, tb, i, j)


# -- block-scaled 8-bit operands (OCP MX formats) ---------------------------
def fp8_decode_table():
    rows = []
    for line in (GOLDEN / "decode_fp8.txt").read_text().splitlines():
        if not line.strip() or line.startswith("#"):
            continue
        fmt, code, val = line.split()[:3]
        rows.append((fmt, int(code, 16), math.nan if val == "nan" else _parse_value(val)))
    return rows


def _same(got: float, want: float) -> bool:
    if math.isnan(want):
        return math.isnan(got)
    return got == want and math.copysign(1, got) == math.copysign(1, want)


def _mx_decode(o, fmt, code):
    if fmt == "e8m0":
        return o.decode_e8m0(code)
    if fmt == "e2m1":
        return o.decode_fp4(code)
    return o.decode_fp8(fmt, code)


def _torch_values(fmt: str, codes: np.ndarray) -> np.ndarray:
    """Values of uint8 codes by torch's own float8 / e8m0 types, as float64."""
    import torch
    t = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2, "e8m0": torch.float8_e8m0fnu}[fmt]
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(t).to(torch.float64).numpy()


def pin_mx_decode_table(o):
    """8-bit element and scale decoding matches the hand-worked table."""
    for fmt, code, val in fp8_decode_table():
        got = _mx_decode(o, fmt, code)
        assert _same(got, val), (fmt, hex(code), got, val)


def pin_mx_decode_library(o):
    """All 256 codes of each 8-bit format decode to what torch's float8_e4m3fn,
    float8_e5m2 and float8_e8m0fnu types give."""
    codes = np.arange(256, dtype=np.uint8)
    for fmt in ("e4m3", "e5m2", "e8m0"):
        ref = _torch_values(fmt, codes)
        for c in range(256):
            got = _mx_decode(o, fmt, c)
            assert _same(got, float(ref[c])), (fmt, hex(c), got, ref[c])


def _mx_random(rng, M, N, K, fa, fb, slo, shi):
    """Random finite codes of every magnitude and random scale codes."""
    def finite(fmt, shape):
        c = rng.integers(0, 256, size=shape, dtype=np.uint8)
        bad = np.isnan(_torch_values(fmt, c)) | np.isinf(_torch_values(fmt, c))
        return np.where(bad, np.uint8(0x38 if fmt == "e4m3" else 0x3C), c).astype(np.uint8)
    A, Bt = finite(fa, (M, K)), finite(fb, (N, K))
    SA = rng.integers(slo, shi + 1, size=(M, K // 32), dtype=np.uint8)
    SB = rng.integers(slo, shi + 1, size=(N, K // 32), dtype=np.uint8)
    return A, SA, Bt, SB


def _mx_exact_terms(fa, fb, A, SA, Bt, SB, i, j):
    """The K products of element (i, j) as exact rationals, from torch-decoded
    codes and scales."""
    K = A.shape[1]
    a = _torch_values(fa, A[i]); b = _torch_values(fb, Bt[j])
    sa = _torch_values("e8m0", SA[i]); sb = _torch_values("e8m0", SB[j])
    return [Fraction(float(a[k])) * Fraction(float(sa[k // 32])) * Fraction(float(b[k])) *
            Fraction(float(sb[k // 32])) for k in range(K)]


def pin_mx_bruteforce(o):
    """Random codes and scales of every magnitude: each element is within the
    recursive-summation bound (K-1)*u*sum|terms| of the exact rational sum of
    the definition (terms from torch-decoded values), and equal to it when
    the terms are all multiples of one power of two that keeps the sums exact."""
    rng = np.random.default_rng(120)
    u = Fraction(1, 2 ** 53)
    for (M, N, K, fa, fb) in [(3, 4, 32, "e4m3", "e4m3"), (2, 5, 64, "e5m2", "e4m3"),
                              (4, 3, 96, "e4m3", "e5m2"), (1, 2, 128, "e5m2", "e5m2")]:
        A, SA, Bt, SB = _mx_random(rng, M, N, K, fa, fb, 100, 154)
        got = o.gemm_mxfp8(fa, fb, A, SA, Bt, SB)
        for i in range(M):
            for j in range(N):
                terms = _mx_exact_terms(fa, fb, A, SA, Bt, SB, i, j)
                want = sum(terms, Fraction(0))
                bound = (K - 1) * u * sum((abs(t) for t in terms), Fraction(0))
                assert abs(Fraction(got[i, j]) - want) <= bound, (fa, fb, M, N, K, i, j)
    import sam_inputs as si
    for fa, fb in [("e4m3", "e4m3"), ("e5m2", "e4m3"), ("e4m3", "e5m2")]:
        w = si.Workload("pin", "mxfp8", 3, 5, 160, "mx_dyadic", 121, fmt_a=fa, fmt_b=fb)
        A, SA, Bt, SB = si.make_mx_operands(w)
        got = o.gemm_mxfp8(fa, fb, A, SA, Bt, SB)
        for i in range(3):
            for j in range(5):
                want = sum(_mx_exact_terms(fa, fb, A, SA, Bt, SB, i, j), Fraction(0))
                assert Fraction(got[i, j]) == want, (fa, fb, i, j)


def pin_mx_unit_scales(o):
    """With every scale code 127 (scale 1) the block-scaled product is the
    plain product of the decoded values: bit for bit the FP32 oracle run on
    torch-decoded A and on B = Bt transposed (same values, same ascending-k
    double sums)."""
    rng = np.random.default_rng(122)
    for (M, N, K, fa, fb) in [(5, 7, 64, "e4m3", "e4m3"), (6, 3, 96, "e5m2", "e4m3"), (4, 4, 32, "e5m2", "e5m2")]:
        A, SA, Bt, SB = _mx_random(rng, M, N, K, fa, fb, 127, 127)
        got = o.gemm_mxfp8(fa, fb, A, SA, Bt, SB)
        Ad = _torch_values(fa, A).astype(np.float32)
        Bd = np.ascontiguousarray(_torch_values(fb, Bt).astype(np.float32).T)
        ref = o.gemm("f32", Ad, Bd)
        assert np.array_equal(_bits(got), _bits(ref)), (M, N, K, fa, fb)


def pin_mx_scale_closed_form(o):
    """All elements 1 (e4m3 0x38) with SA[i][b] = 127 + b and SB[j][b] = 127 + j
    gives C[i][j] = 32 * 2^j * (2^(K/32) - 1): each block scale reaches its
    own block of its own row / column only."""
    M, N, K = 3, 5, 128
    A = np.full((M, K), 0x38, np.uint8); Bt = np.full((N, K), 0x38, np.uint8)
    SA = np.tile(np.arange(127, 127 + K // 32, dtype=np.uint8), (M, 1))
    SB = np.repeat(np.arange(127, 127 + N, dtype=np.uint8)[:, None], K // 32, axis=1)
    got = o.gemm_mxfp8("e4m3", "e4m3", A, SA, Bt, SB)
    for i in range(M):
        for j in range(N):
            assert got[i, j] == 32.0 * 2.0 ** j * (2.0 ** (K // 32) - 1), (i, j, got[i, j])


def pin_mx_points_and_degenerate(o):
    """Single points are the full product's sums bit for bit; K = 0 gives +0;
    K not a multiple of 32 is rejected."""
    rng = np.random.default_rng(123)
    A, SA, Bt, SB = _mx_random(rng, 6, 9, 64, "e4m3", "e5m2", 110, 140)
    full = o.gemm_mxfp8("e4m3", "e5m2", A, SA, Bt, SB)
    rows = np.array([0, 5, 3, 5, 0]); cols = np.array([0, 8, 4, 0, 8])
    pts = o.gemm_mxfp8_points("e4m3", "e5m2", A, SA, Bt, SB, rows, cols)
    assert np.array_equal(_bits(pts), _bits(full[rows, cols]))
    z = o.gemm_mxfp8("e4m3", "e4m3", np.zeros((2, 0), np.uint8), np.zeros((2, 0), np.uint8),
                     np.zeros((3, 0), np.uint8), np.zeros((3, 0), np.uint8))
    assert z.shape == (2, 3) and (z == 0).all() and not np.signbit(z).any()
    try:
        o.gemm_mxfp8("e4m3", "e4m3", np.zeros((2, 48), np.uint8), np.zeros((2, 1), np.uint8),
                     np.zeros((3, 48), np.uint8), np.zeros((3, 1), np.uint8))
    except ValueError:
        pass
    else:
        raise AssertionError("K = 48 accepted")


# -- block-scaled 4-bit operands (MXFP4) ---------------------------------------
def _e2m1_values(codes: np.ndarray) -> np.ndarray:
    """E2M1 values through torch's E4M3 decoder: a normal E2M1 code (exponent
    field e >= 1, bias 1, fraction f) is the E4M3 code with exponent field
    e + 6 (bias 7) and fraction 4 f; the subnormal 0.5 is E4M3 0x30."""
    codes = np.asarray(codes, dtype=np.uint8)
    sign, e, f = (codes >> 3) & 1, (codes >> 1) & 3, codes & 1
    mag = np.where(e == 0, np.where(f == 1, 0x30, 0x00), ((e + 6) << 3) | (f << 2)).astype(np.uint8)
    return _torch_values("e4m3", (sign.astype(np.uint8) << 7) | mag)


def _unpack4(b: np.ndarray) -> np.ndarray:
    """Rows of packed bytes -> rows of 4-bit codes, element 2i in the low nibble."""
    b = np.asarray(b, dtype=np.uint8)
    out = np.empty((b.shape[0], 2 * b.shape[1]), dtype=np.uint8)
    out[:, 0::2] = b & 0xF
    out[:, 1::2] = b >> 4
    return out


def _mx4_random(rng, M, N, K, slo, shi):
    A = rng.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    Bt = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    SA = rng.integers(slo, shi + 1, size=(M, K // 32), dtype=np.uint8)
    SB = rng.integers(slo, shi + 1, size=(N, K // 32), dtype=np.uint8)
    return A, SA, Bt, SB


def pin_mx4_decode_via_e4m3(o):
    """Every E2M1 code decodes to the value torch's E4M3 type gives for the
    same number written in E4M3."""
    codes = np.arange(16, dtype=np.uint8)
    ref = _e2m1_values(codes)
    for c in range(16):
        assert _same(o.decode_fp4(c), float(ref[c])), (hex(c), o.decode_fp4(c), ref[c])


def pin_mx4_bruteforce(o):
    """Random packed codes and scales: within (K-1)*u*sum|terms| of the exact
    rational sum (values unpacked and decoded independently), and exactly
    equal with scales near 1."""
    rng = np.random.default_rng(130)
    u = Fraction(1, 2 ** 53)
    for (M, N, K, slo, shi) in [(3, 4, 32, 100, 154), (2, 5, 96, 100, 154), (4, 3, 64, 126, 128)]:
        A, SA, Bt, SB = _mx4_random(rng, M, N, K, slo, shi)
        got = o.gemm_mxfp4(A, SA, Bt, SB)
        a, b = _e2m1_values(_unpack4(A)), _e2m1_values(_unpack4(Bt))
        sa, sb = _torch_values("e8m0", SA), _torch_values("e8m0", SB)
        for i in range(M):
            for j in range(N):
                terms = [Fraction(float(a[i, k])) * Fraction(float(sa[i, k // 32])) * Fraction(float(b[j, k])) *
                         Fraction(float(sb[j, k // 32])) for k in range(K)]
                want = sum(terms, Fraction(0))
                if shi - slo <= 2:
                    assert Fraction(got[i, j]) == want, (M, N, K, i, j)
                else:
                    bound = (K - 1) * u * sum((abs(t) for t in terms), Fraction(0))
                    assert abs(Fraction(got[i, j]) - want) <= bound, (M, N, K, i, j)


def pin_mx4_unit_scales(o):
    """Scales of 1 reduce the MXFP4 product bit for bit to the FP32 oracle on
    the unpacked, independently decoded values (B = Bt transposed)."""
    rng = np.random.default_rng(131)
    for (M, N, K) in [(5, 7, 64), (3, 2, 160)]:
        A, SA, Bt, SB = _mx4_random(rng, M, N, K, 127, 127)
        got = o.gemm_mxfp4(A, SA, Bt, SB)
        Ad = _e2m1_values(_unpack4(A)).astype(np.float32)
        Bd = np.ascontiguousarray(_e2m1_values(_unpack4(Bt)).astype(np.float32).T)
        assert np.array_equal(_bits(got), _bits(o.gemm("f32", Ad, Bd))), (M, N, K)


def pin_mx4_packing_closed_form(o):
    """Byte 0 of A's row = 0x21 puts 0.5 at k = 0 and 1.0 at k = 1; a B column
    that is one-hot at k = 0 (byte 0x02) or k = 1 (byte 0x20) picks each out;
    a scale of 2 on block 1 reaches only k >= 32 (A value 3 at k = 33)."""
    K = 64
    A = np.zeros((1, K // 2), np.uint8); A[0, 0] = 0x21; A[0, 16] = 0x50   # k = 33: code 5 = 3
    Bt = np.zeros((3, K // 2), np.uint8); Bt[0, 0] = 0x02; Bt[1, 0] = 0x20; Bt[2, 16] = 0x20
    SA = np.array([[127, 128]], np.uint8); SB = np.full((3, 2), 127, np.uint8)
    got = o.gemm_mxfp4(A, SA, Bt, SB)
    assert got.tolist() == [[0.5, 1.0, 6.0]], got


def pin_mx4_points(o):
    """Single MXFP4 points equal the full product's sums bit for bit, at
    corners, interior positions and with an odd number of 32-value blocks;
    with scales near 1 they also equal the exact rational sum of the
    independently unpacked and decoded values. M != N, and rows and cols are
    drawn apart, so a row/column mix-up or a nibble picked from the wrong half
    of a byte on one operand changes the result."""
    rng = np.random.default_rng(132)
    for (M, N, K, slo, shi) in [(7, 5, 96, 100, 154), (6, 9, 160, 126, 128), (5, 4, 32, 120, 134)]:
        A, SA, Bt, SB = _mx4_random(rng, M, N, K, slo, shi)
        full = o.gemm_mxfp4(A, SA, Bt, SB)
        lim = min(M, N)
        rows = np.array([0, lim - 1, 1, lim - 1, 2, 0, lim - 2], dtype=np.int64)
        cols = np.array([0, lim - 1, 3 % lim, 0, 1, lim - 1, 2], dtype=np.int64)
        pts = o.gemm_mxfp4_points(A, SA, Bt, SB, rows, cols)
        assert np.array_equal(_bits(pts), _bits(full[rows, cols])), (M, N, K)
        if shi - slo <= 2:
            a, b = _e2m1_values(_unpack4(A)), _e2m1_values(_unpack4(Bt))
            sa, sb = _torch_values("e8m0", SA), _torch_values("e8m0", SB)
            for p, (i, j) in enumerate(zip(rows, cols)):
                want = sum((Fraction(float(a[i, k])) * Fraction(float(sa[i, k // 32])) *
                            Fraction(float(b[j, k])) * Fraction(float(sb[j, k // 32])) for k in range(K)),
                           Fraction(0))
                assert Fraction(pts[p]) == want, (M, N, K, i, j)
    z = o.gemm_mxfp4_points(np.zeros((2, 0), np.uint8), np.zeros((2, 0), np.uint8), np.zeros((3, 0), np.uint8),
                            np.zeros((3, 0), np.uint8), [1], [2])
    assert z.tolist() == [0.0] and not np.signbit(z).any()


ALL_PINS = [pin_golden_small, pin_decode_table, pin_decode_library,
            pin_bruteforce_ints, pin_bruteforce_16bit, pin_fsum_bound,
            pin_closed_forms, pin_identity_permutation,
            pin_associativity_linearity, pin_numpy_matmul,
            pin_rows_points_consistent, pin_degenerate, pin_ex_bruteforce, pin_ex_inexact_scales,
            pin_mx_decode_table, pin_mx_decode_library, pin_mx_bruteforce,
            pin_mx_unit_scales, pin_mx_scale_closed_form, pin_mx_points_and_degenerate,
            pin_mx4_decode_via_e4m3, pin_mx4_bruteforce, pin_mx4_unit_scales, pin_mx4_packing_closed_form,
            pin_mx4_points]
