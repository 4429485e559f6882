/*
 * oracle.c -- reference GEMM in double precision.
 *
 * TEST INFRASTRUCTURE ONLY. The test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load this library; the product path (the
 * HIP library and its Python binding) never does, and this file shares no
 * code, header or table with it.
 *
 * What it computes. C = A*B for compact row-major A[M,K] and B[K,N], with no
 * scale on the product and nothing taken from the old contents of C (page
 * "Scale coverage exposes a remaining GEMM gap", section "Measurement contract
 * and evidence": the GEMM there has alpha one, beta zero, no transpose and no
 * prepacked operand). Operands are FP32, or bfloat16 / IEEE binary16 bit
 * patterns (the 16-bit operand port of page "Measured data point on fixed-tile
 * vs shape-adaptive GEMM", section "One more result that surprised us").
 *
 * How. Each operand value is decoded exactly to double. Each product a*b is
 * then exact in double (two significands of at most 24 bits make at most 48
 * bits), and the products of one output element are added in double in
 * ascending k, starting from +0.0. The loop order is i, then k, then j with
 * a double row accumulator: for every element the additions still happen in
 * ascending k, so the bits equal those of the i-j-k dot-product order. No
 * blocking and no reassociation; build with -O2 -fno-fast-math
 * -ffp-contract=off.
 *
 * The double result is handed back as is; rounding it (for a bit-exact
 * comparison) is the caller's business.
 *
 * A second family, at the end of the file, does the same for block-scaled
 * 8-bit operands (OCP MX formats): each value is its element times its
 * block's power-of-two scale, then the same exact products and ascending-k
 * double sum.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_F16 = 2 };

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits. It is
 * the upper half of an IEEE binary32, so the value follows binary32's rules:
 * exponent field 0 is zero/subnormal with scale 2^-126, field 255 is inf/NaN. */
double oracle_decode_bf16(uint16_t bits)
{
    int sign = bits >> 15;
    int e = (bits >> 7) & 0xFF;
    int f = bits & 0x7F;
    double v;
    if (e == 0xFF)
        v = f ? NAN : INFINITY;
    else if (e == 0)
        v = ldexp((double)f, -126 - 7);          /* 0.f * 2^-126 */
    else
        v = ldexp((double)(0x80 | f), e - 127 - 7); /* 1.f * 2^(e-127) */
    return sign ? -v : v;
}

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits;
 * field 0 is zero/subnormal with scale 2^-14, field 31 is inf/NaN. */
double oracle_decode_f16(uint16_t bits)
{
    int sign = bits >> 15;
    int e = (bits >> 10) & 0x1F;
    int f = bits & 0x3FF;
    double v;
    if (e == 0x1F)
        v = f ? NAN : INFINITY;
    else if (e == 0)
        v = ldexp((double)f, -14 - 10);
    else
        v = ldexp((double)(0x400 | f), e - 15 - 10);
    return sign ? -v : v;
}

static double load_val(int dtype, const void* p, int64_t idx)
{
    switch (dtype) {
    case ORACLE_F32:  return (double)((const float*)p)[idx];
    case ORACLE_BF16: return oracle_decode_bf16(((const uint16_t*)p)[idx]);
    default:          return oracle_decode_f16(((const uint16_t*)p)[idx]);
    }
}

static int check_args(int dtype, const void* A, const void* B, int64_t M,
                      int64_t N, int64_t K)
{
    if (dtype < ORACLE_F32 || dtype > ORACLE_F16) return -1;
    if (M < 0 || N < 0 || K < 0) return -1;
    if (K > 0 && ((M > 0 && !A) || (N > 0 && !B))) return -1;
    return 0;
}

static void set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

/* Number of threads an OpenMP region would use now (1 without OpenMP). */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Rows [row0, row0+nrows) of C into Cslab[nrows][N].  Returns 0 or -1. */
int oracle_gemm_rows(int dtype, const void* A, const void* B, int64_t M,
                     int64_t N, int64_t K, int64_t row0, int64_t nrows,
                     double* Cslab, int nthreads)
{
    if (check_args(dtype, A, B, M, N, K)) return -1;
    if (row0 < 0 || nrows < 0 || row0 + nrows > M) return -1;
    if (nrows == 0 || N == 0) return 0;
    if (!Cslab) return -1;

    /* B decoded once into double; the conversion is exact, and it is the
     * same value load_val would give inside the loop. */
    double* Bd = NULL;
    if (K > 0) {
        Bd = (double*)malloc((size_t)K * (size_t)N * sizeof(double));
        if (!Bd) return -1;
        set_threads(nthreads);
#pragma omp parallel for schedule(static)
        for (int64_t k = 0; k < K; ++k)
            for (int64_t j = 0; j < N; ++j)
                Bd[k * N + j] = load_val(dtype, B, k * N + j);
    }

    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t i = row0 + r;
        double* acc = Cslab + r * N;
        for (int64_t j = 0; j < N; ++j) acc[j] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double a = load_val(dtype, A, i * K + k);
            const double* brow = Bd + k * N;
            for (int64_t j = 0; j < N; ++j) acc[j] = acc[j] + a * brow[j];
        }
    }
    free(Bd);
    return 0;
}

/* The whole of C into C[M][N]. */
int oracle_gemm(int dtype, const void* A, const void* B, int64_t M, int64_t N,
                int64_t K, double* C, int nthreads)
{
    return oracle_gemm_rows(dtype, A, B, M, N, K, 0, M, C, nthreads);
}

/* Single elements: out[p] = C[rows[p]][cols[p]], each one its own
 * ascending-k sum. */
int oracle_gemm_points(int dtype, const void* A, const void* B, int64_t M,
                       int64_t N, int64_t K, const int64_t* rows,
                       const int64_t* cols, int64_t npts, double* out,
                       int nthreads)
{
    if (check_args(dtype, A, B, M, N, K)) return -1;
    if (npts < 0 || (npts > 0 && (!rows || !cols || !out))) return -1;
    for (int64_t p = 0; p < npts; ++p)
        if (rows[p] < 0 || rows[p] >= M || cols[p] < 0 || cols[p] >= N)
            return -1;
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t p = 0; p < npts; ++p) {
        const int64_t i = rows[p], j = cols[p];
        double s = 0.0;
        for (int64_t k = 0; k < K; ++k)
            s = s + load_val(dtype, A, i * K + k) * load_val(dtype, B, k * N + j);
        out[p] = s;
    }
    return 0;
}

/* The general form out = alpha * op(A) * op(B) + beta * C0, the usual BLAS
 * definition (the pages fix alpha = 1, beta = 0 and no transposes; this
 * wider form is the reading used for the general entry point). Storage is
 * row-major with explicit row strides:
 *   op(A) = A (M rows of K, stride lda) or A^T (A holds K rows of M, stride lda);
 *   op(B) = B (K rows of N, stride ldb) or B^T (B holds N rows of K, stride ldb).
 * C0 is compact [M][N] and is read only when beta != 0; the product is not
 * evaluated when alpha == 0 or K == 0 (so nothing in A or B can reach out).
 * Per element: P = sum over ascending k of exact products, in double from
 * +0.0; out = alpha * P + beta * C0 in double, returned unrounded. */
int oracle_gemm_ex(int dtype, int trans_a, int trans_b, int64_t M, int64_t N,
                   int64_t K, double alpha, const void* A, int64_t lda,
                   const void* B, int64_t ldb, double beta, const float* C0,
                   double* out, int nthreads)
{
    if (dtype < ORACLE_F32 || dtype > ORACLE_F16) return -1;
    if (M < 0 || N < 0 || K < 0 || (trans_a != 0 && trans_a != 1) ||
        (trans_b != 0 && trans_b != 1)) return -1;
    if (lda < (trans_a ? M : K) || ldb < (trans_b ? K : N)) return -1;
    const int product = alpha != 0.0 && K > 0;
    if (product && M > 0 && N > 0 && (!A || !B)) return -1;
    if (beta != 0.0 && M > 0 && N > 0 && !C0) return -1;
    if (M > 0 && N > 0 && !out) return -1;
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t j = 0; j < N; ++j) {
            double p = 0.0;
            if (product) {
                for (int64_t k = 0; k < K; ++k) {
                    const double a = load_val(dtype, A, trans_a ? k * lda + i : i * lda + k);
                    const double b = load_val(dtype, B, trans_b ? j * ldb + k : k * ldb + j);
                    p = p + a * b;
                }
            }
            double v = product ? alpha * p : 0.0;
            if (beta != 0.0) v = v + beta * (double)C0[i * N + j];
            out[i * N + j] = v;
        }
    }
    return 0;
}

/* ---- Block-scaled 8-bit operands (OCP Microscaling, MXFP8) ---------------
 *
 * The FP4 GEMM of page "fix(fp4_gemm autotune) SM107 kernel family excluded
 * from autotune candidates and heuristics update - #4856" runs on
 * block-scaled operands but the page does not define a format. This oracle
 * takes the formats of the OCP Microscaling (MX) specification v1.0 that
 * gfx950's matrix cores implement, with 8-bit elements:
 *
 *   E4M3: 1 sign, 4 exponent bits (bias 7), 3 fraction bits. Exponent field
 *         0 is zero/subnormal (0.f * 2^-6); S.1111.111 is NaN; there is no
 *         infinity, so S.1111.110 is the largest finite value, 448.
 *   E5M2: 1 sign, 5 exponent bits (bias 15), 2 fraction bits, IEEE rules:
 *         field 0 is zero/subnormal (0.f * 2^-14), field 31 is Inf (f = 0)
 *         or NaN.
 *   E8M0 scale: 2^(code - 127); code 255 is NaN.
 *
 * A block is 32 consecutive values of K. Every row i of A carries one scale
 * per block, SA[i][b], and every column j of B carries one, SB[j][b], and the
 * operand value at k is the element times the scale of its block:
 *   a(i,k) = 2^(SA[i][k/32]-127) * A[i][k],  b(k,j) = 2^(SB[j][k/32]-127) * B[k][j]
 *   C[i][j] = sum over ascending k of a(i,k) * b(k,j).
 * Storage (both operands K-contiguous, the form block scaling along K is
 * given in): A is M rows of K codes; B is given as Bt, N rows of K codes
 * (Bt[j][k] = B[k][j]); SA is M rows and SB N rows of K/32 scale codes.
 * K must be a multiple of 32.
 *
 * How: the scaled values are exact in double (an element has at most 4
 * significant bits and the scale is a power of two within double's range),
 * so each product is exact; products are added in double in ascending k
 * from +0.0, as in the plain GEMM above. */
enum { ORACLE_E4M3 = 0, ORACLE_E5M2 = 1 };

double oracle_decode_fp8(int fmt, uint8_t code)
{
    const int sign = code >> 7;
    double v;
    if (fmt == ORACLE_E4M3) {
        const int e = (code >> 3) & 0xF, f = code & 0x7;
        if (e == 0xF && f == 0x7)
            v = NAN;
        else if (e == 0)
            v = ldexp((double)f, -6 - 3);
        else
            v = ldexp((double)(0x8 | f), e - 7 - 3);
    } else {
        const int e = (code >> 2) & 0x1F, f = code & 0x3;
        if (e == 0x1F)
            v = f ? NAN : INFINITY;
        else if (e == 0)
            v = ldexp((double)f, -14 - 2);
        else
            v = ldexp((double)(0x4 | f), e - 15 - 2);
    }
    return sign ? -v : v;
}

double oracle_decode_e8m0(uint8_t code)
{
    return code == 0xFF ? NAN : ldexp(1.0, (int)code - 127);
}

static double mx_val(int fmt, const uint8_t* codes, const uint8_t* scales, int64_t row, int64_t K, int64_t k)
{
    return oracle_decode_fp8(fmt, codes[row * K + k]) * oracle_decode_e8m0(scales[row * (K / 32) + k / 32]);
}

/* out[i][j] (M x N doubles) for every i, j. Returns 0 or -1. */
int oracle_gemm_mxfp8(int fmt_a, int fmt_b, const uint8_t* A, const uint8_t* SA, const uint8_t* Bt,
                      const uint8_t* SB, int64_t M, int64_t N, int64_t K, double* out, int nthreads)
{
    if ((fmt_a != ORACLE_E4M3 && fmt_a != ORACLE_E5M2) || (fmt_b != ORACLE_E4M3 && fmt_b != ORACLE_E5M2))
        return -1;
    if (M < 0 || N < 0 || K < 0 || K % 32 != 0) return -1;
    if (M == 0 || N == 0) return 0;
    if (!out || (K > 0 && (!A || !SA || !Bt || !SB))) return -1;
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t j = 0; j < N; ++j) {
            double s = 0.0;
            for (int64_t k = 0; k < K; ++k)
                s = s + mx_val(fmt_a, A, SA, i, K, k) * mx_val(fmt_b, Bt, SB, j, K, k);
            out[i * N + j] = s;
        }
    }
    return 0;
}

/* Single elements out[p] = C[rows[p]][cols[p]] of the product above. */
int oracle_gemm_mxfp8_points(int fmt_a, int fmt_b, const uint8_t* A, const uint8_t* SA, const uint8_t* Bt,
                             const uint8_t* SB, int64_t M, int64_t N, int64_t K, const int64_t* rows,
                             const int64_t* cols, int64_t npts, double* out, int nthreads)
{
    if ((fmt_a != ORACLE_E4M3 && fmt_a != ORACLE_E5M2) || (fmt_b != ORACLE_E4M3 && fmt_b != ORACLE_E5M2))
        return -1;
    if (M < 0 || N < 0 || K < 0 || K % 32 != 0 || npts < 0) return -1;
    if (npts > 0 && (!rows || !cols || !out || (K > 0 && (!A || !SA || !Bt || !SB)))) return -1;
    for (int64_t p = 0; p < npts; ++p)
        if (rows[p] < 0 || rows[p] >= M || cols[p] < 0 || cols[p] >= N) return -1;
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t p = 0; p < npts; ++p) {
        double s = 0.0;
        for (int64_t k = 0; k < K; ++k)
            s = s + mx_val(fmt_a, A, SA, rows[p], K, k) * mx_val(fmt_b, Bt, SB, cols[p], K, k);
        out[p] = s;
    }
    return 0;
}

/* ---- Block-scaled 4-bit operands (OCP MX, MXFP4) ---------------------------
 *
 * E2M1 elements: 1 sign, 2 exponent bits (bias 1), 1 fraction bit; exponent
 * field 0 is zero/subnormal (0.f * 2^0); no infinity or NaN, so the largest
 * magnitude is 6. Two elements per byte: element k of a row is the low
 * nibble of byte k/2 when k is even and the high nibble when k is odd (the
 * reading taken for the packing, which the pages do not give). Scales and
 * blocks as for MXFP8: E8M0 per 32 values of K, per row of A and per column
 * of B. Storage: A is M rows of K/2 bytes, B is given as Bt, N rows of K/2
 * bytes; SA and SB as above. Every value is exact in double and the products
 * are summed in ascending k from +0.0. */
double oracle_decode_fp4(uint8_t code)
{
    const int sign = (code >> 3) & 1, e = (code >> 1) & 3, f = code & 1;
    const double v = e == 0 ? ldexp((double)f, -1) : ldexp((double)(0x2 | f), e - 1 - 1);
    return sign ? -v : v;
}

static double mx4_val(const uint8_t* codes, const uint8_t* scales, int64_t row, int64_t K, int64_t k)
{
    const uint8_t byte = codes[row * (K / 2) + k / 2];
    const uint8_t code = (k & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 0xF);
    return oracle_decode_fp4(code) * oracle_decode_e8m0(scales[row * (K / 32) + k / 32]);
}

int oracle_gemm_mxfp4(const uint8_t* A, const uint8_t* SA, const uint8_t* Bt, const uint8_t* SB, int64_t M,
                      int64_t N, int64_t K, double* out, int nthreads)
{
    if (M < 0 || N < 0 || K < 0 || K % 32 != 0) return -1;
    if (M == 0 || N == 0) return 0;
    if (!out || (K > 0 && (!A || !SA || !Bt || !SB))) return -1;
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t j = 0; j < N; ++j) {
            double s = 0.0;
            for (int64_t k = 0; k < K; ++k)
                s = s + mx4_val(A, SA, i, K, k) * mx4_val(Bt, SB, j, K, k);
            out[i * N + j] = s;
        }
    }
    return 0;
}

int oracle_gemm_mxfp4_points(const uint8_t* A, const uint8_t* SA, const uint8_t* Bt, const uint8_t* SB, int64_t M,
                             int64_t N, int64_t K, const int64_t* rows, const int64_t* cols, int64_t npts,
                             double* out, int nthreads)
{
    if (M < 0 || N < 0 || K < 0 || K % 32 != 0 || npts < 0) return -1;
    if (npts > 0 && (!rows || !cols || !out || (K > 0 && (!A || !SA || !Bt || !SB)))) return -1;
    for (int64_t p = 0; p < npts; ++p)
        if (rows[p] < 0 || rows[p] >= M || cols[p] < 0 || cols[p] >= N) return -1;
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t p = 0; p < npts; ++p) {
        double s = 0.0;
        for (int64_t k = 0; k < K; ++k)
            s = s + mx4_val(A, SA, rows[p], K, k) * mx4_val(Bt, SB, cols[p], K, k);
        out[p] = s;
    }
    return 0;
}
