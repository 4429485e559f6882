/*
 * sam.h -- C ABI of the shape-adaptive GEMM library for MI355X (gfx950).
 *
 * Operation (page "Scale coverage exposes a remaining GEMM gap", section
 * "Measurement contract and evidence"): C = A*B with compact row-major
 * A[M][K], B[K][N], C[M][N] (leading dimensions K, N, N), alpha one, beta
 * zero: C is write-only and its old contents are never read. Operands are
 * FP32, or bfloat16 / IEEE binary16 passed as raw 16-bit patterns; products
 * are accumulated in FP32 and C is always FP32 (the 16-bit operand runs of
 * page "Measured data point on fixed-tile vs shape-adaptive GEMM", section
 * "One more result that surprised us", there on other hardware).
 *
 * Shape adaptivity (same page, sections "The wall, and why we think it's
 * structural" and "The actual question"; page "Post-mortem: a GPU stack
 * without nvcc, cuBLAS, or LLVM", section 2.1): a dispatcher picks one of
 * several macro-tile / schedule variants from (M, N, K, dtype) alone, through
 * a frozen, source-controlled table. No timing happens at run time.
 *
 * Determinism (page "Measured data point ...", question 2; page
 * "Post-mortem ...", section 7): no atomics anywhere; the K sum of every
 * output runs in a fixed order per variant, and split-K partials are added
 * in split order 0, 1, ..., S-1 by a separate kernel. The same (M, N, K,
 * dtype) on the same library build gives the same plan and the same bits.
 *
 * Conventions shared by every entry point:
 *   - All pointers to operands, C and workspace are DEVICE pointers of the
 *     current HIP device; `stream` is a hipStream_t (NULL = default stream).
 *   - Calls are asynchronous: work is enqueued on `stream` and the call
 *     returns. The library never synchronises the host and keeps no pointer
 *     after returning; buffers must live until the stream work completes.
 *   - The caller owns and allocates everything (A, B, C, workspace). The
 *     library never allocates device memory on these paths.
 *   - Errors found before enqueueing (arguments, workspace size, device,
 *     launch) are returned as a negative sam_status; detail text is in
 *     sam_last_error() (per thread). Faults inside kernels surface at the
 *     caller's next synchronisation. No C++ exception crosses this ABI.
 *   - Sizes: M, N, K >= 0. M == 0 or N == 0 is a no-op returning SAM_OK.
 *     K == 0 writes +0.0f to every element of C. M*N, M*K and K*N must fit
 *     in int64 and every index below 2^31 elements per operand.
 *   - A, B, C, workspace base addresses must be 16-byte aligned, else
 *     SAM_ERR_MISALIGNED. Odd K or N are fine: such shapes take load paths
 *     that never form an unaligned vector address.
 *   - C must not overlap A, B or the workspace (SAM_ERR_INVALID_ARG).
 *   - Thread-safe: the variant table is immutable and module state is
 *     initialised once.
 */
#ifndef SAM_H
#define SAM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* SAM_MXFP8 / SAM_MXFP4 name block-scaled 8-bit / 4-bit operands
 * (sam_gemm_mxfp8, sam_gemm_mxfp4) in plan queries; the other entry points
 * take the first three. */
typedef enum { SAM_F32 = 0, SAM_BF16 = 1, SAM_F16 = 2, SAM_MXFP8 = 3, SAM_MXFP4 = 4 } sam_dtype;

typedef enum {
    SAM_OK = 0,
    SAM_ERR_INVALID_ARG = -1,        /* bad size, null or overlapping pointer */
    SAM_ERR_MISALIGNED = -2,         /* a base pointer not 16-byte aligned   */
    SAM_ERR_WORKSPACE = -3,          /* workspace smaller than the plan needs */
    SAM_ERR_UNSUPPORTED = -4,        /* forced variant cannot take this case  */
    SAM_ERR_UNSUPPORTED_DEVICE = -5, /* no gfx950 device / kernels not loadable */
    SAM_ERR_LAUNCH = -6,             /* the HIP runtime refused a launch      */
    SAM_ERR_INTERNAL = -7
} sam_status;

/* One dispatch decision. Plain old data; struct_size is set by the library
 * to sizeof(sam_plan) for ABI versioning. */
typedef struct {
    uint32_t struct_size;
    int32_t variant_id;        /* stable index into the variant table        */
    char name[64];             /* e.g. "f32_t256x256_w2x2_b32" + "_s4" ...    */
    int32_t dtype;             /* sam_dtype                                   */
    int32_t tile_m, tile_n, tile_k; /* macro tile; tile_k = K per LDS stage  */
    int32_t waves_m, waves_n;  /* wave grid inside a workgroup               */
    int32_t mfma_m;            /* MFMA block edge: 32 or 16                   */
    int32_t split_k;           /* 1 = single pass; >1 = partials + ordered sum;
                                  -1 = stream-K: grid_wgs persistent workgroups
                                  share the tiles' K iterations evenly, shared
                                  tiles are summed in a fixed order after */
    int32_t group_m;           /* grouped-raster height in tiles             */
    int32_t xcd_remap;         /* 1 = workgroup ids remapped per XCD          */
    int32_t a_vector, b_vector;/* 1 = 16-byte loads of A / B rows            */
    int64_t grid_wgs;          /* workgroups of the main kernel              */
    uint64_t workspace_bytes;  /* device workspace the call needs (0 if none) */
    double est_us;             /* the dispatcher's cost estimate, microseconds */
    int32_t raster_n;          /* 0: groups of group_m tile rows sweep the tile
                                  columns (M-major); 1: groups of group_m tile
                                  columns sweep the rows (N-major)           */
    int32_t operand_swap;      /* 1: the MFMA takes B's fragment as its first
                                  operand, so accumulators hold the transposed
                                  block (stored 16 bytes per lane)           */
    int64_t sk_dp_tiles;       /* stream-K: leading tiles run one per
                                  workgroup before the shared ones (16-bit)  */
    int32_t tuned;             /* 0 cost model, 1 frozen table (this shape),
                                  2 frozen table (a measured shape in the same
                                  half-octave bucket)                        */
} sam_plan;

/* The plan sam_gemm_<dtype> would run for this shape. Host only: touches no
 * device state and needs no GPU. Returns SAM_ERR_INVALID_ARG for negative
 * sizes or a null `out`. */
sam_status sam_gemm_plan(int64_t M, int64_t N, int64_t K, sam_dtype dtype,
                         sam_plan* out);

/* C = A*B, FP32 operands. `workspace` may be NULL when the plan's
 * workspace_bytes is 0; otherwise it must hold at least that many bytes
 * (else SAM_ERR_WORKSPACE: the call never falls back to another plan). */
sam_status sam_gemm_f32(const float* A, const float* B, float* C, int64_t M,
                        int64_t N, int64_t K, void* workspace,
                        uint64_t workspace_bytes, void* stream);

/* C = A*B, bfloat16 operands as raw bit patterns, FP32 accumulate/output. */
sam_status sam_gemm_bf16(const uint16_t* A, const uint16_t* B, float* C,
                         int64_t M, int64_t N, int64_t K, void* workspace,
                         uint64_t workspace_bytes, void* stream);

/* C = A*B, IEEE binary16 operands as raw bit patterns, FP32 accumulate/out. */
sam_status sam_gemm_f16(const uint16_t* A, const uint16_t* B, float* C,
                        int64_t M, int64_t N, int64_t K, void* workspace,
                        uint64_t workspace_bytes, void* stream);

/* Element formats of block-scaled 8-bit operands (OCP Microscaling
 * specification v1.0): E4M3 (bias 7, 3 fraction bits, no infinity, largest
 * finite 448) and E5M2 (bias 15, 2 fraction bits, IEEE-style Inf/NaN). */
typedef enum { SAM_E4M3 = 0, SAM_E5M2 = 1 } sam_fp8_format;

/* Block-scaled 8-bit GEMM (the block-scaled low-precision operands whose
 * tile variants page "fix(fp4_gemm autotune) SM107 kernel family excluded
 * from autotune candidates and heuristics update - #4856" tunes; the page
 * fixes no format, this takes the OCP MX formats gfx950's matrix cores
 * implement):
 *   C[i][j] = sum over k of (2^(scale_a[i][k/32] - 127) * A[i][k])
 *                         * (2^(scale_b[j][k/32] - 127) * Bt[j][k])
 * with products accumulated in FP32 and C written in FP32.
 *   A       device, M rows of K element codes (format fmt_a), row stride K.
 *   Bt      device, N rows of K element codes (format fmt_b): B given
 *           K-contiguous, Bt[j][k] = B[k][j], row stride K.
 *   scale_a device, M rows of K/32 E8M0 codes (2^(code-127)), row stride K/32.
 *   scale_b device, N rows of K/32 E8M0 codes, row stride K/32.
 *   C       device, M rows of N floats, row stride N; write-only.
 * K must be a multiple of 32 (SAM_ERR_INVALID_ARG otherwise). A, Bt, C and
 * the workspace must be 16-byte aligned; the scale arrays may have any
 * alignment. Codes that encode NaN or Inf, and the scale code 255, are not
 * valid inputs: the elements of C they reach are then unspecified (no
 * fault). Workspace as for sam_gemm_f32 (sam_gemm_plan with SAM_MXFP8 gives
 * the plan and its workspace_bytes). Asynchronous on `stream`. */
sam_status sam_gemm_mxfp8(sam_fp8_format fmt_a, sam_fp8_format fmt_b,
                          const uint8_t* A, const uint8_t* scale_a,
                          const uint8_t* Bt, const uint8_t* scale_b, float* C,
                          int64_t M, int64_t N, int64_t K, void* workspace,
                          uint64_t workspace_bytes, void* stream);

/* The same with a forced block-scaled variant `id` and split (0 = the
 * variant's own choice; stream-K is not offered). SAM_ERR_UNSUPPORTED when
 * the variant is not a block-scaled one or the split is not admissible. */
sam_status sam_gemm_mxfp8_variant(int32_t id, int32_t split_k,
                                  sam_fp8_format fmt_a, sam_fp8_format fmt_b,
                                  const uint8_t* A, const uint8_t* scale_a,
                                  const uint8_t* Bt, const uint8_t* scale_b,
                                  float* C, int64_t M, int64_t N, int64_t K,
                                  void* workspace, uint64_t workspace_bytes,
                                  void* stream);

/* Block-scaled 4-bit GEMM (MXFP4, OCP Microscaling v1.0): the product of
 * sam_gemm_mxfp8 with E2M1 elements (1 sign, 2 exponent bits with bias 1, 1
 * fraction bit; values 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives) packed
 * two per byte: element k of a row is the low nibble of byte k/2 for even k
 * and the high nibble for odd k.
 *   A       device, M rows of K/2 bytes, row stride K/2.
 *   Bt      device, N rows of K/2 bytes (Bt[j] holds column j of B).
 *   scale_a, scale_b, C, K, alignment, workspace and errors as for
 *           sam_gemm_mxfp8 (sam_gemm_plan with SAM_MXFP4 gives the plan). */
sam_status sam_gemm_mxfp4(const uint8_t* A, const uint8_t* scale_a,
                          const uint8_t* Bt, const uint8_t* scale_b, float* C,
                          int64_t M, int64_t N, int64_t K, void* workspace,
                          uint64_t workspace_bytes, void* stream);

/* The same with a forced block-scaled variant `id` and split (0 = the
 * variant's own choice). */
sam_status sam_gemm_mxfp4_variant(int32_t id, int32_t split_k,
                                  const uint8_t* A, const uint8_t* scale_a,
                                  const uint8_t* Bt, const uint8_t* scale_b,
                                  float* C, int64_t M, int64_t N, int64_t K,
                                  void* workspace, uint64_t workspace_bytes,
                                  void* stream);

/* Operand forms of the general entry point. */
typedef enum { SAM_OP_N = 0, SAM_OP_T = 1 } sam_op;

/* General form C = alpha * op(A) * op(B) + beta * C, the usual BLAS
 * definition (the pages' GEMM is its alpha = 1, beta = 0, no-transpose
 * case: page "Scale coverage exposes a remaining GEMM gap", section
 * "Measurement contract and evidence"). Row-major storage with row strides:
 *   op(A) is M x K: SAM_OP_N reads A as M rows of K values (lda >= K),
 *                   SAM_OP_T reads A as K rows of M values (lda >= M);
 *   op(B) is K x N: SAM_OP_N reads K rows of N (ldb >= N), SAM_OP_T N rows of
 *                   K (ldb >= K);
 *   C is M rows of N values, ldc >= N.
 * Element types as for sam_gemm_<dtype>; alpha and beta are FP32. C is read
 * only when beta != 0 (with beta == 0 whatever C held never reaches the
 * result); A and B are not read when alpha == 0 or K == 0. The result is
 * fmaf(alpha, P, beta * C) with P the FP32 product of the GEMM path (alpha * P
 * when beta == 0).
 * How: a call with SAM_OP_N, SAM_OP_N, compact strides, alpha 1 and beta 0 is
 * exactly sam_gemm_<dtype>. Otherwise the plan for (M, N, K, dtype) decides:
 *  - ring plans (FP32 "f..." and 16-bit "r..." variants) read A and B rows
 *    with their strides in place when each row stays whole 16-byte pieces
 *    (or the plan reads that operand one value at a time, or copies it into
 *    padded rows anyway), and store C themselves with row stride ldc (a
 *    multiple of 4) and alpha / beta applied where C is written: in the
 *    kernel, the split-K reduce or the stream-K fix-up. 16-bit 16x16x32 ring
 *    plans also read transposed operands (SAM_OP_T) straight, when K, N and
 *    the transposed operand's leading dimension are multiples of 8 (a
 *    192-row tile hands a transposed A to its 256-row twin); FP32 ring plans
 *    with tiles up to 128 x 256 read a transposed B straight when K and ldb
 *    are multiples of 4, and those and the 256 x 256 tile a transposed A
 *    when N and lda are multiples of 4; FP32 with both operands transposed
 *    runs as the
 *    plain product B A of the operands as stored, whose ring plan stores C
 *    transposed;
 *  - whatever remains (a transposed operand the plan cannot read, other
 *    strides, other plan kinds) is copied into compact rows in the
 *    workspace first, the product goes to a workspace temporary unless the
 *    plan stores C itself or ldc == N and beta == 0, and a last pass applies
 *    alpha and beta; those copies cost extra HBM traffic.
 * Base pointers must be 16-byte aligned; the workspace must hold
 * sam_gemm_ex_workspace() bytes (SAM_ERR_WORKSPACE otherwise).
 * Asynchronous on `stream`, like the other entry points. */
sam_status sam_gemm_ex(sam_dtype dtype, sam_op trans_a, sam_op trans_b,
                       int64_t M, int64_t N, int64_t K, float alpha,
                       const void* A, int64_t lda, const void* B, int64_t ldb,
                       float beta, float* C, int64_t ldc, void* workspace,
                       uint64_t workspace_bytes, void* stream);

/* Workspace bytes sam_gemm_ex needs for these arguments (host only). */
sam_status sam_gemm_ex_workspace(sam_dtype dtype, sam_op trans_a,
                                 sam_op trans_b, int64_t M, int64_t N,
                                 int64_t K, int64_t lda, int64_t ldb,
                                 int64_t ldc, float alpha, float beta,
                                 uint64_t* bytes);

/* sam_gemm_ex with a forced plan: variant `id`, split_k and raster_n as for
 * sam_gemm_variant_r (SAM_ERR_UNSUPPORTED / SAM_ERR_INVALID_ARG likewise);
 * everything else as for sam_gemm_ex, with the workspace from
 * sam_gemm_ex_variant_workspace. For tests and tuning of the general forms. */
sam_status sam_gemm_ex_variant(int32_t id, int32_t split_k, int32_t raster_n,
                               sam_dtype dtype, sam_op trans_a,
                               sam_op trans_b, int64_t M, int64_t N,
                               int64_t K, float alpha, const void* A,
                               int64_t lda, const void* B, int64_t ldb,
                               float beta, float* C, int64_t ldc,
                               void* workspace, uint64_t workspace_bytes,
                               void* stream);

/* Workspace bytes sam_gemm_ex_variant needs for these arguments (host only). */
sam_status sam_gemm_ex_variant_workspace(int32_t id, int32_t split_k,
                                         int32_t raster_n, sam_dtype dtype,
                                         sam_op trans_a, sam_op trans_b,
                                         int64_t M, int64_t N, int64_t K,
                                         int64_t lda, int64_t ldb, int64_t ldc,
                                         float alpha, float beta,
                                         uint64_t* bytes);

/* Number of entries in the variant table (ids 0 .. count-1). */
int32_t sam_variant_count(void);

/* Static description of variant `id` (no shape: split_k = 1, grid 0). */
sam_status sam_variant_info(int32_t id, sam_plan* out);

/* The plan for a forced variant and split. split_k = 0 lets the dispatcher
 * pick the split for that variant, -1 asks for its stream-K form (FP32 ring
 * variants with tiles up to 128 x 256, when the shape has at least as many K
 * iterations as resident workgroups). SAM_ERR_UNSUPPORTED if the variant does
 * not take `dtype` or the split is not admissible for the shape;
 * SAM_ERR_INVALID_ARG for split_k < -1. The 16-bit 16x16x32 ring variants
 * have a stream-K form too: whole waves of tiles run one per workgroup and
 * the tiles of the last, partial wave share their K iterations. */
sam_status sam_variant_plan(int32_t id, int64_t M, int64_t N, int64_t K,
                            sam_dtype dtype, int32_t split_k, sam_plan* out);

/* The same with a forced raster order: raster_n = 0 (M-major), 1 (N-major)
 * or -1 (the one the cost model prefers for this variant and split; ties go
 * to M-major). The raster order decides which tiles run together and so how
 * much of each A and B panel the XCD's L2 serves to several of them (page
 * "fix(fp4_gemm autotune) SM107 kernel family excluded from autotune
 * candidates and heuristics update - #4856", section "Swap × raster
 * experiment: tile reuse root cause"). SAM_ERR_INVALID_ARG for other
 * raster_n; SAM_ERR_UNSUPPORTED where the variant has no tiles (the streaming
 * skinny kernels) and raster_n is 1. */
sam_status sam_variant_plan_r(int32_t id, int64_t M, int64_t N, int64_t K,
                              sam_dtype dtype, int32_t split_k, int32_t raster_n,
                              sam_plan* out);

/* The cost model's own plan for this shape, ignoring the frozen table of
 * measured shapes (host only; for calibration reports and tests). */
sam_status sam_gemm_plan_model(int64_t M, int64_t N, int64_t K, sam_dtype dtype,
                               sam_plan* out);

/* Run a forced variant (tests, profiling and calibration). Operands as for
 * sam_gemm_<dtype> (16-bit ones as uint16_t patterns). SAM_MXFP8 and
 * SAM_MXFP4 are refused with SAM_ERR_INVALID_ARG: block-scaled operands go
 * through sam_gemm_mxfp8_variant / sam_gemm_mxfp4_variant. */
sam_status sam_gemm_variant(int32_t id, sam_dtype dtype, int32_t split_k,
                            const void* A, const void* B, float* C, int64_t M,
                            int64_t N, int64_t K, void* workspace,
                            uint64_t workspace_bytes, void* stream);

/* Bytes of the device scratch array behind sam_gemm_noalloc (64 MiB per GPU). */
#define SAM_SCRATCH_BYTES (64ull << 20)

/* C = A*B exactly as sam_gemm_f32 / sam_gemm_bf16 / sam_gemm_f16 (`dtype`
 * SAM_F32, SAM_BF16 or SAM_F16; the same plan, kernels and bits) without a
 * caller workspace and without any allocation: for callers that cannot
 * allocate device memory (code under graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). The plan's workspace (padded operand
 * copies, split-K partials, stream-K slots) goes to a file-scope device array of SAM_SCRATCH_BYTES that each GPU holds from
 * its first such call until the process ends. A plan whose workspace_bytes
 * exceeds SAM_SCRATCH_BYTES is refused with SAM_ERR_WORKSPACE (use
 * sam_gemm_<dtype> with a workspace for it). Nothing in the array needs to
 * start at zero: every plan writes each workspace value before reading it.
 * Every call on one GPU shares that GPU's array, so calls that overlap in
 * time on one GPU (on different streams, or from different threads without
 * ordering) race and may return wrong results; calls in order on one stream
 * are safe. Other arguments, alignment and errors as for sam_gemm_f32. */
sam_status sam_gemm_noalloc(sam_dtype dtype, const void* A, const void* B,
                            float* C, int64_t M, int64_t N, int64_t K,
                            void* stream);

/* sam_gemm_variant with a forced raster order (raster_n as for
 * sam_variant_plan_r). */
sam_status sam_gemm_variant_r(int32_t id, sam_dtype dtype, int32_t split_k,
                              int32_t raster_n, const void* A, const void* B,
                              float* C, int64_t M, int64_t N, int64_t K,
                              void* workspace, uint64_t workspace_bytes,
                              void* stream);

/* Checks once per process that the current device is gfx950 and that the
 * library's kernels are loadable on it. SAM_ERR_UNSUPPORTED_DEVICE if not. */
sam_status sam_device_check(void);

/* Static text for a status code. */
const char* sam_status_string(sam_status s);

/* Detail of the last failing call on this thread ("" if none). */
const char* sam_last_error(void);

/* Build stamp: library version, git revision, ROCm/HIP version, target. */
const char* sam_build_info(void);

#ifdef __cplusplus
}
#endif

#endif /* SAM_H */
