// Internal declarations shared by the dispatcher, the kernels and the C ABI.
#pragma once

#include <stdint.h>
#include <hip/hip_runtime.h>

namespace sam {

// DT_MX8: block-scaled 8-bit elements (E4M3 / E5M2 with E8M0 scales per 32 of K);
// DT_MX4: block-scaled E2M1 elements, two per byte.
enum Dt : int { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2, DT_MX8 = 3, DT_MX4 = 4 };

// Fixed facts of one MI355X (gfx950) used by the cost model. They are frozen
// here rather than queried so that a plan is a pure function of the shape.
struct DeviceModel {
    int cus = 256;                 // 8 XCDs x 32 CUs
    int xcds = 8;
    int lds_bytes = 160 * 1024;    // LDS per CU
    double clock_ghz = 2.4;
    double f32_flop_per_clk_cu = 256.0;    // 4 SIMDs x 64 (32x32x2 f32 in 64 clk)
    double h16_flop_per_clk_cu = 4096.0;   // 4 SIMDs x 1024
    double mx8_flop_per_clk_cu = 8192.0;   // 4 SIMDs x 2048 (32x32x64 8-bit in 64 clk)
    double mx4_flop_per_clk_cu = 16384.0;  // 4 SIMDs x 4096 (32x32x64 4-bit in 32 clk)
    double hbm_gbs = 5900.0;       // measured streaming read rate
    double tiled_hbm_frac = 0.75;  // share of it the LDS-tiled kernels reach when HBM-bound (calibrated)
    double hbm_write_gbs = 6000.0; // rate the epilogue write phase drains at (calibrated)
    double l2_gbs = 16000.0;       // operand delivery from L2 into LDS, chip-wide (calibrated)
    double fabric_gbs = 7000.0;    // L2 misses: delivery from beyond L2, chip-wide (measured)
    double launch_us = 4.0;        // per kernel launch, rough
};

// Static description of a tile/schedule variant.
enum Kind : int { KIND_STAGED = 0, KIND_DMA = 1, KIND_STREAM = 2, KIND_F32RING = 3, KIND_MX8 = 4, KIND_KQ = 5, KIND_KP = 6 };

struct Variant {
    int id;
    const char* name;
    int kind;            // Kind
    int dtype_mask;      // bit (1 << Dt)
    int bm, bn;          // macro tile
    int wm, wn;          // wave grid
    int blk;             // MFMA block edge (32 or 16)
    int nbuf;            // LDS stages (2 for staged variants, the ring depth otherwise)
    int bk;              // K per LDS stage for ring variants (0: by dtype, staged variants),
                         // K block of a workgroup for streaming variants
    int group_m;         // grouped raster height (tiles)
    int xcd_remap;       // 1: remap workgroup ids so each XCD gets a contiguous range
    int max_split;       // largest split-K the variant is planned with
    int elem_loads;      // takes rows that are not whole 16-byte pieces (K or N odd for FP32)
    int swap;            // MFMA operands exchanged: the accumulators hold the transposed block
    double eff_f32;      // calibrated fraction of MFMA peak it sustains in steady state
                         // (streaming variants: fraction of the HBM read rate)
    double eff_h16;
    double eff_mx8;      // block-scaled 8-bit variants
    double eff_mx4;      // ... running E2M1 elements
    int pad;             // FP32 ring: takes rows that are not whole 16-byte pieces through padded copies
};

int variant_count();
const Variant* variant_get(int id);

// Arguments of one main-kernel launch.
struct GemmArgs {
    const void* A;
    const void* B;
    float* out;          // C when split == 1, else workspace partials [split][M][N]
    int M, N, K;
    int k_chunk;         // K range per split, a multiple of the LDS K-stage
    int split;
    int tiles_m, tiles_n;
    int group_m;
    int xcd_remap;
    long long part_stride;  // M*N (elements between consecutive partials)
    float* ws;           // stream-K: partial-tile slots (2 per workgroup, BM*BN floats each)
    int sk_iters;        // stream-K: K iterations per tile (0: data-parallel launch)
    int sk_grid;         // stream-K: workgroups sharing the stream-K tiles' iterations
    int sk_dp;           // stream-K: leading tiles run one per workgroup before them (16-bit form)
    int raster_n;        // 1: raster groups of group_m tile columns walk the rows (N-major)
    int lda, ldb;        // row strides of A and B in elements (ring kernels; K and N otherwise)
    // Final store of C (not of split-K partials; ring kernels and their
    // stream-K fix-up only): row stride ldc, and with epi = 1 the stored
    // value is alpha t + beta C for the product t, as the general entry
    // point defines it (C read only when beta != 0). Otherwise ldc = N,
    // epi = 0.
    int ldc;
    int epi;
    float alpha, beta;
    // FP32 ring kernels, their stream-K fix-up and the general split-K
    // reduce: the product D (M x N here) is stored transposed, D[i][j] at
    // C[j * ldc + i] (the general entry point's A^T B^T, computed as B A).
    int ct;
    const unsigned char* sa;   // block-scaled operands: scale codes of A (M x K/32)
    const unsigned char* sb;   // ... and of B (N x K/32); B is then N rows of K codes
    int fmt_a, fmt_b;    // element formats: 0 E4M3, 1 E5M2
};

// Fully resolved plan (internal form of sam_plan).
struct Plan {
    int variant_id;
    int kind;
    int dtype;
    int bm, bn, bk;
    int wm, wn, blk;
    int split;
    int k_chunk;
    int group_m;
    int xcd_remap;
    int a_vec, b_vec;
    int c_vec;           // FP32 ring: C rows are whole 16-byte pieces (N % 4 == 0), stored 16 bytes at a time
    int tiles_m, tiles_n;
    long long grid;
    unsigned long long ws_bytes;
    double est_us;
    int tuned;           // 1: taken from the frozen table of measured shapes
    int sk;              // 1: stream-K (grid = persistent workgroups, split == 1)
    int sk_dp;           // stream-K: tiles run one per workgroup ahead of the shared ones
    int sk_g;            // stream-K: workgroups sharing the remaining tiles' iterations
    int raster_n;        // 0: groups of group_m tile rows sweep the columns; 1: the transpose
    int swap;            // 1: MFMA operands exchanged (accumulators hold the transposed block)
    // 16-bit operands whose rows are not whole 16-byte pieces: A (K % 8 != 0)
    // and / or B (N % 8 != 0) are first copied into the workspace with row
    // strides lda / ldb rounded up to a multiple of 8 and zeros in the gap,
    // then the ring kernel reads the copies. ws_inner is where the plan's own
    // split-K / stream-K workspace starts.
    int pad_a, pad_b;
    long long lda, ldb;
    unsigned long long ws_inner;
    // 16-bit ring plans of the general entry point: operands given
    // transposed and read straight by the kernel, bit 0 B (N rows of K
    // values, row stride ldb), bit 1 A (K rows of M values, row stride lda).
    int tr;
};

// Dispatcher (sam_plan.cpp). Host only, pure.
// raster_req: -1 lets the cost model pick the raster order, 0 / 1 forces it.
bool plan_for_variant(int vid, long long M, long long N, long long K, int dtype,
                      int split_req, Plan* out, int raster_req = -1);
bool plan_auto(long long M, long long N, long long K, int dtype, Plan* out);
// The cost model's own choice, ignoring the frozen table.
bool plan_model(long long M, long long N, long long K, int dtype, Plan* out);
void plan_name(const Plan& p, char* buf, int n);
int k_stage(const Variant& v, int dtype);   // K per LDS stage
// The operand-swap form of a variant (same tile and schedule, 16-byte
// stores and loads of C), or -1.
int swap_twin(int id);
// The 16-bit ring variant with the same schedule on 256-row tiles (for a
// tile that has no A-given-transposed form), or -1.
int tile256_twin(int id);
// Whether an FP32 ring variant has the form that reads B given transposed
// (N rows of K values) straight, in its data-parallel or stream-K form.
bool f32_has_bt(int variant_id, bool stream_k);
// Whether it has the form that reads A given transposed (K rows of M
// values) straight, with B's and C's rows whole 16-byte pieces.
bool f32_has_at(int variant_id, bool stream_k);

// Kernel launchers (sam_kernels.hip). Return hipSuccess or the launch error.
hipError_t launch_gemm(const Plan& p, const GemmArgs& a, hipStream_t s);
hipError_t launch_gemm_dma(const Plan& p, const GemmArgs& a, hipStream_t s);
hipError_t launch_stream(const Plan& p, const GemmArgs& a, hipStream_t s);
hipError_t launch_f32_ring(const Plan& p, const GemmArgs& a, hipStream_t s);
hipError_t launch_sk_fixup(const Plan& p, const GemmArgs& a, hipStream_t s);
typedef void (*KernelFn)(GemmArgs);
// 16-bit ring kernels for operands given transposed (layout: bit 0 B,
// bit 1 A), and whether a variant has both forms of a layout.
KernelFn dma_t_kernel(int variant_id, int layout, bool stream_k, int dtype);
bool dma_has_layout(int variant_id, int layout, int dtype);
hipError_t launch_sk_fixup_dma(const Plan& p, const GemmArgs& a, hipStream_t s);
hipError_t launch_mx8(const Plan& p, const GemmArgs& a, hipStream_t s);
hipError_t launch_kq(const Plan& p, const GemmArgs& a, hipStream_t s);
hipError_t launch_kp(const Plan& p, const GemmArgs& a, hipStream_t s);
hipError_t launch_reduce(const float* parts, int split, long long part_stride,
                         float* C, long long count, hipStream_t s);
// Split-K sum into C with row stride ldc through the general entry point's
// epilogue (alpha t + beta C), transposed when ct.
hipError_t launch_reduce_ex(const float* parts, int split, long long part_stride, float* C, long long M, long long N,
                            long long ldc, float alpha, float beta, int ct, hipStream_t s);
hipError_t launch_zero(float* C, long long count, hipStream_t s);
// General entry point (sam_kernels_ex.hip): pack an operand (transposing
// when `trans`) into compact rows, and C = alpha T + beta C.
hipError_t launch_pack(const void* in, long long ld, void* out, long long rows, long long cols, int elem_bytes,
                       int trans, hipStream_t s);
hipError_t launch_axpby(const float* T, long long ldt, float* C, long long ldc, long long M, long long N, float alpha,
                        float beta, hipStream_t s);
// 16-bit rows x cols (row stride lds elements) into dst with row stride ldd
// (a multiple of 8, dst 16-byte aligned), zeros in columns cols .. ldd - 1.
// One padded copy of an operand: rows x cols values of es bytes (2 or 4)
// with row stride lds into rows of ldd values (ldd es a multiple of 16),
// zeros past cols.
struct PadCopy {
    const void* src;
    long long lds;
    void* dst;
    long long ldd, rows, cols;
};
// Both operands' copies in one launch; a copy with no rows is skipped.
hipError_t launch_pad(const PadCopy& a, const PadCopy& b, int es, hipStream_t s);
// A representative kernel symbol for loadability checks.
const void* probe_kernel();

}  // namespace sam
