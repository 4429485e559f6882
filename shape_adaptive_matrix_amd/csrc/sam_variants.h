// The variant table. Ids are stable (new variants are appended) and run
// consecutively over both lists below.
//
// Staged variants (sam_kernels.hip): operands pass through registers into
// double-buffered LDS; compiled for FP32, bfloat16 and binary16 and for
// vector/element loads of A and B rows.
//   X(id, name, BM, BN, WM, WN, BLK, group_m, xcd_remap, max_split, eff_f32, eff_h16, pf_f32, pf_h16)
// LDS-ring variants (sam_kernels_dma.hip): 16-bit operands with K % 8 == 0
// and N % 8 == 0 only; loads write LDS directly into a ring of NBUF stages.
//   D(id, name, BM, BN, WM, WN, BK, NBUF, MODE, BLK, group_m, xcd_remap, max_split, eff_h16)
// BLK is the MFMA block edge: 32 (32x32x16) or 16 (16x16x32, names "..._b16",
// ids 45.., listed after the block-scaled variants).
// MODE 0 loads straight into LDS; MODE 1 loads into registers and writes LDS
// (names start with "q"); MODE 2 loads A straight into LDS and B through
// registers, transposed to K-contiguous rows (names start with "h").
// Streaming variants (sam_kernels_stream.hip): FP32 only, M <= 16 (tile
// 16 x 64) or N <= 16 (tile 64 x 16); the large operand streams from HBM into
// registers, KB values of K per workgroup block.
//   S(id, name, BM, BN, KB, max_split, eff_hbm)
// FP32 LDS-ring variants (sam_kernels_f32ring.hip): K % 4 == 0 and
// N % 4 == 0 only; both operands load straight into a ring of NBUF LDS
// stages of BK values of K; wave tiles of 32-row blocks x 32 V-column groups
// (B read V columns at a time); KS = 2 runs two waves per tile position, each
// on half of every stage's K steps (names "...s2"); BLK is the MFMA block
// edge, 32 (32x32x2) or 16 (16x16x4, names "...b16"); EL = 1: the variant
// also has an element-load form for K or N not a multiple of 4.
//   F(id, name, BM, BN, WM, WN, BK, NBUF, V, KS, BLK, EL, group_m, xcd_remap, max_split, eff_f32)
// Block-scaled variants (ids 40..): sam_variants_mx.h.
// eff_* is the fraction of the MFMA peak the variant sustains in steady
// state, the calibration the cost model uses.
#pragma once

#define SAM_STAGED_VARIANTS(X)                                                           \
    X(0, "t64x64_w2x2_b32",    64,  64, 2, 2, 32, 8, 1, 16, 0.74, 0.12, 1, 2)            \
    X(1, "t128x128_w2x2_b32", 128, 128, 2, 2, 32, 8, 1, 16, 0.84, 0.28, 1, 2)            \
    X(2, "t128x256_w2x2_b32", 128, 256, 2, 2, 32, 8, 1,  8, 0.78, 0.31, 1, 2)            \
    X(3, "t256x128_w2x2_b32", 256, 128, 2, 2, 32, 8, 1,  8, 0.78, 0.31, 1, 2)            \
    X(4, "t256x256_w2x2_b32", 256, 256, 2, 2, 32, 8, 1,  8, 0.825, 0.40, 1, 1)           \
    X(5, "t16x256_w1x4_b16",   16, 256, 1, 4, 16, 1, 1, 32, 0.45, 0.05, 1, 2)            \
    X(6, "t256x16_w4x1_b16",  256,  16, 4, 1, 16, 8, 1, 32, 0.54, 0.05, 1, 2)            \
    X(7, "t256x256_w2x4_b32", 256, 256, 2, 4, 32, 8, 1,  8, 0.88, 0.35, 1, 1)

#define SAM_DMA_VARIANTS(D)                                                              \
    D(8, "r256x256_w2x2_k32n4", 256, 256, 2, 2, 32, 4, 0, 32, 8, 1, 8, 0.45)                   \
    D(9, "r128x256_w2x2_k32n4", 128, 256, 2, 2, 32, 4, 0, 32, 8, 1, 8, 0.37)                   \
    D(10, "r256x128_w2x2_k32n4", 256, 128, 2, 2, 32, 4, 0, 32, 8, 1, 8, 0.36)                   \
    D(11, "r128x128_w2x2_k32n4", 128, 128, 2, 2, 32, 4, 0, 32, 8, 1, 16, 0.34)                  \
    D(12, "r256x256_w2x2_k64n2", 256, 256, 2, 2, 64, 2, 0, 32, 8, 1, 8, 0.47)                   \
    D(13, "r256x128_w2x2_k64n3", 256, 128, 2, 2, 64, 3, 0, 32, 8, 1, 8, 0.38)                   \
    D(14, "r128x256_w2x2_k64n3", 128, 256, 2, 2, 64, 3, 0, 32, 8, 1, 8, 0.37)                \
    D(15, "q256x256_w2x2_k64", 256, 256, 2, 2, 64, 2, 1, 32, 8, 1, 8, 0.44)                \
    D(16, "h256x256_w2x2_k64", 256, 256, 2, 2, 64, 2, 2, 32, 8, 1, 8, 0.36)                \
    D(17, "r256x256_w2x4_k64n2", 256, 256, 2, 4, 64, 2, 0, 32, 8, 1, 8, 0.50)                \
    D(18, "r256x256_w4x2_k64n2", 256, 256, 4, 2, 64, 2, 0, 32, 8, 1, 8, 0.495)                \
    D(19, "r256x256_w2x4_k32n4", 256, 256, 2, 4, 32, 4, 0, 32, 8, 1, 8, 0.47)

#define SAM_STREAM_VARIANTS(S)                                                           \
    S(20, "sm16x64_k2048", 16, 64, 2048, 32, 0.92)                                       \
    S(21, "sn64x16_k2048", 64, 16, 2048, 32, 0.75)                                       \
    S(22, "sm16x64_k1024", 16, 64, 1024, 32, 0.97)                                       \
    S(23, "sn64x16_k1024", 64, 16, 1024, 32, 0.81)

#define SAM_F32RING_VARIANTS(F)                                                          \
    F(24, "f128x128_w4x1_k64n2", 128, 128, 4, 1, 64, 2, 4, 1, 32, 0, 8, 1, 16, 0.84)               \
    F(25, "f128x128_w4x1_k32n4", 128, 128, 4, 1, 32, 4, 4, 1, 32, 0, 8, 1, 16, 0.82)               \
    F(26, "f256x128_w8x1_k32n3", 256, 128, 8, 1, 32, 3, 4, 1, 32, 1, 8, 1,  8, 0.89)               \
    F(27, "f128x256_w4x2_k32n3", 128, 256, 4, 2, 32, 3, 4, 1, 32, 1, 8, 1,  8, 0.89)               \
    F(28, "f64x128_w2x1_k32n2",   64, 128, 2, 1, 32, 2, 4, 1, 32, 1, 8, 1, 16, 0.5)               \
    F(29, "f256x256_w4x2_k32n2", 256, 256, 4, 2, 32, 2, 4, 1, 32, 1, 8, 1,  8, 0.94)               \
    F(30, "f128x128_w4x2_k64n2", 128, 128, 4, 2, 64, 2, 2, 1, 32, 1, 8, 1, 16, 0.885)               \
    F(31, "f128x128_w4x2_k32n4", 128, 128, 4, 2, 32, 4, 2, 1, 32, 1, 8, 1, 16, 0.875)               \
    F(32, "f256x128_w8x2_k32n3", 256, 128, 8, 2, 32, 3, 2, 1, 32, 1, 8, 1,  8, 0.89)                \
    F(33, "f128x128_w2x2s2_k64n2", 128, 128, 2, 2, 64, 2, 2, 2, 32, 1, 8, 1, 16, 0.895)            \
    F(34, "f128x128_w2x2s2_k32n4", 128, 128, 2, 2, 32, 4, 2, 2, 32, 1, 8, 1, 16, 0.885)            \
    F(35, "f128x128_w2x2s2_k64n2_b16", 128, 128, 2, 2, 64, 2, 4, 2, 16, 1, 8, 1, 16, 0.91)   \
    F(36, "f256x256_w4x2_k32n2_b16",   256, 256, 4, 2, 32, 2, 4, 1, 16, 0, 8, 1,  8, 0.95)   \
    F(37, "f128x128_w4x2_k64n2_b16",   128, 128, 4, 2, 64, 2, 4, 1, 16, 1, 8, 1, 16, 0.895)            \
    F(38, "f128x128_w4x2_k32n2_b16",   128, 128, 4, 2, 32, 2, 4, 1, 16, 1, 8, 1, 16, 0.88)   \
    F(39, "f128x128_w4x2_k32n2",       128, 128, 4, 2, 32, 2, 2, 1, 32, 1, 8, 1, 16, 0.87)

#include "sam_variants_mx.h"

#define SAM_DMA16_VARIANTS(D)                                                            \
    D(45, "r256x256_w2x4_k64n2_b16", 256, 256, 2, 4, 64, 2, 0, 16, 8, 1, 8, 0.58)         \
    D(46, "r256x256_w4x2_k64n2_b16", 256, 256, 4, 2, 64, 2, 0, 16, 8, 1, 8, 0.575)         \
    D(47, "r128x128_w2x2_k64n2_b16", 128, 128, 2, 2, 64, 2, 0, 16, 8, 1, 16, 0.34)

// Single-launch small-tile variants (sam_kernels_kq.hip): FP32 only, a
// 16 TB x 16 TB tile per workgroup whose NW waves (4 or 8, names "..._w8")
// each take a share of K and sum their partial tiles in LDS in a fixed
// order; any K and N.
//   Q(id, name, TB, NW, group_m, xcd_remap, eff_f32)
#define SAM_KQ_VARIANTS(Q)                                                               \
    Q(48, "kq32x32", 2, 4, 8, 1, 0.55)                                                   \
    Q(49, "kq48x48", 3, 4, 8, 1, 0.65)                                                   \
    Q(50, "kq64x64", 4, 4, 8, 1, 0.70)

// Persistent short-K variants (sam_kernels_kp.hip): FP32 only, K <= KP,
// K % 4 == 0 and N % 4 == 0; 128 x 128 tiles, resident workgroups walk their
// tiles with the next tile's panels loading and the last tile's stores
// draining while the current one is multiplied.
//   P(id, name, KP, group_m, xcd_remap, eff_f32)
#define SAM_KP_VARIANTS(P)                                                               \
    P(51, "kp128x128_k32", 32, 8, 1, 0.80)                                              \
    P(52, "kp128x128_k64", 64, 8, 1, 0.85)

// Eight-wave forms of the single-launch small-tile variants (same list format).
#define SAM_KQ8_VARIANTS(Q)                                                              \
    Q(53, "kq32x32_w8", 2, 8, 8, 1, 0.62)                                                \
    Q(54, "kq48x48_w8", 3, 8, 8, 1, 0.73)                                                \
    Q(55, "kq64x64_w8", 4, 8, 8, 1, 0.78)

// Operand-swap forms of the 16x16x32 ring variants (same list format as
// SAM_DMA16_VARIANTS plus SW = 1): the MFMA computes the transposed block, so
// each lane stores four adjacent columns of C with one 16-byte store.
//   D(id, name, BM, BN, WM, WN, BK, NBUF, MODE, BLK, SW, group_m, xcd_remap, max_split, eff_h16)
#define SAM_DMA16S_VARIANTS(D)                                                           \
    D(56, "r256x256_w2x4_k64n2_b16_sw", 256, 256, 2, 4, 64, 2, 0, 16, 1, 8, 1, 8, 0.575)  \
    D(57, "r256x256_w4x2_k64n2_b16_sw", 256, 256, 4, 2, 64, 2, 0, 16, 1, 8, 1, 8, 0.57)  \
    D(58, "r128x128_w2x2_k64n2_b16_sw", 128, 128, 2, 2, 64, 2, 0, 16, 1, 8, 1, 16, 0.34)

// 192-row tiles of the 16x16x32 ring (same list format as SAM_DMA16S_VARIANTS):
// for shapes whose 256-row tile count leaves a large part of the CUs idle or
// adds a partial round (M = 2049: nine 256-row tiles, the last holding one
// row; M = 6144: 32 row tiles instead of 24), three quarters of the work per
// workgroup in more workgroups. A 192-row tile is not a power of two, so it
// has no transposed-A form (its A^T rows would not be whole 1 KB loads).
#define SAM_DMA16M_VARIANTS(D)                                                           \
    D(59, "r192x256_w2x4_k64n2_b16", 192, 256, 2, 4, 64, 2, 0, 16, 0, 8, 1, 8, 0.55)    \
    D(60, "r192x256_w2x4_k64n2_b16_sw", 192, 256, 2, 4, 64, 2, 0, 16, 1, 8, 1, 8, 0.545)

// Padding forms of FP32 ring variants (same list format as
// SAM_F32RING_VARIANTS; EL 0): for K or N not a multiple of 4 they copy the
// operand whose rows are not whole 16-byte pieces into the workspace with
// its rows padded to a multiple of 4 values (zeros in the gap), and run the
// 16-byte-load kernel on the copy instead of the element-load form. Not
// admitted when K and N are multiples of 4 (then they are their base
// variant).
#define SAM_F32PAD_VARIANTS(F)                                                           \
    F(61, "f128x128_w4x2_k32n2_b16_pad",   128, 128, 4, 2, 32, 2, 4, 1, 16, 0, 8, 1, 16, 0.88)   \
    F(62, "f256x256_w4x2_k32n2_b16_pad",   256, 256, 4, 2, 32, 2, 4, 1, 16, 0, 8, 1,  8, 0.95)   \
    F(63, "f128x128_w2x2s2_k64n2_b16_pad", 128, 128, 2, 2, 64, 2, 4, 2, 16, 0, 8, 1, 16, 0.91)

// A deeper ring for 128 x 128 16-bit tiles (same list format as
// SAM_DMA16S_VARIANTS): such a tile moves half the bytes per stage of a
// 256 x 256 one, so four stages (three in flight) fit where two do there,
// and eight waves of 64 x 32 keep enough loads and MFMAs in flight per CU
// for shapes whose tile counts leave no room for larger tiles.
#define SAM_DMA16D_VARIANTS(D)                                                           \
    D(64, "r128x128_w2x4_k64n4_b16", 128, 128, 2, 4, 64, 4, 0, 16, 0, 8, 1, 16, 0.40)
