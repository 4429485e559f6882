// The variant table. Ids are stable (new variants are appended) and run
// consecutively over both lists below.
//
// Staged variants (sam_kernels.hip): operands pass through registers into
// double-buffered LDS; compiled for FP32, bfloat16 and binary16 and for
// vector/element loads of A and B rows.
//   X(id, name, BM, BN, WM, WN, BLK, group_m, xcd_remap, max_split, eff_f32, eff_h16, pf_f32, pf_h16)
// LDS-ring variants (sam_kernels_dma.hip): 16-bit operands with K % 8 == 0
// and N % 8 == 0 only; loads write LDS directly into a ring of NBUF stages.
//   D(id, name, BM, BN, WM, WN, BK, NBUF, group_m, xcd_remap, max_split, eff_h16)
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
    D(8, "r256x256_w2x2_k32n4",  256, 256, 2, 2, 32, 4, 8, 1, 8, 0.45)                   \
    D(9, "r128x256_w2x2_k32n4",  128, 256, 2, 2, 32, 4, 8, 1, 8, 0.37)                   \
    D(10, "r256x128_w2x2_k32n4", 256, 128, 2, 2, 32, 4, 8, 1, 8, 0.36)                   \
    D(11, "r128x128_w2x2_k32n4", 128, 128, 2, 2, 32, 4, 8, 1, 16, 0.34)                  \
    D(12, "r256x256_w2x2_k64n2", 256, 256, 2, 2, 64, 2, 8, 1, 8, 0.47)                   \
    D(13, "r256x128_w2x2_k64n3", 256, 128, 2, 2, 64, 3, 8, 1, 8, 0.38)                   \
    D(14, "r128x256_w2x2_k64n3", 128, 256, 2, 2, 64, 3, 8, 1, 8, 0.37)
