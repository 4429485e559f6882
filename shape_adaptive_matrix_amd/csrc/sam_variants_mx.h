// Block-scaled variants (sam_kernels_mx.hip), ids continuing the table of
// sam_variants.h: E4M3 / E5M2 elements with E8M0 scales per 32 values of K,
// both operands K-contiguous, K % 32 == 0; a ring of two LDS stages of BK
// values of K. SD = 1: with K % 128 == 0 the scales travel through LDS with
// the operands (SD = 0, or other K: each lane loads its own scale bytes).
// The same variants run E2M1 elements (MXFP4) with 2 BK values of K per
// stage in the same LDS rows.
//   M8(id, name, BM, BN, WM, WN, BK, SD, group_m, xcd_remap, max_split, eff_mx8, eff_mx4)
// eff_* is the fraction of the MFMA peak the variant sustains in steady
// state, the calibration the cost model uses.
#pragma once

#define SAM_MX8_VARIANTS(M8)                                                             \
    M8(40, "x256x256_w2x2_k128", 256, 256, 2, 2, 128, 1, 8, 1,  8, 0.44, 0.31)           \
    M8(41, "x256x128_w4x2_k128", 256, 128, 4, 2, 128, 1, 8, 1,  8, 0.30, 0.25)           \
    M8(42, "x128x128_w2x2_k128", 128, 128, 2, 2, 128, 1, 8, 1, 16, 0.33, 0.215)          \
    M8(43, "x128x128_w2x2_k256", 128, 128, 2, 2, 256, 1, 8, 1, 16, 0.28, 0.23)           \
    M8(44, "x128x256_w2x4_k128", 128, 256, 2, 4, 128, 1, 8, 1,  8, 0.28, 0.255)
