// The variant table: macro tile, wave grid, MFMA block edge, raster and the
// calibrated steady-state efficiency used by the cost model. Every variant is
// compiled for FP32, bfloat16 and binary16 operands and for aligned/unaligned
// A and B rows. Ids are stable: new variants are appended.
//
//   X(id, name, BM, BN, WM, WN, BLK, group_m, xcd_remap, max_split, eff_f32, eff_h16)
#pragma once

#define SAM_VARIANT_LIST(X)                                                        \
    X(0, "t64x64_w2x2_b32",    64,  64, 2, 2, 32, 8, 1, 16, 0.45, 0.25)          \
    X(1, "t128x128_w2x2_b32", 128, 128, 2, 2, 32, 8, 1, 16, 0.70, 0.45)          \
    X(2, "t128x256_w2x2_b32", 128, 256, 2, 2, 32, 8, 1,  8, 0.72, 0.50)          \
    X(3, "t256x128_w2x2_b32", 256, 128, 2, 2, 32, 8, 1,  8, 0.72, 0.50)          \
    X(4, "t256x256_w2x2_b32", 256, 256, 2, 2, 32, 8, 1,  8, 0.75, 0.55)          \
    X(5, "t16x256_w1x4_b16",   16, 256, 1, 4, 16, 1, 1, 32, 0.40, 0.30)          \
    X(6, "t256x16_w4x1_b16",  256,  16, 4, 1, 16, 8, 1, 32, 0.40, 0.30)
