"""Planted mistakes in copies of the oracle must each fail some pin (CPU only).

Each mutant is a one-line textual change to a copy of ``oracle/oracle.c`` (a
dropped term, a sign error, a wrong index, a wrong format constant, a wrong
zero, a narrower accumulator), built into its own library under a temporary
directory. The real oracle is never modified.
"""
import pytest

import oracle
from tests import pins

MUTANTS = {
    "drop_last_k": ("for (int64_t k = 0; k < K; ++k) {\n            const double a",
                    "for (int64_t k = 0; k < K - 1; ++k) {\n            const double a"),
    "sign_flip": ("acc[j] = acc[j] + a * brow[j]", "acc[j] = acc[j] - a * brow[j]"),
    "reversed_k_in_A": ("const double a = load_val(dtype, A, i * K + k);",
                        "const double a = load_val(dtype, A, i * K + (K - 1 - k));"),
    "transposed_B_decode": ("Bd[k * N + j] = load_val(dtype, B, k * N + j);",
                            "Bd[k * N + j] = load_val(dtype, B, (k * N + j) % K * N + (k * N + j) / K);"),
    "bf16_bias": ("v = ldexp((double)(0x80 | f), e - 127 - 7);",
                  "v = ldexp((double)(0x80 | f), e - 126 - 7);"),
    "f16_subnormal_scale": ("v = ldexp((double)f, -14 - 10);", "v = ldexp((double)f, -15 - 10);"),
    "f16_hidden_bit": ("v = ldexp((double)(0x400 | f), e - 15 - 10);",
                       "v = ldexp((double)f, e - 15 - 10);"),
    "negative_zero_start": ("acc[j] = 0.0;", "acc[j] = -0.0;"),
    "float_point_accumulator": ("double s = 0.0;\n        for (int64_t k = 0; k < K; ++k)\n            s = s + load_val",
                                "float s = 0.0f;\n        for (int64_t k = 0; k < K; ++k)\n            s = s + load_val"),
    "points_column_reversed": ("load_val(dtype, B, k * N + j);\n        out[p]",
                               "load_val(dtype, B, k * N + (N - 1 - j));\n        out[p]"),
    "ex_ignores_trans_a": ("trans_a ? k * lda + i : i * lda + k", "i * lda + k"),
    "ex_ldb_taken_as_n": ("trans_b ? j * ldb + k : k * ldb + j", "trans_b ? j * ldb + k : k * N + j"),
    "ex_beta_sign": ("v = v + beta * (double)C0[i * N + j];", "v = v - beta * (double)C0[i * N + j];"),
    "ex_product_when_alpha_zero": ("const int product = alpha != 0.0 && K > 0;", "const int product = K > 0;"),
    "ex_reads_c_when_beta_zero": ("if (beta != 0.0) v = v + beta", "if (C0) v = v + beta"),
    "mx_e4m3_bias": ("v = ldexp((double)(0x8 | f), e - 7 - 3);", "v = ldexp((double)(0x8 | f), e - 8 - 3);"),
    "mx_e4m3_subnormal_scale": ("v = ldexp((double)f, -6 - 3);", "v = ldexp((double)f, -7 - 3);"),
    "mx_e4m3_nan_taken_as_value": ("if (e == 0xF && f == 0x7)", "if (e == 0xF && f == 0x7 && sign)"),
    "mx_e5m2_hidden_bit": ("v = ldexp((double)(0x4 | f), e - 15 - 2);", "v = ldexp((double)f, e - 15 - 2);"),
    "mx_e5m2_no_inf": ("v = f ? NAN : INFINITY;\n        else if (e == 0)\n            v = ldexp((double)f, -14 - 2);",
                       "v = NAN;\n        else if (e == 0)\n            v = ldexp((double)f, -14 - 2);"),
    "mx_e8m0_bias": ("ldexp(1.0, (int)code - 127)", "ldexp(1.0, (int)code - 126)"),
    "mx_scale_block_shifted": ("codes[row * K + k]) * oracle_decode_e8m0(scales[row * (K / 32) + k / 32]",
                               "codes[row * K + k]) * oracle_decode_e8m0(scales[row * (K / 32) + (k / 32 + 1) % (K / 32)]"),
    "mx_scale_row_ignored": ("codes[row * K + k]) * oracle_decode_e8m0(scales[row * (K / 32) + k / 32]",
                             "codes[row * K + k]) * oracle_decode_e8m0(scales[k / 32]"),
    "mx_block_of_16": ("codes[row * K + k]) * oracle_decode_e8m0(scales[row * (K / 32) + k / 32]",
                       "codes[row * K + k]) * oracle_decode_e8m0(scales[row * (K / 32) + (k / 16) % (K / 32)]"),
    "mx_format_b_ignored": ("s = s + mx_val(fmt_a, A, SA, i, K, k) * mx_val(fmt_b, Bt, SB, j, K, k);",
                            "s = s + mx_val(fmt_a, A, SA, i, K, k) * mx_val(fmt_a, Bt, SB, j, K, k);"),
    "mx_b_taken_row_major": ("s = s + mx_val(fmt_a, A, SA, i, K, k) * mx_val(fmt_b, Bt, SB, j, K, k);",
                             "s = s + mx_val(fmt_a, A, SA, i, K, k) * oracle_decode_fp8(fmt_b, Bt[k * N + j]) * "
                             "oracle_decode_e8m0(SB[j * (K / 32) + k / 32]);"),
    "mx4_bias": ("ldexp((double)(0x2 | f), e - 1 - 1)", "ldexp((double)(0x2 | f), e - 2 - 1)"),
    "mx4_subnormal_scale": ("e == 0 ? ldexp((double)f, -1)", "e == 0 ? ldexp((double)f, 0)"),
    "mx4_hidden_bit": ("ldexp((double)(0x2 | f), e - 1 - 1)", "ldexp((double)f, e - 1 - 1)"),
    "mx4_byte_index_shifted": ("const uint8_t byte = codes[row * (K / 2) + k / 2];",
                               "const uint8_t byte = codes[row * (K / 2) + (k / 2 + 1) % (K / 2)];"),
    "mx4_one_nibble_for_both": ("(k & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 0xF)",
                                "(uint8_t)(byte & 0xF)"),
    "mx4_scale_row_ignored": ("return oracle_decode_fp4(code) * oracle_decode_e8m0(scales[row * (K / 32) + k / 32]);",
                              "return oracle_decode_fp4(code) * oracle_decode_e8m0(scales[k / 32]);"),
    "mx4_points_rows_cols_swapped": ("s = s + mx4_val(A, SA, rows[p], K, k) * mx4_val(Bt, SB, cols[p], K, k);",
                                     "s = s + mx4_val(A, SA, cols[p], K, k) * mx4_val(Bt, SB, rows[p], K, k);"),
    "mx4_points_b_nibble_inverted": ("s = s + mx4_val(A, SA, rows[p], K, k) * mx4_val(Bt, SB, cols[p], K, k);",
                                     "s = s + mx4_val(A, SA, rows[p], K, k) * mx4_val(Bt, SB, cols[p], K, k ^ 1);"),
    "mx_last_block_dropped": ("for (int64_t k = 0; k < K; ++k)\n                s = s + mx_val(fmt_a, A, SA, i, K, k)",
                              "for (int64_t k = 0; k < K - 32; ++k)\n                s = s + mx_val(fmt_a, A, SA, i, K, k)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = oracle.SRC.read_text()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique/present"
    msrc = tmp_path / "oracle_mutant.c"
    msrc.write_text(src.replace(old, new))
    lib = oracle.build(src=msrc, out=tmp_path / "liboracle_mutant.so")
    o = oracle.Oracle(lib)
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(o)
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught mutant {name}"
