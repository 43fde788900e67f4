"""The oracle's pins are discriminating: plant a plausible mistake in a copy of
oracle.c (on the CPU, in a temporary directory), load that copy in place of
the oracle, and check that at least one pin of ``test_oracle.py`` fails.

Each mutant is a one-token slip of the kind a hand-written loop nest invites:
a dropped term, a wrong sign, a transposed operand, a wrong index, a start
value other than zero, binary32 accumulation, a misdecoded binary16 or
bfloat16 field, an ignored leading dimension or scale factor, a second
rounding, a misdecoded FP8 field, a sign or width slip in the INT8 sum, or
a convolution index slip (filter axes, dilation, padding, stride, channel).
"""
import ctypes
import shutil
import subprocess

import pytest

import oracle
import test_oracle as pins

MUTANTS = {
    # f32 routine
    "f32_drops_last_term": ("for (int k = 0; k < K; ++k) {\n                const double a = (double)A",
                            "for (int k = 0; k < K - 1; ++k) {\n                const double a = (double)A"),
    "f32_subtracts": ("acc[j] += a * (double)brow[j];", "acc[j] -= a * (double)brow[j];"),
    "f32_B_transposed": ("acc[j] += a * (double)brow[j];",
                         "acc[j] += a * (double)B[((size_t)j * K + k) % ((size_t)K * N)];"),
    "f32_A_transposed": ("const double a = (double)A[(size_t)i * K + k];",
                         "const double a = (double)A[((size_t)k * M + i) % ((size_t)M * K)];"),
    "f32_accumulates_into_C": ("for (int j = 0; j < N; ++j)\n                acc[j] = 0.0;\n            for (int k = 0; k < K; ++k) {\n                const double a = (double)A",
                               "for (int j = 0; j < N; ++j)\n                acc[j] = C[(size_t)i * N + j];\n            for (int k = 0; k < K; ++k) {\n                const double a = (double)A"),
    "f32_float_accumulator": ("double *acc = (double *)malloc((size_t)N * sizeof(double));\n        if (!acc)\n            failed = 1;\n#pragma omp for schedule(static)\n        for (int i = 0; i < M; ++i) {\n            if (!acc)\n                continue;\n            for (int j = 0; j < N; ++j)\n                acc[j] = 0.0;\n            for (int k = 0; k < K; ++k) {\n                const double a = (double)A",
                              "float *acc = (float *)malloc((size_t)N * sizeof(float));\n        if (!acc)\n            failed = 1;\n#pragma omp for schedule(static)\n        for (int i = 0; i < M; ++i) {\n            if (!acc)\n                continue;\n            for (int j = 0; j < N; ++j)\n                acc[j] = 0.0;\n            for (int k = 0; k < K; ++k) {\n                const double a = (double)A"),
    "f32_row_offset_slip": ("C[(size_t)i * N + j] = (float)acc[j];\n        }\n        free(acc);\n    }\n    return failed ? ORACLE_ERR_ALLOC : ORACLE_OK;\n}\n\n/*\n * Full product, binary16",
                            "C[(size_t)i * N + (j + 1) % N] = (float)acc[j];\n        }\n        free(acc);\n    }\n    return failed ? ORACLE_ERR_ALLOC : ORACLE_OK;\n}\n\n/*\n * Full product, binary16"),
    # f16 routine and decoder
    "f16_drops_first_term": ("for (int k = 0; k < K; ++k) {\n                const double a = dec",
                             "for (int k = 1; k < K; ++k) {\n                const double a = dec"),
    "f16_B_transposed": ("acc[j] += a * dec[brow[j]];",
                         "acc[j] += a * dec[B[((size_t)j * K + k) % ((size_t)K * N)]];"),
    "f16_subnormal_scale": ("v = ldexp((double)frac, -24);", "v = ldexp((double)frac, -25);"),
    "f16_exponent_bias": ("v = ldexp((double)(1024 + frac), expo - 25);",
                          "v = ldexp((double)(1024 + frac), expo - 24);"),
    "f16_hidden_bit": ("v = ldexp((double)(1024 + frac), expo - 25);",
                       "v = ldexp((double)(frac), expo - 15);"),
    # bfloat16 routine and decoder
    "bf16_subnormal_scale": ("v = ldexp((double)frac, -133);", "v = ldexp((double)frac, -134);"),
    "bf16_exponent_bias": ("v = ldexp((double)(128 + frac), expo - 134);",
                           "v = ldexp((double)(128 + frac), expo - 133);"),
    "bf16_hidden_bit": ("v = ldexp((double)(128 + frac), expo - 134);",
                        "v = ldexp((double)(frac), expo - 127);"),
    "bf16_B_transposed": ("acc[j] += a * bdec[brow[j]];",
                          "acc[j] += a * bdec[B[((size_t)j * K + k) % ((size_t)K * N)]];"),
    "bf16_fraction_field": ("const int frac = h & 0x7f;", "const int frac = h & 0x3f;"),
    # general-layout routine
    "ex_lda_ignored": ("const size_t ia = opA ? (size_t)k * lda + i : (size_t)i * lda + k;",
                       "const size_t ia = opA ? (size_t)k * M + i : (size_t)i * lda + k;"),
    "ex_ldb_ignored": ("const size_t ib = opB ? (size_t)j * ldb + k : (size_t)k * ldb + j;",
                       "const size_t ib = opB ? (size_t)j * ldb + k : (size_t)k * N + j;"),
    "ex_ldc_ignored": ("C[(size_t)i * ldc + j] = (float)v;", "C[(size_t)i * N + j] = (float)v;"),
    "ex_alpha_dropped": ("double v = alpha * acc;", "double v = acc;"),
    "ex_beta_as_one": ("v += beta * (double)C[(size_t)i * ldc + j];", "v += (double)C[(size_t)i * ldc + j];"),
    "ex_reads_C_when_beta_zero": ("if (beta != 0.0)\n                v += beta", "if (1)\n                v += beta"),
    "ex_rounds_sum_before_alpha": ("double v = alpha * acc;", "double v = alpha * (double)(float)acc;"),
    "ex_decoders_swapped": ("return in == 1 ? oracle_f16_to_f64(h) : oracle_bf16_to_f64(h);",
                            "return in == 2 ? oracle_f16_to_f64(h) : oracle_bf16_to_f64(h);"),
    # 8-bit routines and decoders
    "e4m3_exponent_bias": ("v = ldexp((double)(8 + frac), expo - 10);", "v = ldexp((double)(8 + frac), expo - 11);"),
    "e4m3_nan_as_number": ("else if (expo == 15 && frac == 7)\n        v = NAN;", "else if (expo == 16)\n        v = NAN;"),
    "e4m3_subnormal_scale": ("v = ldexp((double)frac, -9);", "v = ldexp((double)frac, -10);"),
    "e5m2_hidden_bit": ("v = ldexp((double)(4 + frac), expo - 17);", "v = ldexp((double)(frac), expo - 15);"),
    "e5m2_fraction_field": ("const int frac = b & 0x3;", "const int frac = b & 0x1;"),
    "fp8_B_transposed": ("acc[j] += a * dec[brow[j]];",
                         "acc[j] += a * dec[B[((size_t)j * K + k) % ((size_t)K * N)]];"),
    "i8_unsigned_A": ("const int64_t a = A[(size_t)i * K + k];", "const int64_t a = (uint8_t)A[(size_t)i * K + k];"),
    "i8_narrow_accumulator": ("int64_t *acc = (int64_t *)malloc((size_t)N * sizeof(int64_t));",
                              "int32_t *acc = (int32_t *)malloc((size_t)N * sizeof(int32_t));"),
    # convolution
    "conv_r_s_swapped": ("const size_t iw = (((size_t)k * C + c) * R + r) * S + s;",
                         "const size_t iw = (((size_t)k * C + c) * R + s % R) * S + r % S;"),
    "conv_no_row_dilation": ("const int h = p * sh - ph + r * dh, v = q * sw - pw + s * dw;",
                             "const int h = p * sh - ph + r, v = q * sw - pw + s * dw;"),
    "conv_padding_sign": ("const int h = p * sh - ph + r * dh, v = q * sw - pw + s * dw;",
                          "const int h = p * sh + ph + r * dh, v = q * sw - pw + s * dw;"),
    "conv_column_stride_ignored": ("const int h = p * sh - ph + r * dh, v = q * sw - pw + s * dw;",
                                   "const int h = p * sh - ph + r * dh, v = q - pw + s * dw;"),
    "conv_wrong_channel": ("const size_t ix = (((size_t)n * C + c) * H + h) * W + v;",
                           "const size_t ix = (((size_t)n * C + (c + 1) % C) * H + h) * W + v;"),
    # selected-element routine
    "at_wrong_column": ("* (double)B[(size_t)k * N + j];", "* (double)B[(size_t)k * N + i % N];"),
}

PINS = [
    lambda: pins.test_f16_decoder_matches_numpy_on_every_bit_pattern(),
    lambda: pins.test_f16_decoder_spot_values(),
    lambda: pins.test_identity_right_and_left(7, 13),
    lambda: pins.test_identity_right_and_left(64, 33),
    lambda: pins.test_permutation_products(5, 9, 11),
    lambda: pins.test_rank1_closed_form(6, 17, 9),
    lambda: pins.test_all_ones_gives_K(),
    lambda: pins.test_K1_is_the_correctly_rounded_product(),
    lambda: pins.test_K0_writes_zeros_and_overwrites(),
    lambda: pins.test_bruteforce_dyadic_all_shapes_up_to_6(),
    lambda: pins.test_bruteforce_final_rounding_is_round_to_nearest_even(),
    lambda: pins.test_numpy_float64_matmul_within_one_ulp(),
    lambda: pins.test_small_integer_products_are_exact(),
    lambda: pins.test_selected_elements_match_full_product_bit_for_bit(),
    lambda: pins.test_f16_product_equals_f32_product_of_the_decoded_values(),
    lambda: pins.test_f16_bruteforce_exact(),
    lambda: pins.test_f16_accepts_raw_bit_patterns_and_small_integers_are_exact(),
    lambda: pins.test_bf16_decoder_matches_torch_on_every_bit_pattern(),
    lambda: pins.test_bf16_decoder_spot_values(),
    lambda: pins.test_bf16_product_equals_f32_product_of_the_decoded_values(),
    lambda: pins.test_bf16_bruteforce_exact(),
    lambda: pins.test_bf16_small_integers_are_exact(),
    lambda: pins.test_ex_transposed_and_padded_operands_match_the_plain_product("f32"),
    lambda: pins.test_ex_transposed_and_padded_operands_match_the_plain_product("f16"),
    lambda: pins.test_ex_transposed_and_padded_operands_match_the_plain_product("bf16"),
    lambda: pins.test_ex_bruteforce_alpha_beta_single_rounding(),
    lambda: pins.test_ex_small_integers_alpha_beta_closed_form(),
    lambda: pins.test_ex_beta_zero_never_reads_C_and_K0_scales_C(),
    lambda: pins.test_ex_16bit_equals_f32_on_the_decoded_values("f16"),
    lambda: pins.test_ex_16bit_equals_f32_on_the_decoded_values("bf16"),
    lambda: pins.test_fp8_decoder_matches_torch_on_every_code("e4m3"),
    lambda: pins.test_fp8_decoder_matches_torch_on_every_code("e5m2"),
    lambda: pins.test_fp8_decoder_spot_values(),
    lambda: pins.test_fp8_product_equals_f32_product_of_the_decoded_values("e4m3"),
    lambda: pins.test_fp8_product_equals_f32_product_of_the_decoded_values("e5m2"),
    lambda: pins.test_fp8_bruteforce_exact("e4m3"),
    lambda: pins.test_fp8_bruteforce_exact("e5m2"),
    lambda: pins.test_i8_product_is_numpy_int64_product(),
    lambda: pins.test_i8_extremes_and_overflow(),
    *[(lambda c=c: pins.test_conv2d_matches_torch_float64_within_one_ulp(c)) for c in pins.CONV_CASES],
    lambda: pins.test_conv2d_one_by_one_is_the_gemm_per_image(),
    *[(lambda c=c: pins.test_conv2d_all_ones_counts_the_taps_inside_the_image(c)) for c in pins.CONV_CASES],
    *[(lambda c=c: pins.test_conv2d_single_input_pixel_picks_out_the_weights(c)) for c in pins.CONV_CASES],
    lambda: pins.test_conv2d_16bit_equals_f32_on_the_decoded_values("f16"),
    lambda: pins.test_conv2d_16bit_equals_f32_on_the_decoded_values("bf16"),
]


def _build_mutant(tmp_path, old, new):
    src = open(oracle._SRC).read()
    assert old in src, "mutation anchor not found in oracle.c"
    mutated = src.replace(old, new, 1)
    assert mutated != src
    c = tmp_path / "mutant.c"
    c.write_text(mutated)
    so = tmp_path / "libmutant.so"
    subprocess.run(["gcc", *oracle.CFLAGS, "-w", str(c), "-o", str(so), "-lm"], check=True)
    return oracle.configure(ctypes.CDLL(str(so)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path, monkeypatch):
    lib = _build_mutant(tmp_path, *MUTANTS[name])
    monkeypatch.setattr(oracle, "_lib", lib)
    caught = 0
    for pin in PINS:
        try:
            pin()
        except (AssertionError, RuntimeError, ValueError, pytest.fail.Exception):
            caught += 1
    assert caught > 0, f"no pin notices mutant {name}"


def test_unmutated_oracle_passes_every_pin():
    for pin in PINS:
        pin()
