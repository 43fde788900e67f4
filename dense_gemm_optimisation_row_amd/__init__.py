"""MI355X (gfx950) dense row-major GEMM: C = A x B with FP32 accumulation.

The computation runs in hand-written HIP kernels behind the C ABI of
``include/gemm.h`` (``libdgor_gemm.so``, built by ``build.py``); this package
only marshals torch tensors into it (``binding``).  The shared library is
loaded on first use, and every entry point raises if it is missing.
"""
from .binding import (  # noqa: F401
    AUTO, BF16_VARIANTS, EIGHT_BIT_VARIANTS, F16_VARIANTS, F32_VARIANTS, GEMM_OP_N, GEMM_OP_T,
    GemmError, R0_NAIVE, R1_LDS_TILED, R8_MFMA_8BIT,
    R2_VECTOR_LOADS, R3_LDS_PADDED, R4_DOUBLE_BUFFER, R5_REGISTER_BLOCKED, R6_MFMA_F32,
    R7_MFMA_F16, gemm_bf16_f32acc, gemm_bf16_f32acc_ex, gemm_bf16_f32acc_variant,
    gemm_f16_f32acc, gemm_f16_f32acc_ex, gemm_f16_f32acc_variant, gemm_f32, gemm_f32_ex,
    gemm_f32_variant, gemm_e4m3_f32acc, gemm_e4m3_f32acc_variant, gemm_e5m2_f32acc,
    gemm_e5m2_f32acc_variant, gemm_i8_i32acc, gemm_i8_i32acc_variant, kind_of, plan, status_string,
    CONV_IM2COL, CONV_IMPLICIT, CONV_IMPLICIT_NHWC, conv2d, conv2d_algorithm, conv2d_workspace, conv_params,
    variant_name,
)
