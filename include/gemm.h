/*
 * gemm.h -- C ABI of the MI355X (gfx950) dense row-major GEMM library.
 *
 * Operation (all entry points): C = A x B, where
 *   A is M x K, B is K x N, C is M x N, each row-major with packed leading
 *   dimensions:  A[i*K + k],  B[k*N + j],  C[i*N + j];
 *   C[i][j] = sum over k in [0, K) of A[i][k] * B[k][j], accumulated in FP32.
 * Definition: "Lesson 8: how a GPU does matrix multiply", section 1 (element
 * formula) and section 2 (row-major index expressions); "SGEMM optimisation
 * journey", Level 1 (argument order M, N, K, A, B, C); "4. GEMM optimisation",
 * section 4.1 (shapes; C written once, not accumulated into).
 *
 * Conventions shared by every call:
 *   - A, B, C are DEVICE pointers owned by the caller.  The library allocates
 *     and frees nothing, keeps no per-call state, and never copies to the host.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *     and the call returns without waiting: the caller synchronises.
 *   - C is overwritten.  C must not overlap A or B.  Inputs must be finite.
 *   - Pointers need only natural element alignment.  16-byte alignment of a
 *     base pointer, with K (for A) or N (for B, C) a multiple of the vector
 *     width, is detected and used for 128-bit accesses; it is never required.
 *   - Dimensions are `int`; every offset is computed in 64 bits.
 *   - Edge cases: M, N or K negative -> GEMM_ERR_INVALID_DIM.  M == 0 or
 *     N == 0 -> GEMM_OK with nothing launched or written.  K == 0 -> C is set
 *     to 0.0f (an empty sum).  A NULL pointer whose extent is nonzero ->
 *     GEMM_ERR_NULL_PTR (extents: A M*K, B K*N, C M*N; checked before
 *     the M == 0 / N == 0 early return).  Nothing is launched when a status
 *     other than GEMM_OK is returned, except GEMM_ERR_LAUNCH.
 *   - Errors are returned, never printed or thrown.  A current device that is
 *     not gfx950 -> GEMM_ERR_UNSUPPORTED_DEVICE.  A failed launch ->
 *     GEMM_ERR_LAUNCH.  A failed HIP runtime query -> GEMM_ERR_RUNTIME.
 *   - Calls are thread-safe; concurrent calls on different streams are fine.
 */
#ifndef DGOR_GEMM_H
#define DGOR_GEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GEMM_OK = 0,
    GEMM_ERR_INVALID_DIM = -1,
    GEMM_ERR_NULL_PTR = -2,
    GEMM_ERR_LAUNCH = -3,
    GEMM_ERR_UNSUPPORTED_DEVICE = -4,
    GEMM_ERR_INVALID_VARIANT = -5,
    GEMM_ERR_RUNTIME = -6,
    GEMM_ERR_INVALID_LAYOUT = -7,
    GEMM_ERR_WORKSPACE = -8,
    GEMM_ERR_SCRATCH_LIMIT = -9
} gemm_status;

/*
 * Kernel variants ("rungs"), in the order the pages build them up:
 *   R0 one thread per output element            ("4. GEMM optimisation" 4.1;
 *                                                 Lesson 8 section 4)
 *   R1 16x16 LDS tiles, masked loads, two barriers (Lesson 8 section 10,
 *                                                 section 26 for the masking)
 *   R2 R1 with 128-bit global loads             ("4. GEMM optimisation" 4.3)
 *   R3 R2 with padded LDS rows                  (Lesson 8 section 27;
 *                                                 SGEMM journey Level 3)
 *   R4 R3 with two LDS stages, one barrier/step (Lesson 8 section 24;
 *                                                 SGEMM journey Level 4)
 *   R5 register-blocked 8x8 outputs per thread  (Lesson 8 section 18;
 *                                                 SGEMM journey Level 5)
 *   R6 FP32 matrix-core (MFMA) tiles             (Lesson 8 section 21)
 *   R7 16-bit-input matrix-core (MFMA) tiles,     (SGEMM journey Level 6;
 *      FP32 accumulation (binary16 or bfloat16)   Lesson 8 section 22)
 *   R8 8-bit-input matrix-core (MFMA) tiles:      (Lesson 8 section 22)
 *      FP8 with FP32, INT8 with INT32 accumulation
 * GEMM_VARIANT_AUTO lets the library choose from the shape and alignment.
 */
typedef enum {
    GEMM_VARIANT_AUTO = -1,
    GEMM_R0_NAIVE = 0,
    GEMM_R1_LDS_TILED = 1,
    GEMM_R2_VECTOR_LOADS = 2,
    GEMM_R3_LDS_PADDED = 3,
    GEMM_R4_DOUBLE_BUFFER = 4,
    GEMM_R5_REGISTER_BLOCKED = 5,
    GEMM_R6_MFMA_F32 = 6,
    GEMM_R7_MFMA_F16 = 7,
    GEMM_R8_MFMA_8BIT = 8,
    GEMM_VARIANT_COUNT = 9
} gemm_variant;

/* FP32 inputs, FP32 accumulation and output.  Chooses the fastest variant
 * for the shape (R6 in practice).  See the conventions above. */
int gemm_f32(int M, int N, int K, const float *A, const float *B, float *C,
             void *stream);

/* IEEE binary16 inputs (raw 16-bit patterns), exact products, FP32
 * accumulation and FP32 output ("SGEMM optimisation journey", Level 6: half
 * operands with a float accumulator).  Chooses R7 in practice. */
int gemm_f16_f32acc(int M, int N, int K, const uint16_t *A, const uint16_t *B,
                    float *C, void *stream);

/* bfloat16 inputs (raw 16-bit patterns: the high half of a binary32, 8
 * exponent and 7 fraction bits), exact products, FP32 accumulation and FP32
 * output -- one of the input formats "Lesson 8: how a GPU does matrix
 * multiply", section 22, lists for matrix units.  Same tiles as the binary16
 * path with the bfloat16 matrix-core instructions.  Chooses R7 in practice. */
int gemm_bf16_f32acc(int M, int N, int K, const uint16_t *A, const uint16_t *B,
                     float *C, void *stream);

/*
 * 8-bit inputs, the FP8 and INT8 formats "Lesson 8: how a GPU does matrix
 * multiply", section 22, lists for matrix units.  One byte per element,
 * row-major with packed leading dimensions as above.
 *   gemm_e4m3_f32acc: OCP FP8 E4M3 codes (4 exponent bits, bias 7, 3
 *     fraction bits, no infinities; 0x7F / 0xFF are NaN);
 *   gemm_e5m2_f32acc: OCP FP8 E5M2 codes (5 exponent bits, bias 15, 2
 *     fraction bits);
 *   both with unscaled values, exact products and FP32 accumulation and
 *   output.  The matrix cores add each group of eight products of a k-step
 *   at a fixed point aligned to the group's largest product, keeping about
 *   13 bits below it, before the FP32 accumulation: a product more than
 *   2^13 times smaller than the largest of its group is lost.
 *   gemm_i8_i32acc: signed INT8 inputs, exact INT32 accumulation and output
 *     (C is int32_t).  K above 131072 -> GEMM_ERR_INVALID_DIM, since
 *     128 * 128 * K must fit int32.
 * Calls with 16-byte aligned A and B, K and N multiples of 16, K and N
 * below 2^22 take R8 (256 x 256 x 64 tiles through a four-stage LDS ring,
 * or 128 x 128 x 64 tiles where they spread better over the compute units,
 * as the plan reports); others take R0.  Same conventions and errors as
 * gemm_f32 otherwise.
 */
int gemm_e4m3_f32acc(int M, int N, int K, const uint8_t *A, const uint8_t *B,
                     float *C, void *stream);
int gemm_e5m2_f32acc(int M, int N, int K, const uint8_t *A, const uint8_t *B,
                     float *C, void *stream);
int gemm_i8_i32acc(int M, int N, int K, const int8_t *A, const int8_t *B,
                   int32_t *C, void *stream);

/* Same operations with the variant forced (GEMM_VARIANT_AUTO allowed), for
 * benchmarking and testing every rung.  gemm_f32_variant accepts R0..R6;
 * gemm_f16_f32acc_variant and gemm_bf16_f32acc_variant accept R0 and R7;
 * the 8-bit ones accept R0 and R8 (R8 on a call its tiles cannot take runs
 * R0, which the plan reports).  Any other value -> GEMM_ERR_INVALID_VARIANT.
 * Same semantics and errors otherwise. */
int gemm_f32_variant(int variant, int M, int N, int K, const float *A,
                     const float *B, float *C, void *stream);
int gemm_f16_f32acc_variant(int variant, int M, int N, int K,
                            const uint16_t *A, const uint16_t *B, float *C,
                            void *stream);
int gemm_bf16_f32acc_variant(int variant, int M, int N, int K,
                             const uint16_t *A, const uint16_t *B, float *C,
                             void *stream);
int gemm_e4m3_f32acc_variant(int variant, int M, int N, int K,
                             const uint8_t *A, const uint8_t *B, float *C,
                             void *stream);
int gemm_e5m2_f32acc_variant(int variant, int M, int N, int K,
                             const uint8_t *A, const uint8_t *B, float *C,
                             void *stream);
int gemm_i8_i32acc_variant(int variant, int M, int N, int K, const int8_t *A,
                           const int8_t *B, int32_t *C, void *stream);

/*
 * Launch plan: what a call with these arguments would launch.  Pure host
 * arithmetic (no device is touched), so it can be queried without a GPU.
 * Pointers are used only for their alignment; they are never dereferenced.
 * `variant` may be GEMM_VARIANT_AUTO.  Fills *plan and returns GEMM_OK, or
 * returns GEMM_ERR_INVALID_DIM / GEMM_ERR_INVALID_VARIANT /
 * GEMM_ERR_NULL_PTR (plan == NULL).  For M == 0 or N == 0 the plan has
 * launches == 0; for K == 0 it describes the zero-fill launch.
 */
typedef struct {
    int variant;        /* rung that runs (a gemm_variant value) */
    int launches;       /* kernels enqueued: 0 or 1 */
    int tile_m;         /* output rows per workgroup */
    int tile_n;         /* output columns per workgroup */
    int tile_k;         /* k extent of one LDS stage (0 for R0 / zero-fill) */
    int threads;        /* threads per workgroup */
    int grid_x;         /* workgroups along N */
    int grid_y;         /* workgroups along M */
    int k_stages;       /* ceil(K / tile_k): k-stages of one workgroup */
    int lds_stages;     /* LDS k-stages in flight (1, 2, or a ring of 4) */
    int lds_bytes;      /* LDS per workgroup, padding included */
    int tile_bytes;     /* bytes of one unpadded A tile plus one B tile */
    int outputs_per_thread; /* C elements each thread accumulates (over its
                               group's share of k, where a workgroup runs
                               two groups of wavefronts over halves of k) */
    int vector_a;       /* 1 if A is read with 128-bit loads */
    int vector_b;       /* 1 if B is read with 128-bit loads */
    int vector_c;       /* 1 if C is written with 128-bit stores */
} gemm_plan;

int gemm_f32_plan(int variant, int M, int N, int K, const float *A,
                  const float *B, const float *C, gemm_plan *plan);
int gemm_f16_f32acc_plan(int variant, int M, int N, int K, const uint16_t *A,
                         const uint16_t *B, const float *C, gemm_plan *plan);
int gemm_bf16_f32acc_plan(int variant, int M, int N, int K, const uint16_t *A,
                          const uint16_t *B, const float *C, gemm_plan *plan);
int gemm_e4m3_f32acc_plan(int variant, int M, int N, int K, const uint8_t *A,
                          const uint8_t *B, const float *C, gemm_plan *plan);
int gemm_e5m2_f32acc_plan(int variant, int M, int N, int K, const uint8_t *A,
                          const uint8_t *B, const float *C, gemm_plan *plan);
int gemm_i8_i32acc_plan(int variant, int M, int N, int K, const int8_t *A,
                        const int8_t *B, const int32_t *C, gemm_plan *plan);

/*
 * General operand layouts and scaling, the interface "Lesson 8: how a GPU
 * does matrix multiply", section 28, describes libraries exposing (with the
 * D = A x B + C of its section 21):
 *     C = alpha * op(A) * op(B) + beta * C,   op(A) M x K, op(B) K x N,
 * where op(X) is X (GEMM_OP_N) or its transpose (GEMM_OP_T), all matrices
 * row-major with the given leading dimensions (row strides, in elements):
 *     opA N: A is M x K, A[i*lda + k], lda >= K;  opA T: A is K x M, lda >= M;
 *     opB N: B is K x N, B[k*ldb + j], ldb >= N;  opB T: B is N x K, ldb >= K;
 *     C is M x N, C[i*ldc + j], ldc >= N.
 * Products are exact and summed in FP32 as in the plain entry points.  When
 * beta == 0, C is not read (it may hold anything); when K == 0 or alpha == 0,
 * A and B are not used and C = beta * C.
 * Calls with 16-byte aligned A and B, leading dimensions (and the
 * dimension read along rows of a transposed operand) in whole 16-byte
 * vectors take the 256 x 256 ring kernels; C = alpha A B + beta C is then
 * formed from C = A B or C += A B and separate scaling passes over C
 * (alpha != 1 and beta != 0 together: C *= beta / alpha first, C *= alpha
 * last, so the beta C term may differ from the one-step value by a few
 * units in its last place).  Other calls take a plain kernel that forms
 * alpha * sum + beta * C directly.  The plain row-major case (N, N,
 * lda = K, ldb = ldc = N, alpha 1, beta 0) is exactly gemm_f32 /
 * gemm_f16_f32acc / gemm_bf16_f32acc.
 * Errors as for those, plus GEMM_ERR_INVALID_LAYOUT for an op flag other
 * than GEMM_OP_N / GEMM_OP_T or a leading dimension below its minimum
 * (checked before anything else but negative dimensions).
 */
typedef enum { GEMM_OP_N = 0, GEMM_OP_T = 1 } gemm_op;

int gemm_f32_ex(int opA, int opB, int M, int N, int K, float alpha,
                const float *A, int lda, const float *B, int ldb, float beta,
                float *C, int ldc, void *stream);
int gemm_f16_f32acc_ex(int opA, int opB, int M, int N, int K, float alpha,
                       const uint16_t *A, int lda, const uint16_t *B, int ldb,
                       float beta, float *C, int ldc, void *stream);
int gemm_bf16_f32acc_ex(int opA, int opB, int M, int N, int K, float alpha,
                        const uint16_t *A, int lda, const uint16_t *B, int ldb,
                        float beta, float *C, int ldc, void *stream);

/*
 * Two-dimensional convolution as matrix multiplication (through im2col and
 * one GEMM, or an implicit GEMM that forms no im2col matrix) -- the operator
 * "Lesson 8: how a GPU does matrix multiply" names as the next lesson
 * (convolution as matrix multiplication; input feature maps, weights and
 * output feature maps; direct convolution against im2col).  As deep-learning
 * frameworks define it (a cross-correlation), all tensors row-major:
 *   x: N x C x H x W (NCHW), w: K x C x R x S, y: N x K x P x Q,
 *   P = (H + 2 pad_h - dilation_h (R - 1) - 1) / stride_h + 1, Q likewise,
 *   y[n][k][p][q] = sum over c, r, s of
 *       x[n][c][p stride_h - pad_h + r dilation_h][q stride_w - pad_w + s dilation_w]
 *       * w[k][c][r][s],  input positions outside the image contributing 0.
 * Products are exact and summed in FP32 by the GEMM kernels (16-bit inputs:
 * FP32 accumulation and output, as gemm_f16_f32acc / gemm_bf16_f32acc).
 * 16-bit layers with C a multiple of 32, filters of at most 64 taps (R S)
 * and at least 96 tiles (64 filters x 256 output pixels when K <= 64, else
 * 128 filters x 64 pixels) take an
 * implicit GEMM on a channels-last copy of x: one pass writes that copy
 * (N x (H + 2 pad_h) x (W + 2 pad_w) x C, zeros in the border) and the
 * weights reordered to K x R x S x C; the GEMM kernel then sums each output
 * over r, s, c (c fastest) and writes y.  The workspace holds the reordered
 * weights and then the copy, each starting on a 256-byte boundary.
 * Other 16-bit layers with at least 256 tiles of 128 filters x 256 output pixels
 * (ceil(K / 128) * ceil(N P Q / 256) >= 256) take an implicit GEMM that
 * gathers the patches from x straight into on-chip memory, sums each output
 * over c, r, s in 32-deep steps and writes y.  The padded weights are used
 * only when C R S is not a multiple of 8 or w is not 16-byte aligned; with
 * stride_w 1 and Q a multiple of 4 the kernel first writes a zero-padded copy
 * of x (N x C x (H + 2 pad_h) x (W + 2 pad_w rounded up to a multiple of 8))
 * that the gather reads with wide loads; the workspace then holds only the
 * padded weights and that copy.  gemm_conv2d_algorithm reports the path.
 * The library allocates nothing: the caller passes a device workspace of at
 * least the size gemm_conv2d_workspace reports.  On the im2col path it holds
 * the padded weights (K x CRSp), the im2col matrix (CRSp x NPQp) and the GEMM
 * result (K x NPQp, FP32), where CRS = C R S and NPQ = N P Q are rounded up
 * to multiples of 8.  When K >= 192 and CRSp >= 64 the GEMM is split over k into chunks of
 * a multiple of 64 (at least 64) until its 256 x 256 tiles times the splits
 * reach 256, and the workspace holds one FP32 result per split; the output
 * pass adds them in split order.  Errors: negative sizes, R, S, strides or dilations below
 * 1, negative padding, an empty output (P or Q below 1), or sizes whose
 * products overflow int -> GEMM_ERR_INVALID_DIM; NULL params or a NULL
 * tensor with nonzero extent -> GEMM_ERR_NULL_PTR; a workspace that is NULL,
 * not 256-byte aligned, or too small -> GEMM_ERR_WORKSPACE; otherwise as
 * gemm_f32.  N == 0 or
 * K == 0 writes nothing; C == 0 writes zeros.  Work is enqueued on `stream`;
 * the workspace must not be reused until it completes.
 */
typedef struct {
    int N, C, H, W;            /* input: N images, C channels, H x W pixels */
    int K, R, S;               /* K filters of C x R x S */
    int stride_h, stride_w;    /* >= 1 */
    int pad_h, pad_w;          /* >= 0, zero padding on each side */
    int dilation_h, dilation_w;/* >= 1 */
} gemm_conv2d_params;

/* Workspace bytes for a convolution with these parameters and input element
 * size (4 for gemm_conv2d_f32, 2 for the 16-bit forms), in *bytes.  Host
 * arithmetic only.  Errors as the convolution entry points. */
int gemm_conv2d_workspace(const gemm_conv2d_params *params, int input_bytes, size_t *bytes);

/* Which path a convolution with these parameters and input element size
 * takes, in *algorithm: GEMM_CONV_IM2COL (im2col matrix, then the GEMM
 * kernels), GEMM_CONV_IMPLICIT (the implicit GEMM gathering from x; 16-bit
 * inputs only) or GEMM_CONV_IMPLICIT_NHWC (the implicit GEMM on a
 * channels-last copy of x; 16-bit inputs with C a multiple of 32).  Host
 * arithmetic only.  Errors as gemm_conv2d_workspace. */
typedef enum { GEMM_CONV_IM2COL = 0, GEMM_CONV_IMPLICIT = 1, GEMM_CONV_IMPLICIT_NHWC = 2 } gemm_conv_algorithm;
int gemm_conv2d_algorithm(const gemm_conv2d_params *params, int input_bytes, int *algorithm);

int gemm_conv2d_f32(const gemm_conv2d_params *params, const float *x, const float *w, float *y,
                    void *workspace, size_t workspace_bytes, void *stream);
int gemm_conv2d_f16_f32acc(const gemm_conv2d_params *params, const uint16_t *x, const uint16_t *w,
                           float *y, void *workspace, size_t workspace_bytes, void *stream);
int gemm_conv2d_bf16_f32acc(const gemm_conv2d_params *params, const uint16_t *x, const uint16_t *w,
                            float *y, void *workspace, size_t workspace_bytes, void *stream);

/* gemm_conv2d_f16_f32acc without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  The workspace is a fixed 16 MiB
 * array inside the library (one per GPU, held from the library's load on
 * that GPU until the process ends); the call allocates nothing and launches
 * the same kernels as gemm_conv2d_f16_f32acc, so y is bit for bit the same.
 * A layer whose gemm_conv2d_workspace size (input_bytes 2) exceeds 16 MiB ->
 * GEMM_ERR_SCRATCH_LIMIT, with nothing launched; its first call on a device
 * looks up that device's array (a failure -> GEMM_ERR_RUNTIME); other errors
 * as gemm_conv2d_f16_f32acc.  Every call on one GPU uses that GPU's one
 * array and leaves its contents behind (each call writes all it reads):
 * calls that overlap on one GPU -- on different streams, or from different
 * threads without ordering -- race on it. */
int gemm_conv2d_f16_f32acc_noalloc(const gemm_conv2d_params *params, const uint16_t *x, const uint16_t *w,
                                   float *y, void *stream);

/* Static, NUL-terminated descriptions; never NULL ("unknown ..." for values
 * outside the enums). */
const char *gemm_status_string(int status);
const char *gemm_variant_name(int variant);

#ifdef __cplusplus
}
#endif

#endif /* DGOR_GEMM_H */
