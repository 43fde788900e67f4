// The vector-ALU rungs R0..R5 of the FP32 path, the binary16 naive kernel and
// the K = 0 zero fill.  Each rung adds one idea from the pages on top of the
// previous one; they exist to be measured against each other and against the
// matrix-core kernels, and every one computes the same C = A x B.
//
// All kernels: row-major A (M x K), B (K x N), C (M x N); 64-bit offsets;
// every load outside the matrix reads as 0 and every store outside C is
// skipped ("Lesson 8: how a GPU does matrix multiply", section 26).
#include "common.h"

namespace dgor {
namespace {

// ---------------------------------------------------------------- helpers --

// Four consecutive floats of row r, starting at column c, of a rows x cols
// row-major matrix; elements outside the matrix read as 0.  VEC means every
// row starts 16-byte aligned and cols % 4 == 0, so a vector either lies fully
// inside or fully outside and one 128-bit load serves.
template <bool VEC>
__device__ __forceinline__ float4 load4(const float *__restrict__ p, int rows, int cols,
                                        int r, int c)
{
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (r < rows) {
        const float *q = p + (size_t)r * cols + c;
        if (VEC) {
            if (c < cols)
                v = *reinterpret_cast<const float4 *>(q);
        } else {
            if (c + 0 < cols) v.x = q[0];
            if (c + 1 < cols) v.y = q[1];
            if (c + 2 < cols) v.z = q[2];
            if (c + 3 < cols) v.w = q[3];
        }
    }
    return v;
}

__device__ __forceinline__ float load1(const float *__restrict__ p, int rows, int cols,
                                       int r, int c)
{
    return (r < rows && c < cols) ? p[(size_t)r * cols + c] : 0.f;
}

// --------------------------------------------------------------- K = 0 ---

__global__ __launch_bounds__(256) void zero_fill(float *__restrict__ C, size_t n)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        C[i] = 0.f;
}

// C = s C on an M x N block with row stride ldc (s == 0: zeros, C unread).
__global__ __launch_bounds__(256) void scale_c(float *__restrict__ C, int M, int N, int ldc, float s)
{
    // rows blockIdx.y, blockIdx.y + gridDim.y, ...; 1024 columns per block
    for (int row = blockIdx.y; row < M; row += gridDim.y) {
        float *c = C + (size_t)row * ldc;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int col = blockIdx.x * 1024 + u * 256 + threadIdx.x;
            if (col < N)
                c[col] = s == 0.f ? 0.f : s * c[col];
        }
    }
}

// The strided plain kernel for any operand layout and input format: one
// thread per element, the k-sum in FP32 in ascending k, then
// C = alpha sum + beta C (C read only when beta != 0).  A is M x K (lda) or,
// with TA, K x M; B is K x N (ldb) or, with TB, N x K.
__device__ __forceinline__ float widen16(uint16_t h, bool bf16)
{
    return bf16 ? __uint_as_float((uint32_t)h << 16) : (float)__builtin_bit_cast(_Float16, h);
}

__device__ __forceinline__ float widen_in(const void *p, size_t idx, int in16)
{
    if (in16 == 0)
        return ((const float *)p)[idx];
    const uint16_t h = ((const uint16_t *)p)[idx];
    return widen16(h, in16 == 2);
}

template <bool TA, bool TB>
__global__ __launch_bounds__(256) void naive_ex(int M, int N, int K, const void *A, int lda, const void *B,
                                                int ldb, float *C, int ldc, float alpha, float beta, int in16)
{
    const int row = blockIdx.y * 16 + threadIdx.y;
    const int col = blockIdx.x * 16 + threadIdx.x;
    if (row < M && col < N) {
        float sum = 0.f;
        for (int k = 0; k < K; ++k) {
            const float a = widen_in(A, TA ? (size_t)k * lda + row : (size_t)row * lda + k, in16);
            const float b = widen_in(B, TB ? (size_t)col * ldb + k : (size_t)k * ldb + col, in16);
            sum = fmaf(a, b, sum);
        }
        float *c = C + (size_t)row * ldc + col;
        const float v = alpha * sum;
        *c = beta == 0.f ? v : fmaf(beta, *c, v);
    }
}

// The plain kernel for 8-bit inputs: one thread per element, the k-sum in
// ascending k, FP32 for the FP8 formats (the products of two FP8 values are
// exact in FP32) and INT32 for INT8 (exact).  The FP8 codes are decoded here
// from the OCP definitions: E4M3 has 4 exponent bits (bias 7) and 3 fraction
// bits, E5M2 5 exponent bits (bias 15) and 2 fraction bits; exponent 0 is
// subnormal.  Inputs are finite by contract.
__device__ __forceinline__ float fp8_value(uint32_t b, int fmt)
{
    const bool e4 = fmt == kFmtE4M3;
    const uint32_t man_bits = e4 ? 3u : 2u;
    const int bias = e4 ? 7 : 15;
    const uint32_t expo = (b & 0x7fu) >> man_bits;
    const uint32_t frac = b & ((1u << man_bits) - 1u);
    const float mag = expo ? ldexpf((float)(frac + (1u << man_bits)), (int)expo - bias - (int)man_bits)
                           : ldexpf((float)frac, 1 - bias - (int)man_bits);
    return (b & 0x80u) ? -mag : mag;
}

template <int FMT>
__global__ __launch_bounds__(256) void naive_8bit(int M, int N, int K, const uint8_t *__restrict__ A,
                                                  const uint8_t *__restrict__ B, float *__restrict__ C)
{
    const int row = blockIdx.y * 16 + threadIdx.y;
    const int col = blockIdx.x * 16 + threadIdx.x;
    if (row < M && col < N) {
        if (FMT == kFmtI8) {
            int sum = 0;
            for (int k = 0; k < K; ++k)
                sum += (int)(int8_t)A[(size_t)row * K + k] * (int)(int8_t)B[(size_t)k * N + col];
            reinterpret_cast<int *>(C)[(size_t)row * N + col] = sum;
        } else {
            float sum = 0.f;
            for (int k = 0; k < K; ++k)
                sum = fmaf(fp8_value(A[(size_t)row * K + k], FMT), fp8_value(B[(size_t)k * N + col], FMT), sum);
            C[(size_t)row * N + col] = sum;
        }
    }
}

// ------------------------------------------------------------- R0 naive ---
// One thread per element of C, 16 x 16 threads per workgroup, the k-sum held
// in a register and C written once ("4. GEMM optimisation", 4.1; Lesson 8
// sections 3 and 4).  Neighbouring threads read neighbouring B columns, but
// every thread walks its own A row and B column straight from HBM.
__global__ __launch_bounds__(256) void naive_f32(int M, int N, int K,
                                                 const float *__restrict__ A,
                                                 const float *__restrict__ B,
                                                 float *__restrict__ C)
{
    const int row = blockIdx.y * 16 + threadIdx.y;
    const int col = blockIdx.x * 16 + threadIdx.x;
    if (row < M && col < N) {
        const float *a = A + (size_t)row * K;
        const float *b = B + col;
        float sum = 0.f;
        for (int k = 0; k < K; ++k)
            sum = fmaf(a[k], b[(size_t)k * N], sum);
        C[(size_t)row * N + col] = sum;
    }
}

// 16-bit operands (binary16 or bfloat16 bit patterns), FP32 accumulation:
// each product of two 16-bit values is exact in FP32, so this computes the
// same sum as the 16-bit matrix-core kernels.  A bfloat16 pattern is the high
// half of the binary32 with the same value.

template <bool BF16>
__global__ __launch_bounds__(256) void naive_16(int M, int N, int K,
                                                const uint16_t *__restrict__ A,
                                                const uint16_t *__restrict__ B,
                                                float *__restrict__ C)
{
    const int row = blockIdx.y * 16 + threadIdx.y;
    const int col = blockIdx.x * 16 + threadIdx.x;
    if (row < M && col < N) {
        const uint16_t *a = A + (size_t)row * K;
        const uint16_t *b = B + col;
        float sum = 0.f;
        for (int k = 0; k < K; ++k)
            sum = fmaf(widen16(a[k], BF16), widen16(b[(size_t)k * N], BF16), sum);
        C[(size_t)row * N + col] = sum;
    }
}

// ------------------------------------------------------ R1 LDS 16 x 16 ---
// Each 16 x 16 workgroup stages a 16 x 16 tile of A and of B in LDS per
// k-step; the first barrier publishes the tile, the second keeps it alive
// until every thread has used it (Lesson 8 sections 10 to 12).
__global__ __launch_bounds__(256) void lds16_f32(int M, int N, int K,
                                                 const float *__restrict__ A,
                                                 const float *__restrict__ B,
                                                 float *__restrict__ C)
{
    __shared__ float As[16][16];
    __shared__ float Bs[16][16];
    const int tx = threadIdx.x, ty = threadIdx.y;
    const int row = blockIdx.y * 16 + ty;
    const int col = blockIdx.x * 16 + tx;
    float sum = 0.f;
    const int steps = (K + 15) / 16;
    for (int t = 0; t < steps; ++t) {
        As[ty][tx] = load1(A, M, K, row, t * 16 + tx);
        Bs[ty][tx] = load1(B, K, N, t * 16 + ty, col);
        __syncthreads();
#pragma unroll
        for (int k = 0; k < 16; ++k)
            sum = fmaf(As[ty][k], Bs[k][tx], sum);
        __syncthreads();
    }
    if (row < M && col < N)
        C[(size_t)row * N + col] = sum;
}

// ------------------------------------------- R2 / R3 / R4: 16 x 16 x 64 ---
// Output tile 16 x 16 (one element per thread) with a 64-deep k-stage, so
// that every thread moves exactly one 128-bit vector of A and one of B per
// stage ("4. GEMM optimisation", 4.3: four floats per load).
//   R2: PAD = 0, one LDS stage, two barriers per step.
//   R3: padded LDS rows (PAD_A extra floats per A row, PAD_B per B row) so
//       that the 4 distinct A rows one wavefront reads at the same k fall in
//       different banks (Lesson 8 section 27; SGEMM journey Level 3).
//   R4: R3 with two LDS stages: the next stage is fetched into registers
//       while the current one is consumed, then written to the other buffer;
//       one barrier per step (Lesson 8 section 24; SGEMM journey Level 4).
template <bool VEC_A, bool VEC_B, int PAD_A, int PAD_B, int STAGES>
__global__ __launch_bounds__(256) void vec16_f32(int M, int N, int K,
                                                 const float *__restrict__ A,
                                                 const float *__restrict__ B,
                                                 float *__restrict__ C)
{
    constexpr int BK = 64;
    __shared__ float As[STAGES][16][BK + PAD_A];
    __shared__ float Bs[STAGES][BK][16 + PAD_B];
    const int tid = threadIdx.y * 16 + threadIdx.x;
    const int m0 = blockIdx.y * 16, n0 = blockIdx.x * 16;
    // loader coordinates: A is 16 rows x 16 vectors, B is 64 rows x 4 vectors
    const int ar = tid >> 4, ac = (tid & 15) * 4;
    const int br = tid >> 2, bc = (tid & 3) * 4;
    const int tx = threadIdx.x, ty = threadIdx.y;
    const int steps = (K + BK - 1) / BK;
    float sum = 0.f;

    auto store = [&](int buf, const float4 &ra, const float4 &rb) {
        As[buf][ar][ac + 0] = ra.x; As[buf][ar][ac + 1] = ra.y;
        As[buf][ar][ac + 2] = ra.z; As[buf][ar][ac + 3] = ra.w;
        Bs[buf][br][bc + 0] = rb.x; Bs[buf][br][bc + 1] = rb.y;
        Bs[buf][br][bc + 2] = rb.z; Bs[buf][br][bc + 3] = rb.w;
    };
    auto compute = [&](int buf) {
#pragma unroll
        for (int k = 0; k < BK; ++k)
            sum = fmaf(As[buf][ty][k], Bs[buf][k][tx], sum);
    };

    if (STAGES == 1) {
        // load, barrier, use, barrier: loads and arithmetic take turns
        for (int t = 0; t < steps; ++t) {
            store(0, load4<VEC_A>(A, M, K, m0 + ar, t * BK + ac),
                  load4<VEC_B>(B, K, N, t * BK + br, n0 + bc));
            __syncthreads();
            compute(0);
            __syncthreads();
        }
    } else {
        store(0, load4<VEC_A>(A, M, K, m0 + ar, ac), load4<VEC_B>(B, K, N, br, n0 + bc));
        __syncthreads();
        for (int t = 0; t < steps; ++t) {
            const int buf = t & 1;
            float4 ra, rb;
            if (t + 1 < steps) {  // fetch the next stage while this one is used
                ra = load4<VEC_A>(A, M, K, m0 + ar, (t + 1) * BK + ac);
                rb = load4<VEC_B>(B, K, N, (t + 1) * BK + br, n0 + bc);
            }
            compute(buf);
            if (t + 1 < steps) {
                // the other buffer was last read one step ago, before the
                // barrier that ended that step
                store(buf ^ 1, ra, rb);
                __syncthreads();
            }
        }
    }
    const int row = m0 + ty, col = n0 + tx;
    if (row < M && col < N)
        C[(size_t)row * N + col] = sum;
}

// ------------------------------------------- R5 register-blocked 8 x 8 ---
// 128 x 128 output tile, 8-deep k-stage, 256 threads each accumulating an
// 8 x 8 block in registers (SGEMM journey Level 5 with BM = BN = 128,
// BK = TM = TN = 8; Lesson 8 section 18).  Double-buffered, 128-bit loads.
// A is stored k-major in LDS (As[k][m]) so a thread fetches its 8 A values
// with two 128-bit LDS reads; its rows are ty*4+{0..3} and 64+ty*4+{0..3}
// and its columns tx*4+{0..3} and 64+tx*4+{0..3}, so the 16 threads of a row
// of the thread grid read 256 contiguous bytes of B.  The transposed A rows
// are padded by 8 floats so that the two k rows one wavefront writes at once
// land in opposite halves of the banks.
template <bool VEC_A, bool VEC_B, bool VEC_C>
__global__ __launch_bounds__(256) void regblock_f32(int M, int N, int K,
                                                    const float *__restrict__ A,
                                                    const float *__restrict__ B,
                                                    float *__restrict__ C)
{
    constexpr int BM = 128, BN = 128, BK = 8, PAD = kRegblockPad;
    __shared__ float As[2][BK][BM + PAD];
    __shared__ float Bs[2][BK][BN];
    const int tid = threadIdx.x;
    const int tx = tid & 15, ty = tid >> 4;
    const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
    const int ar = tid >> 1, ac = (tid & 1) * 4;   // A: 128 rows x 2 vectors
    const int br = tid >> 5, bc = (tid & 31) * 4;  // B: 8 rows x 32 vectors
    const int steps = (K + BK - 1) / BK;

    float acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
            acc[i][j] = 0.f;

    float4 ra = load4<VEC_A>(A, M, K, m0 + ar, ac);
    float4 rb = load4<VEC_B>(B, K, N, br, n0 + bc);
    As[0][ac + 0][ar] = ra.x; As[0][ac + 1][ar] = ra.y;
    As[0][ac + 2][ar] = ra.z; As[0][ac + 3][ar] = ra.w;
    *reinterpret_cast<float4 *>(&Bs[0][br][bc]) = rb;
    __syncthreads();

    for (int t = 0; t < steps; ++t) {
        const int buf = t & 1;
        if (t + 1 < steps) {
            ra = load4<VEC_A>(A, M, K, m0 + ar, (t + 1) * BK + ac);
            rb = load4<VEC_B>(B, K, N, (t + 1) * BK + br, n0 + bc);
        }
#pragma unroll
        for (int k = 0; k < BK; ++k) {
            const float4 a0 = *reinterpret_cast<const float4 *>(&As[buf][k][ty * 4]);
            const float4 a1 = *reinterpret_cast<const float4 *>(&As[buf][k][64 + ty * 4]);
            const float4 b0 = *reinterpret_cast<const float4 *>(&Bs[buf][k][tx * 4]);
            const float4 b1 = *reinterpret_cast<const float4 *>(&Bs[buf][k][64 + tx * 4]);
            const float a[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
            const float b[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
        if (t + 1 < steps) {
            const int nb = buf ^ 1;
            As[nb][ac + 0][ar] = ra.x; As[nb][ac + 1][ar] = ra.y;
            As[nb][ac + 2][ar] = ra.z; As[nb][ac + 3][ar] = ra.w;
            *reinterpret_cast<float4 *>(&Bs[nb][br][bc]) = rb;
            __syncthreads();
        }
    }

#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = m0 + (i < 4 ? ty * 4 + i : 64 + ty * 4 + (i - 4));
        if (row >= M)
            continue;
        float *crow = C + (size_t)row * N;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int col = n0 + h * 64 + tx * 4;
            const float4 v = make_float4(acc[i][h * 4 + 0], acc[i][h * 4 + 1],
                                         acc[i][h * 4 + 2], acc[i][h * 4 + 3]);
            if (VEC_C) {
                if (col < N)
                    *reinterpret_cast<float4 *>(crow + col) = v;
            } else {
                if (col + 0 < N) crow[col + 0] = v.x;
                if (col + 1 < N) crow[col + 1] = v.y;
                if (col + 2 < N) crow[col + 2] = v.z;
                if (col + 3 < N) crow[col + 3] = v.w;
            }
        }
    }
}

}  // namespace

// ------------------------------------------------------------- launchers --

hipError_t launch_scale_c(float *C, int M, int N, int ldc, float s, hipStream_t stream)
{
    const unsigned gx = (unsigned)((N + 1023) / 1024);
    const unsigned gy = (unsigned)(M < 8192 ? M : 8192);
    hipLaunchKernelGGL(scale_c, dim3(gx, gy), dim3(256), 0, stream, C, M, N, ldc, s);
    return hipGetLastError();
}

hipError_t launch_naive_ex(const RingArgs &a, float alpha, float beta, int in16, hipStream_t stream)
{
    const dim3 grid((a.N + 15) / 16, (a.M + 15) / 16), blk(16, 16);
    if (a.trans_a && a.trans_b)
        hipLaunchKernelGGL((naive_ex<true, true>), grid, blk, 0, stream, a.M, a.N, a.K, a.A, a.lda, a.B, a.ldb,
                           a.C, a.ldc, alpha, beta, in16);
    else if (a.trans_a)
        hipLaunchKernelGGL((naive_ex<true, false>), grid, blk, 0, stream, a.M, a.N, a.K, a.A, a.lda, a.B, a.ldb,
                           a.C, a.ldc, alpha, beta, in16);
    else if (a.trans_b)
        hipLaunchKernelGGL((naive_ex<false, true>), grid, blk, 0, stream, a.M, a.N, a.K, a.A, a.lda, a.B, a.ldb,
                           a.C, a.ldc, alpha, beta, in16);
    else
        hipLaunchKernelGGL((naive_ex<false, false>), grid, blk, 0, stream, a.M, a.N, a.K, a.A, a.lda, a.B, a.ldb,
                           a.C, a.ldc, alpha, beta, in16);
    return hipGetLastError();
}

hipError_t launch_naive_8bit(const Problem &p, int fmt, hipStream_t stream)
{
    const dim3 grid((p.N + 15) / 16, (p.M + 15) / 16), blk(16, 16);
    const uint8_t *A = (const uint8_t *)p.A, *B = (const uint8_t *)p.B;
    if (fmt == kFmtE4M3)
        hipLaunchKernelGGL(naive_8bit<kFmtE4M3>, grid, blk, 0, stream, p.M, p.N, p.K, A, B, p.C);
    else if (fmt == kFmtE5M2)
        hipLaunchKernelGGL(naive_8bit<kFmtE5M2>, grid, blk, 0, stream, p.M, p.N, p.K, A, B, p.C);
    else
        hipLaunchKernelGGL(naive_8bit<kFmtI8>, grid, blk, 0, stream, p.M, p.N, p.K, A, B, p.C);
    return hipGetLastError();
}

hipError_t launch_zero_fill(const Problem &p, hipStream_t stream)
{
    const size_t n = (size_t)p.M * p.N;
    const size_t blocks = (n + 255) / 256;
    const unsigned grid = (unsigned)(blocks < 65536 ? blocks : 65536);
    hipLaunchKernelGGL(zero_fill, dim3(grid), dim3(256), 0, stream, p.C, n);
    return hipGetLastError();
}

hipError_t launch_naive_f16(const Problem &p, const gemm_plan &plan, hipStream_t stream, bool bf16)
{
    const uint16_t *A = (const uint16_t *)p.A, *B = (const uint16_t *)p.B;
    if (bf16)
        hipLaunchKernelGGL(naive_16<true>, dim3(plan.grid_x, plan.grid_y), dim3(16, 16), 0, stream,
                           p.M, p.N, p.K, A, B, p.C);
    else
        hipLaunchKernelGGL(naive_16<false>, dim3(plan.grid_x, plan.grid_y), dim3(16, 16), 0, stream,
                           p.M, p.N, p.K, A, B, p.C);
    return hipGetLastError();
}

namespace {
template <int PA, int PB, int ST>
void launch_vec16(const Problem &p, dim3 grid, hipStream_t s)
{
    const float *A = (const float *)p.A, *B = (const float *)p.B;
    const dim3 blk(16, 16);
    if (p.vec_a && p.vec_b)
        hipLaunchKernelGGL((vec16_f32<true, true, PA, PB, ST>), grid, blk, 0, s, p.M, p.N, p.K, A, B, p.C);
    else if (p.vec_a)
        hipLaunchKernelGGL((vec16_f32<true, false, PA, PB, ST>), grid, blk, 0, s, p.M, p.N, p.K, A, B, p.C);
    else if (p.vec_b)
        hipLaunchKernelGGL((vec16_f32<false, true, PA, PB, ST>), grid, blk, 0, s, p.M, p.N, p.K, A, B, p.C);
    else
        hipLaunchKernelGGL((vec16_f32<false, false, PA, PB, ST>), grid, blk, 0, s, p.M, p.N, p.K, A, B, p.C);
}

template <bool VA, bool VB>
void launch_regblock_c(const Problem &p, dim3 grid, hipStream_t s)
{
    const float *A = (const float *)p.A, *B = (const float *)p.B;
    if (p.vec_c)
        hipLaunchKernelGGL((regblock_f32<VA, VB, true>), grid, dim3(256), 0, s, p.M, p.N, p.K, A, B, p.C);
    else
        hipLaunchKernelGGL((regblock_f32<VA, VB, false>), grid, dim3(256), 0, s, p.M, p.N, p.K, A, B, p.C);
}
}  // namespace

hipError_t launch_ladder_f32(const Problem &p, const gemm_plan &plan, hipStream_t s)
{
    const float *A = (const float *)p.A, *B = (const float *)p.B;
    const dim3 grid(plan.grid_x, plan.grid_y);
    switch (plan.variant) {
    case GEMM_R0_NAIVE:
        hipLaunchKernelGGL(naive_f32, grid, dim3(16, 16), 0, s, p.M, p.N, p.K, A, B, p.C);
        break;
    case GEMM_R1_LDS_TILED:
        hipLaunchKernelGGL(lds16_f32, grid, dim3(16, 16), 0, s, p.M, p.N, p.K, A, B, p.C);
        break;
    case GEMM_R2_VECTOR_LOADS:
        launch_vec16<0, 0, 1>(p, grid, s);
        break;
    case GEMM_R3_LDS_PADDED:
        launch_vec16<kLadderPadA, kLadderPadB, 1>(p, grid, s);
        break;
    case GEMM_R4_DOUBLE_BUFFER:
        launch_vec16<kLadderPadA, kLadderPadB, 2>(p, grid, s);
        break;
    case GEMM_R5_REGISTER_BLOCKED:
        if (p.vec_a && p.vec_b) launch_regblock_c<true, true>(p, grid, s);
        else if (p.vec_a) launch_regblock_c<true, false>(p, grid, s);
        else if (p.vec_b) launch_regblock_c<false, true>(p, grid, s);
        else launch_regblock_c<false, false>(p, grid, s);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace dgor
