// R7: binary16-input GEMM with FP32 accumulation on the CDNA4 matrix cores
// (v_mfma_f32_32x32x16_f16): half operands, float accumulator, as in the
// "SGEMM optimisation journey", Level 6, but with row-major B and fragments
// staged through LDS ("Lesson 8: how a GPU does matrix multiply", sections
// 19, 21, 23 and 24).  Every product of two halves is exact in FP32; only
// the FP32 accumulation rounds.
//
// Operand layout of v_mfma_f32_32x32x16_f16 (wave64): lane l supplies eight
// halves A[l % 32][8*(l/32) + 0..7] and B[8*(l/32) + 0..7][l % 32] and holds
// 16 accumulators C[8*(r/4) + 4*(l/32) + r%4][l % 32], r = 0..15.
//
// A is row-major, so a lane's eight A halves are 16 contiguous bytes of one
// LDS row: one 128-bit read.  B is row-major too (N contiguous), but a lane
// needs eight k values of one column, and each 32-bit register holds two
// consecutive k.  So B is stored in LDS as "k-pair rows": row p holds, for
// every column n, the 32-bit word (B[2p][n], B[2p+1][n]).  The words are
// built in registers from two 128-bit global loads of rows 2p and 2p+1 while
// staging, and a lane then fetches its fragment with four 32-bit reads of
// consecutive pair rows, 32 lanes reading 32 consecutive columns each.
#include "common.h"

namespace dgor {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));

// Eight halves of row r from column c of a rows x cols row-major binary16
// matrix, zero outside it.  VEC: rows start 16-byte aligned and cols % 8 == 0.
template <bool VEC>
__device__ __forceinline__ uint4 load8h(const uint16_t *__restrict__ p, int rows, int cols,
                                        int r, int c)
{
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (r < rows) {
        const uint16_t *q = p + (size_t)r * cols + c;
        if (VEC) {
            if (c < cols)
                v = *reinterpret_cast<const uint4 *>(q);
        } else {
            uint32_t h[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                h[e] = (c + e < cols) ? (uint32_t)q[e] : 0u;
            v.x = h[0] | (h[1] << 16);
            v.y = h[2] | (h[3] << 16);
            v.z = h[4] | (h[5] << 16);
            v.w = h[6] | (h[7] << 16);
        }
    }
    return v;
}

// Interleave two rows of eight halves (x: row 2p, y: row 2p+1, columns
// n..n+7) into eight k-pair words for columns n..n+7.
__device__ __forceinline__ void pair_words(const uint4 &x, const uint4 &y, uint4 &lo, uint4 &hi)
{
    lo.x = (x.x & 0xffffu) | (y.x << 16);
    lo.y = (x.x >> 16) | (y.x & 0xffff0000u);
    lo.z = (x.y & 0xffffu) | (y.y << 16);
    lo.w = (x.y >> 16) | (y.y & 0xffff0000u);
    hi.x = (x.z & 0xffffu) | (y.z << 16);
    hi.y = (x.z >> 16) | (y.z & 0xffff0000u);
    hi.z = (x.w & 0xffffu) | (y.w << 16);
    hi.w = (x.w >> 16) | (y.w & 0xffff0000u);
}

// BM x BN workgroup tile, BK-deep k-stages, WM x WN wavefronts each owning a
// (BM/WM) x (BN/WN) tile of 32 x 32 MFMA blocks.  A rows in LDS hold BK
// halves plus kF16PadA; pair rows of B hold BN words plus kF16PadB.
template <int BM, int BN, int BK, int WM, int WN, bool VEC_A, bool VEC_B>
__global__ __launch_bounds__(64 * WM * WN) void mfma_f16_kernel(
    int M, int N, int K, const uint16_t *__restrict__ A, const uint16_t *__restrict__ B,
    float *__restrict__ C, int tiles_m, int tiles_n, int group_m)
{
    constexpr int NT = 64 * WM * WN;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    constexpr int LDA = BK + kF16PadA;       // halves
    constexpr int LDB = BN + kF16PadB;       // 32-bit words
    constexpr int A_VECS = BM * BK / 8 / NT; // 128-bit loads of A per thread
    constexpr int B_UNITS = (BK / 2) * (BN / 8) / NT;  // (pair row, 8 columns) units
    static_assert(FM * 32 == WTM && FN * 32 == WTN, "wave tile must be whole 32x32 blocks");
    static_assert(A_VECS * NT * 8 == BM * BK, "A loads must divide");
    static_assert(B_UNITS * NT * 16 == BK * BN, "B loads must divide");
    static_assert(BK % 16 == 0 && LDA % 8 == 0, "k-stage must be whole 16-wide slices");

    __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LDA];
    __shared__ __attribute__((aligned(16))) uint32_t Bp[2][(BK / 2) * LDB];

    int tm, tn;
    dgor_tile_of_block(blockIdx.x, tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = (wave / WN) * WTM, wc = (wave % WN) * WTN;
    const int l32 = lane & 31, g = lane >> 5;

    floatx16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[i][j][r] = 0.f;

    uint4 ra[A_VECS], rb0[B_UNITS], rb1[B_UNITS];
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < A_VECS; ++i) {
            const int idx = tid + i * NT;
            const int r = idx / (BK / 8), c = (idx % (BK / 8)) * 8;
            ra[i] = load8h<VEC_A>(A, M, K, m0 + r, k0 + c);
        }
#pragma unroll
        for (int i = 0; i < B_UNITS; ++i) {
            const int idx = tid + i * NT;
            const int pr = idx / (BN / 8), c = (idx % (BN / 8)) * 8;
            rb0[i] = load8h<VEC_B>(B, K, N, k0 + 2 * pr, n0 + c);
            rb1[i] = load8h<VEC_B>(B, K, N, k0 + 2 * pr + 1, n0 + c);
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < A_VECS; ++i) {
            const int idx = tid + i * NT;
            const int r = idx / (BK / 8), c = (idx % (BK / 8)) * 8;
            *reinterpret_cast<uint4 *>(&As[buf][r * LDA + c]) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < B_UNITS; ++i) {
            const int idx = tid + i * NT;
            const int pr = idx / (BN / 8), c = (idx % (BN / 8)) * 8;
            uint4 lo, hi;
            pair_words(rb0[i], rb1[i], lo, hi);
            *reinterpret_cast<uint4 *>(&Bp[buf][pr * LDB + c]) = lo;
            *reinterpret_cast<uint4 *>(&Bp[buf][pr * LDB + c + 4]) = hi;
        }
    };
    auto compute = [&](int buf) {
        const uint16_t *as = As[buf];
        const uint32_t *bp = Bp[buf];
#pragma unroll
        for (int s = 0; s < BK / 16; ++s) {
            halfx8 a[FM], b[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i)
                a[i] = *reinterpret_cast<const halfx8 *>(&as[(wr + i * 32 + l32) * LDA + 16 * s + 8 * g]);
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                uint32_t w[4];
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    w[q] = bp[(8 * s + 4 * g + q) * LDB + wc + j * 32 + l32];
                b[j] = __builtin_bit_cast(halfx8, w);
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
    };

    const int steps = (K + BK - 1) / BK;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int t = 0; t < steps; ++t) {
        const int buf = t & 1;
        if (t + 1 < steps)
            gload((t + 1) * BK);
        compute(buf);
        if (t + 1 < steps) {
            sstore(buf ^ 1);  // last read one step ago, before that step's barrier
            __syncthreads();
        }
    }

#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int col = n0 + wc + j * 32 + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wr + i * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
                if (row < M && col < N)
                    C[(size_t)row * N + col] = acc[i][j][r];
            }
        }
}

template <int BM, int BN, int BK, int WM, int WN>
hipError_t launch_cfg(const Problem &p, const gemm_plan &plan, hipStream_t s)
{
    const uint16_t *A = (const uint16_t *)p.A, *B = (const uint16_t *)p.B;
    const dim3 grid(plan.grid_x * plan.grid_y), blk(64 * WM * WN);
    const int gm = 4;
    if (p.vec_a && p.vec_b)
        hipLaunchKernelGGL((mfma_f16_kernel<BM, BN, BK, WM, WN, true, true>), grid, blk, 0, s,
                           p.M, p.N, p.K, A, B, p.C, plan.grid_y, plan.grid_x, gm);
    else if (p.vec_a)
        hipLaunchKernelGGL((mfma_f16_kernel<BM, BN, BK, WM, WN, true, false>), grid, blk, 0, s,
                           p.M, p.N, p.K, A, B, p.C, plan.grid_y, plan.grid_x, gm);
    else if (p.vec_b)
        hipLaunchKernelGGL((mfma_f16_kernel<BM, BN, BK, WM, WN, false, true>), grid, blk, 0, s,
                           p.M, p.N, p.K, A, B, p.C, plan.grid_y, plan.grid_x, gm);
    else
        hipLaunchKernelGGL((mfma_f16_kernel<BM, BN, BK, WM, WN, false, false>), grid, blk, 0, s,
                           p.M, p.N, p.K, A, B, p.C, plan.grid_y, plan.grid_x, gm);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_mfma_f16(const Problem &p, const gemm_plan &plan, hipStream_t s)
{
    if (plan.tile_m == 256 && plan.tile_n == 256)
        return launch_cfg<256, 256, 32, 2, 2>(p, plan, s);
    if (plan.tile_m == 128 && plan.tile_n == 128)
        return launch_cfg<128, 128, 32, 2, 2>(p, plan, s);
    if (plan.tile_m == 64 && plan.tile_n == 64)
        return launch_cfg<64, 64, 32, 1, 2>(p, plan, s);
    return hipErrorInvalidValue;
}

}  // namespace dgor
