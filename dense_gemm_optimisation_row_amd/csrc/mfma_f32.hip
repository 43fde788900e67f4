// R6: FP32 GEMM on the CDNA4 matrix cores (v_mfma_f32_32x32x2_f32).
//
// The multi-level tiling of "Lesson 8: how a GPU does matrix multiply",
// section 19 (workgroup tile -> wavefront tile -> per-lane fragments) with the
// matrix-multiply-accumulate unit of section 21 doing the arithmetic, fed
// from LDS tiles that are double-buffered (section 24), padded (section 27)
// and loaded with 128-bit coalesced reads (section 15; "4. GEMM
// optimisation", 4.3).  Edges are zero-filled on load and masked on store
// (section 26).
//
// Operand layout of v_mfma_f32_32x32x2_f32 (wave64): lane l supplies
// A[l % 32][l / 32] and B[l / 32][l % 32] of a 32x2 by 2x32 product and holds
// 16 accumulators C[8*(r/4) + 4*(l/32) + r%4][l % 32], r = 0..15.
// Which k a lane's "k index" stands for is free as long as A and B agree, so
// for four consecutive instructions j = 0..3 lane l uses k = 4*(l/32) + j of
// an 8-wide k slice: its four A values are then contiguous in an A row and
// come from one 128-bit LDS read, and its four B values are one column of
// four consecutive B rows (four 32-bit reads, 32 lanes per row).
#include "common.h"

namespace dgor {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));

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

// BM x BN workgroup tile, BK-deep k-stages, WM x WN wavefronts each owning a
// (BM/WM) x (BN/WN) tile made of 32 x 32 MFMA blocks.  LDS rows are padded:
// A rows (BK floats) by 4 floats, so 16 lanes reading 16 consecutive rows at
// the same k hit 16 distinct groups of 4 banks; B rows (BN floats) by 8
// floats, so the two B rows one 32-bit read touches (k and k + 4) sit in
// opposite halves of the banks.
template <int BM, int BN, int BK, int WM, int WN, bool VEC_A, bool VEC_B>
__global__ __launch_bounds__(64 * WM * WN) void mfma_f32_kernel(
    int M, int N, int K, const float *__restrict__ A, const float *__restrict__ B,
    float *__restrict__ C, int tiles_m, int tiles_n, int group_m)
{
    constexpr int NT = 64 * WM * WN;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    constexpr int LDA = BK + kF32PadA;
    constexpr int LDB = BN + kF32PadB;
    constexpr int A_VECS = BM * BK / 4 / NT;
    constexpr int B_VECS = BK * BN / 4 / NT;
    static_assert(FM * 32 == WTM && FN * 32 == WTN, "wave tile must be whole 32x32 blocks");
    static_assert(A_VECS * NT * 4 == BM * BK && B_VECS * NT * 4 == BK * BN, "loads must divide");
    static_assert(BK % 8 == 0, "k-stage must be whole 8-wide slices");

    __shared__ __attribute__((aligned(16))) float As[2][BM * LDA];
    __shared__ __attribute__((aligned(16))) float Bs[2][BK * LDB];

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

    float4 ra[A_VECS], rb[B_VECS];
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < A_VECS; ++i) {
            const int idx = tid + i * NT;
            const int r = idx / (BK / 4), c = (idx % (BK / 4)) * 4;
            ra[i] = load4<VEC_A>(A, M, K, m0 + r, k0 + c);
        }
#pragma unroll
        for (int i = 0; i < B_VECS; ++i) {
            const int idx = tid + i * NT;
            const int r = idx / (BN / 4), c = (idx % (BN / 4)) * 4;
            rb[i] = load4<VEC_B>(B, K, N, k0 + r, n0 + c);
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < A_VECS; ++i) {
            const int idx = tid + i * NT;
            const int r = idx / (BK / 4), c = (idx % (BK / 4)) * 4;
            *reinterpret_cast<float4 *>(&As[buf][r * LDA + c]) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < B_VECS; ++i) {
            const int idx = tid + i * NT;
            const int r = idx / (BN / 4), c = (idx % (BN / 4)) * 4;
            *reinterpret_cast<float4 *>(&Bs[buf][r * LDB + c]) = rb[i];
        }
    };
    auto compute = [&](int buf) {
        const float *as = As[buf];
        const float *bs = Bs[buf];
#pragma unroll
        for (int kk = 0; kk < BK; kk += 8) {
            float4 a[FM];
            float b[FN][4];
#pragma unroll
            for (int i = 0; i < FM; ++i)
                a[i] = *reinterpret_cast<const float4 *>(&as[(wr + i * 32 + l32) * LDA + kk + 4 * g]);
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    b[j][q] = bs[(kk + 4 * g + q) * LDB + wc + j * 32 + l32];
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j) {
                        const float av = q == 0 ? a[i].x : q == 1 ? a[i].y : q == 2 ? a[i].z : a[i].w;
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, b[j][q], acc[i][j], 0, 0, 0);
                    }
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
    const float *A = (const float *)p.A, *B = (const float *)p.B;
    const dim3 grid(plan.grid_x * plan.grid_y), blk(64 * WM * WN);
    const int gm = 8;
    if (p.vec_a && p.vec_b)
        hipLaunchKernelGGL((mfma_f32_kernel<BM, BN, BK, WM, WN, true, true>), grid, blk, 0, s,
                           p.M, p.N, p.K, A, B, p.C, plan.grid_y, plan.grid_x, gm);
    else if (p.vec_a)
        hipLaunchKernelGGL((mfma_f32_kernel<BM, BN, BK, WM, WN, true, false>), grid, blk, 0, s,
                           p.M, p.N, p.K, A, B, p.C, plan.grid_y, plan.grid_x, gm);
    else if (p.vec_b)
        hipLaunchKernelGGL((mfma_f32_kernel<BM, BN, BK, WM, WN, false, true>), grid, blk, 0, s,
                           p.M, p.N, p.K, A, B, p.C, plan.grid_y, plan.grid_x, gm);
    else
        hipLaunchKernelGGL((mfma_f32_kernel<BM, BN, BK, WM, WN, false, false>), grid, blk, 0, s,
                           p.M, p.N, p.K, A, B, p.C, plan.grid_y, plan.grid_x, gm);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_mfma_f32(const Problem &p, const gemm_plan &plan, hipStream_t s)
{
    if (plan.tile_m == 128 && plan.tile_n == 128)
        return launch_cfg<128, 128, 16, 2, 2>(p, plan, s);
    if (plan.tile_m == 64 && plan.tile_n == 64)
        return launch_cfg<64, 64, 16, 2, 2>(p, plan, s);
    if (plan.tile_m == 32 && plan.tile_n == 64)
        return launch_cfg<32, 64, 16, 1, 2>(p, plan, s);
    return hipErrorInvalidValue;
}

}  // namespace dgor
