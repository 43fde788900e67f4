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
    const int tid = threadIdx.x, lane = tid & 63;
    // wave-uniform, so per-wave offsets and buffer descriptors stay scalar
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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

// ---------------------------------------------------------------------------
// 128 x 128 x 16 tile with direct global->LDS loads, for 16-byte aligned rows.
// Same wavefront tiling and k-mapping as above; what changes is the supply:
// * Loads: buffer_load_dwordx4 ... lds, 1 KB of LDS per instruction (lane p
//   -> byte 16 p); the matrix chunk each lane fetches is permuted so the LDS
//   layout comes out swizzled, and a lane with an out-of-range offset writes
//   zeros, which masks every edge.  Units are 16 bytes (4 floats):
//     A tile (128 m x 16 k, 4 units per row):  unit c of row r at
//       4 r + (c ^ ((r >> 2) & 3));
//     B tile (16 k x 128 n, 32 units per row): unit u of row k at
//       32 k + (u ^ (8 ((k >> 2) & 1))).
//   A reads (128-bit, 16 consecutive rows at one unit) and B reads (32-bit,
//   32 consecutive columns of rows k and k + 4) then touch each bank once per
//   256-byte LDS cycle.
// * Order: a wavefront's LDS reads wait for its own earlier global->LDS loads,
//   so each stage issues all of its fragment reads first, then the next
//   stage's loads, then its 32 MFMAs.  Several workgroups share a compute
//   unit, so their MFMAs cover one another's waits.
namespace f32dma {
constexpr int BM = 128, BN = 128, BK = 16;
constexpr int A_BYTES = BM * BK * 4;            // 8 KB
constexpr int B_BYTES = BK * BN * 4;            // 8 KB
constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
constexpr int LDS_BYTES = 2 * STAGE_BYTES;      // 32 KB
}  // namespace f32dma

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, long long bytes)
{
    const int n = bytes <= 0 ? 0 : (bytes > 0x7fffffffLL ? 0x7fffffff : (int)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, n, 0x00020000);
}

__global__ __launch_bounds__(256) void mfma_f32_dma_kernel(
    int M, int N, int K, const float *__restrict__ A, const float *__restrict__ B,
    float *__restrict__ C, int tiles_m, int tiles_n, int group_m)
{
    using namespace f32dma;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[LDS_BYTES];

    int tm, tn;
    dgor_tile_of_block(blockIdx.x, tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int tid = threadIdx.x, lane = tid & 63;
    // wave-uniform, so per-wave offsets and buffer descriptors stay scalar
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wr = (wave >> 1) * 64, wc = (wave & 1) * 64;
    const int l32 = lane & 31, g = lane >> 5;
    constexpr uint32_t OOB = 0x80000000u;

    // loader: wave w fills A blocks 2w, 2w+1 (16 rows each) and B blocks
    // 2w, 2w+1 (2 rows each)
    uint32_t a_off[2], b_off[2];
    int a_c[2], b_k[2];
    bool a_row_ok[2], b_col_ok[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int blk = 2 * wave + q;
        const int r = 16 * blk + (lane >> 2);
        const int c = (lane & 3) ^ ((r >> 2) & 3);
        a_c[q] = c;
        a_row_ok[q] = m0 + r < M;
        a_off[q] = (uint32_t)(r * K + 4 * c) * 4u;
        const int k = 2 * blk + (lane >> 5);
        const int u = (lane & 31) ^ (8 * ((k >> 2) & 1));
        b_k[q] = k;
        b_col_ok[q] = n0 + 4 * u < N;
        b_off[q] = (uint32_t)(k * N + 4 * u) * 4u;
    }
    auto issue = [&](int stage) {
        const int k0 = stage * BK;
        uint8_t *base = lds + (stage & 1) * STAGE_BYTES;
        const __amdgpu_buffer_rsrc_t ra =
            make_rsrc(A + (size_t)m0 * K + k0, ((long long)(M - m0) * K - k0) * 4);
        const __amdgpu_buffer_rsrc_t rb =
            make_rsrc(B + (size_t)k0 * N + n0, ((long long)(K - k0) * N - n0) * 4);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const bool ok = a_row_ok[q] && k0 + 4 * a_c[q] < K;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void *)(base + (2 * wave + q) * 1024), 16,
                                                     ok ? a_off[q] : OOB, 0, 0, 0);
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const bool ok = b_col_ok[q] && k0 + b_k[q] < K;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void *)(base + A_BYTES + (2 * wave + q) * 1024),
                                                     16, ok ? b_off[q] : OOB, 0, 0, 0);
        }
    };

    // fragment addresses (bytes within a stage)
    const int a_swz = (l32 >> 2) & 3;
    const uint32_t a_lane = (uint32_t)(4 * (wr + l32)) * 16u;
    const uint32_t a_unit0 = (uint32_t)((0 + g) ^ a_swz) * 16u;   // k 0..7 of the stage
    const uint32_t a_unit1 = (uint32_t)((2 + g) ^ a_swz) * 16u;   // k 8..15
    // B value of block fn, k = 8 s + 4 g + q: row k, unit 16 (wc/64) + 8 (fn ^ g) + l32/4
    const uint32_t b_lane = (uint32_t)(512 * (4 * g) + 16 * (16 * (wc >> 6) + (l32 >> 2)) + 4 * (l32 & 3));

    float4 fa[2][2];     // [k-slice s][block fm]
    float fb[2][2][4];   // [s][fn][q]
    auto fread = [&](int stage) {
        const uint8_t *base = lds + (stage & 1) * STAGE_BYTES;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
                fa[s][i] = *reinterpret_cast<const float4 *>(base + a_lane + (s ? a_unit1 : a_unit0) + i * 32 * 64);
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    fb[s][j][q] = *reinterpret_cast<const float *>(
                        base + A_BYTES + b_lane + 512 * (8 * s + q) + 16 * 8 * (j ^ g));
        }
    };

    floatx16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[i][j][r] = 0.f;

    const int steps = (K + BK - 1) / BK;
    issue(0);
    for (int t = 0; t < steps; ++t) {
        __builtin_amdgcn_s_waitcnt((0) | (7 << 4) | (15 << 8));   // vmcnt(0): own loads of stage t
        __syncthreads();   // everyone's loads of stage t landed; stage t-1 fully read
        fread(t);
        if (t + 1 < steps)
            issue(t + 1);  // into the other buffer, read by no one any more
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const float av = q == 0 ? fa[s][i].x : q == 1 ? fa[s][i].y : q == 2 ? fa[s][i].z : fa[s][i].w;
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, fb[s][j][q], acc[i][j], 0, 0, 0);
                    }
    }

#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
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
    if (plan.tile_m == 128 && plan.tile_n == 128) {
        if (direct_lds_applies(plan.tile_m, 128, p.vec_a, p.vec_b, p.N, p.K)) {
            hipLaunchKernelGGL(mfma_f32_dma_kernel, dim3(plan.grid_x * plan.grid_y), dim3(256), 0, s,
                               p.M, p.N, p.K, (const float *)p.A, (const float *)p.B, p.C,
                               plan.grid_y, plan.grid_x, 8);
            return hipGetLastError();
        }
        return launch_cfg<128, 128, 16, 2, 2>(p, plan, s);
    }
    if (plan.tile_m == 64 && plan.tile_n == 64)
        return launch_cfg<64, 64, 16, 2, 2>(p, plan, s);
    if (plan.tile_m == 32 && plan.tile_n == 64)
        return launch_cfg<32, 64, 16, 1, 2>(p, plan, s);
    return hipErrorInvalidValue;
}

}  // namespace dgor
