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
#include <type_traits>

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

// Buffer descriptor over [base, base + bytes): loads past the end read as
// zero, stores past it are dropped (bytes <= 0 gives an empty range).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, long long bytes)
{
    const int n = bytes <= 0 ? 0 : (bytes > 0x7fffffffLL ? 0x7fffffff : (int)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, n, 0x00020000);
}

// ---------------------------------------------------------------------------
// Large-tile kernel with direct global->LDS loads (the gfx950 path).
// 256 x 256 workgroup tile, 64-deep k-stages, two LDS buffers, four
// wavefronts of 128 x 128 (16 MFMA 32x32x16 blocks, 256 accumulators).
//
// * Loads: buffer_load_dwordx4 ... lds.  One instruction moves 64 lanes x 16
//   bytes into 1 KB of LDS, lane p landing at byte 16 p of the block; which
//   16-byte chunk of the matrix lane p fetches is free, so the LDS layout is
//   chosen by permuting the lanes' sources.  A lane whose offset is out of
//   range writes zeros, which zero-fills every edge without a branch.
// * LDS layout, in 16-byte units (8 halves):
//     A tile (256 m x 64 k, 8 units per row):   unit c of row r sits at
//       8 r + (c ^ ((r >> 1) & 7));
//     B tile (64 k x 256 n, 32 units per row, row-major as in memory): unit u
//       of row k sits at 32 k + (u ^ (4 (k & 3))).
//   A fragments are 128-bit reads of 16 consecutive rows at one unit; B
//   fragments are transposing reads (ds_read_b64_tr_b16): in each group of 16
//   lanes, source lane s points at 4 halves of row kb + s/4, columns
//   nb + 4 (s % 4), and output lane i receives rows kb..kb+3 of column nb + i,
//   so two reads give a lane eight consecutive k of its column.  With these
//   swizzles every 256-byte LDS cycle of either read touches each bank once.
// * Ordering: on this chip a wavefront's LDS reads wait for its own earlier
//   global->LDS loads to land.  So each stage starts (after the barrier that
//   publishes it) by issuing all 32 fragment reads of the stage, then the
//   loads of the next stage into the other buffer, then the 64 MFMAs; the
//   next LDS read comes a full stage of MFMAs later, by when the loads have
//   landed.
namespace dma {
constexpr int BM = 256, BN = 256, BK = 64;
constexpr int A_BYTES = BM * BK * 2;                 // 32 KB
constexpr int B_BYTES = BK * BN * 2;                 // 32 KB
constexpr int STAGE_BYTES = A_BYTES + B_BYTES;       // 64 KB
constexpr int LDS_BYTES = 2 * STAGE_BYTES;
}  // namespace dma

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

__device__ __forceinline__ void load_to_lds(__amdgpu_buffer_rsrc_t r, uint8_t *lds_block,
                                            uint32_t voff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)lds_block, 16, voff, 0, 0, 0);
}

__global__ __launch_bounds__(256) void mfma_f16_dma_kernel(
    int M, int N, int K, const uint16_t *__restrict__ A, const uint16_t *__restrict__ B,
    float *__restrict__ C, int tiles_m, int tiles_n, int group_m)
{
    using namespace dma;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[LDS_BYTES];

    int tm, tn;
    dgor_tile_of_block(blockIdx.x, tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = (wave >> 1) * 128, wc = (wave & 1) * 128;
    const int l32 = lane & 31, g = lane >> 5;
    constexpr uint32_t OOB = 0x80000000u;

    // ---- loader: wave w fills A blocks 8w..8w+7 (8 rows each) and B blocks
    // 8w..8w+7 (2 rows each); per lane, offsets relative to the stage base.
    uint32_t a_off[8], b_off[8];
    int a_c[8], b_k[8];
    bool a_row_ok[8], b_col_ok[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int blk = 8 * wave + q;
        const int r = 8 * blk + (lane >> 3);                     // A row in the tile
        const int c = (lane & 7) ^ ((r >> 1) & 7);               // its logical unit
        a_c[q] = c;
        a_row_ok[q] = m0 + r < M;
        a_off[q] = (uint32_t)(r * K + 8 * c) * 2u;
        const int k = 2 * blk + (lane >> 5);                     // B row in the tile
        const int u = (lane & 31) ^ (4 * (k & 3));               // its logical unit
        b_k[q] = k;
        b_col_ok[q] = n0 + 8 * u < N;
        b_off[q] = (uint32_t)(k * N + 8 * u) * 2u;
    }
    auto issue = [&](int stage) {
        const int k0 = stage * BK;
        uint8_t *base = lds + (stage & 1) * STAGE_BYTES;
        const __amdgpu_buffer_rsrc_t ra =
            make_rsrc(A + (size_t)m0 * K + k0, ((long long)(M - m0) * K - k0) * 2);
        const __amdgpu_buffer_rsrc_t rb =
            make_rsrc(B + (size_t)k0 * N + n0, ((long long)(K - k0) * N - n0) * 2);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const bool ok = a_row_ok[q] && k0 + 8 * a_c[q] < K;
            load_to_lds(ra, base + (8 * wave + q) * 1024, ok ? a_off[q] : OOB);
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const bool ok = b_col_ok[q] && k0 + b_k[q] < K;
            load_to_lds(rb, base + A_BYTES + (8 * wave + q) * 1024, ok ? b_off[q] : OOB);
        }
    };

    // ---- fragment readers (per k-step s = 0..3 of a stage)
    const int a_swz = (l32 >> 1) & 7;
    const uint32_t a_lane = (uint32_t)(8 * (wr + l32)) * 16u;
    uint32_t a_unit[4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
        a_unit[s] = (uint32_t)((2 * s + g) ^ a_swz) * 16u;
    const int sl = lane & 15, grp = lane >> 4;
    const uint32_t b_lane = (uint32_t)(512 * (8 * (grp >> 1) + (sl >> 2)) + 8 * (sl & 1));
    uint32_t b_unit[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int u = (wc >> 3) + 4 * j + 2 * (grp & 1) + ((sl & 3) >> 1);
        b_unit[j] = (uint32_t)(u ^ (4 * (sl >> 2))) * 16u;
    }

    halfx8 fa[4][4], fb[4][4];   // [k-step][block]
    auto fread = [&](int stage) {
        const uint8_t *base = lds + (stage & 1) * STAGE_BYTES;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                fa[s][i] = *reinterpret_cast<const halfx8 *>(base + a_lane + a_unit[s] + i * 32 * 128);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint8_t *bp = base + A_BYTES + b_lane + b_unit[j] + 512 * 16 * s;
                const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4 *)(bp));
                const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4 *)(bp + 512 * 4));
                fb[s][j] = __builtin_bit_cast(halfx8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            }
        }
    };

    floatx16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[i][j][r] = 0.f;

    const int steps = (K + BK - 1) / BK;
    issue(0);
    for (int t = 0; t < steps; ++t) {
        // this wave's loads of stage t are the only ones outstanding
        __builtin_amdgcn_s_waitcnt((0) | (7 << 4) | (15 << 8));   // vmcnt(0)
        __syncthreads();   // everyone's loads of stage t landed; stage t-1 fully read
        fread(t);
        if (t + 1 < steps)
            issue(t + 1);  // into the buffer of stage t-1, read by no one any more
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[s][i], fb[s][j], acc[i][j], 0, 0, 0);
    }

    // Epilogue: buffer stores; an element outside C gets an out-of-range lane
    // offset, so it is dropped.
    const int col = n0 + wc + l32;
    const int rows_left = M - m0 - wr - 4 * g;
    const __amdgpu_buffer_rsrc_t rc =
        make_rsrc(C + (size_t)(m0 + wr) * N + n0 + wc, ((long long)(M - m0 - wr) * N - n0 - wc) * 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t cv = (col + 32 * j < N) ? (uint32_t)((4 * g) * N + l32 + 32 * j) * 4u : OOB;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int ro = 32 * i + 8 * (r >> 2) + (r & 3);
                const float v = acc[i][j][r];
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rc, ro < rows_left ? cv : OOB,
                                                      (uint32_t)(ro * N) * 4u, 0);
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
    if (plan.tile_m == 256 && plan.tile_n == 256) {
        if (p.vec_a && p.vec_b && p.K <= (1 << 22) && p.N <= (1 << 22)) {
            hipLaunchKernelGGL(mfma_f16_dma_kernel, dim3(plan.grid_x * plan.grid_y), dim3(256), 0, s,
                               p.M, p.N, p.K, (const uint16_t *)p.A, (const uint16_t *)p.B, p.C,
                               plan.grid_y, plan.grid_x, 4);
            return hipGetLastError();
        }
        return launch_cfg<256, 256, 32, 2, 2>(p, plan, s);
    }
    if (plan.tile_m == 128 && plan.tile_n == 128)
        return launch_cfg<128, 128, 32, 2, 2>(p, plan, s);
    if (plan.tile_m == 64 && plan.tile_n == 64)
        return launch_cfg<64, 64, 32, 1, 2>(p, plan, s);
    return hipErrorInvalidValue;
}

}  // namespace dgor
