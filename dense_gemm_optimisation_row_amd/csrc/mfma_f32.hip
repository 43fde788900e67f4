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
#include "lds_dma.h"

namespace dgor {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

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

// ---------------------------------------------------------------------------
// Large FP32 tile (16-byte aligned operands, at least one 256 x 256 tile per
// compute unit): 256 x 256 workgroup tile, 16-deep k-stages in a ring of four
// LDS buffers, four wavefronts of 128 x 128 (4 x 4 blocks of 32 x 32, 256
// accumulators per lane).  The structure is that of the FP16 ring kernel:
// direct global->LDS loads issued from assembly, one vmcnt wait and one
// barrier per stage, the reads of stage t + 1 and the loads of stage t + 3
// spread between the 128 MFMAs of stage t.
// * LDS layout of one stage, in 16-byte units (4 floats):
//     A (256 m x 16 k, 4 units per row): unit c of row r at 4 r + (c ^ ((r >> 2) & 3));
//     B (16 k x 256 n, 64 units per row): unit u of row k at 64 k + (u ^ (8 ((k >> 2) & 1))).
//   For k-slice q (8 deep) of a stage, lane l reads with one 128-bit read the
//   four A values k = 8q + 4 (l / 32) + 0..3 of its row, and with four 32-bit
//   reads the B values of the same four k in its column; 32 lanes read 32
//   rows at one unit (A) or 32 columns of one row (B), and the swizzles keep
//   both on distinct banks.
namespace f32ring {
constexpr int BM = 256, BN = 256, BK = 16, NBUF = 4;
constexpr int A_BYTES = BM * BK * 4;                 // 16 KB
constexpr int B_BYTES = BK * BN * 4;                 // 16 KB
constexpr int STAGE_BYTES = A_BYTES + B_BYTES;       // 32 KB
constexpr int LDS_BYTES = NBUF * STAGE_BYTES;        // 128 KB
constexpr int LOADS_PER_STAGE = 8;                   // per wavefront: 4 of A, 4 of B
}  // namespace f32ring

__global__ __launch_bounds__(256) void mfma_f32_ring_kernel(
    int M, int N, int K, const float *__restrict__ A, const float *__restrict__ B,
    float *__restrict__ C, int tiles_m, int tiles_n, int group_m)
{
    using namespace f32ring;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[LDS_BYTES];
    const uint32_t ring = lds_address(lds);

    int tm, tn;
    dgor_tile_of_block(blockIdx.x, tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int lane = threadIdx.x & 63;
    // wave-uniform, so per-wave offsets and descriptors stay scalar
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int wr = (wave >> 1) * 128, wc = (wave & 1) * 128;
    constexpr uint32_t OOB = 0x80000000u;

    // ---- loader.  Per stage, wavefront w fills A blocks 4w..4w+3 (16 rows
    // each) and B blocks 4w..4w+3 (one k row of 256 floats each).  Lane
    // offsets are relative to the stage's first element; columns past N get
    // OOB.  The descriptor ranges end at the last row of A and at row K of B;
    // A columns past K are masked per lane in the last stage; a stage past
    // the last one gets empty ranges, so its loads write zeros.
    const int a_c = (lane & 3) ^ ((lane >> 4) & 3);   // logical unit; same in every block
    uint32_t a_off[4], b_off[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int r = 16 * (4 * wave + q) + (lane >> 2);
        a_off[q] = (uint32_t)(r * K + 4 * a_c) * 4u;
        const int k = 4 * wave + q;
        const int u = lane ^ (8 * ((k >> 2) & 1));
        b_off[q] = n0 + 4 * u < N ? (uint32_t)(k * N + 4 * u) * 4u : OOB;
    }
    const bool a_full = m0 + BM <= M;
    const uint32_t a_rows_bytes = (uint32_t)(M - m0) * (uint32_t)K * 4u;   // < 2^31 when !a_full
    const uint32_t lds_a = ring + (uint32_t)(4 * wave * 1024);
    const uint32_t lds_b = ring + (uint32_t)(A_BYTES + 4 * wave * 1024);
    struct StageLoads { intx4 ra, rb; uint32_t lds; bool a_tail; int k_left; };
    auto prep = [&](int st) {
        StageLoads L;
        const int k0 = st * BK;
        const int k_left = K - k0;
        L.ra = rsrc_words(A + (size_t)m0 * K + k0, 0);
        L.ra.z = k_left <= 0 ? 0 : (a_full ? 0x7fffffff : (int)(a_rows_bytes - (uint32_t)k0 * 4u));
        L.rb = rsrc_words(B + (size_t)k0 * N + n0, 0);
        L.rb.z = k_left >= BK ? 0x7fffffff
                              : (k_left <= 0 ? 0 : (int)(((uint32_t)k_left * (uint32_t)N - (uint32_t)n0) * 4u));
        L.lds = (uint32_t)((st % NBUF) * STAGE_BYTES);
        L.a_tail = k_left < BK;
        L.k_left = k_left;
        return L;
    };
    auto load = [&](const StageLoads &L, int q) {
        if (q < 4) {
            const uint32_t off = (L.a_tail && 4 * a_c >= L.k_left) ? OOB : a_off[q];
            load_to_lds(L.ra, lds_a + L.lds + (uint32_t)(q * 1024), off);
        } else {
            load_to_lds(L.rb, lds_b + L.lds + (uint32_t)((q - 4) * 1024), b_off[q - 4]);
        }
    };

    // ---- fragment reads.  Lane (g, l32) = (lane / 32, lane % 32).
    const int l32 = lane & 31, g = lane >> 5;
    const uint32_t a_lane = (uint32_t)((wr + l32) * 64);
    const int a_sw = (l32 >> 2) & 3;
    // B value (k-slice q, sub-step j', block j): row 8q + 4g + j', unit
    // (wc + 32 j + l32) / 4 ^ 8g, float l32 % 4 of the unit
    const uint32_t b_lane = (uint32_t)(A_BYTES + (4 * g) * 1024 + 4 * (l32 & 3));
    uint32_t b_unit[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        b_unit[j] = (uint32_t)((((wc + 32 * j + l32) >> 2) ^ (8 * g)) * 16);

    // read r (0..39) of stage `stage`: k-slice r / 20; within it the four A
    // blocks, then the B values in the order the MFMAs use them (sub-step
    // j' outer, block j inner)
    auto fread = [&](int stage, int r, floatx4 *fa, float *fb) {
        const uint8_t *buf = lds + (stage % NBUF) * STAGE_BYTES;
        const int q = r / 20, x = r % 20;
        if (x < 4) {
            fa[4 * q + x] = *reinterpret_cast<const floatx4 *>(
                buf + a_lane + x * 32 * 64 + (((2 * q + g) ^ a_sw) * 16));
        } else {
            const int jp = (x - 4) >> 2, j = (x - 4) & 3;
            fb[16 * q + 4 * jp + j] =
                *reinterpret_cast<const float *>(buf + b_lane + (8 * q + jp) * 1024 + b_unit[j]);
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

    // One stage: the 128 MFMAs of stage t from (ca, cb); the 40 reads of
    // stage t + 1 into (na, nb), one after each of the first 40 MFMAs; the 8
    // loads of stage t + 3, one after every eleventh MFMA from the 44th.
    const int steps = (K + BK - 1) / BK;
    auto stage = [&](int t, floatx4 *ca, float *cb, floatx4 *na, float *nb) {
        __builtin_amdgcn_s_waitcnt(wait_vmcnt(LOADS_PER_STAGE));
        __builtin_amdgcn_s_barrier();
        const StageLoads L = prep(t + 3);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < 128; ++m) {
            const int q = m >> 6, jp = (m >> 4) & 3, i = (m >> 2) & 3, j = m & 3;
            const floatx4 av = ca[4 * q + i];
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[jp], cb[16 * q + 4 * jp + j], acc[i][j], 0, 0, 0);
            if (m < 40)
                fread(t + 1, m, na, nb);
            if (m >= 44 && (m - 44) % 11 == 0 && (m - 44) / 11 < 8)
                load(L, (m - 44) / 11);
            // keep this order: the compiler would otherwise cluster the reads
            // and loads, and move MFMAs across the barrier
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // prologue: loads of stages 0, 1, 2, then the reads of stage 0
    floatx4 fa0[8], fa1[8];
    float fb0[32], fb1[32];
#pragma unroll
    for (int st = 0; st < 3; ++st) {
        const StageLoads L = prep(st);
#pragma unroll
        for (int q = 0; q < 8; ++q)
            load(L, q);
    }
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(2 * LOADS_PER_STAGE));
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int r = 0; r < 40; ++r)
        fread(0, r, fa0, fb0);

    for (int t = 0; t < steps; t += 2) {
        stage(t, fa0, fb0, fa1, fb1);
        if (t + 1 < steps)
            stage(t + 1, fa1, fb1, fa0, fb0);
    }
    // no load may still be writing this workgroup's LDS when it ends
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));

    // Epilogue: buffer stores; an element outside C gets an out-of-range lane
    // offset and is dropped.  Lane (g, l32) holds rows 8 (r / 4) + 4 g + r % 4.
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
    if (plan.tile_m == kF32RingTile) {   // the planner chose it only where f32_ring_applies
        if (!f32_ring_applies(p.M, p.N, p.K, p.vec_a, p.vec_b))
            return hipErrorInvalidValue;
        hipLaunchKernelGGL(mfma_f32_ring_kernel, dim3(plan.grid_x * plan.grid_y), dim3(256), 0, s,
                           p.M, p.N, p.K, (const float *)p.A, (const float *)p.B, p.C,
                           plan.grid_y, plan.grid_x, 4);
        return hipGetLastError();
    }
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
