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
// Large FP32 tile (16-byte aligned operands): 256 x 256 workgroup tile,
// 16-deep k-stages in a ring of four LDS buffers, four wavefronts of
// 128 x 128 (4 x 4 blocks of 32 x 32, 256 accumulators per lane).  The
// structure is that of the 16-bit ring kernel: direct global->LDS loads
// issued from assembly, one vmcnt wait and one barrier per stage, the reads
// of stage t + 1 and the loads of stage t + 3 spread between the 128 MFMAs
// of stage t.
// * Each operand tile is stored in one of two ways (16-byte units of 4
//   floats):
//     k-contiguous (A, or B given as N x K): 256 rows of 16 k, unit c of
//       row r at 4 r + (c ^ ((r >> 2) & 3));
//     k-strided (B, or A given as K x M): 16 k rows of 256, unit u of row k
//       at 64 k + (u ^ (8 ((k >> 2) & 1))).
//   For k-slice q (8 deep) of a stage, lane l wants, of its row of op(A) or
//   column of op(B), the four values k = 8q + 4 (l / 32) + 0..3, one per
//   MFMA of a group of four: from the k-contiguous layout that is one
//   128-bit read, from the k-strided one four 32-bit reads (32 lanes read 32
//   consecutive values of one row).  The swizzles keep both on distinct banks.
namespace f32ring {
constexpr int BM = 256, BN = 256, BK = 16, NBUF = 4;
constexpr int A_BYTES = BM * BK * 4;                 // 16 KB
constexpr int B_BYTES = BK * BN * 4;                 // 16 KB
constexpr int STAGE_BYTES = A_BYTES + B_BYTES;       // 32 KB
constexpr int LDS_BYTES = NBUF * STAGE_BYTES;        // 128 KB

// Lane offsets of wave w's LPO 1 KB loads of one operand tile per stage
// (loads LPO w .. LPO w + LPO - 1 of the stage's 16), relative to the stage's
// first element (as for the 16-bit ring).
template <bool KSTRIDED, int LPO>
__device__ __forceinline__ void load_offsets(int wave, int lane, int t0, int ext, int ld,
                                             uint32_t off[LPO], int &kc)
{
    constexpr uint32_t OOB = 0x80000000u;
#pragma unroll
    for (int q = 0; q < LPO; ++q) {
        if (!KSTRIDED) {
            const int r = 16 * (LPO * wave + q) + (lane >> 2);
            kc = 4 * ((lane & 3) ^ ((lane >> 4) & 3));   // same in every block
            off[q] = (uint32_t)(r * ld + kc) * 4u;
        } else {
            const int k = LPO * wave + q;
            const int u = lane ^ (8 * ((k >> 2) & 1));
            off[q] = t0 + 4 * u < ext ? (uint32_t)(k * ld + 4 * u) * 4u : OOB;
            kc = 0;
        }
    }
}

// Range in bytes of one stage's descriptor (first element: row t0, k0 for
// the k-contiguous layout; row k0, column t0 for the k-strided one).
template <bool KSTRIDED>
__device__ __forceinline__ int stage_range(int k0, int K, int t0, int ext, int ld)
{
    const int k_left = K - k0;
    if (k_left <= 0)
        return 0;
    if (!KSTRIDED) {
        if (t0 + 256 <= ext)
            return 0x7fffffff;
        return (int)(((uint32_t)(ext - t0 - 1) * (uint32_t)ld + (uint32_t)k_left) * 4u);
    }
    if (k_left >= 16)
        return 0x7fffffff;
    return (int)(((uint32_t)(k_left - 1) * (uint32_t)ld + (uint32_t)(ext - t0)) * 4u);
}
}  // namespace f32ring

template <bool TA, bool TB, bool ACC, int W>
__global__ __launch_bounds__(64 * W) void mfma_f32_ring_kernel(RingArgs args)
{
    const int bid = dgor_ring_split(args, 4);   // split-K: this workgroup's k-range and tile
    using namespace f32ring;
    // W wavefronts of 128 x 256 / (W / 2): BI x BJ blocks of 32 x 32 each;
    // LPO loads per operand and wavefront per stage
    constexpr int WN = W / 2, BI = 4, BJ = 8 / WN, LPO = 16 / W, LOADS_PER_STAGE = 2 * LPO;
    constexpr int MFMAS = 8 * BI * BJ;   // per stage: 2 k-slices x 4 k-steps x the blocks
    static_assert(W == 4 || W == 8, "four or eight wavefronts");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[LDS_BYTES];
    const uint32_t ring = lds_address(lds);
    const int M = args.M, N = args.N, K = args.K, lda = args.lda, ldb = args.ldb;
    const float *__restrict__ A = (const float *)args.A;
    const float *__restrict__ B = (const float *)args.B;

    int tm, tn;
    dgor_tile_of_block(bid, args.tiles_m, args.tiles_n, args.group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int lane = threadIdx.x & 63;
    // wave-uniform, so per-wave offsets and descriptors stay scalar
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int wr = (wave / WN) * 128, wc = (wave % WN) * (256 / WN);
    constexpr uint32_t OOB = 0x80000000u;

    // ---- loader (see the 16-bit ring kernel for the range rules)
    uint32_t a_off[LPO], b_off[LPO];
    int a_kc, b_kc;
    load_offsets<TA, LPO>(wave, lane, m0, M, lda, a_off, a_kc);
    load_offsets<!TB, LPO>(wave, lane, n0, N, ldb, b_off, b_kc);
    const uint32_t lds_a = ring + (uint32_t)(LPO * wave * 1024);
    const uint32_t lds_b = ring + (uint32_t)(A_BYTES + LPO * wave * 1024);
    struct StageLoads { intx4 ra, rb; uint32_t lds; bool tail; int k_left; };
    auto prep = [&](int st) {
        StageLoads L;
        const int k0 = st * BK;
        L.ra = rsrc_words(TA ? A + (size_t)k0 * lda + m0 : A + (size_t)m0 * lda + k0, 0);
        L.ra.z = stage_range<TA>(k0, K, m0, M, lda);
        L.rb = rsrc_words(TB ? B + (size_t)n0 * ldb + k0 : B + (size_t)k0 * ldb + n0, 0);
        L.rb.z = stage_range<!TB>(k0, K, n0, N, ldb);
        L.lds = (uint32_t)((st % NBUF) * STAGE_BYTES);
        L.k_left = K - k0;
        L.tail = L.k_left < BK;
        return L;
    };
    auto load = [&](const StageLoads &L, int q) {
        if (q < LPO) {
            const uint32_t off = (!TA && L.tail && a_kc >= L.k_left) ? OOB : a_off[q];
            load_to_lds(L.ra, lds_a + L.lds + (uint32_t)(q * 1024), off);
        } else {
            const uint32_t off = (TB && L.tail && b_kc >= L.k_left) ? OOB : b_off[q - LPO];
            load_to_lds(L.rb, lds_b + L.lds + (uint32_t)((q - LPO) * 1024), off);
        }
    };

    // ---- fragment reads.  Lane (g, l32) = (lane / 32, lane % 32).
    const int l32 = lane & 31, g = lane >> 5;
    const int kc_sw = (l32 >> 2) & 3;
    auto kc_lane = [&](uint32_t region, int base) { return region + (uint32_t)((base + l32) * 64); };
    auto ks_lane = [&](uint32_t region) { return region + (uint32_t)((4 * g) * 1024 + 4 * (l32 & 3)); };
    uint32_t a_unit[BI], b_unit[BJ];   // k-strided column units of each block
#pragma unroll
    for (int j = 0; j < BI; ++j)
        a_unit[j] = (uint32_t)((((wr + 32 * j + l32) >> 2) ^ (8 * g)) * 16);
#pragma unroll
    for (int j = 0; j < BJ; ++j)
        b_unit[j] = (uint32_t)((((wc + 32 * j + l32) >> 2) ^ (8 * g)) * 16);
    const uint32_t a_lane = TA ? ks_lane(0) : kc_lane(0, wr);
    const uint32_t b_lane = TB ? kc_lane(A_BYTES, wc) : ks_lane(A_BYTES);
    // One read instruction of operand X (k-slice q, block blk of nblk,
    // sub-step e of a k-strided block) into x[nblk q + blk].
    auto read_one = [&](const uint8_t *buf, uint32_t lane_off, const uint32_t *unit, bool kstrided, int nblk,
                        int q, int blk, int e, floatx4 *x) {
        if (!kstrided)
            x[nblk * q + blk] = *reinterpret_cast<const floatx4 *>(
                buf + lane_off + blk * 32 * 64 + (((2 * q + g) ^ kc_sw) * 16));
        else
            x[nblk * q + blk][e] =
                *reinterpret_cast<const float *>(buf + lane_off + (8 * q + e) * 1024 + unit[blk]);
    };
    // Read r of stage `stage`, in k-slice order; within a slice, A's reads
    // (NA per block) then B's (NB per block).
    constexpr int NA = TA ? 4 : 1, NB = TB ? 1 : 4, RPS = BI * NA + BJ * NB;
    constexpr int READS = 2 * RPS;
    static_assert(READS <= MFMAS, "one read after each of the first MFMAs");
    auto fread = [&](int stage, int r, floatx4 *fa, floatx4 *fb) {
        const uint8_t *buf = lds + (stage % NBUF) * STAGE_BYTES;
        const int q = r / RPS, x = r % RPS;
        if (x < BI * NA)
            read_one(buf, a_lane, a_unit, TA, BI, q, x / NA, x % NA, fa);
        else
            read_one(buf, b_lane, b_unit, !TB, BJ, q, (x - BI * NA) / NB, (x - BI * NA) % NB, fb);
    };

    // ---- C tile: lane (g, l32) owns rows 32 i + 8 (r / 4) + 4 g + r % 4 and
    // columns 32 j + l32 of the wave's block.
    const int ldc = args.ldc;
    const int c_col = n0 + wc + l32;
    const int c_rows_left = M - m0 - wr - 4 * g;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(
        args.C + (size_t)(m0 + wr) * ldc + n0 + wc, ((long long)(M - m0 - wr - 1) * ldc + N - n0 - wc) * 4);
    auto c_offset = [&](int col, int rows_left, int i, int j, int r, uint32_t &vo, uint32_t &so) {
        const int ro = 32 * i + 8 * (r >> 2) + (r & 3);
        vo = (ro < rows_left && col + 32 * j < N) ? (uint32_t)((4 * g) * ldc + l32 + 32 * j) * 4u : OOB;
        so = (uint32_t)(ro * ldc) * 4u;
    };

    // Accumulators start at zero, or at C itself (ACC: C = alpha (C + op(A) op(B))).
    floatx16 acc[BI][BJ];
#pragma unroll
    for (int i = 0; i < BI; ++i)
#pragma unroll
        for (int j = 0; j < BJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                if (ACC) {
                    uint32_t vo, so;
                    c_offset(c_col, c_rows_left, i, j, r, vo, so);
                    acc[i][j][r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rc, vo, so, 0));
                } else {
                    // an AGPR write, so the compiler keeps the array in AGPRs
                    asm("v_accvgpr_write_b32 %0, 0" : "=a"(acc[i][j][r]));
                }
            }

    // One stage: the MFMAS matrix instructions of stage t from (ca, cb); the
    // reads of stage t + 1 into (na, nb), one after each of the first READS
    // MFMAs; the loads of stage t + 3 spread over the second half.  The loads'
    // descriptors are set up behind the first MFMA: scalar work between the
    // barrier and the first MFMA leaves the matrix core idle.
    const int steps = (K + BK - 1) / BK;
    auto stage = [&](int t, floatx4 *ca, floatx4 *cb, floatx4 *na, floatx4 *nb) {
        __builtin_amdgcn_s_waitcnt(wait_vmcnt(LOADS_PER_STAGE));
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        StageLoads L;
#pragma unroll
        for (int m = 0; m < MFMAS; ++m) {
            const int q = m / (4 * BI * BJ), jp = (m / (BI * BJ)) & 3, i = (m / BJ) % BI, j = m % BJ;
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(ca[BI * q + i][jp], cb[BJ * q + j][jp], acc[i][j],
                                                              0, 0, 0);
            if (m == 1)
                L = prep(t + 3);
            if (m < READS)
                fread(t + 1, m, na, nb);
            constexpr int HALF = MFMAS / 2, EVERY = HALF / LOADS_PER_STAGE;
            if (m >= HALF && (m - HALF) % EVERY == 0)
                load(L, (m - HALF) / EVERY);
            // keep this order: the compiler would otherwise cluster the reads
            // and loads, and move MFMAs across the barrier
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // prologue: loads of stages 0, 1, 2, then the reads of stage 0
    floatx4 fa0[2 * BI], fa1[2 * BI], fb0[2 * BJ], fb1[2 * BJ];
#pragma unroll
    for (int st = 0; st < 3; ++st) {
        const StageLoads L = prep(st);
#pragma unroll
        for (int q = 0; q < LOADS_PER_STAGE; ++q)
            load(L, q);
    }
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(2 * LOADS_PER_STAGE));
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int r = 0; r < READS; ++r)
        fread(0, r, fa0, fb0);

    for (int t = 0; t < steps; t += 2) {
        stage(t, fa0, fb0, fa1, fb1);
        if (t + 1 < steps)
            stage(t + 1, fa1, fb1, fa0, fb0);
    }
    // no load may still be writing this workgroup's LDS when it ends
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));

    // Epilogue: write alpha times the accumulators, one at a time (see the
    // 16-bit ring kernel); offsets are recomputed from opaque copies.
    int col_e = c_col, rows_e = c_rows_left;
    asm volatile("" : "+v"(col_e), "+v"(rows_e));
    dgor_acc_hazard_wait();
#pragma unroll
    for (int j = 0; j < BJ; ++j)
#pragma unroll
        for (int i = 0; i < BI; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                uint32_t vo, so;
                c_offset(col_e, rows_e, i, j, r, vo, so);
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(dgor_acc_read(acc[i][j][r]) * args.alpha), rc,
                                                      vo, so, 0);
            }
}

template <bool TA, bool TB>
hipError_t launch_ring32_t(const RingArgs &a, hipStream_t s)
{
    const dim3 grid(a.tiles_m * a.tiles_n * (a.splits > 1 ? a.splits : 1));
    constexpr int W = kF32RingWaves;
    if (a.accumulate)
        hipLaunchKernelGGL((mfma_f32_ring_kernel<TA, TB, true, W>), grid, dim3(64 * W), 0, s, a);
    else
        hipLaunchKernelGGL((mfma_f32_ring_kernel<TA, TB, false, W>), grid, dim3(64 * W), 0, s, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Mid-size FP32 problems (16-byte aligned operands, too few 256 x 256 tiles
// to fill the chip, so 64 x 64 tiles): one workgroup per tile computes only
// about 260 K flops per 16-deep k-step, far less than one memory latency
// takes, so k-stages come through a deep ring of LDS buffers, NBUF of BK k,
// loaded straight from global memory NBUF - 1 stages ahead ("Lesson 8: how a
// GPU does matrix multiply", sections 24 and 25 on overlapping loads with
// compute, taken several stages deep).  2 WN wavefronts of 32 x 64 / WN, each
// 2 x (4 / WN) blocks of v_mfma_f32_16x16x4_f32 (lane l supplies A[l % 16][l / 16] and
// B[l / 16][l % 16] and holds C[4 (l / 16) + r][l % 16], r = 0..3); for the
// four instructions e = 0..3 of a 16-deep k-slice q, lane l takes
// k = 16 q + 4 (l / 16) + e, so its A values are one 128-bit read and its B
// values four 32-bit reads of one column.
//   A stage: 64 rows of BK floats (U = BK / 4 units of 16 bytes), unit u of
//     row r at U r + (u ^ fa(r)), fa(r) = (r U / 16) mod U: the 16 rows one
//     128-bit read cycle touches land on 16 distinct groups of 4 banks.
//   B stage: BK rows of 64 floats, unit u of row k at 16 k + (u ^ fb(k)),
//     fb(k) = 4 ((k / 4) mod 4): the four rows k, k + 4, k + 8, k + 12 that
//     one 32-bit read touches fall on four distinct quarters of the banks.
// Edges and the k tail are zero-filled through out-of-range lane offsets
// (K and N are multiples of 4, so a 16-byte unit is wholly in or out).
// Each direct load costs its wavefront some issue time in which the matrix
// core has nothing else to run; with eight wavefronts (two per SIMD, WN = 4)
// the other wavefront's MFMAs fill it, 9% faster than four at 1024^3.
// KS = 2 (shapes with at most one tile per compute unit, whose second
// workgroup slot would stay empty): sixteen wavefronts, two groups of eight,
// group g taking the g-th half of the k-stages through a ring of its own
// (128 KB in all); both groups run the same number of stages (the second's
// last one past K loads zeros), so they meet at the same barriers, and at
// the end group 1 hands its sums to group 0 through LDS, which adds them in
// that fixed order and stores C.
namespace f32small {
__host__ __device__ constexpr int fa(int r, int U) { return (r * U / 16) & (U - 1); }
__host__ __device__ constexpr int fb(int k) { return 4 * ((k >> 2) & 3); }
}  // namespace f32small

template <int BK, int NBUF, int WN, int KS>
__global__ __launch_bounds__(128 * WN * KS) void mfma_f32_small_ring_kernel(int M, int N, int K,
                                                                  const float *__restrict__ A,
                                                                  const float *__restrict__ B,
                                                                  float *__restrict__ C, int tiles_m,
                                                                  int tiles_n, int group_m)
{
    using namespace f32small;
    constexpr int BM = 64, BN = 64, U = BK / 4;
    constexpr int W = 2 * WN, BJ = 4 / WN;   // wavefronts; 16-column blocks per wavefront
    constexpr int A_BYTES = BM * BK * 4, STAGE = A_BYTES + BK * BN * 4;
    constexpr int LA = BK / 4 / W, LB = BK / 4 / W, LPS = LA + LB;   // loads per wavefront and stage
    constexpr int RPS = 2 + 4 * BJ;                                   // reads per slice
    constexpr int SLICES = BK / 16, READS = RPS * SLICES, MFMAS = 8 * BJ * SLICES;
    static_assert(LA >= 1 && LA * W * 4 == BK, "whole loads per wavefront");
    static_assert(U == 8 || U == 16, "A rows of 8 or 16 units");
    static_assert((NBUF & (NBUF - 1)) == 0 && NBUF >= 4, "ring of a power of two, at least 4");
    static_assert(READS <= MFMAS, "one read after each of the first MFMAs");
    static_assert(KS == 1 || KS == 2, "one or two groups over k");
    constexpr int RING = NBUF * STAGE;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[KS * RING];
    const int wave_all = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int grp = wave_all / W, wave = wave_all % W;
    uint8_t *const ring = lds + grp * RING;
    const uint32_t lds0 = lds_address(lds) + (uint32_t)(grp * RING);
    const int steps_all = (K + BK - 1) / BK;
    const int steps = (steps_all + KS - 1) / KS;   // stages of each group
    const int kbase = grp * steps * BK;            // the group's first k

    int tm, tn;
    dgor_tile_of_block(blockIdx.x, tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int lane = threadIdx.x & 63;
    const int wr = (wave / WN) * 32, wc = (wave % WN) * 16 * BJ;
    constexpr uint32_t OOB = 0x80000000u;

    // ---- loader: wave w issues A loads w LA .. w LA + LA - 1 and B loads
    // w LB .. w LB + LB - 1 of each stage (1 KB each).  A load j covers rows
    // j 64 / U ..; lane p takes physical unit p % U of row j 64 / U + p / U.
    // B load j covers k-rows 4 j .. 4 j + 3; lane p takes physical unit p % 16
    // of k-row 4 j + p / 16.
    const intx4 ra = rsrc_words(A + (size_t)m0 * K, 0x7fffffff);
    const intx4 rb = rsrc_words(B + n0, 0x7fffffff);
    uint32_t a_row[LA], b_row[LB];   // byte offsets of the lane's row start
    int a_k[LA], b_k[LB];            // the lane's k within a stage (A: of its unit)
    bool a_ok[LA], b_ok[LB];         // row inside A, column inside B
#pragma unroll
    for (int i = 0; i < LA; ++i) {
        const int j = wave * LA + i, r = j * (64 / U) + lane / U;
        const int u = (lane % U) ^ fa(r, U);
        a_row[i] = (uint32_t)(r * K + 4 * u) * 4u;
        a_k[i] = 4 * u;
        a_ok[i] = m0 + r < M;
    }
#pragma unroll
    for (int i = 0; i < LB; ++i) {
        const int j = wave * LB + i, k = 4 * j + lane / 16;
        const int u = (lane % 16) ^ fb(k);
        b_row[i] = (uint32_t)(k * N + 4 * u) * 4u;
        b_k[i] = k;
        b_ok[i] = n0 + 4 * u < N;
    }
    auto load = [&](int st, int x) {   // load x (0 .. LPS - 1) of the group's stage st
        const int k0 = kbase + st * BK;
        const bool in = st < steps;
        const uint32_t buf = lds0 + (uint32_t)((st & (NBUF - 1)) * STAGE);
        if (x < LA) {
            const bool ok = in && a_ok[x] && k0 + a_k[x] < K;
            load_to_lds(ra, buf + (uint32_t)((wave * LA + x) * 1024), ok ? a_row[x] + (uint32_t)k0 * 4u : OOB);
        } else {
            const int i = x - LA;
            const bool ok = in && b_ok[i] && k0 + b_k[i] < K;
            load_to_lds(rb, buf + (uint32_t)(A_BYTES + (wave * LB + i) * 1024),
                        ok ? b_row[i] + (uint32_t)k0 * (uint32_t)N * 4u : OOB);
        }
    };

    // ---- fragment reads (read rd of a stage: slice q = rd / RPS, then A
    // block 0, A block 1, and rows e = 0..3 of each B block).  A block x,
    // slice q: logical unit 4 q + h of row wr + 16 x + l16.  B block b, slice
    // q, row e: k-row 16 q + 4 h + e (so fb = 4 h), column wc + 16 b + l16.
    const int l16 = lane & 15, h = lane >> 4;
    uint32_t a_off[2 * SLICES], b_lane[BJ];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
        const int r = wr + 16 * x + l16;
#pragma unroll
        for (int q = 0; q < SLICES; ++q)
            a_off[2 * q + x] = (uint32_t)(r * U * 16 + (((4 * q + h) ^ fa(r, U)) * 16));
    }
#pragma unroll
    for (int b = 0; b < BJ; ++b) {
        const int col = wc + 16 * b + l16;
        b_lane[b] = (uint32_t)(A_BYTES + (4 * h) * 256 + (((col >> 2) ^ (4 * h)) * 16) + (col & 3) * 4);
    }
    auto fread = [&](int st, int rd, floatx4 *fa_, floatx4 *fb_) {
        const uint8_t *buf = ring + (st & (NBUF - 1)) * STAGE;
        const int q = rd / RPS, x = rd % RPS;
        if (x < 2) {
            fa_[2 * q + x] = *reinterpret_cast<const floatx4 *>(buf + a_off[2 * q + x]);
        } else {
            const int b = (x - 2) >> 2, e = (x - 2) & 3;
            fb_[BJ * q + b][e] = *reinterpret_cast<const float *>(buf + b_lane[b] + (16 * q + e) * 256);
        }
    };

    floatx4 acc[2][BJ];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < BJ; ++j)
            acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    // One stage t: its MFMAS matrix instructions from (ca, cb); the READS
    // reads of stage t + 1 into (na, nb), one after each of the first ones;
    // the LPS loads of stage t + NBUF - 1 spread over the stage.  Before it,
    // this wavefront's loads of stage t + 1 have landed (those of the NBUF - 3
    // later stages may fly) and the workgroup meets at the barrier, so every
    // wavefront's part of stage t + 1 is in LDS and nobody still reads the
    // buffer the new loads refill (stage t - 1's, read during stage t - 2).
    auto stage = [&](int t, floatx4 *ca, floatx4 *cb, floatx4 *na, floatx4 *nb) {
        __builtin_amdgcn_s_waitcnt(wait_vmcnt((NBUF - 3) * LPS));
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < MFMAS; ++m) {
            const int q = m / (8 * BJ), e = (m / (2 * BJ)) & 3, i = (m / BJ) & 1, j = m % BJ;
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(ca[2 * q + i][e], cb[BJ * q + j][e], acc[i][j], 0,
                                                             0, 0);
            if (m < READS)
                fread(t + 1, m, na, nb);
            if (m % (MFMAS / LPS) == MFMAS / LPS / 2)
                load(t + NBUF - 1, m / (MFMAS / LPS));
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // prologue: stages 0 .. NBUF - 2 in flight; once stage 0 has landed, its reads
    floatx4 fa0[2 * SLICES], fb0[BJ * SLICES], fa1[2 * SLICES], fb1[BJ * SLICES];
    for (int st = 0; st < NBUF - 1; ++st)
#pragma unroll
        for (int x = 0; x < LPS; ++x)
            load(st, x);
    __builtin_amdgcn_s_waitcnt(wait_vmcnt((NBUF - 2) * LPS));
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int r = 0; r < READS; ++r)
        fread(0, r, fa0, fb0);

    for (int t = 0; t < steps; t += 2) {
        stage(t, fa0, fb0, fa1, fb1);
        if (t + 1 < steps)
            stage(t + 1, fa1, fb1, fa0, fb0);
    }
    // no load may still be writing this workgroup's LDS when it ends
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
    if constexpr (KS == 2) {
        // group 1 hands its sums to group 0 through its own ring: once every
        // wavefront's reads have returned, block (i, j) of wavefront w at
        // 16 ((((i BJ + j) W + w) 64) + lane); group 0 adds them to its own
        floatx4 *part = reinterpret_cast<floatx4 *>(lds + RING);
        __builtin_amdgcn_s_waitcnt(wait_vmcnt_lgkm0(0));
        __builtin_amdgcn_s_barrier();
        if (grp == 1) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < BJ; ++j)
                    part[((i * BJ + j) * W + wave) * 64 + lane] = acc[i][j];
        }
        __builtin_amdgcn_s_barrier();
        if (grp == 1)
            return;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < BJ; ++j)
                acc[i][j] += part[((i * BJ + j) * W + wave) * 64 + lane];
    }

    const __amdgpu_buffer_rsrc_t rc =
        make_rsrc(C + (size_t)m0 * N + n0, ((long long)(M - m0 - 1) * N + N - n0) * 4);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < BJ; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = wr + 16 * i + 4 * h + r, col = wc + 16 * j + l16;
                const uint32_t vo = (m0 + row < M && n0 + col < N) ? (uint32_t)(row * N + col) * 4u : OOB;
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][j][r]), rc, vo, 0, 0);
            }
}

// ---------------------------------------------------------------------------
// The end of both tall, narrow kernels, after the barrier that follows the
// partial sums: wavefront w's sums of column block c sit at 64 floatx4 from
// sh + w * area + 1024 c, its sums of the last column (FRINGE) at 64 floats
// from sh + w * area + 1024 NB, its tail-row sum at tpart[w].  They are added
// in order of w, and wavefront c < NB stores block c.
template <int NB, bool FRINGE>
__device__ __forceinline__ void skinny_finish(const uint8_t *sh, int area, const float *tpart, int M, int N,
                                              bool tl, float *C)
{
    constexpr uint32_t OOB = 0x80000000u;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int r16 = lane & 15, h = lane >> 4, m0 = blockIdx.x * 16;
    if (wave < NB) {
        floatx4 v = reinterpret_cast<const floatx4 *>(sh)[64 * wave + lane];
#pragma unroll
        for (int w = 1; w < 8; ++w)
            v += reinterpret_cast<const floatx4 *>(sh + w * area)[64 * wave + lane];
        const int col = NB * r16 + wave;
        const __amdgpu_buffer_rsrc_t rc = make_rsrc(C, (long long)M * N * 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int orow = m0 + 4 * h + r;
            const uint32_t vo = (orow < M && col < N) ? (uint32_t)(orow * N + col) * 4u : OOB;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[r]), rc, vo, 0, 0);
        }
    }
    if (FRINGE && wave == 7 && lane < 16 && m0 + lane < M) {
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < 8; ++w)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                v += reinterpret_cast<const float *>(sh + w * area + 1024 * NB)[16 * g + lane];
        C[(size_t)(m0 + lane) * N + N - 1] = v;
    }
    if (tl && wave == 6 && lane == 0) {
        float v = tpart[0];
#pragma unroll
        for (int w = 1; w < 8; ++w)
            v += tpart[w];
        C[(size_t)(M - 1) * N + blockIdx.x] = v;
    }
}

// Tall, narrow FP32 problems (N <= 64, K <= 1024, A and B 4-byte aligned).
// Their time is one read of A from HBM (B and C are small), so every compute
// unit streams its share of A from the start.  This kernel takes three and
// four column blocks; the resident form below takes one and two.  A workgroup takes 16 rows, all
// N columns and all of K with eight wavefronts (two per SIMD); wavefront w
// takes a contiguous run [kb, ke) of the 16-deep k-slices, the runs as even
// as the slice count allows, and streams it through its own ring of LDS
// slots, so no wavefront waits for another until the partial sums are added.
// A slice is LW direct global->LDS loads into one slot:
//   A: lane (r, h) = (l % 16, l / 16) fetches A[m0 + r][k0 + 4h .. + 3] (16
//      bytes, 4-byte aligned; a unit that runs past K brings the next row's
//      values, which are zeroed on reading, and past the end of A reads zero);
//   B: the slice's 16 rows of B's first 16 NB columns, NB loads of 64 units
//      of 16 bytes.  Row 4g + e of the slice sits at position 4g + ((e + g) &
//      3): the four rows the lane groups h read at once then fall in distinct
//      banks;
//   fringe (FRINGE): B's last column of the slice's rows, 4 bytes a lane.
// Rows past ke read zero (B rows past K hold zeros, and a row of the next
// run is never fetched, so no value outside [kb, ke) enters a sum).  D = R - 1
// slices are in flight while one is computed; the wait for slice s counts the
// loads issued after it, and a slot is refilled only once its last reads have
// returned.  A slice's arithmetic: in instruction e, lane l holds A[l % 16][k]
// and, for column block c, B[k][NB (l % 16) + c], with k = k0 + 4 (l / 16) +
// e (column block c holds the columns NB j + c, so a lane's NB values of one
// row are adjacent: one 8-byte read for NB = 2, one 16-byte read for NB = 4).
// The eight partial sums of an output are added in LDS in order of w, so
// results do not depend on timing.
//   FRINGE (N % 16 == 1, N > 16): the last column is not given a 16-column
//     block of its own (that block would cost as much matrix-core time as a
//     full one); its sums are formed on the vector ALUs.
//   tail (M % 16 == 1 with at least N whole row blocks): the last row gets no
//     workgroup of its own (that workgroup would share a compute unit with
//     another and double its matrix-core time); workgroup j < N instead forms
//     C[M - 1][j] as a dot product spread over its 512 lanes (two products a
//     lane, a butterfly sum in each wavefront, then the eight wavefront sums
//     in order).
template <int NB, bool FRINGE>
__global__ __launch_bounds__(512) void mfma_f32_skinny_kernel(int M, int N, int K, int tail, const float *A,
                                                              const float *B, float *C)
{
    constexpr int R = skinny_slots(NB);                  // ring slots per wavefront
    constexpr int D = R - 1;                             // slices in flight ahead of the computed one
    constexpr int SLOT = skinny_slot_bytes(NB, FRINGE);
    constexpr int AREA = skinny_wave_bytes(NB, FRINGE);  // ring + the tail row's products
    constexpr int LW = 1 + NB + (FRINGE ? 1 : 0);        // loads per slice
    constexpr int U = 4 * NB;                            // 16-byte units per B row
    constexpr int QMAX = kF32SkinnyMaxK / (16 * 8);      // slices per wavefront at most
    constexpr uint32_t OOB = 0x80000000u;
    __shared__ __attribute__((aligned(1024))) uint8_t sh[8 * AREA];
    __shared__ float tpart[8];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int r16 = lane & 15, h = lane >> 4;
    const int m0 = blockIdx.x * 16, row = m0 + r16;
    const int total = (K + 15) / 16;
    const int s_lo = wave * total / 8, s_hi = (wave + 1) * total / 8;
    const int slices = s_hi - s_lo, kb = 16 * s_lo, ke = min(K, 16 * s_hi);
    const intx4 ra = rsrc_words(A, (long long)M * K * 4);
    const intx4 rb = rsrc_words(B, (long long)K * N * 4);
    uint8_t *mine = sh + wave * AREA;
    const uint32_t ring = lds_address(mine);

    // this lane's B units: unit t = 64 j + lane of the slice sits at position
    // p = t / U, column unit t % U, and holds row i of the slice
    int b_row[NB];
    uint32_t b_off[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        const int t = 64 * j + lane, p = t / U, u = t % U, g = p >> 2;
        b_row[j] = 4 * g + (((p & 3) - g) & 3);
        b_off[j] = (uint32_t)(b_row[j] * N + 4 * u) * 4u;
    }
    // the positions this lane reads B rows 4h + e from
    int b_rd[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
        b_rd[e] = 1024 + (4 * h + ((e + h) & 3)) * U * 16 + NB * r16 * 4;

    auto issue = [&](int s) __attribute__((always_inline)) {
        const int k0 = kb + 16 * s;
        const uint32_t slot = ring + (uint32_t)((s % R) * SLOT);
        const int ka = k0 + 4 * h;
        load_to_lds(ra, slot, row < M && ka < ke ? (uint32_t)(row * K + ka) * 4u : OOB);
#pragma unroll
        for (int j = 0; j < NB; ++j)
            load_to_lds(rb, slot + 1024u * (j + 1),
                        k0 + b_row[j] < ke ? (uint32_t)(k0 * N) * 4u + b_off[j] : OOB);
        if constexpr (FRINGE)
            load_dword_to_lds(rb, slot + 1024u * (NB + 1),
                              lane < 16 && k0 + lane < ke ? (uint32_t)((k0 + lane) * N + N - 1) * 4u : OOB);
    };

    // the tail row's products, issued first (older than every slice, so the
    // slice waits need not count them): this wavefront's k, two a lane
    const bool tl = tail && (int)blockIdx.x < N;
    if (tl) {
        const uint32_t dst = ring + (uint32_t)(R * SLOT);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int k = kb + lane + 64 * i;
            load_dword_to_lds(ra, dst + 256u * i, k < ke ? (uint32_t)((M - 1) * K + k) * 4u : OOB);
            load_dword_to_lds(rb, dst + 256u * (2 + i), k < ke ? (uint32_t)(k * N + (int)blockIdx.x) * 4u : OOB);
        }
    }
#pragma unroll
    for (int s = 0; s < D; ++s)
        if (s < slices)
            issue(s);

    floatx4 acc[NB];
#pragma unroll
    for (int c = 0; c < NB; ++c)
        acc[c] = floatx4{0.f, 0.f, 0.f, 0.f};
    float f = 0.f;
#pragma unroll
    for (int s = 0; s < QMAX; ++s) {
        if (s < slices) {   // wave-uniform
            if (s + D < slices) {
                // slice s + D refills slice s - 1's slot, whose reads have returned
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                issue(s + D);
            }
            // slice s has landed once no more than the loads of the slices
            // issued after it are outstanding
            switch (min(D, slices - 1 - s)) {
            case 0: __builtin_amdgcn_s_waitcnt(wait_vmcnt(0)); break;
            case 1: __builtin_amdgcn_s_waitcnt(wait_vmcnt(LW)); break;
            case 2: __builtin_amdgcn_s_waitcnt(wait_vmcnt(2 * LW)); break;
            default: __builtin_amdgcn_s_waitcnt(wait_vmcnt(3 * LW)); break;
            }
            asm volatile("" ::: "memory");
            const uint8_t *slot = mine + (s % R) * SLOT;
            floatx4 av = *reinterpret_cast<const floatx4 *>(slot + 16 * lane);
            const int ka = kb + 16 * s + 4 * h;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                av[e] = ka + e < K ? av[e] : 0.f;
            float bv[4][NB];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float *q = reinterpret_cast<const float *>(slot + b_rd[e]);
                if constexpr (NB == 2) {
                    const float2 v = *reinterpret_cast<const float2 *>(q);
                    bv[e][0] = v.x;
                    bv[e][1] = v.y;
                } else if constexpr (NB == 4) {
                    const floatx4 v = *reinterpret_cast<const floatx4 *>(q);
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        bv[e][c] = v[c];
                } else {
#pragma unroll
                    for (int c = 0; c < NB; ++c)
                        bv[e][c] = q[c];
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int c = 0; c < NB; ++c)
                    acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[e], bv[e][c], acc[c], 0, 0, 0);
            if constexpr (FRINGE) {
                const floatx4 fb = *reinterpret_cast<const floatx4 *>(slot + 1024 * (NB + 1) + 16 * h);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    f = fmaf(av[e], fb[e], f);
            }
        }
    }
    // every load has landed (the tail row's too) and no read of the ring is
    // outstanding: the partial sums go into this wavefront's first slot
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    float tv = 0.f;
    if (tl) {   // this wavefront's sum of the tail row's products (butterfly, fixed order)
        const float *tp = reinterpret_cast<const float *>(mine + R * SLOT);
        tv = tp[lane] * tp[128 + lane] + tp[64 + lane] * tp[192 + lane];
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1)
            tv += __shfl_xor(tv, d);
    }
    // wavefront w's block c at part_w[c]; lane l holds rows 4 (l / 16) + r
    // of column NB (l % 16) + c
    floatx4 *part = reinterpret_cast<floatx4 *>(mine);
#pragma unroll
    for (int c = 0; c < NB; ++c)
        part[64 * c + lane] = acc[c];
    if constexpr (FRINGE)
        reinterpret_cast<float *>(mine + 1024 * NB)[lane] = f;
    if (lane == 0)
        tpart[wave] = tv;
    __syncthreads();
    skinny_finish<NB, FRINGE>(sh, AREA, tpart, M, N, tl, C);
}

// The same problems with at most two column blocks (N <= 32, or N = 33 with
// the last column on the vector ALUs) keep a wavefront's whole run of B in
// its LDS (8 slices x NB KB), so every load can be issued at once: first the
// B units of every slice and B's last column (direct global->LDS loads, B in
// the layout above), then the tail row's products and the A units straight
// into registers.  The compiler counts only the loads it issued itself,
// which come last, so its waits on A are exact, and one wait for the B
// copies precedes the first read of them.  Slice s then needs its A
// registers only: the slices start as A lands, and each reads B with
// NB-float reads free of bank conflicts (against twelve conflicting 4-byte
// reads a slice with B rows packed as in memory).
template <int NB, bool FRINGE>
__global__ __launch_bounds__(512) void mfma_f32_skinny_resident_kernel(int M, int N, int K, int tail,
                                                                       const float *A, const float *B, float *C)
{
    static_assert(NB <= 2, "a wavefront's B run must fit its share of LDS");
    constexpr int QMAX = kF32SkinnyMaxK / (16 * 8);            // slices per wavefront at most
    constexpr int U = 4 * NB;                                  // 16-byte units per B row
    constexpr int FCOL = QMAX * 1024 * NB;                     // B's last column: 4 bytes a row
    constexpr int AREA = skinny_resident_wave_bytes(NB, FRINGE);
    constexpr uint32_t OOB = 0x80000000u;
    __shared__ __attribute__((aligned(1024))) uint8_t sh[8 * AREA];
    __shared__ float tpart[8];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int r16 = lane & 15, h = lane >> 4;
    const int m0 = blockIdx.x * 16, row = m0 + r16;
    const int total = (K + 15) / 16;
    const int s_lo = wave * total / 8, s_hi = (wave + 1) * total / 8;
    const int slices = s_hi - s_lo, kb = 16 * s_lo, ke = min(K, 16 * s_hi);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, (long long)M * K * 4);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(B, (long long)K * N * 4);
    const intx4 rbw = rsrc_words(B, (long long)K * N * 4);
    uint8_t *mine = sh + wave * AREA;
    const uint32_t base = lds_address(mine);

    // B: slice s's units at base + 1024 NB s, unit t = 64 j + lane of the
    // slice at position t / U (rows rotated as in the ring kernel)
    {
        int b_row[NB];
        uint32_t b_off[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const int t = 64 * j + lane, p = t / U, u = t % U, g = p >> 2;
            b_row[j] = 4 * g + (((p & 3) - g) & 3);
            b_off[j] = (uint32_t)(b_row[j] * N + 4 * u) * 4u;
        }
#pragma unroll
        for (int s = 0; s < QMAX; ++s) {
            if (s < slices) {
                const int k0 = kb + 16 * s;
#pragma unroll
                for (int j = 0; j < NB; ++j)
                    load_to_lds(rbw, base + (uint32_t)(1024 * (NB * s + j)),
                                k0 + b_row[j] < ke ? (uint32_t)(k0 * N) * 4u + b_off[j] : OOB);
            }
        }
        if constexpr (FRINGE) {   // rows kb .. ke - 1 of the last column
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int k = kb + lane + 64 * i;
                load_dword_to_lds(rbw, base + (uint32_t)(FCOL + 256 * i),
                                  k < ke ? (uint32_t)(k * N + N - 1) * 4u : OOB);
            }
        }
    }
    // the tail row's products: this wavefront's k, two a lane
    const bool tl = tail && (int)blockIdx.x < N;
    float ta[2], tb[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int k = kb + lane + 64 * i;
        const bool ok = tl && k < ke;
        ta[i] = __uint_as_float(
            __builtin_amdgcn_raw_buffer_load_b32(ra, ok ? (uint32_t)((M - 1) * K + k) * 4u : OOB, 0, 0));
        tb[i] = __uint_as_float(
            __builtin_amdgcn_raw_buffer_load_b32(rb, ok ? (uint32_t)(k * N + blockIdx.x) * 4u : OOB, 0, 0));
    }
    // A of every slice, in slice order.  No load sits under a branch: one
    // that did would make the compiler wait for earlier loads at the join.
    // A unit that runs past K brings the next row's values (zeroed below).
    floatx4 a[QMAX];
#pragma unroll
    for (int s = 0; s < QMAX; ++s) {
        const int k = kb + 16 * s + 4 * h;
        a[s] = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(
                                               ra, s < slices && row < M && k < ke ? (uint32_t)(row * K + k) * 4u : OOB,
                                               0, 0));
        __builtin_amdgcn_sched_barrier(0);
    }
    // every load is issued before the first MFMA (none may be sunk into the
    // slice branches below); the B copies have landed once no more than the
    // loads issued after them (tail, A) are outstanding
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(4 + QMAX));
    asm volatile("" ::: "memory");

    int b_rd[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
        b_rd[e] = (4 * h + ((e + h) & 3)) * U * 16 + NB * r16 * 4;
    floatx4 acc[NB];
#pragma unroll
    for (int c = 0; c < NB; ++c)
        acc[c] = floatx4{0.f, 0.f, 0.f, 0.f};
    float f = 0.f;
#pragma unroll
    for (int s = 0; s < QMAX; ++s) {
        if (s < slices) {   // wave-uniform
            floatx4 av = a[s];
            const int ka = kb + 16 * s + 4 * h;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                av[e] = ka + e < K ? av[e] : 0.f;
            float bv[4][NB];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float *q = reinterpret_cast<const float *>(mine + 1024 * NB * s + b_rd[e]);
                if constexpr (NB == 2) {
                    const float2 v = *reinterpret_cast<const float2 *>(q);
                    bv[e][0] = v.x;
                    bv[e][1] = v.y;
                } else {
                    bv[e][0] = q[0];
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int c = 0; c < NB; ++c)
                    acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[e], bv[e][c], acc[c], 0, 0, 0);
            if constexpr (FRINGE) {
                const floatx4 fb = *reinterpret_cast<const floatx4 *>(mine + FCOL + 64 * s + 16 * h);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    f = fmaf(av[e], fb[e], f);
            }
        }
    }
    // the partial sums go into this wavefront's own B slices (their reads
    // have returned)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    floatx4 *part = reinterpret_cast<floatx4 *>(mine);
#pragma unroll
    for (int c = 0; c < NB; ++c)
        part[64 * c + lane] = acc[c];
    if constexpr (FRINGE)
        reinterpret_cast<float *>(mine + 1024 * NB)[lane] = f;
    // tail: this wavefront's sum of its products (butterfly, fixed order)
    float tv = ta[0] * tb[0] + ta[1] * tb[1];
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1)
        tv += __shfl_xor(tv, d);
    if (lane == 0)
        tpart[wave] = tv;
    __syncthreads();
    skinny_finish<NB, FRINGE>(sh, AREA, tpart, M, N, tl, C);
}

template <int NB, bool FRINGE>
void launch_skinny_t(const Problem &p, const F32SkinnyPlan &n, hipStream_t s)
{
    if constexpr (NB <= 2)
        hipLaunchKernelGGL((mfma_f32_skinny_resident_kernel<NB, FRINGE>), dim3((unsigned)n.blocks), dim3(512), 0,
                           s, p.M, p.N, p.K, n.tail ? 1 : 0, (const float *)p.A, (const float *)p.B, p.C);
    else
        hipLaunchKernelGGL((mfma_f32_skinny_kernel<NB, FRINGE>), dim3((unsigned)n.blocks), dim3(512), 0, s, p.M,
                           p.N, p.K, n.tail ? 1 : 0, (const float *)p.A, (const float *)p.B, p.C);
}

void launch_skinny(const Problem &p, const F32SkinnyPlan &n, hipStream_t s)
{
    if (n.fringe) {
        switch (n.nb) {
        case 1: launch_skinny_t<1, true>(p, n, s); break;
        case 2: launch_skinny_t<2, true>(p, n, s); break;
        default: launch_skinny_t<3, true>(p, n, s); break;
        }
        return;
    }
    switch (n.nb) {
    case 1: launch_skinny_t<1, false>(p, n, s); break;
    case 2: launch_skinny_t<2, false>(p, n, s); break;
    case 3: launch_skinny_t<3, false>(p, n, s); break;
    default: launch_skinny_t<4, false>(p, n, s); break;
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
        return launch_ring32_t<false, false>(ring_args_nn(p, plan), s);
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
    if (plan.tile_m == 64 && plan.tile_n == 64) {
        if (f32_small_ring_applies(64, 64, p.N, p.K, p.vec_a, p.vec_b)) {
            const dim3 grid(plan.grid_x * plan.grid_y);
            if (plan.threads == 256 * kF32SmallWavesN)   // two groups over k
                hipLaunchKernelGGL((mfma_f32_small_ring_kernel<kF32SmallDepth, kF32SmallStages, kF32SmallWavesN, 2>),
                                   grid, dim3(256 * kF32SmallWavesN), 0, s, p.M, p.N, p.K, (const float *)p.A,
                                   (const float *)p.B, p.C, plan.grid_y, plan.grid_x, 8);
            else
                hipLaunchKernelGGL((mfma_f32_small_ring_kernel<kF32SmallDepth, kF32SmallStages, kF32SmallWavesN, 1>),
                                   grid, dim3(128 * kF32SmallWavesN), 0, s, p.M, p.N, p.K, (const float *)p.A,
                                   (const float *)p.B, p.C, plan.grid_y, plan.grid_x, 8);
            return hipGetLastError();
        }
        return launch_cfg<64, 64, 16, 2, 2>(p, plan, s);
    }
    F32SkinnyPlan n;
    if (f32_skinny_plan(p.M, p.N, p.K, n) && plan.tile_m == 16 && plan.grid_y == n.blocks) {
        launch_skinny(p, n, s);
        return hipGetLastError();
    }
    if (plan.tile_m == 32 && plan.tile_n == 64)
        return launch_cfg<32, 64, 16, 1, 2>(p, plan, s);
    return hipErrorInvalidValue;
}

hipError_t launch_ring32(const RingArgs &a, hipStream_t s)
{
    if (a.trans_a)
        return a.trans_b ? launch_ring32_t<true, true>(a, s) : launch_ring32_t<true, false>(a, s);
    return a.trans_b ? launch_ring32_t<false, true>(a, s) : launch_ring32_t<false, false>(a, s);
}

}  // namespace dgor
