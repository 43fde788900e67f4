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
constexpr int LOADS_PER_STAGE = 8;                   // per wavefront: 4 per operand

// Lane offsets of wave w's four 1 KB loads of one operand tile per stage,
// relative to the stage's first element (as for the 16-bit ring).
template <bool KSTRIDED>
__device__ __forceinline__ void load_offsets(int wave, int lane, int t0, int ext, int ld,
                                             uint32_t off[4], int &kc)
{
    constexpr uint32_t OOB = 0x80000000u;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        if (!KSTRIDED) {
            const int r = 16 * (4 * wave + q) + (lane >> 2);
            kc = 4 * ((lane & 3) ^ ((lane >> 4) & 3));   // same in every block
            off[q] = (uint32_t)(r * ld + kc) * 4u;
        } else {
            const int k = 4 * wave + q;
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

template <bool TA, bool TB, bool ACC>
__global__ __launch_bounds__(256) void mfma_f32_ring_kernel(RingArgs args)
{
    const int bid = dgor_ring_split(args, 4);   // split-K: this workgroup's k-range and tile
    using namespace f32ring;
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
    const int wr = (wave >> 1) * 128, wc = (wave & 1) * 128;
    constexpr uint32_t OOB = 0x80000000u;

    // ---- loader (see the 16-bit ring kernel for the range rules)
    uint32_t a_off[4], b_off[4];
    int a_kc, b_kc;
    load_offsets<TA>(wave, lane, m0, M, lda, a_off, a_kc);
    load_offsets<!TB>(wave, lane, n0, N, ldb, b_off, b_kc);
    const uint32_t lds_a = ring + (uint32_t)(4 * wave * 1024);
    const uint32_t lds_b = ring + (uint32_t)(A_BYTES + 4 * wave * 1024);
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
        if (q < 4) {
            const uint32_t off = (!TA && L.tail && a_kc >= L.k_left) ? OOB : a_off[q];
            load_to_lds(L.ra, lds_a + L.lds + (uint32_t)(q * 1024), off);
        } else {
            const uint32_t off = (TB && L.tail && b_kc >= L.k_left) ? OOB : b_off[q - 4];
            load_to_lds(L.rb, lds_b + L.lds + (uint32_t)((q - 4) * 1024), off);
        }
    };

    // ---- fragment reads.  Lane (g, l32) = (lane / 32, lane % 32).
    const int l32 = lane & 31, g = lane >> 5;
    const int kc_sw = (l32 >> 2) & 3;
    auto kc_lane = [&](uint32_t region, int base) { return region + (uint32_t)((base + l32) * 64); };
    auto ks_lane = [&](uint32_t region) { return region + (uint32_t)((4 * g) * 1024 + 4 * (l32 & 3)); };
    uint32_t a_unit[4], b_unit[4];   // k-strided column units of each block
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        a_unit[j] = (uint32_t)((((wr + 32 * j + l32) >> 2) ^ (8 * g)) * 16);
        b_unit[j] = (uint32_t)((((wc + 32 * j + l32) >> 2) ^ (8 * g)) * 16);
    }
    const uint32_t a_lane = TA ? ks_lane(0) : kc_lane(0, wr);
    const uint32_t b_lane = TB ? kc_lane(A_BYTES, wc) : ks_lane(A_BYTES);
    // One read instruction of operand X (k-slice q, block blk, sub-step e of
    // a k-strided block) into x[4 q + blk].
    auto read_one = [&](const uint8_t *buf, uint32_t lane_off, const uint32_t *unit, bool kstrided, int q,
                        int blk, int e, floatx4 *x) {
        if (!kstrided)
            x[4 * q + blk] = *reinterpret_cast<const floatx4 *>(
                buf + lane_off + blk * 32 * 64 + (((2 * q + g) ^ kc_sw) * 16));
        else
            x[4 * q + blk][e] = *reinterpret_cast<const float *>(buf + lane_off + (8 * q + e) * 1024 + unit[blk]);
    };
    // Read r of stage `stage`, in k-slice order; within a slice, for each
    // block, A's read(s) then B's.
    constexpr int NA = TA ? 4 : 1, NB = TB ? 1 : 4, PER = NA + NB;
    constexpr int READS = 8 * PER;
    auto fread = [&](int stage, int r, floatx4 *fa, floatx4 *fb) {
        const uint8_t *buf = lds + (stage % NBUF) * STAGE_BYTES;
        const int item = r / PER, x = r % PER, q = item >> 2, blk = item & 3;
        if (x < NA)
            read_one(buf, a_lane, a_unit, TA, q, blk, x, fa);
        else
            read_one(buf, b_lane, b_unit, !TB, q, blk, x - NA, fb);
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
    floatx16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
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

    // One stage: the 128 MFMAs of stage t from (ca, cb); the reads of stage
    // t + 1 into (na, nb), one after each of the first READS MFMAs (at most
    // 64); the 8 loads of stage t + 3, one after every eighth MFMA from the
    // 64th.
    const int steps = (K + BK - 1) / BK;
    auto stage = [&](int t, floatx4 *ca, floatx4 *cb, floatx4 *na, floatx4 *nb) {
        __builtin_amdgcn_s_waitcnt(wait_vmcnt(LOADS_PER_STAGE));
        __builtin_amdgcn_s_barrier();
        const StageLoads L = prep(t + 3);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < 128; ++m) {
            const int q = m >> 6, jp = (m >> 4) & 3, i = (m >> 2) & 3, j = m & 3;
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(ca[4 * q + i][jp], cb[4 * q + j][jp], acc[i][j], 0,
                                                              0, 0);
            if (m < READS)
                fread(t + 1, m, na, nb);
            if (m >= 64 && (m - 64) % 8 == 0)
                load(L, (m - 64) / 8);
            // keep this order: the compiler would otherwise cluster the reads
            // and loads, and move MFMAs across the barrier
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // prologue: loads of stages 0, 1, 2, then the reads of stage 0
    floatx4 fa0[8], fa1[8], fb0[8], fb1[8];
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
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
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
    if (a.accumulate)
        hipLaunchKernelGGL((mfma_f32_ring_kernel<TA, TB, true>), grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((mfma_f32_ring_kernel<TA, TB, false>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
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
    if (plan.tile_m == 64 && plan.tile_n == 64)
        return launch_cfg<64, 64, 16, 2, 2>(p, plan, s);
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
