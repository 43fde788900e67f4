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
#include "lds_dma.h"

namespace dgor {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// The matrix-core operation of each 16-bit input format.  Fragments travel
// as eight 16-bit patterns (halfx8) whatever the format; only the MFMA
// differs (binary16: v_mfma_f32_*_f16, bfloat16: v_mfma_f32_*_bf16).
struct OpF16 {
    static __device__ __forceinline__ floatx4 mfma16(halfx8 a, halfx8 b, floatx4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ floatx16 mfma32(halfx8 a, halfx8 b, floatx16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};
struct OpBF16 {
    static __device__ __forceinline__ floatx4 mfma16(halfx8 a, halfx8 b, floatx4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ floatx16 mfma32(halfx8 a, halfx8 b, floatx16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
};

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
template <class Op, int BM, int BN, int BK, int WM, int WN, bool VEC_A, bool VEC_B>
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
                    acc[i][j] = Op::mfma32(a[i], b[j], acc[i][j]);
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
// Large-tile kernel (the gfx950 path for 16-byte aligned operands):
// 256 x 256 workgroup tile, 32-deep k-stages in a ring of four LDS buffers,
// four wavefronts of 128 x 128, each an 8 x 8 grid of
// v_mfma_f32_16x16x32_f16 blocks (256 accumulators per lane).
//
// v_mfma_f32_16x16x32_f16 (wave64): lane l = 16 g + s supplies eight halves
// A[s][8 g + 0..7] and B[8 g + 0..7][s] and holds C[4 g + r][s], r = 0..3.
//
// * Loads go straight from global memory into LDS (buffer_load_dwordx4 ...
//   lds): one instruction moves 64 lanes x 16 bytes into 1 KB of LDS, lane p
//   landing at byte 16 p; which 16-byte chunk of the matrix lane p fetches is
//   free, so the LDS layout is chosen by permuting the sources.  A lane whose
//   offset is out of range writes zeros, which zero-fills every edge.
// * LDS layout of one stage, in 16-byte units (8 halves):
//     A (256 m x 32 k, 4 units per row): unit c of row r at
//       4 r + (c ^ (2 ((r >> 2) & 1)));
//     B (32 k x 256 n, 32 units per row): unit u of row k at
//       32 k + (u ^ (4 (k & 3) + 2 ((k >> 3) & 1))).
//   A fragments are 128-bit reads of 16 consecutive rows at one unit.  B
//   fragments are transposing reads (ds_read_b64_tr_b16): in a group of 16
//   lanes, source lane s points at 4 halves of row kb + s/4, columns
//   nb + 4 (s % 4), and output lane i receives rows kb..kb+3 of column nb + i;
//   two such reads give a lane its eight k.  The LDS serves 256 bytes (16
//   units) a cycle.  A 128-bit read is served in four cycles, each taking
//   the 16 lanes that agree in lane bit 5 and in the parity of lane bits
//   2..4; a cycle is free of bank conflicts when its 16 units differ modulo
//   16.  (This rule reproduces the bank-conflict counter for thirteen
//   probed patterns.)  The A swizzle keeps every such group apart, and a
//   64-bit transposing read, served 32 lanes a cycle, measures free of
//   conflicts with the B swizzle.
// * Pipeline.  The loads of stage t + 3 and the fragment reads of stage t + 1
//   are spread between the 64 MFMAs of stage t.  Before stage t each
//   wavefront waits for its own loads of stage t + 1 (the loads of t + 2 stay
//   in flight) and the workgroup meets at one barrier: after it every load of
//   stage t + 1 has landed, and every wavefront has consumed stage t - 1, whose
//   buffer stage t + 3 then refills.
// * The hardware lets a wavefront's LDS reads run ahead of its own
//   outstanding global->LDS loads, but the compiler, when it sees such a load
//   in flight, waits for it before every transposing LDS read.  The loads are
//   therefore issued from inline assembly that the compiler does not track,
//   and the kernel orders them itself with the waits and barriers above.
namespace pipe {
constexpr int BM = 256, BN = 256, BK = 32, NBUF = 4;
constexpr int A_BYTES = BM * BK * 2;                 // 16 KB
constexpr int B_BYTES = BK * BN * 2;                 // 16 KB
constexpr int STAGE_BYTES = A_BYTES + B_BYTES;       // 32 KB
constexpr int LDS_BYTES = NBUF * STAGE_BYTES;        // 128 KB
constexpr int LOADS_PER_STAGE = 8;                   // per wavefront: 4 of A, 4 of B
}  // namespace pipe

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

// Ring-kernel support for one operand tile (256 m or n x 32 k per stage).
// A k-contiguous operand (A, or B given as N x K) is stored in LDS as 256
// rows of 32 k (four 16-byte units, unit c of row r at 4 r + (c ^ 2((r>>2)&1)))
// and read with 128-bit reads; a k-strided operand (B, or A given as K x M)
// as 32 k rows of 256 (unit u of row k at 32 k + (u ^ (4 (k&3) + 2 ((k>>3)&1))))
// and read with transposing reads.  Either way the fragment a lane gets holds
// the eight k of its row of op(A) or column of op(B) that the 16x16x32 MFMA
// wants from it.
namespace ring16 {

// Lane offsets of wave w's four 1 KB loads of one stage, relative to the
// stage's first element (k0 for the k-contiguous layout, row k0 for the
// k-strided one).  ext is the extent of the operand's non-k dimension (M or
// N), t0 the tile's first index in it, ld the row stride.
template <bool KSTRIDED>
__device__ __forceinline__ void load_offsets(int wave, int lane, int t0, int ext, int ld,
                                             uint32_t off[4], int &kc)
{
    constexpr uint32_t OOB = 0x80000000u;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        if (!KSTRIDED) {
            const int r = 16 * (4 * wave + q) + (lane >> 2);
            kc = 8 * ((lane & 3) ^ (2 * ((lane >> 4) & 1)));   // same in every block
            off[q] = (uint32_t)(r * ld + kc) * 2u;
        } else {
            const int k = 2 * (4 * wave + q) + (lane >> 5);
            const int u = (lane & 31) ^ (4 * (k & 3) + 2 * ((k >> 3) & 1));
            off[q] = t0 + 8 * u < ext ? (uint32_t)(k * ld + 8 * u) * 2u : OOB;
            kc = 0;
        }
    }
}

// Range in bytes of one stage's descriptor (the first element is row t0, k0
// for the k-contiguous layout, row k0, column t0 for the k-strided one):
// everything past it is a row past the operand, or a k row past K.
template <bool KSTRIDED>
__device__ __forceinline__ int stage_range(int k0, int K, int t0, int ext, int ld)
{
    const int k_left = K - k0;
    if (k_left <= 0)
        return 0;   // a stage past the last: every load writes zeros
    if (!KSTRIDED) {
        if (t0 + 256 <= ext)
            return 0x7fffffff;
        return (int)(((uint32_t)(ext - t0 - 1) * (uint32_t)ld + (uint32_t)k_left) * 2u);
    }
    if (k_left >= 32)
        return 0x7fffffff;
    return (int)(((uint32_t)(k_left - 1) * (uint32_t)ld + (uint32_t)(ext - t0)) * 2u);
}

}  // namespace ring16

// Epilogue of the 16-bit ring kernels.  A wavefront's 128 x 128 block of C
// sits in its accumulators in the 16 x 16 MFMA layout (lane (g, s) holds
// rows 16 i + 4 g + r, column 16 j + s), so a store straight from them
// covers 64-byte pieces of four rows.  Instead the block goes out through
// LDS in four rounds of 32 rows: the wavefront writes alpha times its
// accumulators for those rows into its own LDS region, reads them back 16
// bytes a lane along the rows, and stores those 16 bytes (a wavefront's
// store is two whole 512-byte rows), so C is written once, in whole 128-byte
// lines.  The rows of the region are padded by 16 bytes, which puts the 64
// lanes of every 4-byte write on distinct banks.  Cw is the block's first
// element; rows_left and cols_left count the block's rows and columns
// inside C; vec: Cw is 16-byte aligned and ldc a multiple of 4 (else each
// element is stored on its own).  The caller has made sure that no
// wavefront still reads the ring or has a load in flight into it.
namespace cstage {
constexpr int ROW_BYTES = 128 * 4 + 16;
constexpr int WAVE_BYTES = 32 * ROW_BYTES;   // 16.5 KB a wavefront
}  // namespace cstage

__device__ __forceinline__ void store_c_staged(const floatx4 (&acc)[8][8], float alpha, uint8_t *lds, int wave,
                                               int lane, float *Cw, int ldc, int rows_left, int cols_left, bool vec)
{
    using namespace cstage;
    typedef unsigned uintx4 __attribute__((ext_vector_type(4)));
    constexpr uint32_t OOB = 0x80000000u;
    uint8_t *w = lds + wave * WAVE_BYTES;
    const int g = lane >> 4, s16 = lane & 15;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(
        Cw, rows_left > 0 && cols_left > 0 ? ((long long)(rows_left - 1) * ldc + cols_left) * 4 : 0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
        for (int ii = 0; ii < 2; ++ii)
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    *reinterpret_cast<float *>(w + (16 * ii + 4 * g + r) * ROW_BYTES + (16 * j + s16) * 4) =
                        dgor_acc_read(acc[2 * q + ii][j][r]) * alpha;
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const int u = lane + 64 * t, row = u >> 5, col = 4 * (u & 31);
            const floatx4 v = *reinterpret_cast<const floatx4 *>(w + row * ROW_BYTES + col * 4);
            const int grow = 32 * q + row;
            if (grow < rows_left) {
                const uint32_t o = (uint32_t)(grow * ldc + col) * 4u;
                if (vec && col + 4 <= cols_left) {
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(uintx4, v), rc, o, 0, 0);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[e]), rc,
                                                              col + e < cols_left ? o + 4u * e : OOB, 0, 0);
                }
            }
        }
    }
}

template <class Op, bool TA, bool TB, bool ACC>
__global__ __launch_bounds__(256) void mfma_f16_pipe_kernel(RingArgs args)
{
    const int bid = dgor_ring_split(args, 2);   // split-K: this workgroup's k-range and tile
    using namespace pipe;
    static_assert(4 * cstage::WAVE_BYTES <= LDS_BYTES, "the epilogue stages through the ring's LDS");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[LDS_BYTES];
    const uint32_t ring = lds_address(lds);
    const int M = args.M, N = args.N, K = args.K, lda = args.lda, ldb = args.ldb;
    const uint16_t *__restrict__ A = (const uint16_t *)args.A;
    const uint16_t *__restrict__ B = (const uint16_t *)args.B;

    int tm, tn;
    dgor_tile_of_block(bid, args.tiles_m, args.tiles_n, args.group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int lane = threadIdx.x & 63;
    // wave-uniform, so per-wave offsets and descriptors stay scalar
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int wr = (wave >> 1) * 128, wc = (wave & 1) * 128;
    constexpr uint32_t OOB = 0x80000000u;

    // ---- loader.  Per stage, wavefront w fills blocks 4w..4w+3 of each
    // operand tile.  A is k-strided when given as K x M (TA), B unless given
    // as N x K (TB).  Lane offsets do not change from stage to stage; the
    // descriptors' ranges zero-fill rows past the operand and k rows past K;
    // k-contiguous columns past K are masked per lane in the last stage.  A
    // stage past the last one gets empty ranges: its loads write zeros and
    // keep the wait counts of every stage alike.
    uint32_t a_off[4], b_off[4];
    int a_kc, b_kc;
    ring16::load_offsets<TA>(wave, lane, m0, M, lda, a_off, a_kc);
    ring16::load_offsets<!TB>(wave, lane, n0, N, ldb, b_off, b_kc);
    const uint32_t lds_a = ring + (uint32_t)(4 * wave * 1024);
    const uint32_t lds_b = ring + (uint32_t)(A_BYTES + 4 * wave * 1024);
    struct StageLoads { intx4 ra, rb; uint32_t lds; bool tail; int k_left; };
    auto prep = [&](int st) {
        StageLoads L;
        const int k0 = st * BK;
        L.ra = rsrc_words(TA ? A + (size_t)k0 * lda + m0 : A + (size_t)m0 * lda + k0, 0);
        L.ra.z = ring16::stage_range<TA>(k0, K, m0, M, lda);
        L.rb = rsrc_words(TB ? B + (size_t)n0 * ldb + k0 : B + (size_t)k0 * ldb + n0, 0);
        L.rb.z = ring16::stage_range<!TB>(k0, K, n0, N, ldb);
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

    // ---- fragment reads.  Lane (g, s) = (lane / 16, lane % 16).  A
    // k-contiguous operand block is one 128-bit read of row base + s at unit
    // g; a k-strided one is two transposing reads (k rows 8g..8g+3 and
    // 8g+4..8g+7 of column base + s).
    const int s16 = lane & 15, g = lane >> 4;
    const int kc_sw = 2 * ((s16 >> 2) & 1);
    const int ks_x = 4 * (s16 >> 2) + 2 * (g & 1);
    uint32_t ks_unit[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        ks_unit[j] = (uint32_t)(((2 * j + ((s16 & 3) >> 1)) ^ ks_x) * 16);
    auto kc_lane = [&](uint32_t region, int base) {
        return region + (uint32_t)((base + s16) * 64 + ((g ^ kc_sw) * 16));
    };
    auto ks_lane = [&](uint32_t region, int base) {
        return region + (uint32_t)((8 * g + (s16 >> 2)) * 512 + 8 * (s16 & 1) + 2 * base);
    };
    const uint32_t a_lane = TA ? ks_lane(0, wr) : kc_lane(0, wr);
    const uint32_t b_lane = TB ? kc_lane(A_BYTES, wc) : ks_lane(A_BYTES, wc);
    auto read_block = [&](const uint8_t *buf, uint32_t lane_off, bool kstrided, int blk) -> halfx8 {
        if (!kstrided)
            return *reinterpret_cast<const halfx8 *>(buf + lane_off + blk * 1024);
        const uint8_t *p = buf + lane_off + ks_unit[blk];
        const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4 *)p);
        const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4 *)(p + 2048));
        return __builtin_bit_cast(halfx8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    // read r (0..15) of stage `stage`: A block 0, the eight B blocks, then A
    // blocks 1..7 (the order the next stage's first MFMAs want them)
    auto fread = [&](int stage, int r, halfx8 *fa, halfx8 *fb) {
        const uint8_t *buf = lds + (stage % NBUF) * STAGE_BYTES;
        if (r == 0 || r >= 9) {
            const int i = r == 0 ? 0 : r - 8;
            fa[i] = read_block(buf, a_lane, TA, i);
        } else {
            fb[r - 1] = read_block(buf, b_lane, !TB, r - 1);
        }
    };

    // ---- C tile: lane (g, s) of the wave owns rows 16 i + 4 g + r and
    // columns 16 j + s of the wave's 128 x 128 block.  An element outside C
    // gets an out-of-range lane offset, so it reads zero and is not written.
    const int ldc = args.ldc;
    const int c_col = n0 + wc + s16;
    const int c_rows_left = M - m0 - wr - 4 * g;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(
        args.C + (size_t)(m0 + wr) * ldc + n0 + wc, ((long long)(M - m0 - wr - 1) * ldc + N - n0 - wc) * 4);
    auto c_offset = [&](int col, int rows_left, int i, int j, int r, uint32_t &vo, uint32_t &so) {
        const int ro = 16 * i + r;
        vo = (ro < rows_left && col + 16 * j < N) ? (uint32_t)((4 * g) * ldc + s16 + 16 * j) * 4u : OOB;
        so = (uint32_t)(ro * ldc) * 4u;
    };

    // Accumulators start at zero, or at C itself (ACC: C = alpha (C + op(A) op(B))).
    floatx4 acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (ACC) {
                    uint32_t vo, so;
                    c_offset(c_col, c_rows_left, i, j, r, vo, so);
                    acc[i][j][r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rc, vo, so, 0));
                } else {
                    // an AGPR write, so the compiler keeps the array in AGPRs
                    asm("v_accvgpr_write_b32 %0, 0" : "=a"(acc[i][j][r]));
                }
            }

    // One stage: the 64 MFMAs of stage t from (ca, cb); the 16 fragment
    // reads of stage t + 1 into (na, nb), one after each of the first 16
    // MFMAs, so they complete long before the next stage needs them; the 8
    // loads of stage t + 3, one after every sixth of the remaining MFMAs.
    // Before it: this wavefront's loads of stage t + 1 have landed (those of
    // t + 2 may stay in flight), and the workgroup meets at the barrier.
    // Reads and loads past the last stage touch unused data, harmlessly.
    const int steps = (K + BK - 1) / BK;
    auto stage = [&](int t, halfx8 *ca, halfx8 *cb, halfx8 *na, halfx8 *nb) {
        __builtin_amdgcn_s_waitcnt(wait_vmcnt(LOADS_PER_STAGE));
        __builtin_amdgcn_s_barrier();
        const StageLoads L = prep(t + 3);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < 64; ++m) {
            const int i = m >> 3, j = m & 7;
            acc[i][j] = Op::mfma16(ca[i], cb[j], acc[i][j]);
            if (m < 16)
                fread(t + 1, m, na, nb);
            if (m >= 16 && (m - 16) % 6 == 5)
                load(L, (m - 16) / 6);
            // keep this order: the compiler would otherwise cluster the reads
            // and loads, and move MFMAs across the barrier
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // prologue: loads of stages 0, 1, 2, then the reads of stage 0
    halfx8 fa0[8], fa1[8], fb0[8], fb1[8];
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
    for (int r = 0; r < 16; ++r)
        fread(0, r, fa0, fb0);

    for (int t = 0; t < steps; t += 2) {
        stage(t, fa0, fb0, fa1, fb1);
        if (t + 1 < steps)
            stage(t + 1, fa1, fb1, fa0, fb0);
    }
    // no load may still be writing this workgroup's LDS when it ends
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));

    // Epilogue: alpha times the accumulators (ACC: they started from C),
    // each moved out of its AGPR and scaled on its own (arithmetic on the
    // array as a whole would pull it into ordinary registers, which do not
    // fit beside the fragments), staged through LDS once every wavefront is
    // done with the ring.
    __builtin_amdgcn_s_waitcnt(wait_vmcnt_lgkm0(0));
    __builtin_amdgcn_s_barrier();
    dgor_acc_hazard_wait();
    {
        const int rows_w = M - m0 - wr, cols_w = N - n0 - wc;
        float *Cw = args.C + (size_t)(m0 + wr) * ldc + n0 + wc;
        const bool vec = ((uintptr_t)Cw & 15) == 0 && (ldc & 3) == 0;
        store_c_staged(acc, args.alpha, lds, wave, lane, Cw, ldc, rows_w, cols_w, vec);
    }
}

// The ring kernel for a k-contiguous A (A given as M x K), with A staged two
// k-stages (64 k, 128 bytes of each row) at a time, so that every A row a
// load touches is one whole 128-byte line rather than half of one; B keeps
// one stage per buffer (a k-strided B row of a tile is 512 bytes, whole
// lines already).  Three A pair buffers of 32 KB and four B buffers of
// 16 KB fill the 160 KB of LDS.
//   A pair buffer: 256 rows of 128 bytes (eight 16-byte units), unit c of
//     row r at 8 r + (c ^ ((r >> 1) & 7)); wave w's load j (0..7) fills rows
//     8 n .. 8 n + 7, n = 8 w + j, lane p taking physical unit p % 8 of row
//     8 n + p / 8.  A fragment of stage half h (0: first stage of the pair)
//     is the 128-bit read of unit 4 h + g of row base + s; the swizzle keeps
//     each 16-lane read cycle on distinct banks.
//   B buffers: the layouts, loads and reads of the four-stage ring above.
// Buffers: A pair P is read during stages 2P - 1 and 2P and refilled with
// pair P + 3 during stages 2P + 2 and 2P + 3; B stage t is read during stage
// t - 1 and its buffer refilled with stage t + 4 during stage t + 1.  Each
// stage begins with a wait for the loads issued two stages before (B stage
// t + 1, A pair (t + 1) / 2) and this wavefront's LDS reads, then a barrier.
namespace pair16 {
constexpr int A_PAIR_BYTES = 256 * 64 * 2;           // 32 KB
constexpr int A_PAIRS = 3;
constexpr int B_BYTES = 32 * 256 * 2;                // 16 KB
constexpr int B_REGION = A_PAIRS * A_PAIR_BYTES;     // 96 KB
constexpr int LDS_BYTES = B_REGION + 4 * B_BYTES;    // 160 KB
}  // namespace pair16

template <class Op, bool TB, bool ACC>
__global__ __launch_bounds__(256) void mfma_f16_pair_kernel(RingArgs args)
{
    const int bid = dgor_ring_split(args, 2);   // split-K: this workgroup's k-range and tile
    using namespace pair16;
    constexpr int BK = pipe::BK;                        // 32 k per stage
    static_assert(4 * cstage::WAVE_BYTES <= LDS_BYTES, "the epilogue stages through the ring's LDS");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[LDS_BYTES];
    const uint32_t ring = lds_address(lds);
    const int M = args.M, N = args.N, K = args.K, lda = args.lda, ldb = args.ldb;
    const uint16_t *__restrict__ A = (const uint16_t *)args.A;
    const uint16_t *__restrict__ B = (const uint16_t *)args.B;

    int tm, tn;
    dgor_tile_of_block(bid, args.tiles_m, args.tiles_n, args.group_m, tm, tn);
    const int m0 = tm * 256, n0 = tn * 256;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int wr = (wave >> 1) * 128, wc = (wave & 1) * 128;
    constexpr uint32_t OOB = 0x80000000u;

    // ---- loaders
    // load j's lane offset: a_off[j & 1] plus (j / 2) * 16 rows (wave-uniform)
    uint32_t a_off[2];
    int a_kc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int r = 64 * wave + 8 * j + (lane >> 3);
        const int c = (lane & 7) ^ ((4 * j + (lane >> 4)) & 7);
        a_off[j] = (uint32_t)(r * lda + 8 * c) * 2u;
        a_kc[j] = 8 * c;
    }
    const uint32_t a_row16 = (uint32_t)(16 * lda) * 2u;
    uint32_t b_off[4];
    int b_kc;
    ring16::load_offsets<!TB>(wave, lane, n0, N, ldb, b_off, b_kc);
    const uint32_t lds_a = ring + (uint32_t)(8 * wave * 1024);
    const uint32_t lds_b = ring + (uint32_t)(B_REGION + 4 * wave * 1024);
    struct PairLoads { intx4 r; int k_left; uint32_t dst; };
    auto a_rsrc = [&](int P, uint32_t buf) {
        PairLoads L;
        const int k0 = 2 * BK * P;
        L.k_left = K - k0;
        L.r = rsrc_words(A + (size_t)m0 * lda + k0, 0);
        L.r.z = L.k_left <= 0 ? 0
              : (m0 + 256 <= M ? 0x7fffffff
                               : (int)(((uint32_t)(M - m0 - 1) * (uint32_t)lda + (uint32_t)L.k_left) * 2u));
        L.dst = lds_a + buf;
        return L;
    };
    auto load_a = [&](const PairLoads &L, int j) {
        const uint32_t off = a_kc[j & 1] >= L.k_left ? OOB : a_off[j & 1] + (uint32_t)(j >> 1) * a_row16;
        load_to_lds(L.r, L.dst + (uint32_t)(j * 1024), off);
    };
    struct BLoads { intx4 r; int k_left; uint32_t dst; };
    auto b_rsrc = [&](int st) {
        BLoads L;
        const int k0 = st * BK;
        L.k_left = K - k0;
        L.r = rsrc_words(TB ? B + (size_t)n0 * ldb + k0 : B + (size_t)k0 * ldb + n0, 0);
        L.r.z = ring16::stage_range<!TB>(k0, K, n0, N, ldb);
        L.dst = lds_b + (uint32_t)((st & 3) * B_BYTES);
        return L;
    };
    auto load_b = [&](const BLoads &L, int q) {
        const uint32_t off = (TB && L.k_left < BK && b_kc >= L.k_left) ? OOB : b_off[q];
        load_to_lds(L.r, L.dst + (uint32_t)(q * 1024), off);
    };

    // ---- fragment reads.  Lane (g, s) = (lane / 16, lane % 16).
    const int s16 = lane & 15, g = lane >> 4;
    // A block i of half h: row wr + 16 i + s16, unit 4 h + g, physical unit
    // (4 h + g) ^ ((s16 >> 1) & 7); the bits of 4 h and g do not overlap, so
    // h is applied by XOR on bit 6 of the byte offset.
    const uint32_t a_lane = (uint32_t)((wr + s16) * 128) | (uint32_t)((g ^ ((s16 >> 1) & 7)) * 16);
    // B blocks: as in the four-stage ring
    const int kc_sw = 2 * ((s16 >> 2) & 1);
    const int ks_x = 4 * (s16 >> 2) + 2 * (g & 1);
    uint32_t ks_unit[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        ks_unit[j] = (uint32_t)(((2 * j + ((s16 & 3) >> 1)) ^ ks_x) * 16);
    const uint32_t b_lane = TB ? (uint32_t)(B_REGION + (wc + s16) * 64 + ((g ^ kc_sw) * 16))
                               : (uint32_t)(B_REGION + (8 * g + (s16 >> 2)) * 512 + 8 * (s16 & 1) + 2 * wc);
    struct ReadSrc { uint32_t a_buf; int a_half; uint32_t b_buf; };
    auto read_a = [&](const ReadSrc &R, int i) -> halfx8 {
        const uint32_t addr = (a_lane ^ (uint32_t)(64 * R.a_half)) + R.a_buf + (uint32_t)(i * 2048);
        return *reinterpret_cast<const halfx8 *>(lds + addr);
    };
    auto read_b = [&](const ReadSrc &R, int j) -> halfx8 {
        if (TB)
            return *reinterpret_cast<const halfx8 *>(lds + b_lane + R.b_buf + j * 1024);
        const uint8_t *p = lds + b_lane + R.b_buf + ks_unit[j];
        const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4 *)p);
        const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4 *)(p + 2048));
        return __builtin_bit_cast(halfx8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    // read r (0..15): A block 0, the eight B blocks, then A blocks 1..7
    auto fread = [&](const ReadSrc &R, int r, halfx8 *fa, halfx8 *fb) {
        if (r == 0 || r >= 9)
            fa[r == 0 ? 0 : r - 8] = read_a(R, r == 0 ? 0 : r - 8);
        else
            fb[r - 1] = read_b(R, r - 1);
    };

    // ---- C tile: lane (g, s) of the wave owns rows 16 i + 4 g + r and
    // columns 16 j + s of the wave's 128 x 128 block.  An element outside C
    // gets an out-of-range lane offset, so it reads zero and is not written.
    const int ldc = args.ldc;
    const int c_col = n0 + wc + s16;
    const int c_rows_left = M - m0 - wr - 4 * g;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(
        args.C + (size_t)(m0 + wr) * ldc + n0 + wc, ((long long)(M - m0 - wr - 1) * ldc + N - n0 - wc) * 4);
    auto c_offset = [&](int col, int rows_left, int i, int j, int r, uint32_t &vo, uint32_t &so) {
        const int ro = 16 * i + r;
        vo = (ro < rows_left && col + 16 * j < N) ? (uint32_t)((4 * g) * ldc + s16 + 16 * j) * 4u : OOB;
        so = (uint32_t)(ro * ldc) * 4u;
    };

    // Accumulators start at zero, or at C itself (ACC: C = alpha (C + A op(B))).
    floatx4 acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (ACC) {
                    uint32_t vo, so;
                    c_offset(c_col, c_rows_left, i, j, r, vo, so);
                    acc[i][j][r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rc, vo, so, 0));
                } else {
                    // an AGPR write, so the compiler keeps the array in AGPRs
                    asm("v_accvgpr_write_b32 %0, 0" : "=a"(acc[i][j][r]));
                }
            }

    // One stage t (parity `par` within its pair): the 64 MFMAs from (ca, cb);
    // the 16 fragment reads of stage t + 1 (source R) into (na, nb), one after
    // each of the first 16 MFMAs; the stage's 8 loads (B stage t + 3, then
    // half `par` of A pair t / 2 + 2), one after every sixth of the rest.
    struct StageLoads { BLoads b; PairLoads a; };
    auto stage = [&](int par, const StageLoads &L, const ReadSrc &R, halfx8 *ca, halfx8 *cb, halfx8 *na,
                     halfx8 *nb) {
#pragma unroll
        for (int m = 0; m < 64; ++m) {
            const int i = m >> 3, j = m & 7;
            acc[i][j] = Op::mfma16(ca[i], cb[j], acc[i][j]);
            if (m < 16)
                fread(R, m, na, nb);
            if (m >= 16 && (m - 16) % 6 == 5) {
                const int ld = (m - 16) / 6;   // 0..7
                if (ld < 4)
                    load_b(L.b, ld);
                else
                    load_a(L.a, 4 * par + ld - 4);
            }
            // keep this order: the compiler would otherwise cluster the reads
            // and loads, and move MFMAs across the barrier
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto stage_begin = [&](int t, uint32_t a_load_buf) {
        if (t == 0)
            __builtin_amdgcn_s_waitcnt(wait_vmcnt_lgkm0(12));
        else
            __builtin_amdgcn_s_waitcnt(wait_vmcnt_lgkm0(8));
        __builtin_amdgcn_s_barrier();
        const StageLoads L{b_rsrc(t + 3), a_rsrc((t >> 1) + 2, a_load_buf)};
        __builtin_amdgcn_sched_barrier(0);
        return L;
    };
    auto b_buf = [](int st) { return (uint32_t)((st & 3) * B_BYTES); };
    auto next_pair = [](uint32_t pb) { return pb == (uint32_t)((A_PAIRS - 1) * A_PAIR_BYTES) ? 0u : pb + A_PAIR_BYTES; };

    // prologue: A pair 0, B stages 0 and 1, A pair 1, B stage 2; then the
    // reads of stage 0 (A pair 0 and B stage 0 landed: 16 younger loads fly)
    halfx8 fa0[8], fa1[8], fb0[8], fb1[8];
    {
        const PairLoads L = a_rsrc(0, 0);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            load_a(L, j);
    }
#pragma unroll
    for (int st = 0; st < 2; ++st) {
        const BLoads L = b_rsrc(st);
#pragma unroll
        for (int q = 0; q < 4; ++q)
            load_b(L, q);
    }
    {
        const PairLoads L = a_rsrc(1, A_PAIR_BYTES);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            load_a(L, j);
    }
    {
        const BLoads L = b_rsrc(2);
#pragma unroll
        for (int q = 0; q < 4; ++q)
            load_b(L, q);
    }
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(16));
    __builtin_amdgcn_s_barrier();
    {
        const ReadSrc R0{0u, 0, b_buf(0)};
#pragma unroll
        for (int r = 0; r < 16; ++r)
            fread(R0, r, fa0, fb0);
    }

    // two stages (one A pair) per trip; pa, pa1, pa2: buffers of pairs P, P+1, P+2
    const int steps = (K + BK - 1) / BK;
    uint32_t pa = 0;
    for (int t = 0; t < steps; t += 2) {
        const uint32_t pa1 = next_pair(pa), pa2 = next_pair(pa1);
        StageLoads L = stage_begin(t, pa2);
        stage(0, L, ReadSrc{pa, 1, b_buf(t + 1)}, fa0, fb0, fa1, fb1);
        if (t + 1 < steps) {
            L = stage_begin(t + 1, pa2);
            stage(1, L, ReadSrc{pa1, 0, b_buf(t + 2)}, fa1, fb1, fa0, fb0);
        }
        pa = pa1;
    }
    // no load may still be writing this workgroup's LDS when it ends
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));

    // Epilogue: as in the four-stage ring, through LDS once every
    // wavefront is done with the ring.
    __builtin_amdgcn_s_waitcnt(wait_vmcnt_lgkm0(0));
    __builtin_amdgcn_s_barrier();
    dgor_acc_hazard_wait();
    {
        const int rows_w = M - m0 - wr, cols_w = N - n0 - wc;
        float *Cw = args.C + (size_t)(m0 + wr) * ldc + n0 + wc;
        const bool vec = ((uintptr_t)Cw & 15) == 0 && (ldc & 3) == 0;
        store_c_staged(acc, args.alpha, lds, wave, lane, Cw, ldc, rows_w, cols_w, vec);
    }
}

// Epilogue of the 128 x 128 ring: a wavefront's block of 64 columns and FM
// 16-row MFMA blocks leaves through its own 8 KB LDS region in FM / 2 rounds
// of 32 rows, as in the 256 x 256 rings; element (row, col) of a round sits
// at row 256 + 16 ((col / 4) ^ 4 ((row / 4) % 4)) + 4 (col % 4), which keeps
// both the 4-byte writes (lane (g, s) of block j at unit 4 (j ^ g) + s / 4)
// and the 16-byte reads along the rows free of bank conflicts.  acc holds the
// sums already read out of the accumulator registers.
template <int FM>
__device__ __forceinline__ void store_c_staged_w64(const floatx4 (&acc)[FM][4], float alpha, uint8_t *lds, int wave,
                                                   int lane, float *Cw, int ldc, int rows_left, int cols_left, bool vec)
{
    typedef unsigned uintx4 __attribute__((ext_vector_type(4)));
    constexpr uint32_t OOB = 0x80000000u;
    uint8_t *w = lds + wave * 8192;
    const int g = lane >> 4, s16 = lane & 15;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(
        Cw, rows_left > 0 && cols_left > 0 ? ((long long)(rows_left - 1) * ldc + cols_left) * 4 : 0);
#pragma unroll
    for (int q = 0; q < FM / 2; ++q) {
#pragma unroll
        for (int ii = 0; ii < 2; ++ii)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    *reinterpret_cast<float *>(w + (16 * ii + 4 * g + r) * 256 + (4 * (j ^ g) + (s16 >> 2)) * 16 +
                                               (s16 & 3) * 4) = acc[2 * q + ii][j][r] * alpha;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int row = (lane >> 4) + 4 * t, c = lane & 15;
            const floatx4 v = *reinterpret_cast<const floatx4 *>(w + row * 256 + ((c ^ (4 * (t & 3))) * 16));
            const int grow = 32 * q + row, col = 4 * c;
            if (grow < rows_left) {
                const uint32_t o = (uint32_t)(grow * ldc + col) * 4u;
                if (vec && col + 4 <= cols_left) {
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(uintx4, v), rc, o, 0, 0);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[e]), rc,
                                                              col + e < cols_left ? o + 4u * e : OOB, 0, 0);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// The 128 x 128 ring for mid-size problems (A given as M x K, B as K x N, C =
// A B): the pair ring's design at half the tile, four wavefronts of 64 x 64
// (4 x 4 blocks of v_mfma_f32_16x16x32, 64 accumulators a lane) and 80 KB of
// LDS, so two workgroups share a compute unit and cover each other's waits.
//   A pair buffer (16 KB): 128 rows of 128 bytes, unit c of row r at
//     8 r + (c ^ ((r >> 1) & 7)); wave w's load j (0..3) fills rows
//     32 w + 8 j .. + 7, two loads a stage (half par of the pair).
//   B stage (8 KB): 32 k rows of 256 bytes, unit u of row k at
//     16 k + (u ^ (2 (k & 3) + 8 ((k >> 3) & 1))); wave w's load q (0..1)
//     fills k rows 4 (2 w + q) .. + 3.  A transposing-read cycle (32 lanes)
//     takes two 16-byte units of each of k rows 8 g .. 8 g + 3, g = 0, 1:
//     the swizzle gives the eight rows eight distinct unit pairs.
//   Pipeline, waits and the fragment order as in the pair ring, with 16
//   MFMAs, 8 fragment reads and 4 loads a wavefront and stage.
//   KS = 2 (shapes with at most one tile per compute unit, whose second
//   workgroup slot would stay empty): eight wavefronts in two groups of
//   four, group g over the g-th half of the k-stages (A, B and K shifted to
//   the group's k range) through a ring of its own (160 KB in all); both
//   groups run the same number of stages, so they meet at the same
//   barriers; at the end group 1 hands its sums to group 0 through its ring,
//   which adds them in that fixed order and stores C.
namespace pair128 {
constexpr int A_PAIR_BYTES = 128 * 64 * 2;           // 16 KB
constexpr int A_PAIRS = 3;
constexpr int B_BYTES = 32 * 128 * 2;                // 8 KB
constexpr int B_REGION = A_PAIRS * A_PAIR_BYTES;     // 48 KB
constexpr int LDS_BYTES = B_REGION + 4 * B_BYTES;    // 80 KB: two workgroups a CU
}  // namespace pair128

template <class Op, int KS>
__global__ __launch_bounds__(256 * KS, 2 / KS) void mfma_f16_pair128_kernel(RingArgs args)
{
    using namespace pair128;
    constexpr int BK = pipe::BK;
    __shared__ __attribute__((aligned(1024))) uint8_t lds_all[KS * LDS_BYTES];
    const int wave_all = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int grp = wave_all >> 2;
    uint8_t *const lds = lds_all + grp * LDS_BYTES;
    const uint32_t ring = lds_address(lds);
    const int M = args.M, N = args.N, lda = args.lda, ldb = args.ldb;
    const int steps_all = (args.K + BK - 1) / BK;
    const int steps = (steps_all + KS - 1) / KS;
    const int kbase = grp * steps * BK;
    const int K = args.K < kbase + steps * BK ? args.K - kbase : steps * BK;   // the group's k extent
    const uint16_t *__restrict__ A = (const uint16_t *)args.A + kbase;
    const uint16_t *__restrict__ B = (const uint16_t *)args.B + (size_t)kbase * ldb;

    int tm, tn;
    dgor_tile_of_block((int)blockIdx.x, args.tiles_m, args.tiles_n, args.group_m, tm, tn);
    const int m0 = tm * 128, n0 = tn * 128;
    const int lane = threadIdx.x & 63;
    const int wave = wave_all & 3;
    const int wr = (wave >> 1) * 64, wc = (wave & 1) * 64;
    constexpr uint32_t OOB = 0x80000000u;

    uint32_t a_off[2];
    int a_kc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int r = 32 * wave + 8 * j + (lane >> 3);
        const int c = (lane & 7) ^ ((4 * j + (lane >> 4)) & 7);
        a_off[j] = (uint32_t)(r * lda + 8 * c) * 2u;
        a_kc[j] = 8 * c;
    }
    const uint32_t a_row16 = (uint32_t)(16 * lda) * 2u;
    uint32_t b_off[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int k = 4 * (2 * wave + q) + (lane >> 4);
        const int u = (lane & 15) ^ (2 * (k & 3) + 8 * ((k >> 3) & 1));
        b_off[q] = n0 + 8 * u < N ? (uint32_t)(k * ldb + 8 * u) * 2u : OOB;
    }
    const uint32_t lds_a = ring + (uint32_t)(4 * wave * 1024);
    const uint32_t lds_b = ring + (uint32_t)(B_REGION + 2 * wave * 1024);
    struct PairLoads { intx4 r; int k_left; uint32_t dst; };
    auto a_rsrc = [&](int P, uint32_t buf) {
        PairLoads L;
        const int k0 = 2 * BK * P;
        L.k_left = K - k0;
        L.r = rsrc_words(A + (size_t)m0 * lda + k0, 0);
        L.r.z = L.k_left <= 0 ? 0
              : (m0 + 128 <= M ? 0x7fffffff
                               : (int)(((uint32_t)(M - m0 - 1) * (uint32_t)lda + (uint32_t)L.k_left) * 2u));
        L.dst = lds_a + buf;
        return L;
    };
    auto load_a = [&](const PairLoads &L, int j) {
        const uint32_t off = a_kc[j & 1] >= L.k_left ? OOB : a_off[j & 1] + (uint32_t)(j >> 1) * a_row16;
        load_to_lds(L.r, L.dst + (uint32_t)(j * 1024), off);
    };
    struct BLoads { intx4 r; uint32_t dst; };
    auto b_rsrc = [&](int st) {
        BLoads L;
        const int k0 = st * BK;
        L.r = rsrc_words(B + (size_t)k0 * ldb + n0, 0);
        L.r.z = ring16::stage_range<true>(k0, K, n0, N, ldb);
        L.dst = lds_b + (uint32_t)((st & 3) * B_BYTES);
        return L;
    };
    auto load_b = [&](const BLoads &L, int q) { load_to_lds(L.r, L.dst + (uint32_t)(q * 1024), b_off[q]); };

    const int s16 = lane & 15, g = lane >> 4;
    const uint32_t a_lane = (uint32_t)((wr + s16) * 128) | (uint32_t)((g ^ ((s16 >> 1) & 7)) * 16);
    const int ks_x = 2 * ((s16 >> 2) & 3) + 8 * (g & 1);
    uint32_t ks_unit[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        ks_unit[j] = (uint32_t)(((wc / 8 + 2 * j + ((s16 & 3) >> 1)) ^ ks_x) * 16);
    const uint32_t b_lane = (uint32_t)(B_REGION + (8 * g + (s16 >> 2)) * 256 + 8 * (s16 & 1));
    struct ReadSrc { uint32_t a_buf; int a_half; uint32_t b_buf; };
    auto read_a = [&](const ReadSrc &R, int i) -> halfx8 {
        const uint32_t addr = (a_lane ^ (uint32_t)(64 * R.a_half)) + R.a_buf + (uint32_t)(i * 2048);
        return *reinterpret_cast<const halfx8 *>(lds + addr);
    };
    auto read_b = [&](const ReadSrc &R, int j) -> halfx8 {
        const uint8_t *p = lds + b_lane + R.b_buf + ks_unit[j];
        const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4 *)p);
        const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4 *)(p + 1024));
        return __builtin_bit_cast(halfx8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    // read r (0..7): A block 0, the four B blocks, then A blocks 1..3
    auto fread = [&](const ReadSrc &R, int r, halfx8 *fa, halfx8 *fb) {
        if (r == 0 || r >= 5)
            fa[r == 0 ? 0 : r - 4] = read_a(R, r == 0 ? 0 : r - 4);
        else
            fb[r - 1] = read_b(R, r - 1);
    };

    floatx4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                asm("v_accvgpr_write_b32 %0, 0" : "=a"(acc[i][j][r]));

    struct StageLoads { BLoads b; PairLoads a; };
    auto stage = [&](int par, const StageLoads &L, const ReadSrc &R, halfx8 *ca, halfx8 *cb, halfx8 *na,
                     halfx8 *nb) {
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            const int i = m >> 2, j = m & 3;
            acc[i][j] = Op::mfma16(ca[i], cb[j], acc[i][j]);
            if (m < 8)
                fread(R, m, na, nb);
            if (m >= 8 && (m & 1)) {
                const int ld = (m - 8) >> 1;   // 0..3
                if (ld < 2)
                    load_b(L.b, ld);
                else
                    load_a(L.a, 2 * par + ld - 2);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto stage_begin = [&](int t, uint32_t a_load_buf) {
        if (t == 0)
            __builtin_amdgcn_s_waitcnt(wait_vmcnt_lgkm0(6));
        else
            __builtin_amdgcn_s_waitcnt(wait_vmcnt_lgkm0(4));
        __builtin_amdgcn_s_barrier();
        const StageLoads L{b_rsrc(t + 3), a_rsrc((t >> 1) + 2, a_load_buf)};
        __builtin_amdgcn_sched_barrier(0);
        return L;
    };
    auto b_buf = [](int st) { return (uint32_t)((st & 3) * B_BYTES); };
    auto next_pair = [](uint32_t pb) { return pb == (uint32_t)((A_PAIRS - 1) * A_PAIR_BYTES) ? 0u : pb + A_PAIR_BYTES; };

    halfx8 fa0[4], fa1[4], fb0[4], fb1[4];
    {
        const PairLoads L = a_rsrc(0, 0);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            load_a(L, j);
    }
#pragma unroll
    for (int st = 0; st < 2; ++st) {
        const BLoads L = b_rsrc(st);
#pragma unroll
        for (int q = 0; q < 2; ++q)
            load_b(L, q);
    }
    {
        const PairLoads L = a_rsrc(1, A_PAIR_BYTES);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            load_a(L, j);
    }
    {
        const BLoads L = b_rsrc(2);
#pragma unroll
        for (int q = 0; q < 2; ++q)
            load_b(L, q);
    }
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(8));
    __builtin_amdgcn_s_barrier();
    {
        const ReadSrc R0{0u, 0, b_buf(0)};
#pragma unroll
        for (int r = 0; r < 8; ++r)
            fread(R0, r, fa0, fb0);
    }

    uint32_t pa = 0;
    for (int t = 0; t < steps; t += 2) {
        const uint32_t pa1 = next_pair(pa), pa2 = next_pair(pa1);
        StageLoads L = stage_begin(t, pa2);
        stage(0, L, ReadSrc{pa, 1, b_buf(t + 1)}, fa0, fb0, fa1, fb1);
        if (t + 1 < steps) {
            L = stage_begin(t + 1, pa2);
            stage(1, L, ReadSrc{pa1, 0, b_buf(t + 2)}, fa1, fb1, fa0, fb0);
        }
        pa = pa1;
    }
    __builtin_amdgcn_s_waitcnt(wait_vmcnt_lgkm0(0));
    __builtin_amdgcn_s_barrier();
    dgor_acc_hazard_wait();
    floatx4 tot[4][4];
    if constexpr (KS == 2) {
        floatx4 *part = reinterpret_cast<floatx4 *>(lds_all + LDS_BYTES);
        if (grp == 1) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    floatx4 v;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        v[r] = dgor_acc_read(acc[i][j][r]);
                    part[((i * 4 + j) * 4 + wave) * 64 + lane] = v;
                }
        }
        __builtin_amdgcn_s_barrier();
        if (grp == 1)
            return;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const floatx4 v = part[((i * 4 + j) * 4 + wave) * 64 + lane];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    tot[i][j][r] = dgor_acc_read(acc[i][j][r]) + v[r];
            }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    tot[i][j][r] = dgor_acc_read(acc[i][j][r]);
    }
    {
        const int ldc = args.ldc;
        float *Cw = args.C + (size_t)(m0 + wr) * ldc + n0 + wc;
        const bool vec = ((uintptr_t)Cw & 15) == 0 && (ldc & 3) == 0;
        store_c_staged_w64<4>(tot, args.alpha, lds, wave, lane, Cw, ldc, M - m0 - wr, N - n0 - wc, vec);
    }
}


template <class Op, int BM, int BN, int BK, int WM, int WN>
hipError_t launch_cfg(const Problem &p, const gemm_plan &plan, hipStream_t s)
{
    const uint16_t *A = (const uint16_t *)p.A, *B = (const uint16_t *)p.B;
    const dim3 grid(plan.grid_x * plan.grid_y), blk(64 * WM * WN);
    const int gm = 4;
    if (p.vec_a && p.vec_b)
        hipLaunchKernelGGL((mfma_f16_kernel<Op, BM, BN, BK, WM, WN, true, true>), grid, blk, 0, s,
                           p.M, p.N, p.K, A, B, p.C, plan.grid_y, plan.grid_x, gm);
    else if (p.vec_a)
        hipLaunchKernelGGL((mfma_f16_kernel<Op, BM, BN, BK, WM, WN, true, false>), grid, blk, 0, s,
                           p.M, p.N, p.K, A, B, p.C, plan.grid_y, plan.grid_x, gm);
    else if (p.vec_b)
        hipLaunchKernelGGL((mfma_f16_kernel<Op, BM, BN, BK, WM, WN, false, true>), grid, blk, 0, s,
                           p.M, p.N, p.K, A, B, p.C, plan.grid_y, plan.grid_x, gm);
    else
        hipLaunchKernelGGL((mfma_f16_kernel<Op, BM, BN, BK, WM, WN, false, false>), grid, blk, 0, s,
                           p.M, p.N, p.K, A, B, p.C, plan.grid_y, plan.grid_x, gm);
    return hipGetLastError();
}

template <class Op, bool TA, bool TB>
hipError_t launch_ring(const RingArgs &a, hipStream_t s)
{
    const dim3 grid(a.tiles_m * a.tiles_n * (a.splits > 1 ? a.splits : 1));
    if constexpr (!TA) {   // k-contiguous A: whole-line A loads
        if (a.accumulate)
            hipLaunchKernelGGL((mfma_f16_pair_kernel<Op, TB, true>), grid, dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL((mfma_f16_pair_kernel<Op, TB, false>), grid, dim3(256), 0, s, a);
    } else {
        if (a.accumulate)
            hipLaunchKernelGGL((mfma_f16_pipe_kernel<Op, TA, TB, true>), grid, dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL((mfma_f16_pipe_kernel<Op, TA, TB, false>), grid, dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

template <class Op>
hipError_t launch_ring_any(const RingArgs &a, hipStream_t s)
{
    if (a.trans_a)
        return a.trans_b ? launch_ring<Op, true, true>(a, s) : launch_ring<Op, true, false>(a, s);
    return a.trans_b ? launch_ring<Op, false, true>(a, s) : launch_ring<Op, false, false>(a, s);
}

template <class Op>
hipError_t launch_op(const Problem &p, const gemm_plan &plan, hipStream_t s)
{
    if (plan.tile_m == 256 && plan.tile_n == 256) {
        if (direct_lds_applies(plan.tile_m, 256, p.vec_a, p.vec_b, p.N, p.K)) {
            return launch_ring<Op, false, false>(ring_args_nn(p, plan), s);
        }
        return launch_cfg<Op, 256, 256, 32, 2, 2>(p, plan, s);
    }
    if (plan.tile_m == 128 && plan.tile_n == 128) {
        if (f16_ring128_applies(p.vec_a, p.vec_b, p.N, p.K)) {
            if (plan.threads == 512)   // two groups over k
                hipLaunchKernelGGL((mfma_f16_pair128_kernel<Op, 2>), dim3(plan.grid_x * plan.grid_y), dim3(512), 0,
                                   s, ring_args_nn(p, plan));
            else
                hipLaunchKernelGGL((mfma_f16_pair128_kernel<Op, 1>), dim3(plan.grid_x * plan.grid_y), dim3(256), 0,
                                   s, ring_args_nn(p, plan));
            return hipGetLastError();
        }
        return launch_cfg<Op, 128, 128, 32, 2, 2>(p, plan, s);
    }
    if (plan.tile_m == 64 && plan.tile_n == 64)
        return launch_cfg<Op, 64, 64, 32, 1, 2>(p, plan, s);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_mfma_f16(const Problem &p, const gemm_plan &plan, hipStream_t s, bool bf16)
{
    return bf16 ? launch_op<OpBF16>(p, plan, s) : launch_op<OpF16>(p, plan, s);
}

hipError_t launch_ring16(const RingArgs &a, hipStream_t s, bool bf16)
{
    return bf16 ? launch_ring_any<OpBF16>(a, s) : launch_ring_any<OpF16>(a, s);
}

}  // namespace dgor
