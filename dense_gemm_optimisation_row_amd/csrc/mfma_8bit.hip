// 8-bit inputs on the matrix cores: FP8 (OCP E4M3 and E5M2) with FP32
// accumulation and output, and INT8 with INT32 accumulation and output
// ("Lesson 8: how a GPU does matrix multiply", section 22 lists FP8 and INT8
// among the matrix units' input formats; its sections 24-25 give the
// staged, double-buffered K-loop these kernels deepen into a ring).
//
// Two kernels with one data movement, and half-size variants of both for
// mid-size products (mfma_i8_pair128_kernel, mfma_fp8_pair128_kernel,
// described where they are defined).  A workgroup of four wavefronts computes a 256 x 256 tile of C
// in 64-deep k-steps; each wavefront a 128 x 128 quarter with 256
// accumulator registers per lane.
//   FP8 (mfma_8bit_ring_kernel): 4 x 4 blocks of 32 x 32, one
//     v_mfma_scale_f32_32x32x64_f8f6f4 (unit scales) per block and k-step.
//   INT8 (mfma_i8_pair_kernel): 8 x 8 blocks of 16 x 16, one
//     v_mfma_i32_16x16x64_i8 per block and k-step.
// Why the formats take different blocks.  At 8192^3 both kernels run at the
// socket power limit, where the clock falls until the power fits, so what
// sets their rate is the energy of an operation.  An MFMA reads its A, B and
// C registers and writes D: v_mfma_i32_32x32x32_i8 moves 4 + 4 + 16 + 16
// registers a lane for 64 K operations, v_mfma_i32_16x16x64_i8 4 x 4 for 32 K,
// a fifth less register traffic per operation; on the 16 x 16 blocks the
// INT8 product settles at a 16% higher clock under the limit (2022 against
// 1746 MHz) and runs 4% faster although its matrix cores are less busy per
// cycle.  For FP8, v_mfma_scale_f32_16x16x128_f8f6f4 moves the same register
// bytes per operation as the 32 x 32 x 64 shape, and its 32-byte fragments
// for an 8 x 8 grid of blocks, double-buffered, would not fit beside the
// accumulators.
//
// Shared by both kernels:
// * Loads go straight from global memory into LDS (buffer_load_dwordx4 ...
//   lds): one instruction moves 64 lanes x 16 bytes into 1 KB of LDS, lane p
//   landing at byte 16 p, and a lane whose offset is out of range writes
//   zeros, which zero-fills every edge.
// * LDS: A is staged two k-steps (an "A pair", 128 bytes of each of the
//   tile's 256 rows) at a time, so every A row a load touches is one whole
//   128-byte line, into three 32 KB pair buffers; B one k-step (64 k rows of
//   the tile's 256 bytes, whole lines already) at a time into four 16 KB
//   buffers.  160 KB in all.
//   A pair buffer: unit c (16 bytes) of row r at 8 r + (c ^ ((r >> 1) & 7));
//     wave w's load j (0..7) fills rows 8 n .. 8 n + 7, n = 8 w + j, lane p
//     taking physical unit p % 8 of row 8 n + p / 8.
//   B buffer: unit u of k row k at 16 k + (u ^ x(k)), with x(k) = 2 (k & 7)
//     for FP8 and 2 (k & 7) | ((k >> 4) & 1) for INT8 (below); wave w's load
//     q fills rows 4 n .. 4 n + 3, n = 4 w + q, lane p taking physical unit
//     p % 16 of row 4 n + p / 16.
//   A fragments are 128-bit reads of one row; B fragments are transposing
//   reads (ds_read_b64_tr_b8): in a group of 16 lanes, source lane s points
//   at 8 bytes of k row kb + s / 2, columns nb + 8 (s % 2) .. + 7, and output
//   lane i receives k rows kb .. kb + 7 of column nb + i.  The swizzles keep
//   the reads free of bank conflicts under the LDS rule measured for the
//   16-bit ring (a 128-bit read is served in four cycles of 16 lanes that
//   agree in lane bit 5 and the parity of lane bits 2..4; a 64-bit read 32
//   lanes a cycle; a cycle is conflict-free when its 16-byte units, or
//   8-byte halves, differ modulo the 256-byte row of banks).
// * Pipeline.  The fragments of step s + 1 are read during step s; during
//   step s each wavefront also issues its 8 loads: B step s + 3 (into the
//   buffer of step s - 1) and half s % 2 of A pair s / 2 + 2.  Before step
//   s: one wait for this wavefront's loads of step s + 1 (the later ones stay
//   in flight) and its own LDS reads, then one barrier, after which every
//   load of step s + 1 has landed and no wavefront still reads a buffer the
//   step's loads overwrite.  Descriptor ranges end at the operand's last row
//   and at K, so everything past them loads as zero; A lanes past K in the
//   last pair are masked (K is a multiple of 16).
#include "common.h"
#include "lds_dma.h"

namespace dgor {
namespace {

typedef int intx8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef int intx2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) intx2 lds_intx2;

// FP8: one v_mfma_scale_f32_32x32x64_f8f6f4 per block and k-step, with unit
// block scales (E8M0 127 = 2^0); format code 0 is E4M3, 1 is E5M2.
template <int FMT>
struct OpFp8 {
    __device__ static floatx16 mma(const intx8 &a, const intx8 &b, floatx16 c)
    {
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FMT, FMT, 0, 127, 0, 127);
    }
};

namespace ring8 {
constexpr int BM = 256, BN = 256, BK = 64;
constexpr int A_PAIR_BYTES = BM * 2 * BK;            // 32 KB: A for two k-steps
constexpr int A_PAIRS = 3;
constexpr int B_BYTES = BK * BN;                     // 16 KB: B for one k-step
constexpr int B_BUFS = 4;
constexpr int B_REGION = A_PAIRS * A_PAIR_BYTES;     // 96 KB
constexpr int LDS_BYTES = B_REGION + B_BUFS * B_BYTES;   // 160 KB
constexpr int LOADS_PER_STEP = 8;                    // per wavefront: 4 of A, 4 of B
}  // namespace ring8

// The FP8 product (A M x K, B K x N, row-major).
//   Fragments.  Lane l = (r, g) = (l % 32, l / 32) holds the k-values
//   32 g .. 32 g + 31 of the step of row r of its A block (two 128-bit
//   reads) and of column r of its B block (four transposing reads).  The
//   matrix unit pairs the same register bytes of A and B lanes, so each k of
//   the step is summed exactly once.  Output: element e of lane l is row
//   8 (e / 4) + 4 g + e % 4, column l % 32 of the block.
template <class Op>
__global__ __launch_bounds__(256) void mfma_8bit_ring_kernel(RingArgs args)
{
    using namespace ring8;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[LDS_BYTES];
    const uint32_t ring = lds_address(lds);
    const int M = args.M, N = args.N, K = args.K, lda = args.lda, ldb = args.ldb;
    const uint8_t *__restrict__ A = (const uint8_t *)args.A;
    const uint8_t *__restrict__ B = (const uint8_t *)args.B;

    int tm, tn;
    dgor_tile_of_block(blockIdx.x, args.tiles_m, args.tiles_n, args.group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int wr = (wave >> 1) * 128, wc = (wave & 1) * 128;
    constexpr uint32_t OOB = 0x80000000u;

    // ---- loader.  Step s of B lives in B buffer s % 4; A pair P in A
    // buffer P % 3.  A load j's lane offset: a_off[j & 1] plus (j / 2) * 16
    // rows (wave-uniform).
    uint32_t a_off[2], b_off[4];
    int a_kc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int r = 64 * wave + 8 * j + (lane >> 3);
        const int c = (lane & 7) ^ ((4 * j + (lane >> 4)) & 7);
        a_off[j] = (uint32_t)(r * lda + 16 * c);
        a_kc[j] = 16 * c;
    }
    const uint32_t a_row16 = (uint32_t)(16 * lda);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int k = 4 * (4 * wave + q) + (lane >> 4);
        const int u = (lane & 15) ^ (2 * (k & 7));
        b_off[q] = n0 + 16 * u < N ? (uint32_t)(k * ldb + 16 * u) : OOB;
    }
    const uint32_t lds_a = ring + (uint32_t)(8 * wave * 1024);
    const uint32_t lds_b = ring + (uint32_t)(B_REGION + 4 * wave * 1024);
    // A pair P (into the pair buffer at byte offset buf): its descriptor,
    // and this wave's load j (0..7) of it
    struct PairLoads { intx4 r; int k_left; uint32_t dst; };
    auto a_rsrc = [&](int P, uint32_t buf) {
        PairLoads L;
        const int k0 = 2 * BK * P;
        L.k_left = K - k0;
        L.r = rsrc_words(A + (size_t)m0 * lda + k0, 0);
        L.r.z = L.k_left <= 0 ? 0
              : (m0 + BM <= M ? 0x7fffffff
                              : (int)((uint32_t)(M - m0 - 1) * (uint32_t)lda + (uint32_t)L.k_left));
        L.dst = lds_a + buf;
        return L;
    };
    auto load_a = [&](const PairLoads &L, int j) {
        const uint32_t off = a_kc[j & 1] >= L.k_left ? OOB : a_off[j & 1] + (uint32_t)(j >> 1) * a_row16;
        load_to_lds(L.r, L.dst + (uint32_t)(j * 1024), off);
    };
    // B step st: its descriptor
    auto b_rsrc = [&](int st) {
        const int k0 = BK * st, k_left = K - k0;
        intx4 r = rsrc_words(B + (size_t)k0 * ldb + n0, 0);
        r.z = k_left <= 0 ? 0
            : (k_left >= BK ? 0x7fffffff : (int)((uint32_t)(k_left - 1) * (uint32_t)ldb + (uint32_t)(N - n0)));
        return r;
    };

    // ---- fragment reads
    const int r32 = lane & 31, g = lane >> 5;
    const int s16 = lane & 15, hg = (lane >> 4) & 1;
    // A block blk of a step: row wr + 32 blk + r32 of its pair buffer, logical
    // unit c = 4 half + 2 g + u (u = 0, 1: the lane's two units), physical
    // unit c ^ ((row >> 1) & 7).  The bits of c do not overlap, so the lane
    // part (2 g ^ ((r32 >> 1) & 7)) is folded in once and (half, u) applied by
    // XOR on bits 4..6 of the byte offset, which the row part leaves clear.
    const uint32_t a_lane = (uint32_t)((wr + r32) * 128) | (uint32_t)(((2 * g) ^ ((r32 >> 1) & 7)) * 16);
    auto a_lane_at = [&](int half, int u) { return a_lane ^ (uint32_t)((4 * half + u) * 16); };
    // B block blk, read q (8 k rows): row 32 g + 8 q + s16 / 2, byte
    // 8 (s16 % 2) of logical unit wc / 16 + 2 blk + hg, at physical unit
    // unit ^ (s16 & 14); wc (0 or 128) sets unit bit 8, applied by XOR.
    uint32_t b_lane[4];
#pragma unroll
    for (int b = 0; b < 4; ++b)
        b_lane[b] = (uint32_t)(B_REGION + (32 * g + (s16 >> 1)) * 256 + 8 * (s16 & 1)) +
                    (((uint32_t)(((2 * b) ^ (s16 & 14)) | hg) * 16u) ^ (uint32_t)wc);

    // Where the reads of one step come from: A pair buffer (byte offset) and
    // half (which step of the pair), B buffer (byte offset).
    struct ReadSrc { uint32_t a_buf; int a_half; uint32_t b_buf; };
    auto read_a = [&](const ReadSrc &R, int blk, int part, intx8 &f) {
        const uint32_t addr = a_lane_at(R.a_half, part) + R.a_buf + (uint32_t)(blk * 32 * 128);
        const intx4 v = *reinterpret_cast<const intx4 *>(lds + addr);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            f[4 * part + e] = v[e];
    };
    auto read_b = [&](const ReadSrc &R, int blk, int part, intx8 &f) {
        const uint32_t addr = b_lane[blk] + R.b_buf + (uint32_t)(part * 2048);
        const intx2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_intx2 *)(lds + addr));
        f[2 * part + 0] = v[0];
        f[2 * part + 1] = v[1];
    };
    // The 24 reads of one step in the order its MFMAs want them: A block 0
    // (2 reads), B blocks 0..3 (4 each), A blocks 1..3.
    constexpr int R_STEP = 24;
    auto fread = [&](const ReadSrc &R, int r, intx8 *fa, intx8 *fb) {
        if (r < 2) {
            read_a(R, 0, r, fa[0]);
        } else if (r < 18) {
            const int q = r - 2;
            read_b(R, q / 4, q % 4, fb[q / 4]);
        } else {
            const int q = r - 18;
            read_a(R, 1 + q / 2, q % 2, fa[1 + q / 2]);
        }
    };

    // ---- C tile: lane (r32, g) owns rows 32 i + 8 (e / 4) + 4 g + e % 4 and
    // column 32 j + r32 of the wave's 128 x 128 block.  An element outside C
    // gets an out-of-range lane offset: it is not written.
    const int ldc = args.ldc;
    const int c_col = n0 + wc + r32;
    const int c_rows_left = M - m0 - wr - 4 * g;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(
        args.C + (size_t)(m0 + wr) * ldc + n0 + wc, ((long long)(M - m0 - wr - 1) * ldc + N - n0 - wc) * 4);
    auto c_offset = [&](int col, int rows_left, int i, int j, int e, uint32_t &vo, uint32_t &so) {
        const int ro = 32 * i + 8 * (e >> 2) + (e & 3);
        vo = (ro < rows_left && col + 32 * j < N) ? (uint32_t)((4 * g) * ldc + r32 + 32 * j) * 4u : OOB;
        so = (uint32_t)(ro * ldc) * 4u;
    };

    floatx16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[i][j][e] = 0;

    // One step (parity par within its A pair): its 16 MFMAs (row-major over
    // the blocks) from (ca, cb); the 24 reads of the next step (source R)
    // into (na, nb), two after each of the first 12 MFMAs; the step's 8 loads
    // (B step s + 3, then half par of A pair s / 2 + 2), one after every
    // second MFMA.
    //
    // Buffers: A pair P is read during steps 2P - 1 and 2P and refilled with
    // pair P + 3 during steps 2P + 2, 2P + 3; B step s is read during step
    // s - 1 and its buffer refilled with step s + 4 during step s + 1.  Both
    // refills start after the barrier that ends the last reads.
    struct StepLoads { intx4 rb; uint32_t b_dst; PairLoads a; };
    auto step = [&](int par, const StepLoads &L, const ReadSrc &R, intx8 *ca, intx8 *cb, intx8 *na, intx8 *nb) {
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            acc[m >> 2][m & 3] = Op::mma(ca[m >> 2], cb[m & 3], acc[m >> 2][m & 3]);
            if (m < 12) {
                fread(R, 2 * m, na, nb);
                fread(R, 2 * m + 1, na, nb);
            }
            if (m % 2 == 1) {
                const int ld = m / 2;   // 0..7: B loads 0..3, then the A half
                if (ld < 4)
                    load_to_lds(L.rb, L.b_dst + (uint32_t)(ld * 1024), b_off[ld]);
                else
                    load_a(L.a, 4 * par + ld - 4);
            }
            // keep this order: the compiler would otherwise cluster the reads
            // and loads, and move MFMAs across the barrier
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // Before step s: this wavefront's loads issued before step s - 1 have
    // landed (B step s + 1, A pair (s + 1) / 2), its LDS reads have returned,
    // and the workgroup meets at the barrier.  Step 0 needs B step 1 with 12
    // younger prologue loads in flight; later steps let the previous step's 8
    // loads fly.
    auto step_begin = [&](int s, uint32_t a_load_buf) {
        if (s == 0)
            __builtin_amdgcn_s_waitcnt(wait_vmcnt_lgkm0(12));
        else
            __builtin_amdgcn_s_waitcnt(wait_vmcnt_lgkm0(LOADS_PER_STEP));
        __builtin_amdgcn_s_barrier();
        StepLoads L;
        L.rb = b_rsrc(s + 3);
        L.b_dst = lds_b + (uint32_t)(((s + 3) & 3) * B_BYTES);
        L.a = a_rsrc((s >> 1) + 2, a_load_buf);
        __builtin_amdgcn_sched_barrier(0);
        return L;
    };
    auto b_buf = [](int st) { return (uint32_t)((st & 3) * B_BYTES); };
    auto next_pair = [](uint32_t pb) { return pb == (uint32_t)((A_PAIRS - 1) * A_PAIR_BYTES) ? 0u : pb + A_PAIR_BYTES; };

    // prologue: A pair 0, B steps 0 and 1, A pair 1, B step 2; then the reads
    // of step 0 (A pair 0 and B step 0 landed: 16 younger loads may fly)
    intx8 fa0[4], fa1[4], fb0[4], fb1[4];
    {
        const PairLoads L = a_rsrc(0, 0);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            load_a(L, j);
    }
#pragma unroll
    for (int st = 0; st < 2; ++st) {
        const intx4 rb = b_rsrc(st);
#pragma unroll
        for (int q = 0; q < 4; ++q)
            load_to_lds(rb, lds_b + b_buf(st) + (uint32_t)(q * 1024), b_off[q]);
    }
    {
        const PairLoads L = a_rsrc(1, A_PAIR_BYTES);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            load_a(L, j);
    }
    {
        const intx4 rb = b_rsrc(2);
#pragma unroll
        for (int q = 0; q < 4; ++q)
            load_to_lds(rb, lds_b + b_buf(2) + (uint32_t)(q * 1024), b_off[q]);
    }
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(16));
    __builtin_amdgcn_s_barrier();
    {
        const ReadSrc R0{0u, 0, b_buf(0)};
#pragma unroll
        for (int r = 0; r < R_STEP; ++r)
            fread(R0, r, fa0, fb0);
    }

    // Two steps (one A pair, P = s / 2) per trip, so each step's parity is
    // known here; pa, pa1, pa2 are the buffers of pairs P, P + 1, P + 2.
    const int steps = (K + BK - 1) / BK;
    uint32_t pa = 0;
    for (int s = 0; s < steps; s += 2) {
        const uint32_t pa1 = next_pair(pa), pa2 = next_pair(pa1);
        StepLoads L = step_begin(s, pa2);
        step(0, L, ReadSrc{pa, 1, b_buf(s + 1)}, fa0, fb0, fa1, fb1);
        if (s + 1 < steps) {
            L = step_begin(s + 1, pa2);
            step(1, L, ReadSrc{pa1, 0, b_buf(s + 2)}, fa1, fb1, fa0, fb0);
        }
        pa = pa1;
    }
    // no load may still be writing this workgroup's LDS when it ends
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));

    int col_e = c_col, rows_e = c_rows_left;
    asm volatile("" : "+v"(col_e), "+v"(rows_e));
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                uint32_t vo, so;
                c_offset(col_e, rows_e, i, j, e, vo, so);
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][j][e]), rc, vo, so, 0);
            }
}

// ---------------------------------------------------------------------------
// The INT8 product (A M x K, B K x N, row-major) on 16 x 16 blocks: the
// structure of the 16-bit pair ring with one-byte elements.
//   Fragments.  Lane (g, s) = (l / 16, l % 16) holds the k-values
//   16 g .. 16 g + 15 of the step of row s of its A block (one 128-bit read
//   of logical unit 4 half + g of the row) and of column s of its B block
//   (two transposing reads, k rows 16 g .. + 7 and 16 g + 8 .. + 15).  The
//   matrix unit pairs equal register bytes of A and B lanes, so each k is
//   summed exactly once.  Output: lane (g, s) holds rows 4 g + r, column s of
//   the block (r = 0..3).
//   B swizzle.  The two transposing reads of lanes 0..31 (served in one
//   cycle) take k rows 16 apart at the same columns; x(k) carries bit 4 of k
//   into unit bit 0 so that the two groups' 8-byte halves land on distinct
//   banks.
//   Epilogue.  C leaves through LDS once the ring is done, in four rounds
//   of 32 rows a wavefront (the 16-bit rings' store with 32-bit elements
//   copied as bits), so it is written once, in whole 128-byte lines.
__device__ __forceinline__ int acc_read_i32(int a)
{
    int v;
    asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
    return v;
}

// A wavefront's 128 x 128 block of INT32 C from its accumulators in the
// 16 x 16 layout: four rounds of 32 rows through its own LDS region (rows of
// 512 bytes padded by 16, so the 64 lanes of every 4-byte write fall on
// distinct banks), read back 16 bytes a lane along the rows and stored so.
// Cw: the block's first element; rows_left / cols_left: its rows and columns
// inside C; vec: Cw 16-byte aligned and ldc a multiple of 4.
__device__ __forceinline__ void store_c_staged_i32(const intx4 (&acc)[8][8], uint8_t *lds, int wave, int lane,
                                                   int *Cw, int ldc, int rows_left, int cols_left, bool vec)
{
    constexpr int ROW_BYTES = 128 * 4 + 16, WAVE_BYTES = 32 * ROW_BYTES;
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
                    *reinterpret_cast<int *>(w + (16 * ii + 4 * g + r) * ROW_BYTES + (16 * j + s16) * 4) =
                        acc_read_i32(acc[2 * q + ii][j][r]);
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const int u = lane + 64 * t, row = u >> 5, col = 4 * (u & 31);
            const intx4 v = *reinterpret_cast<const intx4 *>(w + row * ROW_BYTES + col * 4);
            const int grow = 32 * q + row;
            if (grow < rows_left) {
                const uint32_t o = (uint32_t)(grow * ldc + col) * 4u;
                if (vec && col + 4 <= cols_left) {
                    __builtin_amdgcn_raw_buffer_store_b128(v, rc, o, 0, 0);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        __builtin_amdgcn_raw_buffer_store_b32(v[e], rc, col + e < cols_left ? o + 4u * e : OOB, 0, 0);
                }
            }
        }
    }
}

__global__ __launch_bounds__(256) void mfma_i8_pair_kernel(RingArgs args)
{
    using namespace ring8;
    static_assert(4 * 32 * (128 * 4 + 16) <= LDS_BYTES, "the epilogue stages through the ring's LDS");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[LDS_BYTES];
    const uint32_t ring = lds_address(lds);
    const int M = args.M, N = args.N, K = args.K, lda = args.lda, ldb = args.ldb;
    const uint8_t *__restrict__ A = (const uint8_t *)args.A;
    const uint8_t *__restrict__ B = (const uint8_t *)args.B;

    int tm, tn;
    dgor_tile_of_block(blockIdx.x, args.tiles_m, args.tiles_n, args.group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int wr = (wave >> 1) * 128, wc = (wave & 1) * 128;
    constexpr uint32_t OOB = 0x80000000u;

    // ---- loader (the layouts above; B with x(k) = 2 (k & 7) | ((k >> 4) & 1))
    uint32_t a_off[2], b_off[4];
    int a_kc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int r = 64 * wave + 8 * j + (lane >> 3);
        const int c = (lane & 7) ^ ((4 * j + (lane >> 4)) & 7);
        a_off[j] = (uint32_t)(r * lda + 16 * c);
        a_kc[j] = 16 * c;
    }
    const uint32_t a_row16 = (uint32_t)(16 * lda);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int k = 4 * (4 * wave + q) + (lane >> 4);
        const int u = (lane & 15) ^ ((2 * (k & 7)) | ((k >> 4) & 1));
        b_off[q] = n0 + 16 * u < N ? (uint32_t)(k * ldb + 16 * u) : OOB;
    }
    const uint32_t lds_a = ring + (uint32_t)(8 * wave * 1024);
    const uint32_t lds_b = ring + (uint32_t)(B_REGION + 4 * wave * 1024);
    struct PairLoads { intx4 r; int k_left; uint32_t dst; };
    auto a_rsrc = [&](int P, uint32_t buf) {
        PairLoads L;
        const int k0 = 2 * BK * P;
        L.k_left = K - k0;
        L.r = rsrc_words(A + (size_t)m0 * lda + k0, 0);
        L.r.z = L.k_left <= 0 ? 0
              : (m0 + BM <= M ? 0x7fffffff
                              : (int)((uint32_t)(M - m0 - 1) * (uint32_t)lda + (uint32_t)L.k_left));
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
        const int k0 = BK * st, k_left = K - k0;
        L.r = rsrc_words(B + (size_t)k0 * ldb + n0, 0);
        L.r.z = k_left <= 0 ? 0
              : (k_left >= BK ? 0x7fffffff : (int)((uint32_t)(k_left - 1) * (uint32_t)ldb + (uint32_t)(N - n0)));
        L.dst = lds_b + (uint32_t)((st & 3) * B_BYTES);
        return L;
    };
    auto load_b = [&](const BLoads &L, int q) { load_to_lds(L.r, L.dst + (uint32_t)(q * 1024), b_off[q]); };

    // ---- fragment reads.  A block i of half h: row wr + 16 i + s16,
    // physical unit (4 h + g) ^ ((s16 >> 1) & 7); h applied by XOR on bit 6
    // of the byte offset.  B block j, read h: k row 16 g + 8 h + s16 / 2, byte
    // 8 (s16 % 2) of logical unit wc / 16 + j at physical unit
    // unit ^ (s16 & 14 | g & 1).
    const int s16 = lane & 15, g = lane >> 4;
    const uint32_t a_lane = (uint32_t)((wr + s16) * 128) | (uint32_t)((g ^ ((s16 >> 1) & 7)) * 16);
    const int b_x = (s16 & 14) | (g & 1);
    const uint32_t b_lane = (uint32_t)(B_REGION + (16 * g + (s16 >> 1)) * 256 + 8 * (s16 & 1));
    uint32_t b_unit[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        b_unit[j] = (uint32_t)(((wc / 16 + j) ^ b_x) * 16);
    struct ReadSrc { uint32_t a_buf; int a_half; uint32_t b_buf; };
    auto read_a = [&](const ReadSrc &R, int i) -> intx4 {
        const uint32_t addr = (a_lane ^ (uint32_t)(64 * R.a_half)) + R.a_buf + (uint32_t)(i * 2048);
        return *reinterpret_cast<const intx4 *>(lds + addr);
    };
    auto read_b = [&](const ReadSrc &R, int j) -> intx4 {
        const uint8_t *p = lds + b_lane + R.b_buf + b_unit[j];
        const intx2 lo = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_intx2 *)p);
        const intx2 hi = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_intx2 *)(p + 2048));
        return intx4{lo[0], lo[1], hi[0], hi[1]};
    };
    // read r (0..15): A block 0, the eight B blocks, then A blocks 1..7
    auto fread = [&](const ReadSrc &R, int r, intx4 *fa, intx4 *fb) {
        if (r == 0 || r >= 9)
            fa[r == 0 ? 0 : r - 8] = read_a(R, r == 0 ? 0 : r - 8);
        else
            fb[r - 1] = read_b(R, r - 1);
    };

    intx4 acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)   // AGPR writes, so the compiler keeps the array in AGPRs
                asm("v_accvgpr_write_b32 %0, 0" : "=a"(acc[i][j][r]));

    // One step (parity par within its A pair): the 64 MFMAs from (ca, cb);
    // the 16 reads of the next step (source R) into (na, nb), one after each
    // of the first 16 MFMAs; the step's 8 loads (B step s + 3, then half par
    // of A pair s / 2 + 2), one after every sixth of the rest.
    struct StepLoads { BLoads b; PairLoads a; };
    auto step = [&](int par, const StepLoads &L, const ReadSrc &R, intx4 *ca, intx4 *cb, intx4 *na, intx4 *nb) {
#pragma unroll
        for (int m = 0; m < 64; ++m) {
            const int i = m >> 3, j = m & 7;
            acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ca[i], cb[j], acc[i][j], 0, 0, 0);
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
    // Before step s: as in the FP8 kernel (12 younger loads at step 0, 8 later).
    auto step_begin = [&](int s, uint32_t a_load_buf) {
        if (s == 0)
            __builtin_amdgcn_s_waitcnt(wait_vmcnt_lgkm0(12));
        else
            __builtin_amdgcn_s_waitcnt(wait_vmcnt_lgkm0(LOADS_PER_STEP));
        __builtin_amdgcn_s_barrier();
        const StepLoads L{b_rsrc(s + 3), a_rsrc((s >> 1) + 2, a_load_buf)};
        __builtin_amdgcn_sched_barrier(0);
        return L;
    };
    auto b_buf = [](int st) { return (uint32_t)((st & 3) * B_BYTES); };
    auto next_pair = [](uint32_t pb) { return pb == (uint32_t)((A_PAIRS - 1) * A_PAIR_BYTES) ? 0u : pb + A_PAIR_BYTES; };

    // prologue: A pair 0, B steps 0 and 1, A pair 1, B step 2; then the reads
    // of step 0 (A pair 0 and B step 0 landed: 16 younger loads may fly)
    intx4 fa0[8], fa1[8], fb0[8], fb1[8];
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

    const int steps = (K + BK - 1) / BK;
    uint32_t pa = 0;
    for (int s = 0; s < steps; s += 2) {
        const uint32_t pa1 = next_pair(pa), pa2 = next_pair(pa1);
        StepLoads L = step_begin(s, pa2);
        step(0, L, ReadSrc{pa, 1, b_buf(s + 1)}, fa0, fb0, fa1, fb1);
        if (s + 1 < steps) {
            L = step_begin(s + 1, pa2);
            step(1, L, ReadSrc{pa1, 0, b_buf(s + 2)}, fa1, fb1, fa0, fb0);
        }
        pa = pa1;
    }
    // no load may still be writing this workgroup's LDS when it ends, and no
    // wavefront may still read the ring when the epilogue reuses it
    __builtin_amdgcn_s_waitcnt(wait_vmcnt_lgkm0(0));
    __builtin_amdgcn_s_barrier();
    dgor_acc_hazard_wait();
    {
        const int ldc = args.ldc;
        int *Cw = reinterpret_cast<int *>(args.C) + (size_t)(m0 + wr) * ldc + n0 + wc;
        const bool vec = ((uintptr_t)Cw & 15) == 0 && (ldc & 3) == 0;
        store_c_staged_i32(acc, lds, wave, lane, Cw, ldc, M - m0 - wr, N - n0 - wc, vec);
    }
}

// Epilogue of the INT8 128 x 128 ring: a wavefront's 64 x 64 block leaves
// through its own 8 KB LDS region in two rounds of 32 rows; element (row,
// col) of a round sits at row 256 + 16 ((col / 4) ^ 4 ((row / 4) % 4)) +
// 4 (col % 4), so both the 4-byte writes (lane (g, s) of block j at unit
// 4 (j ^ g) + s / 4) and the 16-byte reads along the rows are free of bank
// conflicts.  Arguments as in store_c_staged_i32, except that acc holds the
// sums already read out of the accumulator registers.
__device__ __forceinline__ void store_c_staged_w64_i32(const intx4 (&acc)[4][4], uint8_t *lds, int wave, int lane,
                                                       int *Cw, int ldc, int rows_left, int cols_left, bool vec)
{
    constexpr uint32_t OOB = 0x80000000u;
    uint8_t *w = lds + wave * 8192;
    const int g = lane >> 4, s16 = lane & 15;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(
        Cw, rows_left > 0 && cols_left > 0 ? ((long long)(rows_left - 1) * ldc + cols_left) * 4 : 0);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
#pragma unroll
        for (int ii = 0; ii < 2; ++ii)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    *reinterpret_cast<int *>(w + (16 * ii + 4 * g + r) * 256 + (4 * (j ^ g) + (s16 >> 2)) * 16 +
                                             (s16 & 3) * 4) = acc[2 * q + ii][j][r];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int row = (lane >> 4) + 4 * t, c = lane & 15;
            const intx4 v = *reinterpret_cast<const intx4 *>(w + row * 256 + ((c ^ (4 * (t & 3))) * 16));
            const int grow = 32 * q + row, col = 4 * c;
            if (grow < rows_left) {
                const uint32_t o = (uint32_t)(grow * ldc + col) * 4u;
                if (vec && col + 4 <= cols_left) {
                    __builtin_amdgcn_raw_buffer_store_b128(v, rc, o, 0, 0);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        __builtin_amdgcn_raw_buffer_store_b32(v[e], rc, col + e < cols_left ? o + 4u * e : OOB, 0, 0);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// 8-bit inputs at mid sizes: the pair rings at half the tile.  INT8 first.  A 128 x 128 tile has
// four wavefronts of 64 x 64 (4 x 4 blocks of v_mfma_i32_16x16x64_i8, 64
// accumulators a lane) and 80 KB of LDS, so two workgroups share a compute
// unit and cover each other's waits, and a 2048^3 product has a tile for
// every compute unit where the 256 x 256 tiles leave three quarters idle.
//   A pair buffer (16 KB): 128 rows of 128 bytes, unit c of row r at
//     8 r + (c ^ ((r >> 1) & 7)); wave w's load j (0..3) fills rows
//     32 w + 8 j .. + 7, two loads a step (half par of the pair).
//   B step (8 KB): 64 k rows of 128 bytes, unit u of row k at
//     8 k + (u ^ x(k)), x(k) = ((k >> 1) & 3) + 4 ((k >> 4) & 1); wave w's
//     load q (0..1) fills k rows 8 (2 w + q) .. + 7, lane p taking physical
//     unit p % 8 of row 8 (2 w + q) + p / 8.  A transposing-read cycle (32
//     lanes) takes one 16-byte unit of each of k rows kb .. kb + 7 and of
//     kb + 16 .. kb + 23: the swizzle gives the sixteen rows sixteen distinct
//     units modulo the 256 bytes of banks.
//   Fragments as in the 256 x 256 kernel (A block i: row wr + 16 i + s16,
//   logical unit 4 h + g; B block j: k rows 16 g .. 16 g + 15 of column
//   wc + 16 j + s16, two transposing reads 8 k rows apart).
//   Pipeline, waits and the fragment order as in the pair ring, with 16
//   MFMAs, 8 fragment reads and 4 loads a wavefront and step.
//   KS = 2 (at most one tile per compute unit): eight wavefronts in two
//   groups of four, each over half of the k-steps (A, B and K shifted to the
//   group's range) through its own 80 KB ring; both groups run the same
//   number of steps and meet at the same barriers, and group 1 hands its sums
//   to group 0 through its ring at the end (the FP8 kernel below does the
//   same).
namespace ring8_128 {
constexpr int BK = 64;
constexpr int A_PAIR_BYTES = 128 * 2 * BK;           // 16 KB
constexpr int A_PAIRS = 3;
constexpr int B_BYTES = BK * 128;                    // 8 KB
constexpr int B_REGION = A_PAIRS * A_PAIR_BYTES;     // 48 KB
constexpr int LDS_BYTES = B_REGION + 4 * B_BYTES;    // 80 KB
}  // namespace ring8_128

template <int KS>
__global__ __launch_bounds__(256 * KS, 2 / KS) void mfma_i8_pair128_kernel(RingArgs args)
{
    using namespace ring8_128;
    static_assert(4 * 8192 <= LDS_BYTES, "the epilogue stages through the ring's LDS");
    __shared__ __attribute__((aligned(1024))) uint8_t lds_all[KS * LDS_BYTES];
    const int wave_all = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int grp = wave_all >> 2;
    uint8_t *const lds = lds_all + grp * LDS_BYTES;
    const uint32_t ring = lds_address(lds);
    const int M = args.M, N = args.N, lda = args.lda, ldb = args.ldb;
    // the group's k range: A, B and K shifted to it
    const int steps = ((args.K + BK - 1) / BK + KS - 1) / KS;
    const int kbase = grp * steps * BK;
    const int K = args.K < kbase + steps * BK ? args.K - kbase : steps * BK;
    const uint8_t *__restrict__ A = (const uint8_t *)args.A + kbase;
    const uint8_t *__restrict__ B = (const uint8_t *)args.B + (size_t)kbase * ldb;

    int tm, tn;
    dgor_tile_of_block((int)blockIdx.x, args.tiles_m, args.tiles_n, args.group_m, tm, tn);
    const int m0 = tm * 128, n0 = tn * 128;
    const int lane = threadIdx.x & 63;
    const int wave = wave_all & 3;
    const int wr = (wave >> 1) * 64, wc = (wave & 1) * 64;
    constexpr uint32_t OOB = 0x80000000u;

    uint32_t a_off[2], b_off[2];
    int a_kc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int r = 32 * wave + 8 * j + (lane >> 3);
        const int c = (lane & 7) ^ ((4 * j + (lane >> 4)) & 7);
        a_off[j] = (uint32_t)(r * lda + 16 * c);
        a_kc[j] = 16 * c;
    }
    const uint32_t a_row16 = (uint32_t)(16 * lda);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int k = 8 * (2 * wave + q) + (lane >> 3);
        const int u = (lane & 7) ^ (((k >> 1) & 3) + 4 * ((k >> 4) & 1));
        b_off[q] = n0 + 16 * u < N ? (uint32_t)(k * ldb + 16 * u) : OOB;
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
                               : (int)((uint32_t)(M - m0 - 1) * (uint32_t)lda + (uint32_t)L.k_left));
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
        const int k0 = BK * st, k_left = K - k0;
        L.r = rsrc_words(B + (size_t)k0 * ldb + n0, 0);
        L.r.z = k_left <= 0 ? 0
              : (k_left >= BK ? 0x7fffffff : (int)((uint32_t)(k_left - 1) * (uint32_t)ldb + (uint32_t)(N - n0)));
        L.dst = lds_b + (uint32_t)((st & 3) * B_BYTES);
        return L;
    };
    auto load_b = [&](const BLoads &L, int q) { load_to_lds(L.r, L.dst + (uint32_t)(q * 1024), b_off[q]); };

    const int s16 = lane & 15, g = lane >> 4;
    const uint32_t a_lane = (uint32_t)((wr + s16) * 128) | (uint32_t)((g ^ ((s16 >> 1) & 7)) * 16);
    const int ks_x = ((s16 >> 2) & 3) + 4 * (g & 1);
    const uint32_t b_lane = (uint32_t)(B_REGION + (16 * g + (s16 >> 1)) * 128 + 8 * (s16 & 1));
    uint32_t b_unit[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        b_unit[j] = (uint32_t)(((wc / 16 + j) ^ ks_x) * 16);
    struct ReadSrc { uint32_t a_buf; int a_half; uint32_t b_buf; };
    auto read_a = [&](const ReadSrc &R, int i) -> intx4 {
        const uint32_t addr = (a_lane ^ (uint32_t)(64 * R.a_half)) + R.a_buf + (uint32_t)(i * 2048);
        return *reinterpret_cast<const intx4 *>(lds + addr);
    };
    auto read_b = [&](const ReadSrc &R, int j) -> intx4 {
        const uint8_t *p = lds + b_lane + R.b_buf + b_unit[j];
        const intx2 lo = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_intx2 *)p);
        const intx2 hi = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_intx2 *)(p + 1024));
        return intx4{lo[0], lo[1], hi[0], hi[1]};
    };
    auto fread = [&](const ReadSrc &R, int r, intx4 *fa, intx4 *fb) {
        if (r == 0 || r >= 5)
            fa[r == 0 ? 0 : r - 4] = read_a(R, r == 0 ? 0 : r - 4);
        else
            fb[r - 1] = read_b(R, r - 1);
    };

    intx4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                asm("v_accvgpr_write_b32 %0, 0" : "=a"(acc[i][j][r]));

    struct StepLoads { BLoads b; PairLoads a; };
    auto step = [&](int par, const StepLoads &L, const ReadSrc &R, intx4 *ca, intx4 *cb, intx4 *na, intx4 *nb) {
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            const int i = m >> 2, j = m & 3;
            acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ca[i], cb[j], acc[i][j], 0, 0, 0);
            if (m < 8)
                fread(R, m, na, nb);
            if (m >= 8 && (m & 1)) {
                const int ld = (m - 8) >> 1;
                if (ld < 2)
                    load_b(L.b, ld);
                else
                    load_a(L.a, 2 * par + ld - 2);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto step_begin = [&](int s, uint32_t a_load_buf) {
        if (s == 0)
            __builtin_amdgcn_s_waitcnt(wait_vmcnt_lgkm0(6));
        else
            __builtin_amdgcn_s_waitcnt(wait_vmcnt_lgkm0(4));
        __builtin_amdgcn_s_barrier();
        const StepLoads L{b_rsrc(s + 3), a_rsrc((s >> 1) + 2, a_load_buf)};
        __builtin_amdgcn_sched_barrier(0);
        return L;
    };
    auto b_buf = [](int st) { return (uint32_t)((st & 3) * B_BYTES); };
    auto next_pair = [](uint32_t pb) { return pb == (uint32_t)((A_PAIRS - 1) * A_PAIR_BYTES) ? 0u : pb + A_PAIR_BYTES; };

    intx4 fa0[4], fa1[4], fb0[4], fb1[4];
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
    for (int s = 0; s < steps; s += 2) {
        const uint32_t pa1 = next_pair(pa), pa2 = next_pair(pa1);
        StepLoads L = step_begin(s, pa2);
        step(0, L, ReadSrc{pa, 1, b_buf(s + 1)}, fa0, fb0, fa1, fb1);
        if (s + 1 < steps) {
            L = step_begin(s + 1, pa2);
            step(1, L, ReadSrc{pa1, 0, b_buf(s + 2)}, fa1, fb1, fa0, fb0);
        }
        pa = pa1;
    }
    __builtin_amdgcn_s_waitcnt(wait_vmcnt_lgkm0(0));
    __builtin_amdgcn_s_barrier();
    dgor_acc_hazard_wait();
    intx4 tot[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                tot[i][j][r] = acc_read_i32(acc[i][j][r]);
    if constexpr (KS == 2) {
        // group 1's sums to group 0 through group 1's ring
        intx4 *part = reinterpret_cast<intx4 *>(lds_all + LDS_BYTES);
        if (grp == 1) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    part[((i * 4 + j) * 4 + wave) * 64 + lane] = tot[i][j];
        }
        __builtin_amdgcn_s_barrier();
        if (grp == 1)
            return;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                tot[i][j] += part[((i * 4 + j) * 4 + wave) * 64 + lane];
    }
    {
        const int ldc = args.ldc;
        int *Cw = reinterpret_cast<int *>(args.C) + (size_t)(m0 + wr) * ldc + n0 + wc;
        const bool vec = ((uintptr_t)Cw & 15) == 0 && (ldc & 3) == 0;
        store_c_staged_w64_i32(tot, lds, wave, lane, Cw, ldc, M - m0 - wr, N - n0 - wc, vec);
    }
}

// Epilogue of the FP8 128 x 128 ring: a wavefront's 64 x 64 block in the
// 32 x 32 layout leaves through its own 8 KB LDS region in two rounds (one
// per row of blocks) of 32 rows; element (row, col) of a round sits at
// row 256 + 16 ((col / 4) ^ 8 ((row / 4) % 2)) + 4 (col % 4), so the 4-byte
// writes (lanes 0..31 and 32..63 take rows 4 apart, on the two halves of the
// banks) and the 16-byte reads along the rows are free of bank conflicts.
// acc: the sums, read out of the accumulator registers; Cw: the block's first
// element; rows_left / cols_left: its rows and columns inside C; vec: Cw
// 16-byte aligned and ldc a multiple of 4.
__device__ __forceinline__ void store_c_staged_w64_32(const floatx16 (&acc)[2][2], uint8_t *lds, int wave, int lane,
                                                      float *Cw, int ldc, int rows_left, int cols_left, bool vec)
{
    typedef unsigned uintx4 __attribute__((ext_vector_type(4)));
    constexpr uint32_t OOB = 0x80000000u;
    uint8_t *w = lds + wave * 8192;
    const int r32 = lane & 31, g = lane >> 5;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(
        Cw, rows_left > 0 && cols_left > 0 ? ((long long)(rows_left - 1) * ldc + cols_left) * 4 : 0);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = 8 * (e >> 2) + 4 * g + (e & 3), col = 32 * j + r32;
                *reinterpret_cast<float *>(w + row * 256 + 16 * ((col >> 2) ^ (8 * g)) + 4 * (col & 3)) =
                    acc[i][j][e];
            }
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int row = (lane >> 4) + 4 * t, c = lane & 15;
            const uintx4 v = *reinterpret_cast<const uintx4 *>(w + row * 256 + ((c ^ (8 * (t & 1))) * 16));
            const int grow = 32 * i + row, col = 4 * c;
            if (grow < rows_left) {
                const uint32_t o = (uint32_t)(grow * ldc + col) * 4u;
                if (vec && col + 4 <= cols_left) {
                    __builtin_amdgcn_raw_buffer_store_b128(v, rc, o, 0, 0);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        __builtin_amdgcn_raw_buffer_store_b32(v[e], rc, col + e < cols_left ? o + 4u * e : OOB, 0, 0);
                }
            }
        }
    }
}

// The FP8 128 x 128 ring: the INT8 one's tile, LDS plan, pipeline and waits
// with the FP8 kernel's 32 x 32 blocks (2 x 2 a wavefront, one
// v_mfma_scale_f32_32x32x64_f8f6f4 per block and step).  Its transposing
// reads take 8 k rows of one 32-column block per cycle (32 lanes: two
// 16-column halves of 8 bytes each), so B rows use the swizzle
// x(k) = 2 ((k >> 1) & 3): the four even and the four odd rows of a read
// get four distinct pairs of units, which with the row parity (128 bytes
// apart) puts the 32 lanes' 8-byte pieces on 32 distinct bank pairs.  Each
// of the 4 MFMAs of a step is followed by three of the next step's 12
// fragment reads and one of its 4 loads.
template <class Op, int KS>
__global__ __launch_bounds__(256 * KS, 2 / KS) void mfma_fp8_pair128_kernel(RingArgs args)
{
    using namespace ring8_128;
    static_assert(4 * 8192 <= LDS_BYTES, "the epilogue stages through the ring's LDS");
    __shared__ __attribute__((aligned(1024))) uint8_t lds_all[KS * LDS_BYTES];
    const int wave_all = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int grp = wave_all >> 2;
    uint8_t *const lds = lds_all + grp * LDS_BYTES;
    const uint32_t ring = lds_address(lds);
    const int M = args.M, N = args.N, lda = args.lda, ldb = args.ldb;
    // the group's k range: A, B and K shifted to it
    const int steps = ((args.K + BK - 1) / BK + KS - 1) / KS;
    const int kbase = grp * steps * BK;
    const int K = args.K < kbase + steps * BK ? args.K - kbase : steps * BK;
    const uint8_t *__restrict__ A = (const uint8_t *)args.A + kbase;
    const uint8_t *__restrict__ B = (const uint8_t *)args.B + (size_t)kbase * ldb;

    int tm, tn;
    dgor_tile_of_block((int)blockIdx.x, args.tiles_m, args.tiles_n, args.group_m, tm, tn);
    const int m0 = tm * 128, n0 = tn * 128;
    const int lane = threadIdx.x & 63;
    const int wave = wave_all & 3;
    const int wr = (wave >> 1) * 64, wc = (wave & 1) * 64;
    constexpr uint32_t OOB = 0x80000000u;

    // ---- loader: as in the INT8 128 x 128 ring, B with x(k) = 2 ((k >> 1) & 3)
    uint32_t a_off[2], b_off[2];
    int a_kc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int r = 32 * wave + 8 * j + (lane >> 3);
        const int c = (lane & 7) ^ ((4 * j + (lane >> 4)) & 7);
        a_off[j] = (uint32_t)(r * lda + 16 * c);
        a_kc[j] = 16 * c;
    }
    const uint32_t a_row16 = (uint32_t)(16 * lda);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int k = 8 * (2 * wave + q) + (lane >> 3);
        const int u = (lane & 7) ^ (2 * ((k >> 1) & 3));
        b_off[q] = n0 + 16 * u < N ? (uint32_t)(k * ldb + 16 * u) : OOB;
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
                               : (int)((uint32_t)(M - m0 - 1) * (uint32_t)lda + (uint32_t)L.k_left));
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
        const int k0 = BK * st, k_left = K - k0;
        L.r = rsrc_words(B + (size_t)k0 * ldb + n0, 0);
        L.r.z = k_left <= 0 ? 0
              : (k_left >= BK ? 0x7fffffff : (int)((uint32_t)(k_left - 1) * (uint32_t)ldb + (uint32_t)(N - n0)));
        L.dst = lds_b + (uint32_t)((st & 3) * B_BYTES);
        return L;
    };
    auto load_b = [&](const BLoads &L, int q) { load_to_lds(L.r, L.dst + (uint32_t)(q * 1024), b_off[q]); };

    // ---- fragment reads (the 32 x 32 layout of the 256 x 256 FP8 kernel).
    // A block i: row wr + 32 i + r32, logical units 4 h + 2 g + u (u = 0, 1),
    // physical unit ^ ((row >> 1) & 7).  B block j, read q: k row
    // 32 g + 8 q + s16 / 2, byte 8 (s16 % 2) of logical unit
    // wc / 16 + 2 j + hg, physical unit ^ 2 ((s16 >> 2) & 3).
    const int r32 = lane & 31, g = lane >> 5;
    const int s16 = lane & 15, hg = (lane >> 4) & 1;
    const uint32_t a_lane = (uint32_t)((wr + r32) * 128) | (uint32_t)(((2 * g) ^ ((r32 >> 1) & 7)) * 16);
    uint32_t b_lane[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
        b_lane[j] = (uint32_t)(B_REGION + (32 * g + (s16 >> 1)) * 128 + 8 * (s16 & 1) +
                               16 * (((wc / 16 + 2 * j) | hg) ^ (2 * ((s16 >> 2) & 3))));
    struct ReadSrc { uint32_t a_buf; int a_half; uint32_t b_buf; };
    auto read_a = [&](const ReadSrc &R, int blk, int part, intx8 &f) {
        const uint32_t addr = (a_lane ^ (uint32_t)((4 * R.a_half + part) * 16)) + R.a_buf + (uint32_t)(blk * 32 * 128);
        const intx4 v = *reinterpret_cast<const intx4 *>(lds + addr);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            f[4 * part + e] = v[e];
    };
    auto read_b = [&](const ReadSrc &R, int blk, int part, intx8 &f) {
        const uint32_t addr = b_lane[blk] + R.b_buf + (uint32_t)(part * 1024);
        const intx2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_intx2 *)(lds + addr));
        f[2 * part + 0] = v[0];
        f[2 * part + 1] = v[1];
    };
    // read r (0..11): A block 0 (2 reads), B blocks 0 and 1 (4 each), A block 1
    auto fread = [&](const ReadSrc &R, int r, intx8 *fa, intx8 *fb) {
        if (r < 2)
            read_a(R, 0, r, fa[0]);
        else if (r < 10)
            read_b(R, (r - 2) >> 2, (r - 2) & 3, fb[(r - 2) >> 2]);
        else
            read_a(R, 1, r - 10, fa[1]);
    };

    floatx16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                asm("v_accvgpr_write_b32 %0, 0" : "=a"(acc[i][j][e]));

    // One step: its 4 MFMAs, each followed by three of the next step's reads
    // and one of the step's loads (B step s + 3, then half par of A pair
    // s / 2 + 2).
    struct StepLoads { BLoads b; PairLoads a; };
    auto step = [&](int par, const StepLoads &L, const ReadSrc &R, intx8 *ca, intx8 *cb, intx8 *na, intx8 *nb) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int i = m >> 1, j = m & 1;
            acc[i][j] = Op::mma(ca[i], cb[j], acc[i][j]);
#pragma unroll
            for (int r = 0; r < 3; ++r)
                fread(R, 3 * m + r, na, nb);
            if (m < 2)
                load_b(L.b, m);
            else
                load_a(L.a, 2 * par + m - 2);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto step_begin = [&](int s, uint32_t a_load_buf) {
        if (s == 0)
            __builtin_amdgcn_s_waitcnt(wait_vmcnt_lgkm0(6));
        else
            __builtin_amdgcn_s_waitcnt(wait_vmcnt_lgkm0(4));
        __builtin_amdgcn_s_barrier();
        const StepLoads L{b_rsrc(s + 3), a_rsrc((s >> 1) + 2, a_load_buf)};
        __builtin_amdgcn_sched_barrier(0);
        return L;
    };
    auto b_buf = [](int st) { return (uint32_t)((st & 3) * B_BYTES); };
    auto next_pair = [](uint32_t pb) { return pb == (uint32_t)((A_PAIRS - 1) * A_PAIR_BYTES) ? 0u : pb + A_PAIR_BYTES; };

    intx8 fa0[2], fa1[2], fb0[2], fb1[2];
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
        for (int r = 0; r < 12; ++r)
            fread(R0, r, fa0, fb0);
    }

    uint32_t pa = 0;
    for (int s = 0; s < steps; s += 2) {
        const uint32_t pa1 = next_pair(pa), pa2 = next_pair(pa1);
        StepLoads L = step_begin(s, pa2);
        step(0, L, ReadSrc{pa, 1, b_buf(s + 1)}, fa0, fb0, fa1, fb1);
        if (s + 1 < steps) {
            L = step_begin(s + 1, pa2);
            step(1, L, ReadSrc{pa1, 0, b_buf(s + 2)}, fa1, fb1, fa0, fb0);
        }
        pa = pa1;
    }
    __builtin_amdgcn_s_waitcnt(wait_vmcnt_lgkm0(0));
    __builtin_amdgcn_s_barrier();
    dgor_acc_hazard_wait();
    floatx16 tot[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                tot[i][j][e] = dgor_acc_read(acc[i][j][e]);
    if constexpr (KS == 2) {
        // group 1's sums to group 0 through group 1's ring, 16 bytes a lane
        // per piece; group 0 adds them in that order
        floatx4 *part = reinterpret_cast<floatx4 *>(lds_all + LDS_BYTES);
        if (grp == 1) {
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    part[((b * 4 + c) * 4 + wave) * 64 + lane] =
                        floatx4{tot[b >> 1][b & 1][4 * c], tot[b >> 1][b & 1][4 * c + 1],
                                tot[b >> 1][b & 1][4 * c + 2], tot[b >> 1][b & 1][4 * c + 3]};
        }
        __builtin_amdgcn_s_barrier();
        if (grp == 1)
            return;
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const floatx4 v = part[((b * 4 + c) * 4 + wave) * 64 + lane];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    tot[b >> 1][b & 1][4 * c + e] += v[e];
            }
    }
    {
        const int ldc = args.ldc;
        float *Cw = args.C + (size_t)(m0 + wr) * ldc + n0 + wc;
        const bool vec = ((uintptr_t)Cw & 15) == 0 && (ldc & 3) == 0;
        store_c_staged_w64_32(tot, lds, wave, lane, Cw, ldc, M - m0 - wr, N - n0 - wc, vec);
    }
}

template <int FMT>
hipError_t launch_fp8(const RingArgs &a, int tile, int groups, hipStream_t s)
{
    if (tile == kRing8SmallTile && groups == 2)
        hipLaunchKernelGGL((mfma_fp8_pair128_kernel<OpFp8<FMT>, 2>), dim3(a.tiles_m * a.tiles_n), dim3(512), 0, s, a);
    else if (tile == kRing8SmallTile)
        hipLaunchKernelGGL((mfma_fp8_pair128_kernel<OpFp8<FMT>, 1>), dim3(a.tiles_m * a.tiles_n), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(mfma_8bit_ring_kernel<OpFp8<FMT>>, dim3(a.tiles_m * a.tiles_n), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_ring8(const RingArgs &a, int fmt, int tile, int groups, hipStream_t s)
{
    if (a.accumulate || a.trans_a || a.trans_b || a.splits > 1 || a.alpha != 1.f)
        return hipErrorInvalidValue;
    if ((tile != kRing8Tile && tile != kRing8SmallTile) || groups < 1 || groups > 2 ||
        (groups == 2 && tile != kRing8SmallTile))
        return hipErrorInvalidValue;
    switch (fmt) {
    case kFmtE4M3:
        return launch_fp8<0>(a, tile, groups, s);
    case kFmtE5M2:
        return launch_fp8<1>(a, tile, groups, s);
    case kFmtI8:
        if (tile == kRing8SmallTile && groups == 2)
            hipLaunchKernelGGL(mfma_i8_pair128_kernel<2>, dim3(a.tiles_m * a.tiles_n), dim3(512), 0, s, a);
        else if (tile == kRing8SmallTile)
            hipLaunchKernelGGL(mfma_i8_pair128_kernel<1>, dim3(a.tiles_m * a.tiles_n), dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL(mfma_i8_pair_kernel, dim3(a.tiles_m * a.tiles_n), dim3(256), 0, s, a);
        return hipGetLastError();
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace dgor
