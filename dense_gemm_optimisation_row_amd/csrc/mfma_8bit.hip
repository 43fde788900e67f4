// 8-bit inputs on the matrix cores: FP8 (OCP E4M3 and E5M2) with FP32
// accumulation and output, and INT8 with INT32 accumulation and output
// ("Lesson 8: how a GPU does matrix multiply", section 22 lists FP8 and INT8
// among the matrix units' input formats; its sections 24-25 give the
// staged, double-buffered K-loop this kernel deepens into a ring).
//
// One kernel template covers the three formats.  A workgroup of four
// wavefronts computes a 256 x 256 tile of C; each wavefront a 128 x 128
// quarter as 4 x 4 blocks of 32 x 32 accumulators (256 accumulator
// registers per lane).  Per 64-deep k-step a block takes one
// v_mfma_scale_f32_32x32x64_f8f6f4 (FP8, unit scales) or two
// v_mfma_i32_32x32x32_i8 (INT8).
//
// * Fragments.  Lane l = (r, g) = (l % 32, l / 32) holds k-values of row r
//   of its op(A) block and of column r of its op(B) block: FP8 all 32 of
//   32 g .. 32 g + 31 in one k-step, INT8 16 of them in each of two
//   sub-steps (32 g + 16 h .. + 15 in sub-step h).  The matrix unit pairs
//   the same register bytes of A and B lanes, so each k of the step is
//   summed exactly once.  Output: element e of lane l is row
//   8 (e / 4) + 4 g + e % 4, column l % 32 of the block.
// * Loads go straight from global memory into LDS (buffer_load_dwordx4 ...
//   lds): one instruction moves 64 lanes x 16 bytes into 1 KB of LDS, lane p
//   landing at byte 16 p, and a lane whose offset is out of range writes
//   zeros, which zero-fills every edge.
// * LDS layout of one stage (16-byte units):
//     k-contiguous operand (A, or B given as N x K): 256 rows of 64 k,
//       unit c of row r at 4 r + (c ^ ((r >> 2) & 3));
//     k-strided operand (B, or A given as K x M): 64 k rows of 256,
//       unit u of row k at 16 k + (u ^ (2 (k & 7))).
//   k-contiguous fragments are two 128-bit reads (units 2 g and 2 g + 1).
//   k-strided fragments are four transposing reads (ds_read_b64_tr_b8): in a
//   group of 16 lanes, source lane s points at 8 bytes of row kb + s / 2,
//   columns nb + 8 (s % 2) .. + 7, and output lane i receives rows
//   kb .. kb + 7 of column nb + i.  Both swizzles keep the reads free of
//   bank conflicts under the LDS rule measured for the 16-bit ring (a
//   128-bit read is served in four cycles of 16 lanes that agree in lane
//   bit 5 and the parity of lane bits 2..4; a 64-bit read 32 lanes a cycle;
//   a cycle is conflict-free when its 16-byte units, or 8-byte halves,
//   differ modulo the 256-byte row of banks).
// * Pipeline.  Four LDS buffers of 32 KB.  FP8 reads all fragments of
//   stage t during stage t - 1, so stage t's buffer is free once stage t
//   begins: during stage t each wavefront refills it with the 8 loads of
//   stage t + 4.  INT8 still reads stage t's second sub-step during stage t,
//   so it refills the buffer of stage t - 1 with stage t + 3.  The loads are
//   spread over the stage's MFMAs, and the fragment reads of the next
//   (sub-)step over the first three quarters of those of the current one.
//   Before stage t: one wait for the loads of stage t + 1 (the later ones
//   stay in flight) and for this wavefront's own LDS reads, then one
//   barrier, after which no wavefront still reads the buffer the stage's
//   loads overwrite.
#include "common.h"
#include "lds_dma.h"

namespace dgor {
namespace {

typedef int intx8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef int intx16 __attribute__((ext_vector_type(16)));
typedef int intx2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) intx2 lds_intx2;

// Per-format pieces of the kernel.  kSub: sub-steps per 64-deep k-step;
// kReadsKC / kReadsKS: reads per fragment of a k-contiguous (128-bit) or
// k-strided (64-bit transposing) operand in one sub-step; put16 / put8 place
// read `part` of a sub-step in the fragment.
//
// FP8: one v_mfma_scale_f32_32x32x64_f8f6f4 per block and k-step, with unit
// block scales (E8M0 127 = 2^0); format code 0 is E4M3, 1 is E5M2.
template <int FMT>
struct OpFp8 {
    typedef floatx16 Acc;
    typedef intx8 Frag;
    static constexpr int kSub = 1, kReadsKC = 2, kReadsKS = 4;
    __device__ static void put16(Frag &f, int part, const intx4 &v)
    {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            f[4 * part + e] = v[e];
    }
    __device__ static void put8(Frag &f, int part, const intx2 &v)
    {
        f[2 * part + 0] = v[0];
        f[2 * part + 1] = v[1];
    }
    __device__ static Acc mma(const Frag &a, const Frag &b, Acc c)
    {
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FMT, FMT, 0, 127, 0, 127);
    }
    __device__ static uint32_t bits(float x) { return __float_as_uint(x); }
};

// INT8: one v_mfma_i32_32x32x32_i8 per block and sub-step, two sub-steps per
// k-step, each with its own 16-byte fragments (half the registers of
// 32-byte ones, which the register allocator needs here).
struct OpI8 {
    typedef intx16 Acc;
    typedef intx4 Frag;
    static constexpr int kSub = 2, kReadsKC = 1, kReadsKS = 2;
    __device__ static void put16(Frag &f, int, const intx4 &v) { f = v; }
    __device__ static void put8(Frag &f, int part, const intx2 &v)
    {
        f[2 * part + 0] = v[0];
        f[2 * part + 1] = v[1];
    }
    __device__ static Acc mma(const Frag &a, const Frag &b, Acc c)
    {
        return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
    }
    __device__ static uint32_t bits(int x) { return (uint32_t)x; }
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

// The plain row-major product (A M x K, B K x N).  A is staged two k-steps
// at a time so that every A row a load touches is one whole 128-byte line;
// B rows (256 bytes of a tile) are whole lines already.
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

    // ---- loader.  Step s (k = 64 s .. 64 s + 63) of B lives in B buffer
    // s % 4; steps 2P and 2P + 1 of A (pair P) in A buffer P % 3.
    //   A pair buffer: 256 rows of 128 bytes, 16-byte unit c of row r at
    //     8 r + (c ^ ((r >> 1) & 7)); wave w's load j (0..7) fills rows
    //     8 n .. 8 n + 7, n = 8 w + j, lane p taking physical unit p % 8 of
    //     row 8 n + p / 8.
    //   B buffer: 64 k rows of 256 bytes, unit u of row k at
    //     16 k + (u ^ (2 (k & 7))); wave w's load q fills rows 4 n .. 4 n + 3,
    //     n = 4 w + q, lane p taking physical unit p % 16 of row 4 n + p / 16.
    // Descriptor ranges end at the last row of the operand and at K, so
    // everything past them loads as zero; A lanes past K in the last pair are
    // masked (K is a multiple of 16).
    // A load j's lane offset: a_off[j & 1] plus (j / 2) * 16 rows (wave-uniform)
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

    typedef typename Op::Frag Frag;
    // Where the reads of one sub-step come from: A pair buffer (byte offset)
    // and half (which step of the pair), B buffer (byte offset), sub-step h.
    struct ReadSrc { uint32_t a_buf; int a_half; uint32_t b_buf; int h; };
    auto read_a = [&](const ReadSrc &R, int blk, int part, Frag &f) {
        const int u = R.h * Op::kReadsKC + part;
        const uint32_t addr = a_lane_at(R.a_half, u) + R.a_buf + (uint32_t)(blk * 32 * 128);
        Op::put16(f, part, *reinterpret_cast<const intx4 *>(lds + addr));
    };
    auto read_b = [&](const ReadSrc &R, int blk, int part, Frag &f) {
        const int q = R.h * Op::kReadsKS + part;
        const uint32_t addr = b_lane[blk] + R.b_buf + (uint32_t)(q * 2048);
        Op::put8(f, part, __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_intx2 *)(lds + addr)));
    };
    // The reads of one sub-step in the order its MFMAs want them: A block 0,
    // B blocks 0..3, A blocks 1..3; r runs over 0 .. R_SUB - 1.
    constexpr int PA = Op::kReadsKC, PB = Op::kReadsKS;
    constexpr int R_SUB = 4 * PA + 4 * PB;
    auto fread = [&](const ReadSrc &R, int r, Frag *fa, Frag *fb) {
        if (r < PA) {
            read_a(R, 0, r, fa[0]);
        } else if (r < PA + 4 * PB) {
            const int q = r - PA;
            read_b(R, q / PB, q % PB, fb[q / PB]);
        } else {
            const int q = r - PA - 4 * PB;
            read_a(R, 1 + q / PA, q % PA, fa[1 + q / PA]);
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

    typename Op::Acc acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[i][j][e] = 0;

    // One sub-step h of step s: its 16 MFMAs (row-major over the blocks) from
    // (ca, cb); the reads of the next sub-step (h + 1 of step s, or 0 of step
    // s + 1), described by R, into (na, nb) over the first 12 of them; this
    // sub-step's share of step s's 8 loads (B step s + 3, then half `par` of
    // A pair s / 2 + 2), spread over the step's MFMAs.
    //
    // Buffers: A pair P is read during steps 2P - 1 .. 2P + 1 and refilled
    // with pair P + 3 during steps 2P + 2, 2P + 3; B step s is read during
    // steps s - 1 and s and its buffer refilled with step s + 4 during step
    // s + 1.  Both refills start after the barrier that ends the last reads.
    constexpr int READ_SLOTS = 12;
    constexpr int LOAD_EVERY = 16 * Op::kSub / LOADS_PER_STEP;
    struct StepLoads { intx4 rb; uint32_t b_dst; PairLoads a; };
    auto substep = [&](int h, int par, const StepLoads &L, const ReadSrc &R, Frag *ca, Frag *cb, Frag *na,
                       Frag *nb) {
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            acc[m >> 2][m & 3] = Op::mma(ca[m >> 2], cb[m & 3], acc[m >> 2][m & 3]);
            if (m < READ_SLOTS) {
#pragma unroll
                for (int r = m * R_SUB / READ_SLOTS; r < (m + 1) * R_SUB / READ_SLOTS; ++r)
                    fread(R, r, na, nb);
            }
            const int mg = 16 * h + m;
            if (mg % LOAD_EVERY == LOAD_EVERY - 1) {
                const int ld = mg / LOAD_EVERY;   // 0..7: B loads 0..3, then the A half
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
    Frag fa0[4], fa1[4], fb0[4], fb1[4];
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
        const ReadSrc R0{0u, 0, b_buf(0), 0};
#pragma unroll
        for (int r = 0; r < R_SUB; ++r)
            fread(R0, r, fa0, fb0);
    }

    // Two steps (one A pair, P = s / 2) per trip, so each step's parity is
    // known here; pa, pa1, pa2 are the buffers of pairs P, P + 1, P + 2.
    const int steps = (K + BK - 1) / BK;
    uint32_t pa = 0;
    for (int s = 0; s < steps; s += 2) {
        const uint32_t pa1 = next_pair(pa), pa2 = next_pair(pa1);
        StepLoads L = step_begin(s, pa2);
        if constexpr (Op::kSub == 1) {
            substep(0, 0, L, ReadSrc{pa, 1, b_buf(s + 1), 0}, fa0, fb0, fa1, fb1);
        } else {
            substep(0, 0, L, ReadSrc{pa, 0, b_buf(s), 1}, fa0, fb0, fa1, fb1);
            substep(1, 0, L, ReadSrc{pa, 1, b_buf(s + 1), 0}, fa1, fb1, fa0, fb0);
        }
        if (s + 1 < steps) {
            L = step_begin(s + 1, pa2);
            if constexpr (Op::kSub == 1) {
                substep(0, 1, L, ReadSrc{pa1, 0, b_buf(s + 2), 0}, fa1, fb1, fa0, fb0);
            } else {
                substep(0, 1, L, ReadSrc{pa, 1, b_buf(s + 1), 1}, fa0, fb0, fa1, fb1);
                substep(1, 1, L, ReadSrc{pa1, 0, b_buf(s + 2), 0}, fa1, fb1, fa0, fb0);
            }
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
                __builtin_amdgcn_raw_buffer_store_b32(Op::bits(acc[i][j][e]), rc, vo, so, 0);
            }
}

template <class Op>
hipError_t launch_ring(const RingArgs &a, hipStream_t s)
{
    const dim3 grid(a.tiles_m * a.tiles_n);
    hipLaunchKernelGGL(mfma_8bit_ring_kernel<Op>, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_ring8(const RingArgs &a, int fmt, hipStream_t s)
{
    if (a.accumulate || a.trans_a || a.trans_b || a.splits > 1 || a.alpha != 1.f)
        return hipErrorInvalidValue;
    switch (fmt) {
    case kFmtE4M3:
        return launch_ring<OpFp8<0>>(a, s);
    case kFmtE5M2:
        return launch_ring<OpFp8<1>>(a, s);
    case kFmtI8:
        return launch_ring<OpI8>(a, s);
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace dgor
