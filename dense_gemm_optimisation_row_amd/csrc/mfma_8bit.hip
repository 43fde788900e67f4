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
// * Pipeline: as the 16-bit ring.  Four stages of 32 KB; each wavefront
//   issues the fragment reads of the next (sub-)step over the first three
//   quarters of the current one's MFMAs, and the 8 loads of stage t + 3
//   spread over all of stage t's MFMAs; one vmcnt(8) wait and one barrier
//   precede each stage.
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
constexpr int BM = 256, BN = 256, BK = 64, NBUF = 4;
constexpr int A_BYTES = BM * BK;                     // 16 KB
constexpr int B_BYTES = BK * BN;                     // 16 KB
constexpr int STAGE_BYTES = A_BYTES + B_BYTES;       // 32 KB
constexpr int LDS_BYTES = NBUF * STAGE_BYTES;        // 128 KB
constexpr int LOADS_PER_STAGE = 8;                   // per wavefront: 4 of A, 4 of B

// Lane offsets (bytes) of wave w's four 1 KB loads of one operand tile per
// stage, relative to the stage's first element (k0 of row t0 for the
// k-contiguous layout, column t0 of row k0 for the k-strided one).  ext is
// the extent of the operand's non-k dimension, ld its row stride.
template <bool KSTRIDED>
__device__ __forceinline__ void load_offsets(int wave, int lane, int t0, int ext, int ld, uint32_t off[4],
                                             int &kc)
{
    constexpr uint32_t OOB = 0x80000000u;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        if (!KSTRIDED) {
            const int r = 16 * (4 * wave + q) + (lane >> 2);
            kc = 16 * ((lane & 3) ^ ((lane >> 4) & 3));   // same in every block
            off[q] = (uint32_t)(r * ld + kc);
        } else {
            const int k = 4 * (4 * wave + q) + (lane >> 4);
            const int u = (lane & 15) ^ (2 * (k & 7));
            off[q] = t0 + 16 * u < ext ? (uint32_t)(k * ld + 16 * u) : OOB;
            kc = 0;
        }
    }
}

// Range in bytes of one stage's descriptor: everything past it is a row
// past the operand, or a k row past K.
template <bool KSTRIDED>
__device__ __forceinline__ int stage_range(int k0, int K, int t0, int ext, int ld)
{
    const int k_left = K - k0;
    if (k_left <= 0)
        return 0;   // a stage past the last: every load writes zeros
    if (!KSTRIDED) {
        if (t0 + 256 <= ext)
            return 0x7fffffff;
        return (int)((uint32_t)(ext - t0 - 1) * (uint32_t)ld + (uint32_t)k_left);
    }
    if (k_left >= BK)
        return 0x7fffffff;
    return (int)((uint32_t)(k_left - 1) * (uint32_t)ld + (uint32_t)(ext - t0));
}
}  // namespace ring8

template <class Op, bool TA, bool TB>
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

    // ---- loader (the range rules of the 16-bit ring, in bytes)
    uint32_t a_off[4], b_off[4];
    int a_kc, b_kc;
    ring8::load_offsets<TA>(wave, lane, m0, M, lda, a_off, a_kc);
    ring8::load_offsets<!TB>(wave, lane, n0, N, ldb, b_off, b_kc);
    const uint32_t lds_a = ring + (uint32_t)(4 * wave * 1024);
    const uint32_t lds_b = ring + (uint32_t)(A_BYTES + 4 * wave * 1024);
    struct StageLoads { intx4 ra, rb; uint32_t lds; bool tail; int k_left; };
    auto prep = [&](int st) {
        StageLoads L;
        const int k0 = st * BK;
        L.ra = rsrc_words(TA ? A + (size_t)k0 * lda + m0 : A + (size_t)m0 * lda + k0, 0);
        L.ra.z = ring8::stage_range<TA>(k0, K, m0, M, lda);
        L.rb = rsrc_words(TB ? B + (size_t)n0 * ldb + k0 : B + (size_t)k0 * ldb + n0, 0);
        L.rb.z = ring8::stage_range<!TB>(k0, K, n0, N, ldb);
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

    // ---- fragment reads
    const int r32 = lane & 31, g = lane >> 5;
    const int s16 = lane & 15, hg = (lane >> 4) & 1;
    // k-contiguous block blk: row base + 32 blk + r32, logical units 2 g, 2 g + 1
    auto kc_addr = [&](uint32_t region, int base, int h) {
        return region + (uint32_t)((base + r32) * 64 + (((2 * g + h) ^ ((r32 >> 2) & 3)) * 16));
    };
    // k-strided block blk, read q: row 32 g + 8 q + s16 / 2, byte 8 (s16 % 2)
    // of logical unit base / 16 + 2 blk + hg, at physical unit
    // unit ^ (2 (row & 7)) = unit ^ (s16 & 14); base is 0 or 128, so its unit
    // bit (8) is applied by XOR on the byte offset.
    auto ks_units = [&](int base, uint32_t unit[4]) {
#pragma unroll
        for (int b = 0; b < 4; ++b)
            unit[b] = ((uint32_t)(((2 * b) ^ (s16 & 14)) | hg) * 16u) ^ (uint32_t)base;
    };
    auto ks_row = [&](uint32_t region) {
        return region + (uint32_t)((32 * g + (s16 >> 1)) * 256 + 8 * (s16 & 1));
    };
    uint32_t a_unit[4], b_unit[4];
    if (TA)
        ks_units(wr, a_unit);
    if (!TB)
        ks_units(wc, b_unit);
    const uint32_t a_lane0 = TA ? ks_row(0) : kc_addr(0, wr, 0);
    const uint32_t a_lane1 = kc_addr(0, wr, 1);
    const uint32_t b_lane0 = TB ? kc_addr(A_BYTES, wc, 0) : ks_row(A_BYTES);
    const uint32_t b_lane1 = kc_addr(A_BYTES, wc, 1);

    // Read `part` (0 .. reads per fragment - 1) of sub-step h's fragment of
    // block blk: k-contiguous unit 2 g + h kReadsKC + part, or k-strided rows
    // 32 g + 8 (h kReadsKS + part) + s16 / 2.
    typedef typename Op::Frag Frag;
    auto read_part = [&](uint32_t stage_off, bool kstrided, uint32_t lane0, uint32_t lane1,
                         const uint32_t *unit, int blk, int h, int part, Frag &f) {
        if (!kstrided) {
            const int u = h * Op::kReadsKC + part;   // 0 or 1: which of the lane's two units
            const uint32_t addr = (u ? lane1 : lane0) + stage_off + (uint32_t)(blk * 2048);
            Op::put16(f, part, *reinterpret_cast<const intx4 *>(lds + addr));
        } else {
            const int q = h * Op::kReadsKS + part;
            const uint32_t addr = lane0 + stage_off + (uint32_t)(q * 2048) + unit[blk];
            Op::put8(f, part, __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_intx2 *)(lds + addr)));
        }
    };
    // The reads of one sub-step in the order its MFMAs want them: A block 0,
    // B blocks 0..3, A blocks 1..3; r runs over 0 .. R_SUB - 1.
    constexpr int PA = TA ? Op::kReadsKS : Op::kReadsKC, PB = TB ? Op::kReadsKC : Op::kReadsKS;
    constexpr int R_SUB = 4 * PA + 4 * PB;
    auto fread = [&](int stage, int h, int r, Frag *fa, Frag *fb) {
        const uint32_t so = (uint32_t)((stage % NBUF) * STAGE_BYTES);
        if (r < PA) {
            read_part(so, TA, a_lane0, a_lane1, a_unit, 0, h, r, fa[0]);
        } else if (r < PA + 4 * PB) {
            const int q = r - PA;
            read_part(so, !TB, b_lane0, b_lane1, b_unit, q / PB, h, q % PB, fb[q / PB]);
        } else {
            const int q = r - PA - 4 * PB;
            read_part(so, TA, a_lane0, a_lane1, a_unit, 1 + q / PA, h, q % PA, fa[1 + q / PA]);
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

    // One sub-step h of stage t: its 16 MFMAs (row-major over the blocks)
    // from (ca, cb); the reads of the next sub-step (h + 1 of stage t, or 0
    // of stage t + 1) into (na, nb) over the first 12 of them; this
    // sub-step's share of the 8 loads of stage t + 3, spread evenly over the
    // stage's MFMAs.
    constexpr int READ_SLOTS = 12;
    constexpr int LOAD_EVERY = 16 * Op::kSub / LOADS_PER_STAGE;
    auto substep = [&](int t, int h, const StageLoads &L, Frag *ca, Frag *cb, Frag *na, Frag *nb) {
        const int nt = h + 1 < Op::kSub ? t : t + 1, nh = h + 1 < Op::kSub ? h + 1 : 0;
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            acc[m >> 2][m & 3] = Op::mma(ca[m >> 2], cb[m & 3], acc[m >> 2][m & 3]);
            if (m < READ_SLOTS) {
#pragma unroll
                for (int r = m * R_SUB / READ_SLOTS; r < (m + 1) * R_SUB / READ_SLOTS; ++r)
                    fread(nt, nh, r, na, nb);
            }
            const int mg = 16 * h + m;
            if (mg % LOAD_EVERY == LOAD_EVERY - 1)
                load(L, mg / LOAD_EVERY);
            // keep this order: the compiler would otherwise cluster the reads
            // and loads, and move MFMAs across the barrier
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // Before stage t: this wavefront's loads of stage t + 1 have landed
    // (those of t + 2 may stay in flight), and the workgroup meets at the
    // barrier.  Reads and loads past the last stage touch unused data.
    auto stage_begin = [&](int t) {
        __builtin_amdgcn_s_waitcnt(wait_vmcnt(LOADS_PER_STAGE));
        __builtin_amdgcn_s_barrier();
        const StageLoads L = prep(t + 3);
        __builtin_amdgcn_sched_barrier(0);
        return L;
    };

    // prologue: loads of stages 0, 1, 2, then the reads of stage 0
    Frag fa0[4], fa1[4], fb0[4], fb1[4];
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
    for (int r = 0; r < R_SUB; ++r)
        fread(0, 0, r, fa0, fb0);

    const int steps = (K + BK - 1) / BK;
    if constexpr (Op::kSub == 1) {
        for (int t = 0; t < steps; t += 2) {
            StageLoads L = stage_begin(t);
            substep(t, 0, L, fa0, fb0, fa1, fb1);
            if (t + 1 < steps) {
                L = stage_begin(t + 1);
                substep(t + 1, 0, L, fa1, fb1, fa0, fb0);
            }
        }
    } else {
        for (int t = 0; t < steps; ++t) {
            const StageLoads L = stage_begin(t);
            substep(t, 0, L, fa0, fb0, fa1, fb1);
            substep(t, 1, L, fa1, fb1, fa0, fb0);
        }
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

template <class Op, bool TA, bool TB>
hipError_t launch_ring(const RingArgs &a, hipStream_t s)
{
    const dim3 grid(a.tiles_m * a.tiles_n);
    hipLaunchKernelGGL((mfma_8bit_ring_kernel<Op, TA, TB>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

template <class Op>
hipError_t launch_any(const RingArgs &a, hipStream_t s)
{
    if (a.trans_a && a.trans_b)
        return launch_ring<Op, true, true>(a, s);
    if (a.trans_a)
        return launch_ring<Op, true, false>(a, s);
    if (a.trans_b)
        return launch_ring<Op, false, true>(a, s);
    return launch_ring<Op, false, false>(a, s);
}

}  // namespace

hipError_t launch_ring8(const RingArgs &a, int fmt, hipStream_t s)
{
    if (a.accumulate)
        return hipErrorInvalidValue;
    switch (fmt) {
    case kFmtE4M3:
        return launch_any<OpFp8<0>>(a, s);
    case kFmtE5M2:
        return launch_any<OpFp8<1>>(a, s);
    case kFmtI8:
        return launch_any<OpI8>(a, s);
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace dgor
