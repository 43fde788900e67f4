// Internal declarations shared by the host dispatcher and the kernel files.
// Not part of the public ABI (include/gemm.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm.h"

namespace dgor {

// One GEMM call after validation: row-major A (M x K), B (K x N), C (M x N).
struct Problem {
    int M, N, K;
    const void *A;  // float or binary16 bits
    const void *B;
    float *C;
    bool vec_a;     // A rows start 16-byte aligned and hold whole 128-bit vectors
    bool vec_b;     // same for B
    bool vec_c;     // same for C (FP32, 4 per vector)
};

// One launch of a ring kernel with general operand layouts: op(A) is M x K
// and op(B) is K x N.  A is M x K row-major (lda >= K) or, with trans_a,
// K x M row-major (lda >= M); B is K x N (ldb >= N) or, with trans_b, N x K
// (ldb >= K); C is M x N (ldc >= N).  The kernel writes C = op(A) op(B), or
// with `accumulate` C = C + op(A) op(B) (C read first).  Operands must be
// 16-byte aligned with every leading dimension a multiple of 16 bytes.
// The kernel stores alpha times its accumulators, which start at zero or,
// with accumulate, at C: C = alpha op(A) op(B) or C = alpha (C + op(A) op(B)).
// Split-K (splits > 1, not with accumulate): the launch has tiles_m *
// tiles_n * splits workgroups; workgroup b computes tile b % (tiles_m
// tiles_n) over k-range [s k_chunk, min(K, (s + 1) k_chunk)) with
// s = b / (tiles_m tiles_n), and writes it to C + s c_split_stride.  k_chunk
// is a multiple of 64.
struct RingArgs {
    int M, N, K;
    const void *A;
    int lda;
    const void *B;
    int ldb;
    float *C;
    int ldc;
    int tiles_m, tiles_n, group_m;
    bool trans_a, trans_b, accumulate;
    int splits = 1, k_chunk = 0;
    size_t c_split_stride = 0;
    float alpha = 1.f;
};

// Launchers.  Each enqueues exactly the kernel `plan` describes on `stream`
// and returns the launch status.  Shapes were validated by the caller.
hipError_t launch_zero_fill(const Problem &p, hipStream_t stream);
hipError_t launch_ladder_f32(const Problem &p, const gemm_plan &plan, hipStream_t stream);
// The 16-bit-input launchers take the input format: binary16 (bf16 false) or
// bfloat16 (bf16 true); tiles and data movement are the same for both.
hipError_t launch_naive_f16(const Problem &p, const gemm_plan &plan, hipStream_t stream, bool bf16);
hipError_t launch_mfma_f32(const Problem &p, const gemm_plan &plan, hipStream_t stream);
hipError_t launch_mfma_f16(const Problem &p, const gemm_plan &plan, hipStream_t stream, bool bf16);
// Ring kernels with general layouts (256 x 256 tiles; args.tiles_* set).
hipError_t launch_ring16(const RingArgs &args, hipStream_t stream, bool bf16);
hipError_t launch_ring32(const RingArgs &args, hipStream_t stream);
// C = s C over an M x N block with row stride ldc; s == 0 writes zeros
// without reading C.
hipError_t launch_scale_c(float *C, int M, int N, int ldc, float s, hipStream_t stream);
// The plain strided kernel for any layout: C = alpha op(A) op(B) + beta C
// (C not read when beta == 0).  in16: 0 binary32 inputs, 1 binary16, 2 bfloat16.
hipError_t launch_naive_ex(const RingArgs &args, float alpha, float beta, int in16, hipStream_t stream);

// 8-bit inputs: OCP FP8 E4M3 and E5M2 (FP32 accumulation and output), INT8
// (INT32 accumulation and output).  The ring kernel takes 256 x 256 tiles in
// k-steps of 64 (one byte per element), with A staged two steps at a time in
// three buffers and B one step at a time in four (160 KB of LDS); it needs
// 16-byte aligned operands with K and N multiples of 16.  The plain kernel
// takes anything.
constexpr int kFmtE4M3 = 0, kFmtE5M2 = 1, kFmtI8 = 2;
constexpr int kRing8Tile = 256, kRing8Depth = 64, kRing8Stages = 4;
constexpr int kRing8LdsBytes = 3 * kRing8Tile * 2 * kRing8Depth + kRing8Stages * kRing8Depth * kRing8Tile;
constexpr int kI8MaxK = 131072;   // |sum| <= 128 * 128 * K must fit int32
// Mid sizes: the same ring at a 128 x 128 tile, 80 KB of LDS (three 16 KB
// A pair buffers, four 8 KB B steps), two workgroups a compute unit.
constexpr int kRing8SmallTile = 128;
constexpr int kRing8SmallLdsBytes =
    3 * kRing8SmallTile * 2 * kRing8Depth + kRing8Stages * kRing8Depth * kRing8SmallTile;
// With at most one 128 x 128 tile per compute unit the ring runs two groups
// of four wavefronts over halves of the k-steps (512 threads, two 80 KB
// rings), their sums added in LDS.
inline bool ring8_small_split(int M, int N)
{
    return (long long)((M + 127) / 128) * ((N + 127) / 128) <= 256;
}
// tile: kRing8Tile or kRing8SmallTile; groups: 1, or 2 with kRing8SmallTile.
hipError_t launch_ring8(const RingArgs &args, int fmt, int tile, int groups, hipStream_t stream);

// Convolution through im2col: shape (P, Q derived), and the passes around the
// GEMM (conv.hip).  elem_bytes is 4 (binary32) or 2 (16-bit inputs).
struct Conv2d {
    int N, C, H, W, K, R, S, sh, sw, ph, pw, dh, dw, P, Q;
};
// wp null: W is used as it is (no padded copy); col null: no im2col matrix
hipError_t launch_conv_prepare(const Conv2d &cv, int elem_bytes, const void *x, const void *w, void *wp, void *col,
                               int crsp, int npqp, hipStream_t stream);
hipError_t launch_conv_output(const Conv2d &cv, const float *yp, float *y, int npqp, int splits,
                              size_t split_stride, hipStream_t stream);
// The implicit-GEMM convolution for 16-bit inputs (no im2col matrix): taken
// when its 128-filter x 256-pixel tiles number at least 256.  wa is K x CRSp
// with 16-byte aligned rows; y is written directly.  With stride 1 along w
// and Q a multiple of 4 it gathers with 12-byte loads from a zero-padded
// copy of x that it first writes to xp (N x C x (H + 2 ph) x (W + 2 pw
// rounded up to a multiple of 8): conv_padded_input_elems elements, plus 8
// of slack that are read but never used; xp 16-byte aligned), when x starts
// 4-byte aligned.
bool conv_igemm_applies(const Conv2d &cv, int elem_bytes);
bool conv_igemm_vec_applies(const Conv2d &cv, int elem_bytes);
long long conv_padded_input_elems(const Conv2d &cv);
hipError_t launch_conv_igemm(const Conv2d &cv, bool bf16, const void *x, const void *wa, float *y, int crsp,
                             void *xp, hipStream_t stream);
// The channels-last implicit GEMM for 16-bit inputs with C a multiple of
// 32 (conv_nhwc.hip): tiles of bm filters x bn pixels in bk-deep stages; the
// workspace holds Wr (K x R S C, wr_bytes) and then the zero-padded
// channels-last copy of x (N x (H + 2 ph) x (W + 2 pw) x C, xp_bytes).
struct NhwcPlan { int bm, bn, bk; size_t xp_bytes, wr_bytes; };
bool conv_nhwc_plan(const Conv2d &cv, int elem_bytes, NhwcPlan &np);
hipError_t launch_conv_nhwc(const Conv2d &cv, const NhwcPlan &np, bool bf16, const void *x, const void *w, float *y,
                            void *xp, void *wr, hipStream_t stream);
hipError_t launch_naive_8bit(const Problem &p, int fmt, hipStream_t stream);

// The arguments of the ring kernels for a plain row-major product.
inline RingArgs ring_args_nn(const Problem &p, const gemm_plan &plan)
{
    return RingArgs{p.M, p.N, p.K, p.A, p.K, p.B, p.N, p.C, p.N,
                    plan.grid_y, plan.grid_x, 4, false, false, false};
}

// LDS padding of the ladder rungs, in floats per row.  R3 and R4 pad each
// A row of their 16 x 64 tile by one float, moving consecutive rows to
// consecutive banks (the pages' one extra column); R5 pads each k row of its
// transposed 8 x 128 A tile by 8 floats.
constexpr int kLadderPadA = 1;
constexpr int kLadderPadB = 0;
constexpr int kRegblockPad = 8;

// Tile shapes of the matrix-core rungs.  The dispatcher picks one per call
// and the launcher recognises it by (plan.tile_m, plan.tile_n).
struct MfmaConfig { int bm, bn, bk, waves_m, waves_n; };

// FP32 (R6): LDS rows of A padded by 4 floats, rows of B by 8 floats.
constexpr int kF32PadA = 4;
constexpr int kF32PadB = 8;
constexpr MfmaConfig kF32Configs[] = {
    {128, 128, 16, 2, 2},   // large problems
    {64, 64, 16, 2, 2},     // problems too small to fill the chip with 128^2 tiles
    {32, 64, 16, 1, 2},     // N <= 64
};
constexpr int mfma_f32_lds_bytes(const MfmaConfig &c)
{
    return 2 * (c.bm * (c.bk + kF32PadA) + c.bk * (c.bn + kF32PadB)) * 4;
}

// FP16 (R7): LDS rows of A padded by 8 halves; k-pair rows of B by 8 words.
constexpr int kF16PadA = 8;
constexpr int kF16PadB = 8;
constexpr MfmaConfig kF16Configs[] = {
    {256, 256, 32, 2, 2},   // large problems: 128 x 128 per wavefront
    {128, 128, 32, 2, 2},
    {64, 64, 32, 1, 2},
};
constexpr int mfma_f16_lds_bytes(const MfmaConfig &c)
{
    return 2 * (c.bm * (c.bk + kF16PadA) * 2 + (c.bk / 2) * (c.bn + kF16PadB) * 4);
}

// The largest tile of each type runs a kernel that loads tiles straight from
// global memory into LDS (unpadded, swizzled stages) when both operands take
// 128-bit loads; lane byte offsets inside one tile then stay below 2^31.
// FP32: 128 x 128 x 16, two stages.  FP16: 256 x 256 x 32, B in a ring of
// four stages and (for an A given as M x K) A in three buffers of two stages.
constexpr int kF32DirectStages = 2;
constexpr int kF32DirectLdsBytes = kF32DirectStages * (128 * 16 + 16 * 128) * 4;
constexpr int kF16RingStages = 4;
// A staged two stages at a time (three 32 KB buffers), B one stage at a time
// (four 16 KB buffers): all 160 KB of LDS.
constexpr int kF16RingLdsBytes = 3 * 256 * 64 * 2 + kF16RingStages * 32 * 256 * 2;
inline bool direct_lds_applies(int tile_m, int top_tile, bool vec_a, bool vec_b, int N, int K)
{
    return tile_m == top_tile && vec_a && vec_b && K < (1 << 22) && N < (1 << 22);
}
// The 16-bit 128 x 128 tile (plain layout) runs the same ring at half the
// size: three 16 KB A buffers and four 8 KB B stages, 80 KB, so two
// workgroups share a compute unit.
constexpr int kF16Ring128LdsBytes = 3 * 128 * 64 * 2 + kF16RingStages * 32 * 128 * 2;
inline bool f16_ring128_applies(bool vec_a, bool vec_b, int N, int K)
{
    return vec_a && vec_b && K < (1 << 22) && N < (1 << 22);
}
// With at most one of its tiles per compute unit the 128 x 128 ring runs two
// groups of four wavefronts over halves of the k-stages (512 threads, two
// 80 KB rings), their sums added in LDS in a fixed order.
inline bool f16_ring128_split(int M, int N)
{
    return (long long)((M + 127) / 128) * ((N + 127) / 128) <= 256;
}

// FP32 problems that take the 64 x 64 tile with both operands in 128-bit
// loads run a ring of kF32SmallStages LDS stages kF32SmallDepth deep, loaded
// straight from global memory; lane byte offsets (k + depth) N 4 of B must
// stay below 2^31.  At 32 deep the ring takes 64 KB, so two workgroups share
// a compute unit when the shape has more tiles than there are units.
constexpr int kF32SmallDepth = 32;
constexpr int kF32SmallStages = 4;
constexpr int kF32SmallWavesN = 4;   // wavefronts along N (2 along M): 32 x 64 / kF32SmallWavesN each
constexpr int kF32SmallLdsBytes = kF32SmallStages * (64 * kF32SmallDepth + kF32SmallDepth * 64) * 4;
inline bool f32_small_ring_applies(int tile_m, int tile_n, int N, int K, bool vec_a, bool vec_b)
{
    return tile_m == 64 && tile_n == 64 && vec_a && vec_b && K < (1 << 22) &&
           (long long)(K + kF32SmallDepth) * N < (1LL << 29);
}
// With at most one 64 x 64 tile per compute unit and K of at least
// kF32SmallSplitMinK, the ring's workgroup is two groups of eight wavefronts,
// each over half of the k-stages with a ring of its own (128 KB, 1024
// threads); their sums are added in LDS in a fixed order.
constexpr int kF32SmallSplitMinK = 512;
inline bool f32_small_ring_split(int M, int N, int K)
{
    return (long long)((M + 63) / 64) * ((N + 63) / 64) <= 256 && K >= kF32SmallSplitMinK;
}

// Tall, narrow FP32 problems (1 <= N <= 64, 1 <= K <= kF32SkinnyMaxK, A and
// B 4-byte aligned): workgroups of 16 rows and 8 wavefronts, nb MFMA blocks
// of 16 columns; with fringe (N % 16 == 1, N > 16) the last column is summed
// on the vector ALUs instead of in a block of its own; with tail (M % 16 == 1
// and at least N whole row blocks) the last row is spread over workgroups
// 0..N-1 instead of getting one of its own.  Each wavefront streams its
// 16-deep k-slices through its own ring of skinny_slots(nb) LDS slots of
// skinny_slot_bytes(nb, fringe) bytes (the 16 x 16 piece of A, 16 rows of B's
// first 16 nb columns, B's last column), plus 1 KB for the tail row's
// products: at most 147,456 bytes for the 8 wavefronts.
constexpr int kF32SkinnyMaxK = 1024;
constexpr int skinny_slots(int nb) { return nb <= 3 ? 4 : 3; }
constexpr int skinny_slot_bytes(int nb, bool fringe) { return 1024 * (1 + nb) + (fringe ? 256 : 0); }
constexpr int skinny_wave_bytes(int nb, bool fringe)
{
    return skinny_slots(nb) * skinny_slot_bytes(nb, fringe) + 1024;
}
// With at most two column blocks a wavefront instead keeps its whole run of
// B (8 slices of nb KB) and, with fringe, B's last column (512 bytes) in LDS
// at once.
constexpr int skinny_resident_wave_bytes(int nb, bool fringe)
{
    return (kF32SkinnyMaxK / 128) * 1024 * nb + (fringe ? 512 : 0);
}
struct F32SkinnyPlan { int nb, blocks; bool fringe, tail; };
inline bool f32_skinny_plan(int M, int N, int K, F32SkinnyPlan &n)
{
    if (N < 1 || N > 64 || K < 1 || K > kF32SkinnyMaxK || M < 1 || (long long)M * K * 4 >= (1LL << 31) ||
        (long long)M * N * 4 >= (1LL << 31))
        return false;
    n.fringe = N > 16 && N % 16 == 1;
    n.nb = n.fringe ? N / 16 : (N + 15) / 16;
    const int full = M / 16, rem = M % 16;
    n.tail = rem == 1 && full >= N;
    n.blocks = full + (rem != 0 && !n.tail ? 1 : 0);
    return true;
}

// FP32 problems with both operands in 128-bit loads and at least one
// 256 x 256 tile per compute unit take a 256 x 256 x 16 tile fed through a
// ring of four LDS stages (lane byte offsets inside a tile stay below 2^31).
constexpr int kF32RingTile = 256;
constexpr int kF32RingDepth = 16;
constexpr int kF32RingStages = 4;
constexpr int kF32RingLdsBytes = kF32RingStages * (256 * 16 + 16 * 256) * 4;
constexpr int kF32RingWaves = 8;   // wavefronts per workgroup: 4 (128 x 128 each) or 8 (128 x 64)
inline bool f32_ring_applies(int M, int N, int K, bool vec_a, bool vec_b)
{
    const long tiles = (long)((M + kF32RingTile - 1) / kF32RingTile) * ((N + kF32RingTile - 1) / kF32RingTile);
    return vec_a && vec_b && K < (1 << 21) && N < (1 << 22) && tiles >= 256;
}

}  // namespace dgor

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------

// The part of a split-K launch this workgroup computes: narrows a's k-range
// and moves its A, B and C to that split (elem_bytes: input element size),
// and returns the workgroup's tile index.  Wave-uniform.
__device__ __forceinline__ int dgor_ring_split(dgor::RingArgs &a, int elem_bytes)
{
    int bid = blockIdx.x;
    if (a.splits > 1) {
        const int tiles = a.tiles_m * a.tiles_n;
        const int sp = bid / tiles;
        bid -= sp * tiles;
        const int k0 = sp * a.k_chunk;
        a.K = min(a.k_chunk, a.K - k0);
        a.A = (const char *)a.A + (a.trans_a ? (size_t)k0 * a.lda : (size_t)k0) * elem_bytes;
        a.B = (const char *)a.B + (a.trans_b ? (size_t)k0 : (size_t)k0 * a.ldb) * elem_bytes;
        a.C += (size_t)sp * a.c_split_stride;
    }
    return bid;
}

// The ring kernels keep their 256 accumulators per lane in the AGPRs; VALU
// arithmetic on them written in C++ makes the compiler move the whole array
// into ordinary registers, which do not fit beside the fragments.  The
// epilogue reads one accumulator at a time through an explicit AGPR move
// (and the accumulators are zeroed by AGPR writes, for the same reason).
// dgor_acc_hazard_wait() goes between the last MFMA and the first read: a
// 16-pass MFMA's result may be read by v_accvgpr_read only 19 wait states
// after it issues (CDNA3/CDNA4 instruction set, MFMA dependency rules).
__device__ __forceinline__ void dgor_acc_hazard_wait()
{
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
    __builtin_amdgcn_sched_barrier(0);
}
__device__ __forceinline__ float dgor_acc_read(float acc)
{
    float v;
    asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(acc));
    return v;
}
// Workgroup -> output tile, aware of the chip's 8 XCDs.  Consecutive
// workgroup ids are dealt round-robin to the XCDs, each with its own L2, so
// id b runs on XCD b % 8.  The ids of one XCD are first renumbered into one
// contiguous range of logical tiles; logical tiles are then walked in groups
// of `group_m` tile rows, column by column inside a group, so the tiles that
// one XCD runs at the same time share a few A row-panels and B column-panels.
__host__ __device__ __forceinline__ void dgor_tile_of_block(int bid, int tiles_m, int tiles_n,
                                                   int group_m, int &tm, int &tn)
{
    const int nb = tiles_m * tiles_n;
    const int per = nb >> 3, rem = nb & 7;
    const int xcd = bid & 7, local = bid >> 3;
    const int logical = xcd * per + (xcd < rem ? xcd : rem) + local;
    const int span = group_m * tiles_n;
    const int group = logical / span;
    const int first_m = group * group_m;
    const int gm = min(tiles_m - first_m, group_m);
    const int in_group = logical - group * span;
    tm = first_m + in_group % gm;
    tn = in_group / gm;
}
