// C ABI of the library (declared in include/gemm.h): argument validation,
// launch planning and dispatch.  Host code only; the kernels live in
// ladder.hip, mfma_f32.hip, mfma_f16.hip and mfma_8bit.hip.
//
// Planning is pure arithmetic on the arguments (no HIP call), so the plan
// entry points work on a machine without a GPU.  The grid follows the
// pages' ceil-div rule ("Lesson 8: how a GPU does matrix multiply", section 3):
// ceil(N / tile_n) workgroups along N and ceil(M / tile_m) along M.
#include <atomic>
#include <math.h>
#include <mutex>
#include <stdint.h>

#include "common.h"

namespace {

using dgor::MfmaConfig;

constexpr int kDevCache = 64;
std::atomic<int> g_dev_state[kDevCache];  // 0 unknown, 1 gfx950, 2 other

int ceil_div(int a, int b) { return (a + b - 1) / b; }

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int check_device()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return GEMM_ERR_RUNTIME;
    if (dev >= 0 && dev < kDevCache) {
        const int st = g_dev_state[dev].load(std::memory_order_relaxed);
        if (st == 1)
            return GEMM_OK;
        if (st == 2)
            return GEMM_ERR_UNSUPPORTED_DEVICE;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
        return GEMM_ERR_RUNTIME;
    const char *arch = prop.gcnArchName;
    const bool ok = arch[0] == 'g' && arch[1] == 'f' && arch[2] == 'x' && arch[3] == '9' &&
                    arch[4] == '5' && arch[5] == '0' && (arch[6] == 0 || arch[6] == ':');
    if (dev >= 0 && dev < kDevCache)
        g_dev_state[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
    return ok ? GEMM_OK : GEMM_ERR_UNSUPPORTED_DEVICE;
}

void clear(gemm_plan *p)
{
    *p = gemm_plan{};
}

// Fill the tile-independent fields of a plan.
void finish(gemm_plan *p, int M, int N, int K)
{
    p->launches = 1;
    p->grid_x = ceil_div(N, p->tile_n);
    p->grid_y = ceil_div(M, p->tile_m);
    p->k_stages = p->tile_k ? ceil_div(K, p->tile_k) : 0;
}

// Which matrix-core configuration a shape gets: the largest tile that still
// yields at least two workgroups per compute unit (256 CUs), else the tile
// that yields the most workgroups; N <= 64 takes the narrow FP32 tile.
template <size_t NC>
int pick_config(const MfmaConfig (&cfg)[NC], int M, int N, bool narrow_ok)
{
    if (narrow_ok && N <= 64)
        return (int)NC - 1;
    const int full = narrow_ok ? (int)NC - 1 : (int)NC;
    for (int i = 0; i < full; ++i) {
        const long tiles = (long)ceil_div(M, cfg[i].bm) * ceil_div(N, cfg[i].bn);
        if (tiles >= 512)
            return i;
    }
    return full - 1;
}

// Expected fraction of the matrix peak of a tile choice: the kernel's own
// rate (rate_few with under two tiles per compute unit, whose first loads
// and last stores nothing else hides; rate_many from two up) times how
// evenly the tiles spread over the 256 compute units, since the unit with
// the most tiles sets the time.  Measured rates: the FP32 256 x 256 ring
// 0.93; the 128 x 128 direct-load kernel 0.75 and 0.87; the 64 x 64 ring 0.66
// and 0.83.
double tile_estimate(long tiles, double rate_few, double rate_many)
{
    const long per = (tiles + 255) / 256;
    return (tiles < 512 ? rate_few : rate_many) * (double)tiles / (256.0 * (double)per);
}

// The FP32 tile for operands that take 128-bit direct loads: 256, 128 or 64
// (0: none of the direct-load kernels applies).
int f32_direct_tile(int M, int N, int K, bool vec_a, bool vec_b)
{
    auto tiles = [&](int t) { return (long)ceil_div(M, t) * ceil_div(N, t); };
    const double e256 =
        dgor::f32_ring_applies(M, N, K, vec_a, vec_b) ? tile_estimate(tiles(256), 0.93, 0.93) : -1;
    const double e128 =
        dgor::direct_lds_applies(128, 128, vec_a, vec_b, N, K) ? tile_estimate(tiles(128), 0.75, 0.87) : -1;
    const double e64 =
        dgor::f32_small_ring_applies(64, 64, N, K, vec_a, vec_b) ? tile_estimate(tiles(64), 0.66, 0.83) : -1;
    if (e256 > 0 && e256 >= e128 && e256 >= e64)
        return 256;
    if (e64 > 0 && e64 >= e128)
        return 64;
    return e128 > 0 ? 128 : 0;
}

int plan_f32(int variant, int M, int N, int K, const void *A, const void *B, const void *C,
             gemm_plan *p)
{
    if (!p)
        return GEMM_ERR_NULL_PTR;
    if (M < 0 || N < 0 || K < 0)
        return GEMM_ERR_INVALID_DIM;
    if (variant == GEMM_VARIANT_AUTO)
        variant = GEMM_R6_MFMA_F32;
    if (variant < GEMM_R0_NAIVE || variant > GEMM_R6_MFMA_F32)
        return GEMM_ERR_INVALID_VARIANT;
    clear(p);
    p->variant = variant;
    p->vector_a = (K % 4 == 0) && aligned16(A);
    p->vector_b = (N % 4 == 0) && aligned16(B);
    p->vector_c = (N % 4 == 0) && aligned16(C);
    if (M == 0 || N == 0)
        return GEMM_OK;
    if (K == 0) {  // empty sum: one zero-fill launch
        p->launches = 1;
        p->threads = 256;
        p->vector_a = p->vector_b = p->vector_c = 0;
        return GEMM_OK;
    }
    switch (variant) {
    case GEMM_R0_NAIVE:
        p->tile_m = p->tile_n = 16;
        p->tile_k = 0;
        p->threads = 256;
        p->outputs_per_thread = 1;
        p->vector_a = p->vector_b = p->vector_c = 0;
        break;
    case GEMM_R1_LDS_TILED:
        p->tile_m = p->tile_n = p->tile_k = 16;
        p->threads = 256;
        p->lds_stages = 1;
        p->lds_bytes = 2 * 16 * 16 * 4;
        p->tile_bytes = 2 * 16 * 16 * 4;
        p->outputs_per_thread = 1;
        p->vector_a = p->vector_b = p->vector_c = 0;
        break;
    case GEMM_R2_VECTOR_LOADS:
    case GEMM_R3_LDS_PADDED:
    case GEMM_R4_DOUBLE_BUFFER: {
        const bool pad = variant != GEMM_R2_VECTOR_LOADS;
        p->tile_m = p->tile_n = 16;
        p->tile_k = 64;
        p->threads = 256;
        p->lds_stages = variant == GEMM_R4_DOUBLE_BUFFER ? 2 : 1;
        const int pa = pad ? dgor::kLadderPadA : 0, pb = pad ? dgor::kLadderPadB : 0;
        p->lds_bytes = p->lds_stages * (16 * (64 + pa) + 64 * (16 + pb)) * 4;
        p->tile_bytes = (16 * 64 + 64 * 16) * 4;
        p->outputs_per_thread = 1;
        p->vector_c = 0;
        break;
    }
    case GEMM_R5_REGISTER_BLOCKED:
        p->tile_m = p->tile_n = 128;
        p->tile_k = 8;
        p->threads = 256;
        p->lds_stages = 2;
        p->lds_bytes = 2 * (8 * (128 + dgor::kRegblockPad) + 8 * 128) * 4;
        p->tile_bytes = (128 * 8 + 8 * 128) * 4;
        p->outputs_per_thread = 64;
        break;
    case GEMM_R6_MFMA_F32: {
        const int direct = f32_direct_tile(M, N, K, p->vector_a, p->vector_b);
        if (direct == dgor::kF32RingTile) {
            p->tile_m = p->tile_n = dgor::kF32RingTile;
            p->tile_k = dgor::kF32RingDepth;
            p->threads = 64 * dgor::kF32RingWaves;
            p->lds_stages = dgor::kF32RingStages;
            p->lds_bytes = dgor::kF32RingLdsBytes;
            p->tile_bytes = 2 * dgor::kF32RingTile * dgor::kF32RingDepth * 4;
            p->outputs_per_thread = dgor::kF32RingTile * dgor::kF32RingTile / p->threads;
            p->vector_c = 0;
            break;
        }
        dgor::F32SkinnyPlan nw;
        if (dgor::f32_skinny_plan(M, N, K, nw)) {
            // one workgroup per 16 rows (grid_y), all columns (tile_n: the
            // MFMA blocks, plus 1 for a column summed on the vector ALUs) and
            // all of K in eight runs of 16-deep slices; with at most two
            // blocks each wavefront holds its whole run of B in LDS (8
            // slices), else it streams the run through a ring of LDS slots
            p->tile_m = 16;
            p->tile_n = 16 * nw.nb + (nw.fringe ? 1 : 0);
            p->tile_k = 16 * ((K + 15) / 16);
            p->threads = 512;
            const bool resident = nw.nb <= 2;
            p->lds_stages = resident ? dgor::kF32SkinnyMaxK / 128 : dgor::skinny_slots(nw.nb);
            p->lds_bytes = 8 * (resident ? dgor::skinny_resident_wave_bytes(nw.nb, nw.fringe)
                                         : dgor::skinny_wave_bytes(nw.nb, nw.fringe)) + 32;
            p->tile_bytes = (16 * K + K * N) * 4;
            p->outputs_per_thread = (16 * N + 511) / 512;
            p->vector_c = 0;
            finish(p, M, N, K);
            p->grid_x = 1;
            p->grid_y = nw.blocks;
            return GEMM_OK;
        }
        // the 128 x 128 or 64 x 64 direct-load kernel where one applies and
        // N > 64, else the register-staged tiles
        const int ci = direct == 128 && N > 64 ? 0 : direct == 64 && N > 64 ? 1
                                                    : pick_config(dgor::kF32Configs, M, N, true);
        const MfmaConfig &c = dgor::kF32Configs[ci];
        p->tile_m = c.bm;
        p->tile_n = c.bn;
        p->tile_k = c.bk;
        p->threads = 64 * c.waves_m * c.waves_n;
        int groups = 1;   // groups of wavefronts over k in one workgroup
        if (dgor::direct_lds_applies(c.bm, dgor::kF32Configs[0].bm, p->vector_a, p->vector_b, N, K)) {
            p->lds_stages = dgor::kF32DirectStages;
            p->lds_bytes = dgor::kF32DirectLdsBytes;
        } else if (dgor::f32_small_ring_applies(c.bm, c.bn, N, K, p->vector_a, p->vector_b)) {
            groups = dgor::f32_small_ring_split(M, N, K) ? 2 : 1;
            p->threads = 128 * dgor::kF32SmallWavesN * groups;
            p->tile_k = dgor::kF32SmallDepth;
            p->lds_stages = dgor::kF32SmallStages;
            p->lds_bytes = dgor::kF32SmallLdsBytes * groups;
        } else {
            p->lds_stages = 2;
            p->lds_bytes = dgor::mfma_f32_lds_bytes(c);
        }
        p->tile_bytes = (c.bm * p->tile_k + p->tile_k * c.bn) * 4;
        p->outputs_per_thread = c.bm * c.bn * groups / p->threads;
        p->vector_c = 0;
        break;
    }
    }
    finish(p, M, N, K);
    return GEMM_OK;
}

int plan_f16(int variant, int M, int N, int K, const void *A, const void *B, const void *C,
             gemm_plan *p)
{
    if (!p)
        return GEMM_ERR_NULL_PTR;
    if (M < 0 || N < 0 || K < 0)
        return GEMM_ERR_INVALID_DIM;
    if (variant == GEMM_VARIANT_AUTO)
        variant = GEMM_R7_MFMA_F16;
    if (variant != GEMM_R0_NAIVE && variant != GEMM_R7_MFMA_F16)
        return GEMM_ERR_INVALID_VARIANT;
    clear(p);
    p->variant = variant;
    p->vector_a = (K % 8 == 0) && aligned16(A);
    p->vector_b = (N % 8 == 0) && aligned16(B);
    p->vector_c = 0;
    if (M == 0 || N == 0)
        return GEMM_OK;
    if (K == 0) {
        p->launches = 1;
        p->threads = 256;
        p->vector_a = p->vector_b = 0;
        return GEMM_OK;
    }
    if (variant == GEMM_R0_NAIVE) {
        p->tile_m = p->tile_n = 16;
        p->threads = 256;
        p->outputs_per_thread = 1;
        p->vector_a = p->vector_b = 0;
    } else {
        // operands that take direct loads: the 256 x 256 ring from half a
        // tile per compute unit up, else the 128 x 128 ring (measured: 3072^3,
        // 144 tiles of 256^2, 32% of the peak against 31%; 2560^3, 100
        // tiles, 22% against 33%; the register-staged tiles 15-24% at these
        // sizes); other operands: the register-staged tiles
        const long t256 = (long)ceil_div(M, 256) * ceil_div(N, 256);
        const bool ring = t256 >= 128 && dgor::direct_lds_applies(256, 256, p->vector_a, p->vector_b, N, K);
        const bool ring128 = !ring && dgor::f16_ring128_applies(p->vector_a, p->vector_b, N, K);
        const MfmaConfig &c =
            dgor::kF16Configs[ring ? 0 : ring128 ? 1 : pick_config(dgor::kF16Configs, M, N, false)];
        p->tile_m = c.bm;
        p->tile_n = c.bn;
        p->tile_k = c.bk;
        p->threads = 64 * c.waves_m * c.waves_n;
        int groups = 1;   // groups of wavefronts over k in one workgroup
        if (dgor::direct_lds_applies(c.bm, dgor::kF16Configs[0].bm, p->vector_a, p->vector_b, N, K)) {
            p->lds_stages = dgor::kF16RingStages;
            p->lds_bytes = dgor::kF16RingLdsBytes;
        } else if (c.bm == 128 && dgor::f16_ring128_applies(p->vector_a, p->vector_b, N, K)) {
            groups = dgor::f16_ring128_split(M, N) ? 2 : 1;
            p->threads *= groups;
            p->lds_stages = dgor::kF16RingStages;
            p->lds_bytes = dgor::kF16Ring128LdsBytes * groups;
        } else {
            p->lds_stages = 2;
            p->lds_bytes = dgor::mfma_f16_lds_bytes(c);
        }
        p->tile_bytes = (c.bm * c.bk + c.bk * c.bn) * 2;
        p->outputs_per_thread = c.bm * c.bn * groups / p->threads;
    }
    finish(p, M, N, K);
    return GEMM_OK;
}

bool null_with_extent(const void *A, const void *B, const void *C, int M, int N, int K)
{
    const bool a_needed = (long)M * K > 0, b_needed = (long)K * N > 0, c_needed = (long)M * N > 0;
    return (a_needed && !A) || (b_needed && !B) || (c_needed && !C);
}

// Input format of a call: binary32, binary16 or bfloat16.
enum class In { F32, F16, BF16 };

int run(In in, int variant, int M, int N, int K, const void *A, const void *B, float *C,
        void *stream)
{
    gemm_plan plan;
    const bool half = in != In::F32;
    const int rc = half ? plan_f16(variant, M, N, K, A, B, C, &plan)
                        : plan_f32(variant, M, N, K, A, B, C, &plan);
    if (rc != GEMM_OK)
        return rc;
    if (null_with_extent(A, B, C, M, N, K))
        return GEMM_ERR_NULL_PTR;
    if (plan.launches == 0)
        return GEMM_OK;
    const int dev = check_device();
    if (dev != GEMM_OK)
        return dev;
    dgor::Problem p{M, N, K, A, B, C, plan.vector_a != 0, plan.vector_b != 0, plan.vector_c != 0};
    hipStream_t s = (hipStream_t)stream;
    hipError_t err;
    if (K == 0)
        err = dgor::launch_zero_fill(p, s);
    else if (half)
        err = plan.variant == GEMM_R7_MFMA_F16 ? dgor::launch_mfma_f16(p, plan, s, in == In::BF16)
                                               : dgor::launch_naive_f16(p, plan, s, in == In::BF16);
    else
        err = plan.variant == GEMM_R6_MFMA_F32 ? dgor::launch_mfma_f32(p, plan, s)
                                               : dgor::launch_ladder_f32(p, plan, s);
    return err == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
}

// ----------------------------------------------------------- 8-bit inputs --

// The 8-bit ring tile: 128 when the 128 x 128 ring's estimate beats the
// 256 x 256 ring's.  Both are rate x the balance of tiles over the compute
// units (tile_estimate), with measured fractions of peak.  INT8: the
// 256 x 256 ring 0.48 at one tile a unit and 0.52 with more, the 128 x 128
// ring 0.30 below two tiles a unit and 0.37 with more.  FP8: 0.57 for the
// 256 x 256 ring with several tiles a unit, and 0.55 below two, where fewer
// busy units leave power headroom that raises their clock (3072^3, 144
// tiles, runs at 0.32 against 0.31 on the 128 x 128 ring); the 128 x 128 ring
// 0.33 and 0.40.
int ring8_tile(int fmt, int M, int N)
{
    auto tiles = [&](int t) { return (long)ceil_div(M, t) * ceil_div(N, t); };
    const bool i8 = fmt == dgor::kFmtI8;
    const double e256 = tile_estimate(tiles(dgor::kRing8Tile), i8 ? 0.48 : 0.55, i8 ? 0.52 : 0.57);
    const double e128 = tile_estimate(tiles(dgor::kRing8SmallTile), i8 ? 0.30 : 0.33, i8 ? 0.37 : 0.40);
    return e128 > e256 ? dgor::kRing8SmallTile : dgor::kRing8Tile;
}

// Plan for the 8-bit entry points: R8 (the 256 x 256 x 64 ring, or the
// 128 x 128 one when ring8_tile says so) when both operands can be read with
// 16-byte loads, else R0.  INT8 caps K so that the INT32 sum
// cannot overflow.
int plan_8(int fmt, int variant, int M, int N, int K, const void *A, const void *B, gemm_plan *p)
{
    if (!p)
        return GEMM_ERR_NULL_PTR;
    if (M < 0 || N < 0 || K < 0 || (fmt == dgor::kFmtI8 && K > dgor::kI8MaxK))
        return GEMM_ERR_INVALID_DIM;
    if (variant != GEMM_VARIANT_AUTO && variant != GEMM_R0_NAIVE && variant != GEMM_R8_MFMA_8BIT)
        return GEMM_ERR_INVALID_VARIANT;
    clear(p);
    p->vector_a = (K % 16 == 0) && aligned16(A);
    p->vector_b = (N % 16 == 0) && aligned16(B);
    p->vector_c = 0;
    const bool ring = p->vector_a && p->vector_b && K < (1 << 22) && N < (1 << 22);
    p->variant = (variant != GEMM_R0_NAIVE && ring) ? GEMM_R8_MFMA_8BIT : GEMM_R0_NAIVE;
    if (M == 0 || N == 0)
        return GEMM_OK;
    if (K == 0) {
        p->launches = 1;
        p->threads = 256;
        p->vector_a = p->vector_b = 0;
        return GEMM_OK;
    }
    if (p->variant == GEMM_R0_NAIVE) {
        p->tile_m = p->tile_n = 16;
        p->threads = 256;
        p->outputs_per_thread = 1;
        p->vector_a = p->vector_b = 0;
    } else {
        const int t = ring8_tile(fmt, M, N);
        const int groups = t == dgor::kRing8SmallTile && dgor::ring8_small_split(M, N) ? 2 : 1;
        p->tile_m = p->tile_n = t;
        p->tile_k = dgor::kRing8Depth;
        p->threads = 256 * groups;
        p->lds_stages = dgor::kRing8Stages;
        p->lds_bytes = t == dgor::kRing8Tile ? dgor::kRing8LdsBytes : dgor::kRing8SmallLdsBytes * groups;
        p->tile_bytes = 2 * t * dgor::kRing8Depth;
        p->outputs_per_thread = t * t * groups / p->threads;
    }
    finish(p, M, N, K);
    return GEMM_OK;
}

int run8(int fmt, int variant, int M, int N, int K, const void *A, const void *B, void *C, void *stream)
{
    gemm_plan plan;
    const int rc = plan_8(fmt, variant, M, N, K, A, B, &plan);
    if (rc != GEMM_OK)
        return rc;
    if (null_with_extent(A, B, C, M, N, K))
        return GEMM_ERR_NULL_PTR;
    if (plan.launches == 0)
        return GEMM_OK;
    const int dev = check_device();
    if (dev != GEMM_OK)
        return dev;
    dgor::Problem p{M, N, K, A, B, (float *)C, false, false, false};
    hipStream_t s = (hipStream_t)stream;
    hipError_t err;
    if (K == 0)
        err = dgor::launch_zero_fill(p, s);   // +0.0f and integer 0 share their bits
    else if (plan.variant == GEMM_R0_NAIVE)
        err = dgor::launch_naive_8bit(p, fmt, s);
    else
        err = dgor::launch_ring8(dgor::ring_args_nn(p, plan), fmt, plan.tile_m, plan.threads / 256, s);
    return err == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
}

// ------------------------------------------------------- general layouts --

bool is_finite(float x) { return x - x == 0.f; }

// Whether the ring kernels take this call: 16-byte aligned operands, leading
// dimensions and the vector-read dimensions whole 128-bit vectors, and byte
// offsets inside a tile below 2^31.
bool ring_ok(In in, int opA, int opB, int M, int N, int K, const void *A, int lda, const void *B, int ldb,
             int ldc)
{
    const int v = in == In::F32 ? 4 : 8;               // elements per 16 bytes
    const int ld_max = in == In::F32 ? (1 << 21) : (1 << 22);
    if (!aligned16(A) || !aligned16(B) || lda % v || ldb % v || lda >= ld_max || ldb >= ld_max ||
        ldc >= (1 << 22))
        return false;
    const bool a_ok = opA ? M % v == 0 : K % v == 0;
    const bool b_ok = opB ? K % v == 0 : N % v == 0;
    return a_ok && b_ok;
}

int run_ex(In in, int opA, int opB, int M, int N, int K, float alpha, const void *A, int lda,
           const void *B, int ldb, float beta, float *C, int ldc, void *stream)
{
    if (M < 0 || N < 0 || K < 0)
        return GEMM_ERR_INVALID_DIM;
    if ((opA != GEMM_OP_N && opA != GEMM_OP_T) || (opB != GEMM_OP_N && opB != GEMM_OP_T))
        return GEMM_ERR_INVALID_LAYOUT;
    const int a_cols = opA ? M : K, b_cols = opB ? K : N;
    if (lda < (a_cols > 1 ? a_cols : 1) || ldb < (b_cols > 1 ? b_cols : 1) || ldc < (N > 1 ? N : 1))
        return GEMM_ERR_INVALID_LAYOUT;
    if (null_with_extent(A, B, C, M, N, K))
        return GEMM_ERR_NULL_PTR;
    if (M == 0 || N == 0)
        return GEMM_OK;
    // the plain row-major product takes the tuned path of gemm_* itself
    if (opA == GEMM_OP_N && opB == GEMM_OP_N && lda == K && ldb == N && ldc == N && alpha == 1.f && beta == 0.f)
        return run(in, GEMM_VARIANT_AUTO, M, N, K, A, B, C, stream);
    const int dev = check_device();
    if (dev != GEMM_OK)
        return dev;
    hipStream_t s = (hipStream_t)stream;
    auto ok = [](hipError_t e) { return e == hipSuccess; };
    if (K == 0 || alpha == 0.f)   // C = beta C (zeros when beta == 0, C not read)
        return ok(dgor::launch_scale_c(C, M, N, ldc, beta, s)) ? GEMM_OK : GEMM_ERR_LAUNCH;

    dgor::RingArgs a{M, N, K, A, lda, B, ldb, C, ldc, (M + 255) / 256, (N + 255) / 256, 4,
                     opA == GEMM_OP_T, opB == GEMM_OP_T, false};
    const int in16 = in == In::F32 ? 0 : (in == In::F16 ? 1 : 2);
    // C = alpha A B + beta C from the ring kernels' two forms, C = alpha A B
    // and C = alpha (C + A B), the second after a pass C *= beta / alpha
    // when beta != alpha (beta itself when alpha == 1, so the common cases
    // alpha == 1 with beta in {0, 1} take one kernel and no pass).
    const float ratio = beta == 0.f ? 0.f : (alpha == 1.f ? beta : beta / alpha);
    const bool ratio_ok = beta == 0.f || alpha == 1.f ||
                          (is_finite(ratio) && fabsf(ratio) >= 0x1p-60f && fabsf(ratio) <= 0x1p60f);
    if (!ring_ok(in, opA, opB, M, N, K, A, lda, B, ldb, ldc) || !ratio_ok)
        return ok(dgor::launch_naive_ex(a, alpha, beta, in16, s)) ? GEMM_OK : GEMM_ERR_LAUNCH;
    auto ring = [&]() { return in == In::F32 ? dgor::launch_ring32(a, s) : dgor::launch_ring16(a, s, in == In::BF16); };
    a.alpha = alpha;   // applied by the ring kernel as it stores C
    if (beta != 0.f) {
        if (ratio != 1.f && !ok(dgor::launch_scale_c(C, M, N, ldc, ratio, s)))
            return GEMM_ERR_LAUNCH;
        a.accumulate = true;
    }
    return ok(ring()) ? GEMM_OK : GEMM_ERR_LAUNCH;
}

// ------------------------------------------------------------ convolution --

constexpr size_t kWsAlign = 256;

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Shape checks and the workspace layout of a convolution: padded weights,
// im2col matrix, FP32 GEMM result, each starting on a 256-byte boundary.
struct ConvPlan {
    dgor::Conv2d cv;
    int algorithm;    // gemm_conv_algorithm
    dgor::NhwcPlan nhwc;
    int crsp, npqp;
    bool ring;        // the GEMM runs on the 256 x 256 ring kernels, split over k
    int splits, k_chunk;
    size_t off_col, off_y, split_stride, bytes;
};

int conv_plan(const gemm_conv2d_params *pr, int elem_bytes, ConvPlan &cp)
{
    if (!pr)
        return GEMM_ERR_NULL_PTR;
    const gemm_conv2d_params &q = *pr;
    if (q.N < 0 || q.C < 0 || q.H < 0 || q.W < 0 || q.K < 0 || q.R < 1 || q.S < 1 || q.stride_h < 1 ||
        q.stride_w < 1 || q.pad_h < 0 || q.pad_w < 0 || q.dilation_h < 1 || q.dilation_w < 1 ||
        (elem_bytes != 4 && elem_bytes != 2))
        return GEMM_ERR_INVALID_DIM;
    const long long span_h = (long long)q.H + 2LL * q.pad_h - (long long)q.dilation_h * (q.R - 1) - 1;
    const long long span_w = (long long)q.W + 2LL * q.pad_w - (long long)q.dilation_w * (q.S - 1) - 1;
    if (span_h < 0 || span_w < 0 || span_h > INT32_MAX || span_w > INT32_MAX)
        return GEMM_ERR_INVALID_DIM;
    const long long P = span_h / q.stride_h + 1, Q = span_w / q.stride_w + 1;
    const long long crs = (long long)q.C * q.R * q.S, npq = (long long)q.N * P * Q;
    const long long crsp = (crs + 7) / 8 * 8, npqp = (npq + 7) / 8 * 8;
    if (crsp > INT32_MAX || npqp > INT32_MAX || (long long)q.K * npqp > (1LL << 40) ||
        crsp * npqp > (1LL << 40) || (long long)q.N * q.C * q.H * q.W > (1LL << 40))
        return GEMM_ERR_INVALID_DIM;
    cp.cv = dgor::Conv2d{q.N, q.C, q.H, q.W, q.K, q.R, q.S, q.stride_h, q.stride_w, q.pad_h, q.pad_w,
                         q.dilation_h, q.dilation_w, (int)P, (int)Q};
    cp.crsp = (int)crsp;
    cp.npqp = (int)npqp;
    // The GEMM (K x CRSp by CRSp x NPQp) runs on the 256 x 256 ring kernels
    // when at least 192 filters fill most of a tile's 256 rows and the
    // reduction is at least one 64-deep chunk, split over k until tiles x
    // splits covers the 256 CUs (chunks of at least 64, multiples of 64); the
    // partial results are summed by the output pass.  Otherwise the planner's
    // tiles take it whole.
    cp.ring = q.K >= 192 && crsp >= 64 && npqp < (1 << 21) && crsp < (1 << 21);
    cp.splits = 1;
    cp.k_chunk = (int)crsp;
    if (cp.ring) {
        const long long tiles = ((q.K + 255) / 256) * ((npqp + 255) / 256);
        long long want = (256 + tiles - 1) / tiles;
        want = want < crsp / 64 ? want : crsp / 64;
        want = want > 1 ? want : 1;
        const long long chunk = ((crsp + want - 1) / want + 63) / 64 * 64;
        cp.k_chunk = (int)chunk;
        cp.splits = (int)((crsp + chunk - 1) / chunk);
    }
    cp.split_stride = round_up((size_t)q.K * (size_t)npqp * 4, kWsAlign) / 4;
    if (dgor::conv_nhwc_plan(cp.cv, elem_bytes, cp.nhwc)) {
        // channels-last implicit GEMM: Wr, then the channels-last copy of x
        cp.algorithm = GEMM_CONV_IMPLICIT_NHWC;
        cp.off_col = round_up(cp.nhwc.wr_bytes, kWsAlign);
        cp.off_y = cp.off_col + round_up(cp.nhwc.xp_bytes, kWsAlign);
        cp.bytes = cp.off_y;
        return GEMM_OK;
    }
    cp.off_col = round_up((size_t)q.K * (size_t)crsp * elem_bytes, kWsAlign);
    if (dgor::conv_igemm_applies(cp.cv, elem_bytes)) {
        // implicit GEMM with a gather: the padded weights, then (vector
        // gather only) the zero-padded copy of x; no im2col matrix and no
        // GEMM result
        cp.algorithm = GEMM_CONV_IMPLICIT;
        const size_t xp_bytes = dgor::conv_igemm_vec_applies(cp.cv, elem_bytes)
                                    ? ((size_t)dgor::conv_padded_input_elems(cp.cv) + 8) * 2 : 0;
        cp.off_y = cp.off_col + round_up(xp_bytes, kWsAlign);
        cp.bytes = cp.off_y;
        return GEMM_OK;
    }
    // im2col: the padded weights, the im2col matrix, the GEMM result(s)
    cp.algorithm = GEMM_CONV_IM2COL;
    cp.off_y = cp.off_col + round_up((size_t)crsp * (size_t)npqp * elem_bytes, kWsAlign);
    cp.bytes = cp.off_y + (size_t)cp.splits * cp.split_stride * 4;
    return GEMM_OK;
}

// GEMM_ERR_NULL_PTR for a NULL tensor of nonzero extent; *empty when y has
// no elements (nothing to launch).
int conv_pointers(const ConvPlan &cp, const void *x, const void *w, const float *y, bool &empty)
{
    const dgor::Conv2d &cv = cp.cv;
    const long long xs = (long long)cv.N * cv.C * cv.H * cv.W, wsz = (long long)cv.K * cv.C * cv.R * cv.S;
    const long long ys = (long long)cv.N * cv.K * cv.P * cv.Q;
    empty = ys == 0;
    return (xs > 0 && !x) || (wsz > 0 && !w) || (ys > 0 && !y) ? GEMM_ERR_NULL_PTR : GEMM_OK;
}

int run_conv(In in, const gemm_conv2d_params *pr, const void *x, const void *w, float *y, void *ws,
             size_t ws_bytes, void *stream)
{
    ConvPlan cp;
    const int eb = in == In::F32 ? 4 : 2;
    const int rc = conv_plan(pr, eb, cp);
    if (rc != GEMM_OK)
        return rc;
    const dgor::Conv2d &cv = cp.cv;
    bool empty = false;
    const int pc = conv_pointers(cp, x, w, y, empty);
    if (pc != GEMM_OK || empty)
        return pc;
    if (!ws || ws_bytes < cp.bytes || ((uintptr_t)ws & (kWsAlign - 1)))
        return GEMM_ERR_WORKSPACE;
    const int dev = check_device();
    if (dev != GEMM_OK)
        return dev;
    hipStream_t s = (hipStream_t)stream;
    uint8_t *base = (uint8_t *)ws;
    void *col = base + cp.off_col;
    float *yp = (float *)(base + cp.off_y);
    // W (K x CRS) is already the GEMM's K x CRSp operand when CRS is a
    // multiple of 8 and W is 16-byte aligned: no padded copy then
    if (cp.algorithm == GEMM_CONV_IMPLICIT_NHWC)
        return dgor::launch_conv_nhwc(cv, cp.nhwc, in == In::BF16, x, w, y, col, base, s) == hipSuccess
                   ? GEMM_OK : GEMM_ERR_LAUNCH;
    const bool w_direct = cp.crsp == cv.C * cv.R * cv.S && aligned16(w);
    const void *wp = w_direct ? w : base;
    if (cp.algorithm == GEMM_CONV_IMPLICIT) {   // 16-bit, enough tiles: no im2col matrix
        if (!w_direct &&
            dgor::launch_conv_prepare(cv, eb, x, w, base, nullptr, cp.crsp, cp.npqp, s) != hipSuccess)
            return GEMM_ERR_LAUNCH;
        return dgor::launch_conv_igemm(cv, in == In::BF16, x, wp, y, cp.crsp, col, s) == hipSuccess
                   ? GEMM_OK : GEMM_ERR_LAUNCH;
    }
    if (dgor::launch_conv_prepare(cv, eb, x, w, w_direct ? nullptr : base, col, cp.crsp, cp.npqp, s) !=
        hipSuccess)
        return GEMM_ERR_LAUNCH;
    // the GEMM: K x CRSp by CRSp x NPQp
    if (cp.ring) {
        dgor::RingArgs a{cv.K, cp.npqp, cp.crsp, wp, cp.crsp, col, cp.npqp, yp, cp.npqp,
                         (cv.K + 255) / 256, (cp.npqp + 255) / 256, 4, false, false, false};
        a.splits = cp.splits;
        a.k_chunk = cp.k_chunk;
        a.c_split_stride = cp.split_stride;
        const hipError_t e = in == In::F32 ? dgor::launch_ring32(a, s) : dgor::launch_ring16(a, s, in == In::BF16);
        if (e != hipSuccess)
            return GEMM_ERR_LAUNCH;
    } else {
        const int g = run(in, GEMM_VARIANT_AUTO, cv.K, cp.npqp, cp.crsp, wp, col, yp, stream);
        if (g != GEMM_OK)
            return g;
    }
    return dgor::launch_conv_output(cv, yp, y, cp.npqp, cp.splits, cp.split_stride, s) == hipSuccess
               ? GEMM_OK : GEMM_ERR_LAUNCH;
}

}  // namespace

// Scratch of the no-allocation convolution entry point: a fixed array in
// the code object, so each GPU the library runs on holds its own copy from
// the module's load until the process ends.  Host code never passes the
// array's name to a kernel (on the host it only stands for the symbol): it
// uses the device address hipGetSymbolAddress reports, looked up once per
// device with that device current.
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

std::once_flag g_scratch_once[kDevCache];
void *g_scratch_ptr[kDevCache];
hipError_t g_scratch_err[kDevCache];

// The current device's scratch address in *ptr, or GEMM_ERR_RUNTIME.
int device_scratch(void **ptr)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDevCache)
        return GEMM_ERR_RUNTIME;
    std::call_once(g_scratch_once[dev], [dev] {
        void *p = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = p;
    });
    if (g_scratch_err[dev] != hipSuccess || g_scratch_ptr[dev] == nullptr)
        return GEMM_ERR_RUNTIME;
    *ptr = g_scratch_ptr[dev];
    return GEMM_OK;
}

}  // namespace

extern "C" {

int gemm_f32(int M, int N, int K, const float *A, const float *B, float *C, void *stream)
{
    return run(In::F32, GEMM_VARIANT_AUTO, M, N, K, A, B, C, stream);
}

int gemm_f16_f32acc(int M, int N, int K, const uint16_t *A, const uint16_t *B, float *C,
                    void *stream)
{
    return run(In::F16, GEMM_VARIANT_AUTO, M, N, K, A, B, C, stream);
}

int gemm_bf16_f32acc(int M, int N, int K, const uint16_t *A, const uint16_t *B, float *C,
                     void *stream)
{
    return run(In::BF16, GEMM_VARIANT_AUTO, M, N, K, A, B, C, stream);
}

int gemm_f32_variant(int variant, int M, int N, int K, const float *A, const float *B,
                     float *C, void *stream)
{
    return run(In::F32, variant, M, N, K, A, B, C, stream);
}

int gemm_f16_f32acc_variant(int variant, int M, int N, int K, const uint16_t *A,
                            const uint16_t *B, float *C, void *stream)
{
    return run(In::F16, variant, M, N, K, A, B, C, stream);
}

int gemm_bf16_f32acc_variant(int variant, int M, int N, int K, const uint16_t *A,
                             const uint16_t *B, float *C, void *stream)
{
    return run(In::BF16, variant, M, N, K, A, B, C, stream);
}

int gemm_f32_plan(int variant, int M, int N, int K, const float *A, const float *B,
                  const float *C, gemm_plan *plan)
{
    return plan_f32(variant, M, N, K, A, B, C, plan);
}

int gemm_f16_f32acc_plan(int variant, int M, int N, int K, const uint16_t *A,
                         const uint16_t *B, const float *C, gemm_plan *plan)
{
    return plan_f16(variant, M, N, K, A, B, C, plan);
}

int gemm_bf16_f32acc_plan(int variant, int M, int N, int K, const uint16_t *A,
                          const uint16_t *B, const float *C, gemm_plan *plan)
{
    return plan_f16(variant, M, N, K, A, B, C, plan);
}

int gemm_e4m3_f32acc(int M, int N, int K, const uint8_t *A, const uint8_t *B, float *C, void *stream)
{
    return run8(dgor::kFmtE4M3, GEMM_VARIANT_AUTO, M, N, K, A, B, C, stream);
}

int gemm_e5m2_f32acc(int M, int N, int K, const uint8_t *A, const uint8_t *B, float *C, void *stream)
{
    return run8(dgor::kFmtE5M2, GEMM_VARIANT_AUTO, M, N, K, A, B, C, stream);
}

int gemm_i8_i32acc(int M, int N, int K, const int8_t *A, const int8_t *B, int32_t *C, void *stream)
{
    return run8(dgor::kFmtI8, GEMM_VARIANT_AUTO, M, N, K, A, B, C, stream);
}

int gemm_e4m3_f32acc_variant(int variant, int M, int N, int K, const uint8_t *A, const uint8_t *B, float *C,
                             void *stream)
{
    return run8(dgor::kFmtE4M3, variant, M, N, K, A, B, C, stream);
}

int gemm_e5m2_f32acc_variant(int variant, int M, int N, int K, const uint8_t *A, const uint8_t *B, float *C,
                             void *stream)
{
    return run8(dgor::kFmtE5M2, variant, M, N, K, A, B, C, stream);
}

int gemm_i8_i32acc_variant(int variant, int M, int N, int K, const int8_t *A, const int8_t *B, int32_t *C,
                           void *stream)
{
    return run8(dgor::kFmtI8, variant, M, N, K, A, B, C, stream);
}

int gemm_e4m3_f32acc_plan(int variant, int M, int N, int K, const uint8_t *A, const uint8_t *B, const float *C,
                          gemm_plan *plan)
{
    (void)C;
    return plan_8(dgor::kFmtE4M3, variant, M, N, K, A, B, plan);
}

int gemm_e5m2_f32acc_plan(int variant, int M, int N, int K, const uint8_t *A, const uint8_t *B, const float *C,
                          gemm_plan *plan)
{
    (void)C;
    return plan_8(dgor::kFmtE5M2, variant, M, N, K, A, B, plan);
}

int gemm_i8_i32acc_plan(int variant, int M, int N, int K, const int8_t *A, const int8_t *B, const int32_t *C,
                        gemm_plan *plan)
{
    (void)C;
    return plan_8(dgor::kFmtI8, variant, M, N, K, A, B, plan);
}

int gemm_conv2d_workspace(const gemm_conv2d_params *params, int input_bytes, size_t *bytes)
{
    if (!bytes)
        return GEMM_ERR_NULL_PTR;
    ConvPlan cp;
    const int rc = conv_plan(params, input_bytes, cp);
    if (rc == GEMM_OK)
        *bytes = cp.bytes;
    return rc;
}

int gemm_conv2d_algorithm(const gemm_conv2d_params *params, int input_bytes, int *algorithm)
{
    if (!algorithm)
        return GEMM_ERR_NULL_PTR;
    ConvPlan cp;
    const int rc = conv_plan(params, input_bytes, cp);
    if (rc == GEMM_OK)
        *algorithm = cp.algorithm;
    return rc;
}

int gemm_conv2d_f32(const gemm_conv2d_params *params, const float *x, const float *w, float *y, void *workspace,
                    size_t workspace_bytes, void *stream)
{
    return run_conv(In::F32, params, x, w, y, workspace, workspace_bytes, stream);
}

int gemm_conv2d_f16_f32acc(const gemm_conv2d_params *params, const uint16_t *x, const uint16_t *w, float *y,
                           void *workspace, size_t workspace_bytes, void *stream)
{
    return run_conv(In::F16, params, x, w, y, workspace, workspace_bytes, stream);
}

int gemm_conv2d_bf16_f32acc(const gemm_conv2d_params *params, const uint16_t *x, const uint16_t *w, float *y,
                            void *workspace, size_t workspace_bytes, void *stream)
{
    return run_conv(In::BF16, params, x, w, y, workspace, workspace_bytes, stream);
}

int gemm_conv2d_f16_f32acc_noalloc(const gemm_conv2d_params *params, const uint16_t *x, const uint16_t *w, float *y,
                                   void *stream)
{
    ConvPlan cp;
    const int rc = conv_plan(params, 2, cp);
    if (rc != GEMM_OK)
        return rc;
    bool empty = false;
    const int pc = conv_pointers(cp, x, w, y, empty);
    if (pc != GEMM_OK || empty)
        return pc;
    if (cp.bytes > kNoAllocScratchBytes)
        return GEMM_ERR_SCRATCH_LIMIT;
    void *ws = nullptr;
    const int sc = device_scratch(&ws);
    if (sc != GEMM_OK)
        return sc;
    return run_conv(In::F16, params, x, w, y, ws, kNoAllocScratchBytes, stream);
}

int gemm_f32_ex(int opA, int opB, int M, int N, int K, float alpha, const float *A, int lda, const float *B,
                int ldb, float beta, float *C, int ldc, void *stream)
{
    return run_ex(In::F32, opA, opB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream);
}

int gemm_f16_f32acc_ex(int opA, int opB, int M, int N, int K, float alpha, const uint16_t *A, int lda,
                       const uint16_t *B, int ldb, float beta, float *C, int ldc, void *stream)
{
    return run_ex(In::F16, opA, opB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream);
}

int gemm_bf16_f32acc_ex(int opA, int opB, int M, int N, int K, float alpha, const uint16_t *A, int lda,
                        const uint16_t *B, int ldb, float beta, float *C, int ldc, void *stream)
{
    return run_ex(In::BF16, opA, opB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream);
}

const char *gemm_status_string(int status)
{
    switch (status) {
    case GEMM_OK: return "ok";
    case GEMM_ERR_INVALID_DIM: return "invalid dimension (M, N or K negative)";
    case GEMM_ERR_NULL_PTR: return "null pointer for an operand with nonzero extent";
    case GEMM_ERR_LAUNCH: return "kernel launch failed";
    case GEMM_ERR_UNSUPPORTED_DEVICE: return "current device is not gfx950";
    case GEMM_ERR_INVALID_VARIANT: return "variant not available for this entry point";
    case GEMM_ERR_RUNTIME: return "HIP runtime query failed";
    case GEMM_ERR_INVALID_LAYOUT: return "invalid operand layout (op flag or leading dimension)";
    case GEMM_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case GEMM_ERR_SCRATCH_LIMIT: return "needs more scratch than the no-allocation entry point's fixed array (16 MiB)";
    default: return "unknown status";
    }
}

const char *gemm_variant_name(int variant)
{
    switch (variant) {
    case GEMM_VARIANT_AUTO: return "auto";
    case GEMM_R0_NAIVE: return "R0 naive";
    case GEMM_R1_LDS_TILED: return "R1 LDS 16x16 tiles";
    case GEMM_R2_VECTOR_LOADS: return "R2 128-bit loads";
    case GEMM_R3_LDS_PADDED: return "R3 padded LDS";
    case GEMM_R4_DOUBLE_BUFFER: return "R4 double-buffered LDS";
    case GEMM_R5_REGISTER_BLOCKED: return "R5 register-blocked 8x8";
    case GEMM_R6_MFMA_F32: return "R6 FP32 MFMA";
    case GEMM_R7_MFMA_F16: return "R7 16-bit MFMA, FP32 accumulate";
    case GEMM_R8_MFMA_8BIT: return "R8 8-bit MFMA (FP8: FP32, INT8: INT32 accumulate)";
    default: return "unknown variant";
    }
}

}  // extern "C"
