// Implicit-GEMM convolution on a channels-last copy of x, for 16-bit inputs
// with C a multiple of 32 ("Lesson 8: how a GPU does matrix multiply" names
// convolution as matrix multiplication as its next lesson).
//
// Reorder the reduction over (c, r, s) as (r, s, c), c fastest.  Then
//     y[n][k][p][q] = sum over r, s, c of Wr[k][(r S + s) C + c] xp[n][p sh + r dh][q sw + s dw][c]
// where Wr[k][r][s][c] = w[k][c][r][s] and xp is x channels-last with its zero
// border made explicit: N x Hp x Wp x C, Hp = H + 2 ph, Wp = W + 2 pw.  It is
// the GEMM Y(K x NPQ) = Wr(K x RSC) B(RSC x NPQ) whose column j (pixel n, p, q)
// of B holds, for each tap (r, s), C contiguous values of xp.  So a 32-deep
// k-step of one tap is 64 contiguous bytes of Wr per filter and 64 contiguous
// bytes of xp per pixel: both operand tiles load straight from global memory
// into LDS by the direct loads of the GEMM ring kernels, 16 bytes a lane, and
// no im2col matrix is ever written.  Every product is exact and the sums are
// FP32, as in the GEMM; only their order differs from the direct loop.
//
// Two kernels:
//   nhwc_prepare: xp from x through LDS-tiled transposes (a block per
//     image, run of rows and 64 or 32 channels, or per 64 pixels of xp when
//     W is odd or x not 4-byte aligned), and Wr from w (a block per filter
//     and channel block);
//   conv_nhwc_kernel<BF16, BM, BN, BK, WGM, NST, NW>: BM filters x BN
//     pixels per workgroup, BK-deep stages (a multiple of 32 within one tap:
//     C % BK == 0) in a ring of NST LDS buffers, NW wavefronts in a
//     WGM x (NW / WGM) grid, each a grid of 16 x 16 blocks of
//     v_mfma_f32_16x16x32_f16 (or _bf16) with FP32 accumulators; results
//     straight to y (NKPQ).
//
// What bounds it on gfx950: its operand loads.  A tile this small (set by
// K and the layer's pixel count) needs more bytes per product than the
// GEMM's 256 x 256 tiles, and each XCD's L2 starts every launch cold, so
// the filters and the x rows are first fetched from the memory-side cache
// by every XCD in lockstep; with the loads a CU can keep in flight, that
// latency, not the matrix cores, sets the rate.
#include <type_traits>

#include "common.h"
#include "lds_dma.h"

namespace dgor {
namespace {

typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr uint32_t OOB = 0x80000000u;
constexpr int kNhwcMaxRS = 64;   // filter taps the weight reorder stages in LDS

template <bool BF16>
__device__ __forceinline__ floatx4 nhwc_mma(halfx8 a, halfx8 b, floatx4 c)
{
    if constexpr (BF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                       0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Blocks [0, xp_blocks) write xp, in one of two ways.
//   rows (W even and at most 64, x 4-byte aligned): a block per image n,
//     run of RH = 64 / W image rows h0 .. h0 + RH - 1 and CH channels (64
//     when C allows, else 32).  Each channel's RH W values are one
//     contiguous run of x, read 16 bytes a lane (a compute unit issues
//     memory instructions at a fixed rate whatever their width, so 2-byte
//     loads cost eight times the issue of these) into a row of the LDS tile.
//     The block then writes the xp rows of its image rows, border columns
//     included, and the first and last blocks of an image also the border
//     rows.
//   pixels: a block per 64 consecutive pixels of xp (n, hp, wp flattened),
//     each channel's 64 pixels read one value a lane (zeros in the border).
// Either way the tile is written channels-last, 16 bytes (8 channels of
// one pixel) a thread, CH channels of a pixel contiguous.  Blocks past
// that: filter k and CH channels of w: the CH R S contiguous values are read
// into LDS and written as R S runs of CH channels of Wr.  R S is at most 64.
// Tile rows: 64 values (a run of RH W <= 64, its last 16-byte unit
// included) padded to 66 against bank conflicts.
constexpr int kPrepPix = 64, kPrepRow = 66;

struct PrepRows { int rh, groups; };          // rows mode: image rows per block, blocks per image
inline PrepRows prep_rows(const Conv2d &cv)
{
    PrepRows r;
    r.rh = cv.W <= 64 ? min(64 / cv.W, cv.H) : 1;
    r.groups = (cv.H + r.rh - 1) / r.rh;
    return r;
}
inline bool prep_rows_apply(const Conv2d &cv, const void *x)
{
    return cv.W % 2 == 0 && cv.W <= 64 && ((uintptr_t)x & 3) == 0;
}

__global__ __launch_bounds__(256) void nhwc_prepare(const uint16_t *__restrict__ x, const uint16_t *__restrict__ w,
                                                    uint16_t *__restrict__ xp, uint16_t *__restrict__ wr, Conv2d cv,
                                                    int Hp, int Wp, int ch, int xp_blocks, PrepRows pr, int rows_mode)
{
    __shared__ __attribute__((aligned(16))) uint16_t tile[64 * kPrepRow];
    const int tid = threadIdx.x, cblocks = cv.C / ch, units = ch / 8;
    if ((int)blockIdx.x < xp_blocks && rows_mode) {
        const int cb = blockIdx.x % cblocks, t = blockIdx.x / cblocks;
        const int g = t % pr.groups, n = t / pr.groups;
        const int h0 = g * pr.rh, rows = min(pr.rh, cv.H - h0), run = rows * cv.W, nu = (run + 7) / 8;
        const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, (long long)cv.N * cv.C * cv.H * cv.W * 2);
        const size_t plane = (size_t)cv.H * cv.W;
        const size_t first = ((size_t)n * cv.C + (size_t)cb * ch) * plane + (size_t)h0 * cv.W;
        for (int e = tid; e < ch * nu; e += 256) {
            const int c = e / nu, u = e - c * nu;
            // a unit past the run brings the next values of x (or zeros past
            // its end): they land past the run in the tile row, never read
            const uint4 v = __builtin_bit_cast(
                uint4, __builtin_amdgcn_raw_buffer_load_b128(
                           rx, (uint32_t)((first + (size_t)c * plane + 8 * u) * 2), 0, 0));
            uint32_t *dst = reinterpret_cast<uint32_t *>(tile + c * kPrepRow + 8 * u);
            dst[0] = v.x;
            dst[1] = v.y;
            dst[2] = v.z;
            dst[3] = v.w;
        }
        __syncthreads();
        // xp rows: this block's image rows, and the border rows above the
        // first and below the last
        const int hp_lo = g == 0 ? 0 : h0 + cv.ph;
        const int hp_hi = g == pr.groups - 1 ? Hp : h0 + cv.ph + rows;
        const int count = (hp_hi - hp_lo) * Wp * units;
        for (int e = tid; e < count; e += 256) {
            const int u = e % units, t2 = e / units, wp = t2 % Wp, hp = hp_lo + t2 / Wp;
            const int h = hp - cv.ph - h0, wc = wp - cv.pw;
            uint32_t v[4] = {0u, 0u, 0u, 0u};
            if ((unsigned)h < (unsigned)rows && (unsigned)wc < (unsigned)cv.W) {
                const int px = h * cv.W + wc;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    v[i] = (uint32_t)tile[(8 * u + 2 * i) * kPrepRow + px] |
                           ((uint32_t)tile[(8 * u + 2 * i + 1) * kPrepRow + px] << 16);
            }
            *reinterpret_cast<uint4 *>(xp + (((size_t)n * Hp + hp) * Wp + wp) * cv.C + cb * ch + 8 * u) =
                make_uint4(v[0], v[1], v[2], v[3]);
        }
        return;
    }
    if ((int)blockIdx.x < xp_blocks) {
        const int cb = blockIdx.x % cblocks;
        const long long pix0 = (long long)(blockIdx.x / cblocks) * kPrepPix;
        const long long npix = (long long)cv.N * Hp * Wp;
        {
            const int px = tid & 63;
            const long long pix = pix0 + px;
            const int n = (int)(pix / (Hp * Wp)), rem = (int)(pix - (long long)n * Hp * Wp);
            const int h = rem / Wp - cv.ph, wc = rem % Wp - cv.pw;
            const bool v = pix < npix && (unsigned)h < (unsigned)cv.H && (unsigned)wc < (unsigned)cv.W;
            const size_t plane = (size_t)cv.H * cv.W;
            const uint16_t *src = x + ((size_t)n * cv.C + (size_t)cb * ch) * plane + (size_t)h * cv.W + wc;
            for (int c = tid >> 6; c < ch; c += 4)
                tile[c * kPrepRow + px] = v ? src[(size_t)c * plane] : (uint16_t)0;
        }
        __syncthreads();
        for (int e = tid; e < kPrepPix * units; e += 256) {
            const int px = e / units, u = e - px * units;
            if (pix0 + px >= npix)
                break;
            uint32_t v[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                v[i] = (uint32_t)tile[(8 * u + 2 * i) * kPrepRow + px] |
                       ((uint32_t)tile[(8 * u + 2 * i + 1) * kPrepRow + px] << 16);
            *reinterpret_cast<uint4 *>(xp + (size_t)(pix0 + px) * cv.C + cb * ch + 8 * u) =
                make_uint4(v[0], v[1], v[2], v[3]);
        }
        return;
    }
    // Wr[k][r][s][c] = w[k][c][r][s]
    const int b = blockIdx.x - xp_blocks, k = b / cblocks, cb = b - k * cblocks;
    const int RS = cv.R * cv.S;
    const uint16_t *src = w + ((size_t)k * cv.C + (size_t)cb * ch) * RS;
    for (int e = tid; e < ch * RS; e += 256)
        tile[e] = src[e];
    __syncthreads();
    for (int e = tid; e < RS * units; e += 256) {
        const int rs = e / units, u = e - rs * units;
        uint32_t v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            v[i] = (uint32_t)tile[(8 * u + 2 * i) * RS + rs] | ((uint32_t)tile[(8 * u + 2 * i + 1) * RS + rs] << 16);
        *reinterpret_cast<uint4 *>(wr + ((size_t)k * RS + rs) * cv.C + cb * ch + 8 * u) =
            make_uint4(v[0], v[1], v[2], v[3]);
    }
}

// LDS rows hold the BK values of one filter or pixel: U = BK / 8 units of 16
// bytes.  Unit c of row r sits at physical unit c ^ swz(r), the swizzles of
// the GEMM ring kernels' A tiles for 64- and 128-byte rows, under which the
// 16 lanes of a 128-bit fragment read cycle fall on distinct banks.
template <int U>
__device__ __forceinline__ int nhwc_swz(int r)
{
    return U == 4 ? 2 * ((r >> 2) & 1) : ((r >> 1) & 7);
}

// One workgroup: filters m0..m0+BM, pixels j0..j0+BN, all of R S C in
// BK-deep stages t (tap t BK / C, channels (t BK) % C ..), in a ring of NST
// LDS buffers.  Stage t sits in buffer t % NST: its loads are issued during
// stage t - NST + 1 (the prologue issues stages 0..NST - 2), after the
// barrier opening that stage, which has retired every read of the buffer's
// previous stage t - NST (each wavefront waits for its own LDS reads before
// it).  Stage t opens with a wait for all but this wavefront's loads
// of stages t + 2 .. t + NST - 2, so stages t and t + 1 have landed, and a
// barrier; during stage t the wavefront reads the fragments of its next
// 32-deep step (of stage t, or the first of stage t + 1), one after each of
// its first MFMAs.  Stages past the last load from an empty range (zeros), so
// every stage waits for the same count; no load is in flight when the
// workgroup ends.  The NW wavefronts (4 or 8: with 8, two share each SIMD,
// so one issues MFMAs while the other waits for its loads to be accepted)
// form a WGM x (NW / WGM) grid over the tile.
template <bool BF16, int BM, int BN, int BK, int WGM, int NST, int NW>
__global__ __launch_bounds__(64 * NW) void conv_nhwc_kernel(const uint16_t *__restrict__ xp, const uint16_t *__restrict__ wr,
                                                        float *__restrict__ y, Conv2d cv, int Hp, int Wp, int tiles_m,
                                                        int tiles_n)
{
    constexpr int U = BK / 8, ROWB = 2 * BK, SUB = BK / 32;
    constexpr int A_BYTES = BM * ROWB, B_BYTES = BN * ROWB, STAGE = A_BYTES + B_BYTES;
    constexpr int A_CHUNKS = A_BYTES / 1024, B_CHUNKS = B_BYTES / 1024, LW = (A_CHUNKS + B_CHUNKS) / NW;
    constexpr int ROWS_PER_CHUNK = 64 / U;
    constexpr int WGN = NW / WGM, WTM = BM / WGM, WTN = BN / WGN;   // a wavefront's WTM x WTN
    constexpr int FM = WTM / 16, FN = WTN / 16;                       // in 16 x 16 blocks
    static_assert(A_CHUNKS % NW == 0 && B_CHUNKS % NW == 0 && A_CHUNKS * 1024 == A_BYTES &&
                      B_CHUNKS * 1024 == B_BYTES,
                  "whole 1 KB chunks, the same number for every wavefront");
    static_assert(WGM * WGN == NW && FM >= 1 && FN >= 1 && FM * 16 == WTM && FN * 16 == WTN, "wavefront grid");
    static_assert(NST >= 3 && NST * STAGE <= 163840 && (NST - 1) * LW <= 63, "ring depth");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[NST * STAGE];
    const uint32_t lbase = lds_address(lds);

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    // each XCD takes a contiguous run of pixel tiles (all filter tiles of
    // each), so the x rows a tile shares with its neighbours and the
    // filters stay in that XCD's L2
    int tm, tn;
    dgor_tile_of_block((int)blockIdx.x, tiles_m, tiles_n, tiles_m, tm, tn);
    const int m0 = tm * BM, j0 = tn * BN;
    const int RSC = cv.R * cv.S * cv.C, PQ = cv.P * cv.Q, npq = cv.N * PQ;
    const int steps = RSC / BK;
    const long long xp_bytes = (long long)cv.N * Hp * Wp * cv.C * 2;

    // ---- this wavefront's loads of a stage: slots l < LA take A chunk
    // wave + NW l, the rest B chunk wave + NW (l - LA), so every slot's operand
    // is a compile-time choice.  Lane p fills slot p of its chunk: row p / U
    // of the chunk, physical unit p % U, logical unit c = physical ^ swz(row).
    // Offsets in bytes, fixed for the whole k-range (a stage moves the
    // descriptors' bases); rows past K or NPQ take an out-of-range offset.
    constexpr int LA = A_CHUNKS / NW;
    uint32_t off[LW];
#pragma unroll
    for (int l = 0; l < LW; ++l) {
        const bool is_a = l < LA;
        const int chunk = wave + NW * (is_a ? l : l - LA);
        const int r = chunk * ROWS_PER_CHUNK + lane / U;
        const int c = (lane % U) ^ nhwc_swz<U>(r);
        if (is_a) {
            off[l] = m0 + r < cv.K ? (uint32_t)((m0 + r) * RSC + 8 * c) * 2u : OOB;
        } else {
            const int j = j0 + r;
            if (j < npq) {
                const int n = j / PQ, pq = j - n * PQ, p = pq / cv.Q, q = pq - p * cv.Q;
                off[l] = (uint32_t)((((n * Hp + p * cv.sh) * Wp + q * cv.sw) * cv.C) + 8 * c) * 2u;
            } else {
                off[l] = OOB;
            }
        }
    }
    // The descriptors of one stage's loads, in scalar code once per stage:
    // A along Wr's rows by st BK; B at the stage's tap (r, s) and channel c0,
    // stepped from the previous stage (no division); past the last stage
    // both ranges are empty, so the loads write zeros.
    struct Loads { intx4 ra, rb; uint32_t dst; };
    int ld_st = 0, ld_c0 = 0, ld_r = 0, ld_s = 0;
    auto next_loads = [&]() __attribute__((always_inline)) {
        Loads L;
        const bool live = ld_st < steps;
        L.ra = rsrc_words(wr + (size_t)ld_st * BK, live ? (long long)cv.K * RSC * 2 - (long long)ld_st * BK * 2 : 0);
        const long long toff = (long long)(ld_r * cv.dh * Wp + ld_s * cv.dw) * cv.C + ld_c0;
        L.rb = rsrc_words(xp + toff, live ? xp_bytes - 2 * toff : 0);
        L.dst = lbase + (uint32_t)((ld_st % NST) * STAGE);
        // step by BK channels, wrapping into the next tap (selects, not
        // branches: they would split the MFMA stream)
        ++ld_st;
        const int wrap_c = ld_c0 + BK == cv.C;
        ld_c0 = wrap_c ? 0 : ld_c0 + BK;
        ld_s += wrap_c;
        const int wrap_s = ld_s == cv.S;
        ld_s = wrap_s ? 0 : ld_s;
        ld_r += wrap_s;
        return L;
    };
    auto issue = [&](const Loads &L, int l) __attribute__((always_inline)) {
        if (l < LA)
            load_to_lds(L.ra, L.dst + (uint32_t)((wave + NW * l) * 1024), off[l]);
        else
            load_to_lds(L.rb, L.dst + (uint32_t)(A_BYTES + (wave + NW * (l - LA)) * 1024), off[l]);
    };

    // ---- fragments: wavefront (wm, wn) = (wave / WGN, wave % WGN) owns
    // filters m0 + wm WTM + 16 i + .. and pixels j0 + wn WTN + 16 j + ..; lane
    // (g, s16) reads the 16 bytes of logical unit 4 q + g of row 16 i + s16
    const int wm = wave / WGN, wn = wave % WGN;
    const int g = lane >> 4, s16 = lane & 15;
    auto fa_addr = [&](int st, int q, int i) -> const uint8_t * {
        const int r = wm * WTM + 16 * i + s16;
        return lds + (st % NST) * STAGE + r * ROWB + (((4 * q + g) ^ nhwc_swz<U>(r)) * 16);
    };
    auto fb_addr = [&](int st, int q, int j) -> const uint8_t * {
        const int r = wn * WTN + 16 * j + s16;
        return lds + (st % NST) * STAGE + A_BYTES + r * ROWB + (((4 * q + g) ^ nhwc_swz<U>(r)) * 16);
    };
    constexpr int NREAD = FM + FN;
    auto fread = [&](int st, int q, int rd, halfx8 *fa, halfx8 *fb) __attribute__((always_inline)) {
        if (rd < FM)
            fa[rd] = *reinterpret_cast<const halfx8 *>(fa_addr(st, q, rd));
        else
            fb[rd - FM] = *reinterpret_cast<const halfx8 *>(fb_addr(st, q, rd - FM));
    };

    // accumulators in ordinary registers (at most 64 blocks, 256 a lane):
    // started in the accumulator registers, the compiler moves them between
    // the two files on every stage
    floatx4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
            acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    // prologue: stages 0 .. NST - 2; then stage 0's first fragments
#pragma unroll
    for (int st = 0; st < NST - 1; ++st) {
        const Loads L = next_loads();
#pragma unroll
        for (int l = 0; l < LW; ++l)
            issue(L, l);
    }
    __builtin_amdgcn_s_waitcnt(wait_vmcnt((NST - 2) * LW));
    __builtin_amdgcn_s_barrier();
    halfx8 fa0[FM], fb0[FN], fa1[FM], fb1[FN];
#pragma unroll
    for (int rd = 0; rd < NREAD; ++rd)
        fread(0, 0, rd, fa0, fb0);

    // One 32-deep step (q of stage st): its FM x FN MFMAs from (ca, cb); the
    // next step's reads into (na, nb) after the first NREAD of them; during
    // the stage's first step, the stage's LW loads spread over the rest.
    constexpr int NMF = FM * FN;
    auto step = [&](int st, int q, const Loads &L, const halfx8 *ca, const halfx8 *cb, halfx8 *na, halfx8 *nb)
                    __attribute__((always_inline)) {
        const int nst = q + 1 < SUB ? st : st + 1, nq = q + 1 < SUB ? q + 1 : 0;
#pragma unroll
        for (int m = 0; m < NMF; ++m) {
            const int i = m / FN, j = m % FN;
            acc[i][j] = nhwc_mma<BF16>(ca[i], cb[j], acc[i][j]);
            if (m < NREAD)
                fread(nst, nq, m, na, nb);
            if (q == 0) {
#pragma unroll
                for (int l = 0; l < LW; ++l)
                    if (m == (NMF * (l + 1)) / (LW + 1))
                        issue(L, l);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (NREAD > NMF) {   // fewer MFMAs than reads: the rest now
#pragma unroll
            for (int m = NMF; m < NREAD; ++m)
                fread(nst, nq, m, na, nb);
        }
    };
    // one stage: wait for stage st + 1 (all but this wavefront's loads of
    // stages st + 2 ..) and this wavefront's LDS reads, barrier, then its
    // steps; the step parity alternates the fragment register sets
    auto stage = [&](int st, auto par_c) __attribute__((always_inline)) {
        constexpr int par = decltype(par_c)::value;
        __builtin_amdgcn_s_waitcnt(wait_vmcnt_lgkm0((NST - 3) * LW));
        __builtin_amdgcn_s_barrier();
        const Loads L = next_loads();   // stage st + NST - 1
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < SUB; ++q) {
            if (((q + par * SUB) & 1) == 0)
                step(st, q, L, fa0, fb0, fa1, fb1);
            else
                step(st, q, L, fa1, fb1, fa0, fb0);
        }
    };
    // SUB even: every stage starts from set 0; SUB odd: stages alternate
    if constexpr (SUB % 2 == 0) {
        for (int t = 0; t < steps; ++t)
            stage(t, std::integral_constant<int, 0>{});
    } else {
        for (int t = 0; t < steps; t += 2) {
            stage(t, std::integral_constant<int, 0>{});
            if (t + 1 < steps)
                stage(t + 1, std::integral_constant<int, 1>{});
        }
    }
    // no load may still be writing this workgroup's LDS when it ends
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));

    // ---- y (NKPQ): lane (g, s16) holds filters 16 i + 4 g + r, pixel
    // 16 j + s16 of the wavefront's block; an element outside y gets an
    // out-of-range offset
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(y, (long long)cv.N * cv.K * PQ * 4);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int jj = j0 + wn * WTN + 16 * j + s16;
        const int n = jj / PQ, pq = jj - n * PQ;
        const int base = jj < npq ? n * cv.K * PQ + pq : -1;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int k = m0 + wm * WTM + 16 * i + 4 * g + r;
                const uint32_t o = (base >= 0 && k < cv.K) ? (uint32_t)(base + k * PQ) * 4u : OOB;
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][j][r]), ry, o, 0, 0);
            }
    }
}

template <bool BF16, int BM, int BN, int BK, int WGM, int NST, int NW>
void launch_nhwc_t(const Conv2d &cv, const uint16_t *xp, const uint16_t *wr, float *y, int Hp, int Wp,
                   hipStream_t s)
{
    const long long npq = (long long)cv.N * cv.P * cv.Q;
    const int tiles_m = (cv.K + BM - 1) / BM, tiles_n = (int)((npq + BN - 1) / BN);
    hipLaunchKernelGGL((conv_nhwc_kernel<BF16, BM, BN, BK, WGM, NST, NW>), dim3((unsigned)(tiles_m * tiles_n)),
                       dim3(64 * NW), 0, s, xp, wr, y, cv, Hp, Wp, tiles_m, tiles_n);
}

// The channel block of the prepare kernel: 64 channels when C allows
int nhwc_prepare_ch(const Conv2d &cv) { return cv.C % 64 == 0 ? 64 : 32; }

void launch_nhwc_prepare(const Conv2d &cv, const void *x, const void *w, void *xp, void *wr, hipStream_t s)
{
    const int Hp = cv.H + 2 * cv.ph, Wp = cv.W + 2 * cv.pw, ch = nhwc_prepare_ch(cv);
    const long long npix = (long long)cv.N * Hp * Wp;
    const PrepRows pr = prep_rows(cv);
    const bool rows = prep_rows_apply(cv, x);
    const int xp_blocks = (rows ? cv.N * pr.groups : (int)((npix + kPrepPix - 1) / kPrepPix)) * (cv.C / ch);
    const int w_blocks = cv.K * (cv.C / ch);
    hipLaunchKernelGGL(nhwc_prepare, dim3((unsigned)(xp_blocks + w_blocks)), dim3(256), 0, s, (const uint16_t *)x,
                       (const uint16_t *)w, (uint16_t *)xp, (uint16_t *)wr, cv, Hp, Wp, ch, xp_blocks, pr,
                       rows ? 1 : 0);
}

template <bool BF16>
void launch_nhwc(const Conv2d &cv, const NhwcPlan &np, const uint16_t *xp, const uint16_t *wr, float *y,
                 hipStream_t s)
{
    const int Hp = cv.H + 2 * cv.ph, Wp = cv.W + 2 * cv.pw;
    if (np.bm == 64)
        launch_nhwc_t<BF16, 64, 256, 32, 1, 4, 4>(cv, xp, wr, y, Hp, Wp, s);
    else if (np.bk == 64)
        launch_nhwc_t<BF16, 128, 64, 64, 4, 4, 4>(cv, xp, wr, y, Hp, Wp, s);
    else
        launch_nhwc_t<BF16, 128, 64, 32, 4, 4, 4>(cv, xp, wr, y, Hp, Wp, s);
}

}  // namespace

// The channels-last implicit GEMM's tiles.  K <= 64: 64 filters x 256
// pixels, 32-deep stages (80 KB of LDS, so two workgroups share a CU), the
// four wavefronts side by side along the pixels (64 x 64 each).  K > 64: 128
// filters x 64 pixels, 64-deep stages where C allows (else 32), the
// wavefronts stacked along the filters (32 x 64 each).  Both keep a ring of
// four stages.  It applies to 16-bit inputs with C a multiple of 32, filters
// of at most 64 taps, at least 96 tiles, and every byte offset below 2^31.
bool conv_nhwc_plan(const Conv2d &cv, int elem_bytes, NhwcPlan &np)
{
    if (elem_bytes != 2 || cv.C < 32 || cv.C % 32 != 0 || cv.K < 1 || cv.R * cv.S > kNhwcMaxRS)
        return false;
    const long long npq = (long long)cv.N * cv.P * cv.Q;
    if (cv.K <= 64) {
        np.bm = 64; np.bn = 256; np.bk = 32;
    } else {
        np.bm = 128; np.bn = 64; np.bk = cv.C % 64 == 0 ? 64 : 32;
    }
    const long long tiles = ((cv.K + np.bm - 1) / np.bm) * ((npq + np.bn - 1) / np.bn);
    const long long Hp = cv.H + 2LL * cv.ph, Wp = cv.W + 2LL * cv.pw;
    const long long xp_elems = (long long)cv.N * Hp * Wp * cv.C;
    const long long rsc = (long long)cv.R * cv.S * cv.C;
    np.xp_bytes = (size_t)xp_elems * 2;
    np.wr_bytes = (size_t)(cv.K * rsc) * 2;
    return tiles >= 96 && xp_elems * 2 < (1LL << 31) && cv.K * rsc * 2 < (1LL << 31) &&
           (long long)cv.N * cv.K * cv.P * cv.Q * 4 < (1LL << 31) && npq < (1LL << 30);
}

hipError_t launch_conv_nhwc(const Conv2d &cv, const NhwcPlan &np, bool bf16, const void *x, const void *w, float *y,
                            void *xp, void *wr, hipStream_t s)
{
    launch_nhwc_prepare(cv, x, w, xp, wr, s);
    if (bf16)
        launch_nhwc<true>(cv, np, (const uint16_t *)xp, (const uint16_t *)wr, y, s);
    else
        launch_nhwc<false>(cv, np, (const uint16_t *)xp, (const uint16_t *)wr, y, s);
    return hipGetLastError();
}

}  // namespace dgor
