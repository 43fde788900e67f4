// Convolution through im2col and one GEMM ("Lesson 8: how a GPU does matrix
// multiply" names convolution as matrix multiplication, and direct
// convolution against im2col, as its next lesson).
//
// x is N x C x H x W, w is K x C x R x S, y is N x K x P x Q (all row-major).
// With CRS = C R S and NPQ = N P Q, the product is
//     Y'[k][n PQ + p Q + q] = sum_crs W[k][crs] col[crs][n PQ + p Q + q],
//     col[c R S + r S + s][n PQ + p Q + q] = x[n][c][p sh - ph + r dh][q sw - pw + s dw]
// (zero outside the image), a K x CRS by CRS x NPQ GEMM.  The three memory-
// bound passes here prepare its operands and lay its result out as NKPQ:
//   pad_weights: W (K x CRS) into K x CRSp, zero columns past CRS (skipped
//                when CRS is a multiple of 8: W is then used as it is);
//   im2col:      col into CRSp x NPQp, zero rows past CRS and columns past NPQ;
//   to_nkpq:     Y' (K x NPQp) into y, summing the split-K partials in order
//                (four outputs a thread when PQ is a multiple of 4).
// CRSp and NPQp round CRS and NPQ up to multiples of 8, so both GEMM operands
// take 16-byte loads; the padding adds exact zeros only.
#include "common.h"
#include "lds_dma.h"

#include <type_traits>

namespace dgor {
namespace {

template <typename T>
__global__ __launch_bounds__(256) void pad_weights(const T *__restrict__ w, T *__restrict__ wp, int K, int crs,
                                                   int crsp)
{
    const size_t n = (size_t)K * crsp;
    for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (size_t)gridDim.x * 256) {
        const int k = (int)(e / crsp), j = (int)(e % crsp);
        wp[e] = j < crs ? w[(size_t)k * crs + j] : T(0);
    }
}

// Each thread owns one column j of col (an output pixel: image n, row p,
// column q), decoded once, and writes kRowChunk consecutive rows of it
// (c, r, s stepped without division); blockIdx.y picks the chunk.
// Consecutive threads take consecutive pixels, so reads of x follow its rows
// (stride sw) and writes of col are contiguous.
constexpr int kRowChunk = 32;

template <typename T>
__global__ __launch_bounds__(256) void im2col(const T *__restrict__ x, T *__restrict__ col, Conv2d cv, int crsp,
                                              int npqp)
{
    const int RS = cv.R * cv.S, crs_n = cv.C * RS, PQ = cv.P * cv.Q, npq = cv.N * PQ;
    const int j = blockIdx.x * 256 + threadIdx.x;
    if (j >= npqp)
        return;
    const bool pad_col = j >= npq;
    const int n = pad_col ? 0 : j / PQ, pq = j - n * PQ, p = pq / cv.Q, q = pq - p * cv.Q;
    const int h0 = p * cv.sh - cv.ph, w0 = q * cv.sw - cv.pw;
    const T *img = x + (size_t)n * cv.C * cv.H * cv.W;
    for (int row0 = blockIdx.y * kRowChunk; row0 < crsp; row0 += gridDim.y * kRowChunk) {
        const int rows = min(kRowChunk, crsp - row0);
        T *out = col + (size_t)row0 * npqp + j;
        int c = row0 / RS, rs = row0 - c * RS, r = rs / cv.S, s = rs - r * cv.S;
        for (int i = 0; i < rows; ++i) {
            T v = T(0);
            if (!pad_col && row0 + i < crs_n) {
                const int h = h0 + r * cv.dh, wc = w0 + s * cv.dw;
                if (h >= 0 && h < cv.H && wc >= 0 && wc < cv.W)
                    v = img[((size_t)c * cv.H + h) * cv.W + wc];
            }
            out[(size_t)i * npqp] = v;
            if (++s == cv.S) {
                s = 0;
                if (++r == cv.R) {
                    r = 0;
                    ++c;
                }
            }
        }
    }
}

// y[n][k][p Q + q] = sum over s < splits, ascending, of the split-K partials
// Y'_s[k][n PQ + p Q + q] (one partial without split-K).
__global__ __launch_bounds__(256) void to_nkpq(const float *__restrict__ yp, float *__restrict__ y, int N, int K,
                                               int PQ, int npqp, int splits, size_t split_stride)
{
    const size_t total = (size_t)N * K * PQ;
    for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (size_t)gridDim.x * 256) {
        const int pq = (int)(e % PQ);
        const size_t nk = e / PQ;
        const int k = (int)(nk % K), n = (int)(nk / K);
        const float *src = yp + (size_t)k * npqp + (size_t)n * PQ + pq;
        float v = src[0];
        for (int sp = 1; sp < splits; ++sp)
            v += src[(size_t)sp * split_stride];
        y[e] = v;
    }
}

// The same with four consecutive outputs per thread (PQ a multiple of 4, so
// they share n and k; y and the partials 16-byte aligned).
__global__ __launch_bounds__(256) void to_nkpq4(const float *__restrict__ yp, float *__restrict__ y, int N, int K,
                                                int PQ, int npqp, int splits, size_t split_stride)
{
    const size_t total4 = (size_t)N * K * PQ / 4;
    for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < total4; e += (size_t)gridDim.x * 256) {
        const size_t e0 = 4 * e;
        const int pq = (int)(e0 % PQ);
        const size_t nk = e0 / PQ;
        const int k = (int)(nk % K), n = (int)(nk / K);
        const float *src = yp + (size_t)k * npqp + (size_t)n * PQ + pq;
        float4 v = *reinterpret_cast<const float4 *>(src);
        for (int sp = 1; sp < splits; ++sp) {
            const float4 w = *reinterpret_cast<const float4 *>(src + (size_t)sp * split_stride);
            v.x += w.x;
            v.y += w.y;
            v.z += w.z;
            v.w += w.w;
        }
        *reinterpret_cast<float4 *>(y + e0) = v;
    }
}

// ---------------------------------------------------------------------------
// Implicit GEMM for 16-bit inputs: the same K x CRS by CRS x NPQ product
// with the im2col matrix never written.  Each workgroup computes BM filters x
// 256 output pixels; its 256 threads each own one pixel (decoded once) and
// gather that pixel's 32 values of every 32-deep k-stage straight from x
// (stepping c, r, s; a tap outside the image reads a valid element of x and
// is replaced by zero, so the loads carry no branch and all 32 are in flight
// together), two stages ahead of the MFMAs, in registers.  LDS holds two
// stages, both operands stored with k contiguous (80-byte rows: 32 halves and
// 16 bytes of padding, so the 16 rows one 128-bit read cycle touches fall on
// distinct banks), and each v_mfma_f32_16x16x32 operand is one 128-bit read
// (lane (g, s) takes k = 8 g .. 8 g + 7 of row or pixel s).  Results go
// straight to y (NKPQ).  Wavefront w takes pixels 64 w .. 64 w + 63 and all
// BM filters.
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

template <bool BF16>
__device__ __forceinline__ floatx4 igemm_mma(uint4 a, uint4 b, floatx4 c)
{
    if constexpr (BF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(halfx8, a), __builtin_bit_cast(halfx8, b),
                                                      c, 0, 0, 0);
}

template <bool BF16, int BM>
__global__ __launch_bounds__(256) void conv_igemm(const uint16_t *__restrict__ x, const uint16_t *__restrict__ wa,
                                                  float *__restrict__ y, Conv2d cv, int crsp, int tiles_m)
{
    constexpr int BN = 256, BK = 32, ROWB = 80, FM = BM / 16, AV = BM / 64;
    constexpr int A_BYTES = BM * ROWB, STAGE = A_BYTES + BN * ROWB;
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * STAGE];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tm = blockIdx.x % tiles_m, tn = blockIdx.x / tiles_m;   // a pixel block's filter tiles adjacent
    const int m0 = tm * BM, j0 = tn * BN;
    const int RS = cv.R * cv.S, crs_n = cv.C * RS, PQ = cv.P * cv.Q, npq = cv.N * PQ;

    // this thread's pixel: its offset into x at tap (c, r, s) = (0, 0, 0),
    // and the top-left input position; the tap offset c H W + r dh W + s dw
    // and the gather state (c, r, s, k) are the same in every lane
    constexpr uint32_t OOB = 0x80000000u;
    const int jp = j0 + tid;
    const bool jv = jp < npq;
    const int n = jv ? jp / PQ : 0, pq = jv ? jp - n * PQ : 0, p = pq / cv.Q, q = pq - p * cv.Q;
    const int h0 = p * cv.sh - cv.ph, w0 = q * cv.sw - cv.pw;
    const int lane_base = (n * cv.C * cv.H + h0) * cv.W + w0;   // x < 2^30 elements
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, (long long)cv.N * cv.C * cv.H * cv.W * 2);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(wa, (long long)cv.K * crsp * 2);
    int gc = 0, gr = 0, gs = 0, gk = 0;
    // the next BK values of this pixel; a tap outside the image (or past CRS,
    // or of a pixel past NPQ) has an out-of-range offset and reads zero
    auto gather = [&](uint32_t (&dst)[BK]) __attribute__((always_inline)) {
#pragma unroll
        for (int e = 0; e < BK; ++e) {
            const int rh = gr * cv.dh, sw = gs * cv.dw;
            const bool ok = jv & (gk + e < crs_n) & ((unsigned)(h0 + rh) < (unsigned)cv.H) &
                            ((unsigned)(w0 + sw) < (unsigned)cv.W);
            const uint32_t off = ok ? (uint32_t)(lane_base + (gc * cv.H + rh) * cv.W + sw) * 2u : OOB;
            dst[e] = __builtin_amdgcn_raw_buffer_load_b16(rx, off, 0, 0);
            if (++gs == cv.S) {
                gs = 0;
                if (++gr == cv.R) {
                    gr = 0;
                    ++gc;
                }
            }
        }
        gk += BK;
    };
    // W (K x CRSp, rows 16-byte aligned): thread t loads 16-byte units
    // t + 256 i of the stage's BM x 32 block (zero past K or CRSp)
    auto load_a = [&](int st, uint4 (&dst)[AV]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < AV; ++i) {
            const int u = tid + 256 * i, row = u >> 2, kq = (u & 3) * 8, kk = st * BK + kq;
            const bool ok = (m0 + row < cv.K) & (kk < crsp);
            const uint32_t off = ok ? (uint32_t)((m0 + row) * crsp + kk) * 2u : OOB;
            dst[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, off, 0, 0));
        }
    };
    auto store = [&](int buf, const uint32_t (&rb)[BK], const uint4 (&ra)[AV]) __attribute__((always_inline)) {
        uint8_t *st = lds + buf * STAGE;
#pragma unroll
        for (int i = 0; i < AV; ++i) {
            const int u = tid + 256 * i;
            *reinterpret_cast<uint4 *>(st + (u >> 2) * ROWB + (u & 3) * 16) = ra[i];
        }
        uint32_t pk[BK / 2];
#pragma unroll
        for (int e = 0; e < BK / 2; ++e)
            pk[e] = (rb[2 * e] & 0xffffu) | (rb[2 * e + 1] << 16);
#pragma unroll
        for (int v = 0; v < 4; ++v)
            *reinterpret_cast<uint4 *>(st + A_BYTES + tid * ROWB + 16 * v) =
                make_uint4(pk[4 * v], pk[4 * v + 1], pk[4 * v + 2], pk[4 * v + 3]);
    };

    const int g = lane >> 4, s16 = lane & 15;
    floatx4 acc[FM][4];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int jb = 0; jb < 4; ++jb)
#pragma unroll
            for (int r = 0; r < 4; ++r)   // AGPR writes, so the accumulators stay in AGPRs
                asm("v_accvgpr_write_b32 %0, 0" : "=a"(acc[i][jb][r]));
    auto compute = [&](int buf) __attribute__((always_inline)) {
        const uint8_t *st = lds + buf * STAGE;
        uint4 a[FM], b[4];
#pragma unroll
        for (int i = 0; i < FM; ++i)
            a[i] = *reinterpret_cast<const uint4 *>(st + (16 * i + s16) * ROWB + 16 * g);
#pragma unroll
        for (int jb = 0; jb < 4; ++jb)
            b[jb] = *reinterpret_cast<const uint4 *>(st + A_BYTES + (64 * wave + 16 * jb + s16) * ROWB + 16 * g);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int jb = 0; jb < 4; ++jb)
                acc[i][jb] = igemm_mma<BF16>(a[i], b[jb], acc[i][jb]);
    };

    // stages t and t + 1 gathered before the loop; during stage t the gather
    // of stage t + 2 flies while stage t computes, then stage t + 1 (gathered
    // during t - 1) is stored for the next trip.  A register set is reused
    // once its stage is in LDS; an LDS buffer once the barrier after its
    // stage's MFMAs has passed.
    const int steps = (crsp + BK - 1) / BK;
    uint32_t rb[2][BK];
    uint4 ra[2][AV];
    gather(rb[0]);
    load_a(0, ra[0]);
    gather(rb[1]);   // past the last stage every tap is out of range
    load_a(1, ra[1]);
    store(0, rb[0], ra[0]);
    __syncthreads();
    auto stage = [&](int t, auto cur_c) __attribute__((always_inline)) {
        constexpr int cur = decltype(cur_c)::value;
        gather(rb[cur]);   // stage t + 2 (no condition: a load under one is waited for)
        load_a(t + 2, ra[cur]);
        // keep the order: the store waits for the loads of stage t + 1 only
        // if it stays behind this stage's MFMAs and the new gathers
        __builtin_amdgcn_sched_barrier(0);
        compute(cur);
        __builtin_amdgcn_sched_barrier(0);
        if (t + 1 < steps)
            store(cur ^ 1, rb[cur ^ 1], ra[cur ^ 1]);
        __syncthreads();
    };
    for (int t = 0; t < steps; t += 2) {
        stage(t, std::integral_constant<int, 0>{});
        if (t + 1 < steps)
            stage(t + 1, std::integral_constant<int, 1>{});
    }

    // lane (g, s16) of wavefront w holds filters m0 + 16 i + 4 g + r of pixel
    // j0 + 64 w + 16 jb + s16
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
        const int jo = j0 + 64 * wave + 16 * jb + s16;
        if (jo >= npq)
            continue;
        const int no = jo / PQ, pqo = jo - no * PQ;
        float *yo = y + (size_t)no * cv.K * PQ + pqo;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int k = m0 + 16 * i + 4 * g + r;
                if (k < cv.K)
                    yo[(size_t)k * PQ] = acc[i][jb][r];
            }
    }
}

// Zero-padded copy of x for the vector gather: xp is N x C x Hp x Wp with
// Hp = H + 2 ph and Wp = W + 2 pw rounded up to a multiple of 8, x at rows
// ph.., columns pw.., zeros elsewhere.  One thread per 8 consecutive
// elements of a row of xp, written with one 16-byte store.  A chunk that
// lies wholly inside a row of x (all but the edges) is read with a 16-byte
// and a 4-byte load from the even element at or below its first, shifted
// into place; an edge chunk with eight 2-byte loads, a position outside the
// image taking an out-of-range offset (which reads zero).
__global__ __launch_bounds__(256) void pad_input(const uint16_t *__restrict__ x, uint16_t *__restrict__ xp, Conv2d cv,
                                                 int Hp, int Wp, int chunks)
{
    constexpr uint32_t OOB = 0x80000000u;
    const int x_elems = cv.N * cv.C * cv.H * cv.W;   // < 2^30
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, (long long)x_elems * 2);
    const int per_row = Wp / 8;
    for (int ch = blockIdx.x * 256 + threadIdx.x; ch < chunks; ch += gridDim.x * 256) {
        const int row = ch / per_row, col0 = (ch - row * per_row) * 8;
        const int nc = row / Hp, h = row - nc * Hp - cv.ph, w0 = col0 - cv.pw;
        const bool hv = (unsigned)h < (unsigned)cv.H;
        const int first = (nc * cv.H + h) * cv.W + w0, e0 = first & ~1;
        uint32_t o[4];
        if (hv && w0 >= 0 && w0 + 8 <= cv.W && e0 + 10 <= x_elems) {
            const uint4 d = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, (uint32_t)e0 * 2u, 0, 0));
            const uint32_t d4 = __builtin_amdgcn_raw_buffer_load_b32(rx, (uint32_t)e0 * 2u + 16u, 0, 0);
            const uint32_t sh = (uint32_t)(first - e0) * 2u;
            o[0] = __builtin_amdgcn_alignbyte(d.y, d.x, sh);
            o[1] = __builtin_amdgcn_alignbyte(d.z, d.y, sh);
            o[2] = __builtin_amdgcn_alignbyte(d.w, d.z, sh);
            o[3] = __builtin_amdgcn_alignbyte(d4, d.w, sh);
        } else {
            uint32_t v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const bool ok = hv & ((unsigned)(w0 + e) < (unsigned)cv.W);
                v[e] = __builtin_amdgcn_raw_buffer_load_b16(rx, ok ? (uint32_t)(first + e) * 2u : OOB, 0, 0);
            }
#pragma unroll
            for (int m = 0; m < 4; ++m)
                o[m] = (v[2 * m] & 0xffffu) | (v[2 * m + 1] << 16);
        }
        *reinterpret_cast<uint4 *>(xp + (size_t)ch * 8) = make_uint4(o[0], o[1], o[2], o[3]);
    }
}

// Implicit GEMM with a vector gather, for stride 1 along w and Q a multiple
// of 4: the four pixels j, j + 1, j + 2, j + 3 (j a multiple of 4) then sit
// in one output row and read four adjacent elements of the padded input for
// every tap, so one 12-byte load at the even element at or below the first
// (then shifted by 0 or 2 bytes) fetches them; the padding makes every tap
// inside the copy, so no lane is masked but those past NPQ or CRS.
// Wavefront w gathers taps 8 w .. 8 w + 7 of each 32-deep stage for all 256
// pixels of the tile (lane l: pixels 4 l .. 4 l + 3), transposes them in
// registers and stores, per pixel, 16 bytes (8 taps, k ascending) into slot
// p ^ ((p >> 3) & 3) of the stage's tap-group-w block: the XOR keeps both
// these stores (lanes 4 slots apart) and the MFMA operand reads (16
// consecutive pixels) on distinct banks.  Tiles, A staging, the two-stage
// pipeline and the output are those of the kernel above.
template <bool BF16, int BM>
__global__ __launch_bounds__(256) void conv_igemm_vec(const uint16_t *__restrict__ xp, const uint16_t *__restrict__ wa,
                                                      float *__restrict__ y, Conv2d cv, int crsp, int tiles_m, int Hp,
                                                      int Wp, int xp_elems)
{
    constexpr int BN = 256, BK = 32, ROWB = 80, FM = BM / 16, AV = BM / 64;
    constexpr int A_BYTES = BM * ROWB, GROUP = BN * 16, STAGE = A_BYTES + 4 * GROUP;
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * STAGE];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tm = blockIdx.x % tiles_m, tn = blockIdx.x / tiles_m;
    const int m0 = tm * BM, j0 = tn * BN;
    const int RS = cv.R * cv.S, crs_n = cv.C * RS, PQ = cv.P * cv.Q, npq = cv.N * PQ;

    constexpr uint32_t OOB = 0x80000000u;
    const int jp = j0 + 4 * lane;   // this lane's first pixel; NPQ is a multiple of 4
    const bool jv = jp < npq;
    const int n = jv ? jp / PQ : 0, pq = jv ? jp - n * PQ : 0, p = pq / cv.Q, q = pq - p * cv.Q;
    const int lane_base = (n * cv.C * Hp + p * cv.sh) * Wp + q;   // xp < 2^30 elements
    const uint32_t lb_odd = (uint32_t)lane_base & 1u;
    // the copy plus 8 elements of slack: a load may reach 2 elements past it
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(xp, ((long long)xp_elems + 8) * 2);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(wa, (long long)cv.K * crsp * 2);
    // this wavefront's next tap (c, r, s) and its index; the gather steps
    // through 8 taps, then skips the 24 the other wavefronts take
    int gk = 8 * wave;
    int gc = gk / RS, gr = (gk - gc * RS) / cv.S, gs = gk - gc * RS - gr * cv.S;
    const int skip_c = 24 / RS, skip_r = (24 - skip_c * RS) / cv.S, skip_s = 24 - skip_c * RS - skip_r * cv.S;
    // raw 12-byte loads of the 8 taps, and the parity of each tap's offset
    auto gather = [&](uint32_t (&dst)[8][3], uint32_t &par) __attribute__((always_inline)) {
        uint32_t pm = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int toff = (gc * Hp + gr * cv.dh) * Wp + gs * cv.dw;
            const bool ok = jv & (gk + e < crs_n);
            const uint32_t off = ok ? (uint32_t)((lane_base + toff) & ~1) * 2u : OOB;
            const auto v = __builtin_amdgcn_raw_buffer_load_b96(rx, off, 0, 0);
            dst[e][0] = v[0];
            dst[e][1] = v[1];
            dst[e][2] = v[2];
            pm |= (uint32_t)(toff & 1) << e;
            if (++gs == cv.S) {
                gs = 0;
                if (++gr == cv.R) {
                    gr = 0;
                    ++gc;
                }
            }
        }
        gk += BK;
        gs += skip_s;
        if (gs >= cv.S) {
            gs -= cv.S;
            ++gr;
        }
        gr += skip_r;
        if (gr >= cv.R) {
            gr -= cv.R;
            ++gc;
        }
        gc += skip_c;
        par = pm;
    };
    auto load_a = [&](int st, uint4 (&dst)[AV]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < AV; ++i) {
            const int u = tid + 256 * i, row = u >> 2, kq = (u & 3) * 8, kk = st * BK + kq;
            const bool ok = (m0 + row < cv.K) & (kk < crsp);
            const uint32_t off = ok ? (uint32_t)((m0 + row) * crsp + kk) * 2u : OOB;
            dst[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, off, 0, 0));
        }
    };
    auto slot = [](int px) { return px ^ ((px >> 3) & 3); };
    auto store = [&](int buf, const uint32_t (&rb)[8][3], uint32_t par, const uint4 (&ra)[AV])
                     __attribute__((always_inline)) {
        uint8_t *st = lds + buf * STAGE;
#pragma unroll
        for (int i = 0; i < AV; ++i) {
            const int u = tid + 256 * i;
            *reinterpret_cast<uint4 *>(st + (u >> 2) * ROWB + (u & 3) * 16) = ra[i];
        }
        // pixels (0, 1) and (2, 3) of each tap, shifted into place
        uint32_t lo[8], hi[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t sh = ((((par >> e) & 1u) ^ lb_odd)) * 2u;
            lo[e] = __builtin_amdgcn_alignbyte(rb[e][1], rb[e][0], sh);
            hi[e] = __builtin_amdgcn_alignbyte(rb[e][2], rb[e][1], sh);
        }
        uint8_t *grp = st + A_BYTES + wave * GROUP;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t *src = i < 2 ? lo : hi;
            const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;   // high or low halves
            uint32_t v[4];
#pragma unroll
            for (int m = 0; m < 4; ++m)
                v[m] = __builtin_amdgcn_perm(src[2 * m + 1], src[2 * m], sel);   // taps 2m, 2m + 1
            *reinterpret_cast<uint4 *>(grp + slot(4 * lane + i) * 16) = make_uint4(v[0], v[1], v[2], v[3]);
        }
    };

    const int g = lane >> 4, s16 = lane & 15;
    floatx4 acc[FM][4];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int jb = 0; jb < 4; ++jb)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                asm("v_accvgpr_write_b32 %0, 0" : "=a"(acc[i][jb][r]));
    auto compute = [&](int buf) __attribute__((always_inline)) {
        const uint8_t *st = lds + buf * STAGE;
        uint4 a[FM], b[4];
#pragma unroll
        for (int i = 0; i < FM; ++i)
            a[i] = *reinterpret_cast<const uint4 *>(st + (16 * i + s16) * ROWB + 16 * g);
#pragma unroll
        for (int jb = 0; jb < 4; ++jb)
            b[jb] = *reinterpret_cast<const uint4 *>(st + A_BYTES + g * GROUP + slot(64 * wave + 16 * jb + s16) * 16);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int jb = 0; jb < 4; ++jb)
                acc[i][jb] = igemm_mma<BF16>(a[i], b[jb], acc[i][jb]);
    };

    const int steps = (crsp + BK - 1) / BK;
    uint32_t rb[2][8][3], par[2];
    uint4 ra[2][AV];
    gather(rb[0], par[0]);
    load_a(0, ra[0]);
    gather(rb[1], par[1]);   // past the last stage every tap is past CRS
    load_a(1, ra[1]);
    store(0, rb[0], par[0], ra[0]);
    __syncthreads();
    auto stage = [&](int t, auto cur_c) __attribute__((always_inline)) {
        constexpr int cur = decltype(cur_c)::value;
        gather(rb[cur], par[cur]);
        load_a(t + 2, ra[cur]);
        __builtin_amdgcn_sched_barrier(0);
        compute(cur);
        __builtin_amdgcn_sched_barrier(0);
        if (t + 1 < steps)
            store(cur ^ 1, rb[cur ^ 1], par[cur ^ 1], ra[cur ^ 1]);
        __syncthreads();
    };
    for (int t = 0; t < steps; t += 2) {
        stage(t, std::integral_constant<int, 0>{});
        if (t + 1 < steps)
            stage(t + 1, std::integral_constant<int, 1>{});
    }

#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
        const int jo = j0 + 64 * wave + 16 * jb + s16;
        if (jo >= npq)
            continue;
        const int no = jo / PQ, pqo = jo - no * PQ;
        float *yo = y + (size_t)no * cv.K * PQ + pqo;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int k = m0 + 16 * i + 4 * g + r;
                if (k < cv.K)
                    yo[(size_t)k * PQ] = acc[i][jb][r];
            }
    }
}

unsigned blocks_for(size_t n)
{
    const size_t b = (n + 255) / 256;
    return (unsigned)(b < 65536 ? (b ? b : 1) : 65536);
}

}  // namespace

hipError_t launch_conv_prepare(const Conv2d &cv, int elem_bytes, const void *x, const void *w, void *wp, void *col,
                               int crsp, int npqp, hipStream_t s)
{
    const int crs = cv.C * cv.R * cv.S;
    if (crsp == 0)   // no channels: the GEMM's empty sum writes the zeros
        return hipSuccess;
    const int chunks = (crsp + kRowChunk - 1) / kRowChunk;
    const dim3 g_im((unsigned)((npqp + 255) / 256), (unsigned)(chunks < 65535 ? chunks : 65535));
    if (elem_bytes == 4) {
        if (wp)
            hipLaunchKernelGGL(pad_weights<float>, dim3(blocks_for((size_t)cv.K * crsp)), dim3(256), 0, s,
                               (const float *)w, (float *)wp, cv.K, crs, crsp);
        if (col)
            hipLaunchKernelGGL(im2col<float>, g_im, dim3(256), 0, s, (const float *)x, (float *)col, cv, crsp, npqp);
    } else {
        if (wp)
            hipLaunchKernelGGL(pad_weights<uint16_t>, dim3(blocks_for((size_t)cv.K * crsp)), dim3(256), 0, s,
                               (const uint16_t *)w, (uint16_t *)wp, cv.K, crs, crsp);
        if (col)
            hipLaunchKernelGGL(im2col<uint16_t>, g_im, dim3(256), 0, s, (const uint16_t *)x, (uint16_t *)col, cv,
                               crsp, npqp);
    }
    return hipGetLastError();
}

bool conv_igemm_applies(const Conv2d &cv, int elem_bytes)
{
    if (elem_bytes != 2 || cv.C == 0)
        return false;
    const long long npq = (long long)cv.N * cv.P * cv.Q;
    const long long tiles = (long long)((cv.K + 127) / 128) * ((npq + 255) / 256);
    // byte offsets into x and W stay below 2^31
    return tiles >= 256 && npq < (1LL << 30) && (long long)cv.N * cv.C * cv.H * cv.W < (1LL << 30) &&
           (long long)cv.K * cv.C * cv.R * cv.S < (1LL << 29);
}

long long conv_padded_input_elems(const Conv2d &cv)
{
    return (long long)cv.N * cv.C * (cv.H + 2LL * cv.ph) * ((cv.W + 2LL * cv.pw + 7) / 8 * 8);
}

bool conv_igemm_vec_applies(const Conv2d &cv, int elem_bytes)
{
    return conv_igemm_applies(cv, elem_bytes) && cv.sw == 1 && cv.Q % 4 == 0 &&
           conv_padded_input_elems(cv) + 8 < (1LL << 30);
}

namespace {
template <bool BF16>
hipError_t launch_igemm_t(const Conv2d &cv, const void *x, const void *wa, float *y, int crsp, void *xp,
                          hipStream_t s)
{
    const long long npq = (long long)cv.N * cv.P * cv.Q;
    const int tn = (int)((npq + 255) / 256), bm = cv.K <= 64 ? 64 : 128, tiles_m = (cv.K + bm - 1) / bm;
    const dim3 grid((unsigned)(tiles_m * tn));
    // the padded copy reads x with 4- and 16-byte loads from even elements:
    // x must then start 4-byte aligned (else the element gather, which reads
    // 2 bytes at a time)
    if (conv_igemm_vec_applies(cv, 2) && ((uintptr_t)x & 3) == 0) {
        const int Hp = cv.H + 2 * cv.ph, Wp = (cv.W + 2 * cv.pw + 7) / 8 * 8;
        const int elems = (int)conv_padded_input_elems(cv), chunks = elems / 8;
        const int blocks = (chunks + 255) / 256 < 65536 ? (chunks + 255) / 256 : 65536;
        hipLaunchKernelGGL(pad_input, dim3((unsigned)blocks), dim3(256), 0, s, (const uint16_t *)x, (uint16_t *)xp,
                           cv, Hp, Wp, chunks);
        if (bm == 64)
            hipLaunchKernelGGL((conv_igemm_vec<BF16, 64>), grid, dim3(256), 0, s, (const uint16_t *)xp,
                               (const uint16_t *)wa, y, cv, crsp, tiles_m, Hp, Wp, elems);
        else
            hipLaunchKernelGGL((conv_igemm_vec<BF16, 128>), grid, dim3(256), 0, s, (const uint16_t *)xp,
                               (const uint16_t *)wa, y, cv, crsp, tiles_m, Hp, Wp, elems);
    } else if (bm == 64) {
        hipLaunchKernelGGL((conv_igemm<BF16, 64>), grid, dim3(256), 0, s, (const uint16_t *)x, (const uint16_t *)wa,
                           y, cv, crsp, tiles_m);
    } else {
        hipLaunchKernelGGL((conv_igemm<BF16, 128>), grid, dim3(256), 0, s, (const uint16_t *)x,
                           (const uint16_t *)wa, y, cv, crsp, tiles_m);
    }
    return hipGetLastError();
}
}  // namespace

hipError_t launch_conv_igemm(const Conv2d &cv, bool bf16, const void *x, const void *wa, float *y, int crsp, void *xp,
                             hipStream_t s)
{
    return bf16 ? launch_igemm_t<true>(cv, x, wa, y, crsp, xp, s) : launch_igemm_t<false>(cv, x, wa, y, crsp, xp, s);
}

hipError_t launch_conv_output(const Conv2d &cv, const float *yp, float *y, int npqp, int splits,
                              size_t split_stride, hipStream_t s)
{
    const size_t total = (size_t)cv.N * cv.K * cv.P * cv.Q;
    const int PQ = cv.P * cv.Q;
    // partials: yp 16-byte aligned, rows of npqp (a multiple of 8) floats,
    // split_stride a multiple of 64 floats
    if (PQ % 4 == 0 && ((uintptr_t)y & 15) == 0 && ((uintptr_t)yp & 15) == 0 && split_stride % 4 == 0)
        hipLaunchKernelGGL(to_nkpq4, dim3(blocks_for(total / 4)), dim3(256), 0, s, yp, y, cv.N, cv.K, PQ, npqp,
                           splits, split_stride);
    else
        hipLaunchKernelGGL(to_nkpq, dim3(blocks_for(total)), dim3(256), 0, s, yp, y, cv.N, cv.K, PQ, npqp, splits,
                           split_stride);
    return hipGetLastError();
}

}  // namespace dgor
