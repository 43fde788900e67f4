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
        hipLaunchKernelGGL(im2col<float>, g_im, dim3(256), 0, s, (const float *)x, (float *)col, cv, crsp, npqp);
    } else {
        if (wp)
            hipLaunchKernelGGL(pad_weights<uint16_t>, dim3(blocks_for((size_t)cv.K * crsp)), dim3(256), 0, s,
                               (const uint16_t *)w, (uint16_t *)wp, cv.K, crs, crsp);
        hipLaunchKernelGGL(im2col<uint16_t>, g_im, dim3(256), 0, s, (const uint16_t *)x, (uint16_t *)col, cv, crsp,
                           npqp);
    }
    return hipGetLastError();
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
