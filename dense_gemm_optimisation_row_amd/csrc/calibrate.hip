// Matrix-core rate calibration (measurement instrument, not a GEMM).
//
// Under the socket power limit, a 16-bit GEMM's throughput is set by the
// energy each instruction costs, not by issue cycles alone.  This kernel
// measures the ceiling that leaves: the sustained rate of the 256 x 256 ring
// tile's own matrix-core instruction stream with nothing else running --
// no global or LDS traffic, no waits, no barriers.  It is built into its own
// library (libdgor_calibrate.so), which the GEMM library never loads; only
// the benchmark's calibration mode calls it.
//
// Shape of the work: the same grid as the GEMM of an M x N x K problem
// (ceil(M/256) ceil(N/256) workgroups of four wavefronts), each wavefront
// owning 8 x 8 blocks of 16 x 16 outputs in 256 AGPR accumulators per lane
// and issuing, per 32-deep k-stage, the 64 v_mfma_f32_16x16x32_f16 of the
// GEMM's stage in the same order (A fragment i, B fragment j, j fastest).
// So it executes exactly the GEMM's 2 M' N' K' matrix-core operations (K
// rounded up to a multiple of 64, as the GEMM's tiles round M and N).  The
// operand fragments are taken once from the first 64 k of the wavefront's
// own rows of A and columns of B (the caller passes the GEMM's inputs, so the
// operand bit patterns, and with them the multiplier switching, are the
// workload's) and held in registers; stages alternate between the two
// 32-deep sets.  C receives the accumulators, so none of the work is dead;
// its values are the product over those 64 k repeated K / 64 times, not A B.
#include "common.h"
#include "lds_dma.h"

namespace {

typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void mfma_f16_rate_kernel(const uint16_t *A, const uint16_t *B, float *C, int M,
                                                            int N, int K, int tiles_m)
{
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int tm = blockIdx.x % tiles_m, tn = blockIdx.x / tiles_m;
    const int wr = tm * 256 + (wave >> 1) * 128, wc = tn * 256 + (wave & 1) * 128;
    const int s16 = lane & 15, g = lane >> 4;
    // fragment of block i, set h: eight k 32 h + 8 g .. +7 of row wr + 16 i + s16
    // (A) or of column wc + 16 j + s16 (B); outside the matrices an
    // out-of-range offset reads zero (no branches: they would crowd the
    // accumulators out of their registers)
    constexpr uint32_t OOB = 0x80000000u;
    const __amdgpu_buffer_rsrc_t ra = dgor::make_rsrc(A, (long long)M * K * 2);
    const __amdgpu_buffer_rsrc_t rb = dgor::make_rsrc(B, (long long)K * N * 2);
    halfx8 fa[2][8], fb[2][8];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = wr + 16 * i + s16, c = wc + 16 * i + s16;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int k = 32 * h + 8 * g + e;
                const uint32_t oa = (r < M && k < K) ? (uint32_t)((size_t)r * K + k) * 2u : OOB;
                const uint32_t ob = (c < N && k < K) ? (uint32_t)((size_t)k * N + c) * 2u : OOB;
                fa[h][i][e] = __builtin_bit_cast(_Float16, __builtin_amdgcn_raw_buffer_load_b16(ra, oa, 0, 0));
                fb[h][i][e] = __builtin_bit_cast(_Float16, __builtin_amdgcn_raw_buffer_load_b16(rb, ob, 0, 0));
            }
        }
    floatx4 acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)   // AGPR writes, so the accumulators stay in AGPRs
                asm("v_accvgpr_write_b32 %0, 0" : "=a"(acc[i][j][r]));
    // One stage: the 64 MFMAs as one block of assembly.  Written with the
    // builtin, a loop whose operands stay the same from trip to trip makes
    // the compiler copy the 256 accumulators between registers on every trip;
    // here operand m is accumulator block (m / 8, m % 8), operands 64..71 the
    // A fragments and 72..79 the B fragments.  No two MFMAs in a row share an
    // accumulator, and each is read again only 64 instructions later.
#define DGOR_MF(m, a, b) "v_mfma_f32_16x16x32_f16 %" #m ", %" #a ", %" #b ", %" #m "\n\t"
    auto stage = [&](const halfx8 *ca, const halfx8 *cb) {
        asm volatile(
            "s_nop 4\n\t"   // wait states after whatever wrote the operands last
            DGOR_MF(0, 64, 72) DGOR_MF(1, 64, 73) DGOR_MF(2, 64, 74) DGOR_MF(3, 64, 75)
            DGOR_MF(4, 64, 76) DGOR_MF(5, 64, 77) DGOR_MF(6, 64, 78) DGOR_MF(7, 64, 79)
            DGOR_MF(8, 65, 72) DGOR_MF(9, 65, 73) DGOR_MF(10, 65, 74) DGOR_MF(11, 65, 75)
            DGOR_MF(12, 65, 76) DGOR_MF(13, 65, 77) DGOR_MF(14, 65, 78) DGOR_MF(15, 65, 79)
            DGOR_MF(16, 66, 72) DGOR_MF(17, 66, 73) DGOR_MF(18, 66, 74) DGOR_MF(19, 66, 75)
            DGOR_MF(20, 66, 76) DGOR_MF(21, 66, 77) DGOR_MF(22, 66, 78) DGOR_MF(23, 66, 79)
            DGOR_MF(24, 67, 72) DGOR_MF(25, 67, 73) DGOR_MF(26, 67, 74) DGOR_MF(27, 67, 75)
            DGOR_MF(28, 67, 76) DGOR_MF(29, 67, 77) DGOR_MF(30, 67, 78) DGOR_MF(31, 67, 79)
            DGOR_MF(32, 68, 72) DGOR_MF(33, 68, 73) DGOR_MF(34, 68, 74) DGOR_MF(35, 68, 75)
            DGOR_MF(36, 68, 76) DGOR_MF(37, 68, 77) DGOR_MF(38, 68, 78) DGOR_MF(39, 68, 79)
            DGOR_MF(40, 69, 72) DGOR_MF(41, 69, 73) DGOR_MF(42, 69, 74) DGOR_MF(43, 69, 75)
            DGOR_MF(44, 69, 76) DGOR_MF(45, 69, 77) DGOR_MF(46, 69, 78) DGOR_MF(47, 69, 79)
            DGOR_MF(48, 70, 72) DGOR_MF(49, 70, 73) DGOR_MF(50, 70, 74) DGOR_MF(51, 70, 75)
            DGOR_MF(52, 70, 76) DGOR_MF(53, 70, 77) DGOR_MF(54, 70, 78) DGOR_MF(55, 70, 79)
            DGOR_MF(56, 71, 72) DGOR_MF(57, 71, 73) DGOR_MF(58, 71, 74) DGOR_MF(59, 71, 75)
            DGOR_MF(60, 71, 76) DGOR_MF(61, 71, 77) DGOR_MF(62, 71, 78) DGOR_MF(63, 71, 79)
            : "+a"(acc[0][0]), "+a"(acc[0][1]), "+a"(acc[0][2]), "+a"(acc[0][3]), "+a"(acc[0][4]),
              "+a"(acc[0][5]), "+a"(acc[0][6]), "+a"(acc[0][7]), "+a"(acc[1][0]), "+a"(acc[1][1]),
              "+a"(acc[1][2]), "+a"(acc[1][3]), "+a"(acc[1][4]), "+a"(acc[1][5]), "+a"(acc[1][6]),
              "+a"(acc[1][7]), "+a"(acc[2][0]), "+a"(acc[2][1]), "+a"(acc[2][2]), "+a"(acc[2][3]),
              "+a"(acc[2][4]), "+a"(acc[2][5]), "+a"(acc[2][6]), "+a"(acc[2][7]), "+a"(acc[3][0]),
              "+a"(acc[3][1]), "+a"(acc[3][2]), "+a"(acc[3][3]), "+a"(acc[3][4]), "+a"(acc[3][5]),
              "+a"(acc[3][6]), "+a"(acc[3][7]), "+a"(acc[4][0]), "+a"(acc[4][1]), "+a"(acc[4][2]),
              "+a"(acc[4][3]), "+a"(acc[4][4]), "+a"(acc[4][5]), "+a"(acc[4][6]), "+a"(acc[4][7]),
              "+a"(acc[5][0]), "+a"(acc[5][1]), "+a"(acc[5][2]), "+a"(acc[5][3]), "+a"(acc[5][4]),
              "+a"(acc[5][5]), "+a"(acc[5][6]), "+a"(acc[5][7]), "+a"(acc[6][0]), "+a"(acc[6][1]),
              "+a"(acc[6][2]), "+a"(acc[6][3]), "+a"(acc[6][4]), "+a"(acc[6][5]), "+a"(acc[6][6]),
              "+a"(acc[6][7]), "+a"(acc[7][0]), "+a"(acc[7][1]), "+a"(acc[7][2]), "+a"(acc[7][3]),
              "+a"(acc[7][4]), "+a"(acc[7][5]), "+a"(acc[7][6]), "+a"(acc[7][7])
            : "v"(ca[0]), "v"(ca[1]), "v"(ca[2]), "v"(ca[3]), "v"(ca[4]), "v"(ca[5]), "v"(ca[6]), "v"(ca[7]),
              "v"(cb[0]), "v"(cb[1]), "v"(cb[2]), "v"(cb[3]), "v"(cb[4]), "v"(cb[5]), "v"(cb[6]), "v"(cb[7]));
    };
#undef DGOR_MF
    // K rounded up to a multiple of 64: two stages a trip
    const int pairs = (K + 63) / 64;
    for (int t = 0; t < pairs; ++t) {
        stage(fa[0], fb[0]);
        stage(fa[1], fb[1]);
    }
    dgor_acc_hazard_wait();
    // lane (g, s16) holds rows 16 i + 4 g + r and column 16 j + s16 of the
    // wavefront's block
    const __amdgpu_buffer_rsrc_t rc = dgor::make_rsrc(C, (long long)M * N * 4);
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = wr + 16 * i + 4 * g + r, col = wc + 16 * j + s16;
                const uint32_t oc = (row < M && col < N) ? (uint32_t)((size_t)row * N + col) * 4u : OOB;
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(dgor_acc_read(acc[i][j][r])), rc, oc, 0, 0);
            }
}

}  // namespace

// Enqueue the calibration kernel for an M x N x K binary16 problem (device
// pointers: A M x K and B K x N row-major binary16 bits, C M x N FP32,
// written) on `stream`.  Returns 0, or -1 for a negative or empty shape or a
// null pointer, or -3 if the launch failed.
extern "C" int dgor_calibrate_mfma_f16(const uint16_t *A, const uint16_t *B, float *C, int M, int N, int K,
                                       void *stream)
{
    if (M <= 0 || N <= 0 || K <= 0 || !A || !B || !C)
        return -1;
    const int tiles_m = (M + 255) / 256, tiles_n = (N + 255) / 256;
    hipLaunchKernelGGL(mfma_f16_rate_kernel, dim3((unsigned)(tiles_m * tiles_n)), dim3(256), 0,
                       (hipStream_t)stream, A, B, C, M, N, K, tiles_m);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}
