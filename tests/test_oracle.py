"""Pins for the CPU oracle: each test ties it to something other than itself.

The oracle computes C[i,j] = sum_k A[i,k] B[k,j] ("Lesson 8: how a GPU does
matrix multiply", section 1; "SGEMM optimisation journey", Level 1) with
row-major operands (Lesson 8, section 2), K = 0 giving zeros and C being
overwritten ("4. GEMM optimisation", section 4.1).  The pages print no worked
numeric example of C, so the pins below are closed forms, exact rational
arithmetic, library routines in special cases and invariants.
"""
import ctypes
from fractions import Fraction

import numpy as np
import pytest

import oracle

RNG = np.random.default_rng(12345)


def _wide_f32(shape, rng, lo=-20, hi=20):
    """Random binary32 values with exponents spread over [lo, hi)."""
    mant = rng.uniform(1.0, 2.0, shape)
    sign = rng.choice([-1.0, 1.0], shape)
    expo = rng.integers(lo, hi, shape)
    return (sign * mant * np.exp2(expo)).astype(np.float32)


def _bits(x):
    return np.ascontiguousarray(x, np.float32).view(np.uint32)


# ----------------------------------------------------------------- binary16 --

def test_f16_decoder_matches_numpy_on_every_bit_pattern():
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = pats.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_f64(int(h)) for h in pats])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # sign of zero is kept
    assert np.signbit(oracle.f16_to_f64(0x8000)) and not np.signbit(oracle.f16_to_f64(0))


def test_f16_decoder_spot_values():
    # 0x3C00 = 1.0, 0xC000 = -2.0, 0x0001 = 2^-24 (smallest subnormal),
    # 0x03FF = 1023 * 2^-24 (largest subnormal), 0x0400 = 2^-14, 0x7BFF = 65504.
    cases = {0x3C00: 1.0, 0xC000: -2.0, 0x0001: 2.0 ** -24,
             0x03FF: 1023 * 2.0 ** -24, 0x0400: 2.0 ** -14, 0x7BFF: 65504.0,
             0x3555: 1365 / 4096, 0x7C00: float("inf")}
    for h, v in cases.items():
        assert oracle.f16_to_f64(h) == v, hex(h)


# ------------------------------------------------------- closed-form pins ---

@pytest.mark.parametrize("M,K", [(1, 1), (7, 13), (64, 33), (129, 200)])
def test_identity_right_and_left(M, K):
    A = _wide_f32((M, K), RNG)
    I_k = np.eye(K, dtype=np.float32)
    I_m = np.eye(M, dtype=np.float32)
    assert np.array_equal(oracle.gemm_f32(A, I_k), A)
    assert np.array_equal(oracle.gemm_f32(I_m, A), A)


@pytest.mark.parametrize("M,K,N", [(5, 9, 11), (70, 40, 90)])
def test_permutation_products(M, K, N):
    A = _wide_f32((M, K), RNG)
    B = _wide_f32((K, N), RNG)
    pr = RNG.permutation(M)
    pc = RNG.permutation(N)
    P_rows = np.eye(M, dtype=np.float32)[pr]          # (P A)[i] = A[pr[i]]
    P_cols = np.eye(N, dtype=np.float32)[:, pc]       # (B Q)[:, j] = B[:, pc[j]]
    assert np.array_equal(oracle.gemm_f32(P_rows, A), A[pr])
    assert np.array_equal(oracle.gemm_f32(B, P_cols), B[:, pc])


@pytest.mark.parametrize("M,K,N", [(1, 1, 1), (6, 17, 9), (33, 300, 45)])
def test_rank1_closed_form(M, K, N):
    # A = u v^T, B = w z^T  =>  C = (v . w) u z^T, exact for small integers.
    u = RNG.integers(-4, 5, M)
    v = RNG.integers(-4, 5, K)
    w = RNG.integers(-4, 5, K)
    z = RNG.integers(-4, 5, N)
    A = np.outer(u, v).astype(np.float32)
    B = np.outer(w, z).astype(np.float32)
    expect = (int(v @ w) * np.outer(u, z)).astype(np.float32)
    assert np.array_equal(oracle.gemm_f32(A, B), expect)


def test_all_ones_gives_K():
    for K in (1, 2, 777, 4096):
        C = oracle.gemm_f32(np.ones((3, K), np.float32), np.ones((K, 5), np.float32))
        assert np.all(C == K)


def test_K1_is_the_correctly_rounded_product():
    # One term: C[i,j] = fl32(A[i,0] * B[0,j]).  numpy's binary32 multiply is
    # IEEE correctly rounded, so the bits must agree exactly.
    A = _wide_f32((50, 1), RNG)
    B = _wide_f32((1, 70), RNG)
    expect = A * B                      # float32 x float32 -> float32, RNE
    got = oracle.gemm_f32(A, B)
    assert np.array_equal(_bits(got), _bits(expect))


def test_K0_writes_zeros_and_overwrites():
    out = np.full((4, 6), np.nan, np.float32)
    oracle.gemm_f32(np.empty((4, 0), np.float32), np.empty((0, 6), np.float32), out=out)
    assert np.array_equal(out, np.zeros((4, 6), np.float32))
    # C is overwritten, not accumulated into
    A = np.ones((2, 3), np.float32)
    out = np.full((2, 2), 100.0, np.float32)
    oracle.gemm_f32(A, np.ones((3, 2), np.float32), out=out)
    assert np.all(out == 3.0)


def test_empty_M_or_N_writes_nothing_and_bad_dims_fail():
    lib = oracle._load()
    sentinel = np.full(8, 7.0, np.float32)
    A = np.ones(16, np.float32)
    p = lambda a: ctypes.c_void_p(a.ctypes.data)
    assert lib.oracle_gemm_f32(0, 4, 3, p(A), p(A), p(sentinel), 1) == 0
    assert lib.oracle_gemm_f32(4, 0, 3, p(A), p(A), p(sentinel), 1) == 0
    assert np.all(sentinel == 7.0)
    assert lib.oracle_gemm_f32(-1, 4, 3, p(A), p(A), p(sentinel), 1) == -1
    assert lib.oracle_gemm_f32(1, 1, -3, p(A), p(A), p(sentinel), 1) == -1
    with pytest.raises(ValueError):
        oracle.gemm_f32(np.ones((2, 3), np.float32), np.ones((4, 2), np.float32))


# -------------------------------------------------- exact rational brute force

def _exact_product(A, B):
    M, K = A.shape
    N = B.shape[1]
    Af = [[Fraction(float(x)) for x in row] for row in A]
    Bf = [[Fraction(float(x)) for x in row] for row in B]
    return [[sum((Af[i][k] * Bf[k][j] for k in range(K)), Fraction(0))
             for j in range(N)] for i in range(M)]


def _round_exact_to_f32(q: Fraction) -> np.float32:
    d = float(q)
    # the exact sum must be a binary64 number, so this is a single rounding
    assert Fraction(d) == q
    return np.float32(d)


def test_bruteforce_dyadic_all_shapes_up_to_6():
    # Inputs j/16, j in [-16, 16]: every sum is exact in binary32 and binary64.
    rng = np.random.default_rng(7)
    for M in range(1, 7):
        for N in range(1, 7):
            for K in range(1, 7):
                A = (rng.integers(-16, 17, (M, K)) / 16).astype(np.float32)
                B = (rng.integers(-16, 17, (K, N)) / 16).astype(np.float32)
                ex = _exact_product(A, B)
                expect = np.array([[_round_exact_to_f32(q) for q in r] for r in ex],
                                  np.float32)
                assert np.array_equal(oracle.gemm_f32(A, B), expect), (M, N, K)


def test_bruteforce_final_rounding_is_round_to_nearest_even():
    # 12-bit mantissas with exponents in [-6, 6]: products have 24-bit
    # mantissas, sums of up to 6 of them fit binary64 exactly but need up to
    # ~50 bits, so the result must be the exact sum rounded once (RNE).
    rng = np.random.default_rng(8)
    rounded = 0
    for M in range(1, 7):
        for N in range(1, 7):
            for K in range(1, 7):
                def draw(shape):
                    m = rng.integers(2048, 4096, shape)
                    e = rng.integers(-6, 7, shape)
                    s = rng.choice([-1, 1], shape)
                    return (s * m * np.exp2(e - 11)).astype(np.float32)
                A, B = draw((M, K)), draw((K, N))
                ex = _exact_product(A, B)
                expect = np.array([[_round_exact_to_f32(q) for q in r] for r in ex],
                                  np.float32)
                got = oracle.gemm_f32(A, B)
                assert np.array_equal(_bits(got), _bits(expect)), (M, N, K)
                rounded += sum(Fraction(float(g)) != q
                               for g, q in zip(got.ravel(), sum(ex, [])))
    assert rounded > 100   # the rounding step was really exercised


def test_numpy_float64_matmul_within_one_ulp():
    A = RNG.uniform(-1, 1, (67, 129)).astype(np.float32)
    B = RNG.uniform(-1, 1, (129, 93)).astype(np.float32)
    ref = (A.astype(np.float64) @ B.astype(np.float64)).astype(np.float32)
    got = oracle.gemm_f32(A, B)
    ulp = np.abs(_bits(got).astype(np.int64) - _bits(ref).astype(np.int64))
    same_sign = np.signbit(got) == np.signbit(ref)
    assert np.all(ulp[same_sign] <= 1)
    assert np.all(np.abs(got[~same_sign]) < 1e-30)
    # and against the (much looser) binary32 product numpy computes itself
    assert np.max(np.abs(got - A @ B)) < 1e-4


def test_small_integer_products_are_exact():
    A = RNG.integers(-4, 5, (37, 300))
    B = RNG.integers(-4, 5, (300, 53))
    got = oracle.gemm_f32(A.astype(np.float32), B.astype(np.float32))
    assert np.array_equal(got, (A @ B).astype(np.float32))


def test_result_does_not_depend_on_thread_count():
    A = RNG.standard_normal((203, 301)).astype(np.float32)
    B = RNG.standard_normal((301, 157)).astype(np.float32)
    one = oracle.gemm_f32(A, B, nthreads=1)
    many = oracle.gemm_f32(A, B, nthreads=8)
    assert np.array_equal(_bits(one), _bits(many))
    assert oracle.threads(3) == 3


def test_selected_elements_match_full_product_bit_for_bit():
    A = RNG.standard_normal((97, 211)).astype(np.float32)
    B = RNG.standard_normal((211, 83)).astype(np.float32)
    full = oracle.gemm_f32(A, B)
    r = RNG.integers(0, 97, 500)
    c = RNG.integers(0, 83, 500)
    assert np.array_equal(_bits(oracle.gemm_f32_at(A, B, r, c)), _bits(full[r, c]))
    A16 = A.astype(np.float16)
    B16 = B.astype(np.float16)
    full16 = oracle.gemm_f16(A16, B16)
    assert np.array_equal(_bits(oracle.gemm_f16_at(A16, B16, r, c)), _bits(full16[r, c]))
    with pytest.raises(RuntimeError):
        oracle.gemm_f32_at(A, B, [97], [0])


# ------------------------------------------------------------ binary16 path --

def test_f16_product_equals_f32_product_of_the_decoded_values():
    # binary16 values are exactly binary32 values, so the binary16 routine
    # must give the same bits as the (pinned) binary32 routine on them.
    A = RNG.uniform(-1, 1, (61, 250)).astype(np.float16)
    B = RNG.uniform(-1, 1, (250, 77)).astype(np.float16)
    a32 = A.astype(np.float32)
    b32 = B.astype(np.float32)
    assert np.array_equal(_bits(oracle.gemm_f16(A, B)), _bits(oracle.gemm_f32(a32, b32)))


def test_f16_bruteforce_exact():
    rng = np.random.default_rng(9)
    for M in range(1, 7):
        for N in range(1, 7):
            for K in range(1, 7):
                A = rng.uniform(-1, 1, (M, K)).astype(np.float16)
                B = rng.uniform(-1, 1, (K, N)).astype(np.float16)
                ex = _exact_product(A.astype(np.float64), B.astype(np.float64))
                expect = np.array([[_round_exact_to_f32(q) for q in r] for r in ex],
                                  np.float32)
                assert np.array_equal(_bits(oracle.gemm_f16(A, B)), _bits(expect)), (M, N, K)


def test_f16_accepts_raw_bit_patterns_and_small_integers_are_exact():
    A = RNG.integers(-4, 5, (20, 500))
    B = RNG.integers(-4, 5, (500, 30))
    A16 = A.astype(np.float16).view(np.uint16)
    B16 = B.astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.gemm_f16(A16, B16), (A @ B).astype(np.float32))


# ------------------------------------------------------------ bfloat16 path --
# bfloat16 keeps the sign, the 8 exponent bits and the top 7 fraction bits of
# a binary32 ("Lesson 8: how a GPU does matrix multiply", section 22, names
# the format).  torch's CPU conversion of bfloat16 to float32 is an
# independent implementation of the decode.

def _bf16_to_f32_via_torch(bits):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16)).view(torch.bfloat16)
    with np.errstate(invalid="ignore"):   # NaN patterns widen quietly
        return t.float().numpy().astype(np.float64)


def test_bf16_decoder_matches_torch_on_every_bit_pattern():
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = _bf16_to_f32_via_torch(pats)
    got = np.array([oracle.bf16_to_f64(int(h)) for h in pats])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.signbit(oracle.bf16_to_f64(0x8000)) and not np.signbit(oracle.bf16_to_f64(0))


def test_bf16_decoder_spot_values():
    # 0x3F80 = 1.0, 0xC000 = -2.0, 0x0001 = 2^-133 (smallest subnormal),
    # 0x007F = 127 * 2^-133 (largest subnormal), 0x0080 = 2^-126,
    # 0x7F7F = 255 * 2^120 (largest finite), 0x3EAB = 171 * 2^-9.
    cases = {0x3F80: 1.0, 0xC000: -2.0, 0x0001: 2.0 ** -133, 0x007F: 127 * 2.0 ** -133,
             0x0080: 2.0 ** -126, 0x7F7F: 255 * 2.0 ** 120, 0x3EAB: 171 * 2.0 ** -9,
             0x7F80: float("inf")}
    for h, v in cases.items():
        assert oracle.bf16_to_f64(h) == v, hex(h)


def _bf16_bits(x):
    from dense_gemm_optimisation_row_amd import inputs
    return inputs.to_bf16_bits(np.asarray(x, np.float32))


def test_bf16_input_rounding_matches_torch():
    # the shared input generator's float32 -> bfloat16 rounding (nearest,
    # ties to even) against torch's conversion, including exact ties
    import torch
    rng = np.random.default_rng(21)
    x = (rng.standard_normal(200000) * np.exp2(rng.integers(-60, 60, 200000))).astype(np.float32)
    ties = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 2.0 ** -130], np.float32)
    x = np.concatenate([x, ties])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(_bf16_bits(x), ref)


def test_bf16_product_equals_f32_product_of_the_decoded_values():
    # bfloat16 values are exactly binary32 values: the bfloat16 routine must
    # give the bits of the (pinned) binary32 routine on the decoded inputs.
    A = _bf16_bits(RNG.uniform(-1, 1, (61, 250)))
    B = _bf16_bits(RNG.uniform(-1, 1, (250, 77)))
    a32 = _bf16_to_f32_via_torch(A).astype(np.float32)
    b32 = _bf16_to_f32_via_torch(B).astype(np.float32)
    assert np.array_equal(_bits(oracle.gemm_bf16(A, B)), _bits(oracle.gemm_f32(a32, b32)))
    r = RNG.integers(0, 61, 300)
    c = RNG.integers(0, 77, 300)
    full = oracle.gemm_bf16(A, B)
    assert np.array_equal(_bits(oracle.gemm_bf16_at(A, B, r, c)), _bits(full[r, c]))


def test_bf16_bruteforce_exact():
    rng = np.random.default_rng(10)
    for M in range(1, 7):
        for N in range(1, 7):
            for K in range(1, 7):
                A = _bf16_bits(rng.uniform(-1, 1, (M, K)))
                B = _bf16_bits(rng.uniform(-1, 1, (K, N)))
                a = _bf16_to_f32_via_torch(A).reshape(M, K)
                b = _bf16_to_f32_via_torch(B).reshape(K, N)
                ex = _exact_product(a, b)
                expect = np.array([[_round_exact_to_f32(q) for q in r] for r in ex],
                                  np.float32)
                assert np.array_equal(_bits(oracle.gemm_bf16(A, B)), _bits(expect)), (M, N, K)


def test_bf16_small_integers_are_exact():
    A = RNG.integers(-4, 5, (20, 500))
    B = RNG.integers(-4, 5, (500, 30))
    assert np.array_equal(oracle.gemm_bf16(_bf16_bits(A), _bf16_bits(B)),
                          (A @ B).astype(np.float32))


# ------------------------------------------ general layouts, alpha and beta --
# C = alpha op(A) op(B) + beta C with row strides lda / ldb / ldc ("Lesson 8:
# how a GPU does matrix multiply", section 28 on the library interface; its
# section 21 writes the matrix unit's D = A x B + C).

def _store(X, op, ld, fill, rng=None):
    """Flat storage of the logical matrix X (rows x cols) as op N (X itself,
    row stride ld) or op T (X's transpose stored row-major, row stride ld),
    with every padding element set to ``fill``."""
    S = X.T if op else X
    r, c = S.shape
    buf = np.full(max((r - 1) * ld + c, 0) if r and c else 0, fill, dtype=X.dtype)
    for i in range(r):
        buf[i * ld:i * ld + c] = S[i]
    return buf


def _ex_layouts():
    for op_a in (0, 1):
        for op_b in (0, 1):
            for pad in (0, 3):
                yield op_a, op_b, pad


@pytest.mark.parametrize("fmt", ["f32", "f16", "bf16"])
def test_ex_transposed_and_padded_operands_match_the_plain_product(fmt):
    # alpha 1, beta 0: the same products summed in the same order as the
    # row-major routine, whatever the storage; padding holds NaN (never read)
    # and C's padding columns keep their sentinel.
    rng = np.random.default_rng(31)
    M, N, K = 9, 7, 11
    A32 = rng.standard_normal((M, K)).astype(np.float32)
    B32 = rng.standard_normal((K, N)).astype(np.float32)
    if fmt == "f32":
        A, B, nan = A32, B32, np.float32(np.nan)
        plain = oracle.gemm_f32(A, B)
    elif fmt == "f16":
        A, B, nan = A32.astype(np.float16).view(np.uint16), B32.astype(np.float16).view(np.uint16), 0x7E00
        plain = oracle.gemm_f16(A, B)
    else:
        A, B, nan = _bf16_bits(A32), _bf16_bits(B32), 0x7FC0
        plain = oracle.gemm_bf16(A, B)
    for op_a, op_b, pad in _ex_layouts():
        lda = (M if op_a else K) + pad
        ldb = (K if op_b else N) + pad
        ldc = N + pad
        Cs = np.full(M * ldc, -7.25, np.float32)
        oracle.gemm_ex(fmt, op_a, op_b, M, N, K, 1.0, _store(A, op_a, lda, nan), lda,
                       _store(B, op_b, ldb, nan), ldb, 0.0, Cs, ldc)
        C = Cs.reshape(M, ldc)
        assert np.array_equal(_bits(C[:, :N]), _bits(plain)), (op_a, op_b, pad)
        assert np.all(C[:, N:] == np.float32(-7.25))


def _few_bit(rng, shape, mant_bits, e_lo, e_hi):
    m = rng.integers(1 << (mant_bits - 1), 1 << mant_bits, shape)
    e = rng.integers(e_lo, e_hi + 1, shape)
    s = rng.choice([-1, 1], shape)
    return (s * m * np.exp2(e - (mant_bits - 1))).astype(np.float32)


def test_ex_bruteforce_alpha_beta_single_rounding():
    # Inputs with 8-bit mantissas, alpha and beta with 5, C with 12: every
    # intermediate of alpha * sum + beta * c spans under 46 bits, so binary64
    # holds it exactly and the result must be the exact value rounded once to
    # binary32 (nearest, ties to even).
    rng = np.random.default_rng(41)
    rounded = 0
    for M in range(1, 5):
        for N in range(1, 5):
            for K in range(1, 7):
                A = _few_bit(rng, (M, K), 8, -4, 4)
                B = _few_bit(rng, (K, N), 8, -4, 4)
                C0 = _few_bit(rng, (M, N), 12, -4, 4)
                alpha = float(_few_bit(rng, (), 5, -2, 2))
                beta = float(_few_bit(rng, (), 5, -2, 2))
                op_a, op_b = int(rng.integers(0, 2)), int(rng.integers(0, 2))
                lda, ldb = (M if op_a else K) + 1, (K if op_b else N) + 2
                Cs = C0.ravel().copy()
                oracle.gemm_ex("f32", op_a, op_b, M, N, K, alpha, _store(A, op_a, lda, np.nan), lda,
                               _store(B, op_b, ldb, np.nan), ldb, beta, Cs, N)
                ex = _exact_product(A, B)
                for i in range(M):
                    for j in range(N):
                        q = Fraction(alpha) * ex[i][j] + Fraction(beta) * Fraction(float(C0[i, j]))
                        want = _round_exact_to_f32(q)
                        assert _bits(Cs[i * N + j]) == _bits(want), (M, N, K, i, j)
                        rounded += Fraction(float(want)) != q
    assert rounded > 100


def test_ex_small_integers_alpha_beta_closed_form():
    rng = np.random.default_rng(43)
    M, N, K = 23, 19, 300
    A = rng.integers(-4, 5, (M, K))
    B = rng.integers(-4, 5, (K, N))
    C0 = rng.integers(-1000, 1001, (M, N))
    for alpha, beta in ((1, 0), (3, -2), (-1, 1), (0.5, 0.25), (2, 1)):
        want = alpha * (A @ B).astype(np.float64) + beta * C0
        for op_a, op_b, pad in _ex_layouts():
            lda, ldb = (M if op_a else K) + pad, (K if op_b else N) + pad
            Cs = C0.astype(np.float32).ravel().copy()
            oracle.gemm_ex("f32", op_a, op_b, M, N, K, alpha, _store(A.astype(np.float32), op_a, lda, np.nan),
                           lda, _store(B.astype(np.float32), op_b, ldb, np.nan), ldb, beta, Cs, N)
            assert np.array_equal(Cs.reshape(M, N), want.astype(np.float32)), (alpha, beta, op_a, op_b)


def test_ex_beta_zero_never_reads_C_and_K0_scales_C():
    rng = np.random.default_rng(47)
    M, N, K = 5, 6, 4
    A = rng.standard_normal((M, K)).astype(np.float32)
    B = rng.standard_normal((K, N)).astype(np.float32)
    Cs = np.full(M * N, np.nan, np.float32)
    oracle.gemm_ex("f32", 0, 0, M, N, K, 2.0, A.ravel(), K, B.ravel(), N, 0.0, Cs, N)
    assert np.array_equal(Cs.reshape(M, N), np.float32(2.0) * oracle.gemm_f32(A, B))
    # K = 0: C = beta C (zeros when beta == 0, even over NaN)
    C0 = rng.standard_normal(M * N).astype(np.float32)
    Cs = C0.copy()
    oracle.gemm_ex("f32", 1, 1, M, N, 0, 3.0, np.zeros(1, np.float32), M, np.zeros(1, np.float32), 1, -0.5, Cs, N)
    assert np.array_equal(Cs, (np.float64(-0.5) * C0).astype(np.float32))
    Cs = np.full(M * N, np.nan, np.float32)
    oracle.gemm_ex("f32", 0, 0, M, N, 0, 3.0, np.zeros(1, np.float32), 1, np.zeros(1, np.float32), N, 0.0, Cs, N)
    assert np.all(Cs == 0)
    # operand arrays shorter than the shape and strides need are refused
    with pytest.raises(ValueError):
        oracle.gemm_ex("f32", 0, 0, M, N, K, 1.0, A.ravel()[:3], K, B.ravel(), N, 0.0, Cs, N)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_ex_16bit_equals_f32_on_the_decoded_values(fmt):
    rng = np.random.default_rng(53)
    M, N, K = 6, 10, 13
    A32 = rng.standard_normal((M, K)).astype(np.float32)
    B32 = rng.standard_normal((K, N)).astype(np.float32)
    if fmt == "f16":
        A, B = A32.astype(np.float16), B32.astype(np.float16)
        Ad, Bd = A.astype(np.float32), B.astype(np.float32)
        A, B = A.view(np.uint16), B.view(np.uint16)
    else:
        A, B = _bf16_bits(A32), _bf16_bits(B32)
        Ad = (A.astype(np.uint32) << 16).view(np.float32)
        Bd = (B.astype(np.uint32) << 16).view(np.float32)
    C0 = rng.standard_normal(M * N).astype(np.float32)
    for op_a, op_b, pad in _ex_layouts():
        lda, ldb = (M if op_a else K) + pad, (K if op_b else N) + pad
        got, want = C0.copy(), C0.copy()
        oracle.gemm_ex(fmt, op_a, op_b, M, N, K, -1.5, _store(A, op_a, lda, 0), lda,
                       _store(B, op_b, ldb, 0), ldb, 0.75, got, N)
        oracle.gemm_ex("f32", op_a, op_b, M, N, K, -1.5, _store(Ad, op_a, lda, 0), lda,
                       _store(Bd, op_b, ldb, 0), ldb, 0.75, want, N)
        assert np.array_equal(_bits(got), _bits(want)), (op_a, op_b, pad)


# -------------------------------------------------------------- 8-bit inputs --
# FP8 (OCP E4M3 and E5M2) and INT8 inputs ("Lesson 8: how a GPU does matrix
# multiply", section 22 names both among the matrix units' input formats).

def _fp8_torch(codes, fmt):
    import torch
    td = torch.float8_e4m3fn if fmt == "e4m3" else torch.float8_e5m2
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(td).float().double().numpy()


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fp8_decoder_matches_torch_on_every_code(fmt):
    codes = np.arange(256, dtype=np.uint8)
    ref = _fp8_torch(codes, fmt)
    dec = oracle.e4m3_to_f64 if fmt == "e4m3" else oracle.e5m2_to_f64
    got = np.array([dec(int(c)) for c in codes])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.signbit(got[fin]), np.signbit(ref[fin]))


def test_fp8_decoder_spot_values():
    e4, e5 = oracle.e4m3_to_f64, oracle.e5m2_to_f64
    assert e4(0x38) == 1.0 and e4(0xC0) == -2.0 and e4(0x7E) == 448.0
    assert e4(0x08) == 2.0 ** -6 and e4(0x01) == 2.0 ** -9 and e4(0x07) == 7 * 2.0 ** -9
    assert np.isnan(e4(0x7F)) and np.isnan(e4(0xFF)) and e4(0x78) == 256.0
    assert e5(0x3C) == 1.0 and e5(0x7B) == 57344.0 and e5(0x04) == 2.0 ** -14
    assert e5(0x01) == 2.0 ** -16 and e5(0x7C) == np.inf and e5(0xFC) == -np.inf
    assert np.isnan(e5(0x7D)) and e5(0xBD) == -1.25


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fp8_input_rounding_matches_torch_including_ties(fmt):
    import torch
    from dense_gemm_optimisation_row_amd import inputs
    td = torch.float8_e4m3fn if fmt == "e4m3" else torch.float8_e5m2
    rng = np.random.default_rng(61)
    x = np.concatenate([rng.uniform(-1, 1, 20000), rng.standard_normal(20000) * 20]).astype(np.float32)
    # exact midpoints between neighbouring codes: ties go to the even code
    fin = _fp8_torch(np.arange(127 if fmt == "e4m3" else 124, dtype=np.uint8), fmt)
    mids = ((fin[:-1] + fin[1:]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (fin[:-1] + fin[1:]) / 2)   # exact in binary32
    x = np.concatenate([x, mids, -mids])
    got = inputs.to_fp8_codes(x, fmt)
    ref = torch.from_numpy(x).to(td).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)
    tie_codes = got[-2 * mids.size:-mids.size]
    assert np.all(tie_codes % 2 == 0)


def _finite_fp8(rng, shape, fmt):
    lim = 0x7E if fmt == "e4m3" else 0x7B
    mag = rng.integers(0, lim + 1, shape)
    return (mag | (rng.integers(0, 2, shape) << 7)).astype(np.uint8)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fp8_product_equals_f32_product_of_the_decoded_values(fmt):
    rng = np.random.default_rng(62)
    A, B = _finite_fp8(rng, (23, 57), fmt), _finite_fp8(rng, (57, 31), fmt)
    fn = oracle.gemm_e4m3 if fmt == "e4m3" else oracle.gemm_e5m2
    got = fn(A, B)
    want = oracle.gemm_f32(_fp8_torch(A, fmt).astype(np.float32), _fp8_torch(B, fmt).astype(np.float32))
    assert np.array_equal(_bits(got), _bits(want))
    rows, cols = np.array([0, 22, 5, 11]), np.array([0, 30, 17, 3])
    at = (oracle.gemm_e4m3_at if fmt == "e4m3" else oracle.gemm_e5m2_at)(A, B, rows, cols)
    assert np.array_equal(_bits(at), _bits(got[rows, cols]))


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fp8_bruteforce_exact(fmt):
    rng = np.random.default_rng(63)
    fn = oracle.gemm_e4m3 if fmt == "e4m3" else oracle.gemm_e5m2
    for M, N, K in [(1, 1, 1), (2, 3, 4), (5, 4, 3), (4, 4, 6)]:
        A, B = _finite_fp8(rng, (M, K), fmt), _finite_fp8(rng, (K, N), fmt)
        Ad, Bd = _fp8_torch(A, fmt), _fp8_torch(B, fmt)
        got = fn(A, B)
        for i in range(M):
            for j in range(N):
                q = sum(Fraction(float(Ad[i, k])) * Fraction(float(Bd[k, j])) for k in range(K))
                assert _bits(got[i, j]) == _bits(_round_exact_to_f32(q)), (fmt, M, N, K, i, j)


def test_i8_product_is_numpy_int64_product():
    rng = np.random.default_rng(64)
    A = rng.integers(-128, 128, (37, 300), dtype=np.int8)
    B = rng.integers(-128, 128, (300, 41), dtype=np.int8)
    got = oracle.gemm_i8(A, B)
    assert got.dtype == np.int32
    assert np.array_equal(got.astype(np.int64), A.astype(np.int64) @ B.astype(np.int64))
    rows, cols = np.array([0, 36, 7]), np.array([40, 0, 19])
    assert np.array_equal(oracle.gemm_i8_at(A, B, rows, cols), got[rows, cols])


def test_i8_extremes_and_overflow():
    # all -128: every element is 16384 K, the largest magnitude; it fits int32
    # up to K = 131071 and the routine refuses K = 131072 (2^31).
    K = 131071
    A = np.full((1, K), -128, np.int8)
    B = np.full((K, 2), -128, np.int8)
    assert np.array_equal(oracle.gemm_i8(A, B), np.full((1, 2), 16384 * K, np.int32))
    B[:, 1] = 127
    assert oracle.gemm_i8(A, B)[0, 1] == -128 * 127 * K
    A = np.full((1, K + 1), -128, np.int8)
    B = np.full((K + 1, 1), -128, np.int8)
    with pytest.raises(RuntimeError):
        oracle.gemm_i8(A, B)
    with pytest.raises(RuntimeError):
        oracle.gemm_i8_at(A, B, [0], [0])


# --------------------------------------------------------------- convolution --
# 2-D convolution as deep-learning frameworks define it (cross-correlation,
# NCHW input, KCRS weights, NKPQ output), the operator "Lesson 8: how a GPU
# does matrix multiply" lists next (convolution as matrix multiplication;
# direct convolution and im2col).

CONV_CASES = [
    # (N, C, H, W, K, R, S, stride, pad, dil)
    (1, 1, 5, 5, 1, 3, 3, (1, 1), (0, 0), (1, 1)),
    (2, 3, 7, 6, 4, 3, 2, (2, 1), (1, 0), (1, 2)),
    (1, 4, 9, 9, 5, 3, 3, (1, 1), (1, 1), (1, 1)),
    (3, 2, 8, 11, 3, 5, 3, (2, 3), (2, 1), (1, 1)),
    (2, 5, 10, 7, 2, 2, 4, (1, 2), (0, 2), (2, 1)),
    (1, 3, 6, 6, 6, 1, 1, (2, 2), (0, 0), (1, 1)),
]


def _torch_conv64(x, w, stride, pad, dil):
    import torch
    return torch.nn.functional.conv2d(torch.from_numpy(np.asarray(x, np.float64)),
                                      torch.from_numpy(np.asarray(w, np.float64)),
                                      stride=stride, padding=pad, dilation=dil).numpy()


@pytest.mark.parametrize("case", CONV_CASES, ids=lambda c: "x".join(map(str, c[:7])))
def test_conv2d_matches_torch_float64_within_one_ulp(case):
    N, C, H, W, K, R, S, st, pd, dl = case
    rng = np.random.default_rng(71)
    x = rng.standard_normal((N, C, H, W)).astype(np.float32)
    w = rng.standard_normal((K, C, R, S)).astype(np.float32)
    got = oracle.conv2d("f32", x, w, st, pd, dl)
    ref = _torch_conv64(x, w, st, pd, dl).astype(np.float32)
    assert got.shape == ref.shape
    ulp = np.abs(_bits(got).astype(np.int64) - _bits(ref).astype(np.int64))
    same_sign = np.signbit(got) == np.signbit(ref)
    assert np.all(ulp[same_sign] <= 1)
    assert np.all(np.abs(got[~same_sign]) < 1e-30)


def test_conv2d_one_by_one_is_the_gemm_per_image():
    rng = np.random.default_rng(72)
    N, C, H, W, K = 3, 19, 5, 7, 11
    x = rng.standard_normal((N, C, H, W)).astype(np.float32)
    w = rng.standard_normal((K, C, 1, 1)).astype(np.float32)
    y = oracle.conv2d("f32", x, w)
    for n in range(N):
        want = oracle.gemm_f32(np.ascontiguousarray(w[:, :, 0, 0]), np.ascontiguousarray(x[n].reshape(C, H * W)))
        assert np.array_equal(_bits(y[n].reshape(K, H * W)), _bits(want))


@pytest.mark.parametrize("case", CONV_CASES, ids=lambda c: "x".join(map(str, c[:7])))
def test_conv2d_all_ones_counts_the_taps_inside_the_image(case):
    N, C, H, W, K, R, S, st, pd, dl = case
    y = oracle.conv2d("f32", np.ones((N, C, H, W), np.float32), np.ones((K, C, R, S), np.float32), st, pd, dl)
    P, Q = y.shape[2:]
    for p in range(P):
        rows = sum(0 <= p * st[0] - pd[0] + r * dl[0] < H for r in range(R))
        for q in range(Q):
            cols = sum(0 <= q * st[1] - pd[1] + s * dl[1] < W for s in range(S))
            assert np.all(y[:, :, p, q] == C * rows * cols), (p, q)


@pytest.mark.parametrize("case", CONV_CASES, ids=lambda c: "x".join(map(str, c[:7])))
def test_conv2d_single_input_pixel_picks_out_the_weights(case):
    # x = one 1 at (n0, c0, h0, v0): y[n0][k][p][q] = w[k][c0][r][s] exactly where
    # h0 = p sh - ph + r dh and v0 = q sw - pw + s dw, and 0 everywhere else
    N, C, H, W, K, R, S, st, pd, dl = case
    rng = np.random.default_rng(73)
    w = rng.standard_normal((K, C, R, S)).astype(np.float32)
    for (n0, c0, h0, v0) in [(0, 0, 0, 0), (N - 1, C - 1, H - 1, W - 1), (N // 2, C // 2, H // 2, W // 3)]:
        x = np.zeros((N, C, H, W), np.float32)
        x[n0, c0, h0, v0] = 1.0
        y = oracle.conv2d("f32", x, w, st, pd, dl)
        want = np.zeros_like(y)
        for p in range(y.shape[2]):
            for q in range(y.shape[3]):
                for r in range(R):
                    for s in range(S):
                        if p * st[0] - pd[0] + r * dl[0] == h0 and q * st[1] - pd[1] + s * dl[1] == v0:
                            want[n0, :, p, q] += w[:, c0, r, s]
        assert np.array_equal(y, want), (n0, c0, h0, v0)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_conv2d_16bit_equals_f32_on_the_decoded_values(fmt):
    rng = np.random.default_rng(74)
    N, C, H, W, K, R, S, st, pd, dl = CONV_CASES[1]
    x32 = rng.standard_normal((N, C, H, W)).astype(np.float32)
    w32 = rng.standard_normal((K, C, R, S)).astype(np.float32)
    if fmt == "f16":
        x, w = x32.astype(np.float16), w32.astype(np.float16)
        xd, wd = x.astype(np.float32), w.astype(np.float32)
    else:
        x, w = _bf16_bits(x32), _bf16_bits(w32)
        xd = (x.astype(np.uint32) << 16).view(np.float32)
        wd = (w.astype(np.uint32) << 16).view(np.float32)
    got = oracle.conv2d(fmt, x, w, st, pd, dl)
    assert np.array_equal(_bits(got), _bits(oracle.conv2d("f32", xd, wd, st, pd, dl)))
