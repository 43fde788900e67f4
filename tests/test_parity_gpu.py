"""GPU parity: every kernel, called through the C ABI, against the CPU oracle.

Bars (elementwise, FP32 output):
  * small-integer inputs (values in {-4..4}): bit-exact, every shape;
  * FP32 inputs: |C - C_ref| <= 2e-6 K;
  * binary16 inputs: |C - C_ref| <= 2e-3 sqrt(K) max|C_ref|.
Shapes span several tiles of each kernel configuration and end in ragged
tails in M, N and K.  The full-size workloads are checked in the launch
configuration the benchmark times: the smaller ones in full here; the
headline sizes (FP32 4096^3, 16-bit 8192^3) in full in test_full_gpu.py, and
here as a quick pre-check on sampled elements plus an invariant over every
output (C v = A (B v) for a random +-1 vector v, exact on integer inputs).
"""
import numpy as np
import pytest

import dense_gemm_optimisation_row_amd as dg
from dense_gemm_optimisation_row_amd import binding, inputs

import oracle
from helpers import (as_f32, assert_bits_equal, assert_within, kind, oracle_at, oracle_full,
                     oracle_gemm, say, to_dev, tol_f16, tol_f32, workload)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU (run the CPU suite with -m 'not gpu')")
    binding.load()  # raises if the HIP library was not built
    return torch.device("cuda")


def run(half, variant, A, B, C=None):
    """Run the entry point for A's input format (``half`` is kept for the
    callers' readability; the format comes from the arrays)."""
    import torch
    a, b = to_dev(A), to_dev(B)
    fn = {"f32": dg.gemm_f32_variant, "f16": dg.gemm_f16_f32acc_variant,
          "bf16": dg.gemm_bf16_f32acc_variant}[kind(A)]
    c = fn(variant, a, b, C)
    torch.cuda.synchronize()
    return c.cpu().numpy()


def _fmt(half):
    return half if isinstance(half, str) else ("f16" if half else "f32")


def ints(M, N, K, seed, half=False):
    return inputs.matrices(M, N, K, seed, "int", _fmt(half))


def floats(M, N, K, seed, half=False):
    return inputs.matrices(M, N, K, seed, "uniform", _fmt(half))


SMALL_SHAPES = [
    (1, 1, 1), (1, 1, 37), (5, 3, 2), (16, 16, 16), (17, 33, 65), (64, 64, 64),
    (100, 70, 9), (127, 129, 131), (256, 256, 256), (300, 200, 100), (129, 257, 513),
    (33, 1000, 48), (1000, 33, 777),
]


@pytest.mark.parametrize("variant", dg.F32_VARIANTS)
@pytest.mark.parametrize("shape", SMALL_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_f32_variants_small_shapes(variant, shape):
    M, N, K = shape
    say("f32", dg.variant_name(variant), shape)
    A, B = ints(M, N, K, 11)
    assert_bits_equal(run(False, variant, A, B), oracle.gemm_f32(A, B), f"ints {shape}")
    A, B = floats(M, N, K, 12)
    assert_within(run(False, variant, A, B), oracle.gemm_f32(A, B), tol_f32(K), f"floats {shape}")


@pytest.mark.parametrize("variant", dg.F16_VARIANTS)
@pytest.mark.parametrize("shape", SMALL_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_f16_variants_small_shapes(variant, shape):
    M, N, K = shape
    say("f16", dg.variant_name(variant), shape)
    A, B = ints(M, N, K, 13, half=True)
    assert_bits_equal(run(True, variant, A, B), oracle.gemm_f16(A, B), f"ints {shape}")
    A, B = floats(M, N, K, 14, half=True)
    ref = oracle.gemm_f16(A, B)
    assert_within(run(True, variant, A, B), ref, tol_f16(K, ref), f"floats {shape}")


@pytest.mark.parametrize("variant", dg.BF16_VARIANTS)
@pytest.mark.parametrize("shape", SMALL_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_bf16_variants_small_shapes(variant, shape):
    M, N, K = shape
    say("bf16", dg.variant_name(variant), shape)
    A, B = ints(M, N, K, 15, "bf16")
    assert_bits_equal(run("bf16", variant, A, B), oracle.gemm_bf16(A, B), f"ints {shape}")
    A, B = floats(M, N, K, 16, "bf16")
    ref = oracle.gemm_bf16(A, B)
    assert_within(run("bf16", variant, A, B), ref, tol_f16(K, ref), f"floats {shape}")


# Shapes large enough that the automatic choice takes each matrix-core tile
# configuration, with ragged edges in all three dimensions.
CONFIG_SHAPES = [
    (False, (4000, 4092, 200), (256, 256)),   # FP32 256 x 256 ring, ragged M/N/K
    (False, (4000, 2044, 100), (128, 128)),   # FP32 128 x 128 direct-load tiles (512 of them)
    (False, (1000, 1000, 1000), (64, 64)),    # FP32 64 x 64 tiles
    (False, (4097, 33, 777), (16, 33)),       # FP32 tall, narrow: 2 MFMA blocks + a vector column, tail row
    (False, (4097, 64, 1024), (16, 64)),      # FP32 tall, narrow: 4 MFMA blocks, K = 1024
    (False, (4097, 16, 2048), (32, 64)),      # FP32 narrow tiles (K past 1024)
    (True, (8191, 4097, 72), (256, 256)),     # FP16 256 x 256 tiles, unaligned rows
    (True, (8000, 4104, 200), (256, 256)),    # FP16 256 x 256 tiles, 128-bit rows, ragged M/N/K
    (True, (2047, 4095, 200), (128, 128)),    # FP16 128 x 128 tiles, register-staged (unaligned rows)
    (True, (3000, 3080, 200), (256, 256)),    # FP16 256 x 256 ring with 156 tiles
    (True, (1000, 1000, 1000), (128, 128)),   # FP16 128 x 128 ring
    (True, (1000, 1001, 1000), (64, 64)),     # FP16 64 x 64 tiles (unaligned rows)
    ("bf16", (8000, 4104, 200), (256, 256)),  # BF16 ring, ragged M/N/K
    ("bf16", (8191, 4097, 72), (256, 256)),   # BF16 256 x 256, unaligned rows
    ("bf16", (2047, 4095, 200), (128, 128)),  # BF16 128 x 128 tiles, register-staged
    ("bf16", (1000, 1000, 1000), (128, 128)), # BF16 128 x 128 ring
    ("bf16", (1000, 1001, 1000), (64, 64)),   # BF16 64 x 64 tiles
]


@pytest.mark.parametrize("half,shape,tile", CONFIG_SHAPES,
                         ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) else str(v))
def test_every_matrix_core_configuration(half, shape, tile):
    M, N, K = shape
    p = dg.plan(half, M, N, K)
    assert (p["tile_m"], p["tile_n"]) == tile
    say("auto", _fmt(half), shape, "tile", tile)
    A, B = ints(M, N, K, 21, half)
    ref = oracle_gemm(A, B)
    assert_bits_equal(run(half, dg.AUTO, A, B), ref, f"ints {shape}")
    A, B = floats(M, N, K, 22, half)
    ref = oracle_gemm(A, B)
    tol = tol_f16(K, ref) if half else tol_f32(K)
    assert_within(run(half, dg.AUTO, A, B), ref, tol, f"floats {shape}")


# The large FP16 tile runs a ring of k-stages (32 deep) whose prologue and
# drain differ with the stage count: these K give 1, 1, 2, 2, 3, 3, 4 and 5
# stages, full and ragged, on a shape with ragged M and N that takes the tile.
@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("K", [8, 32, 40, 64, 72, 96, 104, 136])
def test_f16_large_tile_stage_counts(K, fmt):
    M, N = 8000, 4104
    p = dg.plan(True, M, N, K)
    assert (p["tile_m"], p["tile_n"]) == (256, 256)
    say(fmt, "large tile stages", (M, N, K))
    A, B = ints(M, N, K, 61 + K, fmt)
    assert_bits_equal(run(fmt, dg.AUTO, A, B), oracle_gemm(A, B), f"ints K={K}")
    A, B = floats(M, N, K, 62 + K, fmt)
    ref = oracle_gemm(A, B)
    assert_within(run(fmt, dg.AUTO, A, B), ref, tol_f16(K, ref), f"floats K={K}")


# The 128 x 128 16-bit ring: the same stage counts on shapes with ragged M
# and N that take it, with one group of wavefronts (2000 x 2056: 272 tiles)
# and with two groups over halves of the k-stages (1000 x 1032: 64 tiles;
# K = 8 .. 40 leave the second group no stage, or one past K; K = 2088 gives
# 33 + 33 stages with a tail).
@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("M,N,K,groups", [(2000, 2056, K, 1) for K in (8, 32, 40, 64, 72, 96, 104, 136)]
                         + [(1000, 1032, K, 2) for K in (8, 32, 40, 64, 72, 96, 104, 136, 1000, 2088)])
def test_f16_mid_tile_ring_stage_counts(M, N, K, groups, fmt):
    p = dg.plan(True, M, N, K)
    assert (p["tile_m"], p["tile_n"], p["threads"], p["lds_bytes"]) == (128, 128, 256 * groups, 81920 * groups)
    say(fmt, "128 x 128 ring stages", (M, N, K), groups)
    A, B = ints(M, N, K, 63 + K, fmt)
    assert_bits_equal(run(fmt, dg.AUTO, A, B), oracle_gemm(A, B), f"ints K={K}")
    A, B = floats(M, N, K, 64 + K, fmt)
    ref = oracle_gemm(A, B)
    assert_within(run(fmt, dg.AUTO, A, B), ref, tol_f16(K, ref), f"floats K={K}")


# The large FP32 tile runs the same kind of ring with 16-deep stages: these K
# give 1, 1, 2, 2, 3, 3, 4 and 5 stages, full and ragged.
@pytest.mark.parametrize("K", [4, 16, 20, 32, 36, 48, 52, 68])
def test_f32_large_tile_stage_counts(K):
    M, N = 4000, 4092
    p = dg.plan(False, M, N, K)
    assert (p["tile_m"], p["tile_n"]) == (256, 256)
    say("f32 large tile stages", (M, N, K))
    A, B = ints(M, N, K, 71 + K)
    assert_bits_equal(run(False, dg.AUTO, A, B), oracle.gemm_f32(A, B), f"ints K={K}")
    A, B = floats(M, N, K, 72 + K)
    assert_within(run(False, dg.AUTO, A, B), oracle.gemm_f32(A, B), tol_f32(K), f"floats K={K}")


# The 64 x 64 FP32 tile with 128-bit operands runs a ring of four 32-deep
# stages, three loaded ahead: these K give 1, 1, 2, 3, 3, 4, 5, 7, 9 and 11
# stages, full and ragged; the shapes have ragged M and N (1000 = 15 x 64 +
# 40), fewer rows than one tile, and a single row.
@pytest.mark.parametrize("shape", [(1000, 1000, K) for K in (4, 32, 64, 68, 96, 128, 160, 196, 260, 324)]
                         + [(40, 1000, 200), (1, 1024, 128), (1000, 8, 64)],
                         ids=lambda s: "x".join(map(str, s)))
def test_f32_mid_tile_stage_counts(shape):
    M, N, K = shape
    p = dg.plan(False, M, N, K)
    if N > 64:
        assert (p["tile_m"], p["tile_n"], p["tile_k"], p["lds_stages"]) == (64, 64, 32, 4)
    say("f32 mid tile stages", shape)
    A, B = ints(M, N, K, 81 + K)
    assert_bits_equal(run(False, dg.AUTO, A, B), oracle.gemm_f32(A, B), f"ints {shape}")
    A, B = floats(M, N, K, 82 + K)
    assert_within(run(False, dg.AUTO, A, B), oracle.gemm_f32(A, B), tol_f32(K), f"floats {shape}")


# With at most 256 such tiles and K >= 512 the 64 x 64 ring's workgroup is
# two groups of eight wavefronts, each over half of the k-stages: these K
# give 16 + 16, 17 + 17 (the second group's last stage past K), 32 + 32 and
# 33 + 33 stages, and 65 + 65 with a k tail; ragged M and N, one row of
# tiles, a single row.
@pytest.mark.parametrize("shape", [(1000, 1000, K) for K in (512, 528, 1000, 1040, 2084)]
                         + [(40, 1000, 600), (1, 1024, 512), (1024, 1024, 1024)],
                         ids=lambda s: "x".join(map(str, s)))
def test_f32_mid_tile_split_over_k(shape):
    M, N, K = shape
    p = dg.plan(False, M, N, K)
    assert (p["tile_m"], p["tile_n"], p["threads"], p["lds_bytes"]) == (64, 64, 1024, 131072)
    say("f32 mid tile, two groups over k", shape)
    A, B = ints(M, N, K, 91 + K)
    assert_bits_equal(run(False, dg.AUTO, A, B), oracle.gemm_f32(A, B), f"ints {shape}")
    A, B = floats(M, N, K, 92 + K)
    assert_within(run(False, dg.AUTO, A, B), oracle.gemm_f32(A, B), tol_f32(K), f"floats {shape}")


# Tall, narrow FP32 problems (N <= 64, K <= 1024) take a kernel of 16-row
# workgroups that load A and B straight into registers and split K eight
# ways: N across 1..4 column blocks (ragged, and N % 16 == 1 with its last
# column on the vector ALUs), K from 1 to 1024 (K not a multiple of 4, fewer
# slices than wavefronts, uneven runs), the last row spread over the
# workgroups (M % 16 == 1 with at least N whole blocks) or in a block of its
# own, more than 256 workgroups, fewer rows than a block, and base pointers
# one float off 16-byte alignment (the kernel needs 4-byte alignment only;
# there B goes straight into registers instead of being copied into LDS).
NARROW_SHAPES = [(4100, 33, 777), (4097, 33, 777), (4097, 1, 1), (300, 16, 17), (257, 17, 3),
                 (5000, 48, 64), (1000, 63, 600), (4097, 64, 576), (9, 40, 900), (16, 15, 5),
                 (4096, 2, 1024), (8193, 49, 1023), (33, 17, 130), (17, 33, 5), (4097, 64, 1024),
                 (529, 33, 1), (513, 17, 999)]


@pytest.mark.parametrize("shape", NARROW_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_f32_tall_narrow(shape):
    M, N, K = shape
    p = dg.plan(False, M, N, K)
    fringe = N > 16 and N % 16 == 1
    assert p["tile_n"] == (16 * (N // 16) + 1 if fringe else 16 * -(-N // 16))
    assert p["tile_m"] == 16 and p["grid_x"] == 1 and p["threads"] == 512
    tail = M % 16 == 1 and M // 16 >= N
    assert p["grid_y"] == M // 16 + (1 if M % 16 and not tail else 0)
    nb = N // 16 if fringe else -(-N // 16)
    assert p["lds_stages"] == {1: 8, 2: 8, 3: 4, 4: 3}[nb] and p["tile_k"] == 16 * -(-K // 16)
    say("f32 tall narrow", shape)
    A, B = ints(M, N, K, 91)
    assert_bits_equal(run(False, dg.AUTO, A, B), oracle.gemm_f32(A, B), f"ints {shape}")
    A, B = floats(M, N, K, 92)
    ref = oracle.gemm_f32(A, B)
    assert_within(run(False, dg.AUTO, A, B), ref, tol_f32(K), f"floats {shape}")
    # the same through base pointers 4 bytes past 16-byte alignment
    import torch
    a = torch.from_numpy(np.concatenate([np.zeros(1, np.float32), A.ravel()])).to("cuda")
    b = torch.from_numpy(np.concatenate([np.zeros(1, np.float32), B.ravel()])).to("cuda")
    c = torch.empty(M * N + 1, dtype=torch.float32, device="cuda")
    assert binding.raw_gemm("f32", None, M, N, K, a.data_ptr() + 4, b.data_ptr() + 4, c.data_ptr() + 4,
                            None) == binding.GEMM_OK
    torch.cuda.synchronize()
    assert_within(c.cpu().numpy()[1:].reshape(M, N), ref, tol_f32(K), f"misaligned {shape}")


# ------------------------------------------------------ full-size workloads --

FULL = ["f32_256", "f32_1024", "f32_1000", "f32_4097x33x777"]
SAMPLED = ["f32_4096", "f16_8192", "bf16_8192"]


def _gpu_full(name, integer):
    w = inputs.WORKLOADS[name]
    A, B = workload(name, integer)
    return run(w.dtype == "f16", dg.AUTO, A, B)


@pytest.mark.parametrize("name", FULL)
def test_workload_full_compare(name):
    w = inputs.WORKLOADS[name]
    say("workload", name, "integer")
    assert_bits_equal(_gpu_full(name, True), oracle_full(name, True), f"{name} ints")
    say("workload", name, w.dist)
    assert_within(_gpu_full(name, False), oracle_full(name, False), tol_f32(w.K), name)


@pytest.mark.parametrize("name", FULL)
def test_ladder_rungs_on_workloads(name):
    w = inputs.WORKLOADS[name]
    A, B = workload(name, False)
    ref = oracle_full(name, False)
    for v in dg.F32_VARIANTS:
        say("workload", name, dg.variant_name(v))
        assert_within(run(False, v, A, B), ref, tol_f32(w.K), f"{name} {dg.variant_name(v)}")


def _invariant_vector(N, seed):
    rng = np.random.default_rng(seed)
    return rng.choice(np.array([-1.0, 1.0], np.float32), N).astype(np.float32)


@pytest.mark.parametrize("name", SAMPLED)
def test_workload_sampled_and_invariant(name):
    w = inputs.WORKLOADS[name]
    half = w.dtype != "f32"
    rows, cols = inputs.sample_indices(w.M, w.N, 4096, seed=w.seed + 7)

    # integer variant: every output is an exact integer
    say("workload", name, "integer")
    A, B = workload(name, True)
    C = _gpu_full(name, True)
    assert_bits_equal(C[rows, cols], oracle_at(A, B, rows, cols), f"{name} ints sampled")
    v = _invariant_vector(w.N, w.seed)
    v_in = {"f32": v, "f16": v.astype(np.float16), "bf16": inputs.to_bf16_bits(v)}[w.dtype]
    Bv = oracle_gemm(B, v_in.reshape(-1, 1))
    ABv = oracle.gemm_f32(as_f32(A), Bv)                     # exact: |A B v| < 2^24 below
    assert np.max(np.abs(ABv)) < 2 ** 24
    Cv = C.astype(np.float64) @ v.astype(np.float64)
    assert_bits_equal(Cv.reshape(-1, 1), ABv.astype(np.float64), f"{name} C v = A (B v)")
    del C

    say("workload", name, w.dist)
    A, B = workload(name, False)
    C = _gpu_full(name, False)
    ref = oracle_at(A, B, rows, cols)
    tol = tol_f16(w.K, ref) if half else tol_f32(w.K)
    assert_within(C[rows, cols], ref, tol, f"{name} sampled")
    if half:  # report whether the much tighter FP32-path bound also holds
        err = float(np.max(np.abs(C[rows, cols] - ref)))
        print(f"{name}: sampled max |dC| = {err:.3e} (FP32-path bound 2e-6 K = {tol_f32(w.K):.3e})")


# -------------------------------------------------------------- edge cases --

_ENTRY = {"f32": dg.gemm_f32, "f16": dg.gemm_f16_f32acc, "bf16": dg.gemm_bf16_f32acc}
_ENTRY_VARIANT = {"f32": dg.gemm_f32_variant, "f16": dg.gemm_f16_f32acc_variant,
                  "bf16": dg.gemm_bf16_f32acc_variant}


@pytest.mark.parametrize("half", [False, True, "bf16"])
def test_k0_writes_zeros_and_empty_m_n_write_nothing(half):
    import torch
    fmt = _fmt(half)
    say("edge K=0 / M=0 / N=0", fmt)
    dt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[fmt]
    a = torch.empty((5, 0), dtype=dt, device="cuda")
    b = torch.empty((0, 7), dtype=dt, device="cuda")
    c = torch.full((5, 7), float("nan"), device="cuda")
    _ENTRY[fmt](a, b, c)
    torch.cuda.synchronize()
    assert torch.equal(c.cpu(), torch.zeros(5, 7))
    sentinel = torch.full((4,), 3.0, device="cuda")
    fn = binding.raw_gemm
    A = torch.ones(16, dtype=dt, device="cuda")
    assert fn(fmt, None, 0, 4, 4, A.data_ptr(), A.data_ptr(), sentinel.data_ptr(), None) == 0
    assert fn(fmt, None, 4, 0, 4, A.data_ptr(), A.data_ptr(), sentinel.data_ptr(), None) == 0
    torch.cuda.synchronize()
    assert torch.equal(sentinel.cpu(), torch.full((4,), 3.0))


@pytest.mark.parametrize("half", [False, True, "bf16"])
def test_misaligned_base_pointers_take_the_narrow_path(half):
    import torch
    M, N, K = 130, 136, 264
    fmt = _fmt(half)
    say("edge misaligned", fmt, (M, N, K))
    A, B = ints(M, N, K, 31, half)
    ref = oracle_gemm(A, B)
    a_big = to_dev(np.concatenate([np.zeros(1, A.dtype), A.ravel()]))
    b_big = to_dev(np.concatenate([np.zeros(1, B.dtype), B.ravel()]))
    c_big = torch.zeros(M * N + 1, device="cuda")
    a, b, c = a_big[1:].view(M, K), b_big[1:].view(K, N), c_big[1:].view(M, N)
    assert a.data_ptr() % 16 and b.data_ptr() % 16 and c.data_ptr() % 16
    p = dg.plan(half, M, N, K, A=a.data_ptr(), B=b.data_ptr(), C=c.data_ptr())
    assert p["vector_a"] == 0 and p["vector_b"] == 0
    variants = dg.F16_VARIANTS if half else dg.F32_VARIANTS
    for v in variants:
        c.zero_()
        _ENTRY_VARIANT[fmt](v, a, b, c)
        torch.cuda.synchronize()
        assert_bits_equal(c.cpu().numpy(), ref, f"misaligned {dg.variant_name(v)}")
    assert c_big[0].item() == 0.0   # nothing written before C


def test_non_default_stream_and_determinism():
    import torch
    M, N, K = 1000, 1000, 1000
    say("edge stream", (M, N, K))
    A, B = floats(M, N, K, 41)
    a, b = to_dev(A), to_dev(B)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        c1 = dg.gemm_f32(a, b)
        c2 = dg.gemm_f32(a, b)
    s.synchronize()
    assert torch.equal(c1, c2)                  # same bits run to run
    assert_within(c1.cpu().numpy(), oracle.gemm_f32(A, B), tol_f32(K), "stream")
    A16, B16 = floats(M, N, K, 42, half=True)
    h1 = dg.gemm_f16_f32acc(to_dev(A16), to_dev(B16), stream=s)
    h2 = dg.gemm_f16_f32acc(to_dev(A16), to_dev(B16), stream=s)
    s.synchronize()
    assert torch.equal(h1, h2)
    # FP8 on the 128 x 128 ring with two groups over k (their FP32 sums
    # added in a fixed order): the same bits run to run as well
    E = inputs.matrices(1000, 1008, 1024, 43, "uniform", "e4m3")
    assert dg.plan("e4m3", 1000, 1008, 1024)["threads"] == 512
    ea = torch.from_numpy(E[0]).to("cuda").view(torch.float8_e4m3fn)
    eb = torch.from_numpy(E[1]).to("cuda").view(torch.float8_e4m3fn)
    f1 = dg.gemm_e4m3_f32acc(ea, eb, stream=s)
    f2 = dg.gemm_e4m3_f32acc(ea, eb, stream=s)
    s.synchronize()
    assert torch.equal(f1, f2)


def test_concurrent_calls_from_threads_on_their_own_streams():
    """The ABI's calls are thread-safe and may overlap on different streams:
    eight host threads, each with its own stream and its own shape (every
    FP32 and 16-bit path the planner has), call the library 20 times each at
    once (ctypes drops the GIL around the call); every result must equal the
    oracle's bit for bit (integer inputs)."""
    import threading
    import torch
    shapes = [(4096, 4096, 16, "f32"), (1024, 1024, 256, "f32"), (4097, 33, 777, "f32"), (2049, 1000, 100, "f32"),
              (300, 200, 100, "f32"), (8192, 4096, 32, "f16"), (1000, 1000, 200, "bf16"), (513, 257, 129, "f16")]
    cases = []
    for i, (M, N, K, fmt) in enumerate(shapes):
        A, B = inputs.matrices(M, N, K, 8100 + i, "int", fmt)
        cases.append((fmt, M, N, K, to_dev(A), to_dev(B), oracle_gemm(A, B)))
    torch.cuda.synchronize()
    fns = {"f32": dg.gemm_f32, "f16": dg.gemm_f16_f32acc, "bf16": dg.gemm_bf16_f32acc}
    results, errors = [None] * len(cases), []

    def worker(i):
        try:
            fmt, M, N, K, a, b, _ = cases[i]
            s = torch.cuda.Stream()
            outs = [torch.empty((M, N), device="cuda") for _ in range(2)]
            for r in range(20):
                fns[fmt](a, b, outs[r % 2], stream=s)
            s.synchronize()
            results[i] = [o.cpu().numpy() for o in outs]
        except Exception as e:   # reported in the main thread
            errors.append((i, repr(e)))

    say("concurrent threads", len(cases))
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=100)
    assert not any(t.is_alive() for t in threads), "a worker did not finish"
    assert not errors, errors
    for (fmt, M, N, K, _, _, ref), outs in zip(cases, results):
        for o in outs:
            assert_bits_equal(o, ref, f"concurrent {fmt} {(M, N, K)}")


def test_k1_is_a_single_rounded_product():
    M, N = 70, 90
    say("edge K=1")
    A, B = floats(M, N, 1, 51)
    expect = A * B            # one correctly rounded binary32 product
    for v in dg.F32_VARIANTS:
        assert_bits_equal(run(False, v, A, B), expect, f"K=1 {dg.variant_name(v)}")


def test_error_paths_on_the_gpu():
    import torch
    say("edge error paths")
    x = torch.ones(64, device="cuda")
    p = x.data_ptr()
    raw = binding.raw_gemm
    assert raw(False, None, -1, 2, 2, p, p, p, None) == binding.GEMM_ERR_INVALID_DIM
    assert raw(False, None, 2, 2, 2, None, p, p, None) == binding.GEMM_ERR_NULL_PTR
    assert raw(True, 3, 2, 2, 2, p, p, p, None) == binding.GEMM_ERR_INVALID_VARIANT
    with pytest.raises(dg.GemmError):
        dg.gemm_f32_variant(7, x.view(8, 8), x.view(8, 8))
    with pytest.raises(TypeError):
        dg.gemm_f32(x.view(8, 8).half(), x.view(8, 8).half())
    with pytest.raises(ValueError):
        dg.gemm_f32(x.view(8, 8), x[:56].view(7, 8))
