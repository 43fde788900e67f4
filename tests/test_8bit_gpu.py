"""GPU parity of the 8-bit entry points against the CPU oracle: FP8 (OCP E4M3
and E5M2) with FP32 accumulation, INT8 with INT32 accumulation ("Lesson 8:
how a GPU does matrix multiply", section 22 lists both among the matrix
units' input formats).

Bars (elementwise):
  * INT8: bit-exact, every shape and path (integer sums are exact);
  * FP8 on small-integer inputs ({-4..4}, exact in both FP8 formats): bit-exact,
    every shape and path.  Each product is an integer of magnitude <= 16, so a
    group of eight sums at the matrix unit's fixed point with no bit dropped,
    and every FP32 partial sum is an integer below 2^24;
  * FP8 otherwise: |C - C_ref| <= (2^-9 + 2^-26 K) * S, where S = sum_k |a_ik| |b_kj|
    (the oracle's product of the magnitudes).  The matrix cores add each
    group of eight products at a fixed point aligned to the group's largest
    product, about 13 bits below it (a product 2^14 times smaller than the
    largest of its group is dropped): each group errs by less than
    8 * 2^-13 = 2^-10 of its largest product.  Taken twice over for margin,
    plus FP32 accumulation of the K / 8 group sums (below K 2^-27 S, also
    doubled).  The plain kernel sums in FP32 and meets the same bound.
Shapes span several tiles with ragged M and N edges and a k tail; at most of
those sizes the ring takes 128 x 128 tiles, and its 256 x 256 tiles are
checked separately on shapes that have enough tiles for them.
The 8192^3 workloads are compared in full elsewhere (test_full_gpu.py); here
they get a quick sampled pre-check plus an invariant over every output (C v
against A (B v) for a random +-1 vector v).
"""
import numpy as np
import pytest

import dense_gemm_optimisation_row_amd as dg
from dense_gemm_optimisation_row_amd import binding, inputs

import oracle
from helpers import say

pytestmark = pytest.mark.gpu

FMTS = ["e4m3", "e5m2", "i8"]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU (run the CPU suite with -m 'not gpu')")
    binding.load()
    return torch.device("cuda")


def to_dev(a, fmt):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
    if fmt == "e4m3":
        return t.view(torch.float8_e4m3fn)
    if fmt == "e5m2":
        return t.view(torch.float8_e5m2)
    return t


def run(fmt, variant, A, B):
    import torch
    fn = {"e4m3": dg.gemm_e4m3_f32acc_variant, "e5m2": dg.gemm_e5m2_f32acc_variant,
          "i8": dg.gemm_i8_i32acc_variant}[fmt]
    c = fn(variant, to_dev(A, fmt), to_dev(B, fmt))
    torch.cuda.synchronize()
    return c.cpu().numpy()


def oracle_full(fmt, A, B):
    return {"e4m3": oracle.gemm_e4m3, "e5m2": oracle.gemm_e5m2, "i8": oracle.gemm_i8}[fmt](A, B)


def magnitude_sum(fmt, A, B):
    """S = |A| |B| by the oracle (FP8 codes with the sign bit cleared)."""
    f = oracle.gemm_e4m3 if fmt == "e4m3" else oracle.gemm_e5m2
    return f(A & np.uint8(0x7F), B & np.uint8(0x7F)).astype(np.float64)


def fp8_tol(K, S):
    return (2.0 ** -9 + 2.0 ** -26 * K) * S


def check(fmt, got, A, B, what, exact=False):
    """INT8, and FP8 on small-integer inputs (every product and every partial
    sum an integer far below 2^24, so the matrix unit's fixed-point group sums
    and the FP32 additions are all exact): bit-exact.  FP8 otherwise: the
    bound above."""
    ref = oracle_full(fmt, A, B)
    if fmt == "i8" or exact:
        bad = ~(got == ref)
        assert not bad.any(), f"{what}: {int(bad.sum())} elements differ, first at {np.argwhere(bad)[0]}"
        return
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    S = magnitude_sum(fmt, A, B)
    err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    tol = fp8_tol(A.shape[1], S)
    worst = np.unravel_index(np.argmax(err - tol), err.shape)
    assert np.all(err <= tol), f"{what}: |dC| {err[worst]:.3e} > {tol[worst]:.3e} at {worst}"
    rel = float(np.max(err / np.maximum(S, 1e-30)))
    print(f"[{what}] max |dC| / S = {rel:.2e}")


def mats(fmt, M, N, K, seed, dist="uniform"):
    return inputs.matrices(M, N, K, seed, dist, fmt)


# Multiples of 16 in K and N take R8 (ragged tiles in M and N, k tails of
# 16 .. 48 past a 64-deep step); the rest take R0.
RING_SHAPES = [(16, 16, 16), (64, 48, 64), (256, 256, 256), (300, 272, 80), (513, 528, 144),
               (1000, 1008, 1024), (37, 1040, 48), (1040, 32, 1008)]
PLAIN_SHAPES = [(1, 1, 1), (5, 3, 2), (17, 33, 65), (100, 70, 9), (129, 257, 100)]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape", RING_SHAPES + PLAIN_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_8bit_shapes_both_paths(fmt, shape):
    M, N, K = shape
    for variant in (dg.AUTO, dg.R0_NAIVE):
        plan = dg.plan(fmt, M, N, K, variant=variant)
        say("8bit", fmt, shape, dg.variant_name(plan["variant"]))
        A, B = mats(fmt, M, N, K, 4100)
        check(fmt, run(fmt, variant, A, B), A, B, f"{fmt} {shape} {dg.variant_name(plan['variant'])}")
        A, B = mats(fmt, M, N, K, 4200, "normal")
        check(fmt, run(fmt, variant, A, B), A, B, f"{fmt} {shape} normal")
        A, B = mats(fmt, M, N, K, 4250, "int")
        check(fmt, run(fmt, variant, A, B), A, B, f"{fmt} {shape} int", exact=True)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("K", [16, 48, 64, 80, 128, 144, 192, 208, 320])
def test_8bit_ring_stage_counts(fmt, K):
    # 1 to 5 stages of the four-buffer ring, full and with a k tail
    M, N = 520, 784
    assert dg.plan(fmt, M, N, K)["variant"] == dg.R8_MFMA_8BIT
    say("8bit stages", fmt, K)
    A, B = mats(fmt, M, N, K, 4300 + K)
    check(fmt, run(fmt, dg.AUTO, A, B), A, B, f"{fmt} K={K}")
    A, B = mats(fmt, M, N, K, 4350 + K, "int")
    check(fmt, run(fmt, dg.AUTO, A, B), A, B, f"{fmt} K={K} int", exact=True)


@pytest.mark.parametrize("fmt", FMTS)
def test_8bit_extremes(fmt):
    M, N, K = 264, 272, 1024
    if fmt == "i8":
        # every product at its largest magnitude: C = +-16384 K
        A = np.full((M, K), -128, np.int8)
        B = np.full((K, N), -128, np.int8)
        B[:, ::2] = 127
    else:
        big = 0x7E if fmt == "e4m3" else 0x7B     # largest finite magnitude
        rng = np.random.default_rng(4400)
        A = (rng.integers(0, big + 1, (M, K)) | (rng.integers(0, 2, (M, K)) << 7)).astype(np.uint8)
        B = (rng.integers(0, big + 1, (K, N)) | (rng.integers(0, 2, (K, N)) << 7)).astype(np.uint8)
    say("8bit extremes", fmt)
    for variant in (dg.AUTO, dg.R0_NAIVE):
        check(fmt, run(fmt, variant, A, B), A, B, f"{fmt} extremes {variant}")


@pytest.mark.parametrize("fmt", FMTS)
def test_8bit_k0_empty_and_misaligned(fmt):
    import torch
    say("8bit edges", fmt)
    A, B = mats(fmt, 300, 272, 0, 4500)
    out_dtype = torch.int32 if fmt == "i8" else torch.float32
    c = torch.full((300, 272), 7, dtype=out_dtype, device="cuda")
    fn = {"e4m3": dg.gemm_e4m3_f32acc, "e5m2": dg.gemm_e5m2_f32acc, "i8": dg.gemm_i8_i32acc}[fmt]
    fn(to_dev(A, fmt), to_dev(B, fmt), c)
    torch.cuda.synchronize()
    assert torch.count_nonzero(c).item() == 0
    # misaligned bases (one byte in): the plain kernel, same results
    M, N, K = 300, 272, 80
    A, B = mats(fmt, M, N, K, 4501)
    a = torch.from_numpy(np.concatenate([np.zeros(1, A.dtype), A.ravel()])).to("cuda")
    b = torch.from_numpy(np.concatenate([np.zeros(16, B.dtype), B.ravel()])).to("cuda")
    c = torch.empty((M, N), dtype=out_dtype, device="cuda")
    assert dg.plan(fmt, M, N, K, A=a.data_ptr() + 1, B=b.data_ptr() + 16)["variant"] == dg.R0_NAIVE
    assert binding.raw_gemm(fmt, None, M, N, K, a.data_ptr() + 1, b.data_ptr() + 16, c.data_ptr(),
                            None) == binding.GEMM_OK
    torch.cuda.synchronize()
    check(fmt, c.cpu().numpy(), A, B, f"{fmt} misaligned")
    # INT8 K cap
    if fmt == "i8":
        assert binding.raw_gemm("i8", None, 4, 4, 131073, a.data_ptr(), b.data_ptr(), c.data_ptr(),
                                None) == binding.GEMM_ERR_INVALID_DIM


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("c_off", [1, 3])
def test_8bit_ring_with_c_off_16_byte_alignment(fmt, c_off):
    """The ring with aligned A and B and C starting c_off elements (4 c_off
    bytes) past a 16-byte boundary: the stores fall back to one element at a
    time (the LDS-staged epilogues and the 256 x 256 FP8 kernel's direct
    stores alike).  Ragged tiles; every element around C keeps its sentinel."""
    import torch
    M, N, K = 300, 272, 208
    say("8bit ring, C off 16-byte alignment", fmt, c_off)
    A, B = mats(fmt, M, N, K, 4600 + c_off, "int")
    assert dg.plan(fmt, M, N, K)["variant"] == dg.R8_MFMA_8BIT
    out_dtype = torch.int32 if fmt == "i8" else torch.float32
    buf = torch.full((M * N + 8,), -77, dtype=out_dtype, device="cuda")
    a, b = to_dev(A, fmt), to_dev(B, fmt)
    assert binding.raw_gemm(fmt, None, M, N, K, a.data_ptr(), b.data_ptr(), buf.data_ptr() + 4 * c_off,
                            None) == binding.GEMM_OK
    torch.cuda.synchronize()
    got = buf.cpu().numpy()
    assert np.all(got[:c_off] == -77) and np.all(got[c_off + M * N:] == -77), "a store outside C"
    check(fmt, got[c_off:c_off + M * N].reshape(M, N), A, B, f"{fmt} C offset {c_off}", exact=True)


# Shapes for each ring tile: (M, N, K, tile, groups of wavefronts over k);
# ragged M and N edges, k tails of 16 .. 48 past a 64-deep step, one to many
# steps (with two groups: none or one past K for the second group, and odd
# step counts)
TILE_SHAPES = [(4000, 4016, 16, 256, 1), (4000, 4016, 80, 256, 1), (4000, 4016, 208, 256, 1),
               (4000, 4016, 1040, 256, 1),
               (1000, 1008, 1024, 128, 2), (129, 144, 16, 128, 2), (2000, 1008, 4112, 128, 2), (1000, 1008, 208, 128, 2),
               (2500, 2512, 144, 128, 1), (2000, 2064, 1040, 128, 1), (2000, 2064, 16, 128, 1)]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape", TILE_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_8bit_both_ring_tiles(fmt, shape):
    M, N, K, tile, groups = shape
    plan = dg.plan(fmt, M, N, K)
    assert plan["variant"] == dg.R8_MFMA_8BIT and plan["tile_m"] == tile and plan["threads"] == 256 * groups
    say("8bit ring tile", fmt, tile, (M, N, K))
    A, B = mats(fmt, M, N, K, 4800 + K)
    check(fmt, run(fmt, dg.AUTO, A, B), A, B, f"{fmt} {shape}")
    A, B = mats(fmt, M, N, K, 4850 + K, "int")
    check(fmt, run(fmt, dg.AUTO, A, B), A, B, f"{fmt} {shape} int", exact=True)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("c_off", [1, 3])
def test_8bit_256_ring_with_c_off_16_byte_alignment(fmt, c_off):
    """As the test above, on the 256 x 256 rings."""
    import torch
    M, N, K = 4000, 4016, 80
    say("8bit 256^2 ring, C off 16-byte alignment", fmt, c_off)
    A, B = mats(fmt, M, N, K, 4900 + c_off, "int")
    assert dg.plan(fmt, M, N, K)["tile_m"] == 256
    out_dtype = torch.int32 if fmt == "i8" else torch.float32
    buf = torch.full((M * N + 8,), -77, dtype=out_dtype, device="cuda")
    a, b = to_dev(A, fmt), to_dev(B, fmt)
    assert binding.raw_gemm(fmt, None, M, N, K, a.data_ptr(), b.data_ptr(), buf.data_ptr() + 4 * c_off,
                            None) == binding.GEMM_OK
    torch.cuda.synchronize()
    got = buf.cpu().numpy()
    assert np.all(got[:c_off] == -77) and np.all(got[c_off + M * N:] == -77), "a store outside C"
    check(fmt, got[c_off:c_off + M * N].reshape(M, N), A, B, f"{fmt} 256^2 C offset {c_off}", exact=True)


@pytest.mark.parametrize("name", ["e4m3_8192", "e5m2_8192", "i8_8192"])
def test_8bit_workload_sampled_and_invariant(name):
    """The benchmarked configuration: 8192^3 through the ring, 4096 sampled
    elements against the oracle and C v = A (B v) over every row."""
    import torch
    w = inputs.WORKLOADS[name]
    fmt = w.dtype
    say("8bit workload", name)
    for integer in (False, True):
        A, B = inputs.workload_matrices(w, integer)
        got = run(fmt, dg.AUTO, A, B)
        rows, cols = inputs.sample_indices(w.M, w.N, 4096, 4600)
        if fmt == "i8":
            ref = oracle.gemm_i8_at(A, B, rows, cols)
            assert np.array_equal(got[rows, cols], ref)
        elif integer:   # small integers: exact on the FP8 path too
            at = oracle.gemm_e4m3_at if fmt == "e4m3" else oracle.gemm_e5m2_at
            assert np.array_equal(got[rows, cols], at(A, B, rows, cols))
        else:
            at = oracle.gemm_e4m3_at if fmt == "e4m3" else oracle.gemm_e5m2_at
            ref = at(A, B, rows, cols).astype(np.float64)
            S = at(A & np.uint8(0x7F), B & np.uint8(0x7F), rows, cols).astype(np.float64)
            err = np.abs(got[rows, cols] - ref)
            assert np.all(err <= fp8_tol(w.K, S)), float(np.max(err / S))
            print(f"[{name} int={integer}] sampled max |dC| / S = {float(np.max(err / S)):.2e}")
        # invariant over every output: C v = A (B v), v a random +-1 vector
        v = np.random.default_rng(4700).choice([-1, 1], w.N)
        if fmt == "i8":
            lhs = got.astype(np.int64) @ v
            rhs = A.astype(np.int64) @ (B.astype(np.int64) @ v)
            assert np.array_equal(lhs, rhs)
        else:
            td = torch.float8_e4m3fn if fmt == "e4m3" else torch.float8_e5m2
            Ad = torch.from_numpy(A).view(td).to(torch.float64)
            Bd = torch.from_numpy(B).view(td).to(torch.float64)
            vt = torch.from_numpy(v.astype(np.float64))
            lhs = torch.from_numpy(got.astype(np.float64)) @ vt
            rhs = Ad @ (Bd @ vt)
            # bound: the elementwise bound (plus the oracle's own binary32
            # rounding, as rhs is exact) summed over the row
            Sv = (Ad.abs() @ (Bd.abs() @ torch.ones(w.N, dtype=torch.float64)))
            assert torch.all((lhs - rhs).abs() <= fp8_tol(w.K, Sv) + 2.0 ** -23 * Sv).item()
