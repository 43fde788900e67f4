"""GPU parity of the convolution entry points (im2col + GEMM) against the
oracle's direct convolution ("Lesson 8: how a GPU does matrix multiply",
next lesson: convolution as matrix multiplication, direct against im2col).

Bars: small-integer inputs (values in {-4..4}) bit-exact for every format
(every partial sum is an integer below 2^24); otherwise the GEMM bars with
the reduction length CRS = C R S in place of K: FP32 |dy| <= 2e-6 CRS for
inputs in [-1, 1), 16-bit |dy| <= 2e-3 sqrt(CRS) max|y_ref|.  Shapes cover
stride, padding, dilation, rectangular filters and images, a reduction
length that is not a multiple of 8 (padded inside the workspace), and
layer-sized cases that take the matrix-core tiles.
"""
import numpy as np
import pytest

import dense_gemm_optimisation_row_amd as dg
from dense_gemm_optimisation_row_amd import binding, inputs

import oracle
from helpers import say, tol_f16, tol_f32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU (run the CPU suite with -m 'not gpu')")
    binding.load()
    return torch.device("cuda")


def draw(fmt, shape, seed, dist):
    """Seeded tensor in the input format (drawn as an M x K matrix and reshaped)."""
    n = int(np.prod(shape))
    A, _ = inputs.matrices(1, 1, n, seed, dist, fmt)
    return A.reshape(shape)


def to_dev(a):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to("cuda")
    return torch.from_numpy(a).to("cuda")


def run(fmt, x, w, st, pd, dl):
    import torch
    y = dg.conv2d(fmt, to_dev(x), to_dev(w), st, pd, dl)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def check(fmt, got, ref, crs, integer, what):
    assert got.shape == ref.shape, what
    if integer:
        bad = got != ref
        assert not bad.any(), f"{what}: {int(bad.sum())} elements differ, first {np.argwhere(bad)[0]}"
        return
    assert np.all(np.isfinite(got)), what
    tol = tol_f32(crs) if fmt == "f32" else tol_f16(crs, ref)
    err = float(np.max(np.abs(got.astype(np.float64) - ref))) if got.size else 0.0
    assert err <= tol, f"{what}: max |dy| {err:.3e} > {tol:.3e}"


SMALL = [
    # (N, C, H, W, K, R, S, stride, pad, dil)
    (1, 1, 5, 5, 1, 3, 3, (1, 1), (0, 0), (1, 1)),
    (2, 3, 7, 6, 4, 3, 2, (2, 1), (1, 0), (1, 2)),
    (1, 4, 9, 9, 5, 3, 3, (1, 1), (1, 1), (1, 1)),
    (3, 2, 8, 11, 3, 5, 3, (2, 3), (2, 1), (1, 1)),
    (2, 5, 10, 7, 2, 2, 4, (1, 2), (0, 2), (2, 1)),
    (1, 3, 6, 6, 6, 1, 1, (2, 2), (0, 0), (1, 1)),
    (2, 3, 32, 32, 16, 3, 3, (1, 1), (1, 1), (1, 1)),     # CRS 27: padded to 32
    (4, 16, 17, 13, 24, 3, 3, (2, 2), (1, 1), (1, 1)),
]
LAYERS = [
    (8, 64, 56, 56, 64, 3, 3, (1, 1), (1, 1), (1, 1)),    # a 56 x 56 stage
    (4, 128, 28, 28, 256, 3, 3, (2, 2), (1, 1), (1, 1)),  # a strided transition
    (16, 256, 14, 14, 256, 1, 1, (1, 1), (0, 0), (1, 1)), # a 1 x 1 projection
    (2, 3, 224, 224, 64, 7, 7, (2, 2), (3, 3), (1, 1)),   # a 7 x 7 stem (CRS 147)
    (2, 3, 96, 96, 256, 7, 7, (2, 2), (3, 3), (1, 1)),    # split-K with a ragged last chunk (CRSp 152)
]


def _case(fmt, case, seed, integer):
    N, C, H, W, K, R, S, st, pd, dl = case
    dist = "int" if integer else "uniform"
    x = draw(fmt, (N, C, H, W), seed, dist)
    w = draw(fmt, (K, C, R, S), seed + 1, dist)
    what = f"{fmt} {case[:7]} st{st} pd{pd} dl{dl} int={integer}"
    say("conv", what)
    ref = oracle.conv2d(fmt, x, w, st, pd, dl).astype(np.float64)
    check(fmt, run(fmt, x, w, st, pd, dl), ref, C * R * S, integer, what)


@pytest.mark.parametrize("fmt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("case", SMALL, ids=lambda c: "x".join(map(str, c[:7])))
def test_conv2d_small(fmt, case):
    _case(fmt, case, 5100, True)
    _case(fmt, case, 5200, False)


@pytest.mark.parametrize("fmt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("case", LAYERS, ids=lambda c: "x".join(map(str, c[:7])))
def test_conv2d_layers(fmt, case):
    _case(fmt, case, 5300, True)
    _case(fmt, case, 5400, False)


# 16-bit layers with C not a multiple of 32 whose implicit-GEMM tiles (128
# filters x 256 pixels) number at least 256, so they take the gathering
# implicit-GEMM kernels (no im2col matrix):
# BM = 64 and 128 (K <= 64 and K > 64, ragged), C R S a multiple of 8 (W used
# as it is) and not (padded copy), stride, dilation and a 1 x 1 filter, and
# NPQ not a multiple of 256.  Stride 1 along w with Q a multiple of 4 takes
# the vector gather from the padded copy of x (marked vec), the rest the
# element gather.  Few channels keep the oracle quick.
IGEMM = [
    (32, 8, 56, 56, 16, 3, 3, (1, 1), (1, 1), (1, 1)),      # vec, CRS 72, K 16
    (30, 3, 58, 57, 40, 3, 3, (1, 1), (1, 1), (1, 1)),      # Q 57: CRS 27 (padded), NPQ 99180
    (16, 16, 66, 66, 200, 3, 3, (1, 1), (1, 1), (1, 1)),    # Q 66: K 200, two 128-filter tiles
    (16, 8, 130, 130, 24, 5, 5, (2, 2), (2, 2), (1, 1)),    # stride 2, 5 x 5
    (8, 4, 128, 128, 33, 3, 3, (1, 1), (2, 2), (2, 2)),     # vec, dilation 2
    (64, 24, 32, 32, 64, 1, 1, (1, 1), (0, 0), (1, 1)),     # vec, 1 x 1, CRS 24
    (16, 3, 64, 64, 96, 3, 3, (1, 1), (1, 1), (1, 1)),      # vec, K 96 on the 128 tile, CRS 27
    (16, 4, 130, 64, 48, 3, 3, (2, 1), (1, 1), (1, 1)),     # vec, stride 2 along h only
    (16, 4, 64, 63, 40, 2, 2, (1, 1), (1, 1), (1, 1)),      # vec, odd W: odd padded rows
    (16, 8, 64, 64, 130, 3, 3, (1, 1), (1, 1), (1, 1)),     # vec, K 130: a 2-filter second tile
    (16, 8, 62, 62, 128, 1, 1, (1, 1), (1, 1), (1, 1)),     # vec, padded copy above the im2col size
    (16, 5, 64, 65, 40, 2, 4, (1, 1), (1, 1), (1, 1)),      # vec, S 4, odd W, 2 filter rows
    (20, 4, 60, 61, 64, 5, 4, (1, 1), (2, 1), (1, 1)),      # vec, S 4, 5 filter rows, pad (2, 1)
    (16, 6, 66, 65, 64, 3, 4, (1, 1), (1, 1), (2, 1)),      # vec, S 4, dilation 2 along h
]


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("case", IGEMM, ids=lambda c: "x".join(map(str, c[:7])))
def test_conv2d_implicit_gemm_layers(fmt, case):
    N, C, H, W, K, R, S, st, pd, dl = case
    prm = binding.conv_params(N, C, H, W, K, R, S, st, pd, dl)
    assert dg.conv2d_algorithm(prm, 2) == dg.CONV_IMPLICIT
    _case(fmt, case, 5500, True)
    _case(fmt, case, 5600, False)


# 16-bit layers with C a multiple of 32 and at least 96 tiles take the
# implicit GEMM on a channels-last copy of x: every tile configuration
# (filters x pixels x k-depth: 64 x 256 x 32 for K <= 64, 128 x 64 x 64 or
# x 32 by C), with ragged filter and pixel tiles, stride, padding and
# dilation along each axis, rectangular filters and images, a 1 x 1 filter,
# C of 32, 64, 96, 128 and 256, and the 14 x 14, 256-channel layer at half
# its batch.
NHWC = [
    ((32, 32, 28, 28, 64, 3, 3, (1, 1), (1, 1), (1, 1)), (64, 256, 32)),
    ((8, 64, 28, 28, 200, 3, 3, (1, 1), (1, 1), (1, 1)), (128, 64, 64)),
    ((64, 96, 30, 29, 64, 3, 2, (2, 1), (1, 0), (1, 2)), (64, 256, 32)),
    ((2, 64, 112, 112, 64, 3, 3, (1, 1), (1, 1), (1, 1)), (64, 256, 32)),
    ((32, 32, 56, 56, 64, 3, 3, (1, 1), (1, 1), (1, 1)), (64, 256, 32)),
    ((16, 64, 30, 30, 130, 1, 1, (1, 1), (0, 0), (1, 1)), (128, 64, 64)),
    ((32, 32, 40, 40, 40, 3, 3, (1, 1), (1, 1), (1, 1)), (64, 256, 32)),
    ((8, 32, 56, 56, 256, 3, 3, (1, 1), (1, 1), (1, 1)), (128, 64, 32)),
    ((16, 64, 56, 56, 64, 3, 3, (1, 1), (1, 1), (1, 1)), (64, 256, 32)),
    ((32, 32, 33, 35, 96, 3, 3, (2, 2), (2, 1), (2, 2)), (128, 64, 32)),
    ((64, 64, 20, 20, 64, 5, 3, (1, 1), (2, 1), (1, 1)), (64, 256, 32)),
    ((16, 96, 20, 20, 100, 3, 3, (1, 1), (1, 1), (1, 1)), (128, 64, 32)),
    ((16, 256, 14, 14, 256, 3, 3, (1, 1), (1, 1), (1, 1)), (128, 64, 64)),
]


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("case,tile", NHWC, ids=lambda c: "x".join(map(str, c[:7])) if len(c) > 3 else "")
def test_conv2d_channels_last_implicit_gemm_layers(fmt, case, tile):
    N, C, H, W, K, R, S, st, pd, dl = case
    prm = binding.conv_params(N, C, H, W, K, R, S, st, pd, dl)
    assert dg.conv2d_algorithm(prm, 2) == dg.CONV_IMPLICIT_NHWC
    _case(fmt, case, 5800, True)
    _case(fmt, case, 5900, False)


@pytest.mark.parametrize("name", list(inputs.CONV_WORKLOADS))
def test_conv_workloads_in_full(name):
    """The benchmarked convolution layers, every output, on their own draw and
    on small integers (bit-exact)."""
    w = inputs.CONV_WORKLOADS[name]
    case = (w.N, w.C, w.H, w.W, w.K, w.R, w.S, (w.stride, w.stride), (w.pad, w.pad), (1, 1))
    x, wt = inputs.conv_tensors(w)
    say("conv workload", name)
    st, pd = (w.stride, w.stride), (w.pad, w.pad)
    ref = oracle.conv2d(w.dtype, x, wt, st, pd).astype(np.float64)
    check(w.dtype, run(w.dtype, x, wt, st, pd, (1, 1)), ref, w.C * w.R * w.S, False, name)
    _case(w.dtype, case, 6000, True)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("case", [(8, 32, 28, 28, 96, 3, 3, (1, 1), (1, 1), (1, 1)),     # channels last
                                  (32, 8, 56, 56, 16, 3, 3, (1, 1), (1, 1), (1, 1)),     # gather
                                  (1, 4, 9, 9, 5, 3, 3, (1, 1), (1, 1), (1, 1))],        # im2col
                         ids=["nhwc", "gather", "im2col"])
def test_conv2d_inputs_at_odd_element_offsets(fmt, case):
    """x and w handed over as contiguous views that start one element into
    their buffers (2-byte aligned only): every path reads them correctly."""
    import torch
    N, C, H, W, K, R, S, st, pd, dl = case
    x = draw(fmt, (N, C, H, W), 6100, "int")
    w = draw(fmt, (K, C, R, S), 6101, "int")
    xb, wb = to_dev(np.concatenate([x.ravel()[:1], x.ravel()])), to_dev(np.concatenate([w.ravel()[:1], w.ravel()]))
    xv, wv = xb[1:].view(N, C, H, W), wb[1:].view(K, C, R, S)
    assert xv.data_ptr() % 4 == 2 and wv.data_ptr() % 4 == 2
    say("conv odd offsets", fmt, case)
    y = dg.conv2d(fmt, xv, wv, st, pd, dl)
    torch.cuda.synchronize()
    ref = oracle.conv2d(fmt, x, w, st, pd, dl)
    check(fmt, y.cpu().numpy(), ref.astype(np.float64), C * R * S, True, f"odd offsets {case}")


@pytest.mark.parametrize("fmt", ["f32", "f16"])
def test_conv2d_zero_channels_and_empty_batch(fmt):
    import torch
    say("conv edges", fmt)
    dt = torch.float32 if fmt == "f32" else torch.float16
    x = torch.empty((2, 0, 6, 6), dtype=dt, device="cuda")
    w = torch.empty((3, 0, 3, 3), dtype=dt, device="cuda")
    y = torch.full((2, 3, 4, 4), 7.0, device="cuda")
    dg.conv2d(fmt, x, w, y=y)
    torch.cuda.synchronize()
    assert torch.count_nonzero(y).item() == 0          # an empty sum
    x = torch.empty((0, 2, 6, 6), dtype=dt, device="cuda")
    w = torch.ones((3, 2, 3, 3), dtype=dt, device="cuda")
    assert dg.conv2d(fmt, x, w).numel() == 0


def test_conv2d_workspace_errors_on_the_gpu():
    import torch
    say("conv workspace errors")
    x = torch.ones((1, 2, 6, 6), device="cuda")
    w = torch.ones((3, 2, 3, 3), device="cuda")
    y = torch.empty((1, 3, 4, 4), device="cuda")
    p = binding.conv_params(1, 2, 6, 6, 3, 3, 3)
    need = dg.conv2d_workspace(p, 4)
    ws = torch.empty(need + 512, dtype=torch.uint8, device="cuda")
    rc = binding.raw_conv2d("f32", p, x.data_ptr(), w.data_ptr(), y.data_ptr(), ws.data_ptr(), need - 1, None)
    assert rc == binding.GEMM_ERR_WORKSPACE
    rc = binding.raw_conv2d("f32", p, x.data_ptr(), w.data_ptr(), y.data_ptr(), ws.data_ptr() + 8, need, None)
    assert rc == binding.GEMM_ERR_WORKSPACE
    rc = binding.raw_conv2d("f32", p, x.data_ptr(), w.data_ptr(), y.data_ptr(), ws.data_ptr(), need, None)
    torch.cuda.synchronize()
    assert rc == binding.GEMM_OK and torch.all(y == 18.0).item()


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("case", [(32, 8, 56, 56, 16, 3, 3, (1, 1), (1, 1), (1, 1)),
                                  (8, 32, 28, 28, 96, 3, 3, (1, 1), (1, 1), (1, 1))], ids=["gather", "nhwc"])
def test_conv2d_implicit_gemm_inf_reaches_only_its_outputs(fmt, case):
    """An infinite input element on an implicit-GEMM layer (vector gather:
    the wide loads also fetch elements outside each pixel's taps, which must
    never enter a product; channels last: the copy's zero border and the
    stage's channel run) makes exactly the outputs whose receptive field
    covers it infinite, as in the direct convolution; every other output
    stays finite and exact (small-integer inputs, positive weights)."""
    N, C, H, W, K, R, S, st, pd, dl = case
    assert dg.conv2d_algorithm(binding.conv_params(N, C, H, W, K, R, S, st, pd, dl), 2) in (
        dg.CONV_IMPLICIT, dg.CONV_IMPLICIT_NHWC)
    say("conv inf", fmt, case)
    x = draw(fmt, (N, C, H, W), 5700, "int").copy()
    vals = np.random.default_rng(5701).integers(1, 5, (K, C, R, S)).astype(np.float32)
    # weights 1..4 (bfloat16: the top half of the binary32 bits, exact here)
    w = vals.astype(np.float16) if fmt == "f16" else (vals.view(np.uint32) >> 16).astype(np.uint16)
    inf = np.float16(np.inf) if fmt == "f16" else np.uint16(0x7F80)
    x[3, min(5, C - 1), 20, 27] = inf
    x[7, 0, 0, 0] = inf        # the first element of an image: a top-left corner
    ref = oracle.conv2d(fmt, x, w, st, pd, dl).astype(np.float64)
    got = run(fmt, x, w, st, pd, dl)
    assert np.isposinf(ref).sum() > 0
    assert np.array_equal(np.isposinf(got), np.isposinf(ref)) and not np.isnan(got).any()
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
