"""Race check of the kernels that load tiles straight from global memory into
LDS, through the LDS-poisoning build of the library (libdgor_gemm_poison.so:
the same sources compiled with -DDGOR_LDS_POISON).

In that build every global->LDS load first fills the bytes it is about to
write with all-ones -- a NaN in FP32, FP16, BF16 and both FP8 formats, -1 in
INT8 -- after the barrier that retires the region's last reads.  These loads
are issued from inline assembly that the compiler's wait counters do not see,
and the kernels order them with waits and barriers of their own.  A read that
runs ahead of a barrier (a buffer refilled while a wavefront still reads it,
"Lesson 8: how a GPU does matrix multiply", sections 11 and 12 on why each
barrier exists) or of the wait for a load (a stage read before it landed)
returns the poison instead of the operand, and the product is then NaN or
wrong.  So every case here runs on small-integer inputs and must equal the
oracle bit for bit: the stage-count cases of every ring (one to several
stages, full and ragged, prologue and drain), the transposed-A pipe ring, the
128 x 128 two-stage kernel, the tall, narrow kernel's per-wavefront B copies,
FP32 4096^3 in full, and the channels-last convolution kernel's ring (both
tile configurations, 1 to 9 stages).
"""
import numpy as np
import pytest

from dense_gemm_optimisation_row_amd import binding, build, inputs

import oracle
from helpers import assert_bits_equal, say

pytestmark = pytest.mark.gpu

_ORACLE = {"f32": oracle.gemm_f32, "f16": oracle.gemm_f16, "bf16": oracle.gemm_bf16,
           "e4m3": oracle.gemm_e4m3, "e5m2": oracle.gemm_e5m2, "i8": oracle.gemm_i8}
_STEM = {"f32": "gemm_f32", "f16": "gemm_f16_f32acc", "bf16": "gemm_bf16_f32acc",
         "e4m3": "gemm_e4m3_f32acc", "e5m2": "gemm_e5m2_f32acc", "i8": "gemm_i8_i32acc"}


@pytest.fixture(scope="module")
def lib():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU (run the CPU suite with -m 'not gpu')")
    return binding.load(build.POISON_LIB)   # raises if the poison build is missing


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16) if a.dtype == np.uint16 else
                            np.ascontiguousarray(a)).to("cuda")


def _run(lib, fmt, A, B, trans_a=False):
    """The product through the poisoned library (automatic kernel choice); with
    trans_a, A is passed stored transposed (K x M) through the general-layout
    entry point."""
    import torch
    M, K = A.shape
    N = B.shape[1]
    c = torch.full((M, N), 7, dtype=torch.int32 if fmt == "i8" else torch.float32, device="cuda")
    if trans_a:
        at, b = _dev(np.ascontiguousarray(A.T)), _dev(B)
        rc = getattr(lib, _STEM[fmt] + "_ex")(binding.GEMM_OP_T, binding.GEMM_OP_N, M, N, K, 1.0, at.data_ptr(), M,
                                              b.data_ptr(), N, 0.0, c.data_ptr(), N, None)
    else:
        a, b = _dev(A), _dev(B)
        rc = getattr(lib, _STEM[fmt])(M, N, K, a.data_ptr(), b.data_ptr(), c.data_ptr(), None)
    assert rc == binding.GEMM_OK, binding.status_string(rc)
    torch.cuda.synchronize()
    return c.cpu().numpy()


def _check(lib, fmt, M, N, K, seed, trans_a=False):
    A, B = inputs.matrices(M, N, K, seed, "int", fmt)
    got = _run(lib, fmt, A, B, trans_a)
    assert np.all(np.isfinite(got)) if fmt != "i8" else True, "poison (NaN) reached C"
    assert_bits_equal(got, _ORACLE[fmt](A, B), f"{fmt} {M}x{N}x{K}{' TN' if trans_a else ''} (poisoned LDS)")


# (format, M, N, K list): shapes that take each direct-load kernel, K giving
# one to several of its stages, full and with a ragged last stage
CASES = [
    ("f16", 8000, 4104, [8, 32, 40, 64, 72, 96, 104, 136]),     # 16-bit 256^2 pair ring
    ("bf16", 8000, 4104, [8, 40, 104, 136]),
    ("f16", 1000, 1032, [8, 32, 40, 72, 136, 1000]),            # 16-bit 128^2 ring, two groups over k
    ("bf16", 1000, 1032, [8, 40, 136]),
    ("f16", 2000, 2056, [8, 32, 40, 72, 136]),                  # the same, one group
    ("f32", 4000, 4092, [4, 16, 20, 32, 36, 48, 52, 68]),       # FP32 256^2 ring
    ("f32", 1000, 1000, [32, 64, 96, 128, 200, 384]),           # FP32 64^2 ring (32-deep stages)
    ("f32", 1000, 1000, [512, 528, 1040]),                      # the same, two groups over k
    ("f32", 4000, 2044, [16, 100]),                             # FP32 128^2 two-stage kernel
    ("e4m3", 520, 784, [16, 64, 80, 144, 320]),                 # 8-bit 128^2 rings, two groups over k
    ("e5m2", 520, 784, [16, 80, 208]),
    ("i8", 520, 784, [16, 48, 64, 128, 192, 320]),
    ("e4m3", 2000, 2064, [16, 80, 208]),                        # the same, one group
    ("i8", 2000, 2064, [16, 80, 208]),
    ("e4m3", 4000, 4016, [16, 64, 80, 144, 320]),               # 8-bit 256^2 rings
    ("e5m2", 4000, 4016, [16, 80, 208]),
    ("i8", 4000, 4016, [16, 48, 64, 128, 192, 320]),
    # tall, narrow: one and two column blocks hold a wavefront's B run in LDS;
    # three and four stream it through rings of 4 and 3 slots, where K gives
    # 0 to 8 slices a wavefront, so the prologue, the refills and the drain
    # each run with every count of slices in flight
    ("f32", 4097, 33, [777, 1, 100, 200, 500, 1024]),
    ("f32", 4100, 17, [600]),
    ("f32", 1000, 64, [1024, 300, 40]),
    ("f32", 530, 40, [999]),
    ("f32", 600, 49, [800, 70]),
]


@pytest.mark.parametrize("fmt,M,N,Ks", CASES, ids=lambda v: str(v))
def test_ring_stage_counts_with_poisoned_lds(lib, fmt, M, N, Ks):
    for K in Ks:
        say("poisoned LDS", fmt, (M, N, K))
        _check(lib, fmt, M, N, K, 9100 + K)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_transposed_a_pipe_ring_with_poisoned_lds(lib, fmt):
    for K in (32, 72, 136):
        say("poisoned LDS, A stored transposed", fmt, K)
        _check(lib, fmt, 2056, 4104, K, 9200 + K, trans_a=True)


def test_f32_4096_in_full_with_poisoned_lds(lib):
    say("poisoned LDS", "f32_4096 integer variant in full")
    A, B = inputs.workload_matrices("f32_4096", True)
    assert_bits_equal(_run(lib, "f32", A, B), oracle.gemm_f32(A, B), "f32_4096 ints (poisoned LDS)")


# channels-last convolution layers (16-bit, C a multiple of 32): both tile
# configurations, 1, 2, 3 and 9 stages of their ring, ragged filter tiles
CONV_CASES = [
    (32, 32, 28, 28, 64, 1, 1, (1, 1), (0, 0)),    # 64 x 256 x 32 tiles, 1 stage
    (32, 64, 28, 28, 64, 1, 1, (1, 1), (0, 0)),    # 2 stages
    (32, 32, 28, 28, 48, 3, 3, (1, 1), (1, 1)),    # 9 stages, 48 of 64 filters
    (8, 96, 28, 28, 96, 1, 1, (1, 1), (0, 0)),     # 128 x 64 x 32 tiles, 3 stages
    (8, 64, 28, 28, 200, 3, 3, (1, 1), (1, 1)),    # 128 x 64 x 64 tiles, 9 stages, 2 filter tiles
    (8, 128, 28, 28, 128, 1, 1, (1, 1), (0, 0)),   # 2 stages
    (8, 64, 28, 28, 130, 1, 1, (1, 1), (0, 0)),    # 1 stage, a 2-filter last tile
]


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("case", CONV_CASES, ids=lambda c: "x".join(map(str, c[:7])))
def test_channels_last_conv_with_poisoned_lds(lib, fmt, case):
    import torch
    N, C, H, W, K, R, S, st, pd = case
    prm = binding.conv_params(N, C, H, W, K, R, S, st, pd)
    assert binding.conv2d_algorithm(prm, 2) == binding.CONV_IMPLICIT_NHWC
    say("poisoned LDS, channels-last conv", fmt, case)
    x = inputs.matrices(1, 1, N * C * H * W, 9300 + K, "int", fmt)[0].reshape(N, C, H, W)
    w = inputs.matrices(1, 1, K * C * R * S, 9400 + K, "int", fmt)[0].reshape(K, C, R, S)
    P = (H + 2 * pd[0] - R) // st[0] + 1
    Q = (W + 2 * pd[1] - S) // st[1] + 1
    y = torch.full((N, K, P, Q), 7.0, device="cuda")
    ws = torch.empty(binding.conv2d_workspace(prm, 2), dtype=torch.uint8, device="cuda")
    xd, wd = _dev(x), _dev(w)
    stem = "gemm_conv2d_f16_f32acc" if fmt == "f16" else "gemm_conv2d_bf16_f32acc"
    import ctypes
    rc = getattr(lib, stem)(ctypes.byref(prm), xd.data_ptr(), wd.data_ptr(), y.data_ptr(), ws.data_ptr(),
                            ws.numel(), None)
    assert rc == binding.GEMM_OK, binding.status_string(rc)
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    assert np.all(np.isfinite(got)), "poison (NaN) reached y"
    assert_bits_equal(got, oracle.conv2d(fmt, x, w, st, pd), f"{fmt} conv {case} (poisoned LDS)")
