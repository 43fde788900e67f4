"""Seeded random sweep over shapes, base alignments, layouts and formats,
every call through the C ABI against the oracle, bit for bit.

The hand-picked parity tests pin each kernel's stage counts and edges; this
sweep draws shapes near the planner's boundaries (multiples of 4, 8, 16, 64
and 256, one above and one below), base pointers on and one element off
16-byte alignment, so that every path the planner can take is crossed with
shapes nobody chose.  Inputs are small integers (values in {-4..4}), whose
products and sums are exact in every format's accumulator, so each output
must equal the oracle's exactly.  Sizes are bounded so the oracle finishes
each case in well under a second.
"""
import numpy as np
import pytest

import dense_gemm_optimisation_row_amd as dg
from dense_gemm_optimisation_row_amd import binding, inputs

import oracle
from helpers import say

pytestmark = pytest.mark.gpu

ELEM = {"f32": 4, "f16": 2, "bf16": 2, "e4m3": 1, "e5m2": 1, "i8": 1}
ORACLE = {"f32": oracle.gemm_f32, "f16": oracle.gemm_f16, "bf16": oracle.gemm_bf16,
          "e4m3": oracle.gemm_e4m3, "e5m2": oracle.gemm_e5m2, "i8": oracle.gemm_i8}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU (run the CPU suite with -m 'not gpu')")
    binding.load()
    return torch.device("cuda")


def _size(rng, lo, hi):
    """A size in [lo, hi]: half the time a multiple of 4, 8, 16, 64 or 256,
    a quarter one away from one, else uniform."""
    u = rng.random()
    if u < 0.75:
        base = int(rng.choice([4, 8, 16, 64, 256]))
        v = base * int(rng.integers(1, max(2, hi // base + 1)))
        if u >= 0.5:
            v += int(rng.choice([-1, 1]))
    else:
        v = int(rng.integers(lo, hi + 1))
    return min(max(v, lo), hi)


# shape families: mid-size (the 64 x 64 and 128 x 128 tiles), wide M N with
# a short K (the 256 x 256 rings), and tall narrow (N <= 64)
FAMILIES = [((1, 2200), (1, 2200), (1, 1100)), ((4000, 6200), (4000, 6200), (1, 12)),
            ((1, 5000), (1, 64), (1, 1100))]


def _shapes(seed, n, max_work):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        (m0, m1), (n0, n1), (k0, k1) = FAMILIES[len(out) % len(FAMILIES)]
        M, N, K = _size(rng, m0, m1), _size(rng, n0, n1), _size(rng, k0, k1)
        if M * N * K <= max_work:
            off = rng.random() < 0.25   # one element off 16-byte alignment
            out.append((M, N, K, int(off and rng.integers(0, 2)), int(off and rng.integers(0, 2))))
    return out


def _dev_flat(a, off):
    """A device byte buffer holding `a` starting `off` elements in."""
    import torch
    raw = np.ascontiguousarray(a).view(np.uint8).ravel()
    buf = np.zeros(raw.size + 16 + off * a.itemsize, np.uint8)
    buf[off * a.itemsize: off * a.itemsize + raw.size] = raw
    return torch.from_numpy(buf).to("cuda")


def _run(fmt, M, N, K, A, B, off_a, off_b):
    import torch
    a, b = _dev_flat(A, off_a), _dev_flat(B, off_b)
    out_dtype = torch.int32 if fmt == "i8" else torch.float32
    c = torch.full((M * N + 4,), 7, dtype=out_dtype, device="cuda")
    rc = binding.raw_gemm(fmt, None, M, N, K, a.data_ptr() + off_a * ELEM[fmt], b.data_ptr() + off_b * ELEM[fmt],
                          c.data_ptr(), None)
    assert rc == binding.GEMM_OK, binding.status_string(rc)
    torch.cuda.synchronize()
    got = c.cpu().numpy()
    assert np.all(got[M * N:] == 7), "written past C"
    return got[:M * N].reshape(M, N)


CASES = {
    "f32": _shapes(7101, 45, 5e8),
    "f16": _shapes(7102, 30, 5e8),
    "bf16": _shapes(7103, 21, 5e8),
    "e4m3": _shapes(7104, 18, 5e8),
    "e5m2": _shapes(7105, 12, 5e8),
    "i8": _shapes(7106, 18, 5e8),
}


@pytest.mark.parametrize("fmt,case", [(f, c) for f, cs in CASES.items() for c in cs],
                         ids=lambda v: v if isinstance(v, str) else "x".join(map(str, v)))
def test_random_shapes_and_alignment(fmt, case):
    M, N, K, off_a, off_b = case
    p = dg.plan(fmt, M, N, K)
    say("sweep", fmt, (M, N, K), "offsets", off_a, off_b, dg.variant_name(p["variant"]),
        (p["tile_m"], p["tile_n"], p["tile_k"]))
    A, B = inputs.matrices(M, N, K, 7200 + M + N + K, "int", fmt)
    got = _run(fmt, M, N, K, A, B, off_a, off_b)
    ref = ORACLE[fmt](A, B)
    bad = got != ref
    assert not bad.any(), f"{fmt} {case}: {int(bad.sum())} elements differ, first {np.argwhere(bad)[0]}"


# general layouts: random op flags, padded leading dimensions and dyadic scales
EX_CASES = []
_rng = np.random.default_rng(7301)
for _fmt in ("f32", "f16", "bf16"):
    for _ in range(12):
        M, N, K = _size(_rng, 1, 700), _size(_rng, 1, 700), _size(_rng, 1, 600)
        EX_CASES.append((_fmt, M, N, K, int(_rng.integers(0, 2)), int(_rng.integers(0, 2)),
                         int(_rng.choice([0, 0, 8, 3])), float(_rng.choice([1.0, 2.0, -0.5])),
                         float(_rng.choice([0.0, 0.0, 1.0, -2.0, 0.25]))))


def _store(X, ld, fill):
    r, c = X.shape
    buf = np.full((r - 1) * ld + c if r and c else 1, fill, dtype=X.dtype)
    for i in range(r):
        buf[i * ld:i * ld + c] = X[i]
    return buf


@pytest.mark.parametrize("case", EX_CASES, ids=lambda c: "_".join(map(str, c)))
def test_random_general_layouts(case):
    import torch
    from helpers import to_dev
    fmt, M, N, K, op_a, op_b, pad, alpha, beta = case
    say("sweep ex", case)
    A, B = inputs.matrices(M, N, K, 7400 + M + K, "int", fmt)
    As = A.T.copy() if op_a else A
    Bs = B.T.copy() if op_b else B
    lda, ldb, ldc = As.shape[1] + pad, Bs.shape[1] + pad, N + pad
    fa, fb = _store(As, max(lda, 1), 0), _store(Bs, max(ldb, 1), 0)
    C0 = _store(inputs.matrices(M, N, 1, 7500 + N, "int", "f32")[0][:, :1].repeat(N, 1).astype(np.float32),
                max(ldc, 1), 5.0)
    a, b, c = to_dev(fa), to_dev(fb), to_dev(C0)
    rc = binding.raw_gemm_ex(fmt, op_a, op_b, M, N, K, alpha, a.data_ptr(), max(lda, 1), b.data_ptr(),
                             max(ldb, 1), beta, c.data_ptr(), max(ldc, 1), None)
    assert rc == binding.GEMM_OK, binding.status_string(rc)
    torch.cuda.synchronize()
    got = c.cpu().numpy()
    want = oracle.gemm_ex(fmt, op_a, op_b, M, N, K, alpha, fa, max(lda, 1), fb, max(ldb, 1), beta, C0.copy(),
                          max(ldc, 1))
    bad = got != want
    assert not bad.any(), f"{case}: {int(bad.sum())} elements differ"


# convolutions: random small geometries in every format
CONV_CASES = []
_rng = np.random.default_rng(7601)
for _fmt in ("f32", "f16", "bf16"):
    for _ in range(8):
        R, S = int(_rng.integers(1, 6)), int(_rng.integers(1, 6))
        st = (int(_rng.integers(1, 3)), int(_rng.integers(1, 3)))
        dl = (int(_rng.integers(1, 3)), int(_rng.integers(1, 3)))
        pd = (int(_rng.integers(0, 3)), int(_rng.integers(0, 3)))
        H = int(_rng.integers(dl[0] * (R - 1) + 1, 40)) + pd[0] * 0
        W = int(_rng.integers(dl[1] * (S - 1) + 1, 40))
        CONV_CASES.append((_fmt, int(_rng.integers(1, 5)), int(_rng.integers(1, 40)), H, W,
                           int(_rng.integers(1, 300)), R, S, st, pd, dl))


@pytest.mark.parametrize("case", CONV_CASES, ids=lambda c: "_".join(map(str, c[:8])))
def test_random_convolutions(case):
    import torch
    from helpers import to_dev
    fmt, N, C, H, W, K, R, S, st, pd, dl = case
    say("sweep conv", case)
    n = N * C * H * W
    x = inputs.matrices(1, 1, n, 7700 + n, "int", fmt)[0].reshape(N, C, H, W)
    w = inputs.matrices(1, 1, K * C * R * S, 7800 + K, "int", fmt)[0].reshape(K, C, R, S)
    y = dg.conv2d(fmt, to_dev(x), to_dev(w), st, pd, dl)
    torch.cuda.synchronize()
    ref = oracle.conv2d(fmt, x, w, st, pd, dl)
    got = y.cpu().numpy()
    assert got.shape == ref.shape
    bad = got != ref
    assert not bad.any(), f"{case}: {int(bad.sum())} elements differ"


# convolutions that take the implicit GEMMs: seeded random geometries (stride,
# padding and dilation per axis, rectangular filters) sized for enough tiles.
# Channels last: C a multiple of 32 and at least 96 tiles; gathering: C below
# 32 and at least 256 tiles of 128 filters x 256 pixels.  Integer inputs,
# bit-exact; each case asserts the path it takes.
IMPLICIT_CASES = []
_rng = np.random.default_rng(7901)


def _out(n, k, p, d, s):
    return (n + 2 * p - d * (k - 1) - 1) // s + 1


def _nhwc_tiles(N, H, W, K, R, S, st, pd, dl):
    npq = N * _out(H, R, pd[0], dl[0], st[0]) * _out(W, S, pd[1], dl[1], st[1])
    return -(-npq // 256) if K <= 64 else -(-K // 128) * -(-npq // 64), npq


for _fmt in ("f16", "bf16"):
    for _i in range(10):
        nhwc = _i < 6
        while True:   # draw until the case takes the path it is meant for, at a size the oracle finishes quickly
            R, S = int(_rng.integers(1, 4)), int(_rng.integers(1, 4))
            st = (int(_rng.integers(1, 3)), int(_rng.integers(1, 3)))
            dl = (int(_rng.integers(1, 3)), int(_rng.integers(1, 3)))
            pd = (int(_rng.integers(0, 3)), int(_rng.integers(0, 3)))
            if nhwc:
                C = 32 * int(_rng.integers(1, 4))
                K = int(_rng.integers(1, 65)) if _i < 3 else int(_rng.integers(65, 161))
                N, H, W = int(_rng.integers(16, 81)), int(_rng.integers(20, 49)), int(_rng.integers(20, 49))
                tiles, npq = _nhwc_tiles(N, H, W, K, R, S, st, pd, dl)
                if tiles >= 96 and 2 * npq * K * C * R * S <= 4e9:
                    break
            else:
                C, K, N = int(_rng.integers(1, 32)), int(_rng.integers(1, 129)), int(_rng.integers(48, 65))
                H, W = int(_rng.integers(44, 57)), int(_rng.integers(44, 57))
                st = (1, 1)   # enough pixels for 256 tiles
                break
        IMPLICIT_CASES.append((_fmt, nhwc, N, C, H, W, K, R, S, st, pd, dl))


@pytest.mark.parametrize("case", IMPLICIT_CASES, ids=lambda c: "_".join(map(str, c[:9])))
def test_random_implicit_gemm_convolutions(case):
    import torch
    from helpers import to_dev
    fmt, nhwc, N, C, H, W, K, R, S, st, pd, dl = case
    P = (H + 2 * pd[0] - dl[0] * (R - 1) - 1) // st[0] + 1
    Q = (W + 2 * pd[1] - dl[1] * (S - 1) - 1) // st[1] + 1
    prm = binding.conv_params(N, C, H, W, K, R, S, st, pd, dl)
    algo = dg.conv2d_algorithm(prm, 2)
    if nhwc:
        tiles = _nhwc_tiles(N, H, W, K, R, S, st, pd, dl)[0]
        assert (algo == dg.CONV_IMPLICIT_NHWC) == (tiles >= 96), (case, tiles, algo)
    else:
        tiles = -(-K // 128) * -(-(N * P * Q) // 256)
        assert (algo == dg.CONV_IMPLICIT) == (tiles >= 256), (case, tiles, algo)
    say("sweep implicit conv", case, "algorithm", algo)
    n = N * C * H * W
    x = inputs.matrices(1, 1, n, 8000 + n, "int", fmt)[0].reshape(N, C, H, W)
    w = inputs.matrices(1, 1, K * C * R * S, 8100 + K, "int", fmt)[0].reshape(K, C, R, S)
    y = dg.conv2d(fmt, to_dev(x), to_dev(w), st, pd, dl)
    torch.cuda.synchronize()
    ref = oracle.conv2d(fmt, x, w, st, pd, dl)
    got = y.cpu().numpy()
    assert got.shape == ref.shape
    bad = got != ref
    assert not bad.any(), f"{case}: {int(bad.sum())} elements differ"
