"""GPU parity of the general-layout entry points (gemm_*_ex): C = alpha op(A)
op(B) + beta C with transposed operands, padded leading dimensions and the
scale factors, against the oracle's general-layout routine on the same
storage ("Lesson 8: how a GPU does matrix multiply", section 28).

Bars: small-integer inputs with dyadic alpha, beta (every intermediate exact
in binary32) are bit-exact on every path; other inputs meet
|alpha| * (the plain bar for K) + 8 eps32 (|alpha| max|AB| + |beta| max|C0|),
the second term covering the separate scaling passes.  Shapes take both the
256 x 256 ring kernels (whole 16-byte vectors) and the plain strided kernel
(anything else), with ragged tiles in M, N and K.
"""
import numpy as np
import pytest

from dense_gemm_optimisation_row_amd import binding, inputs

import oracle
from helpers import oracle_at, say, to_dev, tol_f16, tol_f32

pytestmark = pytest.mark.gpu

EPS32 = 2.0 ** -23


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU (run the CPU suite with -m 'not gpu')")
    binding.load()
    return torch.device("cuda")


def _store(X, op, ld, fill):
    """Flat storage of the logical matrix X as op N (row stride ld) or op T
    (X's transpose, row stride ld); padding set to ``fill``; no padding after
    the last stored row, so any read past the operand would leave it."""
    S = X.T if op else X
    r, c = S.shape
    buf = np.full((r - 1) * ld + c if r and c else 1, fill, dtype=X.dtype)
    for i in range(r):
        buf[i * ld:i * ld + c] = S[i]
    return buf


def _nan_of(X):
    return np.uint16(0x7FC0) if X.dtype == np.uint16 else X.dtype.type(np.nan)


def _call_gpu(fmt, op_a, op_b, M, N, K, alpha, A, lda, B, ldb, beta, C0, ldc):
    """Run gemm_<fmt>_ex on device copies of the flat arrays; returns the flat C."""
    import torch
    a, b, c = to_dev(A), to_dev(B), to_dev(C0)
    rc = binding.raw_gemm_ex(fmt, op_a, op_b, M, N, K, alpha, a.data_ptr(), lda, b.data_ptr(), ldb,
                             beta, c.data_ptr(), ldc, None)
    assert rc == binding.GEMM_OK, binding.status_string(rc)
    torch.cuda.synchronize()
    return c.cpu().numpy()


def _oracle(fmt, op_a, op_b, M, N, K, alpha, A, lda, B, ldb, beta, C0, ldc):
    C = C0.copy()
    return oracle.gemm_ex(fmt, op_a, op_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc)


def _mats(fmt, M, N, K, seed, dist):
    return inputs.matrices(M, N, K, seed, dist, fmt)


LAYOUTS = [(0, 0), (0, 1), (1, 0), (1, 1)]
# (M, N, K): all multiples of 8 (ring kernels when the leading dimensions
# are), ragged 256-tiles in M and N and a k tail; then odd sizes (plain kernel).
SHAPES = [(264, 520, 72), (520, 264, 136), (300, 201, 77), (37, 45, 1000)]
INT_SCALES = [(1.0, 0.0), (2.0, 0.5), (-1.0, 3.0), (1.0, 1.0), (0.5, 0.0), (0.25, -2.0)]
FLOAT_SCALES = INT_SCALES + [(1.5, -0.25), (-0.7, 0.3)]


def _run_case(fmt, op_a, op_b, shape, pad, alpha, beta, integer, seed):
    M, N, K = shape
    A, B = _mats(fmt, M, N, K, seed, "int" if integer else "uniform")
    rng = np.random.default_rng(seed + 1)
    C0 = (rng.integers(-1000, 1001, (M, N)) if integer else rng.uniform(-1, 1, (M, N))).astype(np.float32)
    lda, ldb, ldc = (M if op_a else K) + pad, (K if op_b else N) + pad, N + pad
    As, Bs = _store(A, op_a, lda, _nan_of(A)), _store(B, op_b, ldb, _nan_of(B))
    Cs = np.full(M * ldc, -3.5, np.float32)
    Cs.reshape(M, ldc)[:, :N] = C0
    got = _call_gpu(fmt, op_a, op_b, M, N, K, alpha, As, lda, Bs, ldb, beta, Cs, ldc).reshape(M, ldc)
    want = _oracle(fmt, op_a, op_b, M, N, K, alpha, As, lda, Bs, ldb, beta, Cs, ldc).reshape(M, ldc)
    what = f"{fmt} op{op_a}{op_b} {shape} pad {pad} alpha {alpha} beta {beta}"
    assert np.all(got[:, N:] == np.float32(-3.5)), f"{what}: C padding written"
    got, want = got[:, :N], want[:, :N]
    if integer:
        bad = got != want
        assert not bad.any(), f"{what}: {int(bad.sum())} elements differ, first {np.argwhere(bad)[0]}"
        return
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    ab = np.abs(want.astype(np.float64) - beta * C0.astype(np.float64)) / max(abs(alpha), 1e-30)
    plain = tol_f32(K) if fmt == "f32" else tol_f16(K, ab)
    tol = abs(alpha) * plain + 8 * EPS32 * (abs(alpha) * float(ab.max()) + abs(beta) * float(np.abs(C0).max()))
    err = float(np.max(np.abs(got.astype(np.float64) - want.astype(np.float64))))
    assert err <= tol, f"{what}: max |dC| {err:.3e} > {tol:.3e}"


@pytest.mark.parametrize("fmt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("layout", LAYOUTS, ids=lambda l: f"op{l[0]}{l[1]}")
def test_ex_layouts_pads_and_scales(fmt, shape, layout):
    op_a, op_b = layout
    for pad in (0, 8, 3):
        say("ex", fmt, layout, shape, "pad", pad)
        for alpha, beta in INT_SCALES:
            _run_case(fmt, op_a, op_b, shape, pad, alpha, beta, True, 3100)
        for alpha, beta in FLOAT_SCALES:
            _run_case(fmt, op_a, op_b, shape, pad, alpha, beta, False, 3200)


@pytest.mark.parametrize("fmt", ["f32", "f16", "bf16"])
def test_ex_beta_zero_ignores_C_and_k0_alpha0_scale_C(fmt):
    M, N, K = 264, 136, 64
    A, B = _mats(fmt, M, N, K, 3300, "int")
    for op_a, op_b in LAYOUTS:
        for pad in (0, 3):
            say("ex beta0", fmt, op_a, op_b, pad)
            lda, ldb = (M if op_a else K) + pad, (K if op_b else N) + pad
            As, Bs = _store(A, op_a, lda, _nan_of(A)), _store(B, op_b, ldb, _nan_of(B))
            Cn = np.full(M * N, np.nan, np.float32)
            got = _call_gpu(fmt, op_a, op_b, M, N, K, 2.0, As, lda, Bs, ldb, 0.0, Cn, N)
            want = _oracle(fmt, op_a, op_b, M, N, K, 2.0, As, lda, Bs, ldb, 0.0, Cn, N)
            assert np.array_equal(got, want)
    C0 = np.random.default_rng(3301).integers(-50, 51, M * N).astype(np.float32)
    dummy = np.zeros(8, np.float32 if fmt == "f32" else np.uint16)
    for K0, alpha, beta in ((0, 1.0, 0.5), (0, 3.0, 0.0), (K, 0.0, -2.0), (K, 0.0, 0.0)):
        say("ex k0/alpha0", fmt, K0, alpha, beta)
        As, Bs = (dummy, dummy) if K0 == 0 else (A.ravel(), B.ravel())
        src = C0 if beta != 0 else np.full(M * N, np.nan, np.float32)
        got = _call_gpu(fmt, 0, 0, M, N, K0, alpha, As, max(K0, 1), Bs, N, beta, src, N)
        assert np.array_equal(got, (np.float32(beta) * C0) if beta != 0 else np.zeros_like(C0))


@pytest.mark.parametrize("fmt", ["f32", "f16", "bf16"])
def test_ex_plain_layout_is_the_plain_entry_point(fmt):
    import torch
    import dense_gemm_optimisation_row_amd as dg
    M, N, K = 1024, 768, 512
    A, B = _mats(fmt, M, N, K, 3400, "uniform")
    a, b = to_dev(A), to_dev(B)
    say("ex plain", fmt)
    plain = {"f32": dg.gemm_f32, "f16": dg.gemm_f16_f32acc, "bf16": dg.gemm_bf16_f32acc}[fmt](a, b)
    ex = {"f32": dg.gemm_f32_ex, "f16": dg.gemm_f16_f32acc_ex, "bf16": dg.gemm_bf16_f32acc_ex}[fmt](a, b)
    torch.cuda.synchronize()
    assert torch.equal(plain, ex)


@pytest.mark.parametrize("fmt", ["f32", "f16", "bf16"])
def test_ex_torch_views(fmt):
    """The torch layer reads op and leading dimension off the strides: a
    transposed view is op T, a column slice of a wider tensor a padded ld."""
    import torch
    import dense_gemm_optimisation_row_amd as dg
    fn = {"f32": dg.gemm_f32_ex, "f16": dg.gemm_f16_f32acc_ex, "bf16": dg.gemm_bf16_f32acc_ex}[fmt]
    M, N, K = 264, 200, 136
    A, B = _mats(fmt, M, N, K, 3500, "int")
    ref = oracle.gemm_ex(fmt, 0, 0, M, N, K, 1.0, A.ravel(), K, B.ravel(), N, 0.0,
                         np.zeros(M * N, np.float32), N).reshape(M, N)
    a, b = to_dev(A), to_dev(B)
    wide_a = torch.zeros((M, K + 24), dtype=a.dtype, device=a.device)
    wide_a[:, :K] = a
    views = {
        "NN": (a, b),
        "TN": (a.t().contiguous().t(), b),
        "NT": (a, b.t().contiguous().t()),
        "TT": (a.t().contiguous().t(), b.t().contiguous().t()),
        "padded": (wide_a[:, :K], b),
    }
    for name, (va, vb) in views.items():
        say("ex view", fmt, name)
        c = fn(va, vb)
        torch.cuda.synchronize()
        assert np.array_equal(c.cpu().numpy(), ref), name
    cbig = torch.full((M, N + 8), 5.0, device=a.device)
    cv = cbig[:, :N]
    cv.fill_(1.0)
    fn(a, b, cv, alpha=2.0, beta=-1.0)
    torch.cuda.synchronize()
    out = cbig.cpu().numpy()
    assert np.array_equal(out[:, :N], 2 * ref - 1) and np.all(out[:, N:] == 5.0)


# The large operands in the launch configuration a transposed caller gets: the
# ring kernels on 4096 (FP32) and 8192 (16-bit) with op T operands and
# alpha/beta, checked on sampled elements against the oracle's value of the
# same product.
LARGE = [("f32", 4096, 4096, 4096, "normal", 1005), ("f16", 8192, 8192, 8192, "uniform", 1006),
         ("bf16", 8192, 8192, 8192, "uniform", 1007)]


@pytest.mark.parametrize("case", LARGE, ids=lambda c: f"{c[0]}_{c[1]}")
@pytest.mark.parametrize("layout", [(1, 0), (0, 1), (1, 1)], ids=lambda l: f"op{l[0]}{l[1]}")
def test_ex_large_transposed_sampled(case, layout):
    import torch
    fmt, M, N, K, dist, seed = case
    op_a, op_b = layout
    say("ex large", fmt, M, layout)
    A, B = inputs.matrices(M, N, K, seed, dist, fmt)
    a, b = to_dev(A), to_dev(B)
    at = a.t().contiguous() if op_a else a
    bt = b.t().contiguous() if op_b else b
    c0 = torch.linspace(-1, 1, M * N, device=a.device, dtype=torch.float32).reshape(M, N).contiguous()
    c = c0.clone()
    alpha, beta = 0.75, -0.5
    rc = binding.raw_gemm_ex(fmt, op_a, op_b, M, N, K, alpha, at.data_ptr(), M if op_a else K,
                             bt.data_ptr(), K if op_b else N, beta, c.data_ptr(), N, None)
    assert rc == binding.GEMM_OK
    torch.cuda.synchronize()
    rows, cols = inputs.sample_indices(M, N, 192, seed + 77)
    ab = oracle_at(A, B, rows, cols).astype(np.float64)
    c0s = c0.cpu().numpy()[rows, cols].astype(np.float64)
    want = alpha * ab + beta * c0s
    got = c.cpu().numpy()[rows, cols]
    plain = tol_f32(K) if fmt == "f32" else tol_f16(K, np.abs(ab))
    tol = alpha * plain + 8 * EPS32 * (alpha * float(np.abs(ab).max()) + abs(beta))
    assert np.max(np.abs(got - want)) <= tol


def _run_c_case(fmt, op_a, op_b, shape, c_pad, c_off, alpha, beta, seed):
    """Unpadded A and B (so the ring kernels run on the multiple-of-8 shapes)
    with C's rows ``c_pad`` elements apart beyond N and C's first element
    ``c_off`` floats into its buffer: the ring epilogue's element-wise stores
    whenever C is not 16-byte aligned or ldc not a multiple of 4.  Integer
    inputs, bit-exact; every element around C must keep its sentinel."""
    import torch
    M, N, K = shape
    A, B = _mats(fmt, M, N, K, seed, "int")
    C0 = np.random.default_rng(seed + 1).integers(-1000, 1001, (M, N)).astype(np.float32)
    lda, ldb, ldc = (M if op_a else K), (K if op_b else N), N + c_pad
    As, Bs = _store(A, op_a, lda, _nan_of(A)), _store(B, op_b, ldb, _nan_of(B))
    Cs = np.full(M * ldc, -3.5, np.float32)
    Cs.reshape(M, ldc)[:, :N] = C0
    buf = np.concatenate([np.full(c_off, -7.25, np.float32), Cs, np.full(4, -7.25, np.float32)])
    a, b, cbuf = to_dev(As), to_dev(Bs), to_dev(buf)
    c_ptr = cbuf.data_ptr() + 4 * c_off
    assert (c_ptr % 16 == 0) == (c_off % 4 == 0)
    rc = binding.raw_gemm_ex(fmt, op_a, op_b, M, N, K, alpha, a.data_ptr(), lda, b.data_ptr(), ldb,
                             beta, c_ptr, ldc, None)
    assert rc == binding.GEMM_OK, binding.status_string(rc)
    torch.cuda.synchronize()
    out = cbuf.cpu().numpy()
    what = f"{fmt} op{op_a}{op_b} {shape} ldc N+{c_pad} C +{c_off} floats alpha {alpha} beta {beta}"
    assert np.all(out[:c_off] == np.float32(-7.25)) and np.all(out[c_off + M * ldc:] == np.float32(-7.25)), \
        f"{what}: written outside C's storage"
    got = out[c_off:c_off + M * ldc].reshape(M, ldc)
    want = _oracle(fmt, op_a, op_b, M, N, K, alpha, As, lda, Bs, ldb, beta, Cs, ldc).reshape(M, ldc)
    assert np.all(got[:, N:] == np.float32(-3.5)), f"{what}: C padding written"
    bad = got[:, :N] != want[:, :N]
    assert not bad.any(), f"{what}: {int(bad.sum())} elements differ, first {np.argwhere(bad)[0]}"


@pytest.mark.parametrize("fmt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("layout", LAYOUTS, ids=lambda l: f"op{l[0]}{l[1]}")
def test_ring_epilogue_with_unaligned_c(fmt, layout):
    op_a, op_b = layout
    for shape in SHAPES[:2]:
        for c_pad, c_off in ((1, 0), (3, 0), (0, 1), (4, 2), (0, 3)):
            say("ex unaligned C", fmt, layout, shape, c_pad, c_off)
            for alpha, beta in ((1.0, 0.0), (2.0, 0.5)):
                _run_c_case(fmt, op_a, op_b, shape, c_pad, c_off, alpha, beta, 3300 + c_pad + 10 * c_off)
