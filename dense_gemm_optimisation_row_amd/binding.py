"""ctypes binding of the C ABI in ``include/gemm.h`` (argument marshalling only).

Two layers:

* ``raw_*`` functions pass integers (device addresses, sizes, a stream
  handle) straight to the library and return its status code;
* ``gemm_f32`` / ``gemm_f16_f32acc`` / ``gemm_bf16_f32acc`` and the 8-bit
  ``gemm_e4m3_f32acc`` / ``gemm_e5m2_f32acc`` / ``gemm_i8_i32acc`` (and
  ``*_variant``) take torch tensors
  that already live on the GPU, check shape / dtype / contiguity, call the
  library on the tensors' current stream and raise ``GemmError`` on a
  non-zero status;
* ``gemm_*_ex`` take strided 2-D views (one unit stride each) and read the
  operand layout (transposed or not, leading dimension) off the strides.

All arithmetic happens in the HIP kernels.  There is no fallback: if the
library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libdgor_gemm.so")

# Mirrors gemm_status / gemm_variant of include/gemm.h.
GEMM_OK = 0
GEMM_ERR_INVALID_DIM = -1
GEMM_ERR_NULL_PTR = -2
GEMM_ERR_LAUNCH = -3
GEMM_ERR_UNSUPPORTED_DEVICE = -4
GEMM_ERR_INVALID_VARIANT = -5
GEMM_ERR_RUNTIME = -6
GEMM_ERR_INVALID_LAYOUT = -7
GEMM_ERR_WORKSPACE = -8
GEMM_ERR_SCRATCH_LIMIT = -9
GEMM_OP_N, GEMM_OP_T = 0, 1

AUTO = -1
R0_NAIVE, R1_LDS_TILED, R2_VECTOR_LOADS, R3_LDS_PADDED = 0, 1, 2, 3
R4_DOUBLE_BUFFER, R5_REGISTER_BLOCKED, R6_MFMA_F32, R7_MFMA_F16 = 4, 5, 6, 7
R8_MFMA_8BIT = 8
F32_VARIANTS = (0, 1, 2, 3, 4, 5, 6)
F16_VARIANTS = (0, 7)
BF16_VARIANTS = (0, 7)
EIGHT_BIT_VARIANTS = (0, 8)

EXPORTS = ("gemm_f32", "gemm_f16_f32acc", "gemm_bf16_f32acc",
           "gemm_f32_variant", "gemm_f16_f32acc_variant", "gemm_bf16_f32acc_variant",
           "gemm_f32_plan", "gemm_f16_f32acc_plan", "gemm_bf16_f32acc_plan",
           "gemm_e4m3_f32acc", "gemm_e5m2_f32acc", "gemm_i8_i32acc",
           "gemm_e4m3_f32acc_variant", "gemm_e5m2_f32acc_variant", "gemm_i8_i32acc_variant",
           "gemm_e4m3_f32acc_plan", "gemm_e5m2_f32acc_plan", "gemm_i8_i32acc_plan",
           "gemm_f32_ex", "gemm_f16_f32acc_ex", "gemm_bf16_f32acc_ex",
           "gemm_conv2d_workspace", "gemm_conv2d_algorithm", "gemm_conv2d_f32", "gemm_conv2d_f16_f32acc", "gemm_conv2d_bf16_f32acc",
           "gemm_conv2d_f16_f32acc_noalloc",
           "gemm_status_string", "gemm_variant_name")

# Entry-point name stem per input format.
_STEM = {"f32": "gemm_f32", "f16": "gemm_f16_f32acc", "bf16": "gemm_bf16_f32acc",
         "e4m3": "gemm_e4m3_f32acc", "e5m2": "gemm_e5m2_f32acc", "i8": "gemm_i8_i32acc"}
# Formats with a general-layout (``_ex``) entry point.
_EX_KINDS = ("f32", "f16", "bf16")


def kind_of(kind) -> str:
    """Input format of a call: "f32", "f16", "bf16", "e4m3", "e5m2" or "i8"; a
    bool means f16 (True) or f32 (False)."""
    if isinstance(kind, bool):
        return "f16" if kind else "f32"
    if kind in _STEM:
        return kind
    raise ValueError(f"unknown input format {kind!r}")


class GemmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class ConvParams(ctypes.Structure):
    """gemm_conv2d_params of include/gemm.h."""
    _fields_ = [(n, ctypes.c_int) for n in (
        "N", "C", "H", "W", "K", "R", "S", "stride_h", "stride_w", "pad_h", "pad_w",
        "dilation_h", "dilation_w")]


_CONV_STEM = {"f32": "gemm_conv2d_f32", "f16": "gemm_conv2d_f16_f32acc", "bf16": "gemm_conv2d_bf16_f32acc"}


class Plan(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in (
        "variant", "launches", "tile_m", "tile_n", "tile_k", "threads", "grid_x", "grid_y",
        "k_stages", "lds_stages", "lds_bytes", "tile_bytes", "outputs_per_thread",
        "vector_a", "vector_b", "vector_c")]

    def as_dict(self) -> dict:
        return {n: getattr(self, n) for n, _ in self._fields_}


_lib = None
_libs = {}


def load(path: str = LIB_PATH):
    """Load the library once (raises if it has not been built).  ``path``
    selects another build of the same ABI (the LDS-poisoning debug build);
    calls through the module's functions always use the product library."""
    global _lib
    if path != LIB_PATH:
        if path not in _libs:
            _libs[path] = _configure(path)
        return _libs[path]
    if _lib is None:
        _lib = _configure(path)
    return _lib


def _configure(path: str):
    if not os.path.exists(path):
        raise RuntimeError(
            f"HIP library {path} is missing: build it with "
            "`python -m dense_gemm_optimisation_row_amd.build`")
    lib = ctypes.CDLL(path)
    i, p = ctypes.c_int, ctypes.c_void_p
    for kind, stem in _STEM.items():
        f = getattr(lib, stem)
        f.argtypes = [i, i, i, p, p, p, p]
        f.restype = i
        f = getattr(lib, stem + "_variant")
        f.argtypes = [i, i, i, i, p, p, p, p]
        f.restype = i
        f = getattr(lib, stem + "_plan")
        f.argtypes = [i, i, i, i, p, p, p, ctypes.POINTER(Plan)]
        f.restype = i
        if kind in _EX_KINDS:
            f = getattr(lib, stem + "_ex")
            f.argtypes = [i, i, i, i, i, ctypes.c_float, p, i, p, i, ctypes.c_float, p, i, p]
            f.restype = i
    lib.gemm_conv2d_workspace.argtypes = [ctypes.POINTER(ConvParams), i, ctypes.POINTER(ctypes.c_size_t)]
    lib.gemm_conv2d_workspace.restype = i
    lib.gemm_conv2d_algorithm.argtypes = [ctypes.POINTER(ConvParams), i, ctypes.POINTER(i)]
    lib.gemm_conv2d_algorithm.restype = i
    for stem in _CONV_STEM.values():
        f = getattr(lib, stem)
        f.argtypes = [ctypes.POINTER(ConvParams), p, p, p, p, ctypes.c_size_t, p]
        f.restype = i
    lib.gemm_conv2d_f16_f32acc_noalloc.argtypes = [ctypes.POINTER(ConvParams), p, p, p, p]
    lib.gemm_conv2d_f16_f32acc_noalloc.restype = i
    lib.gemm_status_string.argtypes = [i]
    lib.gemm_status_string.restype = ctypes.c_char_p
    lib.gemm_variant_name.argtypes = [i]
    lib.gemm_variant_name.restype = ctypes.c_char_p
    return lib


def status_string(status: int) -> str:
    return load().gemm_status_string(int(status)).decode()


def variant_name(variant: int) -> str:
    return load().gemm_variant_name(int(variant)).decode()


# ------------------------------------------------------------- raw layer --

def raw_gemm(kind, variant: int | None, M: int, N: int, K: int,
             A: int | None, B: int | None, C: int | None, stream: int | None) -> int:
    """Call the library with plain integers; returns the status code.
    ``kind`` is the input format ("f32", "f16", "bf16", or a bool for f16)."""
    lib = load()
    stem = _STEM[kind_of(kind)]
    if variant is None:
        return int(getattr(lib, stem)(M, N, K, A, B, C, stream))
    return int(getattr(lib, stem + "_variant")(variant, M, N, K, A, B, C, stream))


def raw_gemm_ex(kind, op_a: int, op_b: int, M: int, N: int, K: int, alpha: float,
                A: int | None, lda: int, B: int | None, ldb: int, beta: float,
                C: int | None, ldc: int, stream: int | None) -> int:
    """``gemm_*_ex`` with plain integers; returns the status code."""
    f = getattr(load(), _STEM[kind_of(kind)] + "_ex")
    return int(f(op_a, op_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream))


def plan(kind, M: int, N: int, K: int, variant: int = AUTO,
         A: int = 0, B: int = 0, C: int = 0) -> dict:
    """Launch plan for these arguments (host arithmetic only; no GPU needed).

    Addresses matter only through their 16-byte alignment; 0 counts as aligned.
    """
    lib = load()
    out = Plan()
    f = getattr(lib, _STEM[kind_of(kind)] + "_plan")
    rc = f(variant, M, N, K, A or None, B or None, C or None, ctypes.byref(out))
    if rc != GEMM_OK:
        raise GemmError(rc, "plan")
    return out.as_dict()


# ----------------------------------------------------------- torch layer --

def _check(A, B, C, in_dtype, out_dtype=None):
    import torch
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    if A.dim() != 2 or B.dim() != 2 or A.shape[1] != B.shape[0]:
        raise ValueError(f"shapes {tuple(A.shape)} x {tuple(B.shape)} do not chain")
    if A.dtype != in_dtype or B.dtype != in_dtype:
        raise TypeError(f"A and B must be {in_dtype}")
    if not (A.is_cuda and B.is_cuda):
        raise ValueError("A and B must be GPU tensors")
    if not (A.is_contiguous() and B.is_contiguous()):
        raise ValueError("A and B must be contiguous (row-major)")
    M, K = A.shape
    N = B.shape[1]
    if C is None:
        C = torch.empty((M, N), dtype=out_dtype, device=A.device)
    elif (tuple(C.shape) != (M, N) or C.dtype != out_dtype or not C.is_contiguous()
          or C.device != A.device):
        raise ValueError(f"C must be a contiguous {out_dtype} M x N tensor on A's device")
    if B.device != A.device:
        raise ValueError("A and B must be on the same device")
    return M, N, K, C


def _stream_handle(device, stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t):
    return t.data_ptr() if t.numel() else None


_DTYPES = {}


def _dtypes(kind):
    """(input dtype, output dtype) of a format."""
    if not _DTYPES:
        import torch
        _DTYPES.update({"f32": (torch.float32, torch.float32), "f16": (torch.float16, torch.float32),
                        "bf16": (torch.bfloat16, torch.float32), "e4m3": (torch.float8_e4m3fn, torch.float32),
                        "e5m2": (torch.float8_e5m2, torch.float32), "i8": (torch.int8, torch.int32)})
    return _DTYPES[kind]


_ENTRY_CACHE = {}


def _entry(kind, variant):
    """The library function of a format (automatic or forced variant), looked
    up once."""
    key = (kind, variant is None)
    f = _ENTRY_CACHE.get(key)
    if f is None:
        f = getattr(load(), _STEM[kind] + ("" if variant is None else "_variant"))
        _ENTRY_CACHE[key] = f
    return f


def _call(kind, variant, A, B, C, stream):
    import torch
    kind = kind_of(kind)
    M, N, K, C = _check(A, B, C, *_dtypes(kind))
    f = _entry(kind, variant)
    args = (M, N, K, _ptr(A), _ptr(B), _ptr(C))
    if variant is not None:
        args = (variant,) + args
    # the call runs on A's device: switch only when another is current (the
    # switch costs more than a small GEMM's launch)
    if A.device.index == torch.cuda.current_device():
        rc = int(f(*args, _stream_handle(A.device, stream)))
    else:
        with torch.cuda.device(A.device):
            rc = int(f(*args, _stream_handle(A.device, stream)))
    if rc != GEMM_OK:
        raise GemmError(rc, _STEM[kind])
    return C


def gemm_f32(A, B, C=None, stream=None):
    """C = A x B for float32 GPU tensors; returns C (allocated if not given)."""
    return _call(False, None, A, B, C, stream)


def gemm_f16_f32acc(A, B, C=None, stream=None):
    """C = A x B for float16 GPU tensors with FP32 accumulation and output."""
    return _call(True, None, A, B, C, stream)


def gemm_f32_variant(variant, A, B, C=None, stream=None):
    """``gemm_f32`` with the kernel variant (rung) forced."""
    return _call(False, int(variant), A, B, C, stream)


def gemm_f16_f32acc_variant(variant, A, B, C=None, stream=None):
    """``gemm_f16_f32acc`` with the kernel variant (rung) forced."""
    return _call(True, int(variant), A, B, C, stream)


def gemm_bf16_f32acc(A, B, C=None, stream=None):
    """C = A x B for bfloat16 GPU tensors with FP32 accumulation and output."""
    return _call("bf16", None, A, B, C, stream)


def gemm_bf16_f32acc_variant(variant, A, B, C=None, stream=None):
    """``gemm_bf16_f32acc`` with the kernel variant (rung) forced."""
    return _call("bf16", int(variant), A, B, C, stream)


def _layout(t, name):
    """(op, leading dimension) of a 2-D view with one unit stride: op N when
    rows are contiguous (X[r][c] at r*ld + c), op T when columns are (the view
    is the transpose of a row-major matrix with row stride ld)."""
    rows, cols = t.shape
    s0, s1 = t.stride()
    if s1 == 1 or cols <= 1:
        return GEMM_OP_N, (s0 if rows > 1 else max(cols, 1))
    if s0 == 1 or rows <= 1:
        return GEMM_OP_T, (s1 if cols > 1 else max(rows, 1))
    raise ValueError(f"{name} needs a unit stride in one dimension (strides {t.stride()})")


def _call_ex(kind, A, B, C, alpha, beta, stream):
    import torch
    kind = kind_of(kind)
    if kind not in _EX_KINDS:
        raise ValueError(f"no general-layout entry point for {kind}")
    dtype = _dtypes(kind)[0]
    if A.dim() != 2 or B.dim() != 2 or A.shape[1] != B.shape[0]:
        raise ValueError(f"shapes {tuple(A.shape)} x {tuple(B.shape)} do not chain")
    if A.dtype != dtype or B.dtype != dtype:
        raise TypeError(f"A and B must be {dtype}")
    if not (A.is_cuda and B.is_cuda) or B.device != A.device:
        raise ValueError("A and B must be GPU tensors on one device")
    M, K = A.shape
    N = B.shape[1]
    if C is None:
        if beta != 0:
            raise ValueError("beta != 0 needs an input C")
        C = torch.empty((M, N), dtype=torch.float32, device=A.device)
    elif tuple(C.shape) != (M, N) or C.dtype != torch.float32 or C.device != A.device:
        raise ValueError("C must be a float32 M x N tensor on A's device")
    op_a, lda = _layout(A, "A")
    op_b, ldb = _layout(B, "B")
    op_c, ldc = _layout(C, "C")
    if op_c != GEMM_OP_N:
        raise ValueError("C must have contiguous rows")
    with torch.cuda.device(A.device):
        rc = raw_gemm_ex(kind, op_a, op_b, M, N, K, float(alpha), _ptr(A), lda, _ptr(B), ldb,
                         float(beta), _ptr(C), ldc, _stream_handle(A.device, stream))
    if rc != GEMM_OK:
        raise GemmError(rc, _STEM[kind] + "_ex")
    return C


def gemm_f32_ex(A, B, C=None, alpha=1.0, beta=0.0, stream=None):
    """C = alpha A B + beta C for float32 GPU views A (M x K) and B (K x N),
    each row- or column-contiguous with any leading dimension (a transposed
    view is passed as op T); C is an M x N float32 view with contiguous rows.
    Returns C (allocated when not given, which needs beta == 0)."""
    return _call_ex("f32", A, B, C, alpha, beta, stream)


def gemm_f16_f32acc_ex(A, B, C=None, alpha=1.0, beta=0.0, stream=None):
    """``gemm_f32_ex`` for float16 A and B (FP32 accumulation and output)."""
    return _call_ex("f16", A, B, C, alpha, beta, stream)


def gemm_bf16_f32acc_ex(A, B, C=None, alpha=1.0, beta=0.0, stream=None):
    """``gemm_f32_ex`` for bfloat16 A and B (FP32 accumulation and output)."""
    return _call_ex("bf16", A, B, C, alpha, beta, stream)


def gemm_e4m3_f32acc(A, B, C=None, stream=None):
    """C = A x B for FP8 E4M3 GPU tensors (torch.float8_e4m3fn), FP32 accumulation and output."""
    return _call("e4m3", None, A, B, C, stream)


def gemm_e5m2_f32acc(A, B, C=None, stream=None):
    """C = A x B for FP8 E5M2 GPU tensors (torch.float8_e5m2), FP32 accumulation and output."""
    return _call("e5m2", None, A, B, C, stream)


def gemm_i8_i32acc(A, B, C=None, stream=None):
    """C = A x B for int8 GPU tensors, exact INT32 accumulation and int32 output."""
    return _call("i8", None, A, B, C, stream)


def gemm_e4m3_f32acc_variant(variant, A, B, C=None, stream=None):
    return _call("e4m3", int(variant), A, B, C, stream)


def gemm_e5m2_f32acc_variant(variant, A, B, C=None, stream=None):
    return _call("e5m2", int(variant), A, B, C, stream)


def gemm_i8_i32acc_variant(variant, A, B, C=None, stream=None):
    return _call("i8", int(variant), A, B, C, stream)


# ------------------------------------------------------------- convolution --

def conv_params(N, C, H, W, K, R, S, stride=(1, 1), pad=(0, 0), dil=(1, 1)) -> ConvParams:
    return ConvParams(N, C, H, W, K, R, S, stride[0], stride[1], pad[0], pad[1], dil[0], dil[1])


def conv2d_workspace(params: ConvParams, input_bytes: int) -> int:
    """Workspace bytes gemm_conv2d_* needs (host arithmetic; raises on bad params)."""
    out = ctypes.c_size_t()
    rc = load().gemm_conv2d_workspace(ctypes.byref(params), int(input_bytes), ctypes.byref(out))
    if rc != GEMM_OK:
        raise GemmError(rc, "gemm_conv2d_workspace")
    return int(out.value)


CONV_IM2COL, CONV_IMPLICIT, CONV_IMPLICIT_NHWC = 0, 1, 2   # gemm_conv_algorithm


def conv2d_algorithm(params: ConvParams, input_bytes: int) -> int:
    """The path gemm_conv2d_* takes: CONV_IM2COL, CONV_IMPLICIT (the gather
    implicit GEMM) or CONV_IMPLICIT_NHWC (the channels-last implicit GEMM);
    host arithmetic; raises on bad params."""
    out = ctypes.c_int()
    rc = load().gemm_conv2d_algorithm(ctypes.byref(params), int(input_bytes), ctypes.byref(out))
    if rc != GEMM_OK:
        raise GemmError(rc, "gemm_conv2d_algorithm")
    return int(out.value)


def raw_conv2d(kind, params: ConvParams, x: int | None, w: int | None, y: int | None,
               workspace: int | None, workspace_bytes: int, stream: int | None) -> int:
    """gemm_conv2d_* with plain integers; returns the status code."""
    f = getattr(load(), _CONV_STEM[kind_of(kind)])
    return int(f(ctypes.byref(params), x, w, y, workspace, workspace_bytes, stream))


def gemm_conv2d_f16_f32acc_noalloc(params: ConvParams, x: int | None, w: int | None, y: int | None,
                                   stream: int | None) -> int:
    """gemm_conv2d_f16_f32acc_noalloc with plain integers (device pointers of
    the binary16 x and w and the FP32 y); returns the status code."""
    return int(load().gemm_conv2d_f16_f32acc_noalloc(ctypes.byref(params), x, w, y, stream))


def conv2d(kind, x, w, stride=(1, 1), padding=(0, 0), dilation=(1, 1), y=None, workspace=None, stream=None):
    """2-D convolution (NCHW x KCRS -> NKPQ, cross-correlation) of contiguous
    GPU tensors through im2col and one GEMM.  ``kind`` is "f32", "f16" or
    "bf16" (FP32 output).  The workspace (a uint8 GPU tensor) is allocated
    here when not given; the library itself allocates nothing."""
    import torch
    kind = kind_of(kind)
    if kind not in _CONV_STEM:
        raise ValueError(f"no convolution entry point for {kind}")
    dtype = _dtypes(kind)[0]
    if x.dim() != 4 or w.dim() != 4 or x.shape[1] != w.shape[1]:
        raise ValueError(f"x {tuple(x.shape)} and w {tuple(w.shape)} must be N x C x H x W and K x C x R x S")
    if x.dtype != dtype or w.dtype != dtype or not (x.is_cuda and w.is_cuda):
        raise TypeError(f"x and w must be {dtype} GPU tensors")
    if not (x.is_contiguous() and w.is_contiguous()):
        raise ValueError("x and w must be contiguous")
    N, C, H, W = x.shape
    K, _, R, S = w.shape
    prm = conv_params(N, C, H, W, K, R, S, stride, padding, dilation)
    P = (H + 2 * padding[0] - dilation[0] * (R - 1) - 1) // stride[0] + 1
    Q = (W + 2 * padding[1] - dilation[1] * (S - 1) - 1) // stride[1] + 1
    if y is None:
        y = torch.empty((N, K, max(P, 0), max(Q, 0)), dtype=torch.float32, device=x.device)
    elif (tuple(y.shape) != (N, K, P, Q) or y.dtype != torch.float32 or not y.is_contiguous()
          or y.device != x.device):
        raise ValueError("y must be a contiguous float32 N x K x P x Q tensor on x's device")
    need = conv2d_workspace(prm, x.element_size())
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    with torch.cuda.device(x.device):
        rc = raw_conv2d(kind, prm, _ptr(x), _ptr(w), _ptr(y), workspace.data_ptr(), workspace.numel(),
                        _stream_handle(x.device, stream))
    if rc != GEMM_OK:
        raise GemmError(rc, _CONV_STEM[kind])
    return y
