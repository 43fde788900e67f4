"""CPU oracle for C = A x B (row-major, FP32 result) -- test infrastructure.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library never loads it, and it
imports nothing from the GPU library: the two share no code.

The arithmetic lives in ``oracle.c`` (plain loops, binary64 accumulation in
ascending k, one rounding to binary32).  This module only compiles that file
with gcc and marshals numpy arrays into it through ctypes.

Sources followed: "Lesson 8: how a GPU does matrix multiply", section 1
(C[i,j] = sum_k A[i,k] B[k,j]) and section 2 (row-major indexing); "SGEMM
optimisation journey", Level 1; "4. GEMM optimisation", section 4.1.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# -ffp-contract=off: no fused multiply-add may merge a product into the sum.
# -fno-fast-math: keep IEEE semantics (no reassociation of the k-sum).
CFLAGS = ["-O2", "-fopenmp", "-fno-fast-math", "-ffp-contract=off", "-fPIC",
          "-shared", "-std=c11", "-Wall", "-Wextra"]

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so beside it (gcc) and return the path."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def configure(lib):
    """Declare the C signatures on a loaded oracle library and return it."""
    p = ctypes.c_void_p
    i = ctypes.c_int
    i64 = ctypes.c_int64
    for name in ("oracle_f16_to_f64", "oracle_bf16_to_f64"):
        f = getattr(lib, name)
        f.argtypes = [ctypes.c_uint16]
        f.restype = ctypes.c_double
    lib.oracle_threads.argtypes = [i]
    lib.oracle_threads.restype = i
    for name in ("oracle_gemm_f32", "oracle_gemm_f16", "oracle_gemm_bf16"):
        f = getattr(lib, name)
        f.argtypes = [i, i, i, p, p, p, i]
        f.restype = i
    for name in ("oracle_gemm_f32_at", "oracle_gemm_f16_at", "oracle_gemm_bf16_at"):
        f = getattr(lib, name)
        f.argtypes = [i, i, i, p, p, i64, p, p, p, i]
        f.restype = i
    for name in ("oracle_e4m3_to_f64", "oracle_e5m2_to_f64"):
        f = getattr(lib, name)
        f.argtypes = [ctypes.c_uint8]
        f.restype = ctypes.c_double
    for name in ("oracle_gemm_e4m3", "oracle_gemm_e5m2", "oracle_gemm_i8"):
        f = getattr(lib, name)
        f.argtypes = [i, i, i, p, p, p, i]
        f.restype = i
    lib.oracle_gemm_fp8_at.argtypes = [i, i, i, i, p, p, i64, p, p, p, i]
    lib.oracle_gemm_fp8_at.restype = i
    lib.oracle_gemm_i8_at.argtypes = [i, i, i, p, p, i64, p, p, p, i]
    lib.oracle_gemm_i8_at.restype = i
    lib.oracle_conv2d.argtypes = [i] * 14 + [p, p, p, i]
    lib.oracle_conv2d.restype = i
    d = ctypes.c_double
    lib.oracle_gemm_ex.argtypes = [i, i, i, i, i, i, d, p, i, p, i, d, p, i, i]
    lib.oracle_gemm_ex.restype = i
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = configure(ctypes.CDLL(_LIB))
    return _lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data) if a.size else None


def _check_inputs(A, B, dtype):
    A = np.ascontiguousarray(A)
    B = np.ascontiguousarray(B)
    if A.dtype != dtype or B.dtype != dtype:
        raise TypeError(f"oracle expects {np.dtype(dtype).name} inputs")
    if A.ndim != 2 or B.ndim != 2 or A.shape[1] != B.shape[0]:
        raise ValueError(f"shapes {A.shape} x {B.shape} do not chain")
    return A, B


def threads(nthreads: int = 0) -> int:
    """Threads the oracle uses for a request of ``nthreads`` (0 = OpenMP default)."""
    return int(_load().oracle_threads(nthreads))


def f16_to_f64(bits: int) -> float:
    """Decode one IEEE binary16 bit pattern exactly."""
    return float(_load().oracle_f16_to_f64(int(bits) & 0xFFFF))


def bf16_to_f64(bits: int) -> float:
    """Decode one bfloat16 bit pattern exactly."""
    return float(_load().oracle_bf16_to_f64(int(bits) & 0xFFFF))


def gemm_f32(A: np.ndarray, B: np.ndarray, out: np.ndarray | None = None,
             nthreads: int = 0) -> np.ndarray:
    """C = A x B for float32 A (M x K), B (K x N); binary64 sum, binary32 result.

    ``out`` (float32, M x N, contiguous) is overwritten when given; with M or N
    zero nothing is written.
    """
    A, B = _check_inputs(A, B, np.float32)
    M, K = A.shape
    N = B.shape[1]
    C = np.empty((M, N), np.float32) if out is None else out
    if C.shape != (M, N) or C.dtype != np.float32 or not C.flags.c_contiguous:
        raise ValueError("out must be a contiguous float32 M x N array")
    rc = _load().oracle_gemm_f32(M, N, K, _ptr(A), _ptr(B), _ptr(C), nthreads)
    if rc != 0:
        raise RuntimeError(f"oracle_gemm_f32 failed ({rc})")
    return C


def gemm_f16(A: np.ndarray, B: np.ndarray, out: np.ndarray | None = None,
             nthreads: int = 0) -> np.ndarray:
    """C = A x B for binary16 A, B (numpy float16 or uint16 bit patterns)."""
    A = np.ascontiguousarray(A).view(np.uint16) if np.asarray(A).dtype == np.float16 else A
    B = np.ascontiguousarray(B).view(np.uint16) if np.asarray(B).dtype == np.float16 else B
    A, B = _check_inputs(A, B, np.uint16)
    M, K = A.shape
    N = B.shape[1]
    C = np.empty((M, N), np.float32) if out is None else out
    if C.shape != (M, N) or C.dtype != np.float32 or not C.flags.c_contiguous:
        raise ValueError("out must be a contiguous float32 M x N array")
    rc = _load().oracle_gemm_f16(M, N, K, _ptr(A), _ptr(B), _ptr(C), nthreads)
    if rc != 0:
        raise RuntimeError(f"oracle_gemm_f16 failed ({rc})")
    return C


def gemm_bf16(A: np.ndarray, B: np.ndarray, out: np.ndarray | None = None,
              nthreads: int = 0) -> np.ndarray:
    """C = A x B for bfloat16 A, B given as uint16 bit patterns."""
    A, B = _check_inputs(A, B, np.uint16)
    M, K = A.shape
    N = B.shape[1]
    C = np.empty((M, N), np.float32) if out is None else out
    if C.shape != (M, N) or C.dtype != np.float32 or not C.flags.c_contiguous:
        raise ValueError("out must be a contiguous float32 M x N array")
    rc = _load().oracle_gemm_bf16(M, N, K, _ptr(A), _ptr(B), _ptr(C), nthreads)
    if rc != 0:
        raise RuntimeError(f"oracle_gemm_bf16 failed ({rc})")
    return C


def _at(fname, A, B, rows, cols, nthreads):
    M, K = A.shape
    N = B.shape[1]
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.shape != cols.shape:
        raise ValueError("rows and cols must have the same shape")
    out = np.empty(rows.shape, np.float32)
    rc = getattr(_load(), fname)(M, N, K, _ptr(A), _ptr(B), rows.size,
                                 _ptr(rows), _ptr(cols), _ptr(out), nthreads)
    if rc != 0:
        raise RuntimeError(f"{fname} failed ({rc})")
    return out


def gemm_f32_at(A, B, rows, cols, nthreads: int = 0) -> np.ndarray:
    """C[rows[t], cols[t]] of A x B for float32 inputs, one dot product each."""
    A, B = _check_inputs(A, B, np.float32)
    return _at("oracle_gemm_f32_at", A, B, rows, cols, nthreads)


def gemm_f16_at(A, B, rows, cols, nthreads: int = 0) -> np.ndarray:
    """C[rows[t], cols[t]] of A x B for binary16 inputs, one dot product each."""
    A = np.ascontiguousarray(A).view(np.uint16) if np.asarray(A).dtype == np.float16 else A
    B = np.ascontiguousarray(B).view(np.uint16) if np.asarray(B).dtype == np.float16 else B
    A, B = _check_inputs(A, B, np.uint16)
    return _at("oracle_gemm_f16_at", A, B, rows, cols, nthreads)


def gemm_bf16_at(A, B, rows, cols, nthreads: int = 0) -> np.ndarray:
    """C[rows[t], cols[t]] of A x B for bfloat16 bit-pattern inputs, one dot product each."""
    A, B = _check_inputs(A, B, np.uint16)
    return _at("oracle_gemm_bf16_at", A, B, rows, cols, nthreads)


_IN_CODE = {"f32": 0, "f16": 1, "bf16": 2}


def gemm_ex(fmt: str, op_a: int, op_b: int, M: int, N: int, K: int, alpha: float,
            A: np.ndarray, lda: int, B: np.ndarray, ldb: int, beta: float,
            C: np.ndarray, ldc: int, nthreads: int = 0) -> np.ndarray:
    """C = alpha op(A) op(B) + beta C in place on the flat float32 array C
    (row stride ldc); A and B are flat arrays holding the operands with the
    given row strides (binary16 as float16 or uint16 bits, bfloat16 as uint16
    bits).  Returns C."""
    code = _IN_CODE[fmt]
    A = np.ascontiguousarray(A)
    B = np.ascontiguousarray(B)
    if fmt == "f16":
        A = A.view(np.uint16) if A.dtype == np.float16 else A
        B = B.view(np.uint16) if B.dtype == np.float16 else B
    want = np.float32 if fmt == "f32" else np.uint16
    if A.dtype != want or B.dtype != want:
        raise TypeError(f"{fmt} oracle expects {np.dtype(want).name} operands")
    if C.dtype != np.float32 or not C.flags.c_contiguous:
        raise ValueError("C must be a contiguous float32 array")
    need_a = ((K - 1) * lda + M if op_a else (M - 1) * lda + K) if M and K else 0
    need_b = ((N - 1) * ldb + K if op_b else (K - 1) * ldb + N) if N and K else 0
    need_c = (M - 1) * ldc + N if M and N else 0
    if A.size < need_a or B.size < need_b or C.size < need_c:
        raise ValueError("operand arrays too small for the given shape and strides")
    rc = _load().oracle_gemm_ex(code, op_a, op_b, M, N, K, float(alpha), _ptr(A), lda, _ptr(B), ldb,
                                float(beta), _ptr(C), ldc, nthreads)
    if rc != 0:
        raise RuntimeError(f"oracle_gemm_ex failed ({rc})")
    return C


# ------------------------------------------------------------ 8-bit inputs --

def e4m3_to_f64(code: int) -> float:
    """Decode one OCP FP8 E4M3 code exactly."""
    return float(_load().oracle_e4m3_to_f64(int(code) & 0xFF))


def e5m2_to_f64(code: int) -> float:
    """Decode one OCP FP8 E5M2 code exactly."""
    return float(_load().oracle_e5m2_to_f64(int(code) & 0xFF))


def _gemm8(fname, A, B, dtype, out_dtype, out, nthreads):
    A, B = _check_inputs(A, B, dtype)
    M, K = A.shape
    N = B.shape[1]
    C = np.empty((M, N), out_dtype) if out is None else out
    if C.shape != (M, N) or C.dtype != out_dtype or not C.flags.c_contiguous:
        raise ValueError(f"out must be a contiguous {np.dtype(out_dtype).name} M x N array")
    rc = getattr(_load(), fname)(M, N, K, _ptr(A), _ptr(B), _ptr(C), nthreads)
    if rc != 0:
        raise RuntimeError(f"{fname} failed ({rc})")
    return C


def gemm_e4m3(A, B, out=None, nthreads: int = 0) -> np.ndarray:
    """C = A x B for FP8 E4M3 codes (uint8) A, B; binary64 sum, binary32 result."""
    return _gemm8("oracle_gemm_e4m3", A, B, np.uint8, np.float32, out, nthreads)


def gemm_e5m2(A, B, out=None, nthreads: int = 0) -> np.ndarray:
    """C = A x B for FP8 E5M2 codes (uint8) A, B; binary64 sum, binary32 result."""
    return _gemm8("oracle_gemm_e5m2", A, B, np.uint8, np.float32, out, nthreads)


def gemm_i8(A, B, out=None, nthreads: int = 0) -> np.ndarray:
    """C = A x B for int8 A, B; exact, int32 result (error if it overflows)."""
    return _gemm8("oracle_gemm_i8", A, B, np.int8, np.int32, out, nthreads)


def _at8(A, B, rows, cols, nthreads, fmt=None):
    M, K = A.shape
    N = B.shape[1]
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.shape != cols.shape:
        raise ValueError("rows and cols must have the same shape")
    lib = _load()
    if fmt is None:
        out = np.empty(rows.shape, np.int32)
        rc = lib.oracle_gemm_i8_at(M, N, K, _ptr(A), _ptr(B), rows.size, _ptr(rows), _ptr(cols),
                                   _ptr(out), nthreads)
    else:
        out = np.empty(rows.shape, np.float32)
        rc = lib.oracle_gemm_fp8_at(fmt, M, N, K, _ptr(A), _ptr(B), rows.size, _ptr(rows), _ptr(cols),
                                    _ptr(out), nthreads)
    if rc != 0:
        raise RuntimeError(f"8-bit sampled oracle failed ({rc})")
    return out


def gemm_e4m3_at(A, B, rows, cols, nthreads: int = 0) -> np.ndarray:
    A, B = _check_inputs(A, B, np.uint8)
    return _at8(A, B, rows, cols, nthreads, 0)


def gemm_e5m2_at(A, B, rows, cols, nthreads: int = 0) -> np.ndarray:
    A, B = _check_inputs(A, B, np.uint8)
    return _at8(A, B, rows, cols, nthreads, 1)


def gemm_i8_at(A, B, rows, cols, nthreads: int = 0) -> np.ndarray:
    A, B = _check_inputs(A, B, np.int8)
    return _at8(A, B, rows, cols, nthreads)


# -------------------------------------------------------------- convolution --

def conv2d_out_size(H: int, W: int, R: int, S: int, stride=(1, 1), pad=(0, 0), dil=(1, 1)):
    """(P, Q) of a convolution of an H x W image with an R x S filter."""
    P = (H + 2 * pad[0] - dil[0] * (R - 1) - 1) // stride[0] + 1
    Q = (W + 2 * pad[1] - dil[1] * (S - 1) - 1) // stride[1] + 1
    return P, Q


def conv2d(fmt: str, x: np.ndarray, w: np.ndarray, stride=(1, 1), pad=(0, 0), dil=(1, 1),
           nthreads: int = 0) -> np.ndarray:
    """Direct 2-D convolution (cross-correlation), x N x C x H x W, w K x C x R x S
    (binary32, binary16 as float16 or uint16 bits, bfloat16 as uint16 bits);
    returns y N x K x P x Q in binary32."""
    code = _IN_CODE[fmt]
    x = np.ascontiguousarray(x)
    w = np.ascontiguousarray(w)
    if fmt == "f16":
        x = x.view(np.uint16) if x.dtype == np.float16 else x
        w = w.view(np.uint16) if w.dtype == np.float16 else w
    want = np.float32 if fmt == "f32" else np.uint16
    if x.dtype != want or w.dtype != want or x.ndim != 4 or w.ndim != 4 or x.shape[1] != w.shape[1]:
        raise ValueError("x must be N x C x H x W and w K x C x R x S of the input format")
    N, C, H, W = x.shape
    K, _, R, S = w.shape
    P, Q = conv2d_out_size(H, W, R, S, stride, pad, dil)
    if P <= 0 or Q <= 0:
        raise ValueError("empty output")
    y = np.empty((N, K, P, Q), np.float32)
    rc = _load().oracle_conv2d(code, N, C, H, W, K, R, S, stride[0], stride[1], pad[0], pad[1], dil[0], dil[1],
                               _ptr(x), _ptr(w), _ptr(y), nthreads)
    if rc != 0:
        raise RuntimeError(f"oracle_conv2d failed ({rc})")
    return y
