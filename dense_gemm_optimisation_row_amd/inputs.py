"""Seeded synthetic inputs for C = A x B (shared by tests, bench and smoke).

This module only draws random matrices; it holds none of the product's
arithmetic and imports neither the GPU library nor the oracle.  Both sides
are fed the very same arrays from here.

Generator: numpy ``default_rng(seed)`` (PCG64).  A is drawn first, then B,
from one generator per (workload, variant).  Distributions:

* ``uniform``: i.i.d. uniform on [-1, 1) in binary32;
* ``normal``: i.i.d. standard normal, rounded to binary32;
* ``int``: i.i.d. integers in {-4, ..., 4}, so every partial sum of a product
  with K <= 8192 is an integer of magnitude <= 16*K < 2^24, exact in binary32
  whatever the summation order;
* for binary16 inputs the binary32 draw is rounded once to binary16 by numpy
  (round to nearest even) and both sides read the same bits;
* for bfloat16 inputs the binary32 draw is rounded once to its upper 16 bits
  (round to nearest, ties to even), given as uint16 bit patterns;
* for the OCP FP8 formats (E4M3, E5M2) the binary32 draw is rounded once to
  the nearest code (ties to the even code), given as uint8 codes;
* for INT8 inputs the uniform draw on [-1, 1) is scaled by 128 and rounded
  down, giving integers uniform on [-128, 127]; the small-integer variant is
  the {-4..4} draw itself.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    dtype: str          # "f32", "f16", "bf16", "e4m3", "e5m2" or "i8" (input type;
                        # the output is f32, or int32 for i8)
    dist: str           # "uniform" or "normal"
    seed: int           # seed of the main draw
    int_seed: int       # seed of the small-integer variant

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K


# The workloads: square FP32 at 256 and 1024 (1024 is the size the pages time),
# ragged FP32 shapes that exercise edge masking, FP32 4096 with normal inputs,
# FP16-input 8192, BF16-input 8192 (the bfloat16 entry point), and the
# 8-bit inputs (FP8 E4M3, FP8 E5M2, INT8) at 8192.
WORKLOADS = {
    w.name: w for w in [
        Workload("f32_256", 256, 256, 256, "f32", "uniform", 1001, 2001),
        Workload("f32_1024", 1024, 1024, 1024, "f32", "uniform", 1002, 2002),
        Workload("f32_1000", 1000, 1000, 1000, "f32", "uniform", 1003, 2003),
        Workload("f32_4097x33x777", 4097, 33, 777, "f32", "uniform", 1004, 2004),
        Workload("f32_4096", 4096, 4096, 4096, "f32", "normal", 1005, 2005),
        Workload("f16_8192", 8192, 8192, 8192, "f16", "uniform", 1006, 2006),
        Workload("bf16_8192", 8192, 8192, 8192, "bf16", "uniform", 1007, 2007),
        Workload("e4m3_8192", 8192, 8192, 8192, "e4m3", "uniform", 1008, 2008),
        Workload("e5m2_8192", 8192, 8192, 8192, "e5m2", "uniform", 1009, 2009),
        Workload("i8_8192", 8192, 8192, 8192, "i8", "uniform", 1010, 2010),
    ]
}


@dataclass(frozen=True)
class ConvWorkload:
    name: str
    N: int
    C: int
    H: int
    W: int
    K: int
    R: int
    S: int
    stride: int
    pad: int
    dtype: str
    seed: int

    @property
    def out_hw(self):
        P = (self.H + 2 * self.pad - (self.R - 1) - 1) // self.stride + 1
        Q = (self.W + 2 * self.pad - (self.S - 1) - 1) // self.stride + 1
        return P, Q

    @property
    def flops(self) -> int:
        P, Q = self.out_hw
        return 2 * self.N * self.K * P * Q * self.C * self.R * self.S


# Convolution workloads (im2col + GEMM): 3 x 3 layers at a 56 x 56 and a
# 14 x 14 feature map, batch 32, as in image networks; uniform[-1, 1) inputs.
CONV_WORKLOADS = {
    w.name: w for w in [
        ConvWorkload("conv_f16_n32_c64_56x56_k64_3x3", 32, 64, 56, 56, 64, 3, 3, 1, 1, "f16", 1101),
        ConvWorkload("conv_f16_n32_c256_14x14_k256_3x3", 32, 256, 14, 14, 256, 3, 3, 1, 1, "f16", 1102),
        ConvWorkload("conv_f32_n32_c256_14x14_k256_3x3", 32, 256, 14, 14, 256, 3, 3, 1, 1, "f32", 1103),
    ]
}


def conv_tensors(w: ConvWorkload):
    """(x, w) of a convolution workload: N x C x H x W and K x C x R x S."""
    return (tensor((w.N, w.C, w.H, w.W), w.seed, "uniform", w.dtype),
            tensor((w.K, w.C, w.R, w.S), w.seed + 1, "uniform", w.dtype))


def _draw(rng: np.random.Generator, shape, dist: str) -> np.ndarray:
    if dist == "uniform":
        return rng.random(shape, dtype=np.float32) * np.float32(2.0) - np.float32(1.0)
    if dist == "normal":
        return rng.standard_normal(shape, dtype=np.float32)
    if dist == "int":
        return rng.integers(-4, 5, size=shape, dtype=np.int8).astype(np.float32)
    raise ValueError(f"unknown distribution {dist!r}")


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bfloat16 (nearest, ties to even); return
    the 16-bit patterns as uint16.  Adding 0x7FFF plus the lowest kept bit and
    truncating rounds the discarded 16 bits to nearest with ties to even."""
    bits = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    keep_lsb = (bits >> np.uint64(16)) & np.uint64(1)
    return ((bits + np.uint64(0x7FFF) + keep_lsb) >> np.uint64(16)).astype(np.uint16)


def _fp8_grid(exp_bits: int, man_bits: int, finite_codes: int) -> np.ndarray:
    """Values of the non-negative FP8 codes 0 .. finite_codes-1, in code order
    (which is value order): subnormals fraction * 2^(1-bias-man_bits), then
    (2^man_bits + fraction) * 2^(exponent-bias-man_bits)."""
    bias = (1 << (exp_bits - 1)) - 1
    codes = np.arange(finite_codes)
    e = codes >> man_bits
    f = codes & ((1 << man_bits) - 1)
    sub = f * 2.0 ** (1 - bias - man_bits)
    nor = (f + (1 << man_bits)) * np.exp2(e - bias - man_bits)
    return np.where(e == 0, sub, nor)


# E4M3: codes 0..126 finite (127 is NaN); E5M2: codes 0..123 finite.
_E4M3 = _fp8_grid(4, 3, 127)
_E5M2 = _fp8_grid(5, 2, 124)


def to_fp8_codes(x: np.ndarray, fmt: str) -> np.ndarray:
    """Round finite float32 values to the nearest OCP FP8 code of ``fmt``
    ("e4m3" or "e5m2"), ties to the even code; magnitudes beyond the largest
    finite value saturate to it.  Returns uint8 codes."""
    grid = _E4M3 if fmt == "e4m3" else _E5M2
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    ax = np.abs(x)
    mid = (grid[:-1] + grid[1:]) / 2
    code = np.searchsorted(mid, ax, side="left")          # first midpoint >= |x|
    tie = (code < mid.size) & (ax == mid[np.minimum(code, mid.size - 1)])
    code = np.where(tie & (code % 2 == 1), code + 1, code)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def matrices(M: int, N: int, K: int, seed: int, dist: str = "uniform",
             dtype: str = "f32"):
    """Return (A, B): A is M x K, B is K x N, C-contiguous numpy arrays.

    ``dtype`` "f32" gives float32; "f16" gives float16 (the float32 draw
    rounded once to binary16); "bf16" gives uint16 bfloat16 bit patterns (the
    float32 draw rounded once to bfloat16); "e4m3" / "e5m2" give uint8 FP8
    codes (the draw rounded once); "i8" gives int8.
    """
    rng = np.random.default_rng(seed)
    A = _draw(rng, (M, K), dist)
    B = _draw(rng, (K, N), dist)
    return _convert(A, dtype, dist), _convert(B, dtype, dist)


def _convert(X: np.ndarray, dtype: str, dist: str) -> np.ndarray:
    """A binary32 draw in the input format ``dtype`` (see the module notes)."""
    if dtype == "f16":
        X = X.astype(np.float16)
    elif dtype == "bf16":
        X = to_bf16_bits(X)
    elif dtype in ("e4m3", "e5m2"):
        X = to_fp8_codes(X, dtype)
    elif dtype == "i8":
        if dist != "int":
            X = np.floor(X.astype(np.float64) * 128)
        X = np.clip(X, -128, 127).astype(np.int8)
    elif dtype != "f32":
        raise ValueError(f"unknown dtype {dtype!r}")
    return np.ascontiguousarray(X)


def tensor(shape, seed: int, dist: str = "uniform", dtype: str = "f32") -> np.ndarray:
    """One seeded array of any shape in the input format ``dtype``."""
    return _convert(_draw(np.random.default_rng(seed), tuple(shape), dist), dtype, dist)


def workload_matrices(w: Workload | str, integer: bool = False):
    """Inputs of a named workload; ``integer`` selects its small-integer variant."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    if integer:
        return matrices(w.M, w.N, w.K, w.int_seed, "int", w.dtype)
    return matrices(w.M, w.N, w.K, w.seed, w.dist, w.dtype)


def sample_indices(M: int, N: int, count: int, seed: int):
    """``count`` (row, col) pairs: the four corners, the last row and column,
    then uniform random positions.  Used to check outputs one by one."""
    rng = np.random.default_rng(seed)
    fixed_r = [0, 0, M - 1, M - 1, M - 1, M // 2]
    fixed_c = [0, N - 1, 0, N - 1, N // 2, N - 1]
    n_rand = max(0, count - len(fixed_r))
    rows = np.concatenate([np.array(fixed_r), rng.integers(0, M, n_rand)])
    cols = np.concatenate([np.array(fixed_c), rng.integers(0, N, n_rand)])
    return rows.astype(np.int64), cols.astype(np.int64)
