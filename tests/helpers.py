"""Shared helpers of the GPU tests: device tensors, tolerances, comparisons."""
import functools
import sys

import numpy as np

import oracle
from dense_gemm_optimisation_row_amd import inputs


def say(*args):
    """Name the case about to run on the GPU, flushed, so a run that dies
    mid-case still shows which one it was."""
    print("[gpu-case]", *args, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray):
    """numpy -> GPU tensor; uint16 arrays hold bfloat16 bit patterns."""
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to("cuda")
    return torch.from_numpy(a).to("cuda")


def kind(a: np.ndarray) -> str:
    """Input format of a numpy operand: float32, float16 or bfloat16 bits."""
    return {np.dtype(np.float32): "f32", np.dtype(np.float16): "f16",
            np.dtype(np.uint16): "bf16"}[a.dtype]


def tol_f32(K: int) -> float:
    """Elementwise bound for FP32 inputs in [-1, 1]: |C - C_ref| <= 2e-6 K.
    The same bound is used for the normal(0, 1) workload (its entries are
    larger, but so is the FP32 headroom the bound leaves: see the tests)."""
    return 2e-6 * max(K, 1)


def tol_f16(K: int, cref: np.ndarray) -> float:
    """Elementwise bound for 16-bit inputs (binary16, and bfloat16 under the
    same reading: products of two 16-bit values are exact in binary32 either
    way, so only the binary32 accumulation errs): 2e-3 sqrt(K) max|C_ref|."""
    m = float(np.max(np.abs(cref))) if cref.size else 0.0
    return 2e-3 * np.sqrt(max(K, 1)) * m


@functools.lru_cache(maxsize=None)
def workload(name: str, integer: bool = False):
    """(A, B) numpy inputs of a named workload (cached)."""
    return inputs.workload_matrices(name, integer)


def as_f32(a: np.ndarray) -> np.ndarray:
    """The binary32 values of a numpy operand of any input format (a
    bfloat16 pattern is the upper half of the binary32 with its value)."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return a.astype(np.float32)


def oracle_gemm(A, B):
    """Full oracle product for any input format."""
    return {"f32": oracle.gemm_f32, "f16": oracle.gemm_f16, "bf16": oracle.gemm_bf16}[kind(A)](A, B)


@functools.lru_cache(maxsize=None)
def oracle_full(name: str, integer: bool = False):
    A, B = workload(name, integer)
    return oracle_gemm(A, B)


def oracle_at(A, B, rows, cols):
    f = {"f32": oracle.gemm_f32_at, "f16": oracle.gemm_f16_at, "bf16": oracle.gemm_bf16_at}[kind(A)]
    return f(A, B, rows, cols)


def assert_bits_equal(got: np.ndarray, ref: np.ndarray, what: str):
    # +0 and -0 compare equal: a zero-filled tile may add -0 terms
    bad = ~(got == ref)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} elements differ, first at "
                             f"{idx.tolist()}: got {got[tuple(idx[0])]} want {ref[tuple(idx[0])]}")


def assert_within(got: np.ndarray, ref: np.ndarray, tol: float, what: str):
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    worst = float(err.max()) if err.size else 0.0
    assert worst <= tol, f"{what}: max |dC| = {worst:.3e} > {tol:.3e} at {np.unravel_index(err.argmax(), err.shape)}"
    return worst
