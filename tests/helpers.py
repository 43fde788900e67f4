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
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def tol_f32(K: int) -> float:
    """Elementwise bound for FP32 inputs in [-1, 1]: |C - C_ref| <= 2e-6 K.
    The same bound is used for the normal(0, 1) workload (its entries are
    larger, but so is the FP32 headroom the bound leaves: see the tests)."""
    return 2e-6 * max(K, 1)


def tol_f16(K: int, cref: np.ndarray) -> float:
    """Elementwise bound for binary16 inputs: 2e-3 sqrt(K) max|C_ref|."""
    m = float(np.max(np.abs(cref))) if cref.size else 0.0
    return 2e-3 * np.sqrt(max(K, 1)) * m


@functools.lru_cache(maxsize=None)
def workload(name: str, integer: bool = False):
    """(A, B) numpy inputs of a named workload (cached)."""
    return inputs.workload_matrices(name, integer)


@functools.lru_cache(maxsize=None)
def oracle_full(name: str, integer: bool = False):
    A, B = workload(name, integer)
    if A.dtype == np.float16:
        return oracle.gemm_f16(A, B)
    return oracle.gemm_f32(A, B)


def oracle_at(A, B, rows, cols):
    if A.dtype == np.float16:
        return oracle.gemm_f16_at(A, B, rows, cols)
    return oracle.gemm_f32_at(A, B, rows, cols)


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
