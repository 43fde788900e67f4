"""Build the HIP libraries in-tree, beside this file: ``libdgor_gemm.so`` (the
product), ``libdgor_calibrate.so`` (the benchmark's matrix-core calibration
kernel) and ``libdgor_gemm_poison.so`` (the product built with LDS poisoning,
for the race tests).

Every source in ``csrc/`` is compiled for gfx950 with hipcc (in parallel),
then linked into one shared library that exports the C ABI of
``include/gemm.h``.  Packed FP32 instructions are disabled for all device
code (``-packed-fp32-ops``).

Run as ``python -m dense_gemm_optimisation_row_amd.build``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build", "obj")
LIB = os.path.join(PKG, "libdgor_gemm.so")

SOURCES = ["api.hip", "ladder.hip", "mfma_f32.hip", "mfma_f16.hip", "mfma_8bit.hip", "conv.hip", "conv_nhwc.hip"]
# The matrix-core rate calibration kernel: a library of its own, which the
# GEMM library never loads (only the benchmark's calibration leg calls it).
CAL_SOURCES = ["calibrate.hip"]
CAL_LIB = os.path.join(PKG, "libdgor_calibrate.so")
# The same GEMM library built with -DDGOR_LDS_POISON: every global->LDS load
# first fills its destination with all-ones, so a read that races a load or
# runs ahead of the barrier retiring a buffer sees NaN (a debug build for the
# race tests; the product loads LIB).
POISON_LIB = os.path.join(PKG, "libdgor_gemm_poison.so")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found: the HIP library cannot be built")
    return exe


# Per-file flags.  The channels-last convolution kernels keep their (at most
# 128 a lane) accumulators in ordinary registers: left to choose, the
# compiler starts them in the accumulator registers and moves them between
# the two register files on every k-stage.
FILE_FLAGS = {"conv_nhwc.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(src: str, poison: bool = False) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ("_poison.o" if poison else ".o"))
    cmd = [hipcc(), *FLAGS, *FILE_FLAGS.get(src, []), *(["-DDGOR_LDS_POISON"] if poison else []), "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile all sources, link the GEMM library and the calibration
    library; return the GEMM library's path."""
    os.makedirs(OBJDIR, exist_ok=True)
    jobs_list = [(src, False) for src in SOURCES + CAL_SOURCES] + [(src, True) for src in SOURCES]
    jobs = min(len(jobs_list), max(1, min(8, os.cpu_count() or 1)))
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs_list))
    n = len(SOURCES)
    _link(objs[:n], LIB)
    _link(objs[n:n + len(CAL_SOURCES)], CAL_LIB)
    _link(objs[n + len(CAL_SOURCES):], POISON_LIB)
    if verbose:
        print(f"built {LIB}, {CAL_LIB} and {POISON_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
