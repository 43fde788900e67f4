"""Host build of the matrix-core kernels' workgroup -> tile remap: it must be a
bijection onto the tile grid for every grid shape (checked in C++ against the
very function the kernels call)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="needs hipcc")
def test_tile_remap_is_a_bijection(tmp_path):
    exe = tmp_path / "tile_map_check"
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    subprocess.run([hipcc, "-O1", "-std=c++17", "--offload-arch=gfx950",
                    f"-I{ROOT}/include", f"-I{ROOT}/dense_gemm_optimisation_row_amd/csrc",
                    os.path.join(ROOT, "tests", "cpp", "tile_map_check.cpp"), "-o", str(exe)],
                   check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0, out.stdout + out.stderr
    assert out.stdout.startswith("ok")
