"""CPU-side checks of the C ABI: the library loads and exports every function
include/gemm.h declares, the header is plain C, the launch planner agrees
with the tile arithmetic the pages print, and argument validation rejects bad
calls before anything touches a device.  No kernel is launched here."""
import ctypes
import os
import re
import shutil
import subprocess

import pytest

import dense_gemm_optimisation_row_amd as dg
from dense_gemm_optimisation_row_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gemm.h")
GOLDEN = os.path.join(ROOT, "tests", "golden", "tile_arithmetic.txt")


def _golden():
    vals = {}
    for line in open(GOLDEN):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split("=")
            vals[k.strip()] = int(v)
    return vals


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gemm_\w+)\s*\(", text)))


def test_header_declares_the_documented_entry_points():
    assert _declared_functions() == sorted(binding.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(binding.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(lib, name), name
    nm = shutil.which("nm")
    if nm:
        out = subprocess.run([nm, "-D", "--defined-only", binding.LIB_PATH],
                             capture_output=True, text=True, check=True).stdout
        exported = set(re.findall(r"\bT (gemm_\w+)$", out, flags=re.M))
        assert exported == set(_declared_functions())


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_header_is_plain_c(tmp_path):
    src = tmp_path / "use.c"
    src.write_text('#include "gemm.h"\n'
                   'int main(void) { gemm_plan p; (void)p;\n'
                   '  return gemm_f32(0, 0, 0, 0, 0, 0, 0) == GEMM_OK ? 0 : 1; }\n')
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
                    f"-I{os.path.dirname(HEADER)}", "-c", str(src), "-o", str(tmp_path / "u.o")],
                   check=True)


def test_status_and_variant_names():
    assert dg.status_string(0) == "ok"
    for s in range(-8, 0):
        assert dg.status_string(s) and dg.status_string(s) != "unknown status"
    assert dg.status_string(-99) == "unknown status"
    for v in range(9):
        assert dg.variant_name(v).startswith(f"R{v} ")
    assert dg.variant_name(42) == "unknown variant"


# ------------------------------------------------ planner vs the pages ---

def test_planner_matches_lesson8_tile_arithmetic():
    gold = _golden()
    p = dg.plan(False, 1000, 1000, 64, variant=dg.R1_LDS_TILED)
    assert p["threads"] == gold["block16_threads"]
    assert p["tile_m"] == p["tile_n"] == p["tile_k"] == 16
    first = (p["grid_y"] - 1) * p["tile_m"]
    assert first == gold["m1000_tile16_last_tile_first_row"]
    assert first + p["tile_m"] - 1 == gold["m1000_tile16_last_tile_last_row"]
    assert 1000 - 1 == gold["m1000_tile16_last_valid_row"]
    assert p["k_stages"] == gold["k64_tile16_stages"]
    assert p["tile_m"] * p["tile_k"] + p["tile_k"] * p["tile_n"] == gold["tile16_stage_loads"]
    assert p["tile_m"] * p["tile_n"] * p["tile_k"] == gold["tile16_stage_multiplies"]
    assert p["lds_bytes"] == p["tile_bytes"] == gold["tile16_pair_bytes"]
    assert 2 * 32 * 32 * 4 == gold["tile32_pair_bytes"]


def test_planner_matches_sgemm_journey_level5_resources():
    gold = _golden()
    p = dg.plan(False, 4096, 4096, 4096, variant=dg.R5_REGISTER_BLOCKED)
    assert (p["tile_m"], p["tile_n"], p["tile_k"]) == (128, 128, 8)
    tm = tn = 8
    assert p["threads"] == (128 // tm) * (128 // tn) == gold["regblock_threads"]
    assert p["tile_bytes"] == gold["regblock_smem_bytes"]
    assert p["outputs_per_thread"] + tm + tn == gold["regblock_registers"]
    assert p["lds_stages"] == 2 and p["lds_bytes"] > p["tile_bytes"]   # double-buffered, padded


# ------------------------------------------------------ planner behaviour --

def test_grid_is_ceil_div_for_every_variant():
    for half, variants in ((False, dg.F32_VARIANTS), (True, dg.F16_VARIANTS)):
        for v in variants:
            for (M, N, K) in [(1, 1, 1), (1000, 1000, 1000), (4097, 33, 777), (256, 256, 256)]:
                p = dg.plan(half, M, N, K, variant=v)
                assert p["variant"] == v and p["launches"] == 1
                if not half and v == dg.R6_MFMA_F32 and N <= 64 and p["tile_m"] == 16:
                    # the tall, narrow kernel: all columns in one workgroup; a
                    # last row of its own is spread over the first N
                    # workgroups when there are at least N whole row blocks
                    tail = M % 16 == 1 and M // 16 >= N
                    assert p["grid_x"] == 1 and p["tile_n"] >= N
                    assert p["grid_y"] == (M // 16 if tail else -(-M // 16))
                    continue
                assert p["grid_x"] == -(-N // p["tile_n"]) and p["grid_y"] == -(-M // p["tile_m"])
                assert (p["grid_x"] - 1) * p["tile_n"] < N and (p["grid_y"] - 1) * p["tile_m"] < M
                if p["tile_k"]:
                    assert p["k_stages"] == -(-K // p["tile_k"])
                assert p["lds_bytes"] <= 160 * 1024
                assert p["threads"] <= 1024 and p["threads"] % 64 == 0


def test_auto_picks_matrix_cores_and_tile_by_size():
    big = dg.plan(False, 4096, 4096, 4096)
    # aligned operands with a tile per compute unit: the 256 x 256 ring
    assert big["variant"] == dg.R6_MFMA_F32 and (big["tile_m"], big["tile_n"]) == (256, 256)
    assert big["grid_x"] * big["grid_y"] == 256 and big["lds_stages"] == 4
    # the same shape with A off 16-byte alignment: 128 x 128, two per compute unit
    odd = dg.plan(False, 4096, 4096, 4096, A=4)
    assert (odd["tile_m"], odd["tile_n"]) == (128, 128) and odd["vector_a"] == 0
    assert odd["grid_x"] * odd["grid_y"] >= 512
    small = dg.plan(False, 1024, 1024, 1024)
    assert small["variant"] == dg.R6_MFMA_F32 and small["grid_x"] * small["grid_y"] >= 256
    # tall and narrow (N <= 64, K <= 1024): one workgroup of 512 threads per
    # 16 rows, all columns and all of K.  4097 x 33: two 16-column MFMA
    # blocks plus the 33rd column on the vector ALUs (tile_n 33), and the
    # 4097th row spread over workgroups 0..32 rather than given a 257th
    skinny = dg.plan(False, 4097, 33, 777)
    assert (skinny["tile_m"], skinny["tile_n"], skinny["grid_x"], skinny["grid_y"]) == (16, 33, 1, 256)
    # two column blocks: each wavefront holds its whole run of B in LDS (8
    # slices of 16 rows x 32 columns, and the last column in 512 bytes)
    assert skinny["tile_k"] == 784 and skinny["threads"] == 512 and skinny["lds_stages"] == 8
    assert skinny["lds_bytes"] == 8 * (8 * 2048 + 512) + 32
    # alignment of B does not change the plan
    odd_b = dg.plan(False, 4097, 33, 777, B=0x1004)
    assert (odd_b["lds_stages"], odd_b["lds_bytes"]) == (skinny["lds_stages"], skinny["lds_bytes"])
    assert dg.plan(False, 4097, 33, 1024)["lds_stages"] == 8
    # three or four blocks: a ring of 4 (3) LDS slots a wavefront (A's 1 KB,
    # B's 16 rows x 16 NB columns, the last column in 256 bytes) plus 1 KB
    # for the tail row's products
    wide = dg.plan(False, 4097, 64, 1024)
    assert wide["tile_n"] == 64 and wide["lds_stages"] == 3
    assert wide["lds_bytes"] == 8 * (3 * (1024 + 4096) + 1024) + 32 <= 160 * 1024
    mid = dg.plan(False, 4097, 49, 777)
    assert mid["tile_n"] == 49 and mid["lds_stages"] == 4
    assert mid["lds_bytes"] == 8 * (4 * (1024 + 3072 + 256) + 1024) + 32 <= 160 * 1024
    assert dg.plan(False, 4097, 64, 256)["lds_stages"] == 3
    # M N past 2^31 bytes of C: not the tall, narrow kernel
    assert dg.plan(False, 1 << 24, 64, 1)["tile_m"] != 16
    # a last row block of 2..15 rows, or one row with fewer whole blocks than
    # columns: a workgroup of its own
    assert dg.plan(False, 4098, 33, 777)["grid_y"] == 257
    assert dg.plan(False, 33, 40, 777)["grid_y"] == 3
    assert dg.plan(False, 4097, 32, 777)["grid_y"] == 256 and dg.plan(False, 4097, 32, 777)["tile_n"] == 32
    assert (dg.plan(False, 4000, 64, 512)["tile_m"], dg.plan(False, 4000, 64, 512)["tile_n"]) == (16, 64)
    assert (dg.plan(False, 4097, 64, 1024)["tile_m"], dg.plan(False, 4097, 64, 1024)["tile_n"]) == (16, 64)
    assert dg.plan(False, 100, 20, 9)["tile_n"] == 32          # N % 16 > 1: a padded block
    # K past 1024: the 32 x 64 tile
    assert (dg.plan(False, 4097, 16, 2048)["tile_m"], dg.plan(False, 4097, 16, 2048)["tile_n"]) == (32, 64)
    h = dg.plan(True, 8192, 8192, 8192)
    assert h["variant"] == dg.R7_MFMA_F16 and (h["tile_m"], h["tile_n"]) == (256, 256)


def test_direct_load_tile_follows_the_spread_of_tiles_over_compute_units():
    """Aligned FP32 operands take whichever of the 256, 128 and 64 square
    direct-load tiles has the best measured rate times the evenness of its
    tiles over the 256 compute units; 16-bit operands take the 256 x 256 ring
    from 128 of its tiles."""
    tile = lambda half, M, N, K: dg.plan(half, M, N, K)["tile_m"]
    assert tile(False, 4096, 4096, 4096) == 256     # 256 tiles, one per unit
    assert tile(False, 8192, 8192, 8192) == 256     # 1024: four per unit
    assert tile(False, 6144, 6144, 6144) == 128     # 576 ring tiles leave a quarter round; 2304 of 128^2
    assert tile(False, 5120, 5120, 5120) == 64      # 400 ring tiles, 1600 of 128^2 (7 on some units)
    assert tile(False, 3072, 3072, 3072) == 64      # 576 of 128^2 (three on some units) against 2304 of 64^2
    assert tile(False, 4096, 2048, 2048) == 128     # 512 of 128^2: two per unit
    assert tile(False, 2048, 2048, 2048) == 64      # 256 of 128^2, one per unit: 1024 of 64^2
    assert tile(False, 1024, 1024, 1024) == 64
    assert tile(True, 4096, 4096, 4096) == 256
    assert tile(True, 3072, 3072, 3072) == 256      # 144 ring tiles
    assert tile(True, 2048, 2048, 2048) == 128      # 64 ring tiles: too few; the 128 x 128 ring
    # one tile per unit: two groups of four wavefronts over halves of k, two 80 KB rings
    assert dg.plan(True, 2048, 2048, 2048)["lds_bytes"] == 163840 and dg.plan(True, 2048, 2048, 2048)["threads"] == 512
    assert tile(True, 2560, 2560, 2560) == 128 and dg.plan(True, 2560, 2560, 2560)["threads"] == 256   # 400 tiles
    assert dg.plan(True, 2560, 2560, 2560)["lds_bytes"] == 81920
    assert tile(True, 1000, 1001, 1000) == 64       # rows not whole 16-byte units: register-staged
    # K % 8 != 0: A's rows are not whole 16-byte units, so no direct loads
    assert tile(True, 4096, 4096, 4095) == 128 and dg.plan(True, 4096, 4096, 4095)["vector_a"] == 0


def test_f32_64_ring_splits_k_over_two_groups_with_one_tile_per_unit():
    """The 64 x 64 ring's workgroup becomes two groups of eight wavefronts
    over halves of the k-stages (1024 threads, two 64 KB rings) when the shape
    has at most 256 of its tiles and K >= 512."""
    for M, N, K in ((1024, 1024, 1024), (1000, 1000, 1000), (1024, 1024, 4096), (512, 512, 512), (40, 1000, 600)):
        p = dg.plan(False, M, N, K)
        assert (p["tile_m"], p["threads"], p["lds_bytes"], p["k_stages"]) == (64, 1024, 131072, -(-K // 32))
    for M, N, K in ((2048, 2048, 2048), (1024, 1024, 256), (256, 256, 256), (1536, 1536, 1536)):
        p = dg.plan(False, M, N, K)
        assert (p["tile_m"], p["threads"], p["lds_bytes"]) == (64, 512, 65536)


def test_vector_path_needs_divisible_rows_and_16_byte_alignment():
    p = dg.plan(False, 64, 64, 64)
    assert p["vector_a"] == p["vector_b"] == 1
    p = dg.plan(False, 4097, 33, 777)
    assert p["vector_a"] == 0 and p["vector_b"] == 0
    p = dg.plan(False, 64, 64, 64, A=0x1004, B=0x1000, C=0x1000)   # A offset by one float
    assert p["vector_a"] == 0 and p["vector_b"] == 1
    p = dg.plan(True, 64, 64, 64)
    assert p["vector_a"] == p["vector_b"] == 1
    p = dg.plan(True, 64, 60, 68)            # f16 needs multiples of 8 halves
    assert p["vector_a"] == 0 and p["vector_b"] == 0


def test_8bit_plans_take_the_ring_when_operands_are_aligned():
    for kind in ("e4m3", "e5m2", "i8"):
        p = dg.plan(kind, 8192, 8192, 8192)
        assert p["variant"] == dg.R8_MFMA_8BIT and (p["tile_m"], p["tile_n"], p["tile_k"]) == (256, 256, 64)
        # A in three two-step buffers, B in four one-step buffers: all 160 KB of LDS
        assert p["lds_stages"] == 4 and p["lds_bytes"] == 163840 and p["k_stages"] == 128
        assert p["grid_x"] * p["grid_y"] == 1024 and p["outputs_per_thread"] == 256
        # rows read along k must be whole 16-byte vectors, and both operands 16-byte aligned
        assert dg.plan(kind, 300, 272, 80)["variant"] == dg.R8_MFMA_8BIT
        assert dg.plan(kind, 300, 272, 88)["variant"] == dg.R0_NAIVE
        assert dg.plan(kind, 300, 264, 80)["variant"] == dg.R0_NAIVE
        assert dg.plan(kind, 256, 256, 256, A=8)["variant"] == dg.R0_NAIVE
        # forcing R8 on a call the ring cannot take runs R0; forcing R0 runs R0
        assert dg.plan(kind, 300, 264, 80, variant=dg.R8_MFMA_8BIT)["variant"] == dg.R0_NAIVE
        assert dg.plan(kind, 256, 256, 256, variant=dg.R0_NAIVE)["variant"] == dg.R0_NAIVE
        for bad in (1, 6, 7, 9):
            with pytest.raises(dg.GemmError) as e:
                dg.plan(kind, 4, 4, 4, variant=bad)
            assert e.value.status == binding.GEMM_ERR_INVALID_VARIANT
        z = dg.plan(kind, 5, 6, 0)
        assert z["launches"] == 1 and z["tile_k"] == 0
    # INT8: 128 * 128 * K must fit int32
    assert dg.plan("i8", 4, 4, 131072)["launches"] == 1
    with pytest.raises(dg.GemmError) as e:
        dg.plan("i8", 4, 4, 131073)
    assert e.value.status == binding.GEMM_ERR_INVALID_DIM
    assert dg.plan("e4m3", 4, 4, 131088)["launches"] == 1


def test_8bit_ring_tile_follows_the_spread_of_tiles_over_compute_units():
    """The 8-bit formats take the 128 x 128 ring where its measured rate times
    the evenness of its tiles over the 256 compute units beats the 256 x 256
    ring's."""
    tile = lambda kind, M, N, K: dg.plan(kind, M, N, K)["tile_m"]
    for kind in ("e4m3", "e5m2", "i8"):
        assert tile(kind, 8192, 8192, 8192) == 256      # 1024 ring tiles
        assert tile(kind, 4096, 4096, 4096) == 256      # 256 ring tiles, one per unit
        assert tile(kind, 6144, 6144, 6144) == 256      # 576 ring tiles against 2304 of 128^2
        assert tile(kind, 4096, 2048, 2048) == 128      # 128 ring tiles: half the units idle
        assert tile(kind, 2560, 2560, 2560) == 128      # 100 ring tiles against 400 of 128^2
        assert tile(kind, 2048, 2048, 2048) == 128
        assert tile(kind, 300, 272, 80) == 128
        p = dg.plan(kind, 2048, 2048, 2048)
        # three 16 KB A pair buffers and four 8 KB B steps; with one tile per
        # unit, two such rings for two groups of wavefronts over halves of k
        assert p["lds_bytes"] == 163840 and p["threads"] == 512 and p["lds_stages"] == 4 and p["tile_k"] == 64
        assert p["grid_x"] * p["grid_y"] == 256 and p["outputs_per_thread"] == 64 and p["tile_bytes"] == 16384
        p = dg.plan(kind, 2560, 2560, 2560)   # 400 tiles: one group, two workgroups a unit
        assert p["tile_m"] == 128 and p["lds_bytes"] == 81920 and p["threads"] == 256
    # 144 ring tiles against 576 of 128^2: INT8 takes the smaller tile, FP8
    # (whose larger tile runs faster with units idle) the larger
    assert tile("i8", 3072, 3072, 3072) == 128
    assert tile("e4m3", 3072, 3072, 3072) == 256 and tile("e5m2", 3072, 3072, 3072) == 256


def test_8bit_entry_points_validate_before_touching_a_device():
    raw = binding.raw_gemm
    for kind in ("e4m3", "e5m2", "i8"):
        assert raw(kind, None, -1, 4, 4, 16, 16, 16, None) == binding.GEMM_ERR_INVALID_DIM
        assert raw(kind, None, 4, 4, 4, None, 16, 16, None) == binding.GEMM_ERR_NULL_PTR
        assert raw(kind, None, 0, 4, 4, None, 16, None, None) == binding.GEMM_OK
        assert raw(kind, 7, 4, 4, 4, 16, 16, 16, None) == binding.GEMM_ERR_INVALID_VARIANT
    assert raw("i8", None, 4, 4, 200000, 16, 16, 16, None) == binding.GEMM_ERR_INVALID_DIM


def test_empty_and_k0_plans():
    assert dg.plan(False, 0, 5, 7)["launches"] == 0
    assert dg.plan(True, 5, 0, 7)["launches"] == 0
    z = dg.plan(False, 5, 6, 0)
    assert z["launches"] == 1 and z["tile_k"] == 0


def test_planner_rejects_bad_arguments():
    with pytest.raises(dg.GemmError) as e:
        dg.plan(False, -1, 4, 4)
    assert e.value.status == binding.GEMM_ERR_INVALID_DIM
    for bad in (7, 8, -2, 100):
        with pytest.raises(dg.GemmError) as e:
            dg.plan(False, 4, 4, 4, variant=bad)
        assert e.value.status == binding.GEMM_ERR_INVALID_VARIANT
    for bad in (1, 2, 3, 4, 5, 6, 8):
        with pytest.raises(dg.GemmError) as e:
            dg.plan(True, 4, 4, 4, variant=bad)
        assert e.value.status == binding.GEMM_ERR_INVALID_VARIANT
    lib = binding.load()
    assert lib.gemm_f32_plan(-1, 1, 1, 1, None, None, None, None) == binding.GEMM_ERR_NULL_PTR


# --------------------------------------- validation before any device use --

def test_entry_points_validate_before_touching_a_device():
    raw = binding.raw_gemm
    for half in (False, True):
        assert raw(half, None, -1, 4, 4, 16, 16, 16, None) == binding.GEMM_ERR_INVALID_DIM
        assert raw(half, None, 4, 4, -4, 16, 16, 16, None) == binding.GEMM_ERR_INVALID_DIM
        assert raw(half, None, 4, 4, 4, None, 16, 16, None) == binding.GEMM_ERR_NULL_PTR
        assert raw(half, None, 4, 4, 4, 16, None, 16, None) == binding.GEMM_ERR_NULL_PTR
        assert raw(half, None, 4, 4, 4, 16, 16, None, None) == binding.GEMM_ERR_NULL_PTR
        assert raw(half, None, 4, 4, 0, None, None, 16, None) != binding.GEMM_ERR_NULL_PTR
        # nothing to do: OK without a launch (C has no extent, so may be NULL)
        assert raw(half, None, 0, 4, 4, None, 16, None, None) == binding.GEMM_OK
        assert raw(half, None, 4, 0, 4, 16, None, None, None) == binding.GEMM_OK
        assert raw(half, None, 0, 0, 0, None, None, None, None) == binding.GEMM_OK
        # the null check comes first: B has extent K * N even when M == 0
        assert raw(half, None, 0, 4, 4, None, None, None, None) == binding.GEMM_ERR_NULL_PTR
        assert raw(half, 99, 4, 4, 4, 16, 16, 16, None) == binding.GEMM_ERR_INVALID_VARIANT


def test_ex_entry_points_validate_layout_before_touching_a_device():
    ex = binding.raw_gemm_ex
    OK, DIM, NUL, LAY = (binding.GEMM_OK, binding.GEMM_ERR_INVALID_DIM, binding.GEMM_ERR_NULL_PTR,
                         binding.GEMM_ERR_INVALID_LAYOUT)
    for kind in ("f32", "f16", "bf16"):
        def call(op_a=0, op_b=0, M=4, N=5, K=6, A=16, lda=None, B=16, ldb=None, C=16, ldc=None,
                 alpha=1.0, beta=0.0):
            lda = max(M if op_a else K, 1) if lda is None else lda
            ldb = max(K if op_b else N, 1) if ldb is None else ldb
            ldc = max(N, 1) if ldc is None else ldc
            return ex(kind, op_a, op_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, None)
        assert call(M=-1) == DIM and call(K=-1) == DIM and call(N=-1, op_a=5) == DIM
        for bad in (2, -1, 7):
            assert call(op_a=bad) == LAY and call(op_b=bad) == LAY
        # leading dimensions below the row length of the stored matrix
        assert call(lda=5) == LAY and call(op_a=1, lda=3) == LAY
        assert call(ldb=4) == LAY and call(op_b=1, ldb=5) == LAY
        assert call(ldc=4) == LAY and call(ldc=0, N=0) == LAY
        assert call(op_a=1, lda=4) != LAY and call(op_b=1, ldb=6) != LAY
        assert call(lda=64, ldb=64, ldc=64) != LAY
        # layout is checked before pointers, pointers before the device
        assert call(lda=1, A=None) == LAY
        assert call(A=None) == NUL and call(B=None) == NUL and call(C=None) == NUL
        assert call(M=0, A=None, C=None) == OK and call(N=0, B=None, C=None) == OK
        assert call(M=0, N=0, K=0, A=None, B=None, C=None) == OK


def _conv_splits(K, crsp, npqp):
    """Split-K count of the convolution GEMM: k-chunks of at least 64 (multiples
    of 64) until tiles x splits reaches 256, when K >= 192 and CRSp >= 64."""
    if crsp < 64 or K < 192:
        return 1
    tiles = -(-K // 256) * -(-npqp // 256)
    want = max(1, min(-(-256 // tiles), crsp // 64))
    chunk = -(-(-(-crsp // want)) // 64) * 64
    return -(-crsp // chunk)


def test_conv2d_workspace_layout_and_validation():
    cp = binding.conv_params
    r = lambda v: -(-v // 256) * 256
    # 32 x 256 x 14 x 14, 256 filters 3 x 3, padding 1: CRS 2304, NPQ 6272 (multiples
    # of 8); 25 tiles, so the GEMM is split over k into chunks of 256 (9 partials)
    # (FP32: im2col; 16-bit: the channels-last implicit GEMM, whose workspace is
    # the reordered weights K x R S C and the copy of x N x 16 x 16 x C)
    p = cp(32, 256, 14, 14, 256, 3, 3, (1, 1), (1, 1))
    assert _conv_splits(256, 2304, 6272) == 9
    assert dg.conv2d_workspace(p, 4) == r(256 * 2304 * 4) + r(2304 * 6272 * 4) + 9 * r(256 * 6272 * 4)
    assert dg.conv2d_workspace(p, 2) == r(256 * 2304 * 2) + r(32 * 16 * 16 * 256 * 2)
    # 392 tiles: no split on the im2col path (FP32); 16-bit channels last
    p = cp(32, 64, 56, 56, 64, 3, 3, (1, 1), (1, 1))
    assert _conv_splits(64, 576, 100352) == 1
    assert dg.conv2d_workspace(p, 4) == r(64 * 576 * 4) + r(576 * 100352 * 4) + r(64 * 100352 * 4)
    assert dg.conv2d_workspace(p, 2) == r(64 * 576 * 2) + r(32 * 58 * 58 * 64 * 2)
    # CRS 27 rounds up to 32 (below one chunk: the planner's tiles, no split)
    p = cp(2, 3, 224, 224, 64, 3, 3, (2, 2), (1, 1))
    assert dg.conv2d_workspace(p, 2) == r(64 * 32 * 2) + r(32 * 25088 * 2) + r(64 * 25088 * 4)
    # a padded 1 x 1 layer on the gathering implicit GEMM's vector form: the
    # padded weights and the padded copy of x (16 x 8 x 64 x 64, plus 8
    # elements), no im2col matrix and no GEMM result
    p = cp(16, 8, 62, 62, 128, 1, 1, (1, 1), (1, 1))
    assert dg.conv2d_algorithm(p, 2) == dg.CONV_IMPLICIT
    assert dg.conv2d_workspace(p, 2) == r(128 * 8 * 2) + r((16 * 8 * 64 * 64 + 8) * 2)
    assert dg.conv2d_workspace(p, 4) == r(128 * 8 * 4) + r(8 * 65536 * 4) + r(128 * 65536 * 4)
    # the element gather (stride 2 along w): the padded weights only
    p = cp(16, 8, 130, 130, 24, 5, 5, (2, 2), (2, 2))
    assert dg.conv2d_algorithm(p, 2) == dg.CONV_IMPLICIT
    assert dg.conv2d_workspace(p, 2) == r(24 * 200 * 2)
    # a 7 x 7 stem with 256 filters: CRS 147 -> 152, 98 tiles -> 2 chunks of 128 and 24
    p = cp(2, 3, 224, 224, 256, 7, 7, (2, 2), (3, 3))
    assert _conv_splits(256, 152, 25088) == 2
    assert dg.conv2d_workspace(p, 2) == r(256 * 152 * 2) + r(152 * 25088 * 2) + 2 * r(256 * 25088 * 4)
    bad = [cp(-1, 1, 4, 4, 1, 1, 1), cp(1, 1, 4, 4, 1, 0, 1), cp(1, 1, 4, 4, 1, 1, 1, (0, 1)),
           cp(1, 1, 4, 4, 1, 1, 1, (1, 1), (-1, 0)), cp(1, 1, 4, 4, 1, 1, 1, dil=(1, 0)),
           cp(1, 1, 2, 2, 1, 5, 1), cp(1, 1, 4, 4, 1, 3, 3, dil=(2, 2))]
    for b in bad:
        with pytest.raises(dg.GemmError) as e:
            dg.conv2d_workspace(b, 4)
        assert e.value.status == binding.GEMM_ERR_INVALID_DIM
    with pytest.raises(dg.GemmError):
        dg.conv2d_workspace(cp(1, 1, 4, 4, 1, 1, 1), 3)
    lib = binding.load()
    assert lib.gemm_conv2d_workspace(None, 4, None) == binding.GEMM_ERR_NULL_PTR


def test_conv2d_algorithm_follows_the_tile_count():
    """16-bit layers with C a multiple of 32, filters of at most 64 taps and at
    least 96 channels-last tiles (64 filters x 256 pixels when K <= 64, else
    128 x 64) take the channels-last implicit GEMM; other 16-bit layers with
    at least 256 gathering tiles (128 filters x 256 output pixels) the
    gathering implicit GEMM; FP32 and smaller layers im2col."""
    cp = binding.conv_params
    alg = dg.conv2d_algorithm
    p56 = cp(32, 64, 56, 56, 64, 3, 3, (1, 1), (1, 1))          # 392 tiles of 64 x 256
    p14 = cp(32, 256, 14, 14, 256, 3, 3, (1, 1), (1, 1))        # 2 x 98 tiles of 128 x 64
    assert alg(p56, 2) == dg.CONV_IMPLICIT_NHWC and alg(p56, 4) == dg.CONV_IM2COL
    assert alg(p14, 2) == dg.CONV_IMPLICIT_NHWC and alg(p14, 4) == dg.CONV_IM2COL
    assert alg(cp(4, 128, 28, 28, 256, 3, 3, (2, 2), (1, 1)), 2) == dg.CONV_IM2COL   # 2 x 13 tiles
    assert alg(cp(384, 32, 8, 8, 64, 1, 1), 2) == dg.CONV_IMPLICIT_NHWC   # NPQ 24576: 96 tiles
    assert alg(cp(380, 32, 8, 8, 64, 1, 1), 2) == dg.CONV_IM2COL          # 95 tiles
    assert alg(cp(2, 32, 8, 8, 96, 3, 3, (1, 1), (1, 1)), 2) == dg.CONV_IM2COL   # 1 x 2 tiles
    assert alg(cp(64, 48, 32, 32, 64, 1, 1), 2) == dg.CONV_IMPLICIT     # C 48: gathering, 256 tiles
    assert alg(cp(4, 64, 16, 600, 64, 1, 1), 2) == dg.CONV_IMPLICIT_NHWC   # wide rows: 150 tiles
    assert alg(cp(4, 32, 40, 40, 64, 9, 9, (1, 1), (4, 4)), 2) == dg.CONV_IM2COL   # 81 taps


def test_conv2d_entry_points_validate_before_touching_a_device():
    cp = binding.conv_params
    p = cp(2, 3, 8, 8, 4, 3, 3, (1, 1), (1, 1))
    need = dg.conv2d_workspace(p, 4)
    for kind in ("f32", "f16", "bf16"):
        raw = lambda *a: binding.raw_conv2d(kind, *a)
        assert raw(cp(1, 1, 2, 2, 1, 5, 1), 256, 256, 256, 256, 1 << 20, None) == binding.GEMM_ERR_INVALID_DIM
        assert raw(p, None, 256, 256, 256, need, None) == binding.GEMM_ERR_NULL_PTR
        assert raw(p, 256, None, 256, 256, need, None) == binding.GEMM_ERR_NULL_PTR
        assert raw(p, 256, 256, None, 256, need, None) == binding.GEMM_ERR_NULL_PTR
        nb = dg.conv2d_workspace(p, 4 if kind == "f32" else 2)
        assert raw(p, 256, 256, 256, None, nb, None) == binding.GEMM_ERR_WORKSPACE
        assert raw(p, 256, 256, 256, 256, nb - 1, None) == binding.GEMM_ERR_WORKSPACE
        assert raw(p, 256, 256, 256, 256 + 16, nb, None) == binding.GEMM_ERR_WORKSPACE
        # nothing to compute: OK without touching anything
        assert raw(cp(0, 3, 8, 8, 4, 3, 3), None, 256, None, None, 0, None) == binding.GEMM_OK
        assert raw(cp(2, 3, 8, 8, 0, 3, 3), 256, None, None, None, 0, None) == binding.GEMM_OK
    lib = binding.load()
    assert lib.gemm_conv2d_f32(None, None, None, None, None, 0, None) == binding.GEMM_ERR_NULL_PTR


def test_no_device_is_reported_not_crashed():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; covered by the GPU tests")
    rc = binding.raw_gemm(False, None, 4, 4, 4, 16, 16, 16, None)
    assert rc in (binding.GEMM_ERR_RUNTIME, binding.GEMM_ERR_UNSUPPORTED_DEVICE)
    for kind in ("f32", "f16", "bf16"):
        rc = binding.raw_gemm_ex(kind, 1, 0, 4, 4, 4, 2.0, 16, 4, 16, 4, 0.5, 16, 4, None)
        assert rc in (binding.GEMM_ERR_RUNTIME, binding.GEMM_ERR_UNSUPPORTED_DEVICE)


def test_no_allocation_conv2d_host_checks():
    """The no-allocation FP16 convolution rejects bad sizes and layers whose
    workspace exceeds its fixed 16 MiB before any HIP call (so this runs
    without a GPU): the 14 x 14 and 56 x 56 benchmarked layers fit; a
    56 x 56 layer at twice the batch (xp 27.6 MB) does not."""
    cp = binding.conv_params
    lim = 16 << 20
    assert dg.conv2d_workspace(cp(32, 256, 14, 14, 256, 3, 3, (1, 1), (1, 1)), 2) <= lim
    assert dg.conv2d_workspace(cp(32, 64, 56, 56, 64, 3, 3, (1, 1), (1, 1)), 2) <= lim
    big = cp(64, 64, 56, 56, 64, 3, 3, (1, 1), (1, 1))
    assert dg.conv2d_workspace(big, 2) > lim
    f = binding.gemm_conv2d_f16_f32acc_noalloc
    assert f(big, 16, 16, 16, None) == binding.GEMM_ERR_SCRATCH_LIMIT
    assert f(cp(1, 4, 9, 9, 5, 3, 3, (0, 1)), 16, 16, 16, None) == binding.GEMM_ERR_INVALID_DIM
    assert f(cp(1, 4, 9, 9, 5, 3, 3), None, 16, 16, None) == binding.GEMM_ERR_NULL_PTR
    assert "16 MiB" in binding.status_string(binding.GEMM_ERR_SCRATCH_LIMIT)
