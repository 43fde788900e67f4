"""Checks on the generated gfx950 code of the ring kernels (CPU only: the
kernel sources are compiled to assembly with the library's own flags).

These kernels issue their global->LDS loads from inline assembly that sets
M0 and is invisible to the compiler's wait counters.  That is sound only if
the compiler keeps nothing of its own in M0 in such a kernel and spills
nothing (a spill reload is a vector-memory load whose wait would also wait on
the in-flight tile loads), so both are checked here on the real output."""
import os
import re
import shutil
import subprocess

import pytest

from dense_gemm_optimisation_row_amd import build as hipbuild

RING_KERNELS = [("mfma_f16.hip", "mfma_f16_pipe_kernel"), ("mfma_f16.hip", "mfma_f16_pair_kernel"),
                ("mfma_f16.hip", "mfma_f16_pair128_kernel"),
                ("mfma_f32.hip", "mfma_f32_ring_kernel"), ("mfma_f32.hip", "mfma_f32_small_ring_kernel"),
                ("mfma_8bit.hip", "mfma_8bit_ring_kernel"), ("mfma_8bit.hip", "mfma_i8_pair_kernel"),
                ("mfma_8bit.hip", "mfma_i8_pair128_kernel"), ("mfma_8bit.hip", "mfma_fp8_pair128_kernel")]


_ASM = {}   # source file -> its generated assembly (each source compiled once)


@pytest.fixture(scope="module", params=RING_KERNELS, ids=lambda v: v[1])
def ring(request, tmp_path_factory):
    if shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc not available")
    src, kernel = request.param
    if src not in _ASM:
        out = tmp_path_factory.mktemp("isa") / (src + ".s")
        cmd = [hipbuild.hipcc(), *hipbuild.FLAGS, "-S", "--cuda-device-only",
               os.path.join(hipbuild.CSRC, src), "-o", str(out)]
        subprocess.run(cmd, check=True, capture_output=True, text=True)
        _ASM[src] = out.read_text()
    return _ASM[src], kernel


def _instances(text, name):
    """(symbol, body) of every instantiation of the kernel template ``name``
    (operand layouts, accumulate-into-C, input formats)."""
    found = []
    for m in re.finditer(rf"^(_Z\S*{name}\S*):.*$", text, flags=re.M):
        # the whole function: blocks the compiler lays out past the first
        # s_endpgm belong to it too
        end = text.index(".Lfunc_end", m.end())
        found.append((m.group(1), text[m.end():end]))
    assert found, f"{name} not found in the generated code"
    return found


def test_every_layout_variant_is_generated(ring):
    asm, kernel = ring
    # 16-bit: op(B) x (overwrite, accumulate) x two formats for each of a
    # k-contiguous A (pair kernel) and a k-strided A (pipe kernel); FP32:
    # op(A) x op(B) x (overwrite, accumulate); 8-bit: the row-major product in
    # the two FP8 formats and once for INT8, at each of the two tiles; the
    # 64 x 64 ring with one and with two groups over k; the 16-bit and 8-bit
    # 128 x 128 rings in each format with one and with two groups over k
    want = {"mfma_f16_pipe_kernel": 8, "mfma_f16_pair_kernel": 8, "mfma_f16_pair128_kernel": 4,
            "mfma_f32_ring_kernel": 8,
            "mfma_f32_small_ring_kernel": 2, "mfma_8bit_ring_kernel": 2, "mfma_i8_pair_kernel": 1,
            "mfma_i8_pair128_kernel": 2, "mfma_fp8_pair128_kernel": 4}[kernel]
    assert len(_instances(asm, kernel)) == want


def test_m0_is_touched_only_by_the_load_helper(ring):
    asm, kernel = ring
    for sym, body in _instances(asm, kernel):
        inside = False
        outside_uses = []
        loads = 0
        for line in body.splitlines():
            if "ASMSTART" in line:
                inside = True
                continue
            if "ASMEND" in line:
                inside = False
                continue
            code = line.split(";")[0]
            if re.search(r"\bm0\b", code) and not inside:
                outside_uses.append(code.strip())
            if inside and re.search(r"buffer_load_dword(x4)?\s", code) and " lds" in code:
                loads += 1
        assert loads > 0, f"{sym}: no global->LDS load found inside inline assembly"
        assert outside_uses == [], f"{sym}: compiler-generated M0 accesses: {outside_uses[:5]}"


def test_ring_kernel_spills_nothing(ring):
    asm, kernel = ring
    # accumulators per lane: 256 x 256 tiles over four wavefronts hold all
    # 256 AGPRs, over eight (the FP32 ring) 128, 128 x 128 over four 64; the
    # 64 x 64 tile holds few (not checked)
    want_agpr = {"mfma_f32_small_ring_kernel": None, "mfma_f32_ring_kernel": 128,
                 "mfma_f16_pair128_kernel": 64, "mfma_i8_pair128_kernel": 64,
                 "mfma_fp8_pair128_kernel": 64}.get(kernel, 256)
    for sym, body in _instances(asm, kernel):
        priv = re.search(rf"^\s*\.set\s+{re.escape(sym)}\.private_seg_size,\s*(\d+)", asm, flags=re.M)
        agpr = re.search(rf"^\s*\.set\s+{re.escape(sym)}\.num_agpr,\s*(\d+)", asm, flags=re.M)
        assert priv and int(priv.group(1)) == 0, f"{sym}: scratch (spill) memory in use"
        if want_agpr is not None:
            assert agpr and int(agpr.group(1)) == want_agpr, f"{sym}: accumulators not held in {want_agpr} AGPRs"
        assert "scratch_" not in body, sym


@pytest.fixture(scope="module")
def conv_asm(tmp_path_factory):
    if shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("isa") / "conv.s"
    cmd = [hipbuild.hipcc(), *hipbuild.FLAGS, "-S", "--cuda-device-only",
           os.path.join(hipbuild.CSRC, "conv.hip"), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return out.read_text()


@pytest.mark.parametrize("kernel", ["conv_igemm_vec", "conv_igemm"])
def test_implicit_gemm_kernels_keep_accumulators_and_gather_as_designed(conv_asm, kernel):
    """Both formats x both tile heights; no spills; the accumulators of BM
    filters x 256 pixels over four wavefronts (BM values per lane) in AGPRs;
    the vector form gathers with 12-byte loads only, the element form with
    2-byte loads only."""
    found = [(sym, body) for sym, body in _instances(conv_asm, kernel)
             if kernel == "conv_igemm_vec" or "conv_igemm_vec" not in sym]
    assert len(found) == 4
    for sym, body in found:
        bm = 64 if "Li64E" in sym else 128
        priv = re.search(rf"^\s*\.set\s+{re.escape(sym)}\.private_seg_size,\s*(\d+)", conv_asm, flags=re.M)
        agpr = re.search(rf"^\s*\.set\s+{re.escape(sym)}\.num_agpr,\s*(\d+)", conv_asm, flags=re.M)
        assert priv and int(priv.group(1)) == 0, f"{sym}: scratch (spill) memory in use"
        assert agpr and int(agpr.group(1)) == bm, f"{sym}: accumulators not held in {bm} AGPRs"
        assert "scratch_" not in body, sym
        wide, narrow = body.count("buffer_load_dwordx3"), body.count("buffer_load_ushort")
        if kernel == "conv_igemm_vec":
            assert wide > 0 and narrow == 0, (sym, wide, narrow)
        else:
            assert wide == 0 and narrow > 0, (sym, wide, narrow)


@pytest.fixture(scope="module")
def f32_asm(tmp_path_factory):
    if shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("isa") / "mfma_f32.s"
    cmd = [hipbuild.hipcc(), *hipbuild.FLAGS, "-S", "--cuda-device-only",
           os.path.join(hipbuild.CSRC, "mfma_f32.hip"), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return out.read_text()


def _loads_and_m0(body):
    """(direct-load helper loads, compiler-generated loads, M0 accesses
    outside the helpers) of a kernel body, in order."""
    helper, compiler, m0, inside = [], [], [], False
    for i, ln in enumerate(body.splitlines()):
        if "ASMSTART" in ln:
            inside = True
            continue
        if "ASMEND" in ln:
            inside = False
            continue
        code = ln.split(";")[0]
        if inside and re.search(r"buffer_load_dword(x4)?\b.* lds", code):
            helper.append(i)
        elif not inside and re.search(r"\b(buffer|global|flat)_load", code):
            compiler.append(i)
        elif re.search(r"\bm0\b", code) and not inside:
            m0.append(code.strip())
    return helper, compiler, m0


def _no_scratch(asm, sym):
    priv = re.search(rf"^\s*\.set\s+{re.escape(sym)}\.private_seg_size,\s*(\d+)", asm, flags=re.M)
    assert priv and int(priv.group(1)) == 0, f"{sym}: scratch (spill) memory in use"


def test_skinny_ring_kernel_streams_through_direct_loads_only(f32_asm):
    """The tall, narrow FP32 kernel for three and four column blocks streams
    each wavefront's slices through its own ring of LDS slots: every global
    read comes from the inline-assembly direct-load helpers (which set M0, so
    the compiler must touch M0 nowhere else), so the only waits on memory
    are the hand-placed ones; its prologue issues three slices (two with four
    blocks) before the first MFMA; nothing spills.  Three instantiations:
    3 and 4 blocks, and 3 with the last column on the vector ALUs."""
    found = _instances(f32_asm, "mfma_f32_skinny_kernel")
    assert len(found) == 3
    for sym, body in found:
        nb = int(re.search(r"kernelILi(\d)E", sym).group(1))
        fringe = "ELb1EE" in sym
        helper, compiler, m0 = _loads_and_m0(body)
        assert compiler == [], f"{sym}: loads outside the direct-load helpers"
        assert m0 == [], f"{sym}: compiler-generated M0 accesses: {m0[:5]}"
        first_mfma = next(i for i, ln in enumerate(body.splitlines()) if "v_mfma" in ln)
        depth = 2 if nb == 4 else 3
        assert sum(i < first_mfma for i in helper) >= depth * (1 + nb + (1 if fringe else 0)), sym
        _no_scratch(f32_asm, sym)


def test_skinny_resident_kernel_issues_every_load_before_its_first_mfma(f32_asm):
    """The tall, narrow FP32 kernel for one and two column blocks issues all
    of a lane's loads before its first MFMA, with no wait among them: first
    the direct global->LDS copies of B (helpers that set M0; the compiler
    touches M0 nowhere else), then its own loads of the tail row and of A,
    at most 63 (what the wait counter tells apart), so that its waits on A
    count only loads issued after; nothing spills.  Four instantiations: 1
    and 2 blocks, each with and without the last column on the vector ALUs."""
    found = _instances(f32_asm, "mfma_f32_skinny_resident_kernel")
    assert len(found) == 4
    for sym, body in found:
        helper, compiler, m0 = _loads_and_m0(body)
        lines = body.splitlines()
        first_mfma = next(i for i, ln in enumerate(lines) if "v_mfma" in ln)
        assert helper and compiler and m0 == [], sym
        assert max(helper) < min(compiler), f"{sym}: a compiler load before a B copy"
        assert max(compiler) < first_mfma, f"{sym}: a load after the first MFMA"
        assert len(compiler) <= 63
        assert not any("vmcnt" in ln for ln in lines[min(helper):max(compiler)]), f"{sym}: a wait among the loads"
        _no_scratch(f32_asm, sym)


def test_poison_build_fills_every_direct_load_destination_first(tmp_path):
    """The LDS-poisoning debug build (-DDGOR_LDS_POISON) writes the poison
    before each global->LDS load, and waits for it: in the 16-bit pair ring,
    every direct load is preceded by LDS writes and an lgkmcnt(0) wait since
    the previous direct load."""
    if shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc not available")
    out = tmp_path / "mfma_f16_poison.s"
    cmd = [hipbuild.hipcc(), *hipbuild.FLAGS, "-DDGOR_LDS_POISON", "-S", "--cuda-device-only",
           os.path.join(hipbuild.CSRC, "mfma_f16.hip"), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    text = out.read_text()
    found = _instances(text, "mfma_f16_pair_kernel")
    assert len(found) == 8
    for sym, body in found:
        writes = waited = False
        loads = 0
        for line in body.splitlines():
            code = line.split(";")[0]
            if "ds_write" in code:
                writes, waited = True, False
            elif "s_waitcnt" in code and "lgkmcnt(0)" in code and writes:
                waited = True
            elif "buffer_load_dwordx4" in code and " lds" in code:
                assert writes and waited, f"{sym}: a direct load without its poison before it"
                writes = waited = False
                loads += 1
        assert loads > 0, sym


def test_channels_last_conv_kernel_streams_cleanly(tmp_path):
    """The channels-last convolution kernel (built with its file's flags): no
    spills, no accumulator moves between register files inside the k-loop,
    and, as it loads through the inline-assembly global->LDS helper, no M0
    access of the compiler's own.  Six instantiations: two formats x three
    tile configurations."""
    if shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc not available")
    out = tmp_path / "conv_nhwc.s"
    cmd = [hipbuild.hipcc(), *hipbuild.FLAGS, *hipbuild.FILE_FLAGS["conv_nhwc.hip"], "-S", "--cuda-device-only",
           os.path.join(hipbuild.CSRC, "conv_nhwc.hip"), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    text = out.read_text()
    found = _instances(text, "conv_nhwc_kernel")
    assert len(found) == 6
    for sym, body in found:
        priv = re.search(rf"^\s*\.set\s+{re.escape(sym)}\.private_seg_size,\s*(\d+)", text, flags=re.M)
        assert priv and int(priv.group(1)) == 0, f"{sym}: scratch (spill) memory in use"
        assert "v_accvgpr_mov" not in body and "scratch_" not in body, sym
        inside, outside_m0, dma = False, [], 0
        for line in body.splitlines():
            if "ASMSTART" in line:
                inside = True
                continue
            if "ASMEND" in line:
                inside = False
                continue
            code = line.split(";")[0]
            if inside and "buffer_load_dwordx4" in code and " lds" in code:
                dma += 1
            elif re.search(r"\bm0\b", code) and not inside:
                outside_m0.append(code.strip())
        assert dma > 0 and outside_m0 == [], (sym, outside_m0[:3])


def test_calibration_loop_is_bare_mfmas(tmp_path):
    """The matrix-core rate calibration kernel (calibrate.hip, its own
    library) measures the ceiling of the 256 x 256 tile's MFMA stream only if
    its k-loop is that stream and nothing else: the loop body holds the two
    stages' 128 v_mfma_f32_16x16x32_f16 of a trip, no accumulator moves, no
    memory instruction, and the kernel spills nothing."""
    if shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc not available")
    out = tmp_path / "calibrate.s"
    cmd = [hipbuild.hipcc(), *hipbuild.FLAGS, "-S", "--cuda-device-only",
           os.path.join(hipbuild.CSRC, "calibrate.hip"), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    text = out.read_text()
    [(sym, body)] = _instances(text, "mfma_f16_rate_kernel")
    priv = re.search(rf"^\s*\.set\s+{re.escape(sym)}\.private_seg_size,\s*(\d+)", text, flags=re.M)
    assert priv and int(priv.group(1)) == 0, "scratch (spill) memory in use"
    # the loop: from the block a backward branch returns to, up to that branch
    loops = []
    for m in re.finditer(r"^\s*s_cbranch_\w+\s+(\.LBB\w+)", body, flags=re.M):
        label = re.search(rf"^{re.escape(m.group(1))}:", body, flags=re.M)
        if label and label.start() < m.start():
            loops.append(body[label.end():m.start()])
    assert len(loops) == 1, f"{len(loops)} loops"
    code = [ln.split(";")[0].strip() for ln in loops[0].splitlines()]
    code = [c for c in code if c and not c.startswith(".")]
    mfma = [c for c in code if c.startswith("v_mfma_f32_16x16x32_f16")]
    assert len(mfma) == 128, len(mfma)
    assert not [c for c in code if c.startswith(("v_accvgpr", "buffer_", "global_", "ds_", "scratch_", "v_mov"))], \
        [c for c in code if not c.startswith("v_mfma")]
