"""The C ABI library on the host: it loads, exports every declared entry point, and rejects
bad arguments with the documented codes before anything reaches the GPU."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8_gemv.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", src, flags=re.M)))


def _codes():
    src = open(HEADER).read()
    return {k: int(v) for k, v in re.findall(r"#define\s+(FP8GEMV_\w+)\s+\(?(-?\d+)\)?", src)}


@pytest.fixture(scope="module")
def fg():
    import fp8_gemv_amd
    return fp8_gemv_amd


def test_header_declares_the_entry_points():
    assert _declared() == sorted(["rms_norm_f32", "quantize_q8_1", "rmsnorm_q8_1",
                                  "silu_mul_f32", "silu_mul_q8_1",
                                  "gated_rms_norm_f32", "gated_rmsnorm_q8_1",
                                  "gemv_q8_0_q81", "gemv_e4m3_q81", "gemv_e4m3_blk128_q81",
                                  "gemv_q8_0_q81_mc", "gemv_e4m3_q81_mc",
                                  "gemv_e4m3_blk128_q81_mc", "requant_e4m3_q8_0", "requant_e4m3_blk128_q8_0",
                                  "fp8gemv_read_bytes", "fp8gemv_read_pattern",
                                  "fp8gemv_gemv_launch_info", "fp8gemv_strerror"])


def test_library_exports_every_declared_symbol(fg):
    out = subprocess.run(["nm", "-D", "--defined-only", fg.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in _declared():
        assert name in exported, name
        assert hasattr(fg.lib(), name)
    assert set(fg.EXPORTS) == set(_declared())


def test_library_is_built_for_gfx950_only(fg):
    blob = open(fg.LIB_PATH, "rb").read()
    targets = set(re.findall(rb"amdgcn-amd-amdhsa--(gfx[0-9a-z]+)", blob))
    assert targets == {b"gfx950"}, targets


def test_python_constants_match_header(fg):
    codes = _codes()
    for k, v in codes.items():
        assert getattr(fg, k) == v, k


def test_strerror(fg):
    assert fg.strerror(0) == "ok"
    for code in (-1, -2, -3, -4, -5, -6):
        assert fg.strerror(code) and fg.strerror(code) != "unknown error"
    assert fg.strerror(-99) == "unknown error"


# Argument checks run on the host and return before any HIP call, so they can be exercised
# here with fake (never dereferenced) addresses.
FAKE = 0x100000  # 16-byte aligned, never dereferenced


def test_producer_argument_errors(fg):
    L = fg.lib()
    assert L.rms_norm_f32(None, FAKE, FAKE, 64, 1, 1e-6, None) == fg.FP8GEMV_ERR_NULL
    assert L.rms_norm_f32(FAKE, FAKE, FAKE, 48, 1, 1e-6, None) == fg.FP8GEMV_ERR_SHAPE
    assert L.rms_norm_f32(FAKE, FAKE, FAKE, 0, 1, 1e-6, None) == fg.FP8GEMV_ERR_SHAPE
    assert L.rms_norm_f32(FAKE, FAKE, FAKE, 64, 0, 1e-6, None) == fg.FP8GEMV_ERR_SHAPE
    assert L.rms_norm_f32(FAKE, FAKE, FAKE, 65536 + 32, 1, 1e-6, None) == fg.FP8GEMV_ERR_TOO_LARGE
    assert L.rms_norm_f32(FAKE + 4, FAKE, FAKE, 64, 1, 1e-6, None) == fg.FP8GEMV_ERR_ALIGN
    assert L.quantize_q8_1(FAKE, None, FAKE, 1, 64, None) == fg.FP8GEMV_ERR_NULL
    assert L.quantize_q8_1(FAKE, FAKE, FAKE, 1, 40, None) == fg.FP8GEMV_ERR_SHAPE
    assert L.quantize_q8_1(FAKE, FAKE, FAKE, 70000, 64, None) == fg.FP8GEMV_ERR_TOO_LARGE
    assert L.quantize_q8_1(FAKE, FAKE + 8, FAKE, 1, 64, None) == fg.FP8GEMV_ERR_ALIGN
    assert L.rmsnorm_q8_1(FAKE, FAKE, None, None, FAKE, 64, 1, 1e-6, None) == fg.FP8GEMV_ERR_NULL
    assert L.rmsnorm_q8_1(FAKE, FAKE, None, FAKE, FAKE, 33, 1, 1e-6, None) == fg.FP8GEMV_ERR_SHAPE
    assert L.rmsnorm_q8_1(FAKE, FAKE, FAKE + 4, FAKE, FAKE, 64, 1, 1e-6, None) == fg.FP8GEMV_ERR_ALIGN


def test_silu_producer_argument_errors(fg):
    L, e = fg.lib(), fg
    assert L.silu_mul_f32(None, FAKE, FAKE, 64, 1, None) == e.FP8GEMV_ERR_NULL
    assert L.silu_mul_f32(FAKE, FAKE, FAKE, 40, 1, None) == e.FP8GEMV_ERR_SHAPE
    assert L.silu_mul_f32(FAKE, FAKE, FAKE, 64, 0, None) == e.FP8GEMV_ERR_SHAPE
    assert L.silu_mul_f32(FAKE, FAKE, FAKE, 65536 + 32, 1, None) == e.FP8GEMV_ERR_TOO_LARGE
    assert L.silu_mul_f32(FAKE, FAKE + 4, FAKE, 64, 1, None) == e.FP8GEMV_ERR_ALIGN
    assert L.silu_mul_q8_1(FAKE, FAKE, None, None, FAKE, 64, 1, None) == e.FP8GEMV_ERR_NULL
    assert L.silu_mul_q8_1(FAKE, FAKE, None, FAKE, FAKE, 33, 1, None) == e.FP8GEMV_ERR_SHAPE
    assert L.silu_mul_q8_1(FAKE, FAKE, FAKE + 4, FAKE, FAKE, 64, 1, None) == e.FP8GEMV_ERR_ALIGN
    assert L.silu_mul_q8_1(FAKE, FAKE, None, FAKE, FAKE + 2, 64, 1, None) == e.FP8GEMV_ERR_ALIGN


def test_gemv_argument_errors(fg):
    L = fg.lib()
    e = fg
    # NULL pointers
    assert L.gemv_e4m3_q81(None, 64, 1.0, FAKE, FAKE, FAKE, 1, 64, 8, None) == e.FP8GEMV_ERR_NULL
    assert L.gemv_q8_0_q81(FAKE, 68, FAKE, FAKE, None, 1, 64, 8, None) == e.FP8GEMV_ERR_NULL
    assert L.gemv_e4m3_blk128_q81(FAKE, 64, None, 1, FAKE, FAKE, FAKE, 1, 64, 8,
                                  None) == e.FP8GEMV_ERR_NULL
    # shapes
    assert L.gemv_e4m3_q81(FAKE, 64, 1.0, FAKE, FAKE, FAKE, 0, 64, 8, None) == e.FP8GEMV_ERR_SHAPE
    assert L.gemv_e4m3_q81(FAKE, 64, 1.0, FAKE, FAKE, FAKE, 1, 48, 8, None) == e.FP8GEMV_ERR_SHAPE
    assert L.gemv_e4m3_q81(FAKE, 64, 1.0, FAKE, FAKE, FAKE, 1, 64, 0, None) == e.FP8GEMV_ERR_SHAPE
    assert L.gemv_q8_0_q81(FAKE, 68, FAKE, FAKE, FAKE, 1, 16, 8, None) == e.FP8GEMV_ERR_SHAPE
    assert L.gemv_e4m3_q81(FAKE, 2 ** 17 + 32, 1.0, FAKE, FAKE, FAKE, 1, 2 ** 17, 8,
                           None) == e.FP8GEMV_ERR_TOO_LARGE
    assert L.gemv_e4m3_q81(FAKE, 64, 1.0, FAKE, FAKE, FAKE, 70000, 64, 8,
                           None) == e.FP8GEMV_ERR_TOO_LARGE
    # row_bytes below the container minimum
    assert L.gemv_e4m3_q81(FAKE, 48, 1.0, FAKE, FAKE, FAKE, 1, 64, 8, None) == e.FP8GEMV_ERR_ROW_BYTES
    assert L.gemv_q8_0_q81(FAKE, 66, FAKE, FAKE, FAKE, 1, 64, 8, None) == e.FP8GEMV_ERR_ROW_BYTES
    # grid columns
    assert L.gemv_e4m3_blk128_q81(FAKE, 256, FAKE, 1, FAKE, FAKE, FAKE, 1, 256, 8,
                                  None) == e.FP8GEMV_ERR_GRID
    # alignment
    assert L.gemv_e4m3_q81(FAKE + 8, 64, 1.0, FAKE, FAKE, FAKE, 1, 64, 8, None) == e.FP8GEMV_ERR_ALIGN
    assert L.gemv_e4m3_q81(FAKE, 72, 1.0, FAKE, FAKE, FAKE, 1, 64, 8, None) == e.FP8GEMV_ERR_ALIGN
    assert L.gemv_q8_0_q81(FAKE + 1, 68, FAKE, FAKE, FAKE, 1, 64, 8, None) == e.FP8GEMV_ERR_ALIGN
    assert L.gemv_q8_0_q81(FAKE, 69, FAKE, FAKE, FAKE, 1, 64, 8, None) == e.FP8GEMV_ERR_ALIGN
    assert L.gemv_q8_0_q81(FAKE, 68, FAKE + 4, FAKE, FAKE, 1, 64, 8, None) == e.FP8GEMV_ERR_ALIGN


def test_requant_argument_errors(fg):
    L, e = fg.lib(), fg
    assert L.requant_e4m3_q8_0(None, 64, 1.0, FAKE, 68, 64, 8, None) == e.FP8GEMV_ERR_NULL
    assert L.requant_e4m3_q8_0(FAKE, 64, 1.0, None, 68, 64, 8, None) == e.FP8GEMV_ERR_NULL
    assert L.requant_e4m3_blk128_q8_0(FAKE, 64, None, 1, FAKE, 68, 64, 8, None) == e.FP8GEMV_ERR_NULL
    assert L.requant_e4m3_q8_0(FAKE, 64, 1.0, FAKE, 68, 48, 8, None) == e.FP8GEMV_ERR_SHAPE
    assert L.requant_e4m3_q8_0(FAKE, 64, 1.0, FAKE, 68, 64, 0, None) == e.FP8GEMV_ERR_SHAPE
    assert L.requant_e4m3_q8_0(FAKE, 2 ** 17, 1.0, FAKE, 2 ** 17 // 32 * 34, 2 ** 17, 8,
                               None) == e.FP8GEMV_ERR_TOO_LARGE
    assert L.requant_e4m3_q8_0(FAKE, 48, 1.0, FAKE, 68, 64, 8, None) == e.FP8GEMV_ERR_ROW_BYTES
    assert L.requant_e4m3_q8_0(FAKE, 64, 1.0, FAKE, 66, 64, 8, None) == e.FP8GEMV_ERR_ROW_BYTES
    assert L.requant_e4m3_blk128_q8_0(FAKE, 256, FAKE, 1, FAKE, 272, 256, 8,
                                      None) == e.FP8GEMV_ERR_GRID
    assert L.requant_e4m3_q8_0(FAKE + 8, 64, 1.0, FAKE, 68, 64, 8, None) == e.FP8GEMV_ERR_ALIGN
    assert L.requant_e4m3_q8_0(FAKE, 72, 1.0, FAKE, 68, 64, 8, None) == e.FP8GEMV_ERR_ALIGN
    assert L.requant_e4m3_q8_0(FAKE, 64, 1.0, FAKE + 1, 68, 64, 8, None) == e.FP8GEMV_ERR_ALIGN
    assert L.requant_e4m3_q8_0(FAKE, 64, 1.0, FAKE, 69, 64, 8, None) == e.FP8GEMV_ERR_ALIGN
    assert L.requant_e4m3_blk128_q8_0(FAKE, 64, FAKE + 2, 1, FAKE, 68, 64, 8,
                                      None) == e.FP8GEMV_ERR_ALIGN


def test_gated_producer_argument_errors(fg):
    L = fg.lib()
    e = fg
    F = FAKE
    assert L.gated_rms_norm_f32(None, F, F, F, 8192, 128, 1, 1e-6, None) == e.FP8GEMV_ERR_NULL
    assert L.gated_rms_norm_f32(F, F, F, None, 8192, 128, 1, 1e-6, None) == e.FP8GEMV_ERR_NULL
    assert L.gated_rmsnorm_q8_1(F, F, None, None, F, F, 8192, 128, 1, 1e-6, None) == e.FP8GEMV_ERR_NULL
    assert L.gated_rmsnorm_q8_1(F, F, F, None, None, F, 8192, 128, 1, 1e-6, None) == e.FP8GEMV_ERR_NULL
    for ncols, hd, nrows in ((8192, 96, 1), (8192, 512, 1), (8160, 128, 1), (8192, 128, 0),
                             (8200, 32, 1), (0, 32, 1)):
        assert L.gated_rmsnorm_q8_1(F, F, F, None, F, F, ncols, hd, nrows, 1e-6,
                                    None) == e.FP8GEMV_ERR_SHAPE, (ncols, hd, nrows)
    assert L.gated_rmsnorm_q8_1(F, F, F, None, F, F, 65536 + 256, 256, 1, 1e-6,
                                None) == e.FP8GEMV_ERR_TOO_LARGE
    assert L.gated_rmsnorm_q8_1(F, F, F, None, F, F, 8192, 128, 65536, 1e-6,
                                None) == e.FP8GEMV_ERR_TOO_LARGE
    assert L.gated_rmsnorm_q8_1(F + 4, F, F, None, F, F, 8192, 128, 1, 1e-6, None) == e.FP8GEMV_ERR_ALIGN
    assert L.gated_rmsnorm_q8_1(F, F, F + 8, None, F, F, 8192, 128, 1, 1e-6, None) == e.FP8GEMV_ERR_ALIGN
    assert L.gated_rmsnorm_q8_1(F, F, F, F + 4, F, F, 8192, 128, 1, 1e-6, None) == e.FP8GEMV_ERR_ALIGN
    assert L.gated_rmsnorm_q8_1(F, F, F, None, F, F + 2, 8192, 128, 1, 1e-6, None) == e.FP8GEMV_ERR_ALIGN
    assert L.gated_rms_norm_f32(F, F, F, F + 8, 8192, 128, 1, 1e-6, None) == e.FP8GEMV_ERR_ALIGN


def test_read_bytes_argument_errors(fg):
    L = fg.lib()
    assert L.fp8gemv_read_bytes(None, 1024, FAKE, None) == fg.FP8GEMV_ERR_NULL
    assert L.fp8gemv_read_bytes(FAKE, 0, FAKE, None) == fg.FP8GEMV_ERR_SHAPE
    assert L.fp8gemv_read_bytes(FAKE + 4, 1024, FAKE, None) == fg.FP8GEMV_ERR_ALIGN
    assert L.fp8gemv_read_bytes(FAKE, (1 << 35) + 1, FAKE, None) == fg.FP8GEMV_ERR_TOO_LARGE


def test_launch_info_argument_errors_and_agreement(fg):
    import ctypes
    L = fg.lib()
    info = fg.LaunchInfo()
    ref = ctypes.byref(info)
    assert L.fp8gemv_gemv_launch_info(0, None, 5440, 1, 5120, 10, ref) == fg.FP8GEMV_ERR_NULL
    assert L.fp8gemv_gemv_launch_info(0, FAKE, 5440, 1, 5120, 10, None) == fg.FP8GEMV_ERR_NULL
    for bad in (-1, 6):
        assert L.fp8gemv_gemv_launch_info(bad, FAKE, 5440, 1, 5120, 10, ref) == fg.FP8GEMV_ERR_SHAPE
    assert L.fp8gemv_gemv_launch_info(0, FAKE, 5440, 0, 5120, 10, ref) == fg.FP8GEMV_ERR_SHAPE
    assert L.fp8gemv_gemv_launch_info(1, FAKE, 5120, 1, 5100, 10, ref) == fg.FP8GEMV_ERR_SHAPE
    assert L.fp8gemv_gemv_launch_info(0, FAKE, 5438, 1, 5120, 10, ref) == fg.FP8GEMV_ERR_ROW_BYTES
    assert L.fp8gemv_gemv_launch_info(1, FAKE + 8, 5120, 1, 5120, 10, ref) == fg.FP8GEMV_ERR_ALIGN
    # every row is covered once per activation-row pass; a misaligned Q8_0 plane takes the
    # generic kernel
    for c in ("q8_0", "e4m3", "blk128"):
        for m in (1, 2, 3, 5, 8, 11):
            for in_f in (5120, 17408, 32768):
                rb = in_f // 32 * 34 if c == "q8_0" else in_f
                i = fg.gemv_launch_info(c, rb, m, in_f, 17408)
                assert i["grid_x"] >= 1 and i["grid_y"] >= 1 and i["workgroup_size"] % 64 == 0
                assert i["kernel"].startswith("k_gemv_") and "Cfg<" in i["config"]
    g = fg.gemv_launch_info("q8_0", 5440, 1, 5120, 100, w_align=2)
    assert g["kernel"] == "k_gemv_q8_0_generic" and g["config"] == ""
    # the plain entry points never leave the vector kernels (rows bit-identical to m = 1); the
    # *_mc ones run the matrix-core kernels for every m where the row layout allows it
    for c in ("q8_0", "e4m3", "blk128"):
        rb = 5440 if c == "q8_0" else 5120
        for m in (1, 2, 3, 4, 8, 9):
            assert "mfma" not in fg.gemv_launch_info(c, rb, m, 5120, 17408)["kernel"]
            mc = fg.gemv_launch_info(c + "_mc", rb, m, 5120, 17408)
            assert mc["kernel"].startswith("k_gemv_" + ("q8_0" if c == "q8_0" else "e4m3") + "_mfma")
            assert mc["grid_y"] == (m + 7) // 8
    # layouts the matrix-core kernels do not take fall back to the plain kernels
    assert fg.gemv_launch_info("q8_0_mc", 5440, 4, 5120, 100, w_align=2)["kernel"] == \
        "k_gemv_q8_0_generic"
    assert "mfma" not in fg.gemv_launch_info("q8_0_mc", 96 // 32 * 34 + 14, 4, 96, 100)["kernel"]
    big = (1 << 26) + 16
    for c in ("q8_0_mc", "e4m3_mc", "blk128_mc"):
        assert "mfma" not in fg.gemv_launch_info(c, big, 4, 5120, 100)["kernel"]


def test_read_pattern_argument_errors(fg):
    L = fg.lib()
    P = fg.READ_PATTERNS
    assert len(P) == fg.FP8GEMV_READ_NUM_PATTERNS
    assert L.fp8gemv_read_pattern(None, 1024, 0, 0, FAKE, None) == fg.FP8GEMV_ERR_NULL
    assert L.fp8gemv_read_pattern(FAKE, 1024, 0, 0, None, None) == fg.FP8GEMV_ERR_NULL
    assert L.fp8gemv_read_pattern(FAKE, 0, 0, 0, FAKE, None) == fg.FP8GEMV_ERR_SHAPE
    assert L.fp8gemv_read_pattern(FAKE, 1024, -1, 0, FAKE, None) == fg.FP8GEMV_ERR_SHAPE
    assert L.fp8gemv_read_pattern(FAKE, 1024, len(P), 0, FAKE, None) == fg.FP8GEMV_ERR_SHAPE
    for rows in ("rows_1k", "rows_816", "rows_aligned", "line_windows"):
        for rb, nbytes in ((0, 4096), (1008, 4032), (1040, 4096), (1024 + 8, 2064),
                           ((1 << 20) + 16, (1 << 20) + 16)):
            assert L.fp8gemv_read_pattern(FAKE, nbytes, P[rows], rb, FAKE,
                                          None) == fg.FP8GEMV_ERR_SHAPE, (rows, rb, nbytes)
    assert L.fp8gemv_read_pattern(FAKE, (1 << 35) + 1, 0, 0, FAKE, None) == fg.FP8GEMV_ERR_TOO_LARGE
    assert L.fp8gemv_read_pattern(FAKE + 4, 1024, 0, 0, FAKE, None) == fg.FP8GEMV_ERR_ALIGN
    assert L.fp8gemv_read_pattern(FAKE, 1024, 0, 0, FAKE + 2, None) == fg.FP8GEMV_ERR_ALIGN


def test_binding_rejects_cpu_tensors_and_short_buffers(fg):
    import torch
    x = torch.zeros(64)
    with pytest.raises(ValueError):
        fg.rms_norm_f32(x, x, x, 64, 1)


def test_byte_counts_match_the_pages(fg):
    # gemv_e4m3_bench.rs, QUESTION: Q8_0 is 34 B per 32 weights = 1.0625 B/weight, e4m3 is
    # exactly 1 B/weight (a 5.88% smaller stream).
    for out_f, in_f in [(5120, 5120), (17408, 5120), (5120, 17408), (2048, 2048), (3, 96)]:
        q, e = fg.q8_0_weight_bytes(out_f, in_f), fg.e4m3_weight_bytes(out_f, in_f)
        assert q * 32 == e * 34 and q / e == 1.0625
        assert abs((1 - e / q) - 0.0588) < 5e-4
    # THE BLOCK-128 ARM: the grid is "~21 KB" and "0.02%" of the weight bytes for the widest
    # 27B projection; exactly 136 x 40 f32 = 21,760 B = 0.0244%.
    g = fg.blk128_grid_bytes(17408, 5120)
    assert g == 21760 and g == fg.blk128_grid_bytes(5120, 17408)
    assert round(100 * g / fg.e4m3_weight_bytes(17408, 5120), 2) == 0.02


def test_public_header_is_plain_c():
    # the C consumer of the ABI (a GPU test runs it) must compile as C11 against the header
    import shutil
    import subprocess
    import sys
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import c_abi_build
    if shutil.which("gcc") is None:
        pytest.skip("gcc not on PATH")
    r = subprocess.run(c_abi_build.compile_cmd("", syntax_only=True), capture_output=True,
                       text=True)
    assert r.returncode == 0, r.stderr


def test_build_script_loads_without_the_package():
    # build() must work on a fresh checkout, where the package (which refuses to import
    # without its library) cannot be imported yet: its build script is loaded by path.
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = ("import importlib.util, os, sys\n"
            f"spec = importlib.util.spec_from_file_location('b', os.path.join({root!r}, "
            "'fp8_gemv_amd', 'build.py'))\n"
            "m = importlib.util.module_from_spec(spec); spec.loader.exec_module(m)\n"
            "assert callable(m.build) and 'fp8_gemv_amd' not in sys.modules\n")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    src = open(os.path.join(root, "__graft_entry__.py")).read()
    assert "from fp8_gemv_amd import build" not in src
