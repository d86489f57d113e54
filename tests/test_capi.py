"""The C-ABI library loads, exports every declared symbol, and rejects invalid
calls with the documented status codes before touching the device.

Runs without a GPU: every call here fails host-side validation (or is a
documented no-op), so no HIP API is reached.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "int8_quantized_gemm_amd", "libq8gemm.so")
HEADER = os.path.join(ROOT, "include", "q8gemm.h")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libq8gemm.so not built")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s+\**([a-z_0-9]+)\s*\(", src, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def q8():
    import int8_quantized_gemm_amd as m
    return m


def test_header_declares_the_five_entry_points():
    names = declared_functions()
    for n in ("quant_8bit", "blockwise_scaled_mm", "scaled_mm_int8", "scaled_mm_fp8", "moe_mm_data",
              "grouped_blockwise_scaled_mm", "shuffle_rows", "q8gemm_last_error"):
        assert n in names


def test_every_declared_symbol_is_exported(q8):
    lib = ctypes.CDLL(LIB)
    names = declared_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(q8.EXPORTS) == names


def test_binding_fails_loudly_without_library(tmp_path):
    import subprocess
    import sys
    code = ("import sys, os; sys.path.insert(0, %r); import builtins;"
            "real = os.path.exists;"
            "os.path.exists = lambda p: False if p.endswith('libq8gemm.so') else real(p);"
            "import int8_quantized_gemm_amd") % ROOT
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True)
    assert r.returncode != 0 and "libq8gemm.so" in r.stderr and "ImportError" in r.stderr


def test_quant_validation(q8):
    L = q8._lib
    f, p = ctypes.c_float, None
    # bad input dtype
    assert q8._quant(p, 7, 4, 128, 128, p, q8.Q8_E4M3FN, p, 128, 0, 1e-10, -448, 448, 0, 0, p, 0, p, 0, p) == q8.Q8_EINVAL
    assert "x_dtype" in q8.last_error()
    # group does not divide K
    assert q8._quant(p, q8.Q8_BF16, 4, 100, 100, p, q8.Q8_E4M3FN, p, 32, 0, 1e-10, -448, 448, 0, 0, p, 0, p, 0, p) == q8.Q8_ESHAPE
    # FP8 clip range beyond 448
    assert q8._quant(p, q8.Q8_BF16, 4, 128, 128, p, q8.Q8_E4M3FN, p, 128, 0, 1e-10, -480, 480, 0, 0, p, 0, p, 0, p) == q8.Q8_EINVAL
    # fused SiLU-and-mul: the input row is [gate | up], so ld_x must cover 2K
    assert q8._quant(p, q8.Q8_BF16, 4, 128, 128, p, q8.Q8_E4M3FN, p, 128, 0, 1e-10, -448, 448, 0, 1, p, 0, p, 0, p) == q8.Q8_ESHAPE
    assert "row width" in q8.last_error()
    assert q8._quant(p, q8.Q8_BF16, 4, 128, 256, p, q8.Q8_E4M3FN, p, 128, 0, 1e-10, -448, 448, 0, 2, p, 0, p, 0, p) == q8.Q8_EINVAL
    # fused / masked need per-group scales
    assert q8._quant(8, q8.Q8_BF16, 4, 128, 256, 8, q8.Q8_E4M3FN, 8, 128, 1, 1e-10, -448, 448, 0, 1, p, 0, 8, 4096, p) == q8.Q8_EUNSUPPORTED
    assert q8._quant(8, q8.Q8_BF16, 4, 128, 128, 8, q8.Q8_E4M3FN, 8, 128, 1, 1e-10, -448, 448, 0, 0, 8, 2, 8, 4096, p) == q8.Q8_EUNSUPPORTED
    # masked rows: max_m must be >= 1 and divide M
    assert q8._quant(8, q8.Q8_BF16, 4, 128, 128, 8, q8.Q8_E4M3FN, 8, 128, 0, 1e-10, -448, 448, 0, 0, 8, 0, p, 0, p) == q8.Q8_ESHAPE
    assert q8._quant(8, q8.Q8_BF16, 6, 128, 128, 8, q8.Q8_E4M3FN, 8, 128, 0, 1e-10, -448, 448, 0, 0, 8, 4, p, 0, p) == q8.Q8_ESHAPE
    assert "max_m" in q8.last_error()
    # a valid fused + masked request with null data pointers stops at the null check
    assert q8._quant(p, q8.Q8_BF16, 6, 128, 256, p, q8.Q8_E4M3FN, p, 128, 0, 1e-10, -448, 448, 0, 1, 8, 3, p, 0, p) == q8.Q8_EINVAL
    assert "null" in q8.last_error()
    # ld_x < K
    assert q8._quant(p, q8.Q8_BF16, 4, 128, 64, p, q8.Q8_E4M3FN, p, 128, 0, 1e-10, -448, 448, 0, 0, p, 0, p, 0, p) == q8.Q8_ESHAPE
    # null pointers with real work
    assert q8._quant(p, q8.Q8_BF16, 4, 128, 128, p, q8.Q8_E4M3FN, p, 128, 0, 1e-10, -448, 448, 0, 0, p, 0, p, 0, p) == q8.Q8_EINVAL
    # per-tensor dynamic needs workspace
    need = q8._quant_ws(4, 128, q8.SCALE_PER_TENSOR_DYNAMIC)
    assert need > 0 and q8._quant_ws(4, 128, q8.SCALE_PER_GROUP) == 0
    assert q8._quant(8, q8.Q8_BF16, 4, 128, 128, 8, q8.Q8_E4M3FN, 8, 128, 1, 1e-10, -448, 448, 0, 0, p, 0, p, 0, p) == q8.Q8_EWORKSPACE
    # UE8M0 with a static scale is rejected
    assert q8._quant(8, q8.Q8_BF16, 4, 128, 128, 8, q8.Q8_E4M3FN, 8, 128, 2, 1e-10, -448, 448, 1, 0, p, 0, p, 0, p) == q8.Q8_EINVAL
    # empty input is a no-op (no pointer needed)
    assert q8._quant(p, q8.Q8_BF16, 0, 128, 128, p, q8.Q8_E4M3FN, p, 128, 0, 1e-10, -448, 448, 0, 0, p, 0, p, 0, p) == q8.Q8_OK
    assert q8.last_error() == ""


def test_blockwise_validation(q8):
    p = None
    args = lambda M, N, K, bn, bk, out=q8.Q8_BF16: (p, p, p, p, p, p, out, M, N, K, bn, bk, p, 0, p)
    assert q8._bmm(*args(4, 256, 500, 128, 128)) == q8.Q8_ESHAPE          # ragged K
    assert "multiple of bk" in q8.last_error()
    assert q8._bmm(*args(4, 256, 512, 128, 64)) == q8.Q8_EUNSUPPORTED     # bk not in {32, 128}
    assert q8._bmm(*args(4, 256, 512, 24, 128)) == q8.Q8_EUNSUPPORTED     # bn not a multiple of 16
    assert q8._bmm(*args(4, 256, 512, 128, 128, q8.Q8_F32)) == q8.Q8_EINVAL
    assert q8._bmm(*args(4, 256, 512, 128, 128)) == q8.Q8_EINVAL          # null pointers
    assert q8._bmm(*args(0, 256, 512, 128, 128)) == q8.Q8_OK              # M = 0
    assert q8._bmm(*args(-1, 256, 512, 128, 128)) == q8.Q8_ESHAPE
    # 17..64 rows split K into ranges whose float32 partials need a workspace:
    # 4 ranges of 1792 bytes for K = 7168 (256 workgroups of 64 weight rows)
    assert q8._bmm_ws(33, 4096, 7168, 32, 32) == 4 * 33 * 4096 * 4
    assert q8._bmm_ws(64, 4096, 7168, 128, 128) == 4 * 64 * 4096 * 4
    assert q8._bmm_ws(17, 1000, 1024, 128, 128) == 4 * 17 * 1000 * 4
    for M, N in ((16, 4096), (33, 1002)):  # other kernels, or N % 4
        assert q8._bmm_ws(M, N, 7168, 128, 128) == 0
    # more than 64 rows: the optional split of a last round of tiles, sized for
    # the current device's compute units (none without a device)
    assert q8._bmm_ws(65, 4096, 7168, 128, 128) % 256 == 0
    assert q8._bmm_ws(65, 4096, 896, 128, 128) == 0     # fewer than 8 K slabs: never split
    wargs = lambda ws, wsb: (8, 8, 8, 8, p, 8, q8.Q8_BF16, 33, 4096, 7168, 32, 32, ws, wsb, p)
    assert q8._bmm(*wargs(p, 0)) == q8.Q8_EWORKSPACE
    assert "workspace" in q8.last_error()
    assert q8._bmm(*wargs(16, 4 * 33 * 4096 * 4 - 1)) == q8.Q8_EWORKSPACE
    assert q8._bmm(*wargs(20, 4 * 33 * 4096 * 4)) == q8.Q8_EINVAL     # misaligned
    assert "aligned" in q8.last_error()


def test_split_wait_setting(q8):
    assert q8._split_wait(-1) == q8.Q8_EINVAL
    assert "outside" in q8.last_error()
    assert q8._split_wait(100001) == q8.Q8_EINVAL
    assert q8._split_wait(0) == q8.Q8_OK
    assert q8._split_wait(200) == q8.Q8_OK


def test_int8_validation(q8):
    p = None
    assert q8._imm(p, p, 1, p, p, 1, p, p, q8.Q8_BF16, 4, 100, 128, p) == q8.Q8_ESHAPE   # N % 16
    assert q8._imm(p, p, 1, p, p, 1, p, p, q8.Q8_BF16, 4, 128, 120, p) == q8.Q8_ESHAPE   # K % 16
    assert q8._imm(p, 8, 3, p, 8, 1, p, p, q8.Q8_BF16, 4, 128, 128, p) == q8.Q8_EUNSUPPORTED
    assert "scales_a" in q8.last_error()
    assert q8._imm(p, 8, 4, p, 8, 7, p, p, q8.Q8_BF16, 4, 128, 128, p) == q8.Q8_EUNSUPPORTED
    assert q8._imm(p, 8, 1, p, p, 1, p, p, q8.Q8_I32, 4, 128, 128, p) == q8.Q8_EINVAL    # scales with I32
    assert q8._imm(p, 8, 1, p, 8, 1, p, p, q8.Q8_F32, 4, 128, 128, p) == q8.Q8_EINVAL
    assert q8._imm(p, 8, 1, p, 8, 1, p, p, q8.Q8_BF16, 0, 128, 128, p) == q8.Q8_OK


def test_fp8_scaled_validation(q8):
    p = None
    assert q8._fmm(p, p, 1, p, p, 1, p, p, q8.Q8_BF16, 4, 100, 128, p) == q8.Q8_ESHAPE   # N % 16
    assert q8._fmm(p, p, 1, p, p, 1, p, p, q8.Q8_BF16, 4, 128, 120, p) == q8.Q8_ESHAPE   # K % 16
    assert q8._fmm(p, 8, 3, p, 8, 1, p, p, q8.Q8_BF16, 4, 128, 128, p) == q8.Q8_EUNSUPPORTED
    assert "scales_a" in q8.last_error()
    assert q8._fmm(p, 8, 4, p, 8, 7, p, p, q8.Q8_BF16, 4, 128, 128, p) == q8.Q8_EUNSUPPORTED
    assert q8._fmm(p, p, 1, p, 8, 1, p, p, q8.Q8_BF16, 4, 128, 128, p) == q8.Q8_EINVAL    # null scale
    assert q8._fmm(p, 8, 1, p, 8, 1, p, p, q8.Q8_I32, 4, 128, 128, p) == q8.Q8_EINVAL    # no raw output
    assert q8._fmm(p, 8, 1, p, 8, 1, p, p, q8.Q8_BF16, 4, 128, 128, p) == q8.Q8_EINVAL   # null operands
    assert q8._fmm(p, 8, 1, p, 8, 1, p, p, q8.Q8_BF16, 0, 128, 128, p) == q8.Q8_OK
    assert q8._fmm(p, 8, 1, p, 8, 1, p, p, q8.Q8_F16, 1 << 20, 128, 4096, p) == q8.Q8_EUNSUPPORTED  # 4 GiB


def test_moe_and_grouped_validation(q8):
    p = None
    assert q8._moe(p, 16, 8, 0, 64, 64, p, p, p, p, p, p, 0, p) == q8.Q8_EUNSUPPORTED   # E = 0
    assert q8._moe(p, 16, 8, 2000, 64, 64, p, p, p, p, p, p, 0, p) == q8.Q8_EUNSUPPORTED
    assert q8._moe(p, 16, 0, 8, 64, 64, p, p, p, p, p, p, 0, p) == q8.Q8_ESHAPE
    assert q8._moe(8, 16, 8, 8, 64, 64, 8, 8, 8, 8, 8, p, 0, p) == q8.Q8_EWORKSPACE
    assert q8._moe_ws(4096, 8, 64) == (4096 * 8 // 256) * 64 * 4
    g = lambda tm, K, cmap=p, ws=p, wsb=0: (8, 8, 8, 8, 8, q8.Q8_BF16, 8, 8, p, cmap, 4, tm, 256, K, 128, 128, ws, wsb, p)
    assert q8._gmm(*g(64, 500)) == q8.Q8_ESHAPE
    assert q8._gmm(*g(64, 512, cmap=8)) == q8.Q8_EWORKSPACE
    assert q8._gmm(*g(0, 512)) == q8.Q8_OK
    assert q8._fin(p, q8.Q8_F32, p, p, 4, 2, 16, p, p) == q8.Q8_EINVAL        # dtype
    assert q8._fin(p, q8.Q8_BF16, p, p, 4, 0, 16, p, p) == q8.Q8_ESHAPE       # topk
    assert q8._fin(p, q8.Q8_BF16, p, p, 4, 2, 16, p, p) == q8.Q8_EINVAL       # null D / out
    assert q8._fin(p, q8.Q8_BF16, p, p, 0, 2, 16, p, p) == q8.Q8_OK           # T = 0
    assert q8._fin(p, q8.Q8_BF16, p, p, 1 << 30, 4, 16, p, p) == q8.Q8_ESHAPE # T * topk
    assert q8._shuf(p, 16, p, 4, p, p) == q8.Q8_EINVAL
    assert q8._shuf(p, 16, p, 0, p, p) == q8.Q8_OK


def test_e8m0_gemm_validation(q8):
    p = None
    args = lambda M, N, K, bn, out=q8.Q8_BF16, ptr=p: (ptr, ptr, ptr, ptr, p, ptr, out, M, N, K, bn, p, 0, p)
    assert q8._bmm8(*args(4, 256, 500, 32)) == q8.Q8_ESHAPE            # K not a multiple of 128
    assert "multiple of 128" in q8.last_error()
    assert q8._bmm8(*args(4, 256, 512, 24)) == q8.Q8_EUNSUPPORTED      # bn not a multiple of 16
    assert q8._bmm8(*args(4, 256, 512, 32, q8.Q8_F32)) == q8.Q8_EINVAL  # output dtype
    assert q8._bmm8(*args(4, 0, 512, 32)) == q8.Q8_ESHAPE              # N = 0
    assert q8._bmm8(*args(4, 256, 512, 32)) == q8.Q8_EINVAL            # null pointers
    assert q8._bmm8(*args(0, 256, 512, 32)) == q8.Q8_OK                # M = 0: no-op
    # scale tables must be 4-byte aligned (the kernels read scale dwords)
    assert q8._bmm8(16, 18, 16, 16, p, 16, q8.Q8_BF16, 4, 256, 512, 32, p, 0, p) == q8.Q8_EINVAL
    assert "aligned" in q8.last_error()
    # A beyond 4 GiB
    assert q8._bmm8(*args(1 << 20, 256, 1 << 12, 32)) == q8.Q8_EUNSUPPORTED
    # 17..64 rows split K: float32 partials of 4 ranges in the workspace
    assert q8._bmm8_ws(64, 4096, 7168, 32) == 4 * 64 * 4096 * 4
    assert q8._bmm8_ws(17, 1000, 1024, 32) == 4 * 17 * 1000 * 4
    for M, N in ((16, 4096), (33, 1002)):
        assert q8._bmm8_ws(M, N, 7168, 32) == 0
    # more than 64 rows: the optional split of a last round of tiles, sized for
    # the current device's compute units (none without a device)
    assert q8._bmm8_ws(65, 4096, 7168, 32) % 256 == 0
    assert q8._bmm8_ws(65, 4096, 896, 32) == 0
    wargs = lambda ws, wsb: (16, 16, 16, 16, p, 16, q8.Q8_BF16, 33, 4096, 7168, 32, ws, wsb, p)
    assert q8._bmm8(*wargs(p, 0)) == q8.Q8_EWORKSPACE
    assert q8._bmm8(*wargs(32, 4 * 33 * 4096 * 4 - 1)) == q8.Q8_EWORKSPACE
    assert q8._bmm8(*wargs(40, 4 * 33 * 4096 * 4)) == q8.Q8_EINVAL      # misaligned
    assert "aligned" in q8.last_error()


def test_quant_scale_ue8m0_range(q8):
    p = None
    assert q8._quant(8, q8.Q8_BF16, 4, 128, 128, 8, q8.Q8_E4M3FN, 8, 32, 0, 1e-10, -448, 448, 3, 0, p, 0, p, 0, p) == q8.Q8_EINVAL
    assert "scale_ue8m0" in q8.last_error()
    assert q8._quant(p, q8.Q8_BF16, 0, 128, 128, p, q8.Q8_E4M3FN, p, 32, 0, 1e-10, -448, 448, 2, 0, p, 0, p, 0, p) == q8.Q8_OK


def test_noalloc_routing_rejects_beyond_its_scratch_on_the_host(q8):
    """moe_mm_data_noalloc holds 4 MiB of counts per device: larger routings
    are refused before any HIP call (so this runs without a GPU)."""
    T, topk, E = 40000, 8, 1024
    assert q8._moe_ws(T, topk, E) > (4 << 20)
    st = q8._moe_na(8, T, topk, E, 16, 16, 8, 8, 8, 8, 8, None)
    assert st == q8.Q8_EUNSUPPORTED and "scratch" in q8.last_error()
    # the shared argument rules apply as for moe_mm_data
    assert q8._moe_na(8, 4, 2, 0, 16, 16, 8, 8, 8, 8, 8, None) == q8.Q8_EUNSUPPORTED
    assert q8._moe_na(8, 4, 2, 8, 16, 16, None, 8, 8, 8, 8, None) == q8.Q8_EINVAL
