"""The Python binding rejects tensors that do not match what the kernels read
and write (scale tensors of the wrong size or dtype, short routing tables)
before anything reaches the device.

Runs without a GPU: the tensors here live on the CPU, and every shape and
dtype check comes before the device check, so a call with a bad shape fails
with that shape's message and a call with good shapes fails only because the
tensors are not on the GPU.
"""
import os

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "int8_quantized_gemm_amd", "libq8gemm.so")
pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libq8gemm.so not built")

F8, F32, BF16 = torch.float8_e4m3fn, torch.float32, torch.bfloat16


@pytest.fixture(scope="module")
def q8():
    import int8_quantized_gemm_amd as m
    return m


def off_gpu(fn, *a, **k):
    with pytest.raises(ValueError, match="on the GPU"):
        fn(*a, **k)


def rejects(msg, fn, *a, **k):
    with pytest.raises(ValueError, match=msg):
        fn(*a, **k)


def test_quant_scale_tensor_size_and_dtype(q8):
    x = torch.zeros((4, 256), dtype=BF16)
    q = torch.empty((4, 256), dtype=F8)
    off_gpu(q8.quant_8bit, x, q, torch.empty((4, 2), dtype=F32), 128)
    # [M, K/128] scales passed with group 32: the kernel would write 4x past them
    rejects("output_s must hold", q8.quant_8bit, x, q, torch.empty((4, 2), dtype=F32), 32)
    # float32 scales expected, one byte given (and the reverse for packed E8M0)
    rejects("float32", q8.quant_8bit, x, q, torch.empty((4, 2), dtype=torch.uint8), 128)
    rejects("E8M0 byte", q8.quant_8bit, x, q, torch.empty((4, 8), dtype=F32), 32, scale_ue8m0=2)
    off_gpu(q8.quant_8bit, x, q, torch.empty((4, 8), dtype=torch.uint8), 32, scale_ue8m0=2)
    rejects("one-element", q8.quant_8bit, x, q, torch.empty((4, 2), dtype=F32), 0,
            mode=q8.SCALE_PER_TENSOR_DYNAMIC)
    rejects("output_q must be", q8.quant_8bit, x, torch.empty((4, 128), dtype=F8),
            torch.empty((4, 2), dtype=F32), 128)
    rejects("output_q must be float8", q8.quant_8bit, x, torch.empty((4, 256), dtype=BF16),
            torch.empty((4, 2), dtype=F32), 128)


def test_block_gemm_scales_and_operands(q8):
    M, N, K = 8, 300, 512
    a, w = torch.empty((M, K), dtype=F8), torch.empty((N, K), dtype=F8)
    sa, sw = torch.empty((M, 4), dtype=F32), torch.empty((3, 4), dtype=F32)
    off_gpu(q8.blockwise_scaled_mm, a, w, sa, sw)
    rejects("scales_a", q8.blockwise_scaled_mm, a, w, torch.empty((M, 2), dtype=F32), sw)
    rejects("scales_b", q8.blockwise_scaled_mm, a, w, sa, torch.empty((2, 4), dtype=F32))
    rejects("float32", q8.blockwise_scaled_mm, a, w, sa.to(BF16), sw)
    rejects("float8", q8.blockwise_scaled_mm, a.to(BF16), w, sa, sw)
    rejects("bias", q8.blockwise_scaled_mm, a, w, sa, sw, bias=torch.empty(N - 1, dtype=BF16))
    rejects("bias dtype", q8.blockwise_scaled_mm, a, w, sa, sw, bias=torch.empty(N, dtype=F32))
    rejects("out must be", q8.blockwise_scaled_mm, a, w, sa, sw, out=torch.empty((M, N - 1), dtype=BF16))
    # block32 weight scales are [ceil(N/32), K/32]
    off_gpu(q8.blockwise_scaled_mm, a, w, torch.empty((M, 16), dtype=F32),
            torch.empty((10, 16), dtype=F32), block=(32, 32))
    rejects("scales_b", q8.blockwise_scaled_mm, a, w, torch.empty((M, 16), dtype=F32),
            torch.empty((9, 16), dtype=F32), block=(32, 32))


def test_e8m0_gemm_scales(q8):
    M, N, K = 4, 64, 256
    a, w = torch.empty((M, K), dtype=F8), torch.empty((N, K), dtype=F8)
    off_gpu(q8.blockwise_scaled_mm_e8m0, a, w, torch.empty((M, 8), dtype=torch.uint8),
            torch.empty((2, 8), dtype=torch.uint8))
    rejects("scales_a", q8.blockwise_scaled_mm_e8m0, a, w, torch.empty((M, 4), dtype=torch.uint8),
            torch.empty((2, 8), dtype=torch.uint8))
    rejects("one byte", q8.blockwise_scaled_mm_e8m0, a, w, torch.empty((M, 8), dtype=F32),
            torch.empty((2, 8), dtype=torch.uint8))


def test_int8_and_fp8_scaled_operands(q8):
    a, w = torch.empty((8, 64), dtype=torch.int8), torch.empty((32, 64), dtype=torch.int8)
    s1, s2 = torch.ones(8), torch.ones(32)
    off_gpu(q8.scaled_mm_int8, a, w, s1, s2)
    rejects("int8", q8.scaled_mm_int8, a.to(F8), w, s1, s2)
    rejects("float32", q8.scaled_mm_int8, a, w, s1.to(BF16), s2)
    rejects("bias", q8.scaled_mm_int8, a, w, s1, s2, bias=torch.empty(31, dtype=BF16))
    af, wf = a.view(F8), w.view(F8)
    off_gpu(q8.scaled_mm_fp8, af, wf, s1, s2)
    rejects("float8", q8.scaled_mm_fp8, a, wf, s1, s2)
    rejects("out must be", q8.scaled_mm_fp8, af, wf, s1, s2, out=torch.empty((8, 31), dtype=BF16))


def test_grouped_gemm_tables(q8):
    E, N, K, T, topk = 4, 256, 512, 16, 2
    tm = T * topk
    d = torch.empty((tm, N), dtype=BF16)
    a, b = torch.empty((T, K), dtype=F8), torch.empty((E, N, K), dtype=F8)
    sa, sb = torch.empty((T, 4), dtype=F32), torch.empty((E, 2, 4), dtype=F32)
    off = torch.zeros(E + 1, dtype=torch.int32)
    ps = torch.zeros((E, 3), dtype=torch.int32)
    ip = torch.zeros(tm, dtype=torch.int32)
    op = torch.arange(tm, dtype=torch.int32)
    off_gpu(q8.grouped_blockwise_scaled_mm, d, a, b, sa, sb, off, ps, a_map=ip, c_map=op)
    rejects("expert_offsets", q8.grouped_blockwise_scaled_mm, d, a, b, sa, sb, off[:E], ps, a_map=ip, c_map=op)
    rejects("problem_sizes", q8.grouped_blockwise_scaled_mm, d, a, b, sa, sb, off, ps[:2], a_map=ip, c_map=op)
    rejects("a_scales", q8.grouped_blockwise_scaled_mm, d, a, b, torch.empty((T, 2), dtype=F32), sb, off, ps,
            a_map=ip, c_map=op)
    rejects("b_scales", q8.grouped_blockwise_scaled_mm, d, a, b, sa, torch.empty((E, 1, 4), dtype=F32), off, ps,
            a_map=ip, c_map=op)
    rejects("a_map", q8.grouped_blockwise_scaled_mm, d, a, b, sa, sb, off, ps, a_map=ip[:5], c_map=op)
    rejects("c_map", q8.grouped_blockwise_scaled_mm, d, a, b, sa, sb, off, ps, a_map=ip, c_map=op[:5])
    rejects("int32", q8.grouped_blockwise_scaled_mm, d, a, b, sa, sb, off.long(), ps, a_map=ip, c_map=op)
    # without a_map, a holds the sorted rows itself: it must have total_m of them
    rejects("total_m sorted rows", q8.grouped_blockwise_scaled_mm, d, a, b, sa, sb, off, ps)


def test_finalize_and_routing_sizes(q8):
    d = torch.empty((32, 64), dtype=BF16)
    off_gpu(q8.moe_finalize, d, torch.ones((16, 2)), 2)
    rejects("out must be", q8.moe_finalize, d, torch.ones((16, 2)), 2, out=torch.empty((8, 64), dtype=BF16))
    ids = torch.zeros((16, 2), dtype=torch.int32)
    i32 = lambda n: torch.empty(n, dtype=torch.int32)  # noqa: E731
    off_gpu(q8.moe_mm_data, ids, i32(5), i32(12), i32(12), i32(32), i32(32), 4, 64, 64)
    rejects("too small", q8.moe_mm_data, ids, i32(4), i32(12), i32(12), i32(32), i32(32), 4, 64, 64)
