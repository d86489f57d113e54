"""On the GPU: the binding rejects mis-sized or mis-typed scale tensors and
routing tables with ValueError before anything is launched, so outputs keep
their previous contents (the kernels would otherwise read or write past the
tensors' allocations)."""
import pytest
import torch

from tests.gpu_util import DEV, q8

pytestmark = pytest.mark.gpu

F8, F32, BF16 = torch.float8_e4m3fn, torch.float32, torch.bfloat16


def sentinel(shape, dtype):
    t = torch.empty(shape, dtype=dtype, device=DEV)
    t.view(torch.uint8).fill_(0x5A)
    return t


def untouched(t):
    torch.cuda.synchronize()
    return bool((t.view(torch.uint8) == 0x5A).all())


def test_quant_rejects_short_scales_on_device():
    m = q8()
    x = torch.randn((8, 512), dtype=BF16, device=DEV)
    q, s = sentinel((8, 512), F8), sentinel((8, 4), F32)
    with pytest.raises(ValueError, match="output_s must hold"):
        m.quant_8bit(x, q, s, 32)  # [M, K/128] scales passed with group 32
    with pytest.raises(ValueError, match="float32"):
        m.quant_8bit(x, q, sentinel((8, 4), torch.uint8), 128)
    assert untouched(q) and untouched(s)


def test_block_gemm_rejects_bad_scales_on_device():
    m = q8()
    M, N, K = 64, 512, 1024
    a, w = sentinel((M, K), F8), sentinel((N, K), F8)
    d = sentinel((M, N), BF16)
    sw = sentinel((N // 128, K // 128), F32)
    with pytest.raises(ValueError, match="scales_a"):
        m.blockwise_scaled_mm(a, w, sentinel((M, K // 256), F32), sw, out=d)
    with pytest.raises(ValueError, match="scales"):
        m.blockwise_scaled_mm(a, w, sentinel((M, K // 128), torch.float16), sw, out=d)
    assert untouched(d)


def test_grouped_gemm_rejects_short_offsets_on_device():
    m = q8()
    E, N, K, rows = 4, 256, 512, 64
    a = sentinel((rows, K), F8)
    b = sentinel((E, N, K), F8)
    sa = sentinel((rows, K // 128), F32)
    sb = sentinel((E, N // 128, K // 128), F32)
    d = sentinel((rows, N), BF16)
    ps = torch.zeros((E, 3), dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError, match="expert_offsets"):
        m.grouped_blockwise_scaled_mm(d, a, b, sa, sb, torch.zeros(E, dtype=torch.int32, device=DEV), ps)
    with pytest.raises(ValueError, match="int32"):
        m.grouped_blockwise_scaled_mm(d, a, b, sa, sb, torch.zeros(E + 1, dtype=torch.int64, device=DEV), ps)
    assert untouched(d)
