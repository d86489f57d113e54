"""GPU parity: 8-bit activation quantization, bit-exact against the oracle.

Codes and scales must equal the oracle's byte for byte (both sides decide in
float32 with round-to-nearest-even), on the pages' shapes (tiny fp32 [4,512]
g=128; decode rows of 7168 with g=32 UE8M0 and 1% x20 outliers; the prefill
activation [4096,7168] bf16 g=128; INT8 per-token and per-tensor [2048,8192])
and on edge cases (ragged M, every group-size kernel path, strided input,
zero groups, signed zeros, the full bf16 cast sweep).
"""
import numpy as np
import pytest
import torch

import synth
from oracle import quant as oq
from tests.gpu_util import DEV, codes, q8, sync

pytestmark = pytest.mark.gpu

EPS = 1e-10


def run_quant(x, g, ue=False, int8=False, mode=0, static_scale=None):
    m = q8()
    M, K = x.shape
    qd = torch.int8 if int8 else torch.float8_e4m3fn
    q = torch.empty((M, K), dtype=qd, device=DEV)
    if mode == m.SCALE_PER_GROUP:
        s = torch.empty((M, K // g), dtype=torch.float32, device=DEV)
    elif mode == m.SCALE_STATIC:
        s = torch.tensor([static_scale], dtype=torch.float32, device=DEV)
    else:
        s = torch.empty((1,), dtype=torch.float32, device=DEV)
    lo, hi = (-128.0, 127.0) if int8 else (-448.0, 448.0)
    m.quant_8bit(x, q, s, g, EPS, lo, hi, ue, mode=mode)
    sync()
    return codes(q), s.cpu().numpy()


def oracle_quant(x_cpu, g, ue=False, int8=False):
    x32 = x_cpu.float().numpy()
    if int8:
        return oq.per_token_group(x32, g, EPS, -128.0, 127.0, ue, "i8")
    return oq.per_token_group(x32, g, EPS, -448.0, 448.0, ue, "e4m3")


def check(x_cpu, g, ue=False, int8=False):
    qg, sg = run_quant(x_cpu.to(DEV), g, ue, int8)
    qo, so = oracle_quant(x_cpu, g, ue, int8)
    assert np.array_equal(sg, so), f"scales differ at {np.argwhere(sg != so)[:5]}"
    bad = np.argwhere(qg.view(np.uint8) != qo.view(np.uint8))
    assert bad.size == 0, f"{len(bad)} codes differ, first {bad[:5]}"


def test_tiny_fp32_g128():
    check(synth.activations(4, 512, "f32", seed=0), 128)


@pytest.mark.parametrize("M", [1, 4, 16, 64])
def test_decode_rows_g32_ue8m0_outliers(M):
    check(synth.activations(M, 7168, "bf16", outlier_frac=0.01, seed=0), 32, ue=True)


def test_prefill_activation_full_size():
    check(synth.activations(4096, 7168, "bf16", seed=0), 128)


def test_prefill_activation_g32_ue8m0_full_size():
    check(synth.activations(4096, 7168, "bf16", seed=1), 32, ue=True)


@pytest.mark.parametrize("g", [8, 16, 64, 256, 512, 1024, 96, 3 * 64])
@pytest.mark.parametrize("M", [1, 3, 130])
def test_group_sizes_and_ragged_rows(g, M):
    K = 3072 if g != 1024 else 4096
    check(synth.activations(M, K, "bf16", sigma=3.0, seed=g + M), g)


@pytest.mark.parametrize("dtype", ["f16", "f32"])
def test_other_input_dtypes(dtype):
    check(synth.activations(33, 1024, dtype, seed=5), 128, ue=True)
    check(synth.activations(33, 1024, dtype, seed=6), 128)


def test_strided_input_rows():
    full = synth.activations(20, 1536, "bf16", seed=7)
    x = full[:, :1024]  # row stride 1536
    qg, sg = run_quant(full.to(DEV)[:, :1024], 128)
    qo, so = oracle_quant(x.contiguous(), 128)
    assert np.array_equal(sg, so) and np.array_equal(qg.view(np.uint8), qo)


@pytest.mark.parametrize("g", [16, 128])
def test_strided_rows_eight_element_lanes(g):
    """A row stride of 1032 elements (a multiple of 8, not of 16) keeps the
    kernel at 8 elements per lane for every group size."""
    full = synth.activations(24, 1032, "bf16", seed=9)
    x = full[:, :1024]
    qg, sg = run_quant(full.to(DEV)[:, :1024], g)
    qo, so = oracle_quant(x.contiguous(), g)
    assert np.array_equal(sg, so) and np.array_equal(qg.view(np.uint8), qo)


def test_cast_sweep_every_bf16_value():
    """Groups headed by 448 have scale 1, so the codes are the convert of every
    finite bf16 value in range: exercises subnormals, ties, signed zeros."""
    bits = np.arange(65536, dtype=np.uint32) << 16
    v = bits.view(np.float32)
    v = v[np.isfinite(v) & (np.abs(v) <= 448.0)]
    g = 128
    n = -(-v.size // (g - 1))
    x = np.zeros((n, g), dtype=np.float32)
    flat = np.zeros(n * (g - 1), dtype=np.float32)
    flat[:v.size] = v
    x[:, 1:] = flat.reshape(n, g - 1)
    x[:, 0] = 448.0
    xt = torch.from_numpy(x).to(torch.bfloat16)
    check(xt, g)
    check(xt.float(), g)


def test_zero_groups_and_signed_zero():
    x = torch.zeros((3, 256), dtype=torch.bfloat16)
    x[1, 128:] = 1.0
    x[2, 0] = 448.0
    x[2, 1] = -0.0
    x[2, 2] = -(2.0 ** -11)
    check(x, 128)
    check(x, 128, ue=True)


def test_int8_per_token_full_size():
    check(synth.activations(2048, 8192, "bf16", seed=0), 8192, int8=True)


def test_int8_per_token_small_and_groups():
    check(synth.activations(5, 1000, "bf16", sigma=2.0, seed=3), 1000, int8=True)
    check(synth.activations(7, 2048, "bf16", seed=4), 128, int8=True)


@pytest.mark.parametrize("K", [2056, 4104, 16384])
def test_per_token_rows_around_register_limit(K):
    """Rows of up to 8192 elements stay in registers (one, two or four
    8-element vectors per thread); longer rows take the two-pass kernel."""
    x = synth.activations(3, K, "bf16", seed=K)
    check(x, K, int8=True)
    check(x, K)


@pytest.mark.parametrize("M,K,g,dtype,ue,int8", [
    (130, 1536, 1536, "bf16", False, False),  # one wave per row, three slots a lane
    (7, 2040, 2040, "f16", True, False),      # the last lanes re-read the row's end
    (9, 3840, 1920, "f32", False, True),      # two groups per row, one wave each
    (65, 2048, 2048, "bf16", False, True),    # per-token rows of 2048
    (11, 7168, 3584, "bf16", True, False),    # two groups per row, one workgroup each
    (257, 7168, 7168, "bf16", False, False),  # FP8 per-token rows of the prefill width
    (5, 6000, 6000, "f32", False, True),      # f32 rows of one workgroup, ragged slots
])
def test_long_groups_wave_and_workgroup_kernels(M, K, g, dtype, ue, int8):
    """Groups longer than 512 or not powers of two: one wave per group up to
    2048 elements, one workgroup per group up to 8192."""
    check(synth.activations(M, K, dtype, sigma=2.0, seed=M + g), g, ue, int8)


@pytest.mark.parametrize("K,g", [(6144, 1536), (7168, 3584)])
def test_e8m0_byte_scales_long_groups(K, g):
    m = q8()
    x = synth.activations(6, K, "bf16", seed=g)
    q = torch.empty((6, K), dtype=torch.float8_e4m3fn, device=DEV)
    s = torch.empty((6, K // g), dtype=torch.uint8, device=DEV)
    m.quant_8bit(x.to(DEV), q, s, g, EPS, -448.0, 448.0, 2)
    sync()
    qo, so = oracle_quant(x, g, ue=True)
    assert np.array_equal(s.cpu().numpy(), (so.view(np.uint32) >> 23).astype(np.uint8))
    assert np.array_equal(codes(q).view(np.uint8), qo.view(np.uint8))


@pytest.mark.parametrize("g", [1000, 3000])
def test_strided_rows_long_groups(g):
    full = synth.activations(20, 3016, "bf16", seed=g)
    x = full[:, :3000]  # row stride 3016
    qg, sg = run_quant(full.to(DEV)[:, :3000], g, int8=True)
    qo, so = oracle_quant(x.contiguous(), g, int8=True)
    assert np.array_equal(sg, so) and np.array_equal(qg.view(np.uint8), qo.view(np.uint8))


@pytest.mark.parametrize("int8", [False, True])
def test_per_tensor_dynamic(int8):
    m = q8()
    x = synth.activations(2048, 8192, "bf16", seed=0)
    qg, sg = run_quant(x.to(DEV), 0, int8=int8, mode=m.SCALE_PER_TENSOR_DYNAMIC)
    lo, hi, qd = (-128.0, 127.0, "i8") if int8 else (-448.0, 448.0, "e4m3")
    qo, so = oq.per_tensor_dynamic(x.float().numpy(), EPS, lo, hi, False, qd)
    assert sg[0] == so[0]
    assert np.array_equal(qg.view(np.uint8), qo.view(np.uint8))


def test_per_tensor_dynamic_ue8m0_small():
    m = q8()
    x = synth.activations(3, 200, "f32", sigma=5.0, seed=2)
    qg, sg = run_quant(x.to(DEV), 0, ue=True, mode=m.SCALE_PER_TENSOR_DYNAMIC)
    qo, so = oq.per_tensor_dynamic(x.numpy(), EPS, -448.0, 448.0, True, "e4m3")
    assert sg[0] == so[0] and np.array_equal(qg.view(np.uint8), qo)


@pytest.mark.parametrize("int8", [False, True])
def test_static_scale(int8):
    m = q8()
    x = synth.activations(64, 4096, "bf16", sigma=2.0, seed=9)
    sc = 0.0123
    qg, sg = run_quant(x.to(DEV), 0, int8=int8, mode=m.SCALE_STATIC, static_scale=sc)
    lo, hi, qd = (-128.0, 127.0, "i8") if int8 else (-448.0, 448.0, "e4m3")
    qo = oq.static(x.float().numpy(), np.float32(sc), lo, hi, qd)
    assert np.array_equal(qg.view(np.uint8), qo.view(np.uint8))


def test_run_twice_identical():
    x = synth.activations(512, 7168, "bf16", seed=11).to(DEV)
    a = run_quant(x, 128)
    b = run_quant(x, 128)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("g", [20, 100])
def test_unaligned_rows_scalar_path(g):
    # K % 8 != 0: the scalar kernels
    check(synth.activations(5, 100, "bf16", sigma=2.0, seed=8), g)
    check(synth.activations(5, 100, "f32", sigma=2.0, seed=8), g, ue=True)
