"""GPU parity: INT8 W8A8 (per-token x per-channel and per-tensor x per-tensor).

The raw int32 accumulators (out_dtype=int32) must equal the oracle's exact
integer products bit for bit; the scaled bf16 output is checked with the FP8
GEMM tolerance. The activation quant is the GPU's own (bit-exact against the
oracle's, checked here too).
"""
import numpy as np
import pytest
import torch

import synth
from oracle import gemm as og
from oracle import quant as oq
from tests.gpu_util import DEV, assert_gemm_close, codes, q8, sync

pytestmark = pytest.mark.gpu

EPS = 1e-10


def gpu_quant_int8(x_dev, per_tensor):
    m = q8()
    M, K = x_dev.shape
    q = torch.empty((M, K), dtype=torch.int8, device=DEV)
    if per_tensor:
        s = torch.empty((1,), dtype=torch.float32, device=DEV)
        m.quant_8bit(x_dev, q, s, 0, EPS, -128.0, 127.0, False, mode=m.SCALE_PER_TENSOR_DYNAMIC)
    else:
        s = torch.empty((M, 1), dtype=torch.float32, device=DEV)
        m.quant_8bit(x_dev, q, s, K, EPS, -128.0, 127.0, False)
    return q, s


def oracle_quant_int8(x_cpu, per_tensor):
    x = x_cpu.float().numpy()
    if per_tensor:
        return oq.per_tensor_dynamic(x, EPS, -128.0, 127.0, False, "i8")
    return oq.per_token_group(x, x.shape[1], EPS, -128.0, 127.0, False, "i8")


def run_case(M, N, K, per_tensor, bias=True, rows=None, seed=0, transposed_b=False):
    m = q8()
    x = synth.activations(M, K, "bf16", seed=seed)
    Wq, ws = synth.int8_weights(N, K, per_channel=not per_tensor, seed=seed)
    b = synth.bias(N, seed=seed) if bias else None
    qa, sa = gpu_quant_int8(x.to(DEV), per_tensor)
    W_dev = Wq.to(DEV)
    Wb = W_dev.t() if transposed_b else W_dev
    acc = m.scaled_mm_int8(qa, Wb, None, None, torch.int32)
    d = m.scaled_mm_int8(qa, Wb, sa, ws.to(DEV), torch.bfloat16, None if b is None else b.to(DEV))
    sync()
    qo, so = oracle_quant_int8(x, per_tensor)
    sel = slice(None) if rows is None else rows
    assert np.array_equal(codes(qa)[sel], qo[sel])
    assert np.array_equal(sa.cpu().numpy().reshape(-1)[sel if not per_tensor else slice(None)],
                          so.reshape(-1)[sel if not per_tensor else slice(None)])
    acc_ref = og.int8_acc(qo[sel], Wq.numpy())
    assert np.array_equal(acc.cpu().numpy()[sel].astype(np.int64), acc_ref)
    sa_ref = so if per_tensor else so.reshape(-1)[sel]
    ref = og.scaled_mm_int8(qo[sel], sa_ref, Wq.numpy(), ws.numpy(),
                            None if b is None else b.float().numpy(), acc=acc_ref)
    assert_gemm_close(d.cpu()[sel] if rows is not None else d, ref, f"int8 M={M} N={N} K={K}")


@pytest.mark.parametrize("per_tensor", [False, True])
def test_full_size_every_element(per_tensor):
    """2048 x 8192 x 8192 as the benchmark launches it: every code, scale and
    int32 accumulator bit for bit, every bf16 output within tolerance."""
    run_case(2048, 8192, 8192, per_tensor)


@pytest.mark.parametrize("x_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("per_tensor", [False, True])
def test_ties_round_half_to_even(x_dtype, per_tensor):
    """Quotients exactly halfway between two integers. Per token, rows whose
    |max| is 127 get s = 1 and hold k + 0.5, rows whose |max| is 254 get s = 2
    and hold odd integers (x / s = k + 0.5 again). Per tensor every row holds
    odd integers and the |max| 254 sits in the last row (s = 2 for all).
    Codes must be rint with ties to even, as the oracle has them and as
    written out here from the values."""
    M, K = 64, 1024
    r = np.random.default_rng(11)
    x = np.empty((M, K), dtype=np.float32)
    for m in range(M):
        if m % 2 == 0 and not per_tensor:
            x[m] = r.integers(-127, 127, size=K) + 0.5    # all in (-127, 127)
            x[m, r.integers(K)] = 127.0 if m % 4 == 0 else -127.0
        else:
            x[m] = 2 * r.integers(-127, 126, size=K) + 1  # odd, |x| <= 253
            if not per_tensor:
                x[m, r.integers(K)] = 254.0 if m % 4 == 1 else -254.0
    if per_tensor:
        x[M - 1, K // 2] = -254.0
    xt = torch.from_numpy(x).to(torch.bfloat16 if x_dtype == "bf16" else torch.float32)
    assert np.array_equal(xt.float().numpy(), x)          # every value exact in bf16
    q, s = gpu_quant_int8(xt.to(DEV), per_tensor)
    sync()
    qo, so = oracle_quant_int8(xt, per_tensor)
    assert np.array_equal(codes(q), qo)
    assert np.array_equal(s.cpu().numpy().reshape(-1), so.reshape(-1))
    if per_tensor:
        scale = np.full((M, 1), 2.0)
    else:
        scale = np.where(np.arange(M) % 2 == 0, 1.0, 2.0)[:, None]
    assert np.array_equal(so.reshape(-1), np.full(1, 2.0) if per_tensor else scale.reshape(-1))
    y = x.astype(np.float64) / scale                      # exact: k + 0.5 or +-127
    halves = y - np.floor(y) == 0.5
    assert halves.mean() > 0.99
    lo = np.floor(y)
    even = np.where(lo % 2 == 0, lo, lo + 1)
    expect = np.where(halves, even, y).astype(np.int64)
    assert np.array_equal(codes(q).astype(np.int64), expect)


@pytest.mark.parametrize("M,N,K", [(1, 16, 16), (5, 48, 1040), (300, 528, 1040), (257, 4096, 2048)])
@pytest.mark.parametrize("per_tensor", [False, True])
def test_shapes_full_compare(M, N, K, per_tensor):
    run_case(M, N, K, per_tensor, seed=M + K)


def test_transposed_weight_view_and_no_bias():
    run_case(70, 256, 512, False, bias=False, transposed_b=True, seed=1)


def test_mixed_scale_combinations_broadcast():
    m = q8()
    M, N, K = 64, 128, 256
    r = np.random.default_rng(3)
    A = torch.from_numpy(r.integers(-128, 128, size=(M, K)).astype(np.int8))
    W = torch.from_numpy(r.integers(-128, 128, size=(N, K)).astype(np.int8))
    sa_t = torch.from_numpy(r.uniform(0.01, 0.1, size=M).astype(np.float32))
    sb_t = torch.from_numpy(r.uniform(0.01, 0.1, size=N).astype(np.float32))
    for sa, sb in ((sa_t, sb_t[:1]), (sa_t[:1], sb_t)):
        d = m.scaled_mm_int8(A.to(DEV), W.to(DEV), sa.to(DEV), sb.to(DEV), torch.bfloat16)
        ref = og.scaled_mm_int8(A.numpy(), sa.numpy(), W.numpy(), sb.numpy())
        assert_gemm_close(d, ref, "broadcast")


def test_extreme_accumulators_exact():
    m = q8()
    M, N, K = 32, 64, 8192
    A = torch.full((M, K), -128, dtype=torch.int8)
    W = torch.full((N, K), -128, dtype=torch.int8)
    W[1::2] = 127
    acc = m.scaled_mm_int8(A.to(DEV), W.to(DEV), None, None, torch.int32)
    assert np.array_equal(acc.cpu().numpy().astype(np.int64), og.int8_acc(A.numpy(), W.numpy()))
