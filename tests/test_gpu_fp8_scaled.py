"""GPU parity: per-tensor / per-token FP8 quant + FP8 scaled GEMM against the oracle.

The activations go through the library's own per-token (one group per row)
or per-tensor dynamic FP8 quant, the weights are checkpoint-style per-channel
(one scale per row) or per-tensor FP8; the oracle quantizes in numpy and
multiplies exactly in float64. Quantized bytes must match exactly; GEMM
outputs must satisfy |D - D_ref| <= 1e-2 |D_ref| + 1e-3 rms(D_ref).
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


def weights(N, K, per_channel, seed):
    # per-channel: one tile per row (bn = 1, bk = K); per-tensor: one tile
    Wq, Ws = synth.fp8_block_weights(N, K, 1 if per_channel else N, K, seed=seed)
    return Wq, Ws.reshape(-1)


def run_case(M, N, K, *, per_token=True, per_channel=True, bias=False, seed=0,
             out_dtype=torch.bfloat16, rows=None, transposed_b=False):
    m = q8()
    x = synth.activations(M, K, "bf16", seed=seed)
    Wq, Ws = weights(N, K, per_channel, seed)
    b = synth.bias(N, "bf16" if out_dtype == torch.bfloat16 else "f16", seed=seed) if bias else None
    # GPU: quant then GEMM
    aq = torch.empty((M, K), dtype=torch.float8_e4m3fn, device=DEV)
    if per_token:
        sa = torch.empty((M, 1), dtype=torch.float32, device=DEV)
        m.quant_8bit(x.to(DEV), aq, sa, K, EPS, -448.0, 448.0, False)
    else:
        sa = torch.empty((1,), dtype=torch.float32, device=DEV)
        m.quant_8bit(x.to(DEV), aq, sa, K, EPS, -448.0, 448.0, False, mode=m.SCALE_PER_TENSOR_DYNAMIC)
    wq_dev = Wq.to(DEV).view(torch.float8_e4m3fn)
    mat_b = wq_dev.t() if transposed_b else wq_dev
    d = m.scaled_mm_fp8(aq, mat_b, sa.reshape(-1), Ws.to(DEV), out_dtype,
                        None if b is None else b.to(DEV))
    sync()
    # oracle
    xn = x.float().numpy()
    if per_token:
        aq_o, sa_o = oq.per_token_group(xn, K, EPS, -448.0, 448.0, False, "e4m3")
    else:
        aq_o, sa_o = oq.per_tensor_dynamic(xn, EPS, -448.0, 448.0, False, "e4m3")
    assert np.array_equal(codes(aq), aq_o)
    assert np.array_equal(sa.cpu().numpy().reshape(-1), np.asarray(sa_o, np.float32).reshape(-1))
    sel = slice(None) if rows is None else rows
    ref = og.scaled_mm_fp8(aq_o[sel], np.asarray(sa_o).reshape(-1)[sel] if per_token else sa_o,
                           Wq.numpy(), Ws.numpy(), None if b is None else b.float().numpy())
    got = d if rows is None else d[torch.as_tensor(rows, device=DEV)]
    assert_gemm_close(got, ref, f"M={M} N={N} K={K} per_token={per_token} per_channel={per_channel}")


@pytest.mark.parametrize("M,N,K", [(1, 256, 512), (130, 512, 1024), (300, 1024, 7168),
                                   (257, 16, 400), (65, 4096, 2064)])
def test_per_token_per_channel_shapes(M, N, K):
    run_case(M, N, K, bias=True, seed=M + N)


@pytest.mark.parametrize("per_token,per_channel", [(False, False), (True, False), (False, True)])
def test_scale_combinations(per_token, per_channel):
    run_case(200, 384, 1024, per_token=per_token, per_channel=per_channel, seed=3)
    run_case(33, 384, 400, per_token=per_token, per_channel=per_channel, seed=4)


def test_f16_output_and_transposed_weight_view():
    run_case(96, 256, 768, bias=True, out_dtype=torch.float16, seed=5)
    run_case(96, 256, 768, transposed_b=True, seed=6)


def test_prefill_full_size_every_element():
    """4096 x 7168 x 7168 per-token x per-channel, as the benchmark launches
    it: every code, scale and output element."""
    run_case(4096, 7168, 7168, seed=0)


def test_zero_m_and_run_twice():
    m = q8()
    a = torch.zeros((0, 256), dtype=torch.float8_e4m3fn, device=DEV)
    w = torch.zeros((128, 256), dtype=torch.float8_e4m3fn, device=DEV)
    one = torch.ones(1, device=DEV)
    assert m.scaled_mm_fp8(a, w, one, one).shape == (0, 128)
    x = synth.activations(300, 1024, "bf16", seed=9).to(DEV)
    aq = torch.empty((300, 1024), dtype=torch.float8_e4m3fn, device=DEV)
    sa = torch.empty((300, 1), dtype=torch.float32, device=DEV)
    m.quant_8bit(x, aq, sa, 1024, EPS, -448.0, 448.0, False)
    Wq, Ws = weights(512, 1024, True, 9)
    wd, sd = Wq.to(DEV).view(torch.float8_e4m3fn), Ws.to(DEV)
    d1 = m.scaled_mm_fp8(aq, wd, sa.reshape(-1), sd)
    d2 = m.scaled_mm_fp8(aq, wd, sa.reshape(-1), sd)
    assert torch.equal(d1, d2)
