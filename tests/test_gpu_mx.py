"""GPU parity: packed E8M0 activation scales (quant_8bit scale_ue8m0=2) and the
E8M0 block-scaled FP8 GEMM (blockwise_scaled_mm_e8m0, MX-scaled MFMA) against
the CPU oracle. Scale bytes and codes bit for bit; GEMM outputs within
|D - D_ref| <= 1e-2 |D_ref| + 1e-3 rms(D_ref). GEMM inputs are quantized by
the oracle on the host, so every expected value comes from oracle/ alone."""
import numpy as np
import pytest
import torch

from gpu_util import DEV, assert_gemm_close, codes, q8, sync
from oracle import gemm as og
from oracle import quant as oq
import synth

pytestmark = pytest.mark.gpu
EPS = 1e-10


def _act(M, K, seed, outliers=0.0):
    x = synth.activations(M, K, "bf16", outlier_frac=outliers, seed=seed)
    aq, s = oq.per_token_group(x.float().numpy(), 32, EPS, -448.0, 448.0, True, "e4m3")
    return x, aq, oq.e8m0_bytes(s)


@pytest.mark.parametrize("M,K", [(1, 7168), (16, 7168), (37, 1024), (300, 2048)])
def test_quant_packed_e8m0(M, K):
    x = synth.activations(M, K, "bf16", outlier_frac=0.01, seed=M)
    m = q8()
    q = torch.empty((M, K), dtype=torch.float8_e4m3fn, device=DEV)
    s = torch.full((M, K // 32), 0x5A, dtype=torch.uint8, device=DEV)
    m.quant_8bit(x.to(DEV), q, s, 32, EPS, -448.0, 448.0, 2)
    sync()
    qo, so = oq.per_token_group(x.float().numpy(), 32, EPS, -448.0, 448.0, True, "e4m3")
    assert np.array_equal(codes(q), qo)
    assert np.array_equal(s.cpu().numpy(), oq.e8m0_bytes(so))


@pytest.mark.parametrize("M,N,K,bn,bias", [
    (1, 256, 512, 32, False),      # K not a multiple of 1024: streaming kernel, one row block
    (4, 4096, 1024, 32, True),
    (37, 200, 1024, 32, False),    # three row blocks, ragged N (17..64 rows: split K)
    (64, 512, 2048, 128, True),
    (24, 4096, 7168, 32, False),   # split K: 4 ranges of 1792 bytes, two row blocks
    (48, 1000, 2048, 64, True),    # split K, bn 64, ragged 64-row weight groups
    (33, 16, 4096, 32, False),     # split K, one weight group of 16 rows
    (20, 1002, 1024, 32, True),    # N not a multiple of 4: the streaming kernel
    (12, 520, 2048, 32, True),     # up to 16 rows: activations staged in LDS, ragged N
    (3, 300, 1024, 32, False),     # staged, three rows
    (9, 48, 3072, 16, False),      # staged, bn 16, three weight-row blocks
    (65, 256, 512, 32, False),     # tile kernel from 65 rows
    (300, 520, 1024, 128, True),   # ragged M and N tiles
    (513, 768, 2048, 32, False),
])
def test_e8m0_gemm_matches_oracle(M, N, K, bn, bias):
    x, aq, asb = _act(M, K, seed=M + N)
    Wq, Wsb = synth.fp8_block_weights_e8m0(N, K, bn, 32, seed=K)
    b = synth.bias(N, seed=1) if bias else None
    ref = og.blockwise_scaled_mm_e8m0(aq, asb, Wq.numpy(), Wsb.numpy(), bn,
                                      None if b is None else b.float().numpy())
    m = q8()
    d = m.blockwise_scaled_mm_e8m0(torch.from_numpy(aq).to(DEV), Wq.to(DEV),
                                   torch.from_numpy(asb).to(DEV), Wsb.to(DEV), torch.bfloat16,
                                   bias=None if b is None else b.to(DEV), block_n=bn)
    sync()
    assert_gemm_close(d, ref, f"e8m0 {M}x{N}x{K} bn={bn}")


def test_e8m0_scale_index_closed_form():
    """Row m of A holds ones only in K block m % KB; activation scales 2^kb,
    weight scales 2^(n // bn - 3): D[m, n] = 32 * 2^(m % KB) * 2^(n // bn - 3),
    a power of two times 32 (exact in bf16). A wrong K-block or N-block index
    changes the power."""
    M, N, K, bn = 80, 96, 512, 32
    KB = K // 32
    A = torch.zeros((M, K), dtype=torch.uint8)
    for r in range(M):
        kb = r % KB
        A[r, 32 * kb:32 * kb + 32] = 0x38
    W = torch.full((N, K), 0x38, dtype=torch.uint8)
    As = torch.from_numpy(np.tile((127 + np.arange(KB)).astype(np.uint8), (M, 1)))
    Ws = torch.from_numpy(np.tile((124 + np.arange(N // bn)).astype(np.uint8)[:, None], (1, KB)))
    want = 32.0 * np.ldexp(1.0, (np.arange(M) % KB)[:, None] + (np.arange(N) // bn)[None, :] - 3)
    ref = og.blockwise_scaled_mm_e8m0(A.numpy(), As.numpy(), W.numpy(), Ws.numpy(), bn)
    assert np.array_equal(ref, want)
    m = q8()
    for M2 in (M, 1, 16):  # tile kernel, then the streaming kernel
        d = m.blockwise_scaled_mm_e8m0(A[:M2].to(DEV), W.to(DEV), As[:M2].to(DEV), Ws.to(DEV),
                                       torch.bfloat16, block_n=bn)
        assert np.array_equal(d.cpu().double().numpy(), want[:M2]), M2


@pytest.mark.parametrize("M", [1, 16, 64])
def test_decode_size(M):
    """Decode block32 shape (N = 4096, K = 7168, 1 % outliers) with power-of-two
    weight scales, every output compared."""
    N, K = 4096, 7168
    x, aq, asb = _act(M, K, seed=0, outliers=0.01)
    Wq, Wsb = synth.fp8_block_weights_e8m0(N, K, 32, 32, seed=0)
    ref = og.blockwise_scaled_mm_e8m0(aq, asb, Wq.numpy(), Wsb.numpy(), 32)
    d = q8().blockwise_scaled_mm_e8m0(torch.from_numpy(aq).to(DEV), Wq.to(DEV),
                                      torch.from_numpy(asb).to(DEV), Wsb.to(DEV), block_n=32)
    sync()
    assert_gemm_close(d, ref, f"decode M={M}")


def test_prefill_size_every_element():
    """4096 x 7168 x 7168 with [32,32] power-of-two blocks, the launch the
    benchmark times: every output element."""
    M, N, K = 4096, 7168, 7168
    x, aq, asb = _act(M, K, seed=0)
    Wq, Wsb = synth.fp8_block_weights_e8m0(N, K, 32, 32, seed=0)
    d = q8().blockwise_scaled_mm_e8m0(torch.from_numpy(aq).to(DEV), Wq.to(DEV),
                                      torch.from_numpy(asb).to(DEV), Wsb.to(DEV), block_n=32)
    sync()
    ref = og.blockwise_scaled_mm_e8m0(aq, asb, Wq.numpy(), Wsb.numpy(), 32)
    assert_gemm_close(d, ref, "prefill e8m0")


def test_quant_then_gemm_pipeline():
    """The GPU quantizer's packed scales feed the GEMM directly (the path a
    caller runs); compared with the oracle's quantize-then-multiply."""
    M, N, K = 200, 384, 1024
    x = synth.activations(M, K, "bf16", seed=5)
    Wq, Wsb = synth.fp8_block_weights_e8m0(N, K, 32, 32, seed=5)
    m = q8()
    q = torch.empty((M, K), dtype=torch.float8_e4m3fn, device=DEV)
    s = torch.empty((M, K // 32), dtype=torch.uint8, device=DEV)
    m.quant_8bit(x.to(DEV), q, s, 32, EPS, -448.0, 448.0, 2)
    d = m.blockwise_scaled_mm_e8m0(q, Wq.to(DEV), s, Wsb.to(DEV), block_n=32)
    sync()
    aq, so = oq.per_token_group(x.float().numpy(), 32, EPS, -448.0, 448.0, True, "e4m3")
    ref = og.blockwise_scaled_mm_e8m0(aq, oq.e8m0_bytes(so), Wq.numpy(), Wsb.numpy(), 32)
    assert_gemm_close(d, ref, "quant + e8m0 gemm")
