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


# ---- split of the last round of tiles ------------------------------------------
def _mx_capi(aq, asb, Wd, Wsd, d, bn, ws=None):
    """blockwise_scaled_mm_e8m0 through the C ABI with an explicit workspace
    (None: no workspace, every tile whole)."""
    m = q8()
    M, K = aq.shape
    N = Wd.shape[0]
    wp, wb = (ws.data_ptr(), ws.numel()) if ws is not None else (None, 0)
    r = m._bmm8(aq.data_ptr(), asb.data_ptr(), Wd.data_ptr(), Wsd.data_ptr(), None, d.data_ptr(),
                m.Q8_BF16, M, N, K, bn, wp, wb, torch.cuda.current_stream().cuda_stream)
    assert r == 0, m.last_error()


def test_e8m0_split_tiles_share_a_workspace_across_calls():
    """768 x 2816 x 2048: 33 tiles, each split in K between an owner and a
    helper. Two calls with different activations on one workspace whose bytes
    start as random garbage: each matches the oracle, and each agrees with the
    unsplit kernel within float32 rounding."""
    m = q8()
    M, N, K, bn = 768, 2816, 2048, 32
    need = m._bmm8_ws(M, N, K, bn)
    assert need >= 33 * 256 * 256 * 4
    ws = torch.randint(0, 256, (need,), dtype=torch.uint8, device=DEV)
    Wq, Wsb = synth.fp8_block_weights_e8m0(N, K, bn, 32, seed=12)
    Wd, Wsd = Wq.to(DEV), Wsb.to(DEV)
    for seed in (51, 52):
        x, aq, asb = _act(M, K, seed=seed)
        aqd, asd = torch.from_numpy(aq).to(DEV), torch.from_numpy(asb).to(DEV)
        d_split = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
        d_whole = torch.empty_like(d_split)
        _mx_capi(aqd, asd, Wd, Wsd, d_split, bn, ws)
        _mx_capi(aqd, asd, Wd, Wsd, d_whole, bn, None)
        sync()
        ref = og.blockwise_scaled_mm_e8m0(aq, asb, Wq.numpy(), Wsb.numpy(), bn)
        assert_gemm_close(d_split, ref, f"e8m0 split seed={seed}")
        assert_gemm_close(d_whole, ref, f"e8m0 whole seed={seed}")
        diff = (d_split.float() - d_whole.float()).abs()
        assert float(diff.max()) <= float(d_whole.float().abs().max()) * 2 ** -6


@pytest.mark.parametrize("M,N,K", [(3072, 7168, 7168), (300, 520, 1024)])
def test_e8m0_split_without_wait_equals_unsplit(M, N, K):
    """With no wait each split tile's owner runs on through the rest of K, the
    same MFMA chain as the unsplit kernel: equal bit for bit (3072 x 7168 x
    7168: 80 split tiles after one whole round). A later call with the default
    wait agrees with the unsplit kernel within float32 rounding."""
    m = q8()
    bn = 32
    x, aq, asb = _act(M, K, seed=61)
    Wq, Wsb = synth.fp8_block_weights_e8m0(N, K, bn, 32, seed=61)
    Wd, Wsd = Wq.to(DEV), Wsb.to(DEV)
    aqd, asd = torch.from_numpy(aq).to(DEV), torch.from_numpy(asb).to(DEV)
    need = m._bmm8_ws(M, N, K, bn)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    d_whole = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    d_nowait = torch.empty_like(d_whole)
    d_split = torch.empty_like(d_whole)
    _mx_capi(aqd, asd, Wd, Wsd, d_whole, bn, None)
    try:
        m.set_split_wait_us(0)
        _mx_capi(aqd, asd, Wd, Wsd, d_nowait, bn, ws)
    finally:
        m.set_split_wait_us(200)
    _mx_capi(aqd, asd, Wd, Wsd, d_split, bn, ws)
    sync()
    assert torch.equal(d_nowait, d_whole)
    diff = (d_split.float() - d_whole.float()).abs()
    assert float(diff.max()) <= float(d_whole.float().abs().max()) * 2 ** -6


def test_e8m0_split_tiles_in_a_graph_replay():
    """The split launch captured in a HIP graph: replays with new activations
    (and eager calls between them) each equal an eager call on the same
    inputs."""
    m = q8()
    M, N, K, bn = 640, 1536, 2048, 32
    Wq, Wsb = synth.fp8_block_weights_e8m0(N, K, bn, 32, seed=71)
    Wd, Wsd = Wq.to(DEV), Wsb.to(DEV)
    _, aq, asb = _act(M, K, seed=71)
    aqd, asd = torch.from_numpy(aq).to(DEV), torch.from_numpy(asb).to(DEV)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        m.blockwise_scaled_mm_e8m0(aqd, Wd, asd, Wsd, block_n=bn, out=out)
    torch.cuda.current_stream().wait_stream(s)
    sync()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        m.blockwise_scaled_mm_e8m0(aqd, Wd, asd, Wsd, block_n=bn, out=out)
    for seed in (72, 73, 74):
        _, aq2, asb2 = _act(M, K, seed=seed)
        aqd.copy_(torch.from_numpy(aq2).to(DEV))
        asd.copy_(torch.from_numpy(asb2).to(DEV))
        eager = m.blockwise_scaled_mm_e8m0(aqd.clone(), Wd, asd.clone(), Wsd, block_n=bn)
        sync()
        g.replay()
        sync()
        assert torch.equal(out, eager), f"replay with seed {seed}"
