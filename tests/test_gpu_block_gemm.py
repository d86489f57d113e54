"""GPU parity: activation quant + block-scaled FP8 GEMM against the oracle.

Each side runs the whole hot path from the same seeded bf16/fp32 activations
and checkpoint-style weights: the GPU quantizes with its kernel and multiplies
with its kernel; the oracle quantizes and multiplies in numpy (exact fp8
decode, float64 accumulation). Quantized bytes must match exactly; GEMM
outputs must satisfy |D - D_ref| <= 1e-2 |D_ref| + 1e-3 rms(D_ref).
Full-size prefill shapes are compared element by element like every other
shape (the oracle computes the whole output).
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


def gpu_path(x_dev, Wq, Ws, g, ue, bn, bk, bias=None, out_dtype=torch.bfloat16):
    m = q8()
    M, K = x_dev.shape
    aq = torch.empty((M, K), dtype=torch.float8_e4m3fn, device=DEV)
    As = torch.empty((M, K // g), dtype=torch.float32, device=DEV)
    m.quant_8bit(x_dev, aq, As, g, EPS, -448.0, 448.0, ue)
    d = m.blockwise_scaled_mm(aq, Wq.to(DEV), As, Ws.to(DEV), out_dtype,
                              None if bias is None else bias.to(DEV), block=(bn, bk))
    sync()
    return aq, As, d


def oracle_path(x_cpu, Wq, Ws, g, ue, bn, bk, bias=None, rows=None):
    x = x_cpu.float().numpy()
    if rows is not None:
        x = x[rows]
    aq, As = oq.per_token_group(x, g, EPS, -448.0, 448.0, ue, "e4m3")
    b = None if bias is None else bias.float().numpy()
    return aq, As, og.blockwise_scaled_mm(aq, As, Wq.numpy(), Ws.numpy(), bn, bk, bias=b)


def run_case(M, N, K, bn, bk, *, ue=False, x_dtype="bf16", outliers=0.0, bias=False,
             rows=None, seed=0, out_dtype=torch.bfloat16):
    x = synth.activations(M, K, x_dtype, outlier_frac=outliers, seed=seed)
    Wq, Ws = synth.fp8_block_weights(N, K, bn, bk, seed=seed)
    b = synth.bias(N, "bf16" if out_dtype == torch.bfloat16 else "f16", seed=seed) if bias else None
    aq_g, as_g, d = gpu_path(x.to(DEV), Wq, Ws, bk, ue, bn, bk, b, out_dtype)
    aq_o, as_o, ref = oracle_path(x, Wq, Ws, bk, ue, bn, bk, b, rows)
    sel = slice(None) if rows is None else rows
    assert np.array_equal(codes(aq_g)[sel], aq_o)
    assert np.array_equal(as_g.cpu().numpy()[sel], as_o)
    assert_gemm_close(d[sel] if rows is None else d[torch.as_tensor(rows, device=DEV)], ref,
                      f"M={M} N={N} K={K} bn={bn} bk={bk}")
    return d


def test_tiny_fp32_block128():
    run_case(4, 256, 512, 128, 128, x_dtype="f32")


@pytest.mark.parametrize("M", [1, 2, 3, 4, 8, 12, 16, 64])
def test_decode_block32_ue8m0(M):
    run_case(M, 4096, 7168, 32, 32, ue=True, outliers=0.01)


@pytest.mark.parametrize("M,N,K", [(8, 1000, 1024), (13, 520, 2048), (16, 4096, 8192),
                                   (9, 48, 3072), (16, 16, 1024), (5, 1000, 1024),
                                   (7, 4096, 7168), (1, 4096, 7168), (3, 520, 3072)])
@pytest.mark.parametrize("bk", [128, 32])
def test_decode_shared_activation_shapes(M, N, K, bk):
    """Up to 16 activation rows (either block width) and
    K a multiple of 1024 take the kernel that stages the activations once per
    workgroup: waves without K chunks (K = 1024), one, two, four, seven or
    eight chunks per wave, ragged N, the largest K it accepts (8192)."""
    run_case(M, N, K, bk, bk, ue=(bk == 32), bias=True, seed=M * 7 + K)


@pytest.mark.parametrize("M,K", [(1, 1536), (3, 2560), (16, 1536)])
def test_decode_unstaged_128_blocks(M, K):
    """128-wide blocks with K not a multiple of 1024: the streaming kernel
    whose waves read the activations from L2."""
    run_case(M, 520, K, 128, 128, bias=True, seed=M + K)


@pytest.mark.parametrize("M", [5, 6, 8])
def test_decode_packed_two_row_groups(M):
    """5..8 rows, 32-wide blocks, K not a multiple of 1024: the packed kernel
    with two four-row MFMA groups (the staged kernel does not apply)."""
    run_case(M, 520, 1536, 32, 32, ue=True, bias=True, seed=M)


@pytest.mark.parametrize("M,K", [(1, 1536), (2, 2560), (4, 7296)])
def test_decode_packed_one_row_group(M, K):
    """1..4 rows, 32-wide blocks, K not a multiple of 1024: the packed kernel
    with one four-row MFMA group (rows past M padded)."""
    run_case(M, 520, K, 32, 32, ue=True, bias=True, seed=M + K)


@pytest.mark.parametrize("M,N,K,bn,bk", [(17, 1000, 1024, 128, 128), (33, 4096, 7168, 32, 32),
                                        (48, 520, 2048, 32, 32), (64, 300, 512, 128, 128),
                                        (40, 4096, 7168, 128, 128), (30, 600, 1024, 48, 128),
                                        (64, 4096, 7168, 32, 32), (20, 1002, 1024, 128, 128),
                                        (24, 16, 4096, 32, 32)])
def test_decode_mid_rows(M, N, K, bn, bk):
    """17 .. 64 activation rows: K split into ranges whose float32 partials
    a second kernel sums (ragged N, bias, a range of two chunks (K = 1024 in
    four), one 64-row workgroup column (N = 16), bn != bk), and N not a
    multiple of 4, which takes the kernel without partials."""
    run_case(M, N, K, bn, bk, ue=(bk == 32), bias=True, seed=M + N)


@pytest.mark.parametrize("N", [7168, 18432])
@pytest.mark.parametrize("bias", [False, True])
def test_prefill_full_size_every_element(N, bias):
    """4096 x N x 7168 with [128,128] blocks, the launches the benchmark times:
    every code, scale and output element."""
    run_case(4096, N, 7168, 128, 128, bias=bias)


@pytest.mark.parametrize("M,N,K", [(65, 256, 256), (300, 520, 1024), (513, 1000, 512),
                                   (257, 16, 384), (96, 4096, 7168)])
@pytest.mark.parametrize("bk", [128, 32])
def test_tile_shapes_ragged(M, N, K, bk):
    run_case(M, N, K, bk, bk, ue=(bk == 32), bias=True, seed=M + N)


@pytest.mark.parametrize("M,N,K", [(300, 256, 128), (130, 512, 8192), (130, 300, 8320), (257, 520, 640)])
def test_tile_k_extent(M, N, K):
    """K extents of the 128-wide-block tile kernel's slab loops: a single slab
    (K = 128), the most K blocks whose weight scales one lane register holds
    (K = 8192, 64 blocks), one more (K = 8320, the other loop), and an odd
    slab count (K = 640)."""
    run_case(M, N, K, 128, 128, bias=True, seed=K)


@pytest.mark.parametrize("M,N,K,bn,bk,out_dtype", [
    (130, 301, 1024, 128, 128, torch.bfloat16), (70, 517, 512, 32, 32, torch.bfloat16),
    (200, 603, 512, 48, 128, torch.bfloat16), (130, 301, 1024, 128, 128, torch.float16)])
def test_bias_unaligned_columns(M, N, K, bn, bk, out_dtype):
    """A bias with N not a multiple of four: the tile kernel's bias instance
    then reads and stores element by element (and with bn = 48 takes the
    general slab loop)."""
    run_case(M, N, K, bn, bk, ue=(bk == 32), bias=True, out_dtype=out_dtype, seed=N)


@pytest.mark.parametrize("bn", [48, 64, 256])
def test_weight_block_rows_differ_from_bk(bn):
    run_case(200, 600, 512, bn, 128, seed=3)
    run_case(10, 600, 512, bn, 128, seed=4)


@pytest.mark.parametrize("M", [3, 100])
def test_k_not_multiple_of_128(M):
    run_case(M, 200, 96, 32, 32, seed=5)


def test_f16_output_and_bias():
    run_case(130, 384, 1024, 128, 128, bias=True, out_dtype=torch.float16, seed=6)
    run_case(7, 384, 1024, 128, 128, bias=True, out_dtype=torch.float16, seed=7)


def test_one_hot_weights_gather_exactly():
    """W row n holds a single 1.0 at column pi(n) with unit weight scales, so
    D[m, n] = As[m, pi(n)/bk] * A[m, pi(n)]: one float32 product, then bf16.
    Equality catches transposed operands and scale mis-indexing."""
    m = q8()
    M, N, K, bk = 130, 256, 1024, 128
    r = np.random.default_rng(0)
    pi = r.permutation(K)[:N]
    Wq = torch.zeros((N, K), dtype=torch.uint8)
    Wq[torch.arange(N), torch.from_numpy(pi)] = 0x38
    Ws = torch.ones(((N + bk - 1) // bk, K // bk), dtype=torch.float32)
    x = synth.activations(M, K, "bf16", seed=1)
    for Mx in (M, 9):
        aq_g, as_g, d = gpu_path(x[:Mx].to(DEV), Wq, Ws, bk, False, bk, bk)
        aq_o, as_o = oq.per_token_group(x[:Mx].float().numpy(), bk, EPS, -448.0, 448.0, False, "e4m3")
        from oracle import e4m3
        expect = as_o[:, pi // bk].astype(np.float32) * e4m3.decode(aq_o[:, pi]).astype(np.float32)
        expect_bf16 = torch.from_numpy(expect).to(torch.bfloat16).double().numpy()
        assert np.array_equal(d.cpu().double().numpy(), expect_bf16)


def test_run_twice_identical_and_zero_m():
    m = q8()
    x = synth.activations(300, 1024, "bf16", seed=2).to(DEV)
    Wq, Ws = synth.fp8_block_weights(512, 1024, 128, 128, seed=2)
    d1 = gpu_path(x, Wq, Ws, 128, False, 128, 128)[2]
    d2 = gpu_path(x, Wq, Ws, 128, False, 128, 128)[2]
    assert torch.equal(d1, d2)
    e = m.blockwise_scaled_mm(torch.empty((0, 1024), dtype=torch.float8_e4m3fn, device=DEV),
                              Wq.to(DEV), torch.empty((0, 8), device=DEV), Ws.to(DEV))
    assert e.shape == (0, 512)


# ---- split of the last round of tiles ------------------------------------------
def _bmm_capi(aq, As, Wd, Wsd, d, bn, bk, ws=None):
    """blockwise_scaled_mm through the C ABI with an explicit workspace (None:
    no workspace, every tile whole)."""
    m = q8()
    M, K = aq.shape
    N = Wd.shape[0]
    wp, wb = (ws.data_ptr(), ws.numel()) if ws is not None else (None, 0)
    r = m._bmm(aq.data_ptr(), As.data_ptr(), Wd.data_ptr(), Wsd.data_ptr(), None, d.data_ptr(),
               m.Q8_BF16, M, N, K, bn, bk, wp, wb, torch.cuda.current_stream().cuda_stream)
    assert r == 0, m.last_error()


def _quantized(M, K, bk, seed):
    m = q8()
    x = synth.activations(M, K, "bf16", seed=seed)
    aq = torch.empty((M, K), dtype=torch.float8_e4m3fn, device=DEV)
    As = torch.empty((M, K // bk), dtype=torch.float32, device=DEV)
    m.quant_8bit(x.to(DEV), aq, As, bk, EPS, -448.0, 448.0, False)
    return x, aq, As


@pytest.mark.parametrize("bk", [128, 32])
def test_split_tiles_share_a_workspace_across_calls(bk):
    """768 x 2816 x 2048: 33 tiles, each split in K between two workgroups.
    Two calls with different activations on one workspace whose bytes start
    as random garbage: each output matches the oracle (a stale partial or a
    flag word that happened to look set would break the second call), and
    both split calls agree with the unsplit kernel within float32 rounding."""
    m = q8()
    M, N, K = 768, 2816, 2048
    need = m._bmm_ws(M, N, K, bk, bk)
    assert need >= 33 * 256 * 256 * 4
    ws = torch.randint(0, 256, (need,), dtype=torch.uint8, device=DEV)
    Wq, Ws = synth.fp8_block_weights(N, K, bk, bk, seed=11)
    Wd, Wsd = Wq.to(DEV), Ws.to(DEV)
    for seed in (21, 22):
        x, aq, As = _quantized(M, K, bk, seed)
        d_split = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
        d_whole = torch.empty_like(d_split)
        _bmm_capi(aq, As, Wd, Wsd, d_split, bk, bk, ws)
        _bmm_capi(aq, As, Wd, Wsd, d_whole, bk, bk, None)
        sync()
        ref = oracle_path(x, Wq, Ws, bk, False, bk, bk)[2]
        assert_gemm_close(d_split, ref, f"split seed={seed}")
        assert_gemm_close(d_whole, ref, f"whole seed={seed}")
        diff = (d_split.float() - d_whole.float()).abs()
        assert float(diff.max()) <= float(d_whole.float().abs().max()) * 2 ** -6


@pytest.mark.parametrize("M,N,K", [(4096, 18432, 7168), (300, 520, 1024)])
def test_split_without_wait_equals_unsplit(M, N, K):
    """With no wait (q8gemm_set_split_wait_us(0)) each tile's first part
    computes the rest of K itself, folding the same products in the same
    order as the unsplit kernel: equal bit for bit, also at 4096 x 18432 x
    7168 (128 split tiles after four whole rounds). The helpers still write
    their partials and flag words; a later call with the default wait must
    still match the oracle (small shape) or the unsplit kernel within float32
    rounding."""
    m = q8()
    x, aq, As = _quantized(M, K, 128, 31)
    Wq, Ws = synth.fp8_block_weights(N, K, 128, 128, seed=31)
    Wd, Wsd = Wq.to(DEV), Ws.to(DEV)
    need = m._bmm_ws(M, N, K, 128, 128)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    d_whole = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    d_nowait = torch.empty_like(d_whole)
    d_split = torch.empty_like(d_whole)
    _bmm_capi(aq, As, Wd, Wsd, d_whole, 128, 128, None)
    try:
        m.set_split_wait_us(0)
        _bmm_capi(aq, As, Wd, Wsd, d_nowait, 128, 128, ws)
    finally:
        m.set_split_wait_us(200)
    _bmm_capi(aq, As, Wd, Wsd, d_split, 128, 128, ws)
    sync()
    assert torch.equal(d_nowait, d_whole)
    if M <= 512:
        assert_gemm_close(d_split, oracle_path(x, Wq, Ws, 128, False, 128, 128)[2], "split after no-wait")
    else:
        diff = (d_split.float() - d_whole.float()).abs()
        assert float(diff.max()) <= float(d_whole.float().abs().max()) * 2 ** -6


def test_split_tiles_in_a_graph_replay():
    """The split launch captured in a HIP graph passes the same token on every
    replay: replays with new activations (and eager calls between them) must
    each equal an eager call on the same inputs."""
    m = q8()
    M, N, K = 640, 1536, 2048
    Wq, Ws = synth.fp8_block_weights(N, K, 128, 128, seed=41)
    Wd, Wsd = Wq.to(DEV), Ws.to(DEV)
    _, aq, As = _quantized(M, K, 128, 41)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        m.blockwise_scaled_mm(aq, Wd, As, Wsd, out=out)  # warm-up: workspace of this stream
    torch.cuda.current_stream().wait_stream(s)
    sync()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        m.blockwise_scaled_mm(aq, Wd, As, Wsd, out=out)
    for seed in (42, 43, 44):
        _, aq2, As2 = _quantized(M, K, 128, seed)
        aq.copy_(aq2)
        As.copy_(As2)
        eager = m.blockwise_scaled_mm(aq2, Wd, As2, Wsd)
        sync()
        g.replay()
        sync()
        assert torch.equal(out, eager), f"replay with seed {seed}"


def test_split_only_half_empty_last_rounds():
    """Tiles of the last round are split only when at most half the compute
    units would run them (a fuller round is left whole): the workspace query
    says which, per shape."""
    m = q8()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for M, N in ((4096, 7168), (4096, 18432), (3072, 7168), (1024, 7168), (4096, 4096), (2048, 7168)):
        tiles = -(-M // 256) * -(-N // 256)
        R = tiles % cus
        want = 0 < 2 * R <= cus
        ws = m._bmm_ws(M, N, 7168, 128, 128)
        assert (ws > 0) == want, (M, N, cus, ws)
        if want:
            assert ws >= R * 256 * 256 * 4 + R * 4


@pytest.mark.parametrize("M", [1, 64, 768])
def test_bound_calls_repeat_the_checked_call(M):
    """bind_blockwise_scaled_mm and bind_blockwise_scaled_mm_e8m0 return a
    call that repeats the checked one on the same buffers with a workspace of
    its own: one row (staged kernel), 64 rows (split K, partials in the
    workspace) and 768 rows (33 tiles split in K, flags in the workspace).
    Outputs equal the checked call's bit for bit, on each of two repeats, with
    a caller's workspace too (one short by a byte is refused), and follow new
    operand contents written into the same buffers."""
    m = q8()
    N, K = 2816, 2048
    Wq, Ws = synth.fp8_block_weights(N, K, 32, 32, seed=M)
    Wd, Wsd = Wq.to(DEV).view(torch.float8_e4m3fn), Ws.to(DEV)
    _, aq, As = _quantized(M, K, 32, seed=M)
    ref = m.blockwise_scaled_mm(aq, Wd, As, Wsd, torch.bfloat16, block=(32, 32))
    d = torch.empty_like(ref)
    call = m.bind_blockwise_scaled_mm(aq, Wd, As, Wsd, d, block=(32, 32))
    need = m.blockwise_scaled_mm_workspace_size(M, N, K, 32, 32)
    assert (need > 0) == (M > 16)
    ws = torch.empty(max(1, need), dtype=torch.uint8, device=DEV)
    d_ws = torch.empty_like(ref)
    call_ws = m.bind_blockwise_scaled_mm(aq, Wd, As, Wsd, d_ws, block=(32, 32), workspace=ws)
    call_ws()
    sync()
    assert torch.equal(d_ws, ref)
    if need:
        with pytest.raises(ValueError):
            m.bind_blockwise_scaled_mm(aq, Wd, As, Wsd, d_ws, block=(32, 32), workspace=ws[:need - 1])
    for _ in range(2):
        d.zero_()
        call()
        sync()
        assert torch.equal(d, ref)
    _, aq2, As2 = _quantized(M, K, 32, seed=M + 1)
    aq.copy_(aq2)
    As.copy_(As2)
    call()
    sync()
    assert torch.equal(d, m.blockwise_scaled_mm(aq2, Wd, As2, Wsd, torch.bfloat16, block=(32, 32)))

    W8, Ws8 = synth.fp8_block_weights_e8m0(N, K, 32, 32, seed=M)
    W8d, Ws8d = W8.to(DEV).view(torch.float8_e4m3fn), Ws8.to(DEV)
    x = synth.activations(M, K, "bf16", seed=M).to(DEV)
    aq8 = torch.empty((M, K), dtype=torch.float8_e4m3fn, device=DEV)
    as8 = torch.empty((M, K // 32), dtype=torch.uint8, device=DEV)
    m.quant_8bit(x, aq8, as8, 32, EPS, -448.0, 448.0, 2)
    ref8 = m.blockwise_scaled_mm_e8m0(aq8, W8d, as8, Ws8d, torch.bfloat16, block_n=32)
    d8 = torch.empty_like(ref8)
    call8 = m.bind_blockwise_scaled_mm_e8m0(aq8, W8d, as8, Ws8d, d8, block_n=32)
    for _ in range(2):
        d8.zero_()
        call8()
        sync()
        assert torch.equal(d8, ref8)
