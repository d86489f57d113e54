"""GPU parity: MoE routing tables (bit-exact), row gather, and the expert-grouped
block-FP8 GEMM with fused gather/un-permute against the oracle."""
import numpy as np
import pytest
import torch

import synth
from oracle import moe as om
from oracle import quant as oq
from tests.gpu_util import DEV, assert_gemm_close, codes, q8, sync

pytestmark = pytest.mark.gpu

EPS = 1e-10


def gpu_routing(ids_dev, E, n, k):
    m = q8()
    T, topk = ids_dev.shape
    off = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    ps1 = torch.empty((E, 3), dtype=torch.int32, device=DEV)
    ps2 = torch.empty((E, 3), dtype=torch.int32, device=DEV)
    ip = torch.empty(T * topk, dtype=torch.int32, device=DEV)
    op = torch.empty(T * topk, dtype=torch.int32, device=DEV)
    m.moe_mm_data(ids_dev, off, ps1, ps2, ip, op, E, n, k)
    sync()
    return off, ps1, ps2, ip, op


@pytest.mark.parametrize("T,E,topk,seed", [(4096, 64, 8, 0), (1, 4, 1, 1), (7, 5, 3, 2),
                                           (1000, 256, 8, 3), (3, 1024, 2, 4),
                                           # chunk counts over several LDS slabs of the scan
                                           (16384, 256, 8, 6), (20000, 1024, 8, 7), (5000, 3, 2, 8)])
def test_routing_bit_exact(T, E, topk, seed):
    ids = synth.zipf_topk_ids(T, E, topk, seed=seed)
    got = [t.cpu().numpy() for t in gpu_routing(ids.to(DEV), E, 2048, 7168)]
    ref = om.moe_mm_data(ids.numpy(), E, 2048, 7168)
    for g, r, name in zip(got, ref, ("offsets", "ps1", "ps2", "input_perm", "output_perm")):
        assert np.array_equal(g.reshape(r.shape), r), name


def test_routing_duplicates_empty_experts_and_zero_tokens():
    r = np.random.default_rng(5)
    ids = torch.from_numpy(r.integers(0, 10, size=(600, 6)).astype(np.int32))
    got = [t.cpu().numpy() for t in gpu_routing(ids.to(DEV), 40, 16, 32)]
    ref = om.moe_mm_data(ids.numpy(), 40, 16, 32)
    for g, rr in zip(got, ref):
        assert np.array_equal(g.reshape(rr.shape), rr)
    empty = torch.empty((0, 8), dtype=torch.int32, device=DEV)
    off, ps1, _, _, _ = gpu_routing(empty, 8, 16, 32)
    assert off.cpu().numpy().tolist() == [0] * 9 and ps1[:, 0].cpu().numpy().tolist() == [0] * 8


def test_routing_run_twice_identical():
    ids = synth.zipf_topk_ids(4096, 64, 8, seed=0).to(DEV)
    a = [t.cpu() for t in gpu_routing(ids, 64, 2048, 7168)]
    b = [t.cpu() for t in gpu_routing(ids, 64, 2048, 7168)]
    assert all(torch.equal(x, y) for x, y in zip(a, b))


def test_shuffle_rows():
    m = q8()
    r = np.random.default_rng(0)
    src = torch.from_numpy(r.integers(0, 255, size=(50, 7168), dtype=np.uint8))
    mp = torch.from_numpy(r.integers(0, 50, size=200).astype(np.int32))
    out = m.shuffle_rows(src.to(DEV), mp.to(DEV), (200, 7168))
    assert torch.equal(out.cpu(), src[mp.long()])
    odd = torch.from_numpy(r.integers(0, 255, size=(9, 13), dtype=np.uint8))
    out2 = m.shuffle_rows(odd.to(DEV), mp[:5].remainder(9).to(DEV), (5, 13))
    assert torch.equal(out2.cpu(), odd[mp[:5].remainder(9).long()])


def run_moe(T, E, topk, N, K, rows=None, seed=0, fused=True):
    """Whole MoE path on both sides: routing, activation quant, grouped GEMM,
    un-permute. Returns nothing; asserts parity."""
    m = q8()
    bk = bn = 128
    ids = synth.zipf_topk_ids(T, E, topk, seed=seed)
    x = synth.activations(T, K, "bf16", seed=seed)
    W, Ws = synth.fp8_block_weights(N, K, bn, bk, experts=E, seed=seed)
    # GPU
    off, ps1, _, ip, op = gpu_routing(ids.to(DEV), E, N, K)
    aq = torch.empty((T, K), dtype=torch.float8_e4m3fn, device=DEV)
    As = torch.empty((T, K // bk), dtype=torch.float32, device=DEV)
    m.quant_8bit(x.to(DEV), aq, As, bk, EPS, -448.0, 448.0, False)
    Wd, Wsd = W.to(DEV), Ws.to(DEV)
    if fused:
        d = torch.empty((T * topk, N), dtype=torch.bfloat16, device=DEV)
        m.grouped_blockwise_scaled_mm(d, aq, Wd, As, Wsd, off, ps1, a_map=ip, c_map=op)
    else:
        a_sorted = m.shuffle_rows(aq.view(torch.uint8), ip, (T * topk, K)).view(torch.float8_e4m3fn)
        as_sorted = m.shuffle_rows(As, ip, (T * topk, K // bk))
        d_sorted = torch.empty((T * topk, N), dtype=torch.bfloat16, device=DEV)
        m.grouped_blockwise_scaled_mm(d_sorted, a_sorted, Wd, as_sorted, Wsd, off, ps1)
        # un-permute: out[i] = d_sorted[output_permutation[i]]
        d = m.shuffle_rows(d_sorted, op, (T * topk, N))
    sync()
    # oracle
    aq_o, as_o = oq.per_token_group(x.float().numpy(), bk, EPS, -448.0, 448.0, False, "e4m3")
    assert np.array_equal(codes(aq), aq_o)
    off_o, _, _, ip_o, op_o = om.moe_mm_data(ids.numpy(), E, N, K)
    if rows is None:
        ref = om.unpermute(om.grouped_blockwise_scaled_mm(aq_o, as_o, W.numpy(), Ws.numpy(), off_o,
                                                          ip_o, bn, bk), op_o)
        assert_gemm_close(d, ref, "moe")
    else:
        # sampled flat choices i = t*topk + j: dense oracle of token t with expert ids[t, j]
        from oracle import gemm as og
        idsn = ids.numpy()
        dc = d.cpu()
        got, ref = [], []
        for i in rows:
            t, j = divmod(int(i), topk)
            e = idsn[t, j]
            ref.append(og.blockwise_scaled_mm(aq_o[t:t + 1], as_o[t:t + 1], W[e].numpy(), Ws[e].numpy(), bn, bk)[0])
            got.append(dc[i])
        assert_gemm_close(torch.stack(got), np.stack(ref), "moe sampled")


@pytest.mark.parametrize("fused", [True, False])
def test_moe_small_full_compare(fused):
    run_moe(64, 8, 4, 384, 512, seed=1, fused=fused)


def test_moe_many_tiny_experts():
    run_moe(40, 33, 3, 256, 256, seed=2)


def test_moe_full_size_every_row():
    """4096 tokens, top-8 of 64 Zipf-skewed experts, N = 2048, K = 7168 with
    the fused gather and un-permute, as the benchmark launches it: all 32768
    routed rows compared with the oracle."""
    run_moe(4096, 64, 8, 2048, 7168, seed=0)


def test_grouped_single_expert_equals_dense():
    m = q8()
    T, N, K, bk = 300, 512, 1024, 128
    x = synth.activations(T, K, "bf16", seed=3).to(DEV)
    W, Ws = synth.fp8_block_weights(N, K, bk, bk, experts=3, seed=3)
    aq = torch.empty((T, K), dtype=torch.float8_e4m3fn, device=DEV)
    As = torch.empty((T, K // bk), dtype=torch.float32, device=DEV)
    m.quant_8bit(x, aq, As, bk, EPS, -448.0, 448.0, False)
    off = torch.tensor([0, T, T, T], dtype=torch.int32, device=DEV)
    ps = torch.tensor([[T, N, K], [0, N, K], [0, N, K]], dtype=torch.int32, device=DEV)
    d = torch.empty((T, N), dtype=torch.bfloat16, device=DEV)
    m.grouped_blockwise_scaled_mm(d, aq, W.to(DEV), As, Ws.to(DEV), off, ps)
    # the dense call would split its tiles in K (a half-empty last round);
    # without the wait every tile comes out whole, as the grouped kernel's do
    try:
        m.set_split_wait_us(0)
        dense = m.blockwise_scaled_mm(aq, W[0].to(DEV), As, Ws[0].to(DEV))
    finally:
        m.set_split_wait_us(200)
    sync()
    assert torch.equal(d, dense)


def finalize_bound(w, D_rows, ref):
    """|out - ref| <= 2^-8 |ref| (the 16-bit output rounding) + 2^-20 sum|w d|
    (float32 accumulation over the top-k terms)."""
    mag = np.einsum("tj,tjn->tn", np.abs(w), np.abs(D_rows))
    return 2.0 ** -8 * np.abs(ref) + 2.0 ** -20 * mag


@pytest.mark.parametrize("T,topk,N,dtype,perm,weights", [
    (4096, 8, 2048, "bf16", True, True), (4096, 8, 2048, "bf16", False, True),
    (37, 3, 100, "f16", True, True), (5, 2, 24, "bf16", False, False), (70000, 1, 16, "bf16", True, True),
    # more than one batch of eight rows per token, full and partial
    (50, 10, 264, "bf16", True, True), (33, 16, 2048, "bf16", True, True), (21, 9, 100, "f16", False, True)])
def test_finalize_parity(T, topk, N, dtype, perm, weights):
    """Synthetic routed rows and gate weights on both sides; with ``perm`` the
    rows are in expert-sorted order and the routing table names them."""
    m = q8()
    D = synth.activations(T * topk, N, dtype, seed=T + N)
    w = synth.topk_weights(T, topk, seed=T) if weights else None
    op = None
    if perm:
        ids = synth.zipf_topk_ids(T, max(topk, 16), topk, seed=T)
        op = om.moe_mm_data(ids.numpy(), max(topk, 16), N, N)[4]
    out = m.moe_finalize(D.to(DEV), None if w is None else w.to(DEV), topk,
                         None if op is None else torch.from_numpy(op).to(DEV))
    sync()
    Dn = D.double().numpy()
    wn = None if w is None else w.double().numpy()
    ref = om.finalize(Dn, wn, topk, op)
    rows = om.unpermute(Dn, op) if perm else Dn
    got = out.double().cpu().numpy()
    bound = finalize_bound(np.ones((T, topk)) if wn is None else wn, rows.reshape(T, topk, N), ref)
    assert np.all(np.abs(got - ref) <= bound)


def test_moe_step_with_finalize():
    """Routing, quant, grouped GEMM into expert-sorted rows (no scatter), then
    the finalize with the output permutation, against the oracle path."""
    m = q8()
    T, E, topk, N, K, bk = 96, 8, 4, 256, 512, 128
    ids = synth.zipf_topk_ids(T, E, topk, seed=7)
    x = synth.activations(T, K, "bf16", seed=7)
    W, Ws = synth.fp8_block_weights(N, K, bk, bk, experts=E, seed=7)
    w = synth.topk_weights(T, topk, seed=7)
    off, ps1, _, ip, op = gpu_routing(ids.to(DEV), E, N, K)
    aq = torch.empty((T, K), dtype=torch.float8_e4m3fn, device=DEV)
    As = torch.empty((T, K // bk), dtype=torch.float32, device=DEV)
    m.quant_8bit(x.to(DEV), aq, As, bk, EPS, -448.0, 448.0, False)
    d_sorted = torch.empty((T * topk, N), dtype=torch.bfloat16, device=DEV)
    m.grouped_blockwise_scaled_mm(d_sorted, aq, W.to(DEV), As, Ws.to(DEV), off, ps1, a_map=ip)
    out = m.moe_finalize(d_sorted, w.to(DEV), topk, op)
    sync()
    aq_o, as_o = oq.per_token_group(x.float().numpy(), bk, EPS, -448.0, 448.0, False, "e4m3")
    off_o, _, _, ip_o, op_o = om.moe_mm_data(ids.numpy(), E, N, K)
    d_ref = om.grouped_blockwise_scaled_mm(aq_o, as_o, W.numpy(), Ws.numpy(), off_o, ip_o, bk, bk)
    wn = w.double().numpy()
    ref = om.finalize(d_ref, wn, topk, op_o)
    # each routed row carries the GEMM tolerance and its rounding to bf16
    # (relative 2^-9); the sum adds float32 accumulation and the final bf16
    # rounding (relative 2^-9, 2^-8 with margin)
    rows = om.unpermute(d_ref, op_o).reshape(T, topk, N)
    rms = float(np.sqrt(np.mean(d_ref * d_ref)))
    per_row = 1e-2 * np.abs(rows) + 1e-3 * rms + 2.0 ** -9 * np.abs(rows)
    bound = np.einsum("tj,tjn->tn", np.abs(wn), per_row) + 2.0 ** -8 * np.abs(ref)
    got = out.double().cpu().numpy()
    assert np.all(np.abs(got - ref) <= bound), float(np.max(np.abs(got - ref) / bound))
