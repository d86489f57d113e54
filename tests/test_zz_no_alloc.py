"""The allocation-free routing entry point (moe_mm_data_noalloc) against the
one with a caller workspace (moe_mm_data), called through the C ABI: every
table bit for bit on two calls in a row, the second smaller than the first
(the shared scratch array then holds the first call's counts), and the size
limit rejected on the host."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from oracle import moe as om
from tests.gpu_util import DEV, q8, sync

pytestmark = pytest.mark.gpu


def tables(T, topk, E):
    i32 = lambda *s: torch.full(s, -7, dtype=torch.int32, device=DEV)  # noqa: E731
    return [i32(E + 1), i32(E, 3), i32(E, 3), i32(max(T * topk, 1)), i32(max(T * topk, 1))]


def call_capi(m, fn_name, ids, E, n, k, out, workspace=None):
    T, topk = ids.shape
    stream = torch._C._cuda_getCurrentRawStream(0)
    ptrs = [t.data_ptr() for t in out]
    if fn_name == "moe_mm_data":
        ws = workspace
        st = m._moe(ids.data_ptr(), T, topk, E, n, k, *ptrs, ws.data_ptr(), ws.numel(), stream)
    else:
        st = m._moe_na(ids.data_ptr(), T, topk, E, n, k, *ptrs, stream)
    assert st == m.Q8_OK, m.last_error()


def compare(m, T, topk, E, seed):
    ids = synth.zipf_topk_ids(T, E, topk, seed=seed).to(DEV)
    ws = torch.empty(max(m._moe_ws(T, topk, E), 1), dtype=torch.uint8, device=DEV)
    ref, got = tables(T, topk, E), tables(T, topk, E)
    call_capi(m, "moe_mm_data", ids, E, 2048, 7168, ref, ws)
    call_capi(m, "moe_mm_data_noalloc", ids, E, 2048, 7168, got)
    sync()
    for r, g, name in zip(ref, got, ("offsets", "ps1", "ps2", "input_perm", "output_perm")):
        assert torch.equal(r.cpu(), g.cpu()), name
    oracle = om.moe_mm_data(ids.cpu().numpy(), E, 2048, 7168)
    for g, o in zip(got, oracle):
        assert np.array_equal(g.cpu().numpy().reshape(-1)[:o.size], o.reshape(-1))


def test_noalloc_matches_workspace_entry_point_twice():
    m = q8()
    # 4096 tokens, top-8 of 64 experts (128 chunks x 64 counts), then a smaller
    # routing on more experts: the second call reads only counts it wrote
    compare(m, 4096, 8, 64, seed=0)
    compare(m, 300, 6, 128, seed=1)


def test_noalloc_rejects_requests_beyond_its_scratch():
    m = q8()
    T, topk, E = 40000, 8, 1024      # 1250 chunks x 1024 counts > 2^20 ints
    assert m._moe_ws(T, topk, E) > (4 << 20)
    ids = torch.zeros((T, topk), dtype=torch.int32, device=DEV)
    out = tables(T, topk, E)
    st = m._moe_na(ids.data_ptr(), T, topk, E, 16, 16, *[t.data_ptr() for t in out],
                   torch._C._cuda_getCurrentRawStream(0))
    assert st == m.Q8_EUNSUPPORTED and "scratch" in m.last_error()
    sync()
    assert int(out[0][0]) == -7      # nothing was launched
