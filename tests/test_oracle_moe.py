"""Pins for the oracle's MoE routing tables and grouped GEMM (CPU only).

Routing is checked against a pure-Python counting-sort written from the
definition and against invariants that hold for any correct table; the
grouped GEMM against the dense block GEMM row by row and in the one-expert
special case.
"""
import numpy as np
import pytest

from oracle import e4m3, gemm, moe
from synth import zipf_topk_ids

F32 = np.float32


def python_routing(ids, E):
    T, topk = len(ids), len(ids[0])
    buckets = [[] for _ in range(E)]
    for t in range(T):
        for j in range(topk):
            buckets[ids[t][j]].append(t * topk + j)
    offsets = [0]
    for e in range(E):
        offsets.append(offsets[-1] + len(buckets[e]))
    inp, outp = [], [0] * (T * topk)
    p = 0
    for e in range(E):
        for i in buckets[e]:
            inp.append(i // topk)
            outp[i] = p
            p += 1
    return offsets, inp, outp


@pytest.mark.parametrize("T,E,topk,seed", [(1, 4, 1, 0), (7, 5, 3, 1), (33, 16, 4, 2), (64, 8, 8, 3)])
def test_routing_matches_python_counting_sort(T, E, topk, seed):
    ids = zipf_topk_ids(T, E, topk, seed=seed).numpy()
    off, ps1, ps2, inp, outp = moe.moe_mm_data(ids, E, 2048, 7168)
    po, pi, pout = python_routing(ids.tolist(), E)
    assert off.tolist() == po and inp.tolist() == pi and outp.tolist() == pout
    cnt = np.diff(off)
    assert ps1.tolist() == [[int(c), 2048, 7168] for c in cnt]
    assert ps2.tolist() == [[int(c), 7168, 2048] for c in cnt]


def test_routing_invariants_with_duplicates_and_empty_experts():
    r = np.random.default_rng(9)
    T, topk, E = 200, 6, 40
    ids = r.integers(0, 10, size=(T, topk)).astype(np.int32)  # experts 10..39 empty; duplicates allowed
    off, ps1, _, inp, outp = moe.moe_mm_data(ids, E, 16, 32)
    n = T * topk
    assert off[0] == 0 and off[-1] == n and np.all(np.diff(off) >= 0)
    assert np.all(off[11:] == n)
    assert np.array_equal(np.sort(outp), np.arange(n))
    flat = ids.reshape(-1)
    assert np.array_equal(inp[outp], np.arange(n) // topk)
    for e in range(E):
        seg = np.flatnonzero(flat == e)
        assert np.array_equal(outp[seg], np.arange(off[e], off[e + 1]))  # ascending flat order
    assert np.array_equal(ps1[:, 0], np.diff(off))


def test_routing_rejects_bad_ids():
    with pytest.raises(ValueError):
        moe.moe_mm_data(np.array([[0, 4]], np.int32), 4, 8, 8)


def test_zipf_generator_shape_and_distinct():
    ids = zipf_topk_ids(4096, 64, 8, seed=0).numpy()
    assert ids.shape == (4096, 8) and ids.dtype == np.int32
    assert all(len(set(row)) == 8 for row in ids[:200])
    cnt = np.bincount(ids.reshape(-1), minlength=64)
    assert cnt[0] > cnt[-1] * 10  # skewed toward low ids


def _rand_codes(r, shape, hi=64.0):
    mag = np.exp2(r.uniform(-6, np.log2(hi), size=shape)).astype(F32)
    return e4m3.encode(np.where(r.random(shape) < 0.5, -mag, mag).astype(F32))


def test_grouped_equals_dense_per_choice():
    r = np.random.default_rng(4)
    T, topk, E, N, K, bk = 12, 3, 5, 64, 256, 128
    ids = zipf_topk_ids(T, E, topk, seed=4).numpy()
    Aq = _rand_codes(r, (T, K))
    As = np.exp2(r.uniform(-8, 0, size=(T, K // bk))).astype(F32)
    W = _rand_codes(r, (E, N, K))
    Ws = np.exp2(r.uniform(-10, -4, size=(E, N // bk + 1, K // bk))).astype(F32)
    off, _, _, inp, outp = moe.moe_mm_data(ids, E, N, K)
    Ds = moe.grouped_blockwise_scaled_mm(Aq, As, W, Ws, off, inp, bk, bk)
    out = moe.unpermute(Ds, outp)
    for t in range(T):
        for j in range(topk):
            e = ids[t, j]
            dense = gemm.blockwise_scaled_mm(Aq[t:t + 1], As[t:t + 1], W[e], Ws[e], bk, bk)
            assert np.array_equal(out[t * topk + j], dense[0])


def test_grouped_single_expert_is_one_gemm():
    r = np.random.default_rng(6)
    T, topk, E, N, K, bk = 10, 1, 3, 32, 128, 32
    ids = np.zeros((T, topk), np.int32)
    Aq = _rand_codes(r, (T, K))
    As = np.ones((T, K // bk), F32) * F32(0.5)
    W = _rand_codes(r, (E, N, K))
    Ws = np.ones((E, N // bk, K // bk), F32)
    off, _, _, inp, outp = moe.moe_mm_data(ids, E, N, K)
    out = moe.unpermute(moe.grouped_blockwise_scaled_mm(Aq, As, W, Ws, off, inp, bk, bk), outp)
    assert np.array_equal(out, gemm.blockwise_scaled_mm(Aq, As, W[0], Ws[0], bk, bk))


def test_finalize_brute_force_and_permutation_fusion():
    """Python-loop brute force, and the fused form (expert-sorted rows named
    by output_permutation) equals un-permuting first."""
    from oracle import moe
    r = np.random.default_rng(41)
    T, topk, E, N = 9, 3, 5, 7
    ids = np.stack([r.choice(E, size=topk, replace=False) for _ in range(T)]).astype(np.int32)
    off, ps1, ps2, ip, op = moe.moe_mm_data(ids, E, N, 4)
    D_sorted = r.standard_normal((T * topk, N))
    w = r.uniform(0.0, 1.0, size=(T, topk))
    fused = moe.finalize(D_sorted, w, topk, op)
    D_unperm = moe.unpermute(D_sorted, op)
    plain = moe.finalize(D_unperm, w, topk)
    assert np.array_equal(fused, plain)
    for t in range(T):
        for n in range(N):
            ref = 0.0
            for j in range(topk):
                ref += w[t, j] * D_unperm[t * topk + j, n]
            assert abs(plain[t, n] - ref) <= 1e-12 * (1 + abs(ref))


def test_finalize_special_cases():
    from oracle import moe
    r = np.random.default_rng(42)
    D = r.standard_normal((8, 5))
    # top-1 with weight 1 is the identity; no weights sums the top-k rows
    assert np.array_equal(moe.finalize(D, np.ones((8, 1)), 1), D)
    assert np.array_equal(moe.finalize(D, None, 2), D[0::2] + D[1::2])
    # one-hot weights pick a row exactly
    w = np.zeros((4, 2)); w[:, 1] = 1.0
    assert np.array_equal(moe.finalize(D, w, 2), D[1::2])
    with pytest.raises(ValueError):
        moe.finalize(D[:7], None, 2)
