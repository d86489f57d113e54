"""Pins for the oracle's block-scaled FP8 GEMM and INT8 W8A8 (CPU only).

* exact rational brute force (``fractions.Fraction``) on tiny shapes;
* one-hot weights, which turn the GEMM into a scaled gather of A and expose
  transposed operands and wrong scale indexing;
* closed forms for the scale indexing along K and along N;
* "per-tensor = one block": constant scales reduce the block GEMM to a
  single library matmul (the vLLM CPU per-tensor kernel runs per-tensor FP8
  as one synthetic block);
* block-size independence when all scales are 1;
* INT8: Python-integer brute force and per-tensor/per-token equivalence;
* FP8 per-tensor / per-token x per-channel: exact rational brute force, and
  the special case "per-channel weight scales = blocks of one weight row"
  of the block GEMM with one K block (and with power-of-two scales, any K
  blocking).
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import e4m3, gemm

F32 = np.float32


def rand_codes(r, shape, lo=0.0, hi=300.0):
    """Random finite e4m3 codes of both signs (no NaN codes)."""
    mag = np.exp2(r.uniform(-9, np.log2(hi), size=shape)).astype(F32)
    mag[r.random(shape) < 0.05] = 0.0
    v = np.where(r.random(shape) < 0.5, -mag, mag).astype(F32)
    return e4m3.encode(v)


def rand_scales(r, shape):
    return np.exp2(r.uniform(-12, 4, size=shape)).astype(F32) * r.uniform(1, 2, size=shape).astype(F32)


def frac_gemm(Aq, As, Wq, Ws, bn, bk):
    M, K = Aq.shape
    N = Wq.shape[0]
    dec = [Fraction(float(v)) if np.isfinite(v) else None for v in e4m3.DECODE]
    out = [[Fraction(0)] * N for _ in range(M)]
    parts = {}
    for m in range(M):
        for n in range(N):
            tot = Fraction(0)
            for kb in range(K // bk):
                p = Fraction(0)
                for k in range(kb * bk, (kb + 1) * bk):
                    p += dec[Aq[m, k]] * dec[Wq[n, k]]
                parts[(m, n, kb)] = p
                tot += Fraction(float(As[m, kb])) * Fraction(float(Ws[n // bn, kb])) * p
            out[m][n] = tot
    return out, parts


@pytest.mark.parametrize("M,N,K,bn,bk", [(3, 5, 256, 128, 128), (2, 7, 96, 32, 32), (4, 40, 64, 32, 32)])
def test_exact_fraction_brute_force(M, N, K, bn, bk):
    r = np.random.default_rng(M * 100 + N)
    Aq = rand_codes(r, (M, K))
    Wq = rand_codes(r, (N, K))
    As = rand_scales(r, (M, K // bk))
    Ws = rand_scales(r, (-(-N // bn), K // bk))
    exact, parts = frac_gemm(Aq, As, Wq, Ws, bn, bk)
    P = gemm.block_partials(Aq, Wq, bk)
    D = gemm.blockwise_scaled_mm(Aq, As, Wq, Ws, bn, bk)
    for (m, n, kb), p in parts.items():
        assert Fraction(float(P[m, n, kb])) == p  # partial sums are exact
    for m in range(M):
        for n in range(N):
            ex = exact[m][n]
            assert abs(Fraction(float(D[m, n])) - ex) <= abs(ex) * Fraction(1, 2 ** 48) + Fraction(1, 2 ** 200)


def test_one_hot_weights_gather_A():
    r = np.random.default_rng(11)
    M, N, K, bk = 6, 48, 256, 32
    Aq = rand_codes(r, (M, K))
    As = rand_scales(r, (M, K // bk))
    pi = r.permutation(K)[:N]
    Wq = np.zeros((N, K), dtype=np.uint8)
    Wq[np.arange(N), pi] = 0x38  # 1.0
    Ws = np.ones((-(-N // bk), K // bk), dtype=F32)
    D = gemm.blockwise_scaled_mm(Aq, As, Wq, Ws, bk, bk)
    expect = As[:, pi // bk].astype(np.float64) * e4m3.decode(Aq[:, pi])
    assert np.array_equal(D, expect)


def test_scale_index_closed_forms():
    M, N, K, bk = 3, 96, 512, 32
    Aq = np.full((M, K), 0x38, dtype=np.uint8)
    Wq = np.full((N, K), 0x38, dtype=np.uint8)
    KB = K // bk
    As = np.tile(np.exp2(np.arange(KB, dtype=F32)), (M, 1))
    Ws = np.ones((N // bk, KB), dtype=F32)
    D = gemm.blockwise_scaled_mm(Aq, As, Wq, Ws, bk, bk)
    assert np.all(D == bk * (2.0 ** KB - 1))
    As1 = np.ones((M, KB), dtype=F32)
    Ws2 = np.tile(np.exp2(np.arange(N // bk, dtype=F32))[:, None], (1, KB))
    D2 = gemm.blockwise_scaled_mm(Aq, As1, Wq, Ws2, bk, bk)
    expect = K * np.exp2(np.arange(N) // bk)
    assert np.all(D2 == expect[None, :])


def test_ragged_n_uses_floor_block_index():
    M, N, K, bn, bk = 2, 100, 128, 32, 32
    Aq = np.full((M, K), 0x38, dtype=np.uint8)
    Wq = np.full((N, K), 0x38, dtype=np.uint8)
    Ws = np.tile(np.arange(1, 5, dtype=F32)[:, None], (1, K // bk))  # ceil(100/32) = 4 rows
    D = gemm.blockwise_scaled_mm(Aq, np.ones((M, K // bk), F32), Wq, Ws, bn, bk)
    assert np.all(D == K * (np.arange(N) // bn + 1)[None, :])


def test_per_tensor_is_one_block():
    r = np.random.default_rng(5)
    M, N, K, bk = 9, 33, 512, 128
    Aq = rand_codes(r, (M, K), hi=8.0)
    Wq = rand_codes(r, (N, K), hi=8.0)
    ref = e4m3.decode(Aq) @ e4m3.decode(Wq).T      # one library matmul, exact
    # power-of-two scales keep every step exact: equality
    sa, sw = F32(2.0 ** -7), F32(2.0 ** -11)
    D = gemm.blockwise_scaled_mm(Aq, np.full((M, K // bk), sa), Wq, np.full((1, K // bk), sw), 1 << 20, bk)
    assert np.array_equal(D, float(sa) * float(sw) * ref)
    # general scales: within float64 rounding of the per-block products
    sa, sw = F32(0.013), F32(0.00071)
    D = gemm.blockwise_scaled_mm(Aq, np.full((M, K // bk), sa), Wq, np.full((1, K // bk), sw), 1 << 20, bk)
    mag = float(sa) * float(sw) * (np.abs(e4m3.decode(Aq)) @ np.abs(e4m3.decode(Wq)).T)
    assert np.all(np.abs(D - float(sa) * float(sw) * ref) <= 1e-15 * mag)


def test_block_size_independence_with_unit_scales():
    r = np.random.default_rng(8)
    M, N, K = 4, 64, 256
    Aq = rand_codes(r, (M, K))
    Wq = rand_codes(r, (N, K))
    d32 = gemm.blockwise_scaled_mm(Aq, np.ones((M, 8), F32), Wq, np.ones((2, 8), F32), 32, 32)
    d128 = gemm.blockwise_scaled_mm(Aq, np.ones((M, 2), F32), Wq, np.ones((1, 2), F32), 128, 128)
    assert np.array_equal(d32, d128)  # both exact: integer multiples of 2^-18 below 2^53


def test_bias_added_per_column():
    M, N, K = 2, 8, 128
    Aq = np.zeros((M, K), np.uint8)
    Wq = np.zeros((N, K), np.uint8)
    b = np.arange(N, dtype=F32) - 3.5
    D = gemm.blockwise_scaled_mm(Aq, np.ones((M, 1), F32), Wq, np.ones((1, 1), F32), 128, 128, bias=b)
    assert np.array_equal(D, np.tile(b.astype(np.float64), (M, 1)))


def test_int8_brute_force_and_scales():
    r = np.random.default_rng(21)
    M, N, K = 5, 7, 48
    A = r.integers(-128, 128, size=(M, K)).astype(np.int8)
    W = r.integers(-128, 128, size=(N, K)).astype(np.int8)
    acc = gemm.int8_acc(A, W)
    for m in range(M):
        for n in range(N):
            assert acc[m, n] == sum(int(A[m, k]) * int(W[n, k]) for k in range(K))
    sa = r.uniform(0.01, 0.1, size=M).astype(F32)
    sb = r.uniform(0.01, 0.1, size=N).astype(F32)
    bias = r.standard_normal(N).astype(F32)
    D = gemm.scaled_mm_int8(A, sa, W, sb, bias)
    for m in range(M):
        for n in range(N):
            ex = Fraction(int(acc[m, n])) * Fraction(float(sa[m])) * Fraction(float(sb[n])) + Fraction(float(bias[n]))
            assert abs(Fraction(float(D[m, n])) - ex) <= abs(ex) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 60)
    # per-tensor x per-tensor == per-token x per-channel with constant scales
    d1 = gemm.scaled_mm_int8(A, np.array([0.5], F32), W, np.array([0.25], F32))
    d2 = gemm.scaled_mm_int8(A, np.full(M, 0.5, F32), W, np.full(N, 0.25, F32))
    assert np.array_equal(d1, d2)
    with pytest.raises(ValueError):
        gemm.scaled_mm_int8(A, np.ones(M + 1, F32), W, sb)


def test_int8_extreme_accumulator_fits_int32():
    K = 8192
    A = np.full((1, K), -128, np.int8)
    W = np.full((2, K), -128, np.int8)
    acc = gemm.int8_acc(A, W)
    assert np.all(acc == 128 * 128 * K)


def test_fp8_scaled_fraction_brute_force():
    r = np.random.default_rng(31)
    M, N, K = 4, 6, 160
    Aq = rand_codes(r, (M, K))
    Wq = rand_codes(r, (N, K))
    sa = rand_scales(r, (M,))
    sb = rand_scales(r, (N,))
    bias = r.standard_normal(N).astype(F32)
    D = gemm.scaled_mm_fp8(Aq, sa, Wq, sb, bias)
    dec = [Fraction(float(v)) if np.isfinite(v) else None for v in e4m3.DECODE]
    for m in range(M):
        for n in range(N):
            acc = sum(dec[Aq[m, k]] * dec[Wq[n, k]] for k in range(K))
            ex = acc * Fraction(float(sa[m])) * Fraction(float(sb[n])) + Fraction(float(bias[n]))
            assert abs(Fraction(float(D[m, n])) - ex) <= abs(ex) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 60)


def test_fp8_scaled_is_block_gemm_with_row_blocks():
    """Per-channel weight scales are weight blocks of one row (bn = 1) and
    per-token activation scales are one value per row for every K block:
    with a single K block the block GEMM computes the same float64 numbers;
    with power-of-two scales every step is exact, so any K blocking agrees."""
    r = np.random.default_rng(32)
    M, N, K = 7, 24, 384
    Aq = rand_codes(r, (M, K))
    Wq = rand_codes(r, (N, K))
    sa = rand_scales(r, (M,))
    sb = rand_scales(r, (N,))
    D = gemm.scaled_mm_fp8(Aq, sa, Wq, sb)
    Db = gemm.blockwise_scaled_mm(Aq, sa[:, None], Wq, sb[:, None], 1, K)
    assert np.allclose(D, Db, rtol=1e-14, atol=0)
    sa2 = np.exp2(r.integers(-8, 4, size=M)).astype(F32)
    sb2 = np.exp2(r.integers(-8, 4, size=N)).astype(F32)
    D2 = gemm.scaled_mm_fp8(Aq, sa2, Wq, sb2)
    Db2 = gemm.blockwise_scaled_mm(Aq, np.tile(sa2[:, None], (1, 3)), Wq, np.tile(sb2[:, None], (1, 3)), 1, 128)
    assert np.array_equal(D2, Db2)
    # per-tensor x per-tensor == per-token x per-channel with constant scales
    d1 = gemm.scaled_mm_fp8(Aq, np.array([0.5], F32), Wq, np.array([0.25], F32))
    d2 = gemm.scaled_mm_fp8(Aq, np.full(M, 0.5, F32), Wq, np.full(N, 0.25, F32))
    assert np.array_equal(d1, d2)
    with pytest.raises(ValueError):
        gemm.scaled_mm_fp8(Aq, np.ones(M + 1, F32), Wq, sb)
