"""Pins for the oracle's E8M0 (power-of-two) block scales (CPU only).

* E8M0 decode: the byte is the biased exponent of a power of two, value
  2^(b - 127), 255 reserved for NaN — checked on all 256 bytes against the
  defining closed form and against the float32 exponent field of 2^j.
* The E8M0 block GEMM: closed forms that exercise the K-block scale index
  (activation scales 2^kb) and the N-block index (weight scales 2^(n // bn)),
  and exact rational brute force on a small random case.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import e4m3, gemm, quant

F32 = np.float32
ONE = 0x38  # e4m3 code of 1.0


def test_e8m0_decode_every_byte():
    b = np.arange(256, dtype=np.uint8)
    v = gemm.e8m0_decode(b)
    assert np.isnan(v[255])
    for i in range(255):
        assert v[i] == 2.0 ** (i - 127)
    assert v[127] == 1.0 and v[0] == 2.0 ** -127 and v[254] == 2.0 ** 127


def test_e8m0_bytes_are_the_float32_exponent_field():
    j = np.arange(-126, 128)
    s = np.ldexp(np.float32(1.0), j).astype(F32)
    b = quant.e8m0_bytes(s)
    assert np.array_equal(b, (s.view(np.uint32) >> 23).astype(np.uint8))
    assert np.array_equal(gemm.e8m0_decode(b), s.astype(np.float64))
    with pytest.raises(ValueError):
        quant.e8m0_bytes(np.array([3.0], dtype=F32))


def test_ue8m0_quant_scales_pack_losslessly():
    r = np.random.default_rng(4)
    x = (r.standard_normal((8, 256)) * np.exp2(r.integers(-20, 20, size=(8, 1)))).astype(F32)
    _, s = quant.per_token_group(x, 32, 1e-10, -448.0, 448.0, True, "e4m3")
    assert np.array_equal(gemm.e8m0_decode(quant.e8m0_bytes(s)), s.astype(np.float64))


def test_k_block_scale_index_closed_form():
    M, N, K, bn = 3, 48, 256, 16
    Aq = np.full((M, K), ONE, dtype=np.uint8)
    Wq = np.full((N, K), ONE, dtype=np.uint8)
    KB = K // 32
    As = np.tile((127 + np.arange(KB)).astype(np.uint8), (M, 1))
    Ws = np.full((N // bn, KB), 127, dtype=np.uint8)
    D = gemm.blockwise_scaled_mm_e8m0(Aq, As, Wq, Ws, bn)
    assert np.all(D == 32.0 * (2.0 ** KB - 1))


def test_n_block_scale_index_closed_form():
    M, N, K, bn = 2, 100, 128, 32  # ragged N: 4 weight-scale rows
    Aq = np.full((M, K), ONE, dtype=np.uint8)
    Wq = np.full((N, K), ONE, dtype=np.uint8)
    As = np.full((M, K // 32), 127, dtype=np.uint8)
    Ws = np.tile((120 + np.arange(4)).astype(np.uint8)[:, None], (1, K // 32))
    D = gemm.blockwise_scaled_mm_e8m0(Aq, As, Wq, Ws, bn)
    want = K * np.ldexp(1.0, 120 - 127 + np.arange(N) // bn)
    assert np.all(D == want[None, :])


def test_brute_force_fraction():
    r = np.random.default_rng(12)
    M, N, K, bn = 3, 5, 64, 2
    Aq = r.integers(0, 256, size=(M, K)).astype(np.uint8)
    Wq = r.integers(0, 256, size=(N, K)).astype(np.uint8)
    Aq[(Aq & 0x7F) == 0x7F] = 0x10  # no NaN codes
    Wq[(Wq & 0x7F) == 0x7F] = 0x11
    As = r.integers(118, 136, size=(M, K // 32)).astype(np.uint8)
    Ws = r.integers(118, 136, size=(-(-N // bn), K // 32)).astype(np.uint8)
    D = gemm.blockwise_scaled_mm_e8m0(Aq, As, Wq, Ws, bn)
    dec = {c: Fraction(float(e4m3.DECODE[c])) for c in range(256) if (c & 0x7F) != 0x7F}
    for m in range(M):
        for n in range(N):
            tot = Fraction(0)
            for kb in range(K // 32):
                p = sum(dec[Aq[m, k]] * dec[Wq[n, k]] for k in range(32 * kb, 32 * kb + 32))
                tot += p * Fraction(2) ** (int(As[m, kb]) - 127) * Fraction(2) ** (int(Ws[n // bn, kb]) - 127)
            assert D[m, n] == float(tot)  # every partial sum is exact in float64
