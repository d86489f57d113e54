"""Pins for the oracle's fused SiLU-and-mul quantization and masked rows (CPU).

* The float32 exponential is checked to be the correctly rounded one on every
  finite bf16 input, against Python's ``decimal`` module (whose exp is
  correctly rounded at the working precision), and at the overflow and
  underflow ends against the float32 range limits.
* SiLU-and-mul is checked against exact decimal arithmetic
  ``g * u / (1 + exp(-g))``: four float32 roundings bound the relative error
  by about 4 * 2^-24, which a dropped term, a wrong sign or swapped halves
  break by orders of magnitude; its limits (g = 0, large positive and
  negative g) are closed forms.
* Masked rows follow their definition on small hand-made cases.
"""
from decimal import Decimal, getcontext

import numpy as np
import pytest

from oracle import e4m3, quant

F32 = np.float32
EPS = 1e-10


def _all_bf16():
    bits = (np.arange(65536, dtype=np.uint32) << 16).view(F32)
    return bits[np.isfinite(bits)]


def _rn32(d: Decimal) -> np.float32:
    """Nearest float32 to a positive decimal (no ties occur for exp(x), x != 0)."""
    c = F32(float(d))
    best, best_err = None, None
    for f in (np.nextafter(c, F32(0)), c, np.nextafter(c, F32(np.inf))):
        if not np.isfinite(f):
            continue
        err = abs(Decimal(float(f)) - d)
        if best is None or err < best_err:
            best, best_err = f, err
    return best


def test_exp_rn32_is_correctly_rounded_on_every_bf16():
    getcontext().prec = 50
    v = _all_bf16()
    inner = v[(v >= -110.0) & (v <= 88.5)]
    got = quant.exp_rn32(inner)
    want = np.array([_rn32(Decimal(float(x)).exp()) for x in inner], dtype=F32)
    bad = got.view(np.uint32) != want.view(np.uint32)
    assert not bad.any(), (inner[bad][:5], got[bad][:5], want[bad][:5])
    # ends of the range: ln(FLT_MAX + half an ulp) = 88.7228..., so every bf16
    # from 89 up overflows to +inf; exp(-104) < 2^-150 (half the smallest
    # subnormal) rounds to +0
    hi = v[v >= 89.0]
    lo = v[v <= -104.0]
    assert np.all(np.isposinf(quant.exp_rn32(hi)))
    assert np.all(quant.exp_rn32(lo).view(np.uint32) == 0)
    assert quant.exp_rn32(F32(0.0)) == 1.0 and quant.exp_rn32(F32(-0.0)) == 1.0


def test_exp_rn32_random_float32():
    getcontext().prec = 50
    r = np.random.default_rng(11)
    x = r.uniform(-100.0, 88.0, size=3000).astype(F32)
    got = quant.exp_rn32(x)
    want = np.array([_rn32(Decimal(float(t)).exp()) for t in x], dtype=F32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def _bf16(a):
    a = np.asarray(a, dtype=F32)
    b = a.view(np.uint32)
    b = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return b.view(F32)


def test_silu_and_mul_against_exact_decimal():
    getcontext().prec = 50
    r = np.random.default_rng(5)
    n = 4000
    g = _bf16(r.standard_normal(n).astype(F32) * F32(4.0))
    u = _bf16(r.standard_normal(n).astype(F32))
    y = quant.silu_and_mul(np.concatenate([g[:, None], u[:, None]], axis=1))[:, 0]
    for gi, ui, yi in zip(g, u, y):
        gd, ud = Decimal(float(gi)), Decimal(float(ui))
        exact = gd * ud / (1 + (-gd).exp())
        if exact == 0:
            assert yi == 0.0
            continue
        rel = abs((Decimal(float(yi)) - exact) / exact)
        assert rel <= Decimal(4.01) * Decimal(2) ** -24, (gi, ui, yi, exact)


def test_silu_and_mul_limits_and_orientation():
    # first half is the gate, second half the multiplier
    x = np.array([[30.0, 1.0, 1.0, 30.0]], dtype=F32)
    y = quant.silu_and_mul(x)
    assert y[0, 0] == F32(30.0)                       # e = exp(-30) < 2^-25: d = 1
    assert y[0, 1] == F32(F32(F32(1.0) / F32(1.0 + np.exp(-1.0))) * F32(30.0))
    assert abs(float(y[0, 1]) - 30.0 / (1.0 + np.exp(-1.0))) < 1e-5
    # g = 0 -> 0 (sign of 0 * u); large negative g -> exp overflows, y = -0 * u
    x = np.array([[0.0, -200.0, -0.0, 3.0, 2.0, -1.5]], dtype=F32)
    y = quant.silu_and_mul(x)
    assert y[0, 0] == 0.0 and not np.signbit(y[0, 0])   # (0 / 2) * 3
    assert y[0, 1] == 0.0 and np.signbit(y[0, 1])       # (-200 / inf) * 2 = -0
    assert y[0, 2] == 0.0 and not np.signbit(y[0, 2])   # (-0 / 2) * -1.5 = +0
    # large positive gate: y = fl32(g * u)
    g = np.array([17.5, 100.0, 3e38], dtype=F32)
    u = np.array([1.25, -3.0, 0.5], dtype=F32)
    y = quant.silu_and_mul(np.concatenate([g, u])[None, :])[0]
    assert np.array_equal(y, (g * u).astype(F32))


def test_fused_quant_is_quant_of_silu_output():
    r = np.random.default_rng(9)
    x = _bf16(r.standard_normal((6, 512)).astype(F32) * F32(2.0))
    q, s, valid = quant.per_token_group_fused(x, 64, EPS, -448.0, 448.0, False, "e4m3", silu=True)
    assert valid.all() and q.shape == (6, 256) and s.shape == (6, 4)
    y = quant.silu_and_mul(x)
    q2, s2 = quant.per_token_group(y, 64, EPS, -448.0, 448.0, False, "e4m3")
    assert np.array_equal(q, q2) and np.array_equal(s, s2)
    # the dequantized codes sit within half an e4m3 step of silu(g) * u
    deq = e4m3.decode(q) * np.repeat(s, 64, axis=1)
    assert np.all(np.abs(deq - y) <= np.abs(y) / 16 + np.repeat(s, 64, axis=1) * 2.0 ** -10)


def test_masked_rows_definition():
    v = quant.masked_rows(12, [0, 3, 4], 4)
    assert v.tolist() == [False] * 4 + [True] * 3 + [False] + [True] * 4
    with pytest.raises(ValueError):
        quant.masked_rows(10, [1, 2], 4)


def test_masked_quant_valid_rows_match_unmasked():
    r = np.random.default_rng(13)
    x = r.standard_normal((3 * 5, 256)).astype(F32)
    q, s, valid = quant.per_token_group_fused(x, 128, EPS, -128.0, 127.0, False, "i8",
                                              masked_m=[2, 0, 5], max_m=5)
    assert valid.tolist() == [True, True, False, False, False] + [False] * 5 + [True] * 5
    q2, s2 = quant.per_token_group(x, 128, EPS, -128.0, 127.0, False, "i8")
    assert np.array_equal(q[valid], q2[valid]) and np.array_equal(s[valid], s2[valid])
    assert np.all(q[~valid] == 0) and np.all(s[~valid] == 0)
