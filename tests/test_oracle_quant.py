"""Pins for the oracle's 8-bit activation quantization (CPU only).

Closed forms fixed by the definition (scale = max(amax, eps) / qmax, UE8M0
rounds up to a power of two, codes by nearest rounding), a cast sweep that
reduces the quantizer to torch's e4m3 cast (a library routine), the e4m3
half-step error bound, and structural invariants (per-token = one group per
row, per-tensor = one group for the whole tensor).
"""
import numpy as np
import pytest
import torch

from oracle import e4m3, quant

F32 = np.float32
EPS = 1e-10


def q8(x, g, ue=False, qd="e4m3"):
    if qd == "e4m3":
        return quant.per_token_group(x, g, EPS, -448.0, 448.0, ue, "e4m3")
    return quant.per_token_group(x, g, EPS, -128.0, 127.0, ue, "i8")


@pytest.mark.parametrize("c", [1.0, -3.5, 0.0123, 1e-3, 300.0, -1e4])
def test_all_equal_group(c):
    x = np.full((3, 256), F32(c), dtype=F32)
    q, s = q8(x, 128)
    assert np.all(s == F32(abs(F32(c)) / F32(448.0)))
    expect = 0x7E if c > 0 else 0xFE
    assert np.all(q == expect)


@pytest.mark.parametrize("j", [-20, -3, 0, 1, 5, 10, 17])
def test_ue8m0_power_of_two_amax(j):
    r = np.random.default_rng(j + 100)
    x = (r.uniform(-1.0, 1.0, size=(2, 64)) * 2.0 ** j * 0.9).astype(F32)
    x[0, 5] = F32(2.0 ** j)
    x[1, 40] = F32(-(2.0 ** j))
    q, s = q8(x, 32, ue=True)
    # 2^j / 448 lies in (2^(j-9), 2^(j-8)); rounded up -> 2^(j-8)
    assert s[0, 0] == F32(2.0 ** (j - 8)) and s[1, 1] == F32(2.0 ** (j - 8))
    # the amax element maps to 256 = 1.0 * 2^8 -> code 0x78 (sign bit for negative)
    assert q[0, 5] == 0x78 and q[1, 40] == 0xF8


def test_ue8m0_ceil_bits():
    s = np.array([1.0, 1.5, 0.75, 2.0 ** -30, 3.0 * 2 ** 20, 1.0000001], dtype=F32)
    out = quant.ue8m0_ceil(s)
    assert list(out) == [1.0, 2.0, 1.0, 2.0 ** -30, 2.0 ** 22, 2.0]
    r = np.random.default_rng(7)
    v = np.exp2(r.uniform(-60, 60, size=10000)).astype(F32)
    u = quant.ue8m0_ceil(v)
    # power of two, >= v, and < 2 v
    m, _ = np.frexp(u.astype(np.float64))
    assert np.all(m == 0.5) and np.all(u >= v) and np.all(u.astype(np.float64) < 2.0 * v)


def test_zero_group():
    x = np.zeros((2, 256), dtype=F32)
    x[1, 128:] = 1.0
    q, s = q8(x, 128)
    assert s[0, 0] == F32(F32(EPS) / F32(448.0)) and s[0, 1] == s[0, 0] and s[1, 0] == s[0, 0]
    assert np.all(q[0] == 0) and np.all(q[1, :128] == 0)
    assert s[1, 1] == F32(1.0 / 448.0)


def test_negative_zero_and_tiny_negatives_keep_sign():
    x = np.zeros((1, 32), dtype=F32)
    x[0, 0] = 448.0            # s = 1 exactly
    x[0, 1] = -0.0
    x[0, 2] = -(2.0 ** -11)    # rounds to -0
    q, s = q8(x, 32)
    assert s[0, 0] == 1.0
    assert q[0, 1] == 0x80 and q[0, 2] == 0x80 and q[0, 3] == 0x00


@pytest.mark.parametrize("c", [1.0, -0.37, 5e-3, 1234.5])
def test_int8_constant_row(c):
    x = np.full((2, 512), F32(c), dtype=F32)
    q, s = q8(x, 512, qd="i8")
    assert np.all(s == F32(abs(F32(c)) / F32(127.0)))
    assert np.all(q == (127 if c > 0 else -127))


def test_int8_rounds_half_to_even():
    # s = 1 exactly (amax 127), so the codes are rint of the inputs themselves
    x = np.array([[127.0, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.49, -126.5] + [0.0] * 7], dtype=F32)
    q, s = q8(x, 16, qd="i8")
    assert s[0, 0] == 1.0
    assert list(q[0, :9]) == [127, 0, 2, 2, 0, -2, -2, 3, -126]


def test_cast_sweep_reduces_to_library_cast():
    """A group holding 448 has scale exactly 1, so the codes must be torch's
    e4m3 cast of the inputs. Sweep every finite bf16 value in range."""
    bits = np.arange(65536, dtype=np.uint32) << 16
    v = bits.view(np.float32)
    v = v[np.isfinite(v) & (np.abs(v) <= 448.0)]
    g = 128
    n = -(-v.size // (g - 1))
    x = np.zeros((n, g), dtype=F32)
    flat = np.zeros(n * (g - 1), dtype=F32)
    flat[:v.size] = v
    x[:, 1:] = flat.reshape(n, g - 1)
    x[:, 0] = 448.0
    q, s = q8(x, g)
    assert np.all(s == 1.0)
    lib = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q, lib)


@pytest.mark.parametrize("g,ue", [(128, False), (32, True), (64, False)])
def test_dequant_error_within_half_step(g, ue):
    r = np.random.default_rng(g)
    x = (r.standard_normal((16, 512)) * np.exp2(r.integers(-8, 8, size=(16, 1)))).astype(F32)
    q, s = q8(x, g, ue)
    sf = np.repeat(s, g, axis=1).astype(np.float64)
    deq = e4m3.decode(q) * sf
    y = x.astype(np.float64) / sf
    # e4m3 step at |y| in [2^e, 2^(e+1)) is 2^(e-3); below 2^-6 it is 2^-9.
    e = np.floor(np.log2(np.maximum(np.abs(y), 2.0 ** -6)))
    half_step = np.exp2(e - 4) * sf
    # y itself was rounded to float32 before encoding: allow one float32 ulp of it
    assert np.all(np.abs(deq - x) <= half_step * (1 + 2 ** -20) + np.abs(x) * 2 ** -23)
    assert np.all(np.abs(y) <= 448.0 * (1 + 2 ** -23))


def test_per_token_is_one_group_per_row_and_per_tensor_is_one_group():
    r = np.random.default_rng(3)
    x = r.standard_normal((5, 384)).astype(F32)
    q, s = q8(x, 384)
    for m in range(5):
        qt, st = quant.per_tensor_dynamic(x[m:m + 1], EPS, -448.0, 448.0)
        assert np.array_equal(q[m:m + 1], qt) and s[m, 0] == st[0]
    qg, sg = q8(x, 128)
    for m in range(5):
        for j in range(3):
            blk = x[m:m + 1, j * 128:(j + 1) * 128]
            qt, st = quant.per_tensor_dynamic(blk, EPS, -448.0, 448.0)
            assert np.array_equal(qg[m:m + 1, j * 128:(j + 1) * 128], qt) and sg[m, j] == st[0]


def test_static_scale():
    x = np.array([[1.0, -2.0, 1000.0, -1000.0]], dtype=F32)
    q = quant.static(x, 0.5, -448.0, 448.0)
    assert list(q[0]) == [int(e4m3.encode(F32(2.0))), int(e4m3.encode(F32(-4.0))), 0x7E, 0xFE]
    qi = quant.static(x, 0.5, -128.0, 127.0, "i8")
    assert list(qi[0]) == [2, -4, 127, -128]


def test_rejects_ragged_group():
    with pytest.raises(ValueError):
        q8(np.zeros((1, 100), dtype=F32), 32)


# ---- per-tensor dynamic scale over several rows -------------------------------
# The expected codes below are written out by hand from the e4m3fn layout
# (value (-1)^s (1 + m/8) 2^(e-7), code = s<<7 | e<<3 | m) and from rint with
# ties to even: they do not come from the oracle. In every case the global
# |max| sits in a later row than rows whose own maximum is smaller, so a scale
# taken per row instead of over the whole tensor changes the codes of the
# earlier rows and fails the pin.

def test_per_tensor_dynamic_takes_the_max_over_all_rows():
    x = np.array([[1.0, 2.0, 4.0, -8.0],
                  [0.5, -16.0, 64.0, 3.0],
                  [1792.0, -0.25, 6.0, 0.0]], dtype=F32)
    q, s = quant.per_tensor_dynamic(x, EPS, -448.0, 448.0)
    # |max| = 1792 = 448 * 4 in the last row: s = 4 exactly, codes of x / 4
    assert s.shape == (1,) and s[0] == 4.0
    # x/4:   0.25  0.5   1     -2   | 0.125  -4    16    0.75 | 448   -0.0625 1.5  0
    expect = [[0x28, 0x30, 0x38, 0xC0], [0x20, 0xC8, 0x58, 0x34], [0x7E, 0x98, 0x3C, 0x00]]
    assert q.tolist() == expect
    # a per-row scale would have mapped row 0's maximum (8) to 448
    assert q[0, 3] != 0xFE


def test_per_tensor_dynamic_ue8m0_across_rows():
    x = np.array([[100.0, -3.0, 2.0, 0.5],
                  [1000.0, 12.0, -40.0, 1.0]], dtype=F32)
    q, s = quant.per_tensor_dynamic(x, EPS, -448.0, 448.0, True)
    # 1000 / 448 = 2.23.. rounds up to the power of two 4
    assert s[0] == 4.0
    # x/4: 25 (1.5625*16: mantissa 4.5 ties to even 4 -> 24), -0.75, 0.5, 0.125 |
    #      250 (1.953*128 rounds up to 256 = 2^8: e=15, m=0), 3, -10, 0.25
    expect = [[0x5C, 0xB4, 0x30, 0x20], [0x78, 0x44, 0xD2, 0x28]]
    assert q.tolist() == expect


def test_per_tensor_dynamic_int8_across_rows_and_ties():
    x = np.array([[1.0, 3.0, 5.0, -7.0],
                  [-1.0, -3.0, 9.0, 0.0],
                  [254.0, 2.5, -5.0, 100.0]], dtype=F32)
    q, s = quant.per_tensor_dynamic(x, EPS, -128.0, 127.0, False, "i8")
    # |max| 254 in the last row: s = 254 / 127 = 2; x/2 = k + 0.5 rounds to even
    assert s[0] == 2.0
    assert q.tolist() == [[0, 2, 2, -4], [0, -2, 4, 0], [127, 1, -2, 50]]
    # per row, row 0 would have had s = 7/127 and codes up to -127
    assert q[0, 3] != -127
