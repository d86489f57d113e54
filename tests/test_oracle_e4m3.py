"""Pins for the oracle's e4m3fn codec (CPU only).

The codec is pinned to (a) the format's own definition at hand-derived
anchor points, (b) exhaustive round trips over every finite code and (c)
torch's CPU ``float8_e4m3fn`` cast, a library routine, on every finite bf16
value in range and on a million random float32 values.
"""
import numpy as np
import pytest
import torch

from oracle import e4m3

# (value, code): each follows from the OCP E4M3 definition (bias 7, 3-bit
# mantissa, subnormal step 2^-9, max 448 = 1.75 * 2^8).
ANCHORS = [
    (1.0, 0x38),                 # e=7, m=0
    (1.0625, 0x38),              # midpoint of 1.0 and 1.125: tie -> even mantissa (m=0)
    (1.1875, 0x3A),              # midpoint of 1.125 (m=1) and 1.25 (m=2): tie -> m=2
    (448.0, 0x7E),               # largest finite
    (-448.0, 0xFE),
    (2.0 ** -9, 0x01),           # smallest subnormal
    (2.0 ** -10, 0x00),          # half the smallest subnormal: tie -> 0 (even)
    (1.5 * 2.0 ** -10, 0x01),    # above the tie -> 2^-9
    (-0.0, 0x80),                # sign kept
    (2.0 ** -7 * 1.0625, 0x04),  # = 4.25 * 2^-9, subnormal: nearest grid point 4 * 2^-9
    (2.0 ** -6, 0x08),           # smallest normal: e=1, m=0
    (7 * 2.0 ** -9, 0x07),       # largest subnormal
    (240.0, 0x77),               # 1.875 * 2^7
    (0.3, 0x2A),                 # between 0.28125 (0x29) and 0.3125 (0x2A): nearer 0x2A
]


def test_decode_table_shape_and_specials():
    assert e4m3.DECODE.shape == (256,)
    assert np.isnan(e4m3.DECODE[0x7F]) and np.isnan(e4m3.DECODE[0xFF])
    assert np.sum(np.isnan(e4m3.DECODE)) == 2
    assert e4m3.DECODE[0x7E] == 448.0 and e4m3.DECODE[0xFE] == -448.0
    assert e4m3.DECODE[0x00] == 0.0 and np.signbit(e4m3.DECODE[0x80])
    pos = e4m3.DECODE[:0x7F]
    assert np.all(np.diff(pos) > 0)
    # every value is a multiple of 2^-9
    assert np.all(np.mod(pos * 512.0, 1.0) == 0.0)


@pytest.mark.parametrize("value,code", ANCHORS)
def test_encode_anchors(value, code):
    assert int(e4m3.encode(np.float32(value))) == code


def test_roundtrip_all_finite_codes():
    codes = np.array([b for b in range(256) if b not in e4m3.NAN_CODES], dtype=np.uint8)
    assert codes.size == 254
    back = e4m3.encode(e4m3.decode(codes).astype(np.float32))
    assert np.array_equal(back, codes)


def _torch_codes(x32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_matches_torch_on_every_bf16_in_range():
    bits = np.arange(65536, dtype=np.uint32) << 16
    v = bits.view(np.float32)
    v = v[np.isfinite(v) & (np.abs(v) <= 448.0)]
    assert v.size > 30000
    assert np.array_equal(e4m3.encode(v), _torch_codes(v))


def test_matches_torch_on_random_f32():
    r = np.random.default_rng(1234)
    mag = np.exp2(r.uniform(-14.0, np.log2(448.0), size=1_000_000)).astype(np.float32)
    mag = np.minimum(mag, np.float32(448.0))
    v = np.where(r.random(mag.size) < 0.5, -mag, mag).astype(np.float32)
    assert np.array_equal(e4m3.encode(v), _torch_codes(v))


def test_rejects_out_of_range():
    with pytest.raises(ValueError):
        e4m3.encode(np.float32(449.0))
    with pytest.raises(ValueError):
        e4m3.encode(np.float32(np.nan))
