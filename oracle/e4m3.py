"""OCP float8 e4m3fn codec, exact (oracle; test infrastructure only).

The block-FP8 paths on the pages store weights and activations as
``torch.float8_e4m3fn`` (block32 DeepGEMM PR, review of the pre-quantized
activation path asserting that dtype). That is the OCP 8-bit "E4M3" format:
1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, no infinities,
exponent 15 with mantissa 7 is NaN, largest finite magnitude 448.

Decoding builds a 256-entry float64 table. Encoding rounds a finite value of
magnitude at most 448 to the nearest representable value, ties to the code
whose mantissa LSB is 0; every midpoint between neighbours is a dyadic
rational, so comparing in float64 is exact. The sign is kept, so negative
values that round to zero give the negative-zero code 0x80.
"""
from __future__ import annotations

import numpy as np

MAX = 448.0
NAN_CODES = (0x7F, 0xFF)


def _decode_one(b: int) -> float:
    s = -1.0 if (b >> 7) & 1 else 1.0
    e = (b >> 3) & 0xF
    m = b & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * m * 2.0 ** -9
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


DECODE = np.array([_decode_one(b) for b in range(256)], dtype=np.float64)

# Positive finite values, codes 0x00..0x7E, strictly increasing.
_POS = DECODE[:0x7F].copy()
_MID = (_POS[:-1] + _POS[1:]) / 2.0


def decode(codes) -> np.ndarray:
    """uint8 codes (any shape) -> exact float64 values."""
    return DECODE[np.asarray(codes, dtype=np.uint8)]


def encode(x) -> np.ndarray:
    """Finite values with ``|x| <= 448`` -> uint8 e4m3fn codes, RNE."""
    x = np.asarray(x)
    a = np.abs(x.astype(np.float64))
    if not np.all(np.isfinite(a)):
        raise ValueError("e4m3 encode: non-finite input")
    if np.any(a > MAX):
        raise ValueError("e4m3 encode: magnitude above 448 (clamp first)")
    j = np.searchsorted(_MID, a, side="left")
    jc = np.minimum(j, _MID.size - 1)
    tie = (j < _MID.size) & (_MID[jc] == a)
    code = np.where(tie & (j % 2 == 1), j + 1, j).astype(np.uint8)
    neg = np.signbit(x)
    return np.where(neg, code | np.uint8(0x80), code).astype(np.uint8)
