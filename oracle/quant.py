"""8-bit activation quantization (oracle; test infrastructure only).

Follows "Implementation: Sgl project Sglang GEMM Interface", Description ›
Quantization Routines:

* sgl_per_token_group_quant_8bit — per token (row) and per group of
  ``group_size`` consecutive K elements, to FP8 or INT8, with an epsilon, a
  clipping range ``[qmin, qmax]`` and an optional UE8M0 (power-of-two) scale;
* sgl_per_token_quant_fp8 — the same with one group spanning the whole row;
* sgl_per_tensor_quant_fp8 — one scale for the tensor, dynamic (from the
  tensor's absolute maximum) or static (given).

The INT8 flavour follows the vLLM scaled_mm page, AiterInt8ScaledMMLinearKernel
(dynamic when no input scale is given, static when a scalar is given;
symmetric only).

Readings where the pages are silent, in this order of operations, all in
IEEE float32 with round-to-nearest-even:

1. ``a = max |x|`` over the group (exact);
2. ``s = max(a, eps) / qmax`` — eps floors the absolute maximum;
3. UE8M0: ``s`` rounded up to the next power of two (kept as that float32
   value), so ``|x / s| <= qmax`` still holds;
4. ``y = x / s`` (a true division, not a multiply by ``1/s``), clamped to
   ``[qmin, qmax]``;
5. FP8: nearest e4m3fn code, ties to even; INT8: round half to even.
"""
from __future__ import annotations

import numpy as np

from . import e4m3

F32 = np.float32


def ue8m0_ceil(s) -> np.ndarray:
    """Round positive float32 values up to a power of two (bitwise).

    A value whose mantissa field is non-zero gets its exponent field raised
    by one and its mantissa cleared; exact powers of two are unchanged.
    """
    s = np.asarray(s, dtype=F32)
    bits = s.view(np.uint32)
    frac = bits & np.uint32(0x007FFFFF)
    up = (bits & np.uint32(0x7F800000)) + np.uint32(0x00800000)
    return np.where(frac != 0, up, bits).astype(np.uint32).view(F32)


def _codes(y: np.ndarray, qdtype: str) -> np.ndarray:
    if qdtype == "e4m3":
        return e4m3.encode(y)
    if qdtype == "i8":
        return np.rint(y).astype(np.int8)
    raise ValueError(qdtype)


def _quantize_with_scale(x32: np.ndarray, s: np.ndarray, qmin, qmax, qdtype):
    y = (x32 / s).astype(F32)
    y = np.minimum(np.maximum(y, F32(qmin)), F32(qmax))
    return _codes(y, qdtype)


def per_token_group(x, group_size: int, eps: float, qmin: float, qmax: float,
                    scale_ue8m0: bool = False, qdtype: str = "e4m3"):
    """``x [M, K]`` -> ``(q [M, K], s [M, K/group_size] float32 row-major)``."""
    x32 = np.asarray(x, dtype=F32)
    M, K = x32.shape
    if K % group_size != 0:
        raise ValueError("group_size must divide K")
    G = K // group_size
    xg = x32.reshape(M, G, group_size)
    a = np.abs(xg).max(axis=2)
    s = (np.maximum(a, F32(eps)) / F32(qmax)).astype(F32)
    if scale_ue8m0:
        s = ue8m0_ceil(s)
    q = _quantize_with_scale(xg, s[:, :, None], qmin, qmax, qdtype)
    return q.reshape(M, K), s


def per_tensor_dynamic(x, eps: float, qmin: float, qmax: float,
                       scale_ue8m0: bool = False, qdtype: str = "e4m3"):
    """One scale from the whole tensor's absolute maximum -> ``(q, s[1])``."""
    x32 = np.asarray(x, dtype=F32)
    a = np.abs(x32).max() if x32.size else F32(0.0)
    s = np.array([np.maximum(a, F32(eps)) / F32(qmax)], dtype=F32)
    if scale_ue8m0:
        s = ue8m0_ceil(s)
    return _quantize_with_scale(x32, s[0], qmin, qmax, qdtype), s


def static(x, scale: float, qmin: float, qmax: float, qdtype: str = "e4m3"):
    """Given scale -> codes (the scale itself is an input, not an output)."""
    x32 = np.asarray(x, dtype=F32)
    return _quantize_with_scale(x32, F32(scale), qmin, qmax, qdtype)


# ---- fused SiLU-and-mul + quant, masked rows ---------------------------------
# "Implementation: Sgl project Sglang GEMM Interface", Description ›
# Quantization Routines: sgl_per_token_group_quant_8bit has a variant with a
# fused SiLU-and-mul and masked-M support (arguments fuse_silu_and_mul and
# masked_m in its signature). The page gives no formula; the readings taken:
#
# * SiLU-and-mul of a row [gate | up] of width 2K is y = silu(gate) * up with
#   silu(g) = g / (1 + exp(-g)), the first half the gate and the second half
#   the multiplier (the gated-MLP convention of the MoE pages' activations);
# * y is evaluated in IEEE float32, one rounding per operation, in the order
#   e = exp(-g), d = 1 + e, h = g / d, y = h * up, where exp is the correctly
#   rounded float32 exponential. Every step is then an exactly defined float32
#   operation, so the code decided from y is unique;
# * masked rows: the input is E blocks of max_m rows ([E, max_m, .] flattened)
#   and masked_m[e] rows of block e are valid; the other rows are neither read
#   nor written.


def exp_rn32(x) -> np.ndarray:
    """Correctly rounded float32 exp of float32 inputs.

    numpy's float64 exp (error well below a float64 ulp) rounded once to
    float32: the float32 result is the correctly rounded one unless the exact
    value lies within about 2^-52 (relative) of a float32 rounding midpoint;
    tests/test_oracle_quant.py checks every bf16 input against an exact
    decimal computation. Overflow gives +inf and deep underflow +0, as IEEE
    rounding of the exact value does."""
    x64 = np.asarray(x, dtype=F32).astype(np.float64)
    with np.errstate(over="ignore"):
        return np.exp(x64).astype(F32)


def silu_and_mul(x, K: int | None = None) -> np.ndarray:
    """``x [M, 2K]`` (gate | up) -> ``y [M, K]`` float32 (readings above)."""
    x32 = np.asarray(x, dtype=F32)
    if K is None:
        if x32.shape[1] % 2:
            raise ValueError("silu_and_mul: odd row width")
        K = x32.shape[1] // 2
    g, u = x32[:, :K], x32[:, K:2 * K]
    with np.errstate(over="ignore", invalid="ignore"):
        e = exp_rn32(-g)
        d = (F32(1.0) + e).astype(F32)
        h = (g / d).astype(F32)
        return (h * u).astype(F32)


def masked_rows(M: int, masked_m, max_m: int) -> np.ndarray:
    """Boolean [M]: row r is valid iff r % max_m < masked_m[r // max_m]."""
    mm = np.asarray(masked_m, dtype=np.int64)
    if max_m <= 0 or M % max_m != 0 or mm.size != M // max_m:
        raise ValueError("masked rows: M must be len(masked_m) * max_m")
    r = np.arange(M)
    return (r % max_m) < mm[r // max_m]


def per_token_group_fused(x, group_size: int, eps: float, qmin: float, qmax: float,
                          scale_ue8m0: bool = False, qdtype: str = "e4m3",
                          silu: bool = False, masked_m=None, max_m: int | None = None):
    """Per-token-group quant of ``silu_and_mul(x)`` (or of ``x``) on the valid
    rows. Returns ``(q, s, valid)``; rows where ``valid`` is False hold zeros
    here and are left untouched by the GPU library."""
    x32 = np.asarray(x, dtype=F32)
    y = silu_and_mul(x32) if silu else x32
    M = y.shape[0]
    valid = np.ones(M, dtype=bool) if masked_m is None else masked_rows(M, masked_m, max_m)
    q = np.zeros(y.shape, dtype=np.uint8 if qdtype == "e4m3" else np.int8)
    s = np.zeros((M, y.shape[1] // group_size), dtype=F32)
    if valid.any():
        qv, sv = per_token_group(y[valid], group_size, eps, qmin, qmax, scale_ue8m0, qdtype)
        q[valid], s[valid] = qv, sv
    return q, s, valid


def e8m0_bytes(s) -> np.ndarray:
    """Power-of-two float32 scales (UE8M0-rounded) -> their E8M0 bytes, the
    biased exponent b with s = 2^(b - 127) (packed UE8M0 storage, the
    float8_e8m0fnu scale dtype of the vLLM scaled_mm page)."""
    s = np.asarray(s, dtype=F32)
    m, e = np.frexp(s.astype(np.float64))        # s = m * 2^e, m in [0.5, 1)
    if not np.all(m == 0.5):
        raise ValueError("e8m0_bytes: scales must be powers of two")
    b = e - 1 + 127
    if np.any(b < 0) or np.any(b > 254):
        raise ValueError("e8m0_bytes: exponent out of range")
    return b.astype(np.uint8)
