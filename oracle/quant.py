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
