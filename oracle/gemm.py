"""Scaled 8-bit matmuls (oracle; test infrastructure only).

Block-scaled FP8 ("nt": both operands K-contiguous), from the block32
DeepGEMM PR for DeepSeek-V4.1, "Modifications" (fp8_gemm_nt with recipe
``(1, bn, bk)``: activation groups of 1 x bk, weight tiles of bn x bk), and the
weight-scale layout ``[n_blocks, k_blocks]`` of the vLLM scaled_mm page
(XPUFp8BlockScaledMMKernel, process_weights_after_loading)::

    D[m, n] = sum_kb As[m, kb] * Ws[n // bn, kb] * P[m, n, kb] (+ bias[n])
    P[m, n, kb] = sum_{k in block kb} dec(Aq[m, k]) * dec(Wq[n, k])

Exactness: every e4m3 value is a multiple of 2^-9 of magnitude at most 448,
so every product is a multiple of 2^-18 below 2^18, and a sum of up to 8192
of them needs fewer than 53 significant bits. A float64 matmul of decoded
codes therefore returns P exactly in any summation order; only the scale
multiply and the sum over blocks round (in float64).

INT8 W8A8, from the vLLM scaled_mm page, AiterInt8ScaledMMLinearKernel
apply_weights: ``out = mm(scale_a * a, scale_b * b)`` with numpy broadcasting,
weights ``[N, K]``; the integer accumulator ``acc = sum_k a[m, k] * w[n, k]``
is exact (integer products below 2^14, sums below 2^27, so float64 BLAS is
exact too), then ``acc * sa * sb + bias`` in float64.

FP8 with per-tensor or per-row / per-column scales, from "Implementation: Sgl
project Sglang GEMM Interface" (fp8_scaled_mm: scales of shape (1,) or per row
of A / per column of B, optional bias) and the same broadcasting rule: the
exact float64 product of the decoded codes over the whole K (the exactness
argument above holds for up to 2^17 terms), times ``sa * sb``, plus bias.
"""
from __future__ import annotations

import numpy as np

from . import e4m3


def block_partials(Aq, Wq, bk: int) -> np.ndarray:
    """Exact per-block partial sums ``P[m, n, kb]`` (float64)."""
    A = e4m3.decode(Aq)
    W = e4m3.decode(Wq)
    M, K = A.shape
    N = W.shape[0]
    if K % bk != 0:
        raise ValueError("K must be a multiple of bk")
    KB = K // bk
    P = np.empty((M, N, KB), dtype=np.float64)
    for kb in range(KB):
        sl = slice(kb * bk, (kb + 1) * bk)
        P[:, :, kb] = A[:, sl] @ W[:, sl].T
    return P


def blockwise_scaled_mm(Aq, As, Wq, Ws, bn: int, bk: int, bias=None) -> np.ndarray:
    """Block-scaled FP8 GEMM -> float64 ``D [M, N]`` (before the output cast).

    ``Aq [M, K]`` / ``Wq [N, K]`` uint8 e4m3fn codes, ``As [M, K/bk]`` and
    ``Ws [ceil(N/bn), K/bk]`` float32, ``bias [N]`` or None.
    """
    A = e4m3.decode(Aq)
    W = e4m3.decode(Wq)
    As = np.asarray(As, dtype=np.float64)
    Ws = np.asarray(Ws, dtype=np.float64)
    M, K = A.shape
    N = W.shape[0]
    if K % bk != 0:
        raise ValueError("K must be a multiple of bk")
    col_block = np.arange(N) // bn
    D = np.zeros((M, N), dtype=np.float64)
    for kb in range(K // bk):
        sl = slice(kb * bk, (kb + 1) * bk)
        P = A[:, sl] @ W[:, sl].T
        D += As[:, kb][:, None] * Ws[col_block, kb][None, :] * P
    if bias is not None:
        D += np.asarray(bias, dtype=np.float64)[None, :]
    return D


def int8_acc(Aq, Wq) -> np.ndarray:
    """Exact int32-range accumulators ``acc [M, N]`` as int64."""
    A = np.asarray(Aq, dtype=np.int8).astype(np.float64)
    W = np.asarray(Wq, dtype=np.int8).astype(np.float64)
    acc = (A @ W.T).astype(np.int64)
    if acc.size and np.abs(acc).max() >= 2 ** 31:
        raise OverflowError("accumulator exceeds int32")
    return acc


def scaled_mm_int8(Aq, sa, Wq, sb, bias=None, acc=None) -> np.ndarray:
    """INT8 W8A8 -> float64 ``D [M, N]``; ``sa`` numel 1 or M, ``sb`` 1 or N."""
    if acc is None:
        acc = int8_acc(Aq, Wq)
    M, N = acc.shape
    sa = np.asarray(sa, dtype=np.float64).reshape(-1)
    sb = np.asarray(sb, dtype=np.float64).reshape(-1)
    if sa.size not in (1, M) or sb.size not in (1, N):
        raise ValueError("scale numel must be 1 or the matching dimension")
    sa_col = sa.reshape(-1, 1)   # [M, 1] or [1, 1]: numpy broadcasting
    sb_row = sb.reshape(1, -1)   # [1, N] or [1, 1]
    D = acc.astype(np.float64) * sa_col * sb_row
    if bias is not None:
        D = D + np.asarray(bias, dtype=np.float64)[None, :]
    return D


def scaled_mm_fp8(Aq, sa, Wq, sb, bias=None) -> np.ndarray:
    """FP8 per-tensor / per-token x per-channel -> float64 ``D [M, N]``.

    ``Aq [M, K]`` / ``Wq [N, K]`` uint8 e4m3fn codes; ``sa`` numel 1 or M,
    ``sb`` numel 1 or N; ``bias [N]`` or None.
    """
    A = e4m3.decode(Aq)
    W = e4m3.decode(Wq)
    M, K = A.shape
    N = W.shape[0]
    if K > 2 ** 17:
        raise ValueError("K above 2^17: the float64 sum is no longer exact")
    sa = np.asarray(sa, dtype=np.float64).reshape(-1)
    sb = np.asarray(sb, dtype=np.float64).reshape(-1)
    if sa.size not in (1, M) or sb.size not in (1, N):
        raise ValueError("scale numel must be 1 or the matching dimension")
    D = (A @ W.T) * sa.reshape(-1, 1) * sb.reshape(1, -1)
    if bias is not None:
        D = D + np.asarray(bias, dtype=np.float64)[None, :]
    return D


# ---- power-of-two (UE8M0) block scales ----------------------------------------
# The vLLM scaled_mm page (XPUFp8BlockScaledMMKernel, process_weights_after_
# loading) accepts weight scales stored as float8_e8m0fnu bytes and upcasts
# them to float32; the block32 DeepGEMM PR keeps UE8M0 activation scales. An
# E8M0 byte b holds the power of two 2^(b - 127) (b = 255 is NaN). With both
# operands' block scales in that form the product is the same block-scaled
# GEMM as above, with the decoded values as the scales.


def e8m0_decode(b) -> np.ndarray:
    """E8M0 bytes -> exact float64 values 2^(b - 127) (255 -> NaN)."""
    b = np.asarray(b, dtype=np.uint8).astype(np.int64)
    v = np.ldexp(1.0, b - 127)
    return np.where(b == 255, np.nan, v)


def blockwise_scaled_mm_e8m0(Aq, As_b, Wq, Ws_b, bn: int, bias=None) -> np.ndarray:
    """Block-scaled FP8 GEMM with E8M0 scales, 32-wide K blocks -> float64.

    ``As_b [M, K/32]`` and ``Ws_b [ceil(N/bn), K/32]`` uint8 E8M0 bytes."""
    return blockwise_scaled_mm(Aq, e8m0_decode(As_b), Wq, e8m0_decode(Ws_b), bn, 32, bias)
