"""Seeded synthetic inputs shared by the CPU oracle checks and the GPU path.

This module only draws inputs. It holds none of the arithmetic that the hot
path computes (activation quantization, the scaled matmuls, the routing
tables): the GPU library and the oracle each implement that on their own and
both consume the tensors made here.

Every tensor has its own random stream, ``numpy.random.default_rng([seed, tag])``
with the tags below, so that changing one tensor's shape never changes another
tensor's values.

Weights arrive already quantized, the way a checkpoint ships them (the block32
DeepGEMM PR for DeepSeek-V4.1, "Modifications": checkpoint FP8 weights are
kept as they are). Weight preparation happens once, offline, on the host:
per ``[bn, bk]`` tile the scale is the tile's absolute maximum over the e4m3
maximum 448, and the codes come from torch's own CPU ``float8_e4m3fn`` cast
(a library routine, not this project's encoder). INT8 weights are symmetric
per channel (row) or per tensor with divisor 127 and numpy's round-half-even.
"""
from __future__ import annotations

import numpy as np
import torch

TAG_A = 1
TAG_W = 2
TAG_OUTLIER = 3
TAG_BIAS = 4
TAG_TOPK = 5
TAG_GATE = 6

E4M3_MAX = 448.0


def rng(seed: int, tag: int) -> np.random.Generator:
    return np.random.default_rng([seed, tag])


def normal_f32(shape, sigma: float, seed: int, tag: int) -> np.ndarray:
    return (rng(seed, tag).standard_normal(size=shape, dtype=np.float32)
            * np.float32(sigma)).astype(np.float32)


def activations(M: int, K: int, dtype: str = "bf16", sigma: float = 1.0,
                outlier_frac: float = 0.0, outlier_mult: float = 20.0,
                seed: int = 0) -> torch.Tensor:
    """Activation matrix ``[M, K]`` ~ N(0, sigma^2) as a CPU torch tensor.

    With ``outlier_frac > 0`` a Bernoulli(outlier_frac) mask drawn from its
    own stream multiplies the selected entries by ``outlier_mult``.
    ``dtype`` is ``"bf16"`` (torch's round-to-nearest-even cast), ``"f16"``
    or ``"f32"``.
    """
    x = normal_f32((M, K), sigma, seed, TAG_A)
    if outlier_frac > 0.0:
        mask = rng(seed, TAG_OUTLIER).random(size=(M, K)) < outlier_frac
        x = np.where(mask, x * np.float32(outlier_mult), x).astype(np.float32)
    t = torch.from_numpy(x)
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    if dtype == "f16":
        return t.to(torch.float16)
    if dtype == "f32":
        return t
    raise ValueError(f"unknown activation dtype {dtype!r}")


def bias(N: int, dtype: str = "bf16", sigma: float = 1.0, seed: int = 0) -> torch.Tensor:
    t = torch.from_numpy(normal_f32((N,), sigma, seed, TAG_BIAS))
    return t.to(torch.bfloat16 if dtype == "bf16" else torch.float16)


def _quantize_block_tile_rows(w: np.ndarray, bn: int, bk: int):
    """One [N, K] float32 weight -> (e4m3fn codes [N, K] uint8, scales [nb, kb])."""
    N, K = w.shape
    nb, kb = -(-N // bn), -(-K // bk)
    pad = np.zeros((nb * bn, kb * bk), dtype=np.float32)
    pad[:N, :K] = np.abs(w)
    amax = pad.reshape(nb, bn, kb, bk).max(axis=(1, 3))
    ws = (np.maximum(amax, np.float32(1e-12)) / np.float32(E4M3_MAX)).astype(np.float32)
    full = np.repeat(np.repeat(ws, bn, axis=0), bk, axis=1)[:N, :K]
    ratio = np.clip(w / full, -E4M3_MAX, E4M3_MAX).astype(np.float32)
    codes = torch.from_numpy(ratio).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, ws


def _pow2_at_least(x: np.ndarray) -> np.ndarray:
    """Smallest power of two >= x (x > 0), via frexp: x = m 2^e, m in [0.5, 1)."""
    m, e = np.frexp(x.astype(np.float64))
    return np.ldexp(1.0, np.where(m == 0.5, e - 1, e)).astype(np.float32)


def fp8_block_weights_e8m0(N: int, K: int, bn: int, bk: int = 32, sigma: float = 0.02,
                           seed: int = 0, tag: int = TAG_W):
    """Block-FP8 weights whose per-tile scales are powers of two, the way a
    checkpoint with float8_e8m0fnu weight scales ships them: the scale of a
    [bn, bk] tile is the smallest power of two >= tile amax / 448, the codes
    are torch's e4m3fn cast of w / scale. Returns ``(Wq [N, K] uint8,
    Ws_e8m0 [ceil(N/bn), ceil(K/bk)] uint8)`` with scale = 2^(byte - 127)."""
    w = normal_f32((N, K), sigma, seed, tag)
    nb, kb = -(-N // bn), -(-K // bk)
    pad = np.zeros((nb * bn, kb * bk), dtype=np.float32)
    pad[:N, :K] = np.abs(w)
    amax = pad.reshape(nb, bn, kb, bk).max(axis=(1, 3))
    ws = _pow2_at_least(np.maximum(amax, np.float32(1e-12)) / np.float32(E4M3_MAX))
    full = np.repeat(np.repeat(ws, bn, axis=0), bk, axis=1)[:N, :K]
    ratio = np.clip(w / full, -E4M3_MAX, E4M3_MAX).astype(np.float32)
    codes = torch.from_numpy(ratio).to(torch.float8_e4m3fn).view(torch.uint8)
    exps = (ws.view(np.uint32) >> np.uint32(23)).astype(np.uint8)
    return codes, torch.from_numpy(exps)


def fp8_block_weights(N: int, K: int, bn: int, bk: int, sigma: float = 0.02,
                      seed: int = 0, tag: int = TAG_W, experts: int | None = None):
    """Checkpoint-style block-FP8 weights.

    Returns ``(Wq, Ws)``: ``Wq`` is ``[N, K]`` (or ``[E, N, K]``) uint8 holding
    e4m3fn codes, ``Ws`` is ``[ceil(N/bn), ceil(K/bk)]`` (or ``[E, ...]``)
    float32, one scale per weight tile. Experts are drawn one after another
    from the same stream, expert 0 first.
    """
    g = rng(seed, tag)
    E = 1 if experts is None else experts
    nb, kb = -(-N // bn), -(-K // bk)
    wq = torch.empty((E, N, K), dtype=torch.uint8)
    ws = np.empty((E, nb, kb), dtype=np.float32)
    for e in range(E):
        w = (g.standard_normal(size=(N, K), dtype=np.float32) * np.float32(sigma)).astype(np.float32)
        wq[e], ws[e] = _quantize_block_tile_rows(w, bn, bk)
    ws_t = torch.from_numpy(ws)
    if experts is None:
        return wq[0].contiguous(), ws_t[0].contiguous()
    return wq, ws_t


def int8_weights(N: int, K: int, per_channel: bool = True, sigma: float = 0.02,
                 seed: int = 0):
    """Symmetric INT8 weights ``[N, K]`` int8 with fp32 scales ``[N]`` or ``[1]``."""
    w = normal_f32((N, K), sigma, seed, TAG_W)
    if per_channel:
        s = (np.abs(w).max(axis=1) / np.float32(127.0)).astype(np.float32)
        q = np.clip(np.rint(w / s[:, None]), -128, 127).astype(np.int8)
    else:
        s = np.array([np.abs(w).max() / np.float32(127.0)], dtype=np.float32)
        q = np.clip(np.rint(w / s[0]), -128, 127).astype(np.int8)
    return torch.from_numpy(q), torch.from_numpy(s)


def zipf_topk_ids(T: int, E: int, topk: int, alpha: float = 1.1, seed: int = 0) -> torch.Tensor:
    """Router output ``[T, topk]`` int32 with Zipf(alpha)-skewed expert load.

    Per token, the ``topk`` distinct experts with the largest
    ``log p_e + Gumbel`` keys, ``p_e`` proportional to ``(e+1)^-alpha``
    (Gumbel-top-k: sampling without replacement in proportion to p), stored in
    decreasing key order.
    """
    if topk > E:
        raise ValueError("topk must not exceed the number of experts")
    logp = -alpha * np.log(np.arange(1, E + 1, dtype=np.float64))
    g = rng(seed, TAG_TOPK).gumbel(size=(T, E))
    keys = logp[None, :] + g
    order = np.argsort(-keys, axis=1, kind="stable")[:, :topk]
    return torch.from_numpy(order.astype(np.int32))


def topk_weights(T: int, topk: int, seed: int = 0) -> torch.Tensor:
    """Router gate weights ``[T, topk]`` float32: a softmax over ``topk``
    standard-normal logits per token (positive, each row sums to about 1)."""
    z = rng(seed, TAG_GATE).standard_normal(size=(T, topk)).astype(np.float32)
    e = np.exp(z - z.max(axis=1, keepdims=True))
    return torch.from_numpy((e / e.sum(axis=1, keepdims=True)).astype(np.float32))
