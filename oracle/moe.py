"""MoE routing tables and the expert-grouped block GEMM (oracle; test only).

From "Implementation: Sgl project Sglang CUTLASS MoE", Description and I/O
Contract: from the router's ``topk_ids`` build ``expert_offsets`` (where each
expert's rows begin), per-expert problem sizes (M x N x K), an input
permutation that shuffles token rows before the grouped GEMM and an output
permutation that restores the original order afterwards. Row shuffling is a
destination-to-source gather ("Implementation: Sgl project Sglang GEMM
Interface", Utility: shuffle_rows).

Readings taken where the page is silent:

* the flat index of choice ``j`` of token ``t`` is ``i = t * topk + j``;
* rows of one expert keep ascending flat order (a stable sort), so every
  index is unique and can be compared exactly;
* ``expert_offsets`` has ``E + 1`` entries, the last equal to ``T * topk``;
* ``problem_sizes1[e] = (m_e, n, k)`` is the GEMM run here (width ``n`` out of
  ``k``); ``problem_sizes2[e] = (m_e, k, n)`` is the follow-on GEMM back to
  width ``k``;
* ``input_permutation[p]`` is the token row feeding sorted slot ``p``;
  ``output_permutation[i]`` is the sorted slot holding flat choice ``i``.

Finalize, from "Implementation: Sgl project Sglang Fused MoE Marlin", I/O
Contract (topk_weights, mul_topk_weights, the reduction of the routed
outputs): every routed row is multiplied by its gate weight and the top-k rows
of each token are summed, ``out[t] = sum_j w[t, j] * D[row(t, j)]``.
"""
from __future__ import annotations

import numpy as np

from . import gemm


def moe_mm_data(topk_ids, E: int, n: int, k: int):
    ids = np.asarray(topk_ids, dtype=np.int64)
    T, topk = ids.shape
    flat = ids.reshape(-1)
    if flat.size and (flat.min() < 0 or flat.max() >= E):
        raise ValueError("expert id out of range")
    cnt = np.bincount(flat, minlength=E).astype(np.int64)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(cnt)
    ps1 = np.stack([cnt, np.full(E, n), np.full(E, k)], axis=1)
    ps2 = np.stack([cnt, np.full(E, k), np.full(E, n)], axis=1)
    order = np.argsort(flat, kind="stable")
    input_perm = order // topk
    output_perm = np.empty(flat.size, dtype=np.int64)
    output_perm[order] = np.arange(flat.size)
    return (offsets.astype(np.int32), ps1.astype(np.int32), ps2.astype(np.int32),
            input_perm.astype(np.int32), output_perm.astype(np.int32))


def grouped_blockwise_scaled_mm(Aq, As, W, Ws, expert_offsets, input_perm,
                                bn: int, bk: int) -> np.ndarray:
    """Sorted-order grouped GEMM: ``D_sorted[p] = blockwise(A[perm[p]], W[e(p)])``.

    ``Aq [T, K]`` / ``As [T, K/bk]`` are the unsorted token rows; ``W [E, N, K]``,
    ``Ws [E, ceil(N/bn), K/bk]``. Returns float64 ``[total_m, N]``.
    """
    off = np.asarray(expert_offsets, dtype=np.int64)
    perm = np.asarray(input_perm, dtype=np.int64)
    E = off.size - 1
    N = W.shape[1]
    out = np.zeros((perm.size, N), dtype=np.float64)
    for e in range(E):
        lo, hi = off[e], off[e + 1]
        if hi == lo:
            continue
        rows = perm[lo:hi]
        out[lo:hi] = gemm.blockwise_scaled_mm(Aq[rows], As[rows], W[e], Ws[e], bn, bk)
    return out


def unpermute(D_sorted, output_perm) -> np.ndarray:
    """``out[i] = D_sorted[output_perm[i]]``."""
    return np.asarray(D_sorted)[np.asarray(output_perm, dtype=np.int64)]


def finalize(D, topk_weights, topk: int, output_perm=None) -> np.ndarray:
    """``out[t] = sum_j w[t, j] * D[row(t, j)]`` in float64 -> ``[T, N]``.

    ``D [T*topk, N]`` is un-permuted (row ``t*topk + j``) or, with
    ``output_perm``, expert-sorted (row ``output_perm[t*topk + j]``).
    ``topk_weights [T, topk]`` or None (weights 1).
    """
    D = np.asarray(D, dtype=np.float64)
    rows = D.shape[0]
    if rows % topk:
        raise ValueError("D must have T * topk rows")
    T = rows // topk
    if output_perm is not None:
        D = unpermute(D, output_perm)
    w = np.ones((T, topk)) if topk_weights is None else np.asarray(topk_weights, np.float64).reshape(T, topk)
    return np.einsum("tj,tjn->tn", w, D.reshape(T, topk, -1))
