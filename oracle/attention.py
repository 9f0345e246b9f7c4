"""Naive softmax attention under an explicit boolean mask, in float64.

For each head h and query row i:
    s_ij = scale * <q_i, k_j>          for keys j with mask[i, j] true,
    p_ij = exp(s_ij - max_j s_ij) / sum_j exp(s_ij - max_j s_ij),
    o_i  = sum_j p_ij v_j.
Masked keys take no part: their probability is exactly 0.

This is the textbook definition of scaled dot-product attention; the only
method-specific input is the mask (``oracle.mask``).  ``numpy.matmul`` serves as
the dot-product step.

Parity: pinned (torch CPU scaled_dot_product_attention in fp64 with the same
boolean mask, pure-Python gather form, closed forms, rows summing to one).
"""
from __future__ import annotations

import numpy as np


def masked_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask: np.ndarray,
                     scale: float, return_probs: bool = False):
    """q [H, M, D], k/v [H, N, D], mask [M, N] bool -> o [H, M, D] float64.

    Also returns the log-sum-exp of the scaled scores per row ([H, M]) and,
    when asked, the probability matrix [H, M, N].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    mask = np.asarray(mask, dtype=bool)
    if not mask.any(axis=1).all():
        raise ValueError("a query row sees no key")
    s = scale * np.matmul(q, np.swapaxes(k, -1, -2))  # [H, M, N]
    s = np.where(mask[None, :, :], s, -np.inf)
    row_max = s.max(axis=-1, keepdims=True)
    e = np.exp(s - row_max)  # exp(-inf) = 0 for masked keys
    denom = e.sum(axis=-1, keepdims=True)
    p = e / denom
    o = np.matmul(p, v)
    lse = (row_max + np.log(denom))[..., 0]
    if return_probs:
        return o, lse, p
    return o, lse
