"""Attention of one chunk-step over [cond | clean chunks 0..c-1 | chunk c].

Follows the pages' description of a streaming step (JoyAI-Video-Edit tutorial,
agifrontier.github.io, sections "From bidirectional editing to a chunk-wise
causal architecture" and "Hardware-software co-deployment" / "constant KV
cache"; neurohive.io review, section "Chunks and fighting drift"):

* chunk c is the chunk being generated: its queries and its own K/V come from
  the current denoise step;
* earlier chunks contribute the *clean* K/V written to the cache after they
  were generated;
* the condition tokens' K/V come first in the sequence.

The full concatenated sequence is built, the explicit mask rows of chunk c are
materialised over it (``oracle.mask.mask_rows``), and naive masked attention is
run (``oracle.attention.masked_attention``).  ``rows`` restricts the queries to
a subset of chunk c's tokens; the keys are always the full sequence.

``attend_queries`` gives other query rows (the condition tokens' own
queries) the key set of chunk c.

Parity: pinned (see ``oracle.mask`` and ``oracle.attention``; the gather
form of the tests pins both functions).
"""
from __future__ import annotations

from typing import Callable, Iterable, Optional, Sequence

import numpy as np

from .attention import masked_attention
from .mask import mask_rows


def attend_chunk(c: int, q: np.ndarray, k_cur: np.ndarray, v_cur: np.ndarray,
                 clean_k: Callable[[int], np.ndarray], clean_v: Callable[[int], np.ndarray],
                 cond_k: np.ndarray, cond_v: np.ndarray, window: int, n_sink: int,
                 scale: float, rows: Optional[Sequence[int]] = None,
                 visible: Optional[Iterable[int]] = None, heads: Optional[Sequence[int]] = None):
    """Output [H', |rows|, D] (float64) and lse [H', |rows|] for chunk ``c``.

    q, k_cur, v_cur: [H, T, D]; cond_k, cond_v: [H, Lc, D];
    clean_k(j), clean_v(j): [H, T, D] clean K/V of earlier chunk j.
    ``heads`` selects a subset of heads (all by default).
    """
    H, T, _ = q.shape
    Lc = cond_k.shape[1]
    hs = list(range(H)) if heads is None else list(heads)
    rs = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    m = mask_rows(c, T, Lc, window, n_sink, visible)[rs]
    ks = [cond_k[hs]] + [clean_k(j)[hs] for j in range(c)] + [k_cur[hs]]
    vs = [cond_v[hs]] + [clean_v(j)[hs] for j in range(c)] + [v_cur[hs]]
    k_all = np.concatenate(ks, axis=1)
    v_all = np.concatenate(vs, axis=1)
    return masked_attention(q[hs][:, rs], k_all, v_all, m, scale)


def attend_queries(c: int, q_rows: np.ndarray, k_cur: np.ndarray, v_cur: np.ndarray,
                   clean_k: Callable[[int], np.ndarray], clean_v: Callable[[int], np.ndarray],
                   cond_k: np.ndarray, cond_v: np.ndarray, window: int, n_sink: int, scale: float,
                   visible: Optional[Iterable[int]] = None, heads: Optional[Sequence[int]] = None):
    """Output [H', M, D] and lse [H', M] for M extra query rows (``q_rows``,
    [H, M, D]) that see exactly the keys of chunk ``c``'s queries.

    The pages do not say what the condition tokens' own queries see in the
    joint attention (neurohive.io review, "Architecture": condition and video
    tokens share the model's attention); the reading taken here gives them the
    key set of the chunk being generated: the condition rows, the visible
    earlier chunks and chunk c.  Every row of chunk c's mask is the same, so
    that row is used for all M queries.
    """
    T = k_cur.shape[1]
    Lc = cond_k.shape[1]
    hs = list(range(q_rows.shape[0])) if heads is None else list(heads)
    key_ok = mask_rows(c, T, Lc, window, n_sink, visible)[0]
    m = np.broadcast_to(key_ok, (q_rows.shape[1], key_ok.size))
    ks = [cond_k[hs]] + [clean_k(j)[hs] for j in range(c)] + [k_cur[hs]]
    vs = [cond_v[hs]] + [clean_v(j)[hs] for j in range(c)] + [v_cur[hs]]
    return masked_attention(q_rows[hs], np.concatenate(ks, axis=1), np.concatenate(vs, axis=1), m, scale)
