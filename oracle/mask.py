"""The visibility rule of chunk-wise block-causal attention, as an explicit mask.

Sources: JoyAI-Video-Edit tutorial (agifrontier.github.io), section "From
bidirectional editing to a chunk-wise causal architecture"; neurohive.io review,
sections "Chunks and fighting drift" and "Architecture" (figure caption: the
attention mask over the token groups visible to the active chunk).

Readings where the pages are silent (each is listed in the design notes):

* The window holds the W most recent chunks *before* the active one; the active
  chunk itself is always visible (bidirectional within the chunk).
* The sink is the first ``n_sink`` chunks (the pages: "the first chunk"); a
  chunk that is both in the window and a sink is counted once (set union).
* Condition tokens are visible to every chunk query.
* Only chunk tokens are queries (condition-token queries are not computed).

Parity: pinned (hand-derived visibility fixture, brute-force gather form,
library SDPA on the single-chunk case).
"""
from __future__ import annotations

from typing import Iterable, Optional

import numpy as np


def visible_chunk(c_query: int, c_key: int, window: int, n_sink: int) -> bool:
    """May a query token of chunk ``c_query`` see a key token of chunk ``c_key``?

    The four clauses of the rule: same chunk (bidirectional inside a chunk);
    never a future chunk; a sink chunk; one of the ``window`` most recent
    earlier chunks.
    """
    if c_key == c_query:
        return True
    if c_key > c_query:
        return False
    if c_key < n_sink:
        return True
    return c_query - window <= c_key <= c_query - 1


def visible_history(c: int, window: int, n_sink: int) -> list[int]:
    """The earlier chunks that chunk ``c`` sees, in increasing order."""
    return [j for j in range(c) if visible_chunk(c, j, window, n_sink)]


def chunk_ids(n_chunks: int, chunk_tokens: int, cond_len: int) -> np.ndarray:
    """Chunk id of every position of [cond | chunk 0 | ... | chunk n-1]; -1 = cond."""
    ids = np.empty(cond_len + n_chunks * chunk_tokens, dtype=np.int64)
    ids[:cond_len] = -1
    for c in range(n_chunks):
        start = cond_len + c * chunk_tokens
        ids[start:start + chunk_tokens] = c
    return ids


def mask_rows(c: int, chunk_tokens: int, cond_len: int, window: int, n_sink: int,
              visible: Optional[Iterable[int]] = None) -> np.ndarray:
    """Boolean mask [T, Lc + (c+1) T] of chunk c's queries over [cond | chunks 0..c].

    ``visible`` optionally replaces the rule by an explicit set of earlier
    chunks (what a cache that was evicted by hand still holds).
    """
    ids = chunk_ids(c + 1, chunk_tokens, cond_len)
    if visible is None:
        key_ok = np.array([True if j < 0 else visible_chunk(c, int(j), window, n_sink)
                           for j in ids])
    else:
        allowed = set(int(x) for x in visible) | {c}
        key_ok = np.array([True if j < 0 else int(j) in allowed for j in ids])
    return np.broadcast_to(key_ok, (chunk_tokens, ids.size)).copy()


def full_stream_mask(n_chunks: int, chunk_tokens: int, cond_len: int, window: int,
                     n_sink: int) -> np.ndarray:
    """Mask [n T, Lc + n T] for all chunk queries of a stream at once.

    Row r belongs to chunk r // T; column j to chunk ``chunk_ids[j]``.  This is
    the teacher-forcing form of the same rule (every chunk in one matrix).
    """
    ids = chunk_ids(n_chunks, chunk_tokens, cond_len)
    m = np.zeros((n_chunks * chunk_tokens, ids.size), dtype=bool)
    for r in range(n_chunks * chunk_tokens):
        cq = r // chunk_tokens
        for j, ck in enumerate(ids):
            m[r, j] = True if ck < 0 else visible_chunk(cq, int(ck), window, n_sink)
    return m
