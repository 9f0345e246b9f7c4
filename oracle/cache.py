"""A plain list model of the bounded KV cache: one sink plus a ring of W slots.

Sources: JoyAI-Video-Edit tutorial (agifrontier.github.io), section
"Hardware-software co-deployment", bullet "constant KV cache" (clean K/V are
written right after a chunk is generated; the cache is always global sink +
sliding local window, so its memory stays level); neurohive.io review, section
"Chunks and fighting drift" (the first chunk stays in context permanently);
aiinking.com article, section "Bounded KV cache" (the cache size is limited).

Readings where the pages are silent:

* Slots 0..n_sink-1 hold the sink chunks, which are never evicted.
* Window slots n_sink..n_sink+W-1 are used in cyclic order: a new window chunk
  goes into the slot after the most recently written window slot.  If that
  slot is occupied, its chunk (always the oldest window chunk) is evicted.
* ``evict(n)`` drops the n oldest window chunks (first in, first out); asking
  for more than the window holds is an error and changes nothing.

Parity: pinned (closed form slot(c) = n_sink + (c - n_sink) mod W, evicted
chunk c - W, occupancy min(c + 1, n_sink + W), hand-written fixture).
"""
from __future__ import annotations

from typing import List, Optional, Tuple


class CacheModel:
    def __init__(self, window: int, n_sink: int = 1):
        if window < 1 or n_sink < 0:
            raise ValueError("window must be >= 1 and n_sink >= 0")
        self.window = window
        self.n_sink = n_sink
        self.reset()

    def reset(self) -> None:
        self.slots: List[Optional[int]] = [None] * (self.n_sink + self.window)
        self.fifo: List[int] = []  # window chunks, oldest first
        self.next_id = 0
        self.last_window_slot = self.n_sink + self.window - 1

    def append(self) -> Tuple[int, int, int]:
        """Append the next chunk; returns (chunk_id, slot, evicted chunk or -1)."""
        c = self.next_id
        evicted = -1
        if c < self.n_sink:
            slot = c
        else:
            slot = self.n_sink + (self.last_window_slot + 1 - self.n_sink) % self.window
            if self.slots[slot] is not None:
                evicted = self.slots[slot]
                assert self.fifo[0] == evicted
                self.fifo.pop(0)
            self.fifo.append(c)
            self.last_window_slot = slot
        self.slots[slot] = c
        self.next_id = c + 1
        return c, slot, evicted

    def evict(self, n: int) -> List[int]:
        """Drop the n oldest window chunks; returns their ids, oldest first."""
        if n < 0 or n > len(self.fifo):
            raise ValueError("cannot evict %d of %d window chunks" % (n, len(self.fifo)))
        gone = self.fifo[:n]
        self.fifo = self.fifo[n:]
        for g in gone:
            self.slots[self.slots.index(g)] = None
        return gone

    def resident(self) -> List[int]:
        """Chunk ids held by the cache, in increasing order."""
        return sorted(c for c in self.slots if c is not None)

    def slot_map(self) -> List[int]:
        """slot -> chunk id (-1 for an empty slot)."""
        return [-1 if c is None else c for c in self.slots]

    def occupancy(self) -> int:
        return sum(c is not None for c in self.slots)
