"""Seeded synthetic inputs for block-causal sink + sliding-window attention.

This module is the only code shared by the oracle side (``oracle/``) and the
device side (``block_causal_kv_amd``).  It draws random numbers and rounds them
to the storage precision of the workload; it holds none of the method's
arithmetic (no masks, no softmax, no cache bookkeeping, no quantisation).

Recipe (stated once, used everywhere):

* Every tensor is a float32 draw from ``numpy.random.default_rng`` (PCG64)
  ``standard_normal``, then rounded to bfloat16 with round-to-nearest-even
  (``to_bf16``), so the oracle and the GPU see the same values.
* Streams are addressed by ``(seed, part)``: the condition tokens use part 0,
  chunk ``c`` uses part ``c + 1``.  Any chunk can therefore be regenerated on
  its own, without drawing the chunks before it.
* Per chunk the draw order is: first the clean ``k_clean, v_clean`` that are
  written to the cache after the chunk is generated, then for each denoise
  step ``s`` the tensors ``q_s, k_s, v_s``.  With ``clean_from_last_step=True``
  no clean tensors are drawn and the last step's K/V are the clean K/V.
* Optional outliers: each (head, token) row of every K tensor is scaled by
  ``outlier_scale`` with probability ``outlier_frac`` (a Bernoulli drawn from the
  same generator right after the K tensor), before the bf16 rounding.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np


def to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns float32 values that are exactly representable in bfloat16.
    Inputs here are finite normal draws, so no NaN handling is needed.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # finite inputs cannot carry past bit 31: the largest finite pattern is 0xFF7FFFFF
    u = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) & np.uint32(0xFFFF0000)
    return u.view(np.float32).reshape(x.shape)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """The uint16 bit patterns of bfloat16-representable float32 values."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


@dataclass(frozen=True)
class StreamSpec:
    """Shapes of one synthetic stream (the problem statement's parameters)."""

    name: str
    n_chunks: int
    chunk_tokens: int  # T = source tokens + target tokens
    cond_len: int  # Lc, condition tokens
    heads: int
    head_dim: int
    window: int  # W recent history chunks
    n_sink: int = 1
    steps: int = 1  # attention calls (denoise steps) per chunk
    seed: int = 0
    outlier_frac: float = 0.0
    outlier_scale: float = 8.0
    clean_from_last_step: bool = True
    kv_dtype: str = "bf16"  # "bf16" or "fp8"

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim))

    def steady_kv_len(self) -> int:
        return self.cond_len + self.chunk_tokens * (self.n_sink + self.window + 1)


# The workloads: tiny and mid are the streams the oracle finishes quickly; the
# 720p-shaped stream has 2 x (45 x 40) latent tokens per chunk.
SPECS: Dict[str, StreamSpec] = {
    "tiny": StreamSpec("tiny", 6, 64, 16, 2, 64, 2, seed=0),
    "mid": StreamSpec("mid", 12, 1024, 128, 16, 128, 3, seed=1),
    "720p": StreamSpec("720p", 30, 3600, 256, 24, 128, 4, steps=2, seed=2,
                       outlier_frac=0.01, clean_from_last_step=False),
    "long": StreamSpec("long", 300, 3600, 256, 32, 128, 8, steps=2, seed=3,
                       outlier_frac=0.01, clean_from_last_step=False),
    "fp8": StreamSpec("fp8", 30, 3600, 256, 24, 128, 4, steps=2, seed=2,
                      outlier_frac=0.01, clean_from_last_step=False, kv_dtype="fp8"),
}


def _draw(rng: np.random.Generator, shape, is_key: bool, spec: StreamSpec) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if is_key and spec.outlier_frac > 0.0:
        rows = rng.random(size=shape[:-1]) < spec.outlier_frac
        x[rows] *= np.float32(spec.outlier_scale)
    return to_bf16(x)


def cond_inputs(spec: StreamSpec, heads: Optional[int] = None):
    """Condition-token K and V, each [H][Lc][D] float32 (bf16 values)."""
    h = spec.heads if heads is None else heads
    rng = np.random.default_rng((spec.seed, 0))
    shape = (h, spec.cond_len, spec.head_dim)
    k = _draw(rng, shape, True, spec)
    v = _draw(rng, shape, False, spec)
    return k, v


@dataclass
class ChunkInputs:
    q: List[np.ndarray] = field(default_factory=list)  # per step [H][T][D]
    k: List[np.ndarray] = field(default_factory=list)
    v: List[np.ndarray] = field(default_factory=list)
    k_clean: Optional[np.ndarray] = None
    v_clean: Optional[np.ndarray] = None


def chunk_inputs(spec: StreamSpec, c: int, heads: Optional[int] = None,
                 clean_only: bool = False) -> ChunkInputs:
    """Inputs of chunk ``c`` (float32 arrays holding bf16 values).

    ``clean_only`` stops after the clean K/V (streams whose clean K/V are drawn
    separately); the values drawn are the same as in a full call.
    """
    h = spec.heads if heads is None else heads
    rng = np.random.default_rng((spec.seed, c + 1))
    shape = (h, spec.chunk_tokens, spec.head_dim)
    out = ChunkInputs()
    if not spec.clean_from_last_step:
        out.k_clean = _draw(rng, shape, True, spec)
        out.v_clean = _draw(rng, shape, False, spec)
        if clean_only:
            return out
    for _ in range(spec.steps):
        out.q.append(_draw(rng, shape, False, spec))
        out.k.append(_draw(rng, shape, True, spec))
        out.v.append(_draw(rng, shape, False, spec))
    if spec.clean_from_last_step:
        out.k_clean, out.v_clean = out.k[-1], out.v[-1]
    return out


def small_spec(name: str, **kw) -> StreamSpec:
    """A custom stream (tests use it for edge cases: ragged T, Lc = 0, W = 1 ...)."""
    return StreamSpec(name=name, **kw)
