"""The OCP 8-bit float format E4M3 ("E4M3FN") and per-block quantisation.

The pages say the DiT runs in FP8 (JoyAI-Video-Edit tutorial,
agifrontier.github.io, section "Hardware-software co-deployment", bullet on
mixed precision; neurohive.io review, section "Where 30 FPS comes from") but
give neither the format nor the scaling.  Reading used here: the OCP E4M3
format (the e4m3 type of the OCP 8-bit floating point specification) with one
float32 scale per (head, chunk) block, scale = amax / 448 (1 when amax is 0).

E4M3 bit layout: sign (1), exponent (4, bias 7), mantissa (3).
* exponent field 0: subnormal, value = (-1)^s * 2^-6 * m/8
* exponent field 1..15: normal, value = (-1)^s * 2^(e-7) * (1 + m/8)
* exponent 15 with mantissa 7 is NaN (no infinities); the largest finite
  magnitude is 448 (exponent 15, mantissa 6).

Encoding rounds to the nearest representable value, ties to the code with an
even mantissa (its lowest bit 0), and saturates to +-448.  The quotient
x / scale is taken in float32, as the device does.

Parity: pinned (exhaustive decode of all 256 codes against the format's
definition, tie and saturation cases, round trip of every finite code).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def decode(codes: np.ndarray) -> np.ndarray:
    """float64 value of each E4M3 code (NaN for the two NaN codes)."""
    c = np.asarray(codes, dtype=np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    sub = np.ldexp(m / 8.0, -6)
    nrm = np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))
    val = sign * np.where(e == 0, sub, nrm)
    return np.where((e == 15) & (m == 7), np.nan, val)


def _positive_table():
    codes = np.arange(0, 0x7F, dtype=np.int64)  # 0x00 .. 0x7E, all finite, increasing
    return codes, decode(codes)


def encode(x: np.ndarray) -> np.ndarray:
    """Nearest E4M3 code (ties to even mantissa), saturating at +-448.

    ``x`` must be finite.  -0.0 encodes as 0x80, +0.0 as 0x00.
    """
    x = np.asarray(x, dtype=np.float64)
    if not np.isfinite(x).all():
        raise ValueError("encode expects finite values")
    codes, vals = _positive_table()
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(vals, a, side="left")  # first table value >= a
    hi = np.minimum(hi, len(vals) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - vals[lo]
    d_hi = vals[hi] - a
    pick_hi = d_hi < d_lo
    tie = d_hi == d_lo
    even_hi = (codes[hi] & 1) == 0
    pick_hi = pick_hi | (tie & even_hi)
    exact = vals[hi] == a
    mag = np.where(exact | pick_hi, codes[hi], codes[lo])
    neg = np.signbit(x)
    return (mag | np.where(neg, 0x80, 0)).astype(np.uint8)


def block_scale(block: np.ndarray) -> np.float32:
    """float32 scale of one block: amax / 448, or 1 for an all-zero block."""
    amax = np.float32(np.max(np.abs(np.asarray(block, dtype=np.float32))))
    if amax == 0:
        return np.float32(1.0)
    return np.float32(amax / np.float32(E4M3_MAX))


def quantize_block(block: np.ndarray):
    """(codes uint8, scale float32) of one block; codes = encode(x / scale)."""
    x = np.asarray(block, dtype=np.float32)
    s = block_scale(x)
    y = (x / s).astype(np.float32)  # float32 quotient
    return encode(y), s


def quantize_heads(x: np.ndarray):
    """Per-head quantisation of [H][N][D]: codes [H][N][D], scales [H]."""
    codes = np.empty(x.shape, dtype=np.uint8)
    scales = np.empty(x.shape[0], dtype=np.float32)
    for h in range(x.shape[0]):
        codes[h], scales[h] = quantize_block(x[h])
    return codes, scales


def dequantize_heads(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """float64 values code * scale, per head."""
    return decode(codes) * np.asarray(scales, dtype=np.float64)[:, None, None]
