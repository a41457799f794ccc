"""Rotary position embedding at absolute positions (oracle; test infrastructure only).

Source: Tiny-GPT post, "Two Gotchas That Break It Quietly", Gotcha 1.  The
angle table is the float32 product of the positions ``start .. start+T-1``
(built as float32) and a per-frequency vector; a cached step must start the
positions at the row's offset, not at 0.

Readings where the post is silent (it shows only the angle line):

* frequencies: ``inv_freq[i] = base ** (-2 i / D)`` for ``i < D/2`` with base
  10000, evaluated in float64 and rounded once to float32, the usual RoPE
  table;
* angle: one float32 product ``theta = f32(f32(p) * inv_freq[i])``, as the
  post builds it;
* pairs: dimension ``i`` rotates with dimension ``i + D/2`` ("half split");
* cos and sin of that float32 angle are taken in float64, and the rotation is
  done in float64; the caller rounds the result into the storage type.

Under these readings position 0 is the identity, the rotation preserves each
pair's length, and a query/key dot product depends only on the distance
between their positions (the post's remark under "Does the Cache Change the
Output?") -- the pins in the tests check exactly these facts.
"""
from __future__ import annotations

import numpy as np

from .numerics import round_to


def inv_freq(head_dim: int, base: float = 10000.0) -> np.ndarray:
    """float32 frequencies of length head_dim/2 (float64 pow, one rounding)."""
    if head_dim % 2:
        raise ValueError("head_dim must be even")
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(np.float64(base), -2.0 * i / head_dim).astype(np.float32)


def angles(positions, head_dim: int, base: float = 10000.0) -> np.ndarray:
    """float32 angle table (n_positions, head_dim/2): f32(f32(p) * inv_freq)."""
    p = np.asarray(positions, dtype=np.int64).astype(np.float32)
    return p[:, None] * inv_freq(head_dim, base)[None, :]  # float32 * float32 -> float32


def rotate(x, positions, base: float = 10000.0) -> np.ndarray:
    """Rotate x (n, heads, D) at positions (n,), float64 result, no rounding.

    Every head of token t uses the angle row of positions[t].
    """
    x = np.asarray(x, dtype=np.float64)
    n, _, d = x.shape
    half = d // 2
    th = angles(positions, d, base).astype(np.float64)  # (n, half)
    c = np.cos(th)[:, None, :]
    s = np.sin(th)[:, None, :]
    a = x[..., :half]
    b = x[..., half:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def rotate_round(x, positions, dtype: str, base: float = 10000.0) -> np.ndarray:
    """``rotate`` then one round-to-nearest-even into the storage type."""
    return round_to(rotate(x, positions, base), dtype)
