"""Rounding into storage types (oracle; test infrastructure only).

The Tiny-GPT post casts the rotated q and k back to the value dtype before
attention ("The Cache, in Code": rope, then ``.to(v.dtype)``), so a rotated
key is rounded once into the cache's storage type.  Both storage types used
here round to nearest, ties to even.

bfloat16 keeps float32's exponent range and 8 significant bits.  A finite
float64 ``x`` with ``2^(e-1) <= |x| < 2^e`` therefore rounds on a grid of
spacing ``2^(e-8)``; below the smallest normal (2^-126) the grid spacing stays
2^-133 (subnormals).  ``numpy.rint`` rounds halves to even.
"""
from __future__ import annotations

import numpy as np

_BF16_MAX = float(np.ldexp(np.float64(0xFF), 120))  # (2 - 2^-7) * 2^127
_BF16_MIN_SPACING = 2.0 ** -133


def round_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value (ties to even); float64 out."""
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    finite = np.isfinite(x) & (x != 0)
    xf = x[finite]
    _, e = np.frexp(xf)  # xf = m * 2^e, 0.5 <= |m| < 1
    spacing = np.maximum(np.ldexp(1.0, e - 8), _BF16_MIN_SPACING)
    r = np.rint(xf / spacing) * spacing
    # Past the largest finite bfloat16 (halfway to 2^128 rounds up) the value is infinite.
    r = np.where(np.abs(r) > _BF16_MAX, np.copysign(np.inf, r), r)
    out[finite] = r
    return out


def round_f32(x) -> np.ndarray:
    """Round float64 values to the nearest float32 value (ties to even); float64 out."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_to(x, dtype: str) -> np.ndarray:
    """Round into the named storage type: ``"f32"`` or ``"bf16"``."""
    if dtype == "f32":
        return round_f32(x)
    if dtype == "bf16":
        return round_bf16(x)
    raise ValueError(f"unknown storage type {dtype!r}")


def f32_to_bf16_bits(x32) -> np.ndarray:
    """uint16 bit patterns of ``round_bf16`` applied to float32 input (for bit comparisons)."""
    r = round_bf16(np.asarray(x32, dtype=np.float32).astype(np.float64)).astype(np.float32)
    return (r.view(np.uint32) >> 16).astype(np.uint16)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """float64 values of uint16 bfloat16 bit patterns."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)
