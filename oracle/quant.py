"""8-bit KV cache quantization (oracle; test infrastructure only).

Cake paper, Section 5.1 ("Compression methods") and Section 5.5 with Table 6:
the KV cache is compressed with the common 8-bit quantization, which shrinks
the bytes to move.  The pages fix no scheme.  Read here as the plainest
symmetric one:

* one scale per cached vector, that is per (layer, row, position, KV head):
  the head_dim values the attention reads together;
* scale s = amax / 127 in float32, where amax is the vector's largest |x|;
* code c_i = x_i / s rounded to the nearest integer (ties to even), in
  [-127, 127];
* dequantized value c_i * s.

An all-zero vector has s = 0 and codes 0.  The quotient and the scale are
float32 operations, correctly rounded, because the codes are integers that a
float decides.  The GPU side must take the same decision in the same
precision, so the oracle does them in float32, and the attention on
dequantized values in float64.

What is quantized is what the bfloat16 cache would hold: the rotated key
rounded to bfloat16, and the value rounded to bfloat16.
"""
from __future__ import annotations

import numpy as np

QMAX = 127


def quantize_int8(x):
    """Per-vector symmetric int8 along the last axis.

    x: float values, exactly representable in float32 (bfloat16 values are).
    Returns (codes int8 of x's shape, scales float32 of x.shape[:-1]).
    """
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    if not np.array_equal(x32.astype(np.float64), np.asarray(x, dtype=np.float64)):
        raise ValueError("quantize_int8 expects float32-exact inputs")
    amax = np.max(np.abs(x32), axis=-1)
    scale = (amax / np.float32(QMAX)).astype(np.float32)  # float32 division, correctly rounded
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    q = (x32 / safe[..., None]).astype(np.float32)  # float32 quotient
    codes = np.clip(np.rint(q), -QMAX, QMAX)  # rint: half to even
    codes = np.where(scale[..., None] > 0, codes, 0.0).astype(np.int8)
    return codes, scale


def dequantize_int8(codes, scales) -> np.ndarray:
    """codes * scale per vector, float64 (exact: an int8 times a float32 fits float64)."""
    return np.asarray(codes, dtype=np.float64) * np.asarray(scales, dtype=np.float64)[..., None]


def appended_slots_int8(k_raw, v_raw, start: int, base: float = 10000.0):
    """What an append into an int8 cache writes for one row's T tokens at start..start+T-1.

    k_raw, v_raw: (T, Hkv, D) raw values.  The key is rotated at its position
    and rounded to bfloat16, the value rounded to bfloat16 (what a bfloat16
    cache would hold), and each (token, head) vector is then quantized.
    Returns (k_codes, k_scales, v_codes, v_scales).
    """
    from .attention import appended_slots
    k_hat, v_hat = appended_slots(k_raw, v_raw, start, "bf16", base)
    kc, ks = quantize_int8(k_hat)
    vc, vs = quantize_int8(v_hat)
    return kc, ks, vc, vs


def decode_over_int8(k_codes, k_scales, v_codes, v_scales, q_raw, k_raw, v_raw, base: float = 10000.0,
                     scale: float | None = None, position: int | None = None) -> np.ndarray:
    """One decode token over a row's stored int8 history.

    k_codes/v_codes (n, Hkv, D), k_scales/v_scales (n, Hkv): the stored
    (already rotated) history.  q_raw (Hq, D), k_raw/v_raw (Hkv, D): the new
    token at absolute position `position` (default n: a linear cache holding
    positions 0..n-1), whose key and value are quantized as the append stores
    them.  The query is rotated and rounded to bfloat16 only.  Attention in
    float64 over the dequantized keys and values.  Returns (Hq, D).
    """
    from .attention import attend
    from .numerics import round_to
    from .rope import rotate_round
    p = np.asarray(k_codes).shape[0] if position is None else int(position)
    kc, ks, vc, vs = appended_slots_int8(np.asarray(k_raw)[None], np.asarray(v_raw)[None], p, base)
    k_all = np.concatenate([dequantize_int8(k_codes, k_scales), dequantize_int8(kc, ks)], axis=0)
    v_all = np.concatenate([dequantize_int8(v_codes, v_scales), dequantize_int8(vc, vs)], axis=0)
    q_hat = rotate_round(round_to(np.asarray(q_raw)[None], "bf16"), [p], "bf16", base)
    return attend(q_hat, k_all, v_all, [k_all.shape[0] - 1], scale)[0]
