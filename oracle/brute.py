"""Pure-Python loops for tiny inputs (oracle; test infrastructure only).

The same definitions as ``rope`` and ``attention`` -- rotation at absolute
positions (Tiny-GPT post, Gotcha 1), absolute-position causal softmax
attention with GQA groups (Tiny-GPT post, Gotcha 2; nanochat post, "What the
KV cache looks like on disk"; Cake paper, Section 3) -- but written with
scalar loops, ``math`` functions and ``struct`` float32 casts instead of
vectorised numpy, so that a broadcasting, axis, mask or head-mapping mistake
in the vectorised code shows up as a disagreement.  Inputs are nested lists.
"""
from __future__ import annotations

import math
import struct


def f32(x: float) -> float:
    """Round a Python float to float32 (IEEE round to nearest even) and back."""
    return struct.unpack("f", struct.pack("f", x))[0]


def bf16(x: float) -> float:
    """Round a Python float to the nearest bfloat16 value (ties to even)."""
    if x == 0.0 or math.isinf(x) or math.isnan(x):
        return x
    _, e = math.frexp(x)
    spacing = max(2.0 ** (e - 8), 2.0 ** -133)
    return round(x / spacing) * spacing  # Python's round() takes halves to even


def to_storage(x: float, dtype: str) -> float:
    return f32(x) if dtype == "f32" else bf16(x)


def rope_vec(x, pos: int, base: float, dtype: str):
    """Rotate one head vector x (list of D floats) at position pos; rounded into dtype."""
    d = len(x)
    half = d // 2
    out = [0.0] * d
    for i in range(half):
        freq = f32(base ** (-2.0 * i / d))
        theta = f32(f32(float(pos)) * freq)
        c, s = math.cos(theta), math.sin(theta)
        a, b = x[i], x[i + half]
        out[i] = to_storage(a * c - b * s, dtype)
        out[i + half] = to_storage(a * s + b * c, dtype)
    return out


def attention_row(q_hat, k_hat, v, q_pos, scale: float):
    """q_hat[t][h][d], k_hat[j][g][d], v[j][g][d]; query t sees keys j <= q_pos[t]."""
    n_q_heads = len(q_hat[0])
    n_kv_heads = len(k_hat[0])
    group = n_q_heads // n_kv_heads
    d = len(q_hat[0][0])
    out = []
    for t in range(len(q_hat)):
        row = []
        for h in range(n_q_heads):
            g = h // group
            scores = []
            for j in range(q_pos[t] + 1):
                dot = 0.0
                for e in range(d):
                    dot += q_hat[t][h][e] * k_hat[j][g][e]
                scores.append(dot * scale)
            m = max(scores)
            weights = [math.exp(s - m) for s in scores]
            total = sum(weights)
            vec = []
            for e in range(d):
                acc = 0.0
                for j, w in enumerate(weights):
                    acc += w * v[j][g][e]
                vec.append(acc / total)
            row.append(vec)
        out.append(row)
    return out


def nocache_row(q_raw, k_raw, v_raw, q_positions, dtype: str, base: float = 10000.0):
    """Rotate the whole raw history at positions 0..n-1 and attend for the given positions."""
    d = len(k_raw[0][0])
    k_hat = [[rope_vec([to_storage(x, dtype) for x in k_raw[j][g]], j, base, dtype)
              for g in range(len(k_raw[j]))] for j in range(len(k_raw))]
    v = [[[to_storage(x, dtype) for x in v_raw[j][g]] for g in range(len(v_raw[j]))] for j in range(len(v_raw))]
    q_hat = [[rope_vec([to_storage(x, dtype) for x in q_raw[p][h]], p, base, dtype)
              for h in range(len(q_raw[p]))] for p in q_positions]
    return attention_row(q_hat, k_hat, v, list(q_positions), 1.0 / math.sqrt(d))
