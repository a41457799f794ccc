"""Attention against a KV cache, defined without a cache (oracle; test infrastructure only).

Sources:

* The attention itself: softmax(Q K^T / sqrt(d_k)) V with d_k the key (head)
  dimension -- Cake paper, Section 3 "Background" (the printed equation is
  lost in the page's text; its surrounding sentence names d_k), and the
  default scale of the scaled-dot-product call in the Tiny-GPT post, "The
  Cache, in Code".
* Visibility: the Tiny-GPT post's Gotcha 2 -- one new query sees the whole
  cache, several prompt queries see a causal triangle.  Read here as
  absolute-position causality: key j is visible to a query at absolute
  position p exactly when j <= p.  That reading equals the post's rule at
  start 0 and at T = 1, and it is what chunked prefill needs, where each chunk
  attends to every earlier token (Cake paper, Section 3 "Chunk Prefill";
  Section 4, Figure 4's growing per-chunk cost).
* GQA: several query heads share one KV head, and the cache holds only the
  KV heads (nanochat post, "What the KV cache looks like on disk").  Read as
  contiguous groups: query head h uses KV head h // (Hq / Hkv).
* No cache: the reference computation reruns every earlier token at every
  step (Tiny-GPT post, "What the No-Cache Loop Wastes"), so the oracle
  rebuilds every rotated key from the raw, unrotated history each time it is
  called and never reuses a value from an earlier call.
* Clone: copy positions [0, P) of every layer of the batch-1 cache into every
  row of an empty batch-N cache and set every row's length to P (nanochat
  post, "The prefill trick, 12 lines").

All arithmetic is float64; ``numpy.matmul`` is the only library routine on
the value path.
"""
from __future__ import annotations

import math

import numpy as np

from .numerics import round_to
from .rope import rotate_round


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)


def attend(q_hat, k_hat, v, q_pos, scale: float | None = None) -> np.ndarray:
    """Softmax attention of one batch row.

    q_hat: (T, Hq, D) rotated queries; k_hat, v: (L, Hkv, D) the row's keys
    and values at positions 0..L-1; q_pos: (T,) absolute query positions.
    Key j is visible to query t iff j <= q_pos[t].  Returns (T, Hq, D) float64.
    """
    q_hat = np.asarray(q_hat, dtype=np.float64)
    k_hat = np.asarray(k_hat, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    t_len, hq, d = q_hat.shape
    n_keys, hkv, _ = k_hat.shape
    if hq % hkv:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    if np.any(q_pos >= n_keys) or np.any(q_pos < 0):
        raise ValueError("a query position has no key at its own position")
    group = hq // hkv
    if scale is None:
        scale = default_scale(d)
    visible = np.arange(n_keys)[None, :] <= q_pos[:, None]  # (T, L)
    out = np.empty((t_len, hq, d), dtype=np.float64)
    for h in range(hq):
        g = h // group
        s = (q_hat[:, h, :] @ k_hat[:, g, :].T) * scale
        s = np.where(visible, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        p = np.exp(s - m)  # exp(-inf) = 0 on hidden keys
        out[:, h, :] = (p @ v[:, g, :]) / p.sum(axis=1, keepdims=True)
    return out


def rebuild_row(q_raw, k_raw, v_raw, dtype: str, base: float = 10000.0):
    """Rotated, rounded q/k and rounded v of a whole history at positions 0..n-1.

    q_raw (n, Hq, D), k_raw/v_raw (n, Hkv, D): raw (unrotated) values.  Each
    is rounded into the storage type once: v directly, q and k after rotation.
    """
    n = k_raw.shape[0]
    pos = np.arange(n)
    q_hat = None if q_raw is None else rotate_round(round_to(q_raw, dtype), pos[: q_raw.shape[0]], dtype, base)
    k_hat = rotate_round(round_to(k_raw, dtype), pos, dtype, base)
    v = round_to(v_raw, dtype)
    return q_hat, k_hat, v


def nocache_outputs(q_raw, k_raw, v_raw, query_positions, dtype: str,
                    base: float = 10000.0, scale: float | None = None) -> np.ndarray:
    """No-cache attention outputs of selected positions of one row.

    The history is the raw q/k/v of tokens 0..n-1.  Every key is rotated
    from scratch at its position; the queries at ``query_positions`` attend
    to keys 0..p.  Returns (len(query_positions), Hq, D) float64.
    """
    query_positions = np.asarray(query_positions, dtype=np.int64)
    n = int(query_positions.max()) + 1
    k_raw = k_raw[:n]
    v_raw = v_raw[:n]
    _, k_hat, v = rebuild_row(None, k_raw, v_raw, dtype, base)
    q_sel = round_to(np.asarray(q_raw, dtype=np.float64)[query_positions], dtype)
    q_hat = rotate_round(q_sel, query_positions, dtype, base)
    return attend(q_hat, k_hat, v, query_positions, scale)


def decode_over_existing(k_cached, v_cached, q_raw, k_raw, v_raw, dtype: str,
                         base: float = 10000.0, scale: float | None = None) -> np.ndarray:
    """One decode token over a row whose first P positions already hold rotated keys.

    k_cached, v_cached: (P, Hkv, D) stored values (taken as already rotated);
    q_raw (Hq, D), k_raw/v_raw (Hkv, D): the new token, placed at position P.
    Returns (Hq, D) float64.
    """
    p = k_cached.shape[0]
    k_new = rotate_round(round_to(k_raw[None], dtype), [p], dtype, base)
    q_new = rotate_round(round_to(q_raw[None], dtype), [p], dtype, base)
    k_all = np.concatenate([np.asarray(k_cached, dtype=np.float64), k_new], axis=0)
    v_all = np.concatenate([np.asarray(v_cached, dtype=np.float64), round_to(v_raw[None], dtype)], axis=0)
    return attend(q_new, k_all, v_all, [p], scale)[0]


def appended_slots(k_raw, v_raw, start: int, dtype: str, base: float = 10000.0):
    """What an append writes for one row: rotated, rounded k and rounded v at start..start+T-1."""
    pos = np.arange(start, start + k_raw.shape[0])
    return rotate_round(round_to(k_raw, dtype), pos, dtype, base), round_to(v_raw, dtype)


def clone_cache(k_src, v_src, src_len: int, k_dst, v_dst):
    """The batch-1 -> batch-N clone on numpy arrays (layers, batch, max_seq, Hkv, D).

    Preconditions follow the post's asserts: source batch 1, same layer and
    head and head_dim counts, destination max_seq at least the source's.
    Positions >= src_len of the destination are left as they were.
    Returns (k, v, seqlens) of the destination.
    """
    if k_src.shape[1] != 1:
        raise ValueError("source batch must be 1")
    if k_src.shape[0] != k_dst.shape[0] or k_src.shape[3:] != k_dst.shape[3:]:
        raise ValueError("layer/head/head_dim mismatch")
    if k_dst.shape[2] < k_src.shape[2]:
        raise ValueError("destination max_seq smaller than the source's")
    k = np.array(k_dst, copy=True)
    v = np.array(v_dst, copy=True)
    for b in range(k.shape[1]):
        k[:, b, :src_len] = k_src[:, 0, :src_len]
        v[:, b, :src_len] = v_src[:, 0, :src_len]
    return k, v, np.full(k.shape[1], src_len, dtype=np.int32)


def cache_bytes(n_layers: int, tokens: int, n_kv_heads: int, head_dim: int, bytes_per_value: int,
                batch: int = 1) -> int:
    """Bytes of a K+V cache: 2 x layers x tokens x (kv heads x head_dim) x bytes x batch.

    The Tiny-GPT post's formula ("What the Cache Costs in Memory") with its
    d_model read as n_kv_heads * head_dim, which is what a GQA cache holds
    (nanochat post, "What the KV cache looks like on disk").
    """
    return 2 * n_layers * tokens * n_kv_heads * head_dim * bytes_per_value * batch


def prefill_units(prompt_len: int, n_samples: int, clone: bool) -> int:
    """The nanochat post's prefill cost units: N x prompt^2 naive, 1 x prompt^2 with the clone."""
    return (1 if clone else n_samples) * prompt_len * prompt_len


def window_outputs(q_raw, k_raw, v_raw, query_positions, window: int, dtype: str,
                   base: float = 10000.0, scale: float | None = None) -> np.ndarray:
    """No-cache attention of selected positions over a sliding window of positions.

    Tiny-GPT post, "The Cache, in Code" and "Does the Cache Change the Output?":
    the rolling cache keeps the last `window` positions, each rotated at its
    absolute position, and the query at position p attends keys
    max(0, p + 1 - window) .. p.  Every key is re-rotated here from its raw
    value at its absolute position.  Returns (len(query_positions), Hq, D).
    """
    query_positions = np.asarray(query_positions, dtype=np.int64)
    outs = []
    for p in query_positions:
        lo = max(0, int(p) + 1 - window)
        pos = np.arange(lo, int(p) + 1)
        k_hat = rotate_round(round_to(np.asarray(k_raw, dtype=np.float64)[lo:p + 1], dtype), pos, dtype, base)
        v = round_to(np.asarray(v_raw, dtype=np.float64)[lo:p + 1], dtype)
        q_hat = rotate_round(round_to(np.asarray(q_raw, dtype=np.float64)[p][None], dtype), [int(p)], dtype, base)
        outs.append(attend(q_hat, k_hat, v, [len(pos) - 1], scale)[0])
    return np.stack(outs)
