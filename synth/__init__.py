"""Seeded synthetic inputs for attention against a KV cache.

This module is shared by the oracle side and the GPU side, and it is the only
thing they share.  It draws random numbers and fixes shapes; it holds none of
the method's arithmetic (no rotation, no rounding to bfloat16, no attention).
Every array it returns is float32 (or int), and each side converts it to its
storage type itself.

Every draw comes from its own numpy ``Generator(PCG64(SeedSequence(path)))``
where ``path`` is ``[workload seed, role, index...]``, so an array never
depends on which other arrays were drawn before it or in what order.

The workloads mirror the shapes of the three pages:

* ``tiny_layer_fp32`` -- the single-layer fp32 attention of the Tiny-GPT
  inference post ("The Cache, in Code"): d_model 256, 4 heads of 64, a
  256-token context, an 8-token random prompt, weights N(0, 0.02).
* ``tiny_gpt6_fp32`` -- the same layer stacked six deep with pre-norm RMSNorm,
  a 4x GELU MLP and a 4096-token vocabulary, batch 16 (the post's benchmark
  setting, "The Benchmark": untrained weights, greedy, fp32).
* ``gqa_prompt_clone_bf16`` -- one 2000-token prompt prefilled at batch 1 and
  cloned to 8 rows (the nanochat post, "The prefill trick, 12 lines" and its
  cost table), GQA 16 q heads over 4 kv heads, head_dim 128.
* ``ragged_decode_b64_bf16`` -- batch 64 decode over ragged cached lengths
  1..32768, 64 q / 8 kv heads (LLaMA 3.1-70B's head counts, Cake paper
  Table 1), one new token per row.
* ``long_context_72k_bf16`` -- a 73,728-token random sequence (the Cake
  paper's 72K-token input, Section 1), chunked prefill in 4096-token chunks
  (Section 3, "Chunk Prefill"), then decode at batch 1 and batch 8.

The datasets the Cake paper evaluates on are not used: the paper itself notes
that only the token length matters for its measurements (Section 5.1), so
N(0, 1) activations of the stated lengths stand in for them.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# Roles: the second element of every seed path.
_ROLE_WEIGHTS = 1
_ROLE_PROMPT = 2
_ROLE_STEP = 3
_ROLE_LENGTHS = 4
_ROLE_POOL = 5
_ROLE_OFFSETS = 6
_ROLE_NEW = 7
_ROLE_TOKENS = 8
_ROLE_CHUNK = 9


def generator(*path: int) -> np.random.Generator:
    """A fresh generator for one seed path (all path entries are ints >= 0)."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(p) for p in path])))


def normal(shape, std: float, *path: int) -> np.ndarray:
    """float32 N(0, std^2) array of ``shape`` from the seed path."""
    g = generator(*path)
    a = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    dtype: str  # "f32" or "bf16": the storage type of q, k, v, out and the cache
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    max_seq: int
    rope_base: float = 10000.0
    extra: dict = field(default_factory=dict)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads


TINY_LAYER = Workload("tiny_layer_fp32", 1, "f32", 4, 4, 64, 256,
                      extra=dict(batch=1, d_model=256, prompt=8, steps=248, w_std=0.02))
TINY_GPT6 = Workload("tiny_gpt6_fp32", 2, "f32", 4, 4, 64, 256,
                     extra=dict(batch=16, d_model=256, prompt=8, steps=248, n_layers=6,
                                vocab=4096, mlp=1024, w_std=0.02, rms_eps=1e-5))
GQA_CLONE = Workload("gqa_prompt_clone_bf16", 3, "bf16", 16, 4, 128, 4096,
                     extra=dict(prompt=2000, n_rows=8, steps=256))
RAGGED_DECODE = Workload("ragged_decode_b64_bf16", 4, "bf16", 64, 8, 128, 33024,
                         extra=dict(batch=64, len_max=32768, logical_layers=80,
                                    physical_layers=2, pool_values=1 << 26))
LONG_CONTEXT = Workload("long_context_72k_bf16", 5, "bf16", 64, 8, 128, 74240,
                        extra=dict(context=73728, chunk=4096, steps=512, clone_rows=8))

WORKLOADS = {w.name: w for w in (TINY_LAYER, TINY_GPT6, GQA_CLONE, RAGGED_DECODE, LONG_CONTEXT)}


# --------------------------------------------------------------------------
# Tiny single layer (fp32): projection weights and the per-token inputs x_t.
# --------------------------------------------------------------------------

def tiny_layer_weights(w: Workload = TINY_LAYER):
    """(W_qkv (C, 3C), W_out (C, C)), float32 N(0, 0.02^2); y = x @ W."""
    c = w.extra["d_model"]
    s = w.extra["w_std"]
    return normal((c, 3 * c), s, w.seed, _ROLE_WEIGHTS, 0), normal((c, c), s, w.seed, _ROLE_WEIGHTS, 1)


def tiny_layer_inputs(w: Workload = TINY_LAYER, batch: int | None = None):
    """x of shape (batch, prompt + steps, C), float32 N(0, 1), one stream per row."""
    b = w.extra["batch"] if batch is None else batch
    n = w.extra["prompt"] + w.extra["steps"]
    return np.stack([normal((n, w.extra["d_model"]), 1.0, w.seed, _ROLE_PROMPT, r) for r in range(b)])


# --------------------------------------------------------------------------
# Six-layer tiny GPT (fp32): weights and prompt token ids.
# --------------------------------------------------------------------------

def tiny_gpt_weights(w: Workload = TINY_GPT6):
    """dict: emb (V, C) and per layer qkv (C, 3C), out (C, C), fc1 (C, 4C), fc2 (4C, C)."""
    c, v, m, s = w.extra["d_model"], w.extra["vocab"], w.extra["mlp"], w.extra["w_std"]
    out = {"emb": normal((v, c), s, w.seed, _ROLE_WEIGHTS, 0, 0)}
    for layer in range(w.extra["n_layers"]):
        out[f"qkv{layer}"] = normal((c, 3 * c), s, w.seed, _ROLE_WEIGHTS, 1 + layer, 0)
        out[f"out{layer}"] = normal((c, c), s, w.seed, _ROLE_WEIGHTS, 1 + layer, 1)
        out[f"fc1{layer}"] = normal((c, m), s, w.seed, _ROLE_WEIGHTS, 1 + layer, 2)
        out[f"fc2{layer}"] = normal((m, c), s, w.seed, _ROLE_WEIGHTS, 1 + layer, 3)
    return out


def tiny_gpt_prompt(w: Workload = TINY_GPT6, batch: int | None = None):
    """(batch, prompt) int64 token ids uniform in [0, vocab)."""
    b = w.extra["batch"] if batch is None else batch
    g = generator(w.seed, _ROLE_TOKENS, 0)
    return g.integers(0, w.extra["vocab"], size=(b, w.extra["prompt"]), dtype=np.int64)


def token_ids(w: Workload, n: int, *path: int):
    """n int64 token ids uniform in [0, vocab) from a seed path (teacher forcing)."""
    return generator(w.seed, _ROLE_TOKENS, 1, *path).integers(0, w.extra["vocab"], size=n, dtype=np.int64)


# --------------------------------------------------------------------------
# Direct q/k/v activations (bf16 workloads): N(0, 1) float32.
# --------------------------------------------------------------------------

def qkv_tokens(w: Workload, n_tokens: int, *path: int):
    """(q (n, Hq, D), k (n, Hkv, D), v (n, Hkv, D)) float32 N(0, 1) for one row/segment."""
    d = w.head_dim
    return (normal((n_tokens, w.n_q_heads, d), 1.0, w.seed, _ROLE_NEW, 0, *path),
            normal((n_tokens, w.n_kv_heads, d), 1.0, w.seed, _ROLE_NEW, 1, *path),
            normal((n_tokens, w.n_kv_heads, d), 1.0, w.seed, _ROLE_NEW, 2, *path))


def prompt_qkv(w: Workload, n_tokens: int | None = None):
    """The single prompt's raw (unrotated) q, k, v: path (PROMPT, 0)."""
    n = w.extra["prompt"] if n_tokens is None else n_tokens
    return qkv_tokens(w, n, _ROLE_PROMPT, 0)


def chunk_qkv(w: Workload, chunk: int, n_tokens: int):
    """Raw q, k, v of prefill chunk ``chunk`` of the long sequence."""
    return qkv_tokens(w, n_tokens, _ROLE_CHUNK, chunk)


def chunk_kv(w: Workload, chunk: int, n_tokens: int):
    """Only k, v of prefill chunk ``chunk`` (the same arrays chunk_qkv returns)."""
    d = w.head_dim
    return (normal((n_tokens, w.n_kv_heads, d), 1.0, w.seed, _ROLE_NEW, 1, _ROLE_CHUNK, chunk),
            normal((n_tokens, w.n_kv_heads, d), 1.0, w.seed, _ROLE_NEW, 2, _ROLE_CHUNK, chunk))


def decode_qkv(w: Workload, step: int, row: int):
    """Raw q (1, Hq, D), k, v (1, Hkv, D) of decode step ``step`` for batch row ``row``."""
    return qkv_tokens(w, 1, _ROLE_STEP, step, row)


def decode_qkv_batch(w: Workload, step: int, rows: int):
    """Stacked decode_qkv over rows: q (rows, 1, Hq, D), k, v (rows, 1, Hkv, D)."""
    parts = [decode_qkv(w, step, r) for r in range(rows)]
    return tuple(np.stack([p[i] for p in parts]) for i in range(3))


# --------------------------------------------------------------------------
# Ragged batch decode: lengths and a pooled cache fill.
# --------------------------------------------------------------------------

def ragged_lengths(w: Workload = RAGGED_DECODE, batch: int | None = None):
    """int32 cached lengths P_b uniform in [1, len_max] (tokens already in each row)."""
    b = w.extra["batch"] if batch is None else batch
    return generator(w.seed, _ROLE_LENGTHS, 0).integers(1, w.extra["len_max"] + 1, size=b).astype(np.int32)


def ragged_pool(w: Workload = RAGGED_DECODE):
    """A pool of float32 N(0, 1) values that pre-existing cache rows are cut from.

    Filling tens of GB of cache with independent draws would dominate every
    run, so each (layer slice, row, K or V) takes one contiguous window of this
    pool; the window offsets are drawn by ``ragged_offsets``.
    """
    return normal((w.extra["pool_values"],), 1.0, w.seed, _ROLE_POOL, 0)


def ragged_offsets(w: Workload = RAGGED_DECODE, batch: int | None = None):
    """int64 offsets (physical_layers, batch, 2) of each row's K and V window in the pool.

    A window holds ``len_max * Hkv * D`` values, the most any row needs.
    """
    b = w.extra["batch"] if batch is None else batch
    span = w.extra["len_max"] * w.n_kv_heads * w.head_dim
    hi = w.extra["pool_values"] - span
    g = generator(w.seed, _ROLE_OFFSETS, 0)
    return g.integers(0, hi + 1, size=(w.extra["physical_layers"], b, 2), dtype=np.int64)


def ragged_new_qkv(w: Workload, logical_layer: int, batch: int | None = None):
    """New raw q (B, 1, Hq, D), k, v (B, 1, Hkv, D) for one logical layer's decode call."""
    b = w.extra["batch"] if batch is None else batch
    d = w.head_dim
    return (normal((b, 1, w.n_q_heads, d), 1.0, w.seed, _ROLE_STEP, 0, logical_layer),
            normal((b, 1, w.n_kv_heads, d), 1.0, w.seed, _ROLE_STEP, 1, logical_layer),
            normal((b, 1, w.n_kv_heads, d), 1.0, w.seed, _ROLE_STEP, 2, logical_layer))
