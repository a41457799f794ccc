"""The fp32 tiny-GPT shapes, rerun from scratch at every step (oracle; test infrastructure only).

Source: Tiny-GPT post, "The Cache, in Code".  One attention layer is a single
bias-free qkv projection split into three d_model-wide parts, each viewed as
(tokens, heads, head_dim); q and k are rotated at their positions and cast to
the value dtype; attention runs causally over the history; an output
projection follows.  ``CachedGPT.step`` stacks blocks as
``x += attn(norm1(x)); x += mlp(norm2(x))`` and reads logits from the final
norm of the last position.  The no-cache loop the post starts from reruns the
whole (window-trimmed) history through every block at every step ("What the
No-Cache Loop Wastes"), and that is what every function here does.

Readings where the post is silent:

* the norm is RMSNorm with unit weight and eps 1e-5; the MLP is
  d_model -> 4 d_model -> d_model with the exact (erf) GELU; no linear layer
  has a bias; the output head is tied to the embedding (logits = x @ emb^T).
  With these choices a 6-layer, d_model 256, vocab 4096 model has 5,767,168
  parameters, 23.1 MB in fp32 -- the post's "5.8M parameters" and "23 MB".
* the window: a history longer than the 256-token context is cut to its last
  256 tokens, which then sit at positions 0..255, as the post's no-cache loop
  reruns them (the configured runs never exceed the window).
"""
from __future__ import annotations

import numpy as np
from scipy.special import erf

from .attention import attend, rebuild_row


def rms_norm(x, eps: float = 1e-5) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def gelu(x) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))


def attention_layer(h, w_qkv, w_out, n_heads: int, dtype: str = "f32", base: float = 10000.0) -> np.ndarray:
    """One causal attention layer over a whole history h (n, C); returns (n, C) float64."""
    h = np.asarray(h, dtype=np.float64)
    n, c = h.shape
    d = c // n_heads
    qkv = h @ np.asarray(w_qkv, dtype=np.float64)
    q, k, v = (qkv[:, i * c:(i + 1) * c].reshape(n, n_heads, d) for i in range(3))
    q_hat, k_hat, v_r = rebuild_row(q, k, v, dtype, base)
    o = attend(q_hat, k_hat, v_r, np.arange(n))
    return o.reshape(n, c) @ np.asarray(w_out, dtype=np.float64)


def tiny_layer_nocache(x_hist, w_qkv, w_out, n_heads: int, context: int = 256,
                       dtype: str = "f32", base: float = 10000.0) -> np.ndarray:
    """Outputs (n, C) of the single layer rerun over the trimmed history x_hist (n, C)."""
    x_hist = np.asarray(x_hist, dtype=np.float64)[-context:]
    return attention_layer(x_hist, w_qkv, w_out, n_heads, dtype, base)


def tiny_gpt_logits_nocache(tokens, weights: dict, n_layers: int, n_heads: int, context: int = 256,
                            eps: float = 1e-5, base: float = 10000.0) -> np.ndarray:
    """Last-position logits (vocab,) of the tiny GPT rerun over the token history."""
    tokens = np.asarray(tokens, dtype=np.int64)[-context:]
    emb = np.asarray(weights["emb"], dtype=np.float64)
    x = emb[tokens]
    for layer in range(n_layers):
        x = x + attention_layer(rms_norm(x, eps), weights[f"qkv{layer}"], weights[f"out{layer}"],
                                n_heads, "f32", base)
        hidden = gelu(rms_norm(x, eps) @ np.asarray(weights[f"fc1{layer}"], dtype=np.float64))
        x = x + hidden @ np.asarray(weights[f"fc2{layer}"], dtype=np.float64)
    return rms_norm(x[-1], eps) @ emb.T


def greedy(logits) -> int:
    """Greedy pick: the largest logit, the lowest index on an exact tie."""
    return int(np.argmax(np.asarray(logits)))


def top2_gap(logits) -> float:
    """Gap between the largest and second-largest logit (how close a greedy pick was)."""
    s = np.sort(np.asarray(logits, dtype=np.float64))
    return float(s[-1] - s[-2])


def param_count(vocab: int, d_model: int, n_layers: int, mlp: int) -> int:
    """Parameters of the tiny GPT under the readings above (tied head, no biases, RMSNorm weights 1)."""
    per_layer = d_model * 3 * d_model + d_model * d_model + 2 * d_model * mlp
    return vocab * d_model + n_layers * per_layer
