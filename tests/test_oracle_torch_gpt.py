"""The tiny GPT oracle's block composition pinned against torch's own layers (CPU).

Tiny-GPT post, "The Cache, in Code": ``CachedGPT.step`` embeds the tokens,
runs every block as ``x += attn(norm1(x)); x += mlp(norm2(x))`` and reads the
logits of the last position through the final norm.  Here that model is put
together from torch modules in float64 -- ``nn.Embedding``, ``nn.RMSNorm``,
bias-free ``nn.Linear``, ``nn.GELU`` and ``scaled_dot_product_attention`` with
``is_causal=True`` -- and run over the whole history with no cache.  Its
logits must match ``oracle.model.tiny_gpt_logits_nocache`` to 1e-9.

Only the pair rotation is restated here (torch has no RoPE layer); it follows
the same reading as the oracle -- float32 angles f32(f32(p) * inv_freq),
half-split pairs -- and is pinned on its own by the worked example and the
identities in test_oracle_pins.  The float32 rounding points (the projected
q, k, v and the rotated q, k, as the post's float32 model holds them) are
those of the oracle.  Every other step comes from torch.

The pin must also catch a plausible slip in the composition: variants of the
torch model with post-norm blocks, a dropped residual, the tanh GELU, an
untied head, a missing final norm or heads taken in the wrong order each
disagree with the oracle by far more than the float32 gate.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F
from torch import nn

import synth
from oracle import model
from tests import gates

F64 = torch.float64


def _f32(x: torch.Tensor) -> torch.Tensor:
    """Round a float64 tensor to float32 and back (where the post's float32 model stores a value)."""
    return x.to(torch.float32).to(F64)


def _rope(x: torch.Tensor, base: float = 10000.0) -> torch.Tensor:
    """x (heads, n, D) rotated at positions 0..n-1, half-split pairs, float32 angles."""
    n, d = x.shape[1], x.shape[2]
    i = torch.arange(d // 2, dtype=F64)
    inv = torch.pow(torch.tensor(base, dtype=F64), -2.0 * i / d).to(torch.float32)
    th = (torch.arange(n, dtype=torch.float32)[:, None] * inv[None, :]).to(F64)  # float32 product
    c, s = torch.cos(th), torch.sin(th)
    a, b = x[..., : d // 2], x[..., d // 2:]
    return torch.cat([a * c - b * s, a * s + b * c], dim=-1)


class Attn(nn.Module):
    def __init__(self, w_qkv, w_out, n_heads, head_order=None):
        super().__init__()
        c = w_out.shape[0]
        self.n_heads, self.c = n_heads, c
        self.qkv = nn.Linear(c, 3 * c, bias=False, dtype=F64)
        self.out = nn.Linear(c, c, bias=False, dtype=F64)
        with torch.no_grad():  # the oracle computes h @ W; a Linear computes h @ weight^T
            self.qkv.weight.copy_(torch.from_numpy(np.asarray(w_qkv, dtype=np.float64)).T)
            self.out.weight.copy_(torch.from_numpy(np.asarray(w_out, dtype=np.float64)).T)
        self.head_order = head_order

    def forward(self, h):
        n = h.shape[0]
        q, k, v = (_f32(t).view(n, self.n_heads, -1).transpose(0, 1) for t in self.qkv(h).split(self.c, dim=-1))
        if self.head_order is not None:
            q = q[self.head_order]
        q, k = _f32(_rope(q)), _f32(_rope(k))
        o = F.scaled_dot_product_attention(q, k.contiguous(), v.contiguous(), is_causal=True)  # (heads, n, d)
        return self.out(o.transpose(0, 1).reshape(n, self.c))


class Block(nn.Module):
    def __init__(self, weights, layer, n_heads, eps, variant):
        super().__init__()
        c = weights["emb"].shape[1]
        m = weights[f"fc1{layer}"].shape[1]
        self.variant = variant
        self.norm1 = nn.RMSNorm(c, eps=eps, elementwise_affine=False, dtype=F64)
        self.norm2 = nn.RMSNorm(c, eps=eps, elementwise_affine=False, dtype=F64)
        order = torch.arange(n_heads).flip(0) if variant == "heads_reversed" else None
        self.attn = Attn(weights[f"qkv{layer}"], weights[f"out{layer}"], n_heads, order)
        self.fc1 = nn.Linear(c, m, bias=False, dtype=F64)
        self.fc2 = nn.Linear(m, c, bias=False, dtype=F64)
        self.act = nn.GELU(approximate="tanh" if variant == "gelu_tanh" else "none")
        with torch.no_grad():
            self.fc1.weight.copy_(torch.from_numpy(np.asarray(weights[f"fc1{layer}"], dtype=np.float64)).T)
            self.fc2.weight.copy_(torch.from_numpy(np.asarray(weights[f"fc2{layer}"], dtype=np.float64)).T)

    def forward(self, x):
        mlp = lambda h: self.fc2(self.act(self.fc1(h)))
        if self.variant == "post_norm":
            x = self.norm1(x + self.attn(x))
            return self.norm2(x + mlp(x))
        if self.variant == "no_attn_residual":
            x = self.attn(self.norm1(x))
            return x + mlp(self.norm2(x))
        x = x + self.attn(self.norm1(x))
        return x + mlp(self.norm2(x))


class TinyGPT(nn.Module):
    """The post's model over a whole token history, built from torch layers (float64, no cache)."""

    def __init__(self, weights, n_layers, n_heads, eps=1e-5, variant=None):
        super().__init__()
        emb = torch.from_numpy(np.asarray(weights["emb"], dtype=np.float64))
        self.emb = nn.Embedding(emb.shape[0], emb.shape[1], dtype=F64)
        with torch.no_grad():
            self.emb.weight.copy_(emb)
        self.blocks = nn.ModuleList(Block(weights, layer, n_heads, eps, variant) for layer in range(n_layers))
        self.norm = nn.RMSNorm(emb.shape[1], eps=eps, elementwise_affine=False, dtype=F64)
        self.variant = variant
        if variant == "untied_head":
            g = torch.Generator().manual_seed(5)
            self.head = torch.randn(emb.shape, generator=g, dtype=F64) * 0.02

    @torch.no_grad()
    def forward(self, tokens):
        x = self.emb(torch.as_tensor(np.asarray(tokens), dtype=torch.int64))
        for blk in self.blocks:
            x = blk(x)
        last = x[-1] if self.variant == "no_final_norm" else self.norm(x[-1])
        return F.linear(last, self.head if self.variant == "untied_head" else self.emb.weight)


def _histories():
    w = synth.TINY_GPT6
    prompt = synth.tiny_gpt_prompt(w, batch=2)
    more = synth.token_ids(w, 56, 9)
    return [prompt[0], np.concatenate([prompt[1], more[:12]]), np.concatenate([prompt[0], more])]


@pytest.fixture(scope="module")
def tiny():
    w = synth.TINY_GPT6
    return synth.tiny_gpt_weights(w), w.extra["n_layers"], w.n_q_heads


def test_oracle_logits_equal_torch_layers(tiny):
    weights, nl, nh = tiny
    gpt = TinyGPT(weights, nl, nh)
    for tokens in _histories():
        want = gpt(tokens).numpy()
        got = model.tiny_gpt_logits_nocache(tokens, weights, nl, nh)
        assert np.max(np.abs(got - want)) <= 1e-9, f"{len(tokens)} tokens"


@pytest.mark.parametrize("variant", ["post_norm", "no_attn_residual", "gelu_tanh", "untied_head",
                                     "no_final_norm", "heads_reversed"])
def test_composition_slips_are_caught(tiny, variant):
    weights, nl, nh = tiny
    bad = TinyGPT(weights, nl, nh, variant=variant)
    tokens = _histories()[1]
    got = model.tiny_gpt_logits_nocache(tokens, weights, nl, nh)
    assert not gates.passes(got, bad(tokens).numpy(), "f32"), f"{variant} agrees with the oracle"
