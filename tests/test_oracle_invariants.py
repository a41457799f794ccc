"""Invariants of the method checked on the CPU oracle, and the gate's sensitivity.

* The Tiny-GPT post's check ("Does the Cache Change the Output?"): greedy
  tokens from a cached loop equal those of the from-scratch loop inside the
  window.  The cached loop here is a small float64 re-implementation of the
  post's ``CachedGPT.step`` written in this file; the from-scratch loop is
  the oracle.
* The post's deliberate-bug runs ("Two Gotchas That Break It Quietly"): a
  RoPE offset of 0 and a top-left mask at T = 1 must be caught -- here as
  mutant oracles that fail the same gate the GPU results must pass, and on
  the tiny GPT as greedy drift.
"""
import numpy as np
import pytest

import synth
from oracle import attention as oatt
from oracle import model, numerics, rope
from tests import gates


# ------------------------------------------------------------- mutants

def _decode_variants(k_hist, v_hist, q_raw, k_raw, v_raw, dtype, group):
    """Correct decode output and four planted mistakes, for one row whose
    first P positions hold rotated keys (k_hist, v_hist: (P, Hkv, D))."""
    p = k_hist.shape[0]
    hkv = k_hist.shape[1]

    def run(q_pos_rot, k_pos_rot, n_visible, head_map):
        k_new = rope.rotate_round(numerics.round_to(k_raw[None], dtype), [k_pos_rot], dtype)
        q_new = rope.rotate_round(numerics.round_to(q_raw[None], dtype), [q_pos_rot], dtype)[0]
        k_all = np.concatenate([k_hist, k_new])[:n_visible]
        v_all = np.concatenate([v_hist, numerics.round_to(v_raw[None], dtype)])[:n_visible]
        d = q_new.shape[-1]
        out = np.empty_like(q_new)
        for h in range(q_new.shape[0]):
            g = head_map(h)
            s = k_all[:, g, :] @ q_new[h] / np.sqrt(d)
            w = np.exp(s - s.max())
            out[h] = w @ v_all[:, g, :] / w.sum()
        return out

    right = run(p, p, p + 1, lambda h: h // group)
    return right, {
        "rope_offset_zero": run(0, 0, p + 1, lambda h: h // group),
        "top_left_mask_at_T1": run(p, p, 1, lambda h: h // group),
        "length_off_by_one": run(p, p, p, lambda h: h // group),
        "head_map_modulo": run(p, p, p + 1, lambda h: h % hkv),
    }


def test_decode_variant_helper_equals_oracle():
    g = np.random.default_rng(20)
    kh = numerics.round_bf16(g.standard_normal((30, 2, 16)))
    vh = numerics.round_bf16(g.standard_normal((30, 2, 16)))
    q, k, v = g.standard_normal((8, 16)), g.standard_normal((2, 16)), g.standard_normal((2, 16))
    right, _ = _decode_variants(kh, vh, q, k, v, "bf16", 4)
    ref = oatt.decode_over_existing(kh, vh, q, k, v, "bf16")
    assert np.max(np.abs(right - ref)) <= 1e-14


@pytest.mark.parametrize("which", ["tiny_layer", "gqa"])
def test_each_mutant_fails_the_gate(which):
    """Every planted mistake moves the output past the gate on the workload's shapes."""
    if which == "tiny_layer":
        w, lengths, dtype = synth.TINY_LAYER, [8, 40, 255], "f32"
        mutants = ["rope_offset_zero", "top_left_mask_at_T1", "length_off_by_one"]  # G = 1: no head map
    else:
        w, lengths, dtype = synth.GQA_CLONE, [2000, 2100], "bf16"
        mutants = ["rope_offset_zero", "top_left_mask_at_T1", "length_off_by_one", "head_map_modulo"]
    g = np.random.default_rng(21)
    for p in lengths:
        rights, bads = [], {name: [] for name in mutants}
        for spiked in (False, True):
            kh = rope.rotate_round(numerics.round_to(g.standard_normal((p, w.n_kv_heads, w.head_dim)), dtype),
                                   np.arange(p), dtype)
            vh = numerics.round_to(g.standard_normal((p, w.n_kv_heads, w.head_dim)), dtype)
            q = g.standard_normal((w.n_q_heads, w.head_dim))
            k = g.standard_normal((w.n_kv_heads, w.head_dim))
            v = g.standard_normal((w.n_kv_heads, w.head_dim))
            if spiked:
                # the new key of every group is parallel to the group's first query: score ~ 12
                for kv in range(w.n_kv_heads):
                    qh = q[kv * w.group]
                    k[kv] = 12.0 * np.sqrt(w.head_dim) * qh / np.dot(qh, qh)
            right, bad = _decode_variants(kh, vh, q, k, v, dtype, w.group)
            rights.append(right)
            for name in mutants:
                bads[name].append(bad[name])
        # a batch holding a plain row and a spiked row, as the GPU parity inputs do
        for name in mutants:
            assert not gates.passes(np.stack(bads[name]), np.stack(rights), dtype), \
                f"{which} P={p}: {name} passes the gate"


# ------------------------------------------------------ tiny GPT cached loop

class _CachedGPT:
    """float64 cached decoding written from the Tiny-GPT post's description:
    a prefill of the prompt at start 0, then one token per step at ``pos``,
    appending each layer's rotated k and v.  ``rope_offset`` and ``decode_mask``
    switch on the post's two deliberate bugs."""

    def __init__(self, weights, n_layers, n_heads, rope_offset=True, decode_mask=False):
        self.w, self.n_layers, self.n_heads = weights, n_layers, n_heads
        self.rope_offset, self.decode_mask = rope_offset, decode_mask
        self.caches = [dict() for _ in range(n_layers)]

    def _attn(self, layer, h, start):
        n, c = h.shape
        d = c // self.n_heads
        qkv = h @ self.w[f"qkv{layer}"].astype(np.float64)
        q, k, v = (numerics.round_f32(qkv[:, i * c:(i + 1) * c]).reshape(n, self.n_heads, d) for i in range(3))
        pos = np.arange(start, start + n) if self.rope_offset else np.arange(n)
        q, k = rope.rotate_round(q, pos, "f32"), rope.rotate_round(k, pos, "f32")
        cache = self.caches[layer]
        if "k" in cache:
            k, v = np.concatenate([cache["k"], k]), np.concatenate([cache["v"], v])
        cache["k"], cache["v"] = k, v
        n_keys = k.shape[0]
        if n > 1 or not self.decode_mask:
            q_pos = np.arange(n_keys - n, n_keys)  # causal for the prompt, everything for one query
        else:
            q_pos = np.array([0])  # the bug: a top-left mask hides all but the first key
        o = oatt.attend(q, k, v, q_pos)
        return o.reshape(n, c) @ self.w[f"out{layer}"].astype(np.float64)

    def step(self, tokens, start):
        x = self.w["emb"].astype(np.float64)[tokens]
        for layer in range(self.n_layers):
            x = x + self._attn(layer, model.rms_norm(x), start)
            hid = model.gelu(model.rms_norm(x) @ self.w[f"fc1{layer}"].astype(np.float64))
            x = x + hid @ self.w[f"fc2{layer}"].astype(np.float64)
        return model.rms_norm(x[-1]) @ self.w["emb"].astype(np.float64).T


def _generate(gpt, prompt, n_steps):
    logits = gpt.step(prompt, 0)
    toks, pos = list(prompt), len(prompt)
    out_logits = [logits]
    for _ in range(n_steps):
        nxt = model.greedy(logits)
        toks.append(nxt)
        logits = gpt.step(np.array([nxt]), pos)
        out_logits.append(logits)
        pos += 1
    return toks, out_logits


@pytest.mark.slow
def test_tiny_gpt_cached_equals_nocache_greedy():
    """Same greedy tokens and logits within 1e-9 at every step (the post's cached.py check)."""
    w = synth.TINY_GPT6
    weights = synth.tiny_gpt_weights(w)
    prompt = synth.tiny_gpt_prompt(w, batch=1)[0]
    nl, nh = w.extra["n_layers"], w.n_q_heads
    toks, logits = _generate(_CachedGPT(weights, nl, nh), prompt, 24)
    for s in range(25):
        hist = np.array(toks[: len(prompt) + s])
        ref = model.tiny_gpt_logits_nocache(hist, weights, nl, nh)
        assert np.max(np.abs(logits[s] - ref)) <= 1e-9
        if s < 24:
            assert toks[len(prompt) + s] == model.greedy(ref)


@pytest.mark.slow
@pytest.mark.parametrize("bug", ["rope_offset", "decode_mask"])
def test_tiny_gpt_deliberate_bugs_are_caught(bug):
    """The post's two gotchas move the logits past the fp32 gate from the first decode step.

    The post sees them as greedy drift after a few tokens on its trained
    model.  With untrained N(0, 0.02) weights the attention's share of the
    residual stream is small and greedy tokens may hold for a while, so the
    logits -- which the GPU tests compare at 1e-5 -- are what must move.
    """
    w = synth.TINY_GPT6
    weights = synth.tiny_gpt_weights(w)
    prompt = synth.tiny_gpt_prompt(w, batch=1)[0]
    nl, nh = w.extra["n_layers"], w.n_q_heads
    good_toks, good = _generate(_CachedGPT(weights, nl, nh), prompt, 6)
    kw = {"rope_offset": False} if bug == "rope_offset" else {"decode_mask": True}
    bad = _CachedGPT(weights, nl, nh, **kw)
    bad.step(prompt, 0)
    for s in range(1, 7):  # teacher-forced with the good run's tokens
        logits = bad.step(np.array([good_toks[len(prompt) + s - 1]]), len(prompt) + s - 1)
        assert not gates.passes(logits, good[s], "f32"), f"step {s}"
