"""The fused single-launch decode step (kvc_decode_step) against the oracle (GPU).

One call does what kvc_rope_append (T = 1) followed by kvc_attn_decode does:
the outputs must meet the oracle's gates, the K/V bytes it writes must be
those kvc_rope_append writes, and a whole tiny-GPT decode step built on it
must replay from a captured HIP graph with the eager result.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import attention as oatt
from oracle import model as omodel
from oracle import numerics, rope
from tests import gates
from tests.gpu_util import bits, dev, host64, make_cache
from tests.test_gpu_kernels import DECODE_LENGTHS, SHAPES, _fill_prefix, _rng

pytestmark = pytest.mark.gpu


def _inputs(dtype, hq, hkv, d, lengths, seed):
    g = _rng(9, hq, d, seed)
    b = len(lengths)
    q = g.standard_normal((b, 1, hq, d)).astype(np.float32)
    k = g.standard_normal((b, 1, hkv, d)).astype(np.float32)
    v = g.standard_normal((b, 1, hkv, d)).astype(np.float32)
    return g, q, k, v


@pytest.mark.parametrize("dtype,hq,hkv,d", SHAPES + [("bf16", 32, 2, 128), ("bf16", 6, 2, 128)])
def test_decode_step_matches_oracle(kvc, dtype, hq, hkv, d):
    """Ragged lengths 0..4095 (one to several 256-key tiles and ragged tails), GQA groups 1 to 16."""
    lengths = DECODE_LENGTHS
    g, q, k, v = _inputs(dtype, hq, hkv, d, lengths, 0)
    cache = make_cache(kvc, 2, len(lengths), max(lengths) + 1, hkv, d, dtype)
    hist_k, hist_v = _fill_prefix(cache, 1, lengths, dtype, g)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = kvc.kvc_decode_step(cache, 1, dev(q, dtype), dev(k, dtype), dev(v, dtype), dev_err=err)
    torch.cuda.synchronize()
    assert err.item() == 0
    ref = np.stack([oatt.decode_over_existing(hist_k[b], hist_v[b], q[b, 0], k[b, 0], v[b, 0], dtype)
                    for b in range(len(lengths))])
    gates.check(host64(out)[:, 0], ref, dtype, f"decode step {dtype} {hq}/{hkv} D{d}")
    assert torch.equal(cache.seqlens.cpu(), torch.tensor(lengths, dtype=torch.int32))  # read, never written


@pytest.mark.parametrize("dtype,hq,hkv,d", [("f32", 4, 4, 64), ("bf16", 64, 8, 128), ("bf16", 12, 4, 64)])
def test_decode_step_writes_rope_append_bytes_and_matches_unfused(kvc, dtype, hq, hkv, d):
    """Slot P gets exactly kvc_rope_append's K/V bits, nothing else in the (poisoned) cache changes,
    and the output agrees with kvc_rope_append + kvc_attn_decode."""
    lengths = [0, 5, 300, 1023]
    g, q, k, v = _inputs(dtype, hq, hkv, d, lengths, 1)
    caches = []
    for _ in range(2):
        c = make_cache(kvc, 2, len(lengths), 1024, hkv, d, dtype)
        _fill_prefix(c, 0, lengths, dtype, _rng(9, hq, d, 1, 99))
        caches.append(c)
    fused, unfused = caches
    out = kvc.kvc_decode_step(fused, 0, dev(q, dtype), dev(k, dtype), dev(v, dtype))
    q_rot = kvc.kvc_rope_append(unfused, 0, dev(q, dtype), dev(k, dtype), dev(v, dtype))
    ref_out = kvc.kvc_attn_decode(unfused, 0, q_rot)
    torch.cuda.synchronize()
    assert np.array_equal(bits(fused.k), bits(unfused.k))
    assert np.array_equal(bits(fused.v), bits(unfused.v))
    gates.check(host64(out), host64(ref_out), dtype, "fused vs unfused decode step")
    # K at position 0 (row 0) is the unrotated key, bit for bit (p = 0 is the identity rotation)
    assert np.array_equal(host64(fused.k[0, 0, 0]), numerics.round_to(k[0, 0], dtype))


def test_decode_step_rope_offset_mutant_fails(kvc):
    """A step that rotated at position 0 instead of the row's offset (Gotcha 1) must fail the gate."""
    dtype, hq, hkv, d = "bf16", 16, 4, 128
    lengths = [40, 700, 2000]
    g, q, k, v = _inputs(dtype, hq, hkv, d, lengths, 2)
    cache = make_cache(kvc, 1, len(lengths), 2048, hkv, d, dtype)
    hist_k, hist_v = _fill_prefix(cache, 0, lengths, dtype, g)
    out = host64(kvc.kvc_decode_step(cache, 0, dev(q, dtype), dev(k, dtype), dev(v, dtype)))[:, 0]
    torch.cuda.synchronize()

    def at_zero(b):
        kn = rope.rotate_round(numerics.round_to(k[b, 0][None], dtype), [0], dtype)
        qn = rope.rotate_round(numerics.round_to(q[b, 0][None], dtype), [0], dtype)
        ka = np.concatenate([hist_k[b], kn])
        va = np.concatenate([hist_v[b], numerics.round_to(v[b, 0][None], dtype)])
        return oatt.attend(qn, ka, va, [len(ka) - 1])[0]

    bad = np.stack([at_zero(b) for b in range(len(lengths))])
    assert not gates.passes(out, bad, dtype)
    ref = np.stack([oatt.decode_over_existing(hist_k[b], hist_v[b], q[b, 0], k[b, 0], v[b, 0], dtype)
                    for b in range(len(lengths))])
    gates.check(out, ref, dtype, "decode step")


def test_decode_step_capacity_row_skipped_and_out_may_alias_q(kvc):
    dtype, hq, hkv, d = "bf16", 16, 4, 128
    lengths = [64, 10]
    g, q, k, v = _inputs(dtype, hq, hkv, d, lengths, 3)
    cache = make_cache(kvc, 1, 2, 64, hkv, d, dtype)  # row 0 is full: no slot for a new token
    hist_k, hist_v = _fill_prefix(cache, 0, lengths, dtype, g)
    k_before, v_before = bits(cache.k), bits(cache.v)
    qd = dev(q, dtype)
    q_bits = bits(qd)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = kvc.kvc_decode_step(cache, 0, qd, dev(k, dtype), dev(v, dtype), out=qd, dev_err=err)  # in place
    torch.cuda.synchronize()
    assert out.data_ptr() == qd.data_ptr()
    assert err.item() == kvc.KVC_DEV_CAPACITY
    assert np.array_equal(bits(qd)[0], q_bits[0])  # the skipped row's queries are untouched
    assert np.array_equal(bits(cache.k)[:, 0], k_before[:, 0]) and np.array_equal(bits(cache.v)[:, 0], v_before[:, 0])
    ref = oatt.decode_over_existing(hist_k[1], hist_v[1], q[1, 0], k[1, 0], v[1, 0], dtype)
    gates.check(host64(qd)[1, 0], ref, dtype, "row 1 in place")


# ------------------------------------------------------------- HIP graphs

class _TinyGPTFused:
    """The six-layer fp32 tiny GPT; decode steps through kvc_decode_step (one launch per layer)."""

    def __init__(self, kvc, weights, w):
        self.kvc, self.w = kvc, w
        self.c, self.hq, self.d = w.extra["d_model"], w.n_q_heads, w.head_dim
        self.n_layers, self.eps = w.extra["n_layers"], w.extra["rms_eps"]
        self.wt = {n: torch.from_numpy(np.ascontiguousarray(a)).float().cuda() for n, a in weights.items()}
        self.cache = kvc.KVCache.empty(self.n_layers, w.extra["batch"], w.max_seq, w.n_kv_heads, self.d,
                                       dtype=torch.float32)
        self.err = torch.zeros(1, dtype=torch.int32, device="cuda")

    def _norm(self, x):
        return x * torch.rsqrt((x * x).mean(-1, keepdim=True) + self.eps)

    def step(self, tokens):
        kvc, c, hq, d = self.kvc, self.c, self.hq, self.d
        b, t = tokens.shape
        x = self.wt["emb"][tokens]
        for layer in range(self.n_layers):
            qkv = self._norm(x) @ self.wt[f"qkv{layer}"]
            q, k, v = (qkv[..., i * c:(i + 1) * c].reshape(b, t, hq, d).contiguous() for i in range(3))
            if t == 1:
                o = kvc.kvc_decode_step(self.cache, layer, q, k, v, dev_err=self.err)
            else:
                q_rot = kvc.kvc_rope_append(self.cache, layer, q, k, v, dev_err=self.err)
                o = kvc.kvc_attn_prefill(self.cache, layer, q_rot, dev_err=self.err)
            x = x + o.reshape(b, t, c) @ self.wt[f"out{layer}"]
            hmid = torch.nn.functional.gelu(self._norm(x) @ self.wt[f"fc1{layer}"], approximate="none")
            x = x + hmid @ self.wt[f"fc2{layer}"]
        self.cache.seqlens += t
        return self._norm(x[:, -1]) @ self.wt["emb"].T


def test_tiny_gpt_decode_step_replays_from_a_hip_graph(kvc):
    """A whole decode step of the six-layer tiny GPT (glue + six kvc_decode_step launches + the
    seqlens advance) captured once and replayed for 40 steps; eager work and host syncs run
    between replays.  Every replay's logits equal the eager twin's, and sampled steps equal
    the oracle's no-cache rerun of the history."""
    old_tf32 = torch.backends.cuda.matmul.allow_tf32
    torch.backends.cuda.matmul.allow_tf32 = False
    try:
        w = synth.TINY_GPT6
        weights = synth.tiny_gpt_weights(w)
        prompts = synth.tiny_gpt_prompt(w)
        eager, graphed = _TinyGPTFused(kvc, weights, w), _TinyGPTFused(kvc, weights, w)
        tok = torch.from_numpy(prompts).cuda()
        lg_e = eager.step(tok)
        lg_g = graphed.step(tok)
        static_tok = torch.zeros((prompts.shape[0], 1), dtype=torch.int64, device="cuda")
        hist = prompts.copy()
        nxt = lg_e.argmax(dim=1)
        # warm the glue's kernels on a side stream, as capture requires, on a scratch model
        scratch = _TinyGPTFused(kvc, weights, w)
        scratch.step(tok)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            static_tok.copy_(nxt[:, None])
            for _ in range(2):
                scratch.step(static_tok)
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            static_logits = graphed.step(static_tok)
        # capture recorded the step without running it: graphed is still at the prompt's length
        torch.cuda.synchronize()
        assert torch.equal(graphed.cache.seqlens, eager.cache.seqlens)
        check = {0, 1, 17, 39}
        for s in range(40):
            static_tok.copy_(nxt[:, None])
            graph.replay()
            lg_e = eager.step(nxt[:, None].contiguous())
            torch.cuda.synchronize()
            ge, gg = lg_e.double().cpu().numpy(), static_logits.double().cpu().numpy()
            gates.check(gg, ge, "f32", f"graph replay {s} vs eager")
            hist = np.concatenate([hist, nxt.cpu().numpy()[:, None]], axis=1)
            if s in check:
                for b in (0, 5, 15):
                    ref = omodel.tiny_gpt_logits_nocache(hist[b], weights, w.extra["n_layers"], w.n_q_heads,
                                                         context=w.max_seq, eps=w.extra["rms_eps"])
                    gates.check(gg[b], ref, "f32", f"graph replay {s} row {b} vs oracle")
            nxt = lg_e.argmax(dim=1)
        assert graphed.err.item() == 0 and eager.err.item() == 0
        assert torch.equal(graphed.cache.seqlens, eager.cache.seqlens)
    finally:
        torch.backends.cuda.matmul.allow_tf32 = old_tf32
