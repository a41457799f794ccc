"""The rolling-window cache on the GPU against the oracle (GPU).

Position p lives in slot p mod max_seq and keeps the rotation of its absolute
position; a decode step attends the window of the last max_seq positions.
The oracle recomputes that window from raw values (sliding-window attention,
Tiny-GPT post, "The Cache, in Code" and "Does the Cache Change the Output?").
"""
import numpy as np
import pytest
import torch

import synth
from oracle import attention as oatt
from oracle import model as omodel
from oracle import numerics, quant, rope
from tests import gates
from tests.gpu_util import TORCH_DTYPE, bits, dev, host64
from tests.test_gpu_kernels import _rng

pytestmark = pytest.mark.gpu

WINDOW = 128
POSITIONS = [0, 1, 127, 128, 129, 300, 1000, 4097]  # before, at and far past the first wrap


def _ring(kvc, path, dtype, hq, hkv, d, seed):
    """A rolling cache whose rows stand at POSITIONS, filled with the rotated history of the
    window; returns (cache, raw q/k/v histories up to each row's position inclusive)."""
    g = _rng(30, hq, d, seed)
    n = max(POSITIONS) + 1
    B = len(POSITIONS)
    q = g.standard_normal((B, n, hq, d)).astype(np.float32)
    k = g.standard_normal((B, n, hkv, d)).astype(np.float32)
    v = g.standard_normal((B, n, hkv, d)).astype(np.float32)
    storage = torch.int8 if path == "int8" else TORCH_DTYPE[dtype]
    cache = kvc.KVCache.empty(1, B, WINDOW, hkv, d, dtype=storage, rolling=True)
    cache.k.zero_()
    cache.v.zero_()
    for b, p in enumerate(POSITIONS):
        pos = np.arange(max(0, p - WINDOW), p)
        if not len(pos):
            continue
        k_hat = rope.rotate_round(numerics.round_to(k[b, pos], dtype), pos, dtype)
        v_hat = numerics.round_to(v[b, pos], dtype)
        slots = torch.from_numpy(pos % WINDOW).cuda()
        if path == "int8":
            kc, ks = quant.quantize_int8(k_hat)
            vc, vs = quant.quantize_int8(v_hat)
            cache.k[0, b, slots] = torch.from_numpy(kc).cuda()
            cache.v[0, b, slots] = torch.from_numpy(vc).cuda()
            cache.k_scale[0, b][:, slots] = torch.from_numpy(np.ascontiguousarray(ks.T)).cuda()  # head-major
            cache.v_scale[0, b][:, slots] = torch.from_numpy(np.ascontiguousarray(vs.T)).cuda()
        else:
            cache.k[0, b, slots] = dev(k_hat, dtype)
            cache.v[0, b, slots] = dev(v_hat, dtype)
    cache.seqlens.copy_(torch.tensor(POSITIONS, dtype=torch.int32))
    return cache, (q, k, v)


@pytest.mark.parametrize("path,dtype,hq,hkv,d", [
    ("decode", "f32", 4, 4, 64), ("decode", "bf16", 16, 4, 128), ("decode", "bf16", 64, 8, 128),
    ("step", "f32", 4, 4, 64), ("step", "bf16", 16, 4, 128),
    ("int8", "bf16", 64, 8, 128), ("int8", "bf16", 8, 8, 64),
])
def test_rolling_decode_matches_window_oracle(kvc, path, dtype, hq, hkv, d):
    cache, (q, k, v) = _ring(kvc, path, dtype, hq, hkv, d, seed={"decode": 1, "step": 2, "int8": 3}[path])
    idx = np.arange(len(POSITIONS))
    qn = dev(q[idx, POSITIONS][:, None], dtype)
    kn = dev(k[idx, POSITIONS][:, None], dtype)
    vn = dev(v[idx, POSITIONS][:, None], dtype)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    if path == "step":
        out = kvc.kvc_decode_step(cache, 0, qn, kn, vn, dev_err=err)
    else:
        q_rot = kvc.kvc_rope_append(cache, 0, qn, kn, vn, dev_err=err)
        out = kvc.kvc_attn_decode(cache, 0, q_rot, dev_err=err)
    torch.cuda.synchronize()
    assert err.item() == 0
    got = host64(out)[:, 0]
    if path == "int8":
        ref = []
        for b, p in enumerate(POSITIONS):
            pos = np.arange(max(0, p + 1 - WINDOW), p)  # the window minus the new token
            k_hat = rope.rotate_round(numerics.round_to(k[b, pos], "bf16"), pos, "bf16")
            kc, ks = quant.quantize_int8(k_hat)
            vc, vs = quant.quantize_int8(numerics.round_to(v[b, pos], "bf16"))
            ref.append(quant.decode_over_int8(kc, ks, vc, vs, q[b, p], k[b, p], v[b, p], position=p))
        ref = np.stack(ref)
    else:
        ref = np.stack([oatt.window_outputs(q[b], k[b], v[b], [p], WINDOW, dtype)[0]
                        for b, p in enumerate(POSITIONS)])
    gates.check(got, ref, "bf16" if path == "int8" else dtype, f"rolling {path} {dtype} {hq}/{hkv} D{d}")
    # the new value went to slot P mod window, bit for bit (the plain caches)
    if path != "int8":
        for b, p in enumerate(POSITIONS):
            assert np.array_equal(bits(cache.v[0, b, p % WINDOW]), bits(vn[b, 0]))
    assert torch.equal(cache.seqlens.cpu(), torch.tensor(POSITIONS, dtype=torch.int32))


@pytest.mark.parametrize("fused", [False, True])
def test_tiny_layer_rolling_past_the_window(kvc, fused):
    """The fp32 tiny layer decoding 600 tokens past its 8-token prompt with a 256-position rolling
    cache: every step equals the page's uncached loop, which reruns the last 256 inputs from
    scratch (one layer carries no context from evicted tokens)."""
    old = torch.backends.cuda.matmul.allow_tf32
    torch.backends.cuda.matmul.allow_tf32 = False
    try:
        w = synth.TINY_LAYER
        c, hq, d = w.extra["d_model"], w.n_q_heads, w.head_dim
        n_prompt, n_steps = w.extra["prompt"], 600
        w_qkv, w_out = synth.tiny_layer_weights(w)
        x = synth.normal((n_prompt + n_steps, c), 1.0, w.seed, 77, 0)
        wq = torch.from_numpy(w_qkv).cuda()
        wo = torch.from_numpy(w_out).cuda()
        cache = kvc.KVCache.empty(1, 1, w.max_seq, w.n_kv_heads, d, dtype=torch.float32, rolling=True)
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        outs = []
        for s in range(n_steps + 1):
            xs = x[:n_prompt] if s == 0 else x[n_prompt + s - 1:n_prompt + s]
            t = xs.shape[0]
            qkv = torch.from_numpy(np.ascontiguousarray(xs)).cuda() @ wq
            q, k, v = (qkv[:, i * c:(i + 1) * c].reshape(1, t, hq, d).contiguous() for i in range(3))
            if t == 1 and fused:
                o = kvc.kvc_decode_step(cache, 0, q, k, v, dev_err=err)
            else:
                q_rot = kvc.kvc_rope_append(cache, 0, q, k, v, dev_err=err)
                o = kvc.kvc_attn_prefill(cache, 0, q_rot, dev_err=err) if t > 1 else \
                    kvc.kvc_attn_decode(cache, 0, q_rot, dev_err=err)
            cache.seqlens += t
            outs.append((o.reshape(t, c) @ wo)[-1])
        got = torch.stack(outs).double().cpu().numpy()
        assert err.item() == 0
        assert cache.seqlens.item() == n_prompt + n_steps
        for s in range(0, n_steps + 1, 7):
            p = n_prompt - 1 + s  # position of the step's (last) query
            ref = omodel.tiny_layer_nocache(x[:p + 1], w_qkv, w_out, hq, context=w.max_seq)[-1]
            gates.check(got[s], ref, "f32", f"step at position {p}")
    finally:
        torch.backends.cuda.matmul.allow_tf32 = old
