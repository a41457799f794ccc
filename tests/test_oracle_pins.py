"""Pins of the CPU oracle against things other than itself (CPU only).

Each test ties one oracle function to a library routine on a special case, a
closed form, an identity the method must satisfy, a value the pages print,
or an independent pure-Python brute force, so that a dropped term, a wrong
sign, a wrong index or a transposed operand fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention as oatt
from oracle import brute, model, numerics, rope

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_values.json")


# ----------------------------------------------------------------- rounding

def test_bf16_rounding_matches_torch():
    """round_bf16 agrees bit for bit with torch's float32 -> bfloat16 cast (RNE)."""
    g = np.random.default_rng(0)
    x = np.concatenate([
        g.standard_normal(200000).astype(np.float32) * np.float32(3.0),
        np.float32(2.0) ** g.integers(-140, 127, 20000).astype(np.float32),
        # exact ties: the 9th significant bit set and nothing below it
        (np.arange(1, 5000, dtype=np.uint32) << 16 | np.uint32(0x8000)).view(np.float32),
        np.array([0.0, -0.0, 1e-45, -1e-45, 3.3e38, -3.3e38], dtype=np.float32),
    ])
    ours = numerics.f32_to_bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)


def test_bf16_hand_cases():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties go to the even mantissa (1).
    assert numerics.round_bf16([1 + 2 ** -8])[0] == 1.0
    # 1 + 3 * 2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6: even is 1 + 2^-6.
    assert numerics.round_bf16([1 + 3 * 2 ** -8])[0] == 1 + 2 ** -6
    assert numerics.round_bf16([1 + 2 ** -8 + 2 ** -30])[0] == 1 + 2 ** -7
    assert numerics.round_bf16([-2.5])[0] == -2.5
    assert numerics.round_f32([1 + 2 ** -24])[0] == 1.0


# --------------------------------------------------------------------- RoPE

def test_rope_worked_example_d4():
    """D = 4, base 10000: inv_freq = (1, 0.01); at p = 1 the angles are (1, f32(0.01)).

    Half-split pairs are (0, 2) and (1, 3).  Each basis vector must land on
    the printed rotation: e0 -> (cos 1, 0, sin 1, 0), e2 -> (-sin 1, 0, cos 1, 0),
    e1 -> (0, cos t, 0, sin t), e3 -> (0, -sin t, 0, cos t) with t = f32(0.01).
    """
    f = rope.inv_freq(4, 10000.0)
    assert f[0] == np.float32(1.0) and f[1] == np.float32(0.01)
    t = float(np.float32(0.01))
    eye = np.eye(4)[:, None, :]  # four tokens, one head each
    out = rope.rotate(eye, [1, 1, 1, 1], 10000.0)[:, 0, :]
    c1, s1, ct, st = math.cos(1.0), math.sin(1.0), math.cos(t), math.sin(t)
    expect = np.array([[c1, 0, s1, 0], [0, ct, 0, st], [-s1, 0, c1, 0], [0, -st, 0, ct]])
    assert np.allclose(out, expect, rtol=0, atol=1e-15)


def test_rope_position_zero_is_identity_bitexact():
    g = np.random.default_rng(1)
    x = numerics.round_bf16(g.standard_normal((5, 3, 128)))
    out = rope.rotate_round(x, np.zeros(5, dtype=int), "bf16")
    assert np.array_equal(out, x)


def test_rope_preserves_pair_norms():
    g = np.random.default_rng(2)
    x = g.standard_normal((64, 2, 128))
    pos = g.integers(0, 80000, 64)
    y = rope.rotate(x, pos)
    n_in = x[..., :64] ** 2 + x[..., 64:] ** 2
    n_out = y[..., :64] ** 2 + y[..., 64:] ** 2
    assert np.allclose(n_in, n_out, rtol=1e-13, atol=0)


def test_rope_scores_depend_only_on_distance():
    """<R_p q, R_j k> = <R_{p+s} q, R_{j+s} k> (Tiny-GPT post, window remark).

    Angles are float32 products, so the identity holds to the float32 angle
    error: |delta theta| <= ulp(p * f) per frequency.  Positions below 2^10
    keep that under 6e-5 rad, hence the 1e-3 bound; a wrong offset or a
    sign error breaks it by O(1).
    """
    g = np.random.default_rng(3)
    q = g.standard_normal((1, 1, 64))
    k = g.standard_normal((1, 1, 64))
    for p, j, s in [(7, 3, 100), (50, 0, 400), (300, 299, 511), (10, 10, 900)]:
        a = np.sum(rope.rotate(q, [p]) * rope.rotate(k, [j]))
        b = np.sum(rope.rotate(q, [p + s]) * rope.rotate(k, [j + s]))
        assert abs(a - b) < 1e-3 * np.linalg.norm(q) * np.linalg.norm(k)
    # a shift of only the query changes the score
    a = np.sum(rope.rotate(q, [40]) * rope.rotate(k, [10]))
    b = np.sum(rope.rotate(q, [41]) * rope.rotate(k, [10]))
    assert abs(a - b) > 1e-2


def test_rope_matches_brute_force():
    g = np.random.default_rng(4)
    for d in (4, 8, 64, 128):
        x = g.standard_normal((6, 2, d))
        pos = [0, 1, 2, 77, 4095, 73727]
        for dtype in ("f32", "bf16"):
            ours = rope.rotate_round(x, pos, dtype)
            ref = np.array([[brute.rope_vec(list(x[t, h]), pos[t], 10000.0, dtype) for h in range(2)]
                            for t in range(6)])
            if dtype == "f32":
                assert np.allclose(ours, ref, rtol=0, atol=4e-7 * np.abs(ref).max())
            else:
                # identical up to a one-ulp flip where the float64 value sits on a rounding edge
                ulp = np.ldexp(1.0, np.frexp(np.abs(ref) + 1e-30)[1] - 8)
                assert np.all(np.abs(ours - ref) <= ulp)
                assert np.mean(ours == ref) > 0.99


# ---------------------------------------------------------------- attention

def _rand_row(g, t_len, n_keys, hq, hkv, d):
    q = g.standard_normal((t_len, hq, d))
    k = g.standard_normal((n_keys, hkv, d))
    v = g.standard_normal((n_keys, hkv, d))
    return q, k, v


def test_attend_matches_brute_force_ragged():
    """Tiny GQA rows with ragged offsets: numpy oracle vs pure-Python loops, <= 1e-12."""
    g = np.random.default_rng(5)
    for (t_len, start, hq, hkv, d) in [(1, 0, 4, 2, 8), (5, 0, 4, 2, 8), (3, 4, 4, 1, 4),
                                        (1, 6, 2, 2, 8), (4, 2, 4, 4, 6), (2, 9, 4, 2, 8)]:
        n_keys = start + t_len
        q, k, v = _rand_row(g, t_len, n_keys, hq, hkv, d)
        q_pos = np.arange(start, start + t_len)
        scale = 1 / math.sqrt(d)
        ours = oatt.attend(q, k, v, q_pos)
        ref = np.array(brute.attention_row(q.tolist(), k.tolist(), v.tolist(), list(q_pos), scale))
        assert np.max(np.abs(ours - ref)) <= 1e-12


def test_nocache_matches_brute_force():
    g = np.random.default_rng(6)
    n, hq, hkv, d = 7, 4, 2, 8
    q, k, v = _rand_row(g, n, n, hq, hkv, d)
    qp = [0, 3, 6]
    for dtype in ("f32", "bf16"):
        ours = oatt.nocache_outputs(q, k, v, qp, dtype)
        ref = np.array(brute.nocache_row(q.tolist(), k.tolist(), v.tolist(), qp, dtype))
        assert np.max(np.abs(ours - ref)) <= 1e-12 if dtype == "f32" else np.max(np.abs(ours - ref)) <= 2e-2
        if dtype == "bf16":
            # a bf16 one-ulp rounding flip in a rotated key is the only allowed difference
            assert np.mean(np.abs(ours - ref) <= 1e-12) > 0.9


def _sdpa(q, k, v, causal):
    """torch CPU float64 SDPA on (heads, T, D) tensors, KV heads repeated per group."""
    hq, hkv = q.shape[1], k.shape[1]
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)[None].contiguous()
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)[None].contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=causal)
    return o[0].permute(1, 0, 2).numpy()


def test_attend_prefill_from_zero_matches_torch_sdpa():
    """start 0 prefill = SDPA with is_causal=True (the post's call, Gotcha 2)."""
    g = np.random.default_rng(7)
    q, k, v = _rand_row(g, 37, 37, 8, 2, 64)
    ours = oatt.attend(q, k, v, np.arange(37))
    assert np.max(np.abs(ours - _sdpa(q, k, v, True))) <= 1e-12


def test_attend_decode_matches_torch_sdpa():
    """one query at the last position = SDPA with is_causal=False (Gotcha 2)."""
    g = np.random.default_rng(8)
    q, k, v = _rand_row(g, 1, 300, 16, 4, 128)
    ours = oatt.attend(q, k, v, [299])
    assert np.max(np.abs(ours - _sdpa(q, k, v, False))) <= 1e-12


def test_attend_closed_forms():
    g = np.random.default_rng(9)
    # one visible key: the softmax weight is exactly 1, the output is that value
    q, k, v = _rand_row(g, 1, 1, 4, 2, 16)
    assert np.array_equal(oatt.attend(q, k, v, [0])[0], v[0][[0, 0, 1, 1]])
    # all keys equal: uniform weights, the output is the mean of the visible values
    q, k, v = _rand_row(g, 3, 10, 4, 2, 16)
    k[:] = k[0]
    out = oatt.attend(q, k, v, [4, 7, 9])
    for i, p in enumerate([4, 7, 9]):
        mean = v[: p + 1].mean(axis=0)[[0, 0, 1, 1]]
        assert np.allclose(out[i], mean, atol=1e-13)
    # all values equal to c: the output is c whatever the scores
    v[:] = 0.375
    assert np.allclose(oatt.attend(q, k, v, [4, 7, 9]), 0.375, atol=1e-14)
    # a spike key parallel to the query dominates: the output is its value
    q, k, v = _rand_row(g, 1, 50, 1, 1, 64)
    k[17, 0] = 40.0 * q[0, 0]
    out = oatt.attend(q, k, v, [49])
    assert np.allclose(out[0, 0], v[17, 0], atol=1e-9)


def test_chunked_equals_one_shot():
    """Queries split into chunks see the same keys as one pass (Cake paper, Section 3)."""
    g = np.random.default_rng(10)
    q, k, v = _rand_row(g, 96, 96, 4, 2, 32)
    whole = oatt.attend(q, k, v, np.arange(96))
    parts = np.concatenate([oatt.attend(q[s:s + 32], k, v, np.arange(s, s + 32)) for s in range(0, 96, 32)])
    assert np.array_equal(whole, parts)


def test_cached_steps_equal_nocache_recompute():
    """The Tiny-GPT post's check, on attention: a cached loop (written here, appending
    rotated keys step by step as the post's code does) equals the oracle's
    from-scratch recompute at every step."""
    g = np.random.default_rng(11)
    n, hq, hkv, d = 40, 4, 2, 16
    q, k, v = (numerics.round_f32(x) for x in _rand_row(g, n, n, hq, hkv, d))
    prompt = 6
    kc = rope.rotate_round(k[:prompt], np.arange(prompt), "f32")
    vc = numerics.round_f32(v[:prompt])
    for p in range(prompt, n):
        kc = np.concatenate([kc, rope.rotate_round(k[p:p + 1], [p], "f32")])
        vc = np.concatenate([vc, numerics.round_f32(v[p:p + 1])])
        qh = rope.rotate_round(q[p:p + 1], [p], "f32")
        cached = oatt.attend(qh, kc, vc, [p])
        fresh = oatt.nocache_outputs(q, k, v, [p], "f32")
        assert np.max(np.abs(cached - fresh)) <= 1e-14


def test_decode_over_existing_equals_nocache_when_history_is_rotated():
    g = np.random.default_rng(12)
    n, hq, hkv, d = 20, 8, 2, 32
    q, k, v = (numerics.round_bf16(x) for x in _rand_row(g, n, n, hq, hkv, d))
    k_hat = rope.rotate_round(k, np.arange(n), "bf16")
    v_r = numerics.round_bf16(v)
    out = oatt.decode_over_existing(k_hat[: n - 1], v_r[: n - 1], q[n - 1], k[n - 1], v[n - 1], "bf16")
    ref = oatt.nocache_outputs(q, k, v, [n - 1], "bf16")[0]
    assert np.max(np.abs(out - ref)) <= 1e-14


# -------------------------------------------------------------------- clone

def test_clone_copies_prefix_to_every_row():
    g = np.random.default_rng(13)
    ks = g.standard_normal((2, 1, 12, 2, 4))
    vs = g.standard_normal((2, 1, 12, 2, 4))
    kd = np.full((2, 3, 16, 2, 4), 7.0)
    vd = np.full((2, 3, 16, 2, 4), -7.0)
    k, v, lens = oatt.clone_cache(ks, vs, 9, kd, vd)
    assert list(lens) == [9, 9, 9]
    for b in range(3):
        assert np.array_equal(k[:, b, :9], ks[:, 0, :9]) and np.array_equal(v[:, b, :9], vs[:, 0, :9])
    assert np.all(k[:, :, 9:] == 7.0) and np.all(v[:, :, 9:] == -7.0)
    with pytest.raises(ValueError):
        oatt.clone_cache(ks, vs, 9, kd[:, :, :10], vd[:, :, :10])
    with pytest.raises(ValueError):
        oatt.clone_cache(ks, vs, 9, kd[:1], vd[:1])


def test_clone_then_decode_equals_independent_rows():
    """N rows decoded after a clone equal N independent batch-1 runs (nanochat post)."""
    g = np.random.default_rng(14)
    prompt, steps, hq, hkv, d = 12, 5, 4, 2, 16
    qp, kp, vp = (numerics.round_bf16(x) for x in _rand_row(g, prompt, prompt, hq, hkv, d))
    for row in range(3):
        qn, kn, vn = (numerics.round_bf16(x) for x in _rand_row(g, steps, steps, hq, hkv, d))
        q_all, k_all, v_all = (np.concatenate(x) for x in ((qp, qn), (kp, kn), (vp, vn)))
        # cloned: prefix keys come from the shared prompt, the rest from this row
        kc = rope.rotate_round(kp, np.arange(prompt), "bf16")
        vc = numerics.round_bf16(vp)
        for s in range(steps):
            out = oatt.decode_over_existing(kc, vc, qn[s], kn[s], vn[s], "bf16")
            ref = oatt.nocache_outputs(q_all, k_all, v_all, [prompt + s], "bf16")[0]
            assert np.max(np.abs(out - ref)) <= 1e-14
            kc = np.concatenate([kc, rope.rotate_round(kn[s:s + 1], [prompt + s], "bf16")])
            vc = np.concatenate([vc, numerics.round_bf16(vn[s:s + 1])])


# ------------------------------------------------------------------ sizing

def test_page_printed_sizes():
    gold = json.load(open(GOLDEN))
    c = gold["tiny_gpt_cache_bytes"]
    b = oatt.cache_bytes(c["n_layers"], c["tokens"], c["n_kv_heads"], c["head_dim"], c["bytes_per_value"])
    assert b == c["bytes"] and f"{b / 2**20:.2f} MiB" == c["printed"]
    for row in gold["kv_bytes_per_token"]["rows"]:
        b = oatt.cache_bytes(row["layers"], 1, row["kv_heads"], row["head_dim"], 2)
        assert b == row["printed_kB"] * 1024, row["model"]
    u = gold["clone_prefill_units"]
    assert oatt.prefill_units(u["prompt_len"], u["n_samples"], clone=False) == u["naive"]
    assert oatt.prefill_units(u["prompt_len"], u["n_samples"], clone=True) == u["clone"]
    s = gold["tiny_gpt_size"]
    n = model.param_count(s["vocab"], s["d_model"], s["n_layers"], s["mlp"])
    assert round(n / 1e6, 1) == s["printed_params_millions"]
    assert round(4 * n / 1e6) == s["printed_weight_MB"]


# -------------------------------------------------------------- model parts

def test_model_parts_match_torch():
    g = np.random.default_rng(15)
    x = g.standard_normal((9, 256))
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (256,), eps=1e-5).numpy()
    assert np.allclose(model.rms_norm(x), ref, rtol=0, atol=1e-13)
    ref = torch.nn.functional.gelu(torch.from_numpy(x)).numpy()
    assert np.allclose(model.gelu(x), ref, rtol=0, atol=1e-14)


def test_attention_layer_matches_torch_sdpa_layer():
    """The single layer at start 0 against a torch float64 build of the post's forward."""
    g = np.random.default_rng(16)
    n, c, heads = 11, 64, 4
    d = c // heads
    h = g.standard_normal((n, c))
    wqkv = g.standard_normal((c, 3 * c)) * 0.1
    wout = g.standard_normal((c, c)) * 0.1
    ours = model.attention_layer(h, wqkv, wout, heads, "f32")
    qkv = h @ wqkv
    q, k, v = (qkv[:, i * c:(i + 1) * c].reshape(n, heads, d) for i in range(3))
    qh = rope.rotate_round(numerics.round_f32(q), np.arange(n), "f32")
    kh = rope.rotate_round(numerics.round_f32(k), np.arange(n), "f32")
    ref = _sdpa(qh, kh, numerics.round_f32(v), True).reshape(n, c) @ wout
    assert np.max(np.abs(ours - ref)) <= 1e-12
