"""Ragged batches -- kvc_rope_append_ragged + kvc_attn_mixed -- against the oracle (GPU).

Cake paper, Section 3: a serving batch holds the prefill chunk of one request
beside the single decode tokens of others.  Each row is checked against the
oracle for its own tokens: T_b = 1 as a decode over its cached prefix, T_b > 1
as a causal chunk at its offset, T_b = 0 left alone; and nothing outside the
appended slots changes.
"""
import numpy as np
import pytest
import torch

from oracle import attention as oatt
from oracle import numerics, rope
from tests import gates
from tests.gpu_util import bits, dev, host64, make_cache, rope_error_ok
from tests.test_gpu_kernels import _fill_prefix, _rng

pytestmark = pytest.mark.gpu

COUNTS = [3, 1, 0, 1, 70, 1, 300, 1]      # new tokens per row: prefill chunks, decode tokens, an idle row
STARTS = [0, 5, 300, 1023, 64, 2000, 7, 511]  # cached positions before the call


def _case(kvc, dtype, hq, hkv, d, seed):
    g = _rng(40, hq, d, seed)
    b_sz = len(COUNTS)
    max_seq = max(s + c for s, c in zip(STARTS, COUNTS)) + 3
    cache = make_cache(kvc, 2, b_sz, max_seq, hkv, d, dtype)  # NaN-poisoned
    hist_k, hist_v = _fill_prefix(cache, 1, STARTS, dtype, g)
    rb = kvc.RaggedBatch(COUNTS)
    n = rb.n_tokens
    q = g.standard_normal((n, hq, d)).astype(np.float32)
    k = g.standard_normal((n, hkv, d)).astype(np.float32)
    v = g.standard_normal((n, hkv, d)).astype(np.float32)
    return cache, rb, (hist_k, hist_v), (q, k, v)


def _row_ref(b, rb, hist, qkv, dtype):
    (hist_k, hist_v), (q, k, v) = hist, qkv
    first, cnt, s = rb.first(b), COUNTS[b], STARTS[b]
    sl = slice(first, first + cnt)
    k_new, v_new = oatt.appended_slots(k[sl], v[sl], s, dtype)
    ka = np.concatenate([hist_k[b], k_new])
    va = np.concatenate([hist_v[b], v_new])
    pos = np.arange(s, s + cnt)
    qh = rope.rotate_round(numerics.round_to(q[sl], dtype), pos, dtype)
    return sl, oatt.attend(qh, ka, va, pos), (k_new, v_new)


@pytest.mark.parametrize("dtype,hq,hkv,d", [("bf16", 16, 4, 128), ("bf16", 64, 8, 128), ("bf16", 12, 4, 64),
                                            ("f32", 4, 4, 64), ("f32", 8, 2, 128)])
def test_mixed_batch_matches_oracle(kvc, dtype, hq, hkv, d):
    cache, rb, hist, qkv = _case(kvc, dtype, hq, hkv, d, 0)
    q, k, v = qkv
    k_before, v_before = bits(cache.k), bits(cache.v)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    q_rot = kvc.kvc_rope_append_ragged(cache, 1, dev(q, dtype), dev(k, dtype), dev(v, dtype), rb, dev_err=err)
    out = kvc.kvc_attn_mixed(cache, 1, q_rot, rb, dev_err=err)
    torch.cuda.synchronize()
    assert err.item() == 0
    o = host64(out)
    written = np.zeros(k_before.shape[:3], dtype=bool)  # (layer, row, position)
    kc, vc = host64(cache.k), host64(cache.v)
    for b, cnt in enumerate(COUNTS):
        if cnt == 0:
            continue
        sl, ref, (k_new, v_new) = _row_ref(b, rb, hist, qkv, dtype)
        kind = "decode" if cnt == 1 else "prefill"
        gates.check(o[sl], ref, dtype, f"mixed {dtype} {hq}/{hkv} D{d} row {b} ({kind}, {cnt} tokens)")
        s = STARTS[b]
        assert np.array_equal(vc[1, b, s:s + cnt], v_new)  # values bit for bit
        # rotated keys within what a float32 rotation allows (an ulp, or 2^-20 of the pair's length)
        assert rope_error_ok(kc[1, b, s:s + cnt], k_new, numerics.round_to(k[sl], dtype), dtype), f"row {b}: K"
        written[1, b, s:s + cnt] = True
    # nothing else in the cache changed: the idle row, other layers and positions past each row's tokens
    assert np.array_equal(bits(cache.k)[~written], k_before[~written])
    assert np.array_equal(bits(cache.v)[~written], v_before[~written])
    assert cache.seqlens.cpu().tolist() == STARTS  # read, never written


def test_mixed_rows_equal_the_uniform_calls(kvc):
    """A prefill row's outputs are bit-identical to kvc_attn_prefill on that row alone; a decode
    row's agree with kvc_attn_decode on that row alone to the bf16 gates (the split-KV partition
    differs, so only the order of float32 additions may)."""
    dtype, hq, hkv, d = "bf16", 64, 8, 128
    cache, rb, hist, qkv = _case(kvc, dtype, hq, hkv, d, 1)
    q, k, v = qkv
    q_rot = kvc.kvc_rope_append_ragged(cache, 1, dev(q, dtype), dev(k, dtype), dev(v, dtype), rb)
    out = kvc.kvc_attn_mixed(cache, 1, q_rot, rb)
    torch.cuda.synchronize()
    for b, cnt in enumerate(COUNTS):
        if cnt == 0:
            continue
        first = rb.first(b)
        one = kvc.KVCache.empty(1, 1, cache.max_seq, hkv, d, dtype=torch.bfloat16)
        one.k[0, 0].copy_(cache.k[1, b])
        one.v[0, 0].copy_(cache.v[1, b])
        one.seqlens.fill_(STARTS[b])
        qb = q_rot[first:first + cnt].reshape(1, cnt, hq, d).contiguous()
        if cnt > 1:
            alone = kvc.kvc_attn_prefill(one, 0, qb)
            torch.cuda.synchronize()
            assert torch.equal(alone[0].view(torch.int16), out[first:first + cnt].view(torch.int16)), f"row {b}"
        else:
            alone = kvc.kvc_attn_decode(one, 0, qb)
            torch.cuda.synchronize()
            gates.check(host64(out[first:first + 1]), host64(alone[0]), dtype, f"decode row {b}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_malformed_token_ranges_are_skipped(kvc, dtype):
    """A row whose range runs past n_tokens, or is longer than max_tokens, sets KVC_DEV_TOKENS and
    writes nothing; the well-formed rows are still computed."""
    hq, hkv, d = 8, 4, 64
    g = _rng(41, hq, d)
    starts = [10, 20, 30]
    cache = make_cache(kvc, 1, 3, 64, hkv, d, dtype)
    hist_k, hist_v = _fill_prefix(cache, 0, starts, dtype, g)
    n = 4
    q = g.standard_normal((n, hq, d)).astype(np.float32)
    k = g.standard_normal((n, hkv, d)).astype(np.float32)
    v = g.standard_normal((n, hkv, d)).astype(np.float32)
    rb = kvc.RaggedBatch([2, 1, 1])  # a valid layout to start from: rows [0, 2), [2, 3), [3, 4)
    for cu, bad_rows in (([0, 2, 9, 9], (1, 2)),   # ends past n_tokens
                         ([0, 1, 4, 4], (1,))):    # row 1 has 3 tokens, more than max_tokens = 2
        c2 = make_cache(kvc, 1, 3, 64, hkv, d, dtype)
        c2.k.copy_(cache.k)
        c2.v.copy_(cache.v)
        c2.seqlens.copy_(cache.seqlens)
        rb.cu_tokens = torch.tensor(cu, dtype=torch.int32, device="cuda")
        rb.n_tokens, rb.max_tokens = n, 2
        before_k, before_v = bits(c2.k), bits(c2.v)
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        q_out = torch.full((n, hq, d), float("nan"), device="cuda").to(c2.dtype)
        kvc.kvc_rope_append_ragged(c2, 0, dev(q, dtype), dev(k, dtype), dev(v, dtype), rb, q_out=q_out, dev_err=err)
        out = kvc.kvc_attn_mixed(c2, 0, q_out, rb, dev_err=err)
        torch.cuda.synchronize()
        assert err.item() & kvc.KVC_DEV_TOKENS
        assert not err.item() & kvc.KVC_DEV_CAPACITY
        for b in bad_rows:
            assert np.array_equal(bits(c2.k)[0, b], before_k[0, b]) and np.array_equal(bits(c2.v)[0, b], before_v[0, b])
        # row 0 (tokens 0..1, a 2-token chunk at position 10) is still right
        cnt = cu[1] - cu[0]
        k_new, v_new = oatt.appended_slots(k[:cnt], v[:cnt], starts[0], dtype)
        pos = np.arange(starts[0], starts[0] + cnt)
        qh = rope.rotate_round(numerics.round_to(q[:cnt], dtype), pos, dtype)
        ref = oatt.attend(qh, np.concatenate([hist_k[0], k_new]), np.concatenate([hist_v[0], v_new]), pos)
        gates.check(host64(out[:cnt]), ref, dtype, f"row 0 beside malformed rows {cu}")


@pytest.mark.parametrize("dtype,hq,hkv,d", [("bf16", 16, 4, 128), ("f32", 4, 4, 64)])
def test_mixed_batch_on_a_rolling_window(kvc, dtype, hq, hkv, d):
    """On a rolling cache the decode rows attend the window of the last max_seq positions and
    the prefill rows keep the linear rule (P + T <= max_seq): checked against the oracle's
    sliding-window attention over the raw history (Tiny-GPT post, "The Cache, in Code")."""
    window = 128
    starts, counts = [0, 130, 300, 50], [5, 1, 1, 2]  # rows 1 and 2 have wrapped; 0 and 3 prefill
    g = _rng(42, hq, d)
    b_sz, n_hist = len(starts), max(s + c for s, c in zip(starts, counts))
    q = g.standard_normal((b_sz, n_hist, hq, d)).astype(np.float32)
    k = g.standard_normal((b_sz, n_hist, hkv, d)).astype(np.float32)
    v = g.standard_normal((b_sz, n_hist, hkv, d)).astype(np.float32)
    cache = make_cache(kvc, 1, b_sz, window, hkv, d, dtype)
    cache = kvc.KVCache(cache.k, cache.v, cache.seqlens, rolling=True)
    for b, p in enumerate(starts):  # the window's history: position i in slot i mod window
        pos = np.arange(max(0, p - window), p)
        if len(pos):
            slots = torch.from_numpy(pos % window).cuda()
            cache.k[0, b, slots] = dev(rope.rotate_round(numerics.round_to(k[b, pos], dtype), pos, dtype), dtype)
            cache.v[0, b, slots] = dev(numerics.round_to(v[b, pos], dtype), dtype)
    cache.seqlens.copy_(torch.tensor(starts, dtype=torch.int32))
    rb = kvc.RaggedBatch(counts)
    qp = np.concatenate([q[b, s:s + c] for b, (s, c) in enumerate(zip(starts, counts))])
    kp = np.concatenate([k[b, s:s + c] for b, (s, c) in enumerate(zip(starts, counts))])
    vp = np.concatenate([v[b, s:s + c] for b, (s, c) in enumerate(zip(starts, counts))])
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    q_rot = kvc.kvc_rope_append_ragged(cache, 0, dev(qp, dtype), dev(kp, dtype), dev(vp, dtype), rb, dev_err=err)
    out = host64(kvc.kvc_attn_mixed(cache, 0, q_rot, rb, dev_err=err))
    torch.cuda.synchronize()
    assert err.item() == 0
    for b, (s, c) in enumerate(zip(starts, counts)):
        first = rb.first(b)
        ref = oatt.window_outputs(q[b], k[b], v[b], list(range(s, s + c)), window, dtype)
        gates.check(out[first:first + c], ref, dtype, f"rolling mixed row {b} ({c} tokens at {s})")
