"""Per-kernel parity of the HIP library against the CPU oracle (GPU).

Small ragged shapes that span several tiles and a ragged tail; the caches
are NaN-poisoned everywhere the call must not read or write, so a stray read
turns an output into NaN and a stray write shows up as a changed byte.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import attention as oatt
from oracle import numerics, rope
from tests import gates
from tests.gpu_util import bits, dev, host64, make_cache, poisoned, rope_error_ok, ulp_distance

pytestmark = pytest.mark.gpu

SHAPES = [  # (dtype, Hq, Hkv, D)
    ("f32", 4, 4, 64),
    ("bf16", 16, 4, 128),
    ("bf16", 64, 8, 128),
    ("bf16", 8, 8, 64),
    ("f32", 8, 2, 128),
    ("bf16", 12, 4, 64),
]


def _rng(*path):
    return synth.generator(777, *path)


def _fill_prefix(cache, layer, lengths, dtype, g):
    """Positions < lengths[b] of every row get N(0, 1) values (taken as rotated keys)."""
    d = cache.head_dim
    hist_k, hist_v = [], []
    for b, n in enumerate(lengths):
        k = numerics.round_to(g.standard_normal((n, cache.n_kv_heads, d)), dtype)
        v = numerics.round_to(g.standard_normal((n, cache.n_kv_heads, d)), dtype)
        if n:
            cache.k[layer, b, :n] = dev(k, dtype)
            cache.v[layer, b, :n] = dev(v, dtype)
        hist_k.append(k)
        hist_v.append(v)
    cache.seqlens.copy_(torch.tensor(lengths, dtype=torch.int32))
    return hist_k, hist_v


# ------------------------------------------------------------- rope + append

@pytest.mark.parametrize("dtype,hq,hkv,d", SHAPES)
@pytest.mark.parametrize("t_len", [1, 3, 70])
def test_rope_append_writes_exactly_the_new_slots(kvc, dtype, hq, hkv, d, t_len):
    g = _rng(1, hq, d, t_len)
    batch, max_seq, n_layers, layer = 3, 400, 2, 1
    cache = make_cache(kvc, n_layers, batch, max_seq, hkv, d, dtype)
    starts = [0, 37, max_seq - t_len]  # empty row, ragged offset, a row ending exactly at max_seq
    cache.seqlens.copy_(torch.tensor(starts, dtype=torch.int32))
    q = g.standard_normal((batch, t_len, hq, d)).astype(np.float32)
    k = g.standard_normal((batch, t_len, hkv, d)).astype(np.float32)
    v = g.standard_normal((batch, t_len, hkv, d)).astype(np.float32)
    k_before, v_before = bits(cache.k), bits(cache.v)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    q_out = kvc.kvc_rope_append(cache, layer, dev(q, dtype), dev(k, dtype), dev(v, dtype), dev_err=err)
    torch.cuda.synchronize()
    assert err.item() == 0
    assert cache.seqlens.cpu().tolist() == starts  # never advanced by the library
    k_after, v_after = bits(cache.k), bits(cache.v)
    touched = np.zeros(k_after.shape, dtype=bool)
    kh, vh, qh = host64(cache.k), host64(cache.v), host64(q_out)
    for b, s in enumerate(starts):
        touched[layer, b, s:s + t_len] = True
        k_ref, v_ref = oatt.appended_slots(k[b], v[b], s, dtype)
        assert np.array_equal(v_after[layer, b, s:s + t_len], bits(dev(v[b], dtype)))  # v: bit copy
        k_in, q_in = numerics.round_to(k[b], dtype), numerics.round_to(q[b], dtype)
        assert rope_error_ok(kh[layer, b, s:s + t_len], k_ref, k_in, dtype), f"row {b}: K"
        if s == 0:  # position 0 rotates by the identity: bit-exact
            assert np.array_equal(kh[layer, b, 0], k_ref[0])
        q_ref = rope.rotate_round(q_in, np.arange(s, s + t_len), dtype)
        assert rope_error_ok(qh[b], q_ref, q_in, dtype), f"row {b}: q"
        if dtype == "bf16":  # rounding flips only where the float32 value sits on a bf16 rounding edge
            assert np.mean(ulp_distance(qh[b], q_ref, dtype) == 0) > 0.97
    assert np.array_equal(k_after[~touched], k_before[~touched])
    assert np.array_equal(v_after[~touched], v_before[~touched])


def test_rope_append_long_positions_and_in_place_q(kvc):
    """Positions up to 73,727 (the long-context workload): full-range sin/cos; q_out may alias q."""
    dtype, hq, hkv, d = "bf16", 64, 8, 128
    g = _rng(2)
    cache = make_cache(kvc, 1, 2, 74240, hkv, d, dtype)
    starts = [73727, 65536]
    cache.seqlens.copy_(torch.tensor(starts, dtype=torch.int32))
    q = g.standard_normal((2, 1, hq, d)).astype(np.float32)
    k = g.standard_normal((2, 1, hkv, d)).astype(np.float32)
    v = g.standard_normal((2, 1, hkv, d)).astype(np.float32)
    qd = dev(q, dtype)
    kvc.kvc_rope_append(cache, 0, qd, dev(k, dtype), dev(v, dtype), q_out=qd)
    torch.cuda.synchronize()
    for b, s in enumerate(starts):
        q_in, k_in = numerics.round_to(q[b], dtype), numerics.round_to(k[b], dtype)
        q_ref = rope.rotate_round(q_in, [s], dtype)
        assert rope_error_ok(host64(qd)[b], q_ref, q_in, dtype)
        k_ref, _ = oatt.appended_slots(k[b], v[b], s, dtype)
        assert rope_error_ok(host64(cache.k)[0, b, s:s + 1], k_ref, k_in, dtype)


def test_rope_append_capacity_row_is_skipped(kvc):
    dtype, hq, hkv, d = "bf16", 16, 4, 128
    g = _rng(3)
    cache = make_cache(kvc, 1, 3, 64, hkv, d, dtype)
    starts = [10, 62, -1]  # row 1 would need 4 slots past 62 (> 64); row 2 is negative
    cache.seqlens.copy_(torch.tensor(starts, dtype=torch.int32))
    q = dev(g.standard_normal((3, 4, hq, d)), dtype)
    k = dev(g.standard_normal((3, 4, hkv, d)), dtype)
    v = dev(g.standard_normal((3, 4, hkv, d)), dtype)
    q_out = poisoned(q.shape, dtype)
    before = bits(cache.k)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    kvc.kvc_rope_append(cache, 0, q, k, v, q_out=q_out, dev_err=err)
    torch.cuda.synchronize()
    assert err.item() == kvc.KVC_DEV_CAPACITY
    after = bits(cache.k)
    assert np.array_equal(after[:, 1:], before[:, 1:])  # skipped rows untouched
    assert not np.array_equal(after[:, 0], before[:, 0])
    assert np.all(np.isnan(host64(q_out)[1:]))  # and their q_out is not written


# -------------------------------------------------------------------- clone

@pytest.mark.parametrize("dtype,hkv,d", [("bf16", 4, 128), ("f32", 4, 64), ("bf16", 8, 64)])
def test_clone_is_bit_exact(kvc, dtype, hkv, d):
    g = _rng(4, hkv, d)
    n_layers, src_len = 3, 333
    src = make_cache(kvc, n_layers, 1, 400, hkv, d, dtype, poison=False)
    src.k.copy_(dev(g.standard_normal(src.k.shape), dtype))
    src.v.copy_(dev(g.standard_normal(src.v.shape), dtype))
    src.seqlens.fill_(src_len)
    dst = make_cache(kvc, n_layers, 5, 512, hkv, d, dtype)
    before_k, before_v = bits(dst.k), bits(dst.v)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    kvc.kvc_prefill_clone(src, src_len, dst, dev_err=err)
    torch.cuda.synchronize()
    assert err.item() == 0
    assert dst.seqlens.cpu().tolist() == [src_len] * 5
    sk, sv, dk, dv = bits(src.k), bits(src.v), bits(dst.k), bits(dst.v)
    for b in range(5):
        assert np.array_equal(dk[:, b, :src_len], sk[:, 0, :src_len])
        assert np.array_equal(dv[:, b, :src_len], sv[:, 0, :src_len])
    assert np.array_equal(dk[:, :, src_len:], before_k[:, :, src_len:])
    assert np.array_equal(dv[:, :, src_len:], before_v[:, :, src_len:])


@pytest.mark.parametrize("dtype", ["bf16", "int8"])
def test_clone_of_an_empty_prompt_and_to_one_row(kvc, dtype):
    """Degenerate clones: src_len = 0 copies nothing, reports nothing and leaves the
    destination rows empty (seqlens 0); a batch-1 destination gets the one copy."""
    hkv, d = 4, 128
    src = make_cache(kvc, 2, 1, 64, hkv, d, "bf16", poison=False)
    src.k.normal_()
    src.v.normal_()
    if dtype == "int8":
        src = kvc.KVCache.empty(2, 1, 64, hkv, d, dtype=torch.int8)
        src.k.random_(-127, 128)
        src.v.random_(-127, 128)
        src.k_scale.uniform_()
        src.v_scale.uniform_()

    def dest(batch):
        if dtype == "int8":
            c = kvc.KVCache.empty(2, batch, 64, hkv, d, dtype=torch.int8)
            for t in (c.k, c.v):
                t.fill_(0x55)
            for t in (c.k_scale, c.v_scale):
                t.fill_(-1.0)
            return c
        return make_cache(kvc, 2, batch, 64, hkv, d, "bf16")

    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    src.seqlens.fill_(0)
    dst = dest(3)
    before = [bits(t) for t in (dst.k, dst.v)] + ([host64(dst.k_scale)] if dtype == "int8" else [])
    kvc.kvc_prefill_clone(src, 0, dst, dev_err=err)
    torch.cuda.synchronize()
    assert err.item() == 0 and dst.seqlens.cpu().tolist() == [0, 0, 0]
    assert np.array_equal(bits(dst.k), before[0]) and np.array_equal(bits(dst.v), before[1])
    if dtype == "int8":
        assert np.array_equal(host64(dst.k_scale), before[2])
    src.seqlens.fill_(17)
    one = dest(1)
    kvc.kvc_prefill_clone(src, 17, one, dev_err=err)
    torch.cuda.synchronize()
    assert err.item() == 0 and one.seqlens.cpu().tolist() == [17]
    assert np.array_equal(bits(one.k)[:, 0, :17], bits(src.k)[:, 0, :17])
    assert np.array_equal(bits(one.v)[:, 0, :17], bits(src.v)[:, 0, :17])
    if dtype == "int8":
        assert np.array_equal(host64(one.k_scale)[:, 0, :, :17], host64(src.k_scale)[:, 0, :, :17])
        assert np.all(host64(one.k_scale)[:, 0, :, 17:] == -1.0)


def test_clone_errors(kvc):
    dtype = "bf16"
    src = make_cache(kvc, 2, 1, 64, 4, 128, dtype, poison=False)
    src.seqlens.fill_(20)
    dst = make_cache(kvc, 2, 3, 64, 4, 128, dtype)
    dst.seqlens.copy_(torch.tensor([0, 5, 0], dtype=torch.int32))
    before = bits(dst.k)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    kvc.kvc_prefill_clone(src, 20, dst, dev_err=err)
    torch.cuda.synchronize()
    assert err.item() == kvc.KVC_DEV_NOT_EMPTY
    assert dst.seqlens.cpu().tolist() == [20, 5, 20]
    assert np.array_equal(bits(dst.k)[:, 1], before[:, 1])  # the non-empty row is skipped
    # host-known length disagreeing with the device length: nothing is written
    dst2 = make_cache(kvc, 2, 3, 64, 4, 128, dtype)
    before2 = bits(dst2.k)
    err.zero_()
    kvc.kvc_prefill_clone(src, 19, dst2, dev_err=err)
    torch.cuda.synchronize()
    assert err.item() == kvc.KVC_DEV_SRC_LEN
    assert np.array_equal(bits(dst2.k), before2) and dst2.seqlens.cpu().tolist() == [0, 0, 0]
    # host-side asserts of the post
    with pytest.raises(kvc.KvcError):
        kvc.kvc_prefill_clone(src, 20, make_cache(kvc, 2, 3, 32, 4, 128, dtype))  # dst.max_seq < src.max_seq
    with pytest.raises(kvc.KvcError):
        kvc.kvc_prefill_clone(src, 20, make_cache(kvc, 1, 3, 64, 4, 128, dtype))  # layer count
    with pytest.raises(kvc.KvcError):
        kvc.kvc_prefill_clone(dst, 20, src)  # source batch must be 1


# ------------------------------------------------------------------- decode

DECODE_LENGTHS = [0, 1, 63, 64, 65, 700, 1500, 4095]


def _decode_case(kvc, dtype, hq, hkv, d, lengths, n_workers, spike=False, seed=0):
    g = _rng(5, hq, d, seed)
    batch, max_seq = len(lengths), max(lengths) + 1
    cache = make_cache(kvc, 2, batch, max_seq, hkv, d, dtype)
    hist_k, hist_v = _fill_prefix(cache, 1, lengths, dtype, g)
    q = g.standard_normal((batch, 1, hq, d)).astype(np.float32)
    k = g.standard_normal((batch, 1, hkv, d)).astype(np.float32)
    v = g.standard_normal((batch, 1, hkv, d)).astype(np.float32)
    if spike:  # the new key of group 0 parallel to its first query: that row's output ~ its value
        k[:, 0, 0] = 12.0 * np.sqrt(d) * q[:, 0, 0] / np.sum(q[:, 0, 0] ** 2, axis=-1, keepdims=True)
    q_rot = kvc.kvc_rope_append(cache, 1, dev(q, dtype), dev(k, dtype), dev(v, dtype))
    out = kvc.kvc_attn_decode(cache, 1, q_rot, n_workers=n_workers)
    torch.cuda.synchronize()
    ref = np.stack([oatt.decode_over_existing(hist_k[b], hist_v[b], q[b, 0], k[b, 0], v[b, 0], dtype)
                    for b in range(batch)])
    return host64(out)[:, 0], ref, (hist_k, hist_v, q, k, v)


@pytest.mark.parametrize("dtype,hq,hkv,d", SHAPES + [("bf16", 32, 2, 128), ("bf16", 6, 2, 128)])
@pytest.mark.parametrize("n_workers", [0, 1, 7, 300])
def test_decode_matches_oracle(kvc, dtype, hq, hkv, d, n_workers):
    """Ragged lengths (1 to 4096 keys) over every head layout: GQA groups 1, 3, 4, 8 and 16."""
    out, ref, _ = _decode_case(kvc, dtype, hq, hkv, d, DECODE_LENGTHS, n_workers)
    gates.check(out, ref, dtype, f"decode {dtype} {hq}/{hkv} D{d} workers {n_workers}")


@pytest.mark.parametrize("dtype,hq,hkv,d", [("bf16", 64, 8, 128), ("f32", 4, 4, 64)])
def test_decode_spike_rows_and_mutants_fail(kvc, dtype, hq, hkv, d):
    """Planted spikes; the oracle's deliberate-bug variants must fail against the GPU output."""
    lengths = [5, 300, 2000, 2047]
    out, ref, (hk, hv, q, k, v) = _decode_case(kvc, dtype, hq, hkv, d, lengths, 0, spike=True, seed=1)
    gates.check(out, ref, dtype, "spiked decode")
    out2, ref2, (hk2, hv2, q2, k2, v2) = _decode_case(kvc, dtype, hq, hkv, d, lengths, 0, spike=False, seed=2)
    gates.check(out2, ref2, dtype, "plain decode")
    both_out = np.concatenate([out, out2])
    group = hq // hkv

    def mutant(name, hk, hv, q, k, v, b):
        p = hk[b].shape[0]
        pos_q = 0 if name == "rope_offset_zero" else p
        kn = rope.rotate_round(numerics.round_to(k[b, 0][None], dtype), [pos_q], dtype)
        qn = rope.rotate_round(numerics.round_to(q[b, 0][None], dtype), [pos_q], dtype)
        ka = np.concatenate([hk[b], kn])
        va = np.concatenate([hv[b], numerics.round_to(v[b, 0][None], dtype)])
        if name == "top_left_mask_at_T1":
            ka, va = ka[:1], va[:1]
        if name == "length_off_by_one":
            ka, va = ka[:-1], va[:-1]
        if name == "head_map_modulo":  # query head h reads KV head h mod Hkv
            out_h = np.empty((hq, d))
            for h in range(hq):
                gg = h % hkv
                s = ka[:, gg] @ qn[0, h] / np.sqrt(d)
                w = np.exp(s - s.max())
                out_h[h] = w @ va[:, gg] / w.sum()
            return out_h
        return oatt.attend(qn, ka, va, [len(ka) - 1])[0]

    names = ["rope_offset_zero", "top_left_mask_at_T1", "length_off_by_one"] + (["head_map_modulo"] if group > 1 else [])
    for name in names:
        bad = np.concatenate([np.stack([mutant(name, hk, hv, q, k, v, b) for b in range(len(lengths))]),
                              np.stack([mutant(name, hk2, hv2, q2, k2, v2, b) for b in range(len(lengths))])])
        assert not gates.passes(both_out, bad, dtype), f"mutant {name} passes against the GPU output"


def test_decode_split_count_independence_and_determinism(kvc):
    """The split-KV partition changes only the float32 addition order (one worker = no split at all)."""
    dtype, hq, hkv, d = "bf16", 64, 8, 128
    outs = {}
    for nw in (1, 3, 64, 1000, 0):
        out, ref, _ = _decode_case(kvc, dtype, hq, hkv, d, [1, 777, 3000, 4095], nw, seed=3)
        gates.check(out, ref, dtype, f"workers {nw}")
        outs[nw] = out
    for nw in (3, 64, 1000, 0):
        gates.check(outs[nw], outs[1], dtype, f"workers {nw} vs one worker")
    again, _, _ = _decode_case(kvc, dtype, hq, hkv, d, [1, 777, 3000, 4095], 64, seed=3)
    assert np.array_equal(again, outs[64])  # run-to-run bit-identical


def test_decode_batch_row_equals_single_row_run(kvc):
    """Row b of a batch decodes like a batch-1 cache holding only row b (nanochat's clone-then-diverge flow)."""
    dtype, hq, hkv, d = "bf16", 16, 4, 128
    lengths = [2000, 5, 2047, 1200]
    out, ref, (hk, hv, q, k, v) = _decode_case(kvc, dtype, hq, hkv, d, lengths, 0, seed=4)
    for b in range(len(lengths)):
        one = make_cache(kvc, 1, 1, max(lengths) + 1, hkv, d, dtype)
        n = lengths[b]
        one.k[0, 0, :n] = dev(hk[b], dtype)
        one.v[0, 0, :n] = dev(hv[b], dtype)
        one.seqlens.fill_(n)
        q_rot = kvc.kvc_rope_append(one, 0, dev(q[b:b + 1], dtype), dev(k[b:b + 1], dtype), dev(v[b:b + 1], dtype))
        single = host64(kvc.kvc_attn_decode(one, 0, q_rot))[0, 0]
        torch.cuda.synchronize()
        gates.check(out[b], single, dtype, f"row {b} in batch vs alone")
        gates.check(single, ref[b], dtype, f"row {b} alone vs oracle")


def test_decode_on_a_side_stream_with_the_binding_workspace(kvc):
    """workspace=None and out=None on a stream other than the current one: the binding's temporary
    buffers are recorded on that stream, so the default stream's allocations made while the decode
    still runs cannot take their memory.  Every output must match the oracle."""
    dtype, hq, hkv, d = "bf16", 64, 8, 128
    lengths = [4000, 3000, 4095, 2500]
    g = _rng(9, hq, d)
    cache = make_cache(kvc, 2, len(lengths), max(lengths) + 1, hkv, d, dtype)
    hist_k, hist_v = _fill_prefix(cache, 1, lengths, dtype, g)
    q = g.standard_normal((len(lengths), 1, hq, d)).astype(np.float32)
    k = g.standard_normal((len(lengths), 1, hkv, d)).astype(np.float32)
    v = g.standard_normal((len(lengths), 1, hkv, d)).astype(np.float32)
    q_rot = kvc.kvc_rope_append(cache, 1, dev(q, dtype), dev(k, dtype), dev(v, dtype))
    ref = np.stack([oatt.decode_over_existing(hist_k[b], hist_v[b], q[b, 0], k[b, 0], v[b, 0], dtype)
                    for b in range(len(lengths))])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs, churn = [], []
    for _ in range(6):
        outs.append(kvc.kvc_attn_decode(cache, 1, q_rot, stream=side))  # the binding allocates both buffers
        # meanwhile the default stream allocates and poisons memory of the freed workspace's size
        churn.append(torch.full((kvc.kvc_decode_workspace_bytes(cache, hq) // 4,), float("nan"), device="cuda"))
        del churn[0]
    torch.cuda.synchronize()
    for i, out in enumerate(outs):
        gates.check(host64(out)[:, 0], ref, dtype, f"side-stream decode {i}")


def test_decode_capacity_and_workspace_errors(kvc):
    dtype = "bf16"
    cache = make_cache(kvc, 1, 2, 1024, 4, 128, dtype)
    cache.seqlens.copy_(torch.tensor([1024, 3], dtype=torch.int32))  # row 0 has no slot for a new token
    q = dev(np.ones((2, 1, 16, 128)), dtype)
    out = poisoned(q.shape, dtype)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    cache.k[0, 1, :4] = 0.5
    cache.v[0, 1, :4] = 0.25
    kvc.kvc_attn_decode(cache, 0, q, out=out, dev_err=err)
    torch.cuda.synchronize()
    assert err.item() == kvc.KVC_DEV_CAPACITY
    o = host64(out)
    assert np.all(np.isnan(o[0])) and np.allclose(o[1], 0.25)
    need = kvc.kvc_decode_workspace_bytes(cache, 16)
    assert need > 0
    small = torch.empty(need - 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(kvc.KvcError) as e:
        kvc.kvc_attn_decode(cache, 0, q, workspace=small)
    assert e.value.status == kvc.KVC_E_WORKSPACE


# ------------------------------------------------------------------ prefill

PREFILL_CASES = [  # (dtype, Hq, Hkv, D, T, start)
    ("bf16", 16, 4, 128, 1, 0),
    ("bf16", 16, 4, 128, 2, 0),
    ("bf16", 16, 4, 128, 129, 0),
    ("bf16", 16, 4, 128, 300, 77),
    ("bf16", 64, 8, 128, 64, 1000),
    ("bf16", 8, 1, 128, 150, 40),    # one KV head: 256-byte K rows
    ("bf16", 32, 32, 128, 100, 5),   # no head sharing: 8 KiB K rows
    ("bf16", 8, 8, 64, 200, 0),
    ("bf16", 12, 4, 64, 131, 129),
    ("f32", 4, 4, 64, 8, 0),
    ("f32", 4, 4, 64, 37, 20),
    ("f32", 8, 2, 128, 17, 3),
]


@pytest.mark.parametrize("dtype,hq,hkv,d,t_len,start", PREFILL_CASES)
def test_prefill_matches_oracle(kvc, dtype, hq, hkv, d, t_len, start):
    g = _rng(6, hq, d, t_len, start)
    batch = 2
    starts = [start, start // 2]
    max_seq = start + t_len + 5
    cache = make_cache(kvc, 1, batch, max_seq, hkv, d, dtype)
    hist_k, hist_v = _fill_prefix(cache, 0, starts, dtype, g)
    q = g.standard_normal((batch, t_len, hq, d)).astype(np.float32)
    k = g.standard_normal((batch, t_len, hkv, d)).astype(np.float32)
    v = g.standard_normal((batch, t_len, hkv, d)).astype(np.float32)
    q_rot = kvc.kvc_rope_append(cache, 0, dev(q, dtype), dev(k, dtype), dev(v, dtype))
    out = kvc.kvc_attn_prefill(cache, 0, q_rot)
    torch.cuda.synchronize()
    o = host64(out)
    for b, s in enumerate(starts):
        k_new, v_new = oatt.appended_slots(k[b], v[b], s, dtype)
        ka = np.concatenate([hist_k[b], k_new])
        va = np.concatenate([hist_v[b], v_new])
        qh = rope.rotate_round(numerics.round_to(q[b], dtype), np.arange(s, s + t_len), dtype)
        ref = oatt.attend(qh, ka, va, np.arange(s, s + t_len))
        gates.check(o[b], ref, dtype, f"prefill row {b} start {s}")


@pytest.mark.parametrize("dtype,hq,hkv,d,t_len", [("bf16", 16, 4, 128, 300), ("bf16", 64, 8, 128, 257),
                                                   ("f32", 8, 2, 64, 33)])
def test_prefill_fills_the_cache_exactly(kvc, dtype, hq, hkv, d, t_len):
    """Rows whose chunk ends exactly at max_seq (start + T == max_seq, the last slot the capacity
    check allows): every key up to the last slot is attended, nothing past the cache is read."""
    g = _rng(9, hq, d, t_len)
    starts = [131, 0]
    max_seq = max(starts) + t_len
    cache = make_cache(kvc, 1, 2, max_seq, hkv, d, dtype)
    hist_k, hist_v = _fill_prefix(cache, 0, starts, dtype, g)
    q = g.standard_normal((2, t_len, hq, d)).astype(np.float32)
    k = g.standard_normal((2, t_len, hkv, d)).astype(np.float32)
    v = g.standard_normal((2, t_len, hkv, d)).astype(np.float32)
    q_rot = kvc.kvc_rope_append(cache, 0, dev(q, dtype), dev(k, dtype), dev(v, dtype))
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = kvc.kvc_attn_prefill(cache, 0, q_rot, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    o = host64(out)
    for b, s in enumerate(starts):
        k_new, v_new = oatt.appended_slots(k[b], v[b], s, dtype)
        ka = np.concatenate([hist_k[b], k_new])
        va = np.concatenate([hist_v[b], v_new])
        qh = rope.rotate_round(numerics.round_to(q[b], dtype), np.arange(s, s + t_len), dtype)
        gates.check(o[b], oatt.attend(qh, ka, va, np.arange(s, s + t_len)), dtype, f"row {b} start {s}")


@pytest.mark.parametrize("hq,hkv,d", [(64, 8, 128), (64, 16, 64)])
def test_prefill_four_and_eight_wave_forms_agree(kvc, hq, hkv, d):
    """A batch of 8 rows at 64 query heads takes the 8-wave prefill (its grid fills the device);
    each row prefilled alone takes the 4-wave form (128 query tiles of 128, fewer workgroups than
    CUs).  Every query's output is computed by one wave in the same order in both, so the rows
    must agree bit for bit, and both with the oracle.  T = 300 leaves a ragged last tile."""
    dtype, batch, t_len = "bf16", 8, 300
    g = _rng(8, hq, d)
    starts = [0, 5, 64, 129, 300, 511, 700, 1000]
    max_seq = max(starts) + t_len + 3
    cache = make_cache(kvc, 1, batch, max_seq, hkv, d, dtype)
    hist_k, hist_v = _fill_prefix(cache, 0, starts, dtype, g)
    q = g.standard_normal((batch, t_len, hq, d)).astype(np.float32)
    k = g.standard_normal((batch, t_len, hkv, d)).astype(np.float32)
    v = g.standard_normal((batch, t_len, hkv, d)).astype(np.float32)
    q_rot = kvc.kvc_rope_append(cache, 0, dev(q, dtype), dev(k, dtype), dev(v, dtype))
    together = bits(kvc.kvc_attn_prefill(cache, 0, q_rot))
    for b, s in enumerate(starts):
        one = kvc.KVCache(cache.k[:, b:b + 1].contiguous(), cache.v[:, b:b + 1].contiguous(),
                          cache.seqlens[b:b + 1].clone())
        alone = kvc.kvc_attn_prefill(one, 0, q_rot[b:b + 1].contiguous())
        torch.cuda.synchronize()
        assert np.array_equal(bits(alone)[0], together[b]), f"row {b}: 4-wave and 8-wave forms differ"
        k_new, v_new = oatt.appended_slots(k[b], v[b], s, dtype)
        ka = np.concatenate([hist_k[b], k_new])
        va = np.concatenate([hist_v[b], v_new])
        qh = rope.rotate_round(numerics.round_to(q[b], dtype), np.arange(s, s + t_len), dtype)
        gates.check(host64(alone)[0], oatt.attend(qh, ka, va, np.arange(s, s + t_len)), dtype, f"row {b}")


def test_prefill_chunked_equals_one_shot(kvc):
    """512 tokens in 4 chunks of 128 vs one pass (Cake paper, Section 3): same outputs within tolerance."""
    dtype, hq, hkv, d, n = "bf16", 16, 4, 128, 512
    g = _rng(7)
    q = g.standard_normal((1, n, hq, d)).astype(np.float32)
    k = g.standard_normal((1, n, hkv, d)).astype(np.float32)
    v = g.standard_normal((1, n, hkv, d)).astype(np.float32)
    one = make_cache(kvc, 1, 1, n, hkv, d, dtype)
    q_rot = kvc.kvc_rope_append(one, 0, dev(q, dtype), dev(k, dtype), dev(v, dtype))
    whole = host64(kvc.kvc_attn_prefill(one, 0, q_rot))
    chunked = make_cache(kvc, 1, 1, n, hkv, d, dtype)
    parts = []
    for c in range(4):
        sl = slice(128 * c, 128 * (c + 1))
        qr = kvc.kvc_rope_append(chunked, 0, dev(q[:, sl], dtype), dev(k[:, sl], dtype), dev(v[:, sl], dtype))
        parts.append(host64(kvc.kvc_attn_prefill(chunked, 0, qr)))
        chunked.seqlens += 128
    torch.cuda.synchronize()
    assert np.array_equal(bits(chunked.k), bits(one.k)) and np.array_equal(bits(chunked.v), bits(one.v))
    gates.check(np.concatenate(parts, axis=1), whole, dtype, "chunked vs one-shot")
    ref = oatt.nocache_outputs(q[0], k[0], v[0], np.arange(n), dtype)
    gates.check(whole[0], ref, dtype, "one-shot vs oracle")
