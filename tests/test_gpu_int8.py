"""The 8-bit KV cache on the GPU against the oracle (GPU).

Appending into an int8 cache must store exactly the oracle's codes and
scales (integers decided by float32 arithmetic on both sides); decoding from
it must meet the bfloat16 gates against the oracle's attention over the
dequantized values; the clone copies codes and scales bit for bit.
"""
import numpy as np
import pytest
import torch

from oracle import numerics, quant
from tests import gates
from tests.gpu_util import dev, host64
from tests.test_gpu_kernels import DECODE_LENGTHS, _rng

pytestmark = pytest.mark.gpu

# (Hq, Hkv, D).  Groups up to 32 run on the matrix-core kernel; the last three (groups 64, 36 and 48)
# on the vector-ALU kernel with the codes widened, 36 leaving four padding heads in its last block.
SHAPES8 = [(16, 4, 128), (64, 8, 128), (8, 8, 64), (12, 4, 64), (32, 2, 128), (6, 2, 128),
           (64, 1, 128), (36, 1, 64), (96, 2, 128)]


def _int8_cache(kvc, n_layers, batch, max_seq, hkv, d, poison=True):
    shape = (n_layers, batch, max_seq, hkv, d)
    k = torch.full(shape, 0x55 if poison else 0, dtype=torch.int8, device="cuda")
    v = torch.full(shape, 0x55 if poison else 0, dtype=torch.int8, device="cuda")
    ks = torch.full(kvc.scale_shape(shape), float("nan") if poison else 0.0, dtype=torch.float32, device="cuda")
    vs = torch.full(kvc.scale_shape(shape), float("nan") if poison else 0.0, dtype=torch.float32, device="cuda")
    return kvc.KVCache(k, v, torch.zeros(batch, dtype=torch.int32, device="cuda"), ks, vs)


def _fill_int8_prefix(cache, layer, lengths, g):
    """Positions < lengths[b] get the quantized codes and scales of N(0, 1) bfloat16 vectors."""
    hkv, d = cache.n_kv_heads, cache.head_dim
    hist = []
    for b, n in enumerate(lengths):
        k = np.asarray(g.standard_normal((n, hkv, d)), dtype=np.float32)
        v = np.asarray(g.standard_normal((n, hkv, d)), dtype=np.float32)
        kc, ks = quant.quantize_int8(numerics.round_bf16(k))
        vc, vs = quant.quantize_int8(numerics.round_bf16(v))
        if n:
            cache.k[layer, b, :n] = torch.from_numpy(kc).cuda()
            cache.v[layer, b, :n] = torch.from_numpy(vc).cuda()
            cache.k_scale[layer, b, :, :n] = torch.from_numpy(np.ascontiguousarray(ks.T)).cuda()  # head-major
            cache.v_scale[layer, b, :, :n] = torch.from_numpy(np.ascontiguousarray(vs.T)).cuda()
        hist.append((kc, ks, vc, vs))
    cache.seqlens.copy_(torch.tensor(lengths, dtype=torch.int32))
    return hist


@pytest.mark.parametrize("hq,hkv,d", [(16, 4, 128), (8, 8, 64)])
@pytest.mark.parametrize("t_len", [1, 3, 70])
def test_int8_append_stores_the_oracle_codes_and_scales(kvc, hq, hkv, d, t_len):
    starts = [0, 5, 100]
    max_seq = 200
    g = _rng(11, hq, d, t_len)
    cache = _int8_cache(kvc, 2, len(starts), max_seq, hkv, d)
    cache.seqlens.copy_(torch.tensor(starts, dtype=torch.int32))
    q = g.standard_normal((len(starts), t_len, hq, d)).astype(np.float32)
    k = g.standard_normal((len(starts), t_len, hkv, d)).astype(np.float32)
    v = g.standard_normal((len(starts), t_len, hkv, d)).astype(np.float32)
    k[0, 0, 0] = 0.0  # one all-zero key vector: scale 0, codes 0
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    q_out = kvc.kvc_rope_append(cache, 1, dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), dev_err=err)
    torch.cuda.synchronize()
    assert err.item() == 0
    # the queries are rotated exactly as on a bfloat16 cache
    ref_cache = kvc.KVCache.empty(2, len(starts), max_seq, hkv, d, dtype=torch.bfloat16)
    ref_cache.k.zero_()  # defined contents everywhere, so reading the whole cache back converts cleanly
    ref_cache.v.zero_()
    ref_cache.seqlens.copy_(torch.tensor(starts, dtype=torch.int32))
    q_ref = kvc.kvc_rope_append(ref_cache, 1, dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"))
    torch.cuda.synchronize()
    assert torch.equal(q_out.view(torch.int16), q_ref.view(torch.int16))
    kc_all, vc_all = cache.k.cpu().numpy(), cache.v.cpu().numpy()
    # scales are stored head-major; compare them in the codes' (layer, row, position, head) order
    ks_all = cache.k_scale.cpu().numpy().transpose(0, 1, 3, 2)
    vs_all = cache.v_scale.cpu().numpy().transpose(0, 1, 3, 2)
    touched = np.zeros(kc_all.shape[:4], dtype=bool)
    k_bf16 = host64(ref_cache.k)  # the rotated, bfloat16-rounded keys (bytes shared with the int8 append)
    for b, p in enumerate(starts):
        sl = slice(p, p + t_len)
        # V: the oracle's codes and scales, bit for bit.  K: the rotation's float32 sin/cos may
        # differ from the oracle's by an ulp (reading 4), which can move a bfloat16 key by one
        # ulp (the key tests allow that); the integer decision itself is checked on the same
        # bfloat16 key, which must quantize to exactly the oracle's codes and scale.
        _, _, vc, vs = quant.appended_slots_int8(k[b], v[b], p)
        kc, ks = quant.quantize_int8(k_bf16[1, b, sl])
        assert np.array_equal(kc_all[1, b, sl], kc) and np.array_equal(vc_all[1, b, sl], vc)
        assert np.array_equal(ks_all[1, b, sl].view(np.uint32), ks.view(np.uint32))
        assert np.array_equal(vs_all[1, b, sl].view(np.uint32), vs.view(np.uint32))
        touched[1, b, sl] = True
        kc_o, _, _, _ = quant.appended_slots_int8(k[b], v[b], p)
        assert np.mean(kc_o != kc_all[1, b, sl]) < 0.01  # and the oracle's own rotation agrees almost everywhere
    assert ks_all[1, 0, 0, 0] == 0 and np.all(kc_all[1, 0, 0, 0] == 0)
    # nothing else written: codes keep their poison byte, scales stay NaN
    assert np.all(kc_all[~touched] == 0x55) and np.all(vc_all[~touched] == 0x55)
    assert np.all(np.isnan(ks_all[~touched])) and np.all(np.isnan(vs_all[~touched]))


def _decode_case8(kvc, hq, hkv, d, lengths, n_workers, seed=0):
    g = _rng(12, hq, d, seed)
    cache = _int8_cache(kvc, 2, len(lengths), max(lengths) + 1, hkv, d, poison=False)
    hist = _fill_int8_prefix(cache, 1, lengths, g)
    q = g.standard_normal((len(lengths), 1, hq, d)).astype(np.float32)
    k = g.standard_normal((len(lengths), 1, hkv, d)).astype(np.float32)
    v = g.standard_normal((len(lengths), 1, hkv, d)).astype(np.float32)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    q_rot = kvc.kvc_rope_append(cache, 1, dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), dev_err=err)
    ws = torch.zeros(max(1, kvc.kvc_decode_workspace_bytes(cache, hq, n_workers)), dtype=torch.uint8,
                     device="cuda")
    out = kvc.kvc_attn_decode(cache, 1, q_rot, n_workers=n_workers, workspace=ws, dev_err=err)
    torch.cuda.synchronize()
    assert err.item() == 0
    ref = np.stack([quant.decode_over_int8(*hist[b], q[b, 0], k[b, 0], v[b, 0]) for b in range(len(lengths))])
    return host64(out)[:, 0], ref, (hist, q, k, v)


@pytest.mark.parametrize("hq,hkv,d", SHAPES8)
@pytest.mark.parametrize("n_workers", [0, 7, 300])
def test_int8_decode_matches_oracle(kvc, hq, hkv, d, n_workers):
    """Ragged lengths 0..4095 over GQA groups 1 to 16, head_dim 64 and 128."""
    out, ref, _ = _decode_case8(kvc, hq, hkv, d, DECODE_LENGTHS, n_workers)
    gates.check(out, ref, "bf16", f"int8 decode {hq}/{hkv} D{d} workers {n_workers}")


def test_int8_decode_scale_mutants_fail(kvc):
    """The same codes read without their K or V scales must fail the gate (the scales matter)."""
    hq, hkv, d = 64, 8, 128
    lengths = [300, 2000, 4000]
    out, ref, (hist, q, k, v) = _decode_case8(kvc, hq, hkv, d, lengths, 0, seed=1)
    gates.check(out, ref, "bf16", "int8 decode")
    for which in ("k", "v"):
        bad = []
        for b in range(len(lengths)):
            kc, ks, vc, vs = hist[b]
            ks2 = np.full_like(ks, ks.mean()) if which == "k" else ks
            vs2 = np.full_like(vs, vs.mean()) if which == "v" else vs
            bad.append(quant.decode_over_int8(kc, ks2, vc, vs2, q[b, 0], k[b, 0], v[b, 0]))
        assert not gates.passes(out, np.stack(bad), "bf16"), f"{which} scales ignored passes"


def test_int8_clone_copies_codes_and_scales(kvc):
    hkv, d, n = 8, 128, 333
    src = _int8_cache(kvc, 2, 1, 512, hkv, d, poison=False)
    for layer in (0, 1):
        _fill_int8_prefix(src, layer, [n], _rng(13, layer))
    dst = _int8_cache(kvc, 2, 4, 600, hkv, d)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    kvc.kvc_prefill_clone(src, n, dst, dev_err=err)
    torch.cuda.synchronize()
    assert err.item() == 0
    assert torch.equal(dst.seqlens.cpu(), torch.full((4,), n, dtype=torch.int32))
    for t_src, t_dst in ((src.k, dst.k), (src.v, dst.v)):
        for r in range(4):
            assert torch.equal(t_dst[:, r, :n].cpu(), t_src[:, 0, :n].cpu())
    for t_src, t_dst in ((src.k_scale, dst.k_scale), (src.v_scale, dst.v_scale)):  # head-major: positions last
        for r in range(4):
            assert torch.equal(t_dst[:, r, :, :n].cpu().view(torch.int32), t_src[:, 0, :, :n].cpu().view(torch.int32))
    # positions at or past n keep their poison
    assert torch.all(dst.k[:, :, n:].cpu() == 0x55) and torch.all(torch.isnan(dst.k_scale[:, :, :, n:].cpu()))
    assert torch.all(torch.isnan(dst.v_scale[:, :, :, n:].cpu()))


def test_int8_cache_rejected_by_prefill_and_decode_step(kvc):
    cache = _int8_cache(kvc, 1, 1, 64, 4, 128)
    x = torch.zeros((1, 4, 16, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(kvc.KvcError) as e:
        kvc.kvc_attn_prefill(cache, 0, x)
    assert e.value.status == kvc.KVC_E_DTYPE
    q1 = torch.zeros((1, 1, 16, 128), dtype=torch.bfloat16, device="cuda")
    k1 = torch.zeros((1, 1, 4, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(kvc.KvcError) as e:
        kvc.kvc_decode_step(cache, 0, q1, k1, k1)
    assert e.value.status == kvc.KVC_E_DTYPE
