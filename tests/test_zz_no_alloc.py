"""kvc_attn_decode_noalloc against kvc_attn_decode (GPU).

The no-allocation decode runs the same kernels with its partial results in the
library's static device scratch.  It is called through the C ABI twice in a
row -- the second call with a smaller input, so the scratch still holds the
first call's partials -- and each output must equal kvc_attn_decode's on the
same cache bit for bit (same kernels, same worker count) and meet the oracle's
gates.  Covered: the bfloat16 vector kernel (query-head blocks of 4 and 8,
head_dim 64 and 128), the int8 matrix-core kernel (the largest partials) and
the float32 split kernel with its combine.
"""
import ctypes

import numpy as np
import pytest
import torch

from oracle import quant
from tests import gates
from tests.gpu_util import dev, host64, make_cache
from tests.test_gpu_int8 import _fill_int8_prefix, _int8_cache
from tests.test_gpu_kernels import _fill_prefix, _rng
from oracle import attention as oatt

pytestmark = pytest.mark.gpu


def _noalloc(kvc, cache, layer, q_rot, out, n_workers, err):
    """One call of the C entry point (ctypes, no binding logic in between)."""
    P = ctypes.c_void_p
    return kvc.lib.kvc_attn_decode_noalloc(cache.desc(), int(layer), P(q_rot.data_ptr()), P(out.data_ptr()),
                                           int(q_rot.shape[2]), 0.0, int(n_workers), P(err.data_ptr()),
                                           P(torch.cuda.current_stream().cuda_stream))


def _setup(kvc, kind, hq, hkv, d, lengths, seed):
    """A one-layer-deep decode case after its append: (cache, layer, rotated q, oracle output)."""
    g = _rng(31, ("bf16", "int8", "f32").index(kind), hq, d, seed)
    batch, layer = len(lengths), 1
    q = g.standard_normal((batch, 1, hq, d)).astype(np.float32)
    k = g.standard_normal((batch, 1, hkv, d)).astype(np.float32)
    v = g.standard_normal((batch, 1, hkv, d)).astype(np.float32)
    if kind == "int8":
        cache = _int8_cache(kvc, 2, batch, max(lengths) + 1, hkv, d, poison=False)
        hist = _fill_int8_prefix(cache, layer, lengths, g)
        q_rot = kvc.kvc_rope_append(cache, layer, dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"))
        ref = np.stack([quant.decode_over_int8(*hist[b], q[b, 0], k[b, 0], v[b, 0]) for b in range(batch)])
        return cache, layer, q_rot, ref, "bf16"
    cache = make_cache(kvc, 2, batch, max(lengths) + 1, hkv, d, kind)
    hk, hv = _fill_prefix(cache, layer, lengths, kind, g)
    q_rot = kvc.kvc_rope_append(cache, layer, dev(q, kind), dev(k, kind), dev(v, kind))
    ref = np.stack([oatt.decode_over_existing(hk[b], hv[b], q[b, 0], k[b, 0], v[b, 0], kind) for b in range(batch)])
    return cache, layer, q_rot, ref, kind


CASES = [  # (kind, Hq, Hkv, D, first call's lengths, second (smaller) call's lengths, workers 1st, 2nd)
    ("bf16", 64, 8, 128, [1, 700, 4095, 3000, 65], [300, 2], 0, 0),
    ("bf16", 16, 4, 128, [4095, 64, 1500], [33], 300, 7),
    ("bf16", 12, 4, 64, [2047, 1, 900, 4000], [129, 5], 0, 0),
    ("int8", 64, 8, 128, [4095, 1, 2000], [64], 0, 0),
    ("int8", 8, 8, 64, [3000, 700], [10], 0, 3),
    ("f32", 4, 4, 64, [1500, 3000, 1], [700], 0, 0),
]


@pytest.mark.parametrize("kind,hq,hkv,d,len1,len2,nw1,nw2", CASES)
def test_noalloc_decode_equals_workspace_decode(kvc, kind, hq, hkv, d, len1, len2, nw1, nw2):
    first = _setup(kvc, kind, hq, hkv, d, len1, 0)
    second = _setup(kvc, kind, hq, hkv, d, len2, 1)
    assert sum(len2) < sum(len1) and len(len2) < len(len1)  # the second call is the smaller one
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    outs = []
    for (cache, layer, q_rot, _, _), nw in ((first, nw1), (second, nw2)):  # back to back on one stream
        out = torch.full_like(q_rot, float("nan"))
        assert _noalloc(kvc, cache, layer, q_rot, out, nw, err) == kvc.KVC_OK
        outs.append(out)
    torch.cuda.synchronize()
    assert err.item() == 0
    for (cache, layer, q_rot, ref, gate), nw, out in ((first, nw1, outs[0]), (second, nw2, outs[1])):
        want = kvc.kvc_attn_decode(cache, layer, q_rot, n_workers=nw)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16) if out.dtype == torch.bfloat16 else out.view(torch.int32),
                           want.view(torch.int16) if want.dtype == torch.bfloat16 else want.view(torch.int32)), \
            f"{kind} {hq}/{hkv} D{d}: no-alloc output differs from the workspace call's"
        gates.check(host64(out)[:, 0], ref, gate, f"no-alloc decode {kind} {hq}/{hkv} D{d}")


def test_noalloc_decode_binding_and_oversize_request(kvc):
    """The binding's wrapper takes the caller's output; a request past the scratch is refused
    before anything runs, and the output stays untouched."""
    cache, layer, q_rot, ref, gate = _setup(kvc, "bf16", 64, 8, 128, [500, 1200], 2)
    out = torch.empty_like(q_rot)
    got = kvc.kvc_attn_decode_noalloc(cache, layer, q_rot, out)
    assert got is out
    torch.cuda.synchronize()
    gates.check(host64(out)[:, 0], ref, gate, "no-alloc decode via the binding")
    per_wg = 2 * 8 * (128 + 2) * 4
    too_many = kvc.KVC_DECODE_SCRATCH_MAX_BYTES // per_wg + 1
    untouched = torch.full_like(q_rot, float("nan"))
    with pytest.raises(kvc.KvcError) as e:
        kvc.kvc_attn_decode_noalloc(cache, layer, q_rot, untouched, n_workers=too_many)
    assert e.value.status == kvc.KVC_E_SCRATCH
    torch.cuda.synchronize()
    assert torch.all(torch.isnan(untouched.float()))
