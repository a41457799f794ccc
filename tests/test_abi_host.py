"""The C ABI on the host (CPU only): every declared symbol is exported, and
argument validation rejects bad calls before anything is launched.

None of these calls reaches the GPU: each one fails host validation (or is a
pure host query), so they run on a machine without a GPU.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "kv_cache_attention_kvcache_amd", "libkvc.so")
HEADER = os.path.join(ROOT, "include", "kvc.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):  # build once if nothing is built yet
        import __graft_entry__

        __graft_entry__._build_module().build()
    import kv_cache_attention_kvcache_amd as kvc

    return kvc


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(kvc_\w+)\s*\(", text, re.M)))


def test_header_declares_the_four_calls_and_helpers():
    assert _declared() == sorted(["kvc_rope_append", "kvc_rope_append_ragged", "kvc_decode_workspace_bytes",
                                  "kvc_attn_decode", "kvc_attn_decode_noalloc", "kvc_attn_prefill",
                                  "kvc_attn_mixed", "kvc_decode_step", "kvc_prefill_clone", "kvc_status_string"])


def test_every_declared_symbol_is_exported(lib):
    raw = ctypes.CDLL(lib.LIB_PATH)  # the build the binding loaded (KVC_LIB_PATH may select another)
    for name in _declared():
        assert hasattr(raw, name), name
    assert set(_declared()) == set(lib.EXPORTS)


def _desc(lib, **kw):
    d = dict(k=0x10000, v=0x20000, seqlens=0x30000, n_layers=2, batch=3, max_seq=100, n_kv_heads=4,
             head_dim=128, dtype=lib.KVC_BF16)
    d.update(kw)
    return lib.kvc_cache(d["k"], d["v"], d["seqlens"], d["n_layers"], d["batch"], d["max_seq"],
                         d["n_kv_heads"], d["head_dim"], d["dtype"])


P = ctypes.c_void_p


def test_status_strings(lib):
    for code in range(-7, 1):
        s = lib.kvc_status_string(code)
        assert s and s != "unknown status"
    assert lib.kvc_status_string(-99) == "unknown status"


def test_workspace_query_is_a_host_function(lib):
    W = lib.lib.kvc_decode_workspace_bytes
    d = _desc(lib, max_seq=4096, batch=8, head_dim=128)
    # bfloat16: two partial slots per workgroup, each (max, sum, o) for a block of 4 (group <= 4) or 8 heads
    assert W(ctypes.byref(d), 16, 64) == 64 * 2 * 4 * (128 + 2) * 4
    assert W(ctypes.byref(d), 32, 64) == 64 * 2 * 8 * (128 + 2) * 4
    assert W(ctypes.byref(_desc(lib, head_dim=64)), 64, 10) == 10 * 2 * 8 * (64 + 2) * 4
    # float32: fixed 512-key splits per (row, query head); the worker count is ignored
    f = _desc(lib, max_seq=4096, batch=8, dtype=lib.KVC_F32)
    assert W(ctypes.byref(f), 16, 0) == 8 * 16 * 8 * (128 + 2) * 4
    assert W(ctypes.byref(f), 16, 7) == 8 * 16 * 8 * (128 + 2) * 4
    assert W(ctypes.byref(_desc(lib, max_seq=512, dtype=lib.KVC_F32)), 16, 0) == 0  # one split: none needed
    assert W(ctypes.byref(d), 6, 4) == 0  # 6 % 4 != 0: invalid
    assert W(ctypes.byref(d), 16, -1) == 0  # negative worker count: invalid


def test_rope_append_validation(lib):
    L = lib.lib
    d = _desc(lib)
    good = dict(layer=0, q=P(0x40000), qo=P(0x40000), k=P(0x50000), v=P(0x60000), T=1, hq=16, base=10000.0)

    def call(desc=d, **kw):
        a = dict(good)
        a.update(kw)
        return L.kvc_rope_append(ctypes.byref(desc), a["layer"], a["q"], a["qo"], a["k"], a["v"], a["T"],
                                 a["hq"], a["base"], None, None)

    assert call(layer=2) == lib.KVC_E_ARG
    assert call(layer=-1) == lib.KVC_E_ARG
    assert call(T=0) == lib.KVC_E_ARG
    assert call(q=None) == lib.KVC_E_ARG
    assert call(k=P(0x50004)) == lib.KVC_E_ARG  # misaligned
    assert call(base=0.0) == lib.KVC_E_ARG
    assert call(hq=6) == lib.KVC_E_SHAPE
    assert call(desc=_desc(lib, head_dim=96)) == lib.KVC_E_SHAPE
    assert call(desc=_desc(lib, dtype=7)) == lib.KVC_E_DTYPE
    assert call(desc=_desc(lib, k=0)) == lib.KVC_E_ARG
    assert L.kvc_rope_append(None, 0, P(16), P(16), P(16), P(16), 1, 4, 1e4, None, None) == lib.KVC_E_ARG


def test_decode_and_prefill_validation(lib):
    L = lib.lib
    d = _desc(lib, max_seq=4096)
    q = P(0x40000)
    assert L.kvc_attn_decode(ctypes.byref(d), 0, q, q, 16, 0.0, 8, None, 0, None, None) == lib.KVC_E_WORKSPACE
    assert L.kvc_attn_decode(ctypes.byref(d), 0, q, q, 16, 0.0, 8, P(0x70000), 8 * 2 * 4 * 130 * 4 - 4, None,
                             None) == lib.KVC_E_WORKSPACE  # one float short
    assert L.kvc_attn_decode(ctypes.byref(d), 0, q, q, 16, 0.0, -1, None, 0, None, None) == lib.KVC_E_ARG
    assert L.kvc_attn_decode(ctypes.byref(d), 0, q, q, 16, float("nan"), 0, P(0x70000), 1 << 30, None,
                             None) == lib.KVC_E_ARG
    assert L.kvc_attn_decode(ctypes.byref(d), 5, q, q, 16, 0.0, 0, P(0x70000), 1 << 30, None, None) == lib.KVC_E_ARG
    assert L.kvc_attn_decode(ctypes.byref(d), 0, q, q, 5, 0.0, 0, P(0x70000), 1 << 30, None, None) == lib.KVC_E_SHAPE
    assert L.kvc_attn_prefill(ctypes.byref(d), 0, q, q, 0, 16, 0.0, None, None) == lib.KVC_E_ARG
    assert L.kvc_attn_prefill(ctypes.byref(d), 0, None, q, 4, 16, 0.0, None, None) == lib.KVC_E_ARG
    assert L.kvc_attn_prefill(ctypes.byref(_desc(lib, head_dim=32)), 0, q, q, 4, 16, 0.0, None,
                              None) == lib.KVC_E_SHAPE


def test_noalloc_decode_validation(lib):
    """kvc_attn_decode_noalloc validates as kvc_attn_decode does, and refuses a call whose partial
    results would not fit its static scratch -- all before any HIP call."""
    L = lib.lib
    d = _desc(lib, max_seq=4096)
    q = P(0x40000)
    assert L.kvc_attn_decode_noalloc(ctypes.byref(d), 2, q, q, 16, 0.0, 8, None, None) == lib.KVC_E_ARG
    assert L.kvc_attn_decode_noalloc(ctypes.byref(d), 0, None, q, 16, 0.0, 8, None, None) == lib.KVC_E_ARG
    assert L.kvc_attn_decode_noalloc(ctypes.byref(d), 0, q, P(0x40004), 16, 0.0, 8, None, None) == lib.KVC_E_ARG
    assert L.kvc_attn_decode_noalloc(ctypes.byref(d), 0, q, q, 5, 0.0, 8, None, None) == lib.KVC_E_SHAPE
    assert L.kvc_attn_decode_noalloc(ctypes.byref(d), 0, q, q, 16, 0.0, -1, None, None) == lib.KVC_E_ARG
    assert L.kvc_attn_decode_noalloc(ctypes.byref(d), 0, q, q, 16, float("inf"), 8, None, None) == lib.KVC_E_ARG
    # bfloat16, group 4: 2 partial slots x 4 heads x (128 + 2) floats per workgroup = 4160 B; 4033 workgroups
    # is the first count past 16 MiB
    per_wg = 2 * 4 * 130 * 4
    first_over = lib.KVC_DECODE_SCRATCH_MAX_BYTES // per_wg + 1
    assert L.kvc_decode_workspace_bytes(ctypes.byref(d), 16, first_over) > lib.KVC_DECODE_SCRATCH_MAX_BYTES
    assert L.kvc_decode_workspace_bytes(ctypes.byref(d), 16, first_over - 1) <= lib.KVC_DECODE_SCRATCH_MAX_BYTES
    assert L.kvc_attn_decode_noalloc(ctypes.byref(d), 0, q, q, 16, 0.0, first_over, None,
                                     None) == lib.KVC_E_SCRATCH
    # float32: fixed 512-key splits per (row, query head): 64 rows x 16 heads x 2048 splits is far past it
    f = _desc(lib, max_seq=1 << 20, batch=64, dtype=lib.KVC_F32)
    assert L.kvc_attn_decode_noalloc(ctypes.byref(f), 0, q, q, 16, 0.0, 0, None, None) == lib.KVC_E_SCRATCH
    assert "scratch" in lib.kvc_status_string(lib.KVC_E_SCRATCH)


def test_clone_validation(lib):
    L = lib.lib
    src = _desc(lib, batch=1, max_seq=100)
    ok = _desc(lib, batch=8, max_seq=100)
    assert L.kvc_prefill_clone(ctypes.byref(src), 10, ctypes.byref(_desc(lib, batch=8, max_seq=99)), None,
                               None) == lib.KVC_E_CAPACITY
    assert L.kvc_prefill_clone(ctypes.byref(src), 101, ctypes.byref(ok), None, None) == lib.KVC_E_CAPACITY
    assert L.kvc_prefill_clone(ctypes.byref(src), -1, ctypes.byref(ok), None, None) == lib.KVC_E_CAPACITY
    assert L.kvc_prefill_clone(ctypes.byref(_desc(lib, batch=2)), 10, ctypes.byref(ok), None,
                               None) == lib.KVC_E_SHAPE
    assert L.kvc_prefill_clone(ctypes.byref(src), 10, ctypes.byref(_desc(lib, batch=8, n_layers=3, max_seq=100)),
                               None, None) == lib.KVC_E_SHAPE
    assert L.kvc_prefill_clone(ctypes.byref(src), 10, ctypes.byref(_desc(lib, batch=8, n_kv_heads=8, max_seq=100)),
                               None, None) == lib.KVC_E_SHAPE
    assert L.kvc_prefill_clone(ctypes.byref(src), 10,
                               ctypes.byref(_desc(lib, batch=8, max_seq=100, dtype=lib.KVC_F32)), None,
                               None) == lib.KVC_E_DTYPE


def test_decode_step_validation(lib):
    L, d = lib.lib, _desc(lib)  # batch 3, 4 KV heads, head_dim 128, bfloat16
    q = P(0x40000)
    ok = (q, q, q, q, 16, 0.0, 1e4, None, None)
    call = lambda desc, layer, *a: L.kvc_decode_step(ctypes.byref(desc), layer, *a)
    assert call(d, 2, *ok) == lib.KVC_E_ARG                         # layer out of range
    assert call(d, -1, *ok) == lib.KVC_E_ARG
    assert call(d, 0, None, q, q, q, 16, 0.0, 1e4, None, None) == lib.KVC_E_ARG
    assert call(d, 0, q, None, q, q, 16, 0.0, 1e4, None, None) == lib.KVC_E_ARG
    assert call(d, 0, q, q, None, q, 16, 0.0, 1e4, None, None) == lib.KVC_E_ARG
    assert call(d, 0, q, q, q, None, 16, 0.0, 1e4, None, None) == lib.KVC_E_ARG
    assert call(d, 0, P(0x40004), q, q, q, 16, 0.0, 1e4, None, None) == lib.KVC_E_ARG  # misaligned
    assert call(d, 0, q, q, q, q, 16, 0.0, 1.0, None, None) == lib.KVC_E_ARG     # rope base <= 1
    assert call(d, 0, q, q, q, q, 16, 0.0, float("inf"), None, None) == lib.KVC_E_ARG
    assert call(d, 0, q, q, q, q, 16, float("nan"), 1e4, None, None) == lib.KVC_E_ARG
    assert call(d, 0, q, q, q, q, 6, 0.0, 1e4, None, None) == lib.KVC_E_SHAPE   # 6 % 4 != 0
    assert call(d, 0, q, q, q, q, 4 * 17, 0.0, 1e4, None, None) == lib.KVC_E_SHAPE  # group of 17 > 16
    assert call(_desc(lib, head_dim=96), 0, *ok) == lib.KVC_E_SHAPE
    assert call(_desc(lib, dtype=7), 0, *ok) == lib.KVC_E_DTYPE


def test_int8_cache_validation(lib):
    L = lib.lib
    q = P(0x40000)
    no_scales = _desc(lib, dtype=lib.KVC_I8)
    assert L.kvc_attn_decode(ctypes.byref(no_scales), 0, q, q, 16, 0.0, 0, P(0x70000), 1 << 30, None,
                             None) == lib.KVC_E_ARG  # an int8 cache needs both scale arrays
    d = _desc(lib, dtype=lib.KVC_I8)
    d.k_scale, d.v_scale = 0x50000, 0x60000
    bad = _desc(lib, dtype=lib.KVC_I8)
    bad.k_scale, bad.v_scale = 0x50002, 0x60000  # misaligned scale array
    assert L.kvc_rope_append(ctypes.byref(bad), 0, q, q, q, q, 1, 16, 1e4, None, None) == lib.KVC_E_ARG
    assert L.kvc_attn_prefill(ctypes.byref(d), 0, q, q, 4, 16, 0.0, None, None) == lib.KVC_E_DTYPE
    assert L.kvc_decode_step(ctypes.byref(d), 0, q, q, q, q, 16, 0.0, 1e4, None, None) == lib.KVC_E_DTYPE
    # the int8 decode on matrix cores keeps one 32-head block per KV head (group <= 32); a larger
    # group takes the vector kernel's 8-head blocks, like bfloat16
    W = L.kvc_decode_workspace_bytes
    assert W(ctypes.byref(d), 16, 10) == 10 * 2 * 32 * 130 * 4
    assert W(ctypes.byref(d), 4 * 40, 10) == W(ctypes.byref(_desc(lib)), 4 * 40, 10) == 10 * 2 * 8 * 130 * 4
    src = _desc(lib, batch=1, dtype=lib.KVC_I8)
    src.k_scale, src.v_scale = 0x50000, 0x60000
    assert L.kvc_prefill_clone(ctypes.byref(src), 10, ctypes.byref(_desc(lib, batch=8)), None,
                               None) == lib.KVC_E_DTYPE  # int8 source, bfloat16 destination


def test_rolling_window_validation(lib):
    L = lib.lib
    q = P(0x40000)
    d = _desc(lib)  # max_seq 100
    d.rolling = 1
    assert L.kvc_rope_append(ctypes.byref(d), 0, q, q, q, q, 101, 16, 1e4, None, None) == lib.KVC_E_ARG  # T > window
    bad = _desc(lib)
    bad.rolling = 2
    assert L.kvc_attn_decode(ctypes.byref(bad), 0, q, q, 16, 0.0, 0, P(0x70000), 1 << 30, None, None) == lib.KVC_E_ARG


def test_ragged_calls_validation(lib):
    """kvc_rope_append_ragged and kvc_attn_mixed reject bad token layouts and caches before launching."""
    L = lib.lib
    q, cu = P(0x40000), P(0x80000)
    d = _desc(lib, max_seq=4096)  # batch 3, 4 KV heads, bfloat16

    def app(desc=d, cu=cu, n=10, mx=8, hq=16, base=1e4):
        return L.kvc_rope_append_ragged(ctypes.byref(desc), 0, q, q, q, q, cu, n, mx, hq, base, None, None)

    assert app(cu=None) == lib.KVC_E_ARG
    assert app(cu=P(0x80002)) == lib.KVC_E_ARG  # misaligned prefix array
    assert app(n=-1) == lib.KVC_E_ARG
    assert app(mx=0) == lib.KVC_E_ARG
    assert app(hq=6) == lib.KVC_E_SHAPE
    assert app(base=1.0) == lib.KVC_E_ARG
    rolling = _desc(lib, max_seq=100)
    rolling.rolling = 1
    assert app(desc=rolling, mx=101) == lib.KVC_E_ARG  # a row longer than the window

    def mix(desc=d, cu=cu, n=10, mx=8, hq=16, ws=P(0x90000), ws_bytes=1 << 30, nw=0, scale=0.0):
        return L.kvc_attn_mixed(ctypes.byref(desc), 0, q, q, cu, n, mx, hq, scale, nw, ws, ws_bytes, None, None)

    assert mix(cu=None) == lib.KVC_E_ARG
    assert mix(mx=0) == lib.KVC_E_ARG
    assert mix(n=-5) == lib.KVC_E_ARG
    assert mix(nw=-1) == lib.KVC_E_ARG
    assert mix(scale=float("nan")) == lib.KVC_E_ARG
    assert mix(hq=5) == lib.KVC_E_SHAPE
    assert mix(ws=None, ws_bytes=0, nw=8) == lib.KVC_E_WORKSPACE  # the decode rows need the split-KV scratch
    assert mix(ws_bytes=8 * 2 * 4 * 130 * 4 - 4, nw=8) == lib.KVC_E_WORKSPACE  # one float short
    i8 = _desc(lib, dtype=lib.KVC_I8)
    i8.k_scale, i8.v_scale = 0x50000, 0x60000
    assert mix(desc=i8) == lib.KVC_E_DTYPE
    assert L.kvc_attn_mixed(None, 0, q, q, cu, 1, 1, 16, 0.0, 0, None, 0, None, None) == lib.KVC_E_ARG


def test_empty_ragged_calls_are_no_ops(lib):
    """n_tokens = 0 (every row idle): validated, then nothing is launched, so null tensors are fine."""
    L = lib.lib
    d = _desc(lib, max_seq=4096)
    cu = P(0x80000)
    assert L.kvc_rope_append_ragged(ctypes.byref(d), 0, None, None, None, None, cu, 0, 1, 16, 1e4, None,
                                    None) == lib.KVC_OK
    assert L.kvc_attn_mixed(ctypes.byref(d), 0, None, None, cu, 0, 1, 16, 0.0, 0, None, 0, None, None) == lib.KVC_OK
    # the layout is still validated first
    assert L.kvc_rope_append_ragged(ctypes.byref(d), 0, None, None, None, None, None, 0, 1, 16, 1e4, None,
                                    None) == lib.KVC_E_ARG
    assert L.kvc_attn_mixed(ctypes.byref(d), 5, None, None, cu, 0, 1, 16, 0.0, 0, None, 0, None, None) == lib.KVC_E_ARG
