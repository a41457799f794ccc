"""The measured-ceiling probes (kv_cache_attention_kvcache_amd.ceilings).

CPU: the separate library loads, exports exactly what ceilings.h declares,
and rejects bad arguments before any launch.  GPU: the probes' rates are
physically plausible for one MI355X (below the published peaks, well above
what a broken probe would give), and the streaming read's byte count follows
its row shape.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CEIL_DIR = os.path.join(ROOT, "kv_cache_attention_kvcache_amd", "ceilings")
LIB = os.path.join(CEIL_DIR, "libkvc_ceilings.so")
HEADER = os.path.join(CEIL_DIR, "ceilings.h")


@pytest.fixture(scope="module")
def ceil():
    if not os.path.exists(LIB):
        import __graft_entry__

        __graft_entry__._build_module().build()
    from kv_cache_attention_kvcache_amd import ceilings

    return ceilings


def _declared():
    return sorted(set(re.findall(r"^\s*int\s+(kvc_\w+)\s*\(", open(HEADER).read(), re.M)))


def test_exports_match_header(ceil):
    assert _declared() == sorted(ceil.EXPORTS)
    raw = ctypes.CDLL(LIB)
    for name in _declared():
        assert hasattr(raw, name), name


def test_libkvc_does_not_export_the_probes():
    import kv_cache_attention_kvcache_amd as kvc

    raw = ctypes.CDLL(kvc.LIB_PATH)
    for name in _declared():
        assert not hasattr(raw, name), name


@pytest.mark.parametrize("rows,row,stride,wg", [
    (0, 256, 256, 1),      # no rows
    (4, 128, 256, 1),      # row not a multiple of 256 bytes
    (4, 512, 256, 1),      # row longer than its stride
    (4, 256, 264, 1),      # stride not 16-byte aligned
    (4, 256, 256, 0),      # no workgroups
])
def test_stream_read_rejects_bad_shapes(ceil, rows, row, stride, wg):
    lib = ceil._load()
    rc = lib.kvc_ceiling_stream_read(ctypes.c_void_p(0x10000), rows, row, stride, 0, wg,
                                     ctypes.c_void_p(0x20000), None)
    assert rc == -1


def test_null_and_misaligned_pointers_rejected(ceil):
    lib = ceil._load()
    assert lib.kvc_ceiling_stream_read(None, 4, 256, 256, 0, 1, ctypes.c_void_p(0x20000), None) == -1
    assert lib.kvc_ceiling_stream_read(ctypes.c_void_p(0x10008), 4, 256, 256, 0, 1,
                                       ctypes.c_void_p(0x20000), None) == -1
    assert lib.kvc_ceiling_stream_read(ctypes.c_void_p(0x10000), 4, 256, 256, 0, 1, None, None) == -1
    for rnd in (0, 1):
        assert lib.kvc_ceiling_mfma_bf16(10, 2, rnd, 1, None, None) == -1
        assert lib.kvc_ceiling_mfma_bf16(0, 2, rnd, 1, ctypes.c_void_p(0x20000), None) == -1
        assert lib.kvc_ceiling_mfma_bf16(10, 3, rnd, 1, ctypes.c_void_p(0x20000), None) == -1
        assert lib.kvc_ceiling_mfma_bf16(10, 2, rnd, 0, ctypes.c_void_p(0x20000), None) == -1
    assert lib.kvc_ceiling_lds_read(10, 1, None, None) == -1
    assert lib.kvc_ceiling_lds_read(0, 1, ctypes.c_void_p(0x20000), None) == -1
    assert lib.kvc_ceiling_lds_read(10, 0, ctypes.c_void_p(0x20000), None) == -1
    k, v, sink = ctypes.c_void_p(0x10000), ctypes.c_void_p(0x40000), ctypes.c_void_p(0x20000)
    assert lib.kvc_ceiling_decode_read(None, v, 8, 64, 8, 4, sink, None) == -1
    assert lib.kvc_ceiling_decode_read(k, ctypes.c_void_p(0x40004), 8, 64, 8, 4, sink, None) == -1
    assert lib.kvc_ceiling_decode_read(k, v, 8, 64, 8, 4, None, None) == -1
    for rows, keys, heads, parts in ((0, 64, 8, 4), (8, 0, 8, 4), (8, 64, 0, 4), (8, 64, 8, 0)):
        assert lib.kvc_ceiling_decode_read(k, v, rows, keys, heads, parts, sink, None) == -1


def test_q8_and_write_probes_reject_bad_arguments(ceil):
    lib = ceil._load()
    k, v, ks, vs, sink = (ctypes.c_void_p(a) for a in (0x10000, 0x40000, 0x80000, 0x90000, 0x20000))
    ok = (4, 64, 64, 8, 0, 4)  # rows, n_keys, max_seq, heads, mode, parts
    bad = [(0, 64, 64, 8, 0, 4), (4, 0, 64, 8, 0, 4), (4, 65, 64, 8, 0, 4), (4, 64, 64, 0, 0, 4),
           (4, 64, 64, 9, 1, 4), (4, 64, 64, 8, 2, 4), (4, 64, 64, 8, 0, 0)]
    for args in bad:
        assert lib.kvc_ceiling_q8_read(k, v, ks, vs, *args, sink, None) == -1, args
    assert lib.kvc_ceiling_q8_read(None, v, ks, vs, *ok, sink, None) == -1
    assert lib.kvc_ceiling_q8_read(k, v, None, vs, *ok, sink, None) == -1
    assert lib.kvc_ceiling_q8_read(k, v, ks, vs, *ok, None, None) == -1
    assert lib.kvc_ceiling_q8_read(ctypes.c_void_p(0x10008), v, ks, vs, *ok, sink, None) == -1
    buf = ctypes.c_void_p(0x10000)
    assert lib.kvc_ceiling_stream_write(None, 4096, 1, 0, None) == -1
    assert lib.kvc_ceiling_stream_write(buf, 4100, 1, 0, None) == -1           # not whole vectors
    assert lib.kvc_ceiling_stream_write(buf, 0, 1, 0, None) == -1
    assert lib.kvc_ceiling_stream_write(ctypes.c_void_p(0x10008), 4096, 1, 0, None) == -1
    assert lib.kvc_ceiling_stream_write(buf, 4096, 0, 8192, None) == -1         # no runs
    assert lib.kvc_ceiling_stream_write(buf, 4096, 2, 2048, None) == -1         # runs overlap
    assert lib.kvc_ceiling_stream_write(buf, 4096, 2, 8200, None) == -1         # stride not whole vectors


@pytest.mark.gpu
def test_measured_ceilings_are_plausible(ceil):
    import torch

    assert torch.cuda.is_available()
    c = ceil.measure(buffer_gib=2, reps=3)
    assert 3000 < c["hbm_read_gbps"]["value"] < 8000
    assert 3000 < c["hbm_read_rows_gbps"]["value"] < 8000
    assert 3000 < c["hbm_read_decode_gbps"]["value"] < 8000
    assert 1500 < c["mfma_bf16_tflops"]["value"] < 2500
    # random operands cost power, never speed: at most the constant-operand rate (plus noise)
    assert 1000 < c["mfma_bf16_random_tflops"]["value"] < c["mfma_bf16_tflops"]["value"] * 1.02
    # 64 banks x 4 bytes per clock per CU at 2.4 GHz over 256 CUs is 157 TB/s
    assert 30 < c["lds_read_tbps"]["value"] < 160


@pytest.mark.gpu
def test_stream_read_counts_row_bytes(ceil):
    import torch

    buf = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    assert ceil.stream_read(buf, 256, 2048, True, 8, sink) == (1 << 20) // 8
    assert ceil.stream_read(buf, 512, 512, False, 8, sink) == 1 << 20
    torch.cuda.synchronize()
    assert int(sink.abs().sum()) == 0  # zeros fold to an XOR of 0, which never matches the sentinel


@pytest.mark.gpu
def test_q8_and_write_probes(ceil):
    """The int8 read probes count 132 bytes per (key, head) for K and V each and read at a
    plausible rate; the write probe writes every byte it is given and nothing past it."""
    import torch

    rows, max_seq, heads, n_keys = 2, 4100, 8, 4099  # a ragged last 32-key tile
    g = torch.Generator(device="cuda").manual_seed(3)
    k = torch.randint(-127, 128, (rows, max_seq, heads, 128), dtype=torch.int8, device="cuda", generator=g)
    v = torch.randint(-127, 128, (rows, max_seq, heads, 128), dtype=torch.int8, device="cuda", generator=g)
    ks = torch.rand(rows, heads, max_seq, device="cuda", generator=g)
    vs = torch.rand(rows, heads, max_seq, device="cuda", generator=g)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    for mode in (0, 1):
        assert ceil.q8_read(k, v, ks, vs, n_keys, mode, 4, sink) == 2 * rows * n_keys * heads * 132
    torch.cuda.synchronize()
    r = ceil.measure_q8(k, v, ks, vs, n_keys, parts=(4, 16), reps=2)
    assert all(10 < x < 8000 for x in r["q8_read_segments_gbps"].values())
    assert 10 < r["q8_read_all_heads_gbps"]["value"] < 8000
    buf = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")
    assert ceil.stream_write(buf, (1 << 20) - 4096) == (1 << 20) - 4096
    torch.cuda.synchronize()
    words = buf.view(torch.int32).view(-1, 4).cpu()
    n16 = ((1 << 20) - 4096) // 16
    assert torch.equal(words[:n16, 0], torch.arange(n16, dtype=torch.int32))
    assert torch.equal(words[:n16, 1:], torch.tensor([0, 2, 3], dtype=torch.int32).expand(n16, 3))
    assert int(words[n16:].abs().sum()) == 0
    # three runs of 80,016 bytes (a ragged last workgroup) at a 262,144-byte stride: only those bytes change
    buf.zero_()
    run, stride = 80016, 1 << 18
    assert ceil.stream_write(buf, run, 3, stride) == 3 * run
    torch.cuda.synchronize()
    words = buf.view(torch.int32).view(-1, 4).cpu()
    want = torch.zeros_like(words)
    for r in range(3):
        v0 = r * stride // 16
        want[v0:v0 + run // 16, 0] = torch.arange(run // 16, dtype=torch.int32)
        want[v0:v0 + run // 16, 1:] = torch.tensor([r, 2, 3], dtype=torch.int32)
    assert torch.equal(words, want)
    big = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
    assert 100 < ceil.measure_write(big, big.numel(), reps=2) < 8000
    assert 100 < ceil.measure_write(big, 16 << 20, 8, 32 << 20, reps=2) < 8000
