"""Measured ceilings of the GPU: a streaming read and a matrix-core loop.

A ctypes binding over ``libkvc_ceilings.so`` (declared in ``ceilings.h``) and
``measure()``, which times the two probes with HIP events on torch's current
stream.  The attention kernels' rates can then be stated against what this
chip measurably reaches, next to the published peaks.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvc_ceilings.so")
EXPORTS = ("kvc_ceiling_stream_read", "kvc_ceiling_mfma_bf16", "kvc_ceiling_lds_read", "kvc_ceiling_decode_read",
           "kvc_ceiling_q8_read", "kvc_ceiling_stream_write")
MFMA_FLOPS = 32768  # one 32x32x16 product: 2 * 32 * 32 * 16 flops

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build()")
        lib = ctypes.CDLL(LIB_PATH)
        lib.kvc_ceiling_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int64,
                                                ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
        lib.kvc_ceiling_stream_read.restype = ctypes.c_int
        lib.kvc_ceiling_mfma_bf16.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                              ctypes.c_void_p, ctypes.c_void_p]
        lib.kvc_ceiling_mfma_bf16.restype = ctypes.c_int
        lib.kvc_ceiling_lds_read.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
        lib.kvc_ceiling_lds_read.restype = ctypes.c_int
        lib.kvc_ceiling_decode_read.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                                ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
        lib.kvc_ceiling_decode_read.restype = ctypes.c_int
        lib.kvc_ceiling_q8_read.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int32] * 6 + [ctypes.c_void_p] * 2
        lib.kvc_ceiling_q8_read.restype = ctypes.c_int
        lib.kvc_ceiling_stream_write.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int64,
                                                 ctypes.c_void_p]
        lib.kvc_ceiling_stream_write.restype = ctypes.c_int
        _lib = lib
    return _lib


def _stream_ptr():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def stream_read(buf: torch.Tensor, row_bytes: int, stride_bytes: int, nontemporal: bool, workgroups: int,
                sink: torch.Tensor) -> int:
    """Launch one streaming read over buf (a contiguous uint8 device tensor); returns the bytes read."""
    if buf.dtype != torch.uint8 or not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous uint8 device tensor")
    rows = buf.numel() // stride_bytes
    rc = _load().kvc_ceiling_stream_read(ctypes.c_void_p(buf.data_ptr()), rows, row_bytes, stride_bytes,
                                         int(nontemporal), workgroups, ctypes.c_void_p(sink.data_ptr()),
                                         _stream_ptr())
    if rc != 0:
        raise RuntimeError(f"kvc_ceiling_stream_read failed ({rc})")
    return rows * row_bytes


def mfma_bf16(iters: int, chains: int, workgroups: int, sink: torch.Tensor, random_operands: bool = False) -> float:
    """Launch the matrix-core loop (8 x chains products per wave per iteration); returns its flops."""
    rc = _load().kvc_ceiling_mfma_bf16(iters, chains, int(random_operands), workgroups,
                                       ctypes.c_void_p(sink.data_ptr()), _stream_ptr())
    if rc != 0:
        raise RuntimeError(f"kvc_ceiling_mfma_bf16 failed ({rc})")
    return float(workgroups) * 4 * iters * 8 * chains * MFMA_FLOPS


def lds_read(iters: int, workgroups: int, sink: torch.Tensor) -> int:
    """Launch the LDS read loop (8 waves per workgroup); returns the bytes it reads from LDS."""
    rc = _load().kvc_ceiling_lds_read(iters, workgroups, ctypes.c_void_p(sink.data_ptr()), _stream_ptr())
    if rc != 0:
        raise RuntimeError(f"kvc_ceiling_lds_read failed ({rc})")
    return workgroups * 8 * iters * 16384


def decode_read(k: torch.Tensor, v: torch.Tensor, rows: int, n_keys: int, heads: int, parts: int,
                sink: torch.Tensor) -> int:
    """Launch the read in the decode kernel's assignment over K and V of (rows, n_keys, heads, 256 bytes);
    returns the bytes it reads."""
    need = rows * n_keys * heads * 256
    for t in (k, v):
        if t.dtype != torch.uint8 or not t.is_cuda or not t.is_contiguous() or t.numel() < need:
            raise ValueError(f"k and v must be contiguous uint8 device tensors of at least {need} bytes")
    rc = _load().kvc_ceiling_decode_read(ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()), rows, n_keys,
                                         heads, parts, ctypes.c_void_p(sink.data_ptr()), _stream_ptr())
    if rc != 0:
        raise RuntimeError(f"kvc_ceiling_decode_read failed ({rc})")
    return 2 * need


def q8_read(k: torch.Tensor, v: torch.Tensor, k_scale: torch.Tensor, v_scale: torch.Tensor, n_keys: int,
            mode: int, parts: int, sink: torch.Tensor) -> int:
    """Launch the int8 cache read over keys [0, n_keys) of every row of k, v (int8 or uint8,
    (rows, max_seq, heads, 128)) and their float32 scales (rows, heads, max_seq); mode 0 reads
    in the decode kernel's assignment, mode 1 all heads of a key range per workgroup.  Returns
    the bytes it reads."""
    rows, max_seq, heads, d = k.shape
    if d != 128 or tuple(v.shape) != tuple(k.shape) or tuple(k_scale.shape) != (rows, heads, max_seq) or \
            tuple(v_scale.shape) != tuple(k_scale.shape):
        raise ValueError("k, v must be (rows, max_seq, heads, 128) and the scales (rows, heads, max_seq)")
    for t in (k, v, k_scale, v_scale):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("every operand must be a contiguous device tensor")
    if k.element_size() != 1 or k_scale.dtype != torch.float32 or v_scale.dtype != torch.float32:
        raise ValueError("codes are one byte, scales float32")
    rc = _load().kvc_ceiling_q8_read(ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
                                     ctypes.c_void_p(k_scale.data_ptr()), ctypes.c_void_p(v_scale.data_ptr()),
                                     rows, n_keys, max_seq, heads, mode, parts, ctypes.c_void_p(sink.data_ptr()),
                                     _stream_ptr())
    if rc != 0:
        raise RuntimeError(f"kvc_ceiling_q8_read failed ({rc})")
    return 2 * rows * n_keys * heads * (128 + 4)


def stream_write(buf: torch.Tensor, run_bytes: int, rows: int = 1, stride_bytes: int = 0) -> int:
    """Launch the streaming write of `rows` runs of run_bytes, stride_bytes apart, into buf (a
    contiguous uint8 device tensor); returns the bytes written."""
    need = (rows - 1) * stride_bytes + run_bytes
    if buf.dtype != torch.uint8 or not buf.is_cuda or not buf.is_contiguous() or need > buf.numel():
        raise ValueError(f"buf must be a contiguous uint8 device tensor of at least {need} bytes")
    rc = _load().kvc_ceiling_stream_write(ctypes.c_void_p(buf.data_ptr()), run_bytes, rows, stride_bytes,
                                          _stream_ptr())
    if rc != 0:
        raise RuntimeError(f"kvc_ceiling_stream_write failed ({rc})")
    return rows * run_bytes


def _timed(fn, reps: int) -> float:
    """Seconds per call: one untimed call, then `reps` calls between HIP events on the current stream."""
    fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    e1.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / reps


def measure(device=None, buffer_gib: int = 4, reps: int = 5, decode_shape=(8, 73729, 8)) -> dict:
    """The best rate of each probe over its launch shapes.

    * hbm_read_gbps: contiguous 16-byte loads over `buffer_gib` GiB (far past
      the 256 MB last-level cache), with and without the non-temporal hint.
    * hbm_read_rows_gbps: decode's access shape, 256-byte rows at a 2 KiB
      stride (one KV head's row of a bfloat16 cache with 8 KV heads of 128
      dims), the bytes of the rows only.
    * hbm_read_decode_gbps: the decode kernel's whole read with no arithmetic:
      K and V of `decode_shape` = (rows, keys, KV heads) with 256-byte head
      rows (the batch-8 call at 73,729 keys by default), every (row, head)
      segment cut into 4, 8 or 16 contiguous key ranges, one per workgroup.
    * mfma_bf16_tflops: two or four independent 32x32x16 bfloat16 chains
      per wave, one or two 4-wave workgroups per CU (one or two waves per
      SIMD), with constant operands.
    * mfma_bf16_random_tflops: the same loop on random operands that change
      from one product to the next, as attention's do.  The matrix cores
      draw more power on such data and the chip lowers its clock, so this is
      the rate a bfloat16 contraction over random data can reach.
    * lds_read_tbps: the prefill kernel's LDS operand reads (16-byte reads
      of a padded 16 KB tile, 8 waves per workgroup) at one or two
      workgroups per CU, in TB/s over the whole chip; `bytes_per_clk_per_cu`
      states it per CU at the 2.4 GHz peak clock.
    """
    dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    with torch.cuda.device(dev):
        buf = torch.empty(buffer_gib << 30, dtype=torch.uint8, device=dev)
        buf.fill_(1)
        sink = torch.zeros(4, dtype=torch.int32, device=dev)
        shapes = {}
        for name, row, stride in (("hbm_read_gbps", 256, 256), ("hbm_read_rows_gbps", 256, 2048)):
            best = 0.0
            for nt in (False, True):
                for wpc in (1, 2, 4):
                    nbytes = (buf.numel() // stride) * row
                    t = _timed(lambda: stream_read(buf, row, stride, nt, cus * wpc, sink), reps)
                    rate = nbytes / t / 1e9
                    if rate > best:
                        best, shapes[name] = rate, {"nontemporal": nt, "workgroups_per_cu": wpc}
            shapes[name]["value"] = round(best, 1)
        del buf
        rows, n_keys, heads = decode_shape
        kbuf = torch.empty(rows * n_keys * heads * 256, dtype=torch.uint8, device=dev)
        vbuf = torch.empty_like(kbuf)
        kbuf.fill_(1)
        vbuf.fill_(2)
        best = 0.0
        for parts in (4, 8, 16):
            nbytes = 2 * kbuf.numel()
            t = _timed(lambda: decode_read(kbuf, vbuf, rows, n_keys, heads, parts, sink), reps)
            if nbytes / t / 1e9 > best:
                best, shapes["hbm_read_decode_gbps"] = nbytes / t / 1e9, {
                    "workgroups": rows * heads * parts, "shape": [rows, n_keys, heads, 256]}
        shapes["hbm_read_decode_gbps"]["value"] = round(best, 1)
        del kbuf, vbuf
        for name, rnd in (("mfma_bf16_tflops", False), ("mfma_bf16_random_tflops", True)):
            best = 0.0
            for chains in (2, 4):
                for wpc in (1, 2):
                    iters = 10000 // chains
                    fl = float(cus * wpc) * 4 * iters * 8 * chains * MFMA_FLOPS
                    t = _timed(lambda: mfma_bf16(iters, chains, cus * wpc, sink, rnd), reps)
                    rate = fl / t / 1e12
                    if rate > best:
                        best, shapes[name] = rate, {"chains": chains, "workgroups_per_cu": wpc,
                                                    "random_operands": rnd}
            shapes[name]["value"] = round(best, 1)
        best = 0.0
        for wpc in (1, 2):
            nbytes = cus * wpc * 8 * 4000 * 16384
            t = _timed(lambda: lds_read(4000, cus * wpc, sink), reps)
            if nbytes / t / 1e12 > best:
                best, shapes["lds_read_tbps"] = nbytes / t / 1e12, {"workgroups_per_cu": wpc}
        shapes["lds_read_tbps"]["value"] = round(best, 1)
        shapes["lds_read_tbps"]["bytes_per_clk_per_cu"] = round(best * 1e12 / cus / 2.4e9, 1)
    return shapes


def measure_q8(k: torch.Tensor, v: torch.Tensor, k_scale: torch.Tensor, v_scale: torch.Tensor, n_keys: int,
               parts=(4, 16, 64), reps: int = 5) -> dict:
    """Read rates (GB/s) of an int8 cache of the caller's shape, whole head rows landing in LDS:

    * q8_read_segments_gbps: one key range of one (row, KV head) segment per
      workgroup, for each count of ranges per segment in `parts` (the decode
      kernel's own assignment is one of them: its persistent grid of one
      workgroup per CU cut into segments);
    * q8_read_all_heads_gbps: one key range of a row per workgroup with every
      KV head of it, so the four waves read whole key rows (heads * 128 bytes)
      at a time; the best of 64, 128 and 256 ranges per row.
    """
    sink = torch.zeros(4, dtype=torch.int32, device=k.device)
    nbytes = 2 * k.shape[0] * n_keys * k.shape[2] * 132
    rate = lambda mode, pp: nbytes / _timed(lambda: q8_read(k, v, k_scale, v_scale, n_keys, mode, pp, sink),
                                            reps) / 1e9
    seg = {str(pp): round(rate(0, pp), 1) for pp in parts}
    allh = {str(pp): round(rate(1, pp), 1) for pp in (64, 128, 256)}
    return {"q8_read_segments_gbps": seg, "q8_read_all_heads_gbps": {"value": max(allh.values()), "by_parts": allh}}


def measure_write(buf: torch.Tensor, run_bytes: int, rows: int = 1, stride_bytes: int = 0, reps: int = 5) -> float:
    """Rate (GB/s) of the streaming write of `rows` runs of run_bytes, stride_bytes apart, into buf."""
    t = _timed(lambda: stream_write(buf, run_bytes, rows, stride_bytes), reps)
    return round(rows * run_bytes / t / 1e9, 1)
