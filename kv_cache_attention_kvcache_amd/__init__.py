"""Attention against a KV cache on AMD Instinct MI355X (gfx950).

A thin ctypes binding over ``libkvc.so`` (declared in ``include/kvc.h``).
The functions keep the C names; this module only marshals torch tensors into
pointers, sizes and the current HIP stream -- every step of the computation
runs in the library's HIP kernels.  Importing fails loudly when the library
has not been built: there is no fallback.

    from kv_cache_attention_kvcache_amd import KVCache, kvc_rope_append, kvc_attn_decode
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# KVC_LIB_PATH selects another build of the same library (the host-sanitizer build the CPU tests use)
LIB_PATH = os.environ.get("KVC_LIB_PATH") or os.path.join(_HERE, "libkvc.so")

KVC_F32 = 0
KVC_BF16 = 1
KVC_I8 = 2
KVC_OK = 0
KVC_E_ARG = -1
KVC_E_SHAPE = -2
KVC_E_CAPACITY = -3
KVC_E_DTYPE = -4
KVC_E_WORKSPACE = -5
KVC_E_LAUNCH = -6
KVC_E_SCRATCH = -7
KVC_DECODE_SCRATCH_MAX_BYTES = 16 << 20  # the static scratch behind kvc_attn_decode_noalloc
KVC_DEV_CAPACITY = 1
KVC_DEV_NOT_EMPTY = 2
KVC_DEV_SRC_LEN = 4
KVC_DEV_TOKENS = 8

EXPORTS = ("kvc_rope_append", "kvc_rope_append_ragged", "kvc_decode_workspace_bytes", "kvc_attn_decode",
           "kvc_attn_decode_noalloc", "kvc_attn_prefill", "kvc_attn_mixed", "kvc_decode_step",
           "kvc_prefill_clone", "kvc_status_string")

_DTYPE_CODE = {torch.float32: KVC_F32, torch.bfloat16: KVC_BF16, torch.int8: KVC_I8}


class kvc_cache(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("seqlens", ctypes.c_void_p),
                ("n_layers", ctypes.c_int32), ("batch", ctypes.c_int32), ("max_seq", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p), ("rolling", ctypes.c_int32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python kv_cache_attention_kvcache_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, F32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    cp = ctypes.POINTER(kvc_cache)
    lib.kvc_rope_append.argtypes = [cp, I32, P, P, P, P, I32, I32, F32, P, P]
    lib.kvc_rope_append.restype = ctypes.c_int
    lib.kvc_rope_append_ragged.argtypes = [cp, I32, P, P, P, P, P, I32, I32, I32, F32, P, P]
    lib.kvc_rope_append_ragged.restype = ctypes.c_int
    lib.kvc_attn_mixed.argtypes = [cp, I32, P, P, P, I32, I32, I32, F32, I32, P, SZ, P, P]
    lib.kvc_attn_mixed.restype = ctypes.c_int
    lib.kvc_decode_workspace_bytes.argtypes = [cp, I32, I32]
    lib.kvc_decode_workspace_bytes.restype = SZ
    lib.kvc_attn_decode.argtypes = [cp, I32, P, P, I32, F32, I32, P, SZ, P, P]
    lib.kvc_attn_decode.restype = ctypes.c_int
    lib.kvc_attn_decode_noalloc.argtypes = [cp, I32, P, P, I32, F32, I32, P, P]
    lib.kvc_attn_decode_noalloc.restype = ctypes.c_int
    lib.kvc_attn_prefill.argtypes = [cp, I32, P, P, I32, I32, F32, P, P]
    lib.kvc_attn_prefill.restype = ctypes.c_int
    lib.kvc_decode_step.argtypes = [cp, I32, P, P, P, P, I32, F32, F32, P, P]
    lib.kvc_decode_step.restype = ctypes.c_int
    lib.kvc_prefill_clone.argtypes = [cp, I32, cp, P, P]
    lib.kvc_prefill_clone.restype = ctypes.c_int
    lib.kvc_status_string.argtypes = [ctypes.c_int]
    lib.kvc_status_string.restype = ctypes.c_char_p
    return lib


lib = _load()


class KvcError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {kvc_status_string(status)} (status {status})")
        self.status = status


def kvc_status_string(status: int) -> str:
    return lib.kvc_status_string(int(status)).decode()


def _check(fn: str, status: int):
    if status != KVC_OK:
        raise KvcError(fn, status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, device):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _scratch(nbytes: int, device, stream):
    """A temporary device buffer for one call on `stream`.  torch's caching allocator ties a block
    to the stream it was allocated on, so a buffer used on another stream is recorded there: its
    memory is not handed to new work until that stream's kernels are done with it."""
    t = torch.empty(nbytes, dtype=torch.uint8, device=device)
    _record(t, stream)
    return t


def _record(t, stream):
    if stream is not None and t is not None:
        t.record_stream(stream)


def scale_shape(cache_shape):
    """Shape of an int8 cache's k_scale / v_scale for a (n_layers, batch, max_seq, n_kv_heads, head_dim)
    cache: (n_layers, batch, n_kv_heads, max_seq), head-major."""
    n_layers, batch, max_seq, n_kv_heads = (int(x) for x in tuple(cache_shape)[:4])
    return (n_layers, batch, n_kv_heads, max_seq)


class KVCache:
    """A cache whose buffers are caller-owned torch tensors.

    k, v: (n_layers, batch, max_seq, n_kv_heads, head_dim), float32,
    bfloat16 or int8 (codes), contiguous, on one GPU; seqlens: (batch,) int32
    on that GPU.  An int8 cache also takes k_scale, v_scale: float32
    (n_layers, batch, n_kv_heads, max_seq), one scale per cached vector; its
    queries and outputs are bfloat16.  rolling=True keeps a window of the last
    max_seq positions: position p in slot p mod max_seq, seqlens counting every
    token seen.
    """

    def __init__(self, k: torch.Tensor, v: torch.Tensor, seqlens: torch.Tensor, k_scale=None, v_scale=None,
                 rolling: bool = False):
        if k.shape != v.shape or k.dim() != 5 or k.dtype != v.dtype or k.dtype not in _DTYPE_CODE:
            raise ValueError("k and v must be matching 5-d float32/bfloat16/int8 tensors")
        if not (k.is_contiguous() and v.is_contiguous()) or not (k.is_cuda and v.is_cuda):
            raise ValueError("k and v must be contiguous device tensors")
        if seqlens.dtype != torch.int32 or seqlens.shape != (k.shape[1],) or not seqlens.is_cuda:
            raise ValueError("seqlens must be an int32 (batch,) device tensor")
        if k.dtype == torch.int8:
            for sc in (k_scale, v_scale):
                if sc is None or sc.dtype != torch.float32 or tuple(sc.shape) != scale_shape(k.shape) \
                        or not sc.is_contiguous() or sc.device != k.device:
                    raise ValueError("an int8 cache needs contiguous float32 k_scale and v_scale of shape "
                                     "(n_layers, batch, n_kv_heads, max_seq) on its device")
        self.k, self.v, self.seqlens = k, v, seqlens
        self.k_scale, self.v_scale = (k_scale, v_scale) if k.dtype == torch.int8 else (None, None)
        self._desc = kvc_cache(k.data_ptr(), v.data_ptr(), seqlens.data_ptr(), *[int(s) for s in k.shape],
                               _DTYPE_CODE[k.dtype],
                               self.k_scale.data_ptr() if self.k_scale is not None else None,
                               self.v_scale.data_ptr() if self.v_scale is not None else None, int(bool(rolling)))
        self.rolling = bool(rolling)

    @classmethod
    def empty(cls, n_layers, batch, max_seq, n_kv_heads, head_dim, dtype=torch.bfloat16, device="cuda",
              rolling: bool = False):
        shape = (n_layers, batch, max_seq, n_kv_heads, head_dim)
        scales = (torch.zeros(scale_shape(shape), dtype=torch.float32, device=device),
                  torch.zeros(scale_shape(shape), dtype=torch.float32, device=device)) \
            if dtype == torch.int8 else (None, None)
        return cls(torch.empty(shape, dtype=dtype, device=device), torch.empty(shape, dtype=dtype, device=device),
                   torch.zeros(batch, dtype=torch.int32, device=device), *scales, rolling=rolling)

    @property
    def n_layers(self):
        return self.k.shape[0]

    @property
    def batch(self):
        return self.k.shape[1]

    @property
    def max_seq(self):
        return self.k.shape[2]

    @property
    def n_kv_heads(self):
        return self.k.shape[3]

    @property
    def head_dim(self):
        return self.k.shape[4]

    @property
    def dtype(self):
        """Element type of q, out, k_new and v_new for this cache (bfloat16 for an int8 cache)."""
        return torch.bfloat16 if self.k.dtype == torch.int8 else self.k.dtype

    @property
    def storage_dtype(self):
        return self.k.dtype

    def desc(self):
        return ctypes.byref(self._desc)


def _like(t: torch.Tensor, cache: KVCache, shape, name: str):
    if t.dtype != cache.dtype or not t.is_contiguous() or t.device != cache.k.device or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected contiguous {cache.dtype} {tuple(shape)} on {cache.k.device}, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}")


def kvc_rope_append(cache: KVCache, layer: int, q, k_new, v_new, q_out=None, rope_base: float = 10000.0,
                    dev_err=None, stream=None):
    """Rotate q/k at each row's offset and append k/v in place; returns q_out (rotated q)."""
    b, t, hq, d = q.shape
    _like(q, cache, (cache.batch, t, hq, cache.head_dim), "q")
    _like(k_new, cache, (cache.batch, t, cache.n_kv_heads, cache.head_dim), "k_new")
    _like(v_new, cache, (cache.batch, t, cache.n_kv_heads, cache.head_dim), "v_new")
    if q_out is None:
        q_out = torch.empty_like(q)
        _record(q_out, stream)
    _like(q_out, cache, q.shape, "q_out")
    st = lib.kvc_rope_append(cache.desc(), int(layer), _ptr(q), _ptr(q_out), _ptr(k_new), _ptr(v_new), int(t),
                             int(hq), float(rope_base), _ptr(dev_err), _stream(stream, cache.k.device))
    _check("kvc_rope_append", st)
    return q_out


def kvc_decode_workspace_bytes(cache: KVCache, n_q_heads: int, n_workers: int = 0) -> int:
    return int(lib.kvc_decode_workspace_bytes(cache.desc(), int(n_q_heads), int(n_workers)))


def kvc_attn_decode(cache: KVCache, layer: int, q_rot, out=None, scale: float = 0.0, n_workers: int = 0,
                    workspace=None, dev_err=None, stream=None):
    """One query token per row against layer `layer`'s cached prefix (keys 0..seqlens[b]); returns out.

    n_workers: workgroups the bfloat16 kernel balances the keys over (0 = fill the device)."""
    b, t, hq, d = q_rot.shape
    _like(q_rot, cache, (cache.batch, 1, hq, cache.head_dim), "q_rot")
    if out is None:
        out = torch.empty_like(q_rot)
        _record(out, stream)
    _like(out, cache, q_rot.shape, "out")
    need = kvc_decode_workspace_bytes(cache, hq, n_workers)
    if workspace is None and need > 0:
        workspace = _scratch(need, cache.k.device, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.kvc_attn_decode(cache.desc(), int(layer), _ptr(q_rot), _ptr(out), int(hq), float(scale),
                             int(n_workers), _ptr(workspace), ws_bytes, _ptr(dev_err),
                             _stream(stream, cache.k.device))
    _check("kvc_attn_decode", st)
    return out


def kvc_attn_decode_noalloc(cache: KVCache, layer: int, q_rot, out, scale: float = 0.0, n_workers: int = 0,
                            dev_err=None, stream=None):
    """kvc_attn_decode with its partial results in the library's static device scratch: the
    library allocates nothing, and so does this wrapper (`out` is the caller's).  Calls that
    overlap on one device race on that scratch; calls ordered on one stream do not.  Returns out."""
    b, t, hq, d = q_rot.shape
    _like(q_rot, cache, (cache.batch, 1, hq, cache.head_dim), "q_rot")
    _like(out, cache, q_rot.shape, "out")
    st = lib.kvc_attn_decode_noalloc(cache.desc(), int(layer), _ptr(q_rot), _ptr(out), int(hq), float(scale),
                                     int(n_workers), _ptr(dev_err), _stream(stream, cache.k.device))
    _check("kvc_attn_decode_noalloc", st)
    return out


def kvc_attn_prefill(cache: KVCache, layer: int, q_rot, out=None, scale: float = 0.0, dev_err=None, stream=None):
    """T query tokens per row, causal by absolute position, against layer `layer`; returns out."""
    b, t, hq, d = q_rot.shape
    _like(q_rot, cache, (cache.batch, t, hq, cache.head_dim), "q_rot")
    if out is None:
        out = torch.empty_like(q_rot)
        _record(out, stream)
    _like(out, cache, q_rot.shape, "out")
    st = lib.kvc_attn_prefill(cache.desc(), int(layer), _ptr(q_rot), _ptr(out), int(t), int(hq), float(scale),
                              _ptr(dev_err), _stream(stream, cache.k.device))
    _check("kvc_attn_prefill", st)
    return out


def kvc_decode_step(cache: KVCache, layer: int, q, k_new, v_new, out=None, scale: float = 0.0,
                    rope_base: float = 10000.0, dev_err=None, stream=None):
    """RoPE + append + decode attention for one new token per row in one launch; returns out."""
    b, t, hq, d = q.shape
    _like(q, cache, (cache.batch, 1, hq, cache.head_dim), "q")
    _like(k_new, cache, (cache.batch, 1, cache.n_kv_heads, cache.head_dim), "k_new")
    _like(v_new, cache, (cache.batch, 1, cache.n_kv_heads, cache.head_dim), "v_new")
    if out is None:
        out = torch.empty_like(q)
        _record(out, stream)
    _like(out, cache, q.shape, "out")
    st = lib.kvc_decode_step(cache.desc(), int(layer), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(out), int(hq),
                             float(scale), float(rope_base), _ptr(dev_err), _stream(stream, cache.k.device))
    _check("kvc_decode_step", st)
    return out


class RaggedBatch:
    """The token layout of a ragged call: row b brings counts[b] new tokens, packed in row order.

    cu_tokens is the (batch + 1,) int32 device prefix array the library reads; n_tokens and
    max_tokens are the host-known total and bound the calls take."""

    def __init__(self, counts, device="cuda"):
        counts = [int(c) for c in counts]
        if any(c < 0 for c in counts):
            raise ValueError("token counts must be >= 0")
        cu = [0]
        for c in counts:
            cu.append(cu[-1] + c)
        self.counts = counts
        self.n_tokens = cu[-1]
        self.max_tokens = max(1, max(counts, default=0))
        self.cu_tokens = torch.tensor(cu, dtype=torch.int32, device=device)

    def first(self, b: int) -> int:
        """Packed row of row b's first token."""
        return sum(self.counts[:b])


def kvc_rope_append_ragged(cache: KVCache, layer: int, q, k_new, v_new, rb: RaggedBatch, q_out=None,
                           rope_base: float = 10000.0, dev_err=None, stream=None):
    """kvc_rope_append for a ragged batch: q (n_tokens, Hq, D), k_new/v_new (n_tokens, Hkv, D),
    row b's tokens at the packed rows rb gives it; returns q_out."""
    n, hq, d = q.shape
    _like(q, cache, (rb.n_tokens, hq, cache.head_dim), "q")
    _like(k_new, cache, (rb.n_tokens, cache.n_kv_heads, cache.head_dim), "k_new")
    _like(v_new, cache, (rb.n_tokens, cache.n_kv_heads, cache.head_dim), "v_new")
    if q_out is None:
        q_out = torch.empty_like(q)
        _record(q_out, stream)
    _like(q_out, cache, q.shape, "q_out")
    if rb.cu_tokens.numel() != cache.batch + 1 or rb.cu_tokens.device != cache.k.device:
        raise ValueError("the ragged batch must have batch + 1 prefix entries on the cache's device")
    st = lib.kvc_rope_append_ragged(cache.desc(), int(layer), _ptr(q), _ptr(q_out), _ptr(k_new), _ptr(v_new),
                                    _ptr(rb.cu_tokens), int(rb.n_tokens), int(rb.max_tokens), int(hq),
                                    float(rope_base), _ptr(dev_err), _stream(stream, cache.k.device))
    _check("kvc_rope_append_ragged", st)
    return q_out


def kvc_attn_mixed(cache: KVCache, layer: int, q_rot, rb: RaggedBatch, out=None, scale: float = 0.0,
                   n_workers: int = 0, workspace=None, dev_err=None, stream=None):
    """Attention for a ragged batch: one-token rows decode, longer rows prefill causally; q_rot and
    out are (n_tokens, Hq, D), packed as rb says.  Returns out."""
    n, hq, d = q_rot.shape
    _like(q_rot, cache, (rb.n_tokens, hq, cache.head_dim), "q_rot")
    if out is None:
        out = torch.empty_like(q_rot)
        _record(out, stream)
    _like(out, cache, q_rot.shape, "out")
    if rb.cu_tokens.numel() != cache.batch + 1 or rb.cu_tokens.device != cache.k.device:
        raise ValueError("the ragged batch must have batch + 1 prefix entries on the cache's device")
    need = kvc_decode_workspace_bytes(cache, hq, n_workers)
    if workspace is None and need > 0:
        workspace = _scratch(need, cache.k.device, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.kvc_attn_mixed(cache.desc(), int(layer), _ptr(q_rot), _ptr(out), _ptr(rb.cu_tokens),
                            int(rb.n_tokens), int(rb.max_tokens), int(hq), float(scale), int(n_workers),
                            _ptr(workspace), ws_bytes, _ptr(dev_err), _stream(stream, cache.k.device))
    _check("kvc_attn_mixed", st)
    return out


def kvc_prefill_clone(src: KVCache, src_len: int, dst: KVCache, dev_err=None, stream=None):
    """Copy positions [0, src_len) of the batch-1 cache into every row of the empty batch-N cache."""
    st = lib.kvc_prefill_clone(src.desc(), int(src_len), dst.desc(), _ptr(dev_err), _stream(stream, dst.k.device))
    _check("kvc_prefill_clone", st)
