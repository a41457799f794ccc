"""Cake's bidirectional KV-cache preparation, simulated on one GPU.

Cake paper, Section 4 "Design of Cake" and Appendix A: the KV cache of a long
prompt can be computed on the GPU or loaded from slow storage.  Computing a
chunk costs more the later it sits in the prompt (every token attends to all
earlier ones), while loading costs the same for every chunk.  So Cake splits
the prompt into chunks and runs two processes at once: the GPU computes from
the first chunk forward, an I/O process loads stored chunks from the last one
backward, and both stop where they meet.  If either resource slows down, the
meeting point moves.

Here the storage is pinned host memory read at a chosen, throttled rate (the
pages measure against SSDs and network links far slower than PCIe), the
compute side is the library's chunked prefill (kvc_rope_append +
kvc_attn_prefill) on one stream, and the loads are asynchronous host-to-device
copies on a second stream.  BidirectionalLoader holds only the scheduling, so
it runs with any compute and load functions.
"""
from __future__ import annotations

import threading
import time
from dataclasses import dataclass, field

import torch

from . import KVCache, kvc_attn_prefill, kvc_rope_append


@dataclass
class LoadResult:
    """Outcome of one preparation: chunks [0, meet) computed, [meet, n_chunks) loaded."""
    n_chunks: int
    meet: int
    seconds: float
    computed: list = field(default_factory=list)
    loaded: list = field(default_factory=list)


class BidirectionalLoader:
    """The two pointers of Cake's Appendix A.

    compute_fn(c) computes chunk c and returns when it is done; load_fn(c)
    loads chunk c and returns when it is resident.  Chunk c is claimed by
    exactly one side under a lock: the compute side claims chunks upward from
    0 while the next one is below the lowest chunk the I/O side has claimed,
    and the I/O side claims chunks downward from n_chunks - 1 while the next
    one is at or above the compute side's next chunk.  Either side may be
    switched off (compute-only or I/O-only preparation).
    """

    def __init__(self, n_chunks: int, compute_fn=None, load_fn=None):
        if n_chunks < 1:
            raise ValueError("n_chunks must be >= 1")
        if compute_fn is None and load_fn is None:
            raise ValueError("need a compute side, a load side or both")
        self.n = n_chunks
        self.compute_fn, self.load_fn = compute_fn, load_fn

    def run(self) -> LoadResult:
        lock = threading.Lock()
        state = {"compute_next": 0, "io_low": self.n}  # chunks [compute_next, io_low) are unclaimed
        computed, loaded, errors = [], [], []

        def compute_side():
            try:
                while True:
                    with lock:
                        c = state["compute_next"]
                        if c >= state["io_low"]:
                            return
                        state["compute_next"] = c + 1
                    self.compute_fn(c)
                    computed.append(c)
            except BaseException as e:  # surfaced after join
                errors.append(e)

        def io_side():
            try:
                while True:
                    with lock:
                        c = state["io_low"] - 1
                        if c < state["compute_next"]:
                            return
                        state["io_low"] = c
                    self.load_fn(c)
                    loaded.append(c)
            except BaseException as e:
                errors.append(e)

        sides = [s for s, fn in ((compute_side, self.compute_fn), (io_side, self.load_fn)) if fn is not None]
        t0 = time.perf_counter()
        threads = [threading.Thread(target=s, daemon=True) for s in sides]
        for th in threads:
            th.start()
        for th in threads:
            th.join()
        seconds = time.perf_counter() - t0
        if errors:
            raise errors[0]
        return LoadResult(self.n, state["compute_next"] if self.compute_fn else 0, seconds,
                          sorted(computed), sorted(loaded))


class ThrottledStorage:
    """A stored prefix KV cache in pinned host memory, read at `gbps` GB/s.

    k, v: host tensors (n_layers, 1, max_seq, n_kv_heads, head_dim) holding the
    cache of the whole prompt.  load(c) copies chunk c (all layers, K and V)
    into the device cache on its own stream and returns once the copy is done
    and the simulated link has carried the chunk's bytes.
    """

    def __init__(self, k: torch.Tensor, v: torch.Tensor, chunk: int, gbps: float, device):
        if not (k.is_pinned() and v.is_pinned()):
            raise ValueError("storage tensors must be in pinned host memory")
        self.k, self.v, self.chunk, self.gbps = k, v, chunk, float(gbps)
        self.stream = torch.cuda.Stream(device=device)
        self.t_free = None  # when the simulated link is next idle

    def chunk_bytes(self) -> int:
        per_tok = self.k[:, :, 0].numel() * self.k.element_size()
        return 2 * per_tok * self.chunk

    def load(self, c: int, cache: KVCache):
        sl = slice(c * self.chunk, (c + 1) * self.chunk)
        now = time.perf_counter()
        start = now if self.t_free is None or self.t_free < now else self.t_free
        done_at = start + self.chunk_bytes() / (self.gbps * 1e9)
        self.t_free = done_at
        with torch.cuda.stream(self.stream):
            cache.k[:, :, sl].copy_(self.k[:, :, sl], non_blocking=True)
            cache.v[:, :, sl].copy_(self.v[:, :, sl], non_blocking=True)
        self.stream.synchronize()
        delay = done_at - time.perf_counter()
        if delay > 0:
            time.sleep(delay)


def prepare(cache: KVCache, chunks, storage: ThrottledStorage | None, chunk: int, mode: str = "cake",
            dev_err=None) -> LoadResult:
    """Fill a batch-1 cache with the whole prompt's KV cache, Cake's way.

    chunks: list of (q, k, v) device tensors, (1, chunk, heads, head_dim) each,
    the raw projections of every chunk; storage: the stored prefix cache (for
    the "cake" and "io" modes).  mode: "cake" (both sides), "compute" (chunked
    prefill only) or "io" (loads only).  On return every layer of the cache
    holds positions [0, n_chunks * chunk) and seqlens[0] is that length.
    """
    if cache.batch != 1:
        raise ValueError("Cake prepares one request's cache: batch must be 1")
    n = len(chunks)
    dev = cache.k.device
    comp_stream = torch.cuda.Stream(device=dev)
    q_rot = torch.empty_like(chunks[0][0])
    out = torch.empty_like(chunks[0][0])

    def compute(c: int):
        # The compute side runs from chunk 0 up, so chunk c always follows chunks [0, c).
        with torch.cuda.stream(comp_stream):
            cache.seqlens.fill_(c * chunk)
            q, k, v = chunks[c]
            for layer in range(cache.n_layers):
                kvc_rope_append(cache, layer, q, k, v, q_out=q_rot, dev_err=dev_err)
                kvc_attn_prefill(cache, layer, q_rot, out=out, dev_err=dev_err)
        comp_stream.synchronize()

    def load(c: int):
        storage.load(c, cache)

    if mode not in ("cake", "compute", "io"):
        raise ValueError(f"unknown mode {mode}")
    if mode != "compute" and storage is None:
        raise ValueError(f"mode {mode} needs the stored cache")
    loader = BidirectionalLoader(n, compute if mode != "io" else None, load if mode != "compute" else None)
    torch.cuda.synchronize(dev)
    res = loader.run()
    cache.seqlens.fill_(n * chunk)
    torch.cuda.synchronize(dev)
    return res
