"""Throughput of attention against a KV cache on one MI355X.

One step = one pass of the whole hot path over the long-context workload
(a 73,728-token random sequence, 64 q / 8 kv heads, head_dim 128, bf16):
  1. chunked prefill: 18 chunks of 4096 tokens, each fused RoPE+append then
     causal prefill attention over everything cached so far;
  2. clone of the batch-1 cache into an empty batch-8 cache;
  3. 512 decode steps at batch 1 and 512 at batch 8 (the cloned rows, each
     with its own new tokens): per step RoPE+append, split-KV decode, and
     the caller's seqlens += 1.
All inputs are seeded, synthetic and resident in HBM before timing starts.

Reported: decode attention K/V bytes per second (the JSON `value`), prefill
attention TFLOP/s, the RoPE+append and clone bandwidths (algorithmic bytes:
q read and written, k/v read, K/V slots written; clone source read once and
written to every row), tokens/s, a roofline record for the decode kernel pair
(HIP events around every decode call, on the stream they run on) and the CPU
oracle timed on a bounded sample of the same work.

    python bench.py [--steps K] [--warmup W] [--decode-steps N] [--no-cpu-baseline] [--no-ceilings]

After the timed steps the default run also measures two ceilings of the chip
(kv_cache_attention_kvcache_amd.ceilings): the best streaming-read rate in
decode's access shape (256-byte rows at a 2 KiB stride) and the best bfloat16
matrix-core rate, with constant operands and with random operands that change
every product (the matrix cores then draw more power and the chip holds a
lower clock), and states each roofline against them as well as against the
published peaks: the prefill against the random-operand rate, the data it
computes on being random.

`--workload long_context_int8` runs the same decode steps on an int8 cache
(codes plus one float32 scale per cached vector): the 72K context is written
by the quantizing append alone (prefill attention reads bfloat16 caches
only), then cloned and decoded as above.  Unless --no-ceilings, it then reads
the final batch-8 cache with no arithmetic (whole head rows straight into LDS)
in the decode kernel's own assignment and with all heads of a key range per
workgroup, and reports both rates beside the decode's.

`--workload clone` times the batch-1 -> batch-8 clone of the 72K cache beside a
fill of the same destination bytes and, unless --no-ceilings, a contiguous
streaming write of that many bytes.

`--workload cake` prepares the 72K prompt's KV cache Cake's way (chunked
prefill from the front while a throttled host link loads stored chunks from
the back) and compares it with computing only and loading only, over a range
of simulated link speeds.

`--workload mixed` times one serving step over a ragged batch of eight 72K-token
rows: seven decode one token while the eighth prefills a 2048-token chunk
(kvc_rope_append_ragged + kvc_attn_mixed), beside the decode-only and
chunk-only steps.

`--workload ragged_b64` times ragged batched decode: 64 rows with cached
lengths uniform in [1, 32768] (64 q / 8 kv heads, head_dim 128, bf16), one new
token per row; a step is 80 logical layers of RoPE+append and split-KV decode
over 4 physical layer slices of 8.66 GB each, then seqlens += 1.

`--workload tiny` instead times the two tiny fp32 workloads' decode steps
(one attention layer at batch 1; the six-layer tiny GPT at batch 16), which
are bound by kernel launches: per step through kvc_rope_append +
kvc_attn_decode, through the single-launch kvc_decode_step, and through
kvc_decode_step with the whole step captured once in a HIP graph and replayed.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0      # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA

# HBM traffic per launch of a kernel, measured with rocprofv3 --pmc FETCH_SIZE /
# WRITE_SIZE and scaled by a known-size copy; valid only for the kernel sources
# it was measured on (their SHA-256 is stored beside the figure).
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
CSRC = os.path.join(ROOT, "kv_cache_attention_kvcache_amd", "csrc")


def source_digest(files) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(name: str):
    """Bytes per launch recorded for `name`, or None if absent or its sources changed since."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)[name]
        return rec["bytes_per_launch"] if rec["source_sha256"] == source_digest(rec["sources"]) else None
    except (OSError, KeyError, ValueError):
        return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--workload", choices=["long_context", "long_context_int8", "tiny", "cake", "mixed", "ragged_b64",
                                           "gqa_clone", "clocks", "clone"],
                    default="long_context")
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--decode-steps", type=int, default=None, help="decode steps per batch size (default 512)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the measured-ceiling probes (a streaming read and a matrix-core loop) after the run")
    ap.add_argument("--quiet", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the run, one plain device-to-device copy of this many MiB (a known-size "
                         "kernel whose HBM counters calibrate the profiler's byte counts)")
    return ap.parse_args()


def log(msg, quiet=False):
    if not quiet:
        print(msg, file=sys.stderr, flush=True)


class Timer:
    """HIP events around calls on the current stream; durations read after a sync."""

    def __init__(self):
        self.pairs = []

    def __enter__(self):
        self.e0 = torch.cuda.Event(enable_timing=True)
        self.e1 = torch.cuda.Event(enable_timing=True)
        self.e0.record()
        return self

    def __exit__(self, *a):
        self.e1.record()
        self.pairs.append((self.e0, self.e1))

    def times_ms(self):
        return [a.elapsed_time(b) for a, b in self.pairs]


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path is single-GPU "
              "by design and every figure it reports is one GPU's.", file=sys.stderr)
        sys.exit(2)
    if args.workload == "tiny":
        return bench_tiny(args)
    if args.workload == "long_context_int8":
        return bench_int8(args)
    if args.workload == "cake":
        return bench_cake(args)
    if args.workload == "mixed":
        return bench_mixed(args)
    if args.workload == "ragged_b64":
        return bench_ragged(args)
    if args.workload == "gqa_clone":
        return bench_gqa_clone(args)
    if args.workload == "clocks":
        return bench_clocks(args)
    if args.workload == "clone":
        return bench_clone(args)
    import kv_cache_attention_kvcache_amd as kvc
    import synth

    w = synth.LONG_CONTEXT
    ctx, chunk = w.extra["context"], w.extra["chunk"]
    n_chunks = ctx // chunk
    n_dec = w.extra["steps"] if args.decode_steps is None else args.decode_steps
    rows = w.extra["clone_rows"]
    hq, hkv, d, max_seq = w.n_q_heads, w.n_kv_heads, w.head_dim, w.max_seq
    bf = torch.bfloat16
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    q_ = args.quiet

    # ---------------- inputs (seeded, resident on the device before timing)
    t0 = time.time()
    to_dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(bf).to(dev)
    pq, pk, pv = [], [], []
    for c in range(n_chunks):
        q, k, v = synth.chunk_qkv(w, c, chunk)
        pq.append(to_dev(q[None]))
        pk.append(to_dev(k[None]))
        pv.append(to_dev(v[None]))
    dq = {1: [], rows: []}
    dk = {1: [], rows: []}
    dv = {1: [], rows: []}
    for s in range(n_dec):
        q, k, v = synth.decode_qkv_batch(w, s, rows)
        for b, sl in ((1, slice(0, 1)), (rows, slice(0, rows))):
            dq[b].append(to_dev(q[sl]))
            dk[b].append(to_dev(k[sl]))
            dv[b].append(to_dev(v[sl]))
    log(f"inputs ready in {time.time() - t0:.1f}s", q_)

    cache1 = kvc.KVCache.empty(1, 1, max_seq, hkv, d, dtype=bf, device=dev)
    cache8 = kvc.KVCache.empty(1, rows, max_seq, hkv, d, dtype=bf, device=dev)
    # Batch-1 decode cycles four layer slices of 0.30 GB each, like a four-layer model, so its
    # 1.2 GB working set is far past the 256 MB last-level cache: slice 0 is the prefilled cache,
    # slices 1-3 are clones of it made once before timing.
    n_slices = 4
    slices1 = [cache1] + [kvc.KVCache.empty(1, 1, max_seq, hkv, d, dtype=bf, device=dev) for _ in range(n_slices - 1)]
    ws = torch.empty(max(kvc.kvc_decode_workspace_bytes(cache8, hq), kvc.kvc_decode_workspace_bytes(cache1, hq)),
                     dtype=torch.uint8, device=dev)
    qrot_p = torch.empty((1, chunk, hq, d), dtype=bf, device=dev)
    out_p = torch.empty_like(qrot_p)
    qrot_d = {b: torch.empty((b, 1, hq, d), dtype=bf, device=dev) for b in (1, rows)}
    out_d = {b: torch.empty((b, 1, hq, d), dtype=bf, device=dev) for b in (1, rows)}
    err = torch.zeros(1, dtype=torch.int32, device=dev)

    t_pre, t_app, t_clone, t_dec = Timer(), Timer(), Timer(), {1: Timer(), rows: Timer()}
    phase = {k: Timer() for k in ("prefill", "clone", "decode1", "decode8")}

    def step(timed: bool):
        cache1.seqlens.zero_()
        cache8.seqlens.zero_()
        for c in slices1[1:]:
            c.seqlens.fill_(ctx)
        with phase["prefill"] if timed else _Null():
            for c in range(n_chunks):
                with t_app if timed else _Null():
                    kvc.kvc_rope_append(cache1, 0, pq[c], pk[c], pv[c], q_out=qrot_p, dev_err=err)
                with t_pre if timed else _Null():
                    kvc.kvc_attn_prefill(cache1, 0, qrot_p, out=out_p, dev_err=err)
                cache1.seqlens += chunk
        with phase["clone"] if timed else _Null():
            with t_clone if timed else _Null():
                kvc.kvc_prefill_clone(cache1, ctx, cache8, dev_err=err)
        for b, caches in ((1, slices1), (rows, [cache8])):
            with phase["decode1" if b == 1 else "decode8"] if timed else _Null():
                for s in range(n_dec):
                    for cache in caches:  # the layers of one decode step
                        kvc.kvc_rope_append(cache, 0, dq[b][s], dk[b][s], dv[b][s], q_out=qrot_d[b], dev_err=err)
                        with t_dec[b] if timed else _Null():
                            kvc.kvc_attn_decode(cache, 0, qrot_d[b], out=out_d[b], workspace=ws, dev_err=err)
                    for cache in caches:  # after every layer of the step
                        cache.seqlens += 1

    # the batch-1 slices 1-3: the prompt's cache, cloned once from a prefill of it
    for c in range(n_chunks):
        kvc.kvc_rope_append(cache1, 0, pq[c], pk[c], pv[c], q_out=qrot_p, dev_err=err)
        cache1.seqlens += chunk
    for c in slices1[1:]:
        kvc.kvc_prefill_clone(cache1, ctx, c, dev_err=err)
    torch.cuda.synchronize()
    for i in range(args.warmup):
        step(False)
        torch.cuda.synchronize()
        log(f"warmup step {i} done", q_)
    torch.cuda.synchronize()
    t_start = time.time()
    for i in range(args.steps):
        step(True)
        log(f"timed step {i} enqueued", q_)
    torch.cuda.synchronize()
    wall = time.time() - t_start
    assert err.item() == 0, f"device error bits {err.item()}"

    # ---------------- algorithmic work
    kv_bytes_tok = 2 * hkv * d * 2  # K and V, bf16
    # K/V bytes of all decode calls of one step: batch 1 over four slices, batch 8 over one
    dec_bytes = {1: n_slices * sum((ctx + s + 1) * kv_bytes_tok for s in range(n_dec)),
                 rows: rows * sum((ctx + s + 1) * kv_bytes_tok for s in range(n_dec))}
    dec_calls = {1: n_slices * n_dec, rows: n_dec}
    # RoPE + append of one prefill chunk: q read and q_out written, k/v read, the K and V slots written
    app_bytes = chunk * d * 2 * (2 * hq + 4 * hkv)
    pairs = sum(chunk * (c * chunk) + chunk * (chunk + 1) // 2 for c in range(n_chunks))
    pre_flops = 4 * d * hq * pairs
    K = args.steps
    ms_pre = sum(t_pre.times_ms())
    ms_dec = {b: sum(t_dec[b].times_ms()) for b in (1, rows)}
    dec_total_bytes = K * (dec_bytes[1] + dec_bytes[rows])
    dec_gbps = dec_total_bytes / ((ms_dec[1] + ms_dec[rows]) * 1e-3) / 1e9
    pre_tflops = K * pre_flops / (ms_pre * 1e-3) / 1e12
    # dominant decode launch: batch 8 (2.4 GB of K/V per call)
    per_launch_bytes = dec_bytes[rows] / n_dec
    avg_launch_ms = ms_dec[rows] / (K * n_dec)
    achieved = per_launch_bytes / (avg_launch_ms * 1e-3) / 1e9
    ph = {k: sum(v.times_ms()) / K for k, v in phase.items()}
    clone_gbps = (ctx * kv_bytes_tok * (1 + rows)) / (sum(t_clone.times_ms()) / K * 1e-3) / 1e9
    app_gbps = K * n_chunks * app_bytes / (sum(t_app.times_ms()) * 1e-3) / 1e9
    tokens = ctx + n_dec * (1 + rows)
    ms_step = wall * 1e3 / K
    gbps_b = {b: K * dec_bytes[b] / (ms_dec[b] * 1e-3) / 1e9 for b in (1, rows)}
    res = {
        "metric": "KV-cache decode attn HBM GB/s (% of peak); prefill attn TFLOP/s",
        "value": round(dec_gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "context": ctx, "chunk": chunk, "q_heads": hq, "kv_heads": hkv,
                   "head_dim": d, "decode_steps": n_dec, "decode_batches": [1, rows], "parallelism": "none"},
        "decode_hbm_frac": round(dec_gbps / HBM_PEAK_GBPS, 4),
        "decode_gbps_by_batch": {str(b): round(gbps_b[b], 1) for b in (1, rows)},
        "decode_hbm_frac_by_batch": {str(b): round(gbps_b[b] / HBM_PEAK_GBPS, 4) for b in (1, rows)},
        "decode_us_per_call_by_batch": {str(b): round(ms_dec[b] * 1e3 / (K * dec_calls[b]), 2) for b in (1, rows)},
        "decode_batch1_slices": {"slices": n_slices, "gb_each": round(ctx * kv_bytes_tok / 1e9, 3),
                                 "note": "batch-1 decode cycles four layer slices, 1.2 GB in all, past the "
                                         "256 MB last-level cache"},
        "targets": {"decode_hbm_frac_min": 0.70, "prefill_mfma_frac_min": 0.50,
                    "decode_batch1_meets": bool(gbps_b[1] / HBM_PEAK_GBPS >= 0.70),
                    "decode_batch8_meets": bool(gbps_b[rows] / HBM_PEAK_GBPS >= 0.70),
                    "prefill_meets": bool(pre_tflops / BF16_PEAK_TFLOPS >= 0.50)},
        "prefill_tflops": round(pre_tflops, 1),
        "prefill_mfma_frac": round(pre_tflops / BF16_PEAK_TFLOPS, 4),
        "prefill_ms": round(ms_pre / K, 2),
        "clone_gbps": round(clone_gbps, 1),
        "clone_hbm_frac": round(clone_gbps / HBM_PEAK_GBPS, 4),
        "append_gbps": round(app_gbps, 1),
        "append_hbm_frac": round(app_gbps / HBM_PEAK_GBPS, 4),
        "append_us_per_chunk": round(sum(t_app.times_ms()) / (K * n_chunks) * 1e3, 1),
        "tokens_per_s": round(tokens / (ms_step * 1e-3), 1),
        "phase_ms": {k: round(v, 3) for k, v in ph.items()},
        "roofline": {"bound": "hbm", "kernel": "decode (decode_bf16_kernel + decode_bf16_combine_kernel), batch 8",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic("decode_bf16_b8_72k"),
                     "bytes_per_launch": int(per_launch_bytes), "avg_launch_us": round(avg_launch_ms * 1e3, 2)},
        "roofline_prefill": {"bound": "mfma", "kernel": "prefill_mfma_kernel", "achieved": round(pre_tflops, 1),
                             "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                             "frac": round(pre_tflops / BF16_PEAK_TFLOPS, 4),
                             "flops_per_step": int(pre_flops), "avg_launch_us": round(ms_pre / (K * n_chunks) * 1e3, 1)},
    }
    if not args.no_ceilings:
        from kv_cache_attention_kvcache_amd import ceilings
        torch.cuda.synchronize()
        c = ceilings.measure(dev)
        res["measured_ceilings"] = c
        res["roofline_prefill"]["measured_ceiling_constant_operands"] = c["mfma_bf16_tflops"]["value"]
        # decode against the chip's best plain streaming read (contiguous, 4 GiB); the read in the
        # decode kernel's own assignment is a diagnostic beside it, not the ceiling
        for key, probe in (("roofline", "hbm_read_gbps"), ("roofline_prefill", "mfma_bf16_random_tflops")):
            res[key]["measured_ceiling"] = c[probe]["value"]
            res[key]["measured_ceiling_probe"] = probe
            res[key]["frac_of_measured"] = round(res[key]["achieved"] / c[probe]["value"], 4)
        res["roofline"]["own_pattern_read_gbps"] = c["hbm_read_decode_gbps"]["value"]
        log(f"measured ceilings: {c}", q_)
    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        res["copy_probe_bytes"] = n
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, kv_bytes_tok, q_, step_decode_bytes=dec_bytes[1] + dec_bytes[rows],
                                           prefill_flops=pre_flops)
    print(json.dumps(res), flush=True)


def bench_cake(args):
    """Time to prepare the 72K prompt's cache: compute only, load only, and Cake; one JSON line."""
    import kv_cache_attention_kvcache_amd as kvc
    from kv_cache_attention_kvcache_amd import cake
    import synth

    w = synth.LONG_CONTEXT
    ctx, chunk = w.extra["context"], w.extra["chunk"]
    hkv, d, max_seq = w.n_kv_heads, w.head_dim, w.max_seq
    bf = torch.bfloat16
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    to_dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(bf).to(dev)
    chunks = [tuple(to_dev(a[None]) for a in synth.chunk_qkv(w, c, chunk)) for c in range(ctx // chunk)]
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    ref = kvc.KVCache.empty(1, 1, ctx, hkv, d, dtype=bf, device=dev)
    for _ in range(max(1, args.warmup)):
        cake.prepare(ref, chunks, None, chunk, mode="compute", dev_err=err)
    K = max(1, args.steps)
    med = lambda xs: sorted(xs)[len(xs) // 2]
    t_comp = med([cake.prepare(ref, chunks, None, chunk, mode="compute", dev_err=err).seconds for _ in range(K)])
    kv_bytes = 2 * ctx * hkv * d * 2
    store_k, store_v = ref.k.cpu().pin_memory(), ref.v.cpu().pin_memory()
    got = kvc.KVCache.empty(1, 1, ctx, hkv, d, dtype=bf, device=dev)
    rows = []
    for gbps in (1.0, 2.0, 4.0, 8.0, 16.0):
        store = cake.ThrottledStorage(store_k, store_v, chunk, gbps, dev)
        t_io = med([cake.prepare(got, chunks, store, chunk, mode="io").seconds for _ in range(K)])
        runs = [cake.prepare(got, chunks, store, chunk, mode="cake", dev_err=err) for _ in range(K)]
        t_cake = med([r.seconds for r in runs])
        same = torch.equal(got.k.view(torch.int16), ref.k.view(torch.int16)) and \
            torch.equal(got.v.view(torch.int16), ref.v.view(torch.int16))
        rows.append({"link_gbps": gbps, "io_only_ms": round(t_io * 1e3, 1), "cake_ms": round(t_cake * 1e3, 1),
                     "meet_chunk": sorted(r.meet for r in runs)[len(runs) // 2],
                     "speedup_vs_best_single": round(min(t_comp, t_io) / t_cake, 2), "cache_identical": bool(same)})
        log(f"cake at {gbps} GB/s: {rows[-1]}", args.quiet)
    assert err.item() == 0, f"device error bits {err.item()}"
    best = max(r["speedup_vs_best_single"] for r in rows)
    print(json.dumps({
        "metric": "Cake prefix-cache preparation speedup over the better of compute-only and load-only",
        "value": best, "unit": "x", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(t_comp * 1e3, 2), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name + "_cake", "context": ctx, "chunk": chunk, "layers": 1,
                   "kv_bytes": kv_bytes, "parallelism": "none"},
        "compute_only_ms": round(t_comp * 1e3, 1),
        "compute_equivalent_gbps": round(kv_bytes / t_comp / 1e9, 2),
        "links": rows,
        "roofline": {"bound": "io+mfma", "note": "a scheduler: the time is set by the slower of the two "
                     "sides at their meeting point, not by one kernel"}}), flush=True)


def bench_mixed(args):
    """One serving step over a ragged batch at the long-context shapes; one JSON line.

    Eight rows of 73,728 cached tokens (64 q / 8 kv heads, head_dim 128, bf16): seven decode one
    token each while the eighth prefills a 2048-token chunk at position 73,728 (Cake paper,
    Section 3: a chunk of one request beside the decode tokens of others).  A step is
    kvc_rope_append_ragged + kvc_attn_mixed over the packed 2055 tokens.  The same step with only
    the decode rows and with only the chunk is timed beside it, so that the mixed step can be
    compared with the sum of its parts.
    """
    import kv_cache_attention_kvcache_amd as kvc
    import synth

    w = synth.LONG_CONTEXT
    ctx, hq, hkv, d = w.extra["context"], w.n_q_heads, w.n_kv_heads, w.head_dim
    rows, chunk = 8, 2048
    max_seq = ctx + chunk + 16
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(20251)
    cache = kvc.KVCache.empty(1, rows, max_seq, hkv, d, dtype=torch.bfloat16, device=dev)
    cache.k.normal_(generator=gen)  # the cached history: N(0, 1) values standing for rotated keys
    cache.v.normal_(generator=gen)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    layouts = {"mixed": [1] * (rows - 1) + [chunk], "decode_only": [1] * (rows - 1) + [0],
               "prefill_only": [0] * (rows - 1) + [chunk]}
    inputs = {}
    for name, counts in layouts.items():
        rb = kvc.RaggedBatch(counts, device=dev)
        n = rb.n_tokens
        q = torch.randn((n, hq, d), generator=gen, device=dev).to(torch.bfloat16)
        k = torch.randn((n, hkv, d), generator=gen, device=dev).to(torch.bfloat16)
        v = torch.randn((n, hkv, d), generator=gen, device=dev).to(torch.bfloat16)
        inputs[name] = (rb, q, k, v, torch.empty_like(q), torch.empty_like(q))
    ws = torch.empty(kvc.kvc_decode_workspace_bytes(cache, hq), dtype=torch.uint8, device=dev)
    K = max(1, args.steps) * 5
    res_t = {}
    for name, (rb, q, k, v, q_rot, out) in inputs.items():
        def step():
            cache.seqlens.fill_(ctx)  # every step writes the same slots: constant work
            kvc.kvc_rope_append_ragged(cache, 0, q, k, v, rb, q_out=q_rot, dev_err=err)
            kvc.kvc_attn_mixed(cache, 0, q_rot, rb, out=out, workspace=ws, dev_err=err)
        for _ in range(max(1, args.warmup) * 2):
            step()
        torch.cuda.synchronize()
        t_step, t_attn = Timer(), Timer()
        for _ in range(K):
            cache.seqlens.fill_(ctx)
            with t_step:
                kvc.kvc_rope_append_ragged(cache, 0, q, k, v, rb, q_out=q_rot, dev_err=err)
                with t_attn:
                    kvc.kvc_attn_mixed(cache, 0, q_rot, rb, out=out, workspace=ws, dev_err=err)
        torch.cuda.synchronize()
        res_t[name] = {"step_us": round(sum(t_step.times_ms()) / K * 1e3, 1),
                       "attention_us": round(sum(t_attn.times_ms()) / K * 1e3, 1),
                       "tokens": rb.n_tokens}
        log(f"{name}: {res_t[name]}", args.quiet)
    assert err.item() == 0, f"device error bits {err.item()}"
    m, dec, pre = res_t["mixed"], res_t["decode_only"], res_t["prefill_only"]
    pre_flops = 4 * d * hq * (chunk * ctx + chunk * (chunk + 1) // 2)
    dec_bytes = (rows - 1) * (ctx + 1) * hkv * d * 2 * 2
    pre_tflops = pre_flops / (pre["attention_us"] * 1e-6) / 1e12
    print(json.dumps({
        "metric": "mixed prefill+decode step: new tokens/s", "value": round(m["tokens"] / (m["step_us"] * 1e-6), 1),
        "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": round(m["step_us"] / 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "long_context_72k_mixed_step", "rows": rows, "context": ctx, "chunk": chunk,
                   "decode_rows": rows - 1, "q_heads": hq, "kv_heads": hkv, "head_dim": d, "parallelism": "none"},
        "steps_us": res_t,
        "sum_of_parts_us": round(dec["step_us"] + pre["step_us"], 1),
        "mixed_over_sum_of_parts": round(m["step_us"] / (dec["step_us"] + pre["step_us"]), 4),
        "roofline": {"bound": "mfma", "kernel": "prefill_mfma_kernel over the chunk row (prefill-only step's attention)",
                     "achieved": round(pre_tflops, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(pre_tflops / BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "flops_per_launch": int(pre_flops), "avg_launch_us": pre["attention_us"]},
        "decode_rows_gbps": round(dec_bytes / (dec["attention_us"] * 1e-6) / 1e9, 1),
    }), flush=True)


def bench_ragged(args):
    """Ragged batched decode over streamed layers; one JSON line.

    Batch 64 (64 q / 8 kv heads, head_dim 128, bf16), cached lengths P_b uniform in
    [1, 32768], one new token per row with RoPE at its own offset (nanochat post: the
    new K/V go in place at each row's cache_seqlens).  A step is 80 logical layers of
    kvc_rope_append + kvc_attn_decode over 4 physical layer slices of 8.66 GB (logical
    layer l uses slice l mod 4), then the caller's seqlens += 1.  Every slice is far
    larger than the 256 MB last-level cache, so each decode call streams its K/V from
    HBM.  The cached rows are windows of one seeded N(0, 1) pool, taken as
    already-rotated keys.
    """
    import dataclasses

    import kv_cache_attention_kvcache_amd as kvc
    import synth

    w = synth.RAGGED_DECODE
    n_phys = 4
    b_sz, hq, hkv, d = w.extra["batch"], w.n_q_heads, w.n_kv_heads, w.head_dim
    n_logical = w.extra["logical_layers"]
    if args.steps + args.warmup > w.max_seq - w.extra["len_max"]:
        raise SystemExit(f"at most {w.max_seq - w.extra['len_max']} steps fit the cache's margin")
    bf = torch.bfloat16
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    lengths = synth.ragged_lengths(w)
    offs = synth.ragged_offsets(dataclasses.replace(w, extra={**w.extra, "physical_layers": n_phys}))
    cache = kvc.KVCache.empty(n_phys, b_sz, w.max_seq, hkv, d, dtype=bf, device=dev)
    pool = torch.from_numpy(synth.ragged_pool(w)).to(dev).to(bf)
    for layer in range(n_phys):
        for b in range(b_sz):
            n_b = int(lengths[b])
            for which, t in ((0, cache.k), (1, cache.v)):
                o = int(offs[layer, b, which])
                t[layer, b, :n_b] = pool[o:o + n_b * hkv * d].view(n_b, hkv, d)
    del pool
    to_dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(bf).to(dev)
    new = [tuple(to_dev(a) for a in synth.ragged_new_qkv(w, ell)) for ell in range(n_logical)]
    q_rot = torch.empty((b_sz, 1, hq, d), dtype=bf, device=dev)
    out = torch.empty_like(q_rot)
    ws = torch.empty(kvc.kvc_decode_workspace_bytes(cache, hq), dtype=torch.uint8, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    kv_bytes_tok = 2 * hkv * d * 2  # K and V, bf16
    t_dec = Timer()

    def step(timed):
        for ell in range(n_logical):
            q, k, v = new[ell]
            kvc.kvc_rope_append(cache, ell % n_phys, q, k, v, q_out=q_rot, dev_err=err)
            with t_dec if timed else _Null():
                kvc.kvc_attn_decode(cache, ell % n_phys, q_rot, out=out, workspace=ws, dev_err=err)
        cache.seqlens += 1

    cache.seqlens.copy_(torch.from_numpy(lengths))
    torch.cuda.synchronize()
    for i in range(args.warmup):
        step(False)
        torch.cuda.synchronize()
        log(f"warmup step {i} done", args.quiet)
    base = int(lengths.astype(np.int64).sum()) + b_sz * args.warmup  # cached tokens entering the first timed step
    torch.cuda.synchronize()
    t0 = time.time()
    for i in range(args.steps):
        step(True)
        log(f"timed step {i} enqueued", args.quiet)
    torch.cuda.synchronize()
    wall = time.time() - t0
    assert err.item() == 0, f"device error bits {err.item()}"
    # step s: every decode call sees P_b + s + 1 keys per row (the new token included)
    step_bytes = [n_logical * (base + b_sz * s + b_sz) * kv_bytes_tok for s in range(args.steps)]
    ms_dec = sum(t_dec.times_ms())
    n_calls = args.steps * n_logical
    gbps = sum(step_bytes) / (ms_dec * 1e-3) / 1e9
    per_launch = sum(step_bytes) / n_calls
    ms_step = wall * 1e3 / args.steps
    res = {
        "metric": "KV-cache decode attn HBM GB/s (% of peak)", "value": round(gbps, 1), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 2),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "batch": b_sz, "len_range": [1, w.extra["len_max"]],
                   "mean_cached_len": round(base / b_sz, 1), "q_heads": hq, "kv_heads": hkv, "head_dim": d,
                   "logical_layers": n_logical, "physical_layer_slices": n_phys,
                   "slice_gb": round(cache.k[0].numel() * 2 * 2 / 1e9, 2), "parallelism": "none"},
        "decode_hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
        "tokens_per_s": round(b_sz / (ms_step * 1e-3), 1),
        "decode_ms_per_step": round(ms_dec / args.steps, 2),
        "roofline": {"bound": "hbm", "kernel": "decode (decode_bf16_kernel + decode_bf16_combine_kernel), batch 64",
                     "achieved": round(per_launch / (ms_dec / n_calls * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(per_launch / (ms_dec / n_calls * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic("decode_bf16_ragged_b64"), "bytes_per_launch": int(per_launch),
                     "avg_launch_us": round(ms_dec / n_calls * 1e3, 2)},
    }
    if not args.no_ceilings:
        from kv_cache_attention_kvcache_amd import ceilings
        del cache
        torch.cuda.empty_cache()
        c = ceilings.measure(dev)
        # against the chip's best plain streaming read (contiguous); the row-shaped read is a diagnostic
        res["roofline"]["measured_ceiling"] = c["hbm_read_gbps"]["value"]
        res["roofline"]["measured_ceiling_probe"] = "hbm_read_gbps"
        res["roofline"]["frac_of_measured"] = round(res["roofline"]["achieved"] / c["hbm_read_gbps"]["value"], 4)
        res["roofline"]["row_shaped_read_gbps"] = c["hbm_read_rows_gbps"]["value"]
        res["measured_ceilings"] = {k: c[k] for k in ("hbm_read_gbps", "hbm_read_rows_gbps")}
    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        res["copy_probe_bytes"] = n
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_ragged(w, lengths, offs, kv_bytes_tok, n_logical, args.quiet)
    print(json.dumps(res), flush=True)


def cpu_baseline_ragged(w, lengths, offs, kv_bytes_tok, n_logical, quiet):
    """The oracle on the host for the ragged batch-64 workload: one no-cache decode call per row of
    logical layer 0 (the row's cached K/V taken as rotated, the new token rotated at its offset),
    rows cycled for about 10 s; rate in K/V bytes per second, and the time one 80-layer step of all
    64 rows would take at that rate (an extrapolation, linear in the K/V bytes)."""
    import synth
    from oracle import attention as oatt
    from oracle import numerics

    pool = synth.ragged_pool(w)
    q, k, v = synth.ragged_new_qkv(w, 0)
    hkv, d = w.n_kv_heads, w.head_dim
    with host_threads() as (threads, affinity):
        t0, done, nbytes, b = time.time(), 0, 0, 0
        while time.time() - t0 < 10.0 and done < 64:
            n_b = int(lengths[b])
            kc = numerics.round_to(pool[offs[0, b, 0]:offs[0, b, 0] + n_b * hkv * d].reshape(n_b, hkv, d), "bf16")
            vc = numerics.round_to(pool[offs[0, b, 1]:offs[0, b, 1] + n_b * hkv * d].reshape(n_b, hkv, d), "bf16")
            oatt.decode_over_existing(kc, vc, q[b, 0], k[b, 0], v[b, 0], "bf16")
            done += 1
            nbytes += (n_b + 1) * kv_bytes_tok
            b = (b + 1) % len(lengths)
        dt = time.time() - t0
    rate = nbytes / dt
    step_bytes = n_logical * int((lengths.astype(np.int64) + 1).sum()) * kv_bytes_tok
    log(f"cpu baseline (ragged batch 64): {done} no-cache decode calls in {dt:.1f}s", quiet)
    return {"value": round(rate / 1e9, 3), "unit": "GB/s", "cores": int(threads), "affinity_cpus": int(affinity),
            "kind": "oracle", "tokens_per_s": round(done / dt, 2),
            "extrapolated_step_s": round(step_bytes / rate, 1),
            "extrapolation": "linear in K/V bytes from the sample to one 80-layer step of all 64 rows",
            "sample": f"{done} no-cache decode calls, one per row of logical layer 0 in row order (cached lengths "
                      f"{int(lengths[:done].min())}..{int(lengths[:done].max())}), {dt:.1f} s"}


def bench_int8(args):
    """Decode on an int8 cache at the long-context workload's shapes; one JSON line."""
    import kv_cache_attention_kvcache_amd as kvc
    import synth

    w = synth.LONG_CONTEXT
    ctx, chunk = w.extra["context"], w.extra["chunk"]
    n_dec = w.extra["steps"] if args.decode_steps is None else args.decode_steps
    rows, hq, hkv, d, max_seq = w.extra["clone_rows"], w.n_q_heads, w.n_kv_heads, w.head_dim, w.max_seq
    bf = torch.bfloat16
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    to_dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(bf).to(dev)
    chunks = [tuple(to_dev(a[None]) for a in synth.chunk_qkv(w, c, chunk)) for c in range(ctx // chunk)]
    dec = {1: [], rows: []}
    for s_ in range(n_dec):
        q, k, v = synth.decode_qkv_batch(w, s_, rows)
        for b in (1, rows):
            dec[b].append((to_dev(q[:b]), to_dev(k[:b]), to_dev(v[:b])))
    cache1 = kvc.KVCache.empty(1, 1, max_seq, hkv, d, dtype=torch.int8, device=dev)
    cache8 = kvc.KVCache.empty(1, rows, max_seq, hkv, d, dtype=torch.int8, device=dev)
    ws = torch.zeros(kvc.kvc_decode_workspace_bytes(cache8, hq), dtype=torch.uint8, device=dev)
    qrot = {b: torch.empty((b, 1, hq, d), dtype=bf, device=dev) for b in (1, rows)}
    out = {b: torch.empty((b, 1, hq, d), dtype=bf, device=dev) for b in (1, rows)}
    qrot_p = torch.empty((1, chunk, hq, d), dtype=bf, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    t_dec = {1: Timer(), rows: Timer()}

    def step(timed):
        cache1.seqlens.zero_()
        cache8.seqlens.zero_()
        for q, k, v in chunks:
            kvc.kvc_rope_append(cache1, 0, q, k, v, q_out=qrot_p, dev_err=err)
            cache1.seqlens += chunk
        kvc.kvc_prefill_clone(cache1, ctx, cache8, dev_err=err)
        for b, cache in ((1, cache1), (rows, cache8)):
            for s_ in range(n_dec):
                q, k, v = dec[b][s_]
                kvc.kvc_rope_append(cache, 0, q, k, v, q_out=qrot[b], dev_err=err)
                with t_dec[b] if timed else _Null():
                    kvc.kvc_attn_decode(cache, 0, qrot[b], out=out[b], workspace=ws, dev_err=err)
                cache.seqlens += 1

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    K = args.steps
    t0 = time.time()
    for i in range(K):
        step(True)
        log(f"timed step {i} enqueued", args.quiet)
    torch.cuda.synchronize()
    wall = time.time() - t0
    assert err.item() == 0, f"device error bits {err.item()}"
    vec_bytes = 2 * hkv * (d + 4)  # K and V codes plus their float32 scales, per token
    dec_bytes = {b: b * sum((ctx + s_ + 1) * vec_bytes for s_ in range(n_dec)) for b in (1, rows)}
    ms = {b: sum(t_dec[b].times_ms()) for b in (1, rows)}
    gbps = {b: K * dec_bytes[b] / (ms[b] * 1e-3) / 1e9 for b in (1, rows)}
    total = K * (dec_bytes[1] + dec_bytes[rows]) / ((ms[1] + ms[rows]) * 1e-3) / 1e9
    per_launch = dec_bytes[rows] / n_dec
    avg_ms = ms[rows] / (K * n_dec)
    probes = None
    if not args.no_ceilings:  # the same cache read with no arithmetic, in two assignments
        from kv_cache_attention_kvcache_amd import ceilings

        n_keys = int(cache8.seqlens.min())
        seg = max(1, torch.cuda.get_device_properties(dev).multi_processor_count // (rows * hkv))
        probes = ceilings.measure_q8(cache8.k[0], cache8.v[0], cache8.k_scale[0], cache8.v_scale[0], n_keys,
                                     parts=tuple(sorted({seg, 16, 64})))
        probes["decode_parts_per_segment"] = seg
        probes["n_keys"] = n_keys
        log(f"int8 read probes: {probes}", args.quiet)
    if args.copy_probe_mib > 0:  # a known-size copy that calibrates the profiler's byte counters
        n = args.copy_probe_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
    cpu = None if args.no_cpu_baseline else cpu_baseline_int8(w, vec_bytes, args.quiet)
    print(json.dumps({
        "metric": "KV-cache decode attn HBM GB/s on an int8 cache (codes + scales)", "value": round(total, 1),
        "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / K, 2),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "i8", "data": "synthetic",
        "config": {"workload": w.name + "_int8_decode", "context": ctx, "q_heads": hq, "kv_heads": hkv,
                   "head_dim": d, "decode_steps": n_dec, "decode_batches": [1, rows], "parallelism": "none"},
        "decode_gbps_by_batch": {str(b): round(gbps[b], 1) for b in (1, rows)},
        "decode_us_by_batch": {str(b): round(ms[b] * 1e3 / (K * n_dec), 2) for b in (1, rows)},
        "decode_tokens_per_s_by_batch": {str(b): round(b * K * n_dec / (ms[b] * 1e-3), 1) for b in (1, rows)},
        "roofline": {"bound": "hbm", "kernel": "decode_q8_mfma_kernel + decode_bf16_combine_kernel, batch 8",
                     "achieved": round(per_launch / (avg_ms * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(per_launch / (avg_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic("decode_q8_b8_72k"), "bytes_per_launch": int(per_launch),
                     "avg_launch_us": round(avg_ms * 1e3, 2),
                     "note": "codes + float32 scales per launch; the products run on bf16 matrix cores, "
                             "one workgroup per CU and one tile in flight per wave",
                     **({"measured_ceiling": probes["q8_read_segments_gbps"][str(probes["decode_parts_per_segment"])],
                         "measured_ceiling_probe": "q8_read_segments_gbps at the decode's own parts per segment"}
                        if probes else {})},
        **({"read_probes": probes} if probes else {}),
        **({"cpu_baseline": cpu} if cpu else {})}),
          flush=True)


def cpu_baseline_int8(w, vec_bytes, quiet):
    """The oracle on the host for the int8 cache: no-cache decode of one token over the 73,728-token
    row's stored codes and scales (dequantized, float64 attention), repeated for about 10 s."""
    import synth
    from oracle import numerics, quant

    ctx, chunk = w.extra["context"], w.extra["chunk"]
    ks, vs = [], []
    for c in range(ctx // chunk):
        k, v = synth.chunk_kv(w, c, chunk)
        ks.append(k)
        vs.append(v)
    # the stored history: values rounded to bfloat16, then quantized per vector (keys taken as rotated)
    kc, ksc = quant.quantize_int8(numerics.round_bf16(np.concatenate(ks)))
    vc, vsc = quant.quantize_int8(numerics.round_bf16(np.concatenate(vs)))
    del ks, vs
    qd, kd, vd = synth.decode_qkv(w, 0, 0)
    with host_threads() as (threads, affinity):
        t0, n = time.time(), 0
        while time.time() - t0 < 10.0 and n < 20:
            quant.decode_over_int8(kc, ksc, vc, vsc, qd[0], kd[0], vd[0])
            n += 1
        dt = time.time() - t0
    log(f"cpu baseline (int8): {n} oracle decode calls in {dt:.1f}s", quiet)
    return {"value": round(n * (ctx + 1) * vec_bytes / dt / 1e9, 3), "unit": "GB/s", "cores": int(threads),
            "affinity_cpus": int(affinity), "kind": "oracle",
            "sample": f"{n} no-cache decode calls of one token over the {ctx}-token row's int8 codes and scales "
                      f"(64 q / 8 kv heads, dequantized, float64 attention), {dt:.1f} s"}


def bench_gqa_clone(args):
    """The 2000-token prompt, its clone to eight rows and 256 decode steps per row; one JSON line.

    16 q / 4 kv heads, head_dim 128, bf16, max_seq 4096 (nanochat post, "The prefill trick, 12
    lines": one prompt pass, then N rows sampled from its cache).  A step is RoPE+append and
    causal prefill of the prompt at batch 1, kvc_prefill_clone into an empty batch-8 cache, then
    256 steps of RoPE+append and split-KV decode at batch 8 with distinct per-row tokens.  The
    whole decode working set (33-37 MB) fits the 256 MB last-level cache, so the decode rate is
    stated as effective K/V bytes per second, not as HBM bandwidth.
    """
    import kv_cache_attention_kvcache_amd as kvc
    import synth

    w = synth.GQA_CLONE
    n_prompt, rows, n_dec = w.extra["prompt"], w.extra["n_rows"], w.extra["steps"]
    if args.decode_steps is not None:
        n_dec = args.decode_steps
    hq, hkv, d, max_seq = w.n_q_heads, w.n_kv_heads, w.head_dim, w.max_seq
    bf = torch.bfloat16
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    to_dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(bf).to(dev)
    q, k, v = (to_dev(a[None]) for a in synth.prompt_qkv(w, n_prompt))
    dec = [tuple(to_dev(a) for a in synth.decode_qkv_batch(w, s, rows)) for s in range(n_dec)]
    one = kvc.KVCache.empty(1, 1, max_seq, hkv, d, dtype=bf, device=dev)
    many = kvc.KVCache.empty(1, rows, max_seq, hkv, d, dtype=bf, device=dev)
    ws = torch.empty(kvc.kvc_decode_workspace_bytes(many, hq), dtype=torch.uint8, device=dev)
    q_rot, out = torch.empty_like(q), torch.empty_like(q)
    qd, od = torch.empty((rows, 1, hq, d), dtype=bf, device=dev), torch.empty((rows, 1, hq, d), dtype=bf, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    t_pre, t_clone, t_dec, t_step = Timer(), Timer(), Timer(), Timer()

    def step(timed):
        one.seqlens.zero_()
        many.seqlens.zero_()
        with t_step if timed else _Null():
            kvc.kvc_rope_append(one, 0, q, k, v, q_out=q_rot, dev_err=err)
            with t_pre if timed else _Null():
                kvc.kvc_attn_prefill(one, 0, q_rot, out=out, dev_err=err)
            one.seqlens += n_prompt
            with t_clone if timed else _Null():
                kvc.kvc_prefill_clone(one, n_prompt, many, dev_err=err)
            for s in range(n_dec):
                kvc.kvc_rope_append(many, 0, *dec[s], q_out=qd, dev_err=err)
                with t_dec if timed else _Null():
                    kvc.kvc_attn_decode(many, 0, qd, out=od, workspace=ws, dev_err=err)
                many.seqlens += 1

    for _ in range(max(1, args.warmup)):
        step(False)
    torch.cuda.synchronize()
    K = max(1, args.steps) * 5
    for i in range(K):
        step(True)
    torch.cuda.synchronize()
    assert err.item() == 0, f"device error bits {err.item()}"
    kv_tok = 2 * hkv * d * 2
    pre_flops = 4 * d * hq * n_prompt * (n_prompt + 1) // 2
    clone_bytes = n_prompt * kv_tok * (1 + rows)
    dec_bytes = rows * sum((n_prompt + s + 1) * kv_tok for s in range(n_dec))
    ms = lambda t: sum(t.times_ms()) / K
    pre_tf = pre_flops / (ms(t_pre) * 1e-3) / 1e12
    clone_gbps = clone_bytes / (ms(t_clone) * 1e-3) / 1e9
    dec_gbps = dec_bytes / (ms(t_dec) * 1e-3) / 1e9
    res = {
        "metric": "prompt prefill TFLOP/s, clone GB/s and decode effective K/V GB/s (2000-token prompt, 8 rows)",
        "value": round(dec_gbps, 1), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": max(1, args.warmup),
        "ms_per_step": round(ms(t_step), 3), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "prompt": n_prompt, "rows": rows, "decode_steps": n_dec, "q_heads": hq,
                   "kv_heads": hkv, "head_dim": d, "max_seq": max_seq, "parallelism": "none"},
        "decode_effective_gbps": round(dec_gbps, 1),
        "decode_note": "the decode working set (33-37 MB of K/V per call) is resident in the 256 MB last-level "
                       "cache: an effective rate, not an HBM bandwidth",
        "decode_us_per_call": round(ms(t_dec) * 1e3 / n_dec, 2),
        "decode_tokens_per_s": round(rows * n_dec / (ms(t_dec) * 1e-3), 1),
        "prefill_tflops": round(pre_tf, 2), "prefill_mfma_frac": round(pre_tf / BF16_PEAK_TFLOPS, 4),
        "prefill_us": round(ms(t_pre) * 1e3, 1),
        "prefill_note": "one 2000-token prompt at 16 query heads is 128 workgroups of 256 queries for 256 "
                        "compute units: half the chip has no work",
        "clone_gbps": round(clone_gbps, 1), "clone_us": round(ms(t_clone) * 1e3, 1),
        "clone_bytes": clone_bytes,
        "prefill_units": {"naive": rows * n_prompt * n_prompt, "with_clone": n_prompt * n_prompt},
        "roofline": {"bound": "mfma", "kernel": "prefill_mfma_kernel, 2000-token prompt",
                     "achieved": round(pre_tf, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(pre_tf / BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "flops_per_launch": pre_flops, "avg_launch_us": round(ms(t_pre) * 1e3, 1)},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_gqa(w, n_prompt, rows, n_dec, args.quiet)
    print(json.dumps(res), flush=True)


def cpu_baseline_gqa(w, n_prompt, rows, n_dec, quiet):
    """The oracle on the host for the 2000-token workload: no-cache decode of sampled steps
    (each re-rotating the row's whole history), repeated for about 10 s; rate in K/V bytes per
    second and decode tokens per second over the sample."""
    import synth
    from oracle import attention as oatt

    kv_tok = 2 * w.n_kv_heads * w.head_dim * 2
    q, k, v = synth.prompt_qkv(w, n_prompt)
    steps = [0, n_dec // 4, n_dec // 2, 3 * n_dec // 4, n_dec - 1]
    hist = []
    for s in steps:
        hq_, hk_, hv_ = [q], [k], [v]
        for s2 in range(s + 1):
            a, b, c = synth.decode_qkv(w, s2, 0)
            hq_.append(a)
            hk_.append(b)
            hv_.append(c)
        hist.append((s, np.concatenate(hq_), np.concatenate(hk_), np.concatenate(hv_)))
    with host_threads() as (threads, affinity):
        t0, done, nbytes = time.time(), 0, 0
        while time.time() - t0 < 10.0 and done < 200:  # the sample, repeated for about 10 s
            for s, qa, ka, va in hist:
                oatt.nocache_outputs(qa, ka, va, [n_prompt + s], "bf16")
                done += 1
                nbytes += (n_prompt + s + 1) * kv_tok
        dt = time.time() - t0
    log(f"cpu baseline (2000-token prompt): {done} no-cache decode calls in {dt:.1f}s", quiet)
    return {"value": round(nbytes / dt / 1e9, 3), "unit": "GB/s", "cores": int(threads),
            "affinity_cpus": int(affinity), "kind": "oracle",
            "tokens_per_s": round(done / dt, 2),
            "sample": f"{done} no-cache decode calls of row 0, cycling steps {steps} (each re-rotating the "
                      f"2000-token prompt and the steps so far), {dt:.1f} s"}


def bench_clone(args):
    """The batch-1 -> batch-8 clone of the 73,728-token prompt's cache, beside a plain fill that
    writes the same destination bytes; one JSON line.

    64 q / 8 kv heads, head_dim 128, bf16, max_seq 74,240 (nanochat post, "The prefill trick, 12
    lines").  The clone reads the 0.30 GB source once and writes 2.42 GB; the fill (torch's own
    fill kernel over the same destination slices) writes the 2.42 GB and reads nothing, so it shows
    the write rate this pattern of destination rows allows.  Also the launch sequence the clone's
    counter runs profile.
    """
    import kv_cache_attention_kvcache_amd as kvc
    import synth

    w = synth.LONG_CONTEXT
    ctx, hkv, d, rows = w.extra["context"], w.n_kv_heads, w.head_dim, w.extra["clone_rows"]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    src = kvc.KVCache.empty(1, 1, w.max_seq, hkv, d, dtype=torch.bfloat16, device=dev)
    src.k.normal_(generator=gen)
    src.v.normal_(generator=gen)
    src.seqlens.fill_(ctx)
    dst = kvc.KVCache.empty(1, rows, w.max_seq, hkv, d, dtype=torch.bfloat16, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    K = max(1, args.steps) + 2
    t_clone, t_fill = Timer(), Timer()
    for i in range(K + 1):
        dst.seqlens.zero_()
        with t_clone if i > 0 else _Null():
            kvc.kvc_prefill_clone(src, ctx, dst, dev_err=err)
    for i in range(K + 1):
        with t_fill if i > 0 else _Null():
            dst.k[:, :, :ctx].fill_(1.0)
            dst.v[:, :, :ctx].fill_(1.0)
    torch.cuda.synchronize()
    assert err.item() == 0, f"device error bits {err.item()}"
    if args.copy_probe_mib > 0:  # a known-size copy that calibrates the profiler's byte counters
        n = args.copy_probe_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        torch.empty_like(a).copy_(a)
        torch.cuda.synchronize()
    tok = 2 * hkv * d * 2
    nbytes = ctx * tok * (1 + rows)
    write_probe = None
    if not args.no_ceilings:  # the bytes the clone writes, with no read: in one run, and in its own rows
        from kv_cache_attention_kvcache_amd import ceilings

        wbuf = torch.empty(ctx * tok * rows, dtype=torch.uint8, device=dev)
        contiguous = ceilings.measure_write(wbuf, wbuf.numel())
        del wbuf
        run, stride = ctx * tok // 2, w.max_seq * tok // 2  # one row's K (or V) positions, row to row
        rk, rv = (ceilings.measure_write(t.view(torch.uint8).view(-1), run, rows, stride) for t in (dst.k, dst.v))
        write_probe = {"contiguous": contiguous, "clone_rows": round(2 / (1 / rk + 1 / rv), 1)}
    med = lambda t: sorted(t.times_ms())[len(t.times_ms()) // 2]
    gbps = nbytes / (med(t_clone) * 1e-3) / 1e9
    fill_gbps = ctx * tok * rows / (med(t_fill) * 1e-3) / 1e9
    print(json.dumps({
        "metric": "prefill clone GB/s (source read once + every row written)", "value": round(gbps, 1),
        "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": 1, "ms_per_step": round(med(t_clone), 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name + "_clone", "context": ctx, "rows": rows, "kv_heads": hkv, "head_dim": d,
                   "parallelism": "none"},
        "clone_us": round(med(t_clone) * 1e3, 1), "fill_same_bytes_us": round(med(t_fill) * 1e3, 1),
        "fill_write_gbps": round(fill_gbps, 1),
        **({"write_probe_gbps": write_probe} if write_probe else {}),
        "roofline": {"bound": "hbm", "kernel": "clone_copy_kernel", "achieved": round(gbps, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic("clone_b8_72k"), "bytes_per_launch": nbytes,
                     "avg_launch_us": round(med(t_clone) * 1e3, 1)}}), flush=True)


def bench_clocks(args):
    """A fixed launch sequence for counter runs that relate the kernels to the chip's clock.

    On cuda:0: the matrix-core ceiling loop three times with constant operands and three times
    with random ones; the causal prefill of the last 4096-token chunk of a 73,728-token context
    six times (64 q / 8 kv heads, head_dim 128, bf16); and twenty batch-8 decodes at that context.
    Under `rocprofv3 --kernel-trace --pmc GRBM_GUI_ACTIVE ...` each dispatch then carries both its
    duration and its active cycles (summed over the 8 XCDs), so its shader clock is
    cycles / 8 / duration, and SQ_VALU_MFMA_BUSY_CYCLES (matrix-core work cycles summed over all
    SIMDs) over cycles / 8 x SIMDs is the fraction of the time the matrix cores had work.  Inputs
    are N(0, 1) from a seeded generator.  Prints one JSON line with the event-timed durations.
    """
    import kv_cache_attention_kvcache_amd as kvc
    from kv_cache_attention_kvcache_amd import ceilings

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    bf = torch.bfloat16
    hq, hkv, d, t_chunk, start = 64, 8, 128, 4096, 69632
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    times = {}
    for rnd in (False, True):
        t = Timer()
        for _ in range(3):
            with t:
                ceilings.mfma_bf16(2500, 4, cus * 2, sink, random_operands=rnd)
        times["mfma_loop_random" if rnd else "mfma_loop_constant"] = t
    cache = kvc.KVCache.empty(1, 1, start + t_chunk, hkv, d, dtype=bf, device=dev)
    cache.k.normal_(generator=gen)
    cache.v.normal_(generator=gen)
    cache.seqlens.fill_(start)
    q = torch.randn((1, t_chunk, hq, d), generator=gen, device=dev).to(bf)
    out = torch.empty_like(q)
    t = Timer()
    for _ in range(6):
        with t:
            kvc.kvc_attn_prefill(cache, 0, q, out=out)
    times["prefill_last_72k_chunk"] = t
    torch.cuda.synchronize()
    del cache, q, out
    rows, ctx = 8, start + t_chunk
    c8 = kvc.KVCache.empty(1, rows, ctx + 1, hkv, d, dtype=bf, device=dev)
    c8.k.normal_(generator=gen)
    c8.v.normal_(generator=gen)
    c8.seqlens.fill_(ctx)
    q8 = torch.randn((rows, 1, hq, d), generator=gen, device=dev).to(bf)
    ws = torch.empty(kvc.kvc_decode_workspace_bytes(c8, hq), dtype=torch.uint8, device=dev)
    t = Timer()
    for _ in range(20):
        with t:
            kvc.kvc_attn_decode(c8, 0, q8, workspace=ws)
    times["decode_batch8_72k"] = t
    torch.cuda.synchronize()
    pre_flops = 4 * d * hq * (t_chunk * start + t_chunk * (t_chunk + 1) // 2)
    ms = {k: [round(x, 4) for x in v.times_ms()] for k, v in times.items()}
    best_pre = min(ms["prefill_last_72k_chunk"])
    print(json.dumps({
        "metric": "counter-run launch sequence (event-timed durations, ms)", "value": round(best_pre, 4),
        "unit": "ms", "n_gpus": 1, "steps": 1, "warmup": 0, "ms_per_step": round(best_pre, 4),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "clock_and_counter_sequence", "parallelism": "none"},
        "durations_ms": ms, "prefill_tflops_best": round(pre_flops / (best_pre * 1e-3) / 1e12, 1),
        "roofline": {"bound": "mfma", "kernel": "prefill_mfma_kernel, last 72K chunk",
                     "achieved": round(pre_flops / (best_pre * 1e-3) / 1e12, 1), "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(pre_flops / (best_pre * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                     "traffic": None}}), flush=True)


class _TinyModel:
    """The tiny fp32 workloads' glue around the library: one attention layer
    (x -> qkv -> attention -> out projection) or the six-layer GPT (pre-norm
    RMSNorm, attention, 4x exact-GELU MLP, tied head).  `mode` picks how a
    decode token reaches the cache: "unfused" (kvc_rope_append then
    kvc_attn_decode) or "fused" (kvc_decode_step)."""

    def __init__(self, kvc, w, gpt: bool, mode: str, dev):
        import synth
        self.kvc, self.gpt, self.mode = kvc, gpt, mode
        self.c, self.hq, self.d = w.extra["d_model"], w.n_q_heads, w.head_dim
        to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).float().to(dev)
        if gpt:
            self.n_layers, self.eps = w.extra["n_layers"], w.extra["rms_eps"]
            self.wt = {n: to(a) for n, a in synth.tiny_gpt_weights(w).items()}
            batch = w.extra["batch"]
        else:
            self.n_layers, self.eps = 1, 0.0
            w_qkv, w_out = synth.tiny_layer_weights(w)
            self.wt = {"qkv0": to(w_qkv), "out0": to(w_out)}
            batch = 1
        self.cache = kvc.KVCache.empty(self.n_layers, batch, w.max_seq, w.n_kv_heads, self.d,
                                       dtype=torch.float32, device=dev)
        self.err = torch.zeros(1, dtype=torch.int32, device=dev)

    def _norm(self, x):
        return x * torch.rsqrt((x * x).mean(-1, keepdim=True) + self.eps)

    def step(self, inp):
        """GPT: token ids (B, T) -> logits (B, vocab); layer: x (1, T, C) -> y (1, T, C)."""
        kvc, c, hq, d = self.kvc, self.c, self.hq, self.d
        x = self.wt["emb"][inp] if self.gpt else inp
        b, t = x.shape[0], x.shape[1]
        for layer in range(self.n_layers):
            h = self._norm(x) if self.gpt else x
            qkv = h @ self.wt[f"qkv{layer}"]
            q, k, v = (qkv[..., i * c:(i + 1) * c].reshape(b, t, hq, d).contiguous() for i in range(3))
            if t == 1 and self.mode == "fused":
                o = kvc.kvc_decode_step(self.cache, layer, q, k, v, dev_err=self.err)
            else:
                q_rot = kvc.kvc_rope_append(self.cache, layer, q, k, v, dev_err=self.err)
                o = kvc.kvc_attn_prefill(self.cache, layer, q_rot, dev_err=self.err) if t > 1 else \
                    kvc.kvc_attn_decode(self.cache, layer, q_rot, dev_err=self.err)
            y = o.reshape(b, t, c) @ self.wt[f"out{layer}"]
            if not self.gpt:
                x = y
                continue
            x = x + y
            hmid = torch.nn.functional.gelu(self._norm(x) @ self.wt[f"fc1{layer}"], approximate="none")
            x = x + hmid @ self.wt[f"fc2{layer}"]
        self.cache.seqlens += t
        return self._norm(x[:, -1]) @ self.wt["emb"].T if self.gpt else x


def bench_tiny(args):
    """Decode steps of the two tiny fp32 workloads, three ways; one JSON line."""
    import kv_cache_attention_kvcache_amd as kvc
    import synth

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    torch.backends.cuda.matmul.allow_tf32 = False
    K = max(1, args.steps)
    out = {}
    for name, w, gpt in (("tiny_layer", synth.TINY_LAYER, False), ("tiny_gpt6", synth.TINY_GPT6, True)):
        n_prompt, n_steps = w.extra["prompt"], w.extra["steps"]
        if gpt:
            prompt = torch.from_numpy(synth.tiny_gpt_prompt(w)).to(dev)
        else:
            xs = torch.from_numpy(synth.tiny_layer_inputs(w)[0]).float().to(dev)[None]  # (1, 256, C)
            prompt = xs[:, :n_prompt].contiguous()
            dec_in = [xs[:, n_prompt + s:n_prompt + s + 1].contiguous() for s in range(n_steps)]
        batch = prompt.shape[0]
        res = {}
        for mode in ("unfused", "fused", "fused_graph"):
            m = _TinyModel(kvc, w, gpt, "fused" if mode == "fused_graph" else mode, dev)
            static_in = torch.zeros((batch, 1), dtype=torch.int64, device=dev) if gpt else \
                torch.zeros((1, 1, m.c), dtype=torch.float32, device=dev)
            graph, static_out = None, None
            if mode == "fused_graph":
                # warm up the glue on a side stream, then capture one decode step
                m.step(prompt)
                side = torch.cuda.Stream()
                side.wait_stream(torch.cuda.current_stream())
                with torch.cuda.stream(side):
                    for _ in range(2):
                        m.step(static_in)
                torch.cuda.current_stream().wait_stream(side)
                graph = torch.cuda.CUDAGraph()
                with torch.cuda.graph(graph):
                    static_out = m.step(static_in)
            times = []
            for rep in range(args.warmup + K):
                m.cache.seqlens.zero_()
                last = m.step(prompt)
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for s in range(n_steps):
                    nxt = last.argmax(dim=1)[:, None] if gpt else dec_in[s]
                    if graph is not None:
                        static_in.copy_(nxt)
                        graph.replay()
                        last = static_out
                    else:
                        last = m.step(nxt)
                e1.record()
                torch.cuda.synchronize()
                if rep >= args.warmup:
                    times.append(e0.elapsed_time(e1))
            assert m.err.item() == 0, f"{name} {mode}: device error bits {m.err.item()}"
            ms = sorted(times)[len(times) // 2]
            res[mode] = {"us_per_step": round(ms * 1e3 / n_steps, 2),
                         "tokens_per_s": round(batch * n_steps / (ms * 1e-3), 1),
                         "launches_per_step_attention": m.n_layers * (1 if mode != "unfused" else 2)}
            log(f"{name} {mode}: {res[mode]}", args.quiet)
        out[name] = {"batch": batch, "layers": w.extra["n_layers"] if gpt else 1,
                     "decode_steps": n_steps, **res}
    g = out["tiny_gpt6"]
    cpu = None if args.no_cpu_baseline else cpu_baseline_tiny(args.quiet)
    if cpu:
        for name in ("tiny_layer", "tiny_gpt6"):
            out[name]["oracle_nocache_tokens_per_s"] = cpu["workloads"][name]["tokens_per_s"]
    print(json.dumps({
        "metric": "tiny GPT decode tokens/s (6 layers, batch 16, fp32)",
        "value": g["fused_graph"]["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(g["fused_graph"]["us_per_step"] / 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "tiny_gpt6_fp32 and tiny_layer_fp32 decode", "prompt": 8, "decode_steps": 248,
                   "parallelism": "none"},
        "roofline": {"bound": "launch", "note": "a few microseconds of GPU work per step: the step time is "
                     "launch and glue latency, so a bandwidth or MFMA fraction is not meaningful here"},
        "workloads": out, **({"cpu_baseline": cpu} if cpu else {})}), flush=True)


def cpu_baseline_tiny(quiet):
    """The oracle's no-cache decode loop on the host, as the Tiny-GPT post's no-cache column: every
    step reruns the model over the whole token history (float64 NumPy).  Timed on five steps spread
    over the 248 (history lengths 9 to 256) for every row of the batch; tokens/s = rows per step over
    the mean step time of the sample."""
    import synth
    from oracle import model

    res = {}
    with host_threads() as (threads, affinity):
        t_all = time.time()
        for name, w, gpt in (("tiny_layer", synth.TINY_LAYER, False), ("tiny_gpt6", synth.TINY_GPT6, True)):
            n_prompt, n_steps = w.extra["prompt"], w.extra["steps"]
            steps = [0, n_steps // 4, n_steps // 2, 3 * n_steps // 4, n_steps - 1]
            if gpt:
                weights = synth.tiny_gpt_weights(w)
                prompt = synth.tiny_gpt_prompt(w)
                batch = prompt.shape[0]
                hist = np.concatenate([prompt, np.stack([synth.token_ids(w, n_steps, r) for r in range(batch)])],
                                      axis=1)
            else:
                w_qkv, w_out = synth.tiny_layer_weights(w)
                xs = synth.tiny_layer_inputs(w)[0]
                batch = 1
            t0 = time.time()
            for s in steps:
                n = n_prompt + s + 1
                for r in range(batch):
                    if gpt:
                        model.tiny_gpt_logits_nocache(hist[r, :n], weights, w.extra["n_layers"], w.n_q_heads)
                    else:
                        model.tiny_layer_nocache(xs[:n], w_qkv, w_out, w.n_q_heads)
            dt = (time.time() - t0) / len(steps)
            res[name] = {"tokens_per_s": round(batch / dt, 2), "ms_per_step": round(dt * 1e3, 2), "batch": batch,
                         "sampled_steps": steps}
            log(f"cpu baseline {name}: {res[name]}", quiet)
        total = time.time() - t_all
    g = res["tiny_gpt6"]
    return {"value": g["tokens_per_s"], "unit": "tokens/s", "cores": int(threads), "affinity_cpus": int(affinity),
            "kind": "oracle", "workloads": res,
            "sample": f"the no-cache oracle (float64, whole history rerun every step) at 5 of the 248 decode steps "
                      f"per workload, every row, {total:.1f} s in all; value is the six-layer GPT at batch 16"}


class _Null:
    def __enter__(self):
        return self

    def __exit__(self, *a):
        return False


def cpu_baseline(w, kv_bytes_tok, quiet, step_decode_bytes=None, prefill_flops=None):
    """The oracle, as it is, on the host: no-cache decode of one token at the full
    73,728-token context (every key re-rotated from its raw value, all 64 heads),
    repeated until about 10 s have passed.  Rate in K/V bytes per second, like `value`.

    With `prefill_flops`, also one no-cache call for 8 query positions spread over
    the last prefill chunk (causal, all 64 heads), timed and stated in GFLOP/s of
    attention, with the time the full chunked prefill would take at that rate."""
    import synth
    from oracle import attention as oatt

    with host_threads() as (threads, affinity):
        return _cpu_baseline(w, kv_bytes_tok, quiet, step_decode_bytes, prefill_flops, threads, affinity)


class host_threads:
    """The host cores the oracle may use: the CPUs this process is allowed to run on
    (os.sched_getaffinity), capped by OMP_NUM_THREADS where the machine sets a share; the BLAS
    pools are limited to that many threads while the oracle runs.  Yields (threads, affinity CPUs)."""

    def __enter__(self):
        affinity = len(os.sched_getaffinity(0))
        env = os.environ.get("OMP_NUM_THREADS", "")
        threads = min(affinity, int(env)) if env.isdigit() and int(env) > 0 else affinity
        from threadpoolctl import threadpool_limits
        self._limit = threadpool_limits(limits=threads)
        return threads, affinity

    def __exit__(self, *a):
        self._limit.restore_original_limits()
        return False


def _cpu_baseline(w, kv_bytes_tok, quiet, step_decode_bytes, prefill_flops, threads, affinity):
    import synth
    from oracle import attention as oatt

    ctx = w.extra["context"]
    ks, vs = [], []
    for c in range(ctx // w.extra["chunk"]):
        k, v = synth.chunk_kv(w, c, w.extra["chunk"])
        ks.append(k)
        vs.append(v)
    qd, kd, vd = synth.decode_qkv(w, 0, 0)
    k_all = np.concatenate(ks + [kd])
    v_all = np.concatenate(vs + [vd])
    q_all = np.zeros((ctx + 1, w.n_q_heads, w.head_dim), dtype=np.float32)
    q_all[ctx] = qd[0]
    n, t0 = 0, time.time()
    while True:
        oatt.nocache_outputs(q_all, k_all, v_all, [ctx], "bf16")
        n += 1
        if time.time() - t0 > 10.0 or n >= 20:
            break
    dt = time.time() - t0
    bytes_per = (ctx + 1) * kv_bytes_tok
    log(f"cpu baseline: {n} oracle decode calls in {dt:.1f}s", quiet)
    rate = n * bytes_per / dt
    res = {"value": round(rate / 1e9, 3), "unit": "GB/s", "cores": int(threads), "affinity_cpus": int(affinity),
           "kind": "oracle",
           "sample": f"{n} no-cache decode calls of one token at context {ctx + 1} (64 q / 8 kv heads, "
                     f"all keys re-rotated from raw), {dt:.1f} s"}
    if step_decode_bytes:
        # the no-cache oracle's cost is linear in the keys it re-reads, so one step's decode
        # calls (batch 1 and batch 8) take their K/V bytes over the sampled rate
        res["extrapolated_step_decode_s"] = round(step_decode_bytes / rate, 1)
        res["extrapolation"] = "linear in K/V bytes from the sample to one timed step's decode calls"
    if prefill_flops:
        chunk = w.extra["chunk"]
        start = ctx - chunk  # the last chunk's first position
        q_all[start:ctx] = synth.chunk_qkv(w, ctx // chunk - 1, chunk)[0]
        pos = [start + 511 + 512 * i for i in range(8)]
        fl = 4 * w.head_dim * w.n_q_heads * sum(p + 1 for p in pos)
        t1 = time.time()
        oatt.nocache_outputs(q_all, k_all, v_all, pos, "bf16")
        dt1 = time.time() - t1
        log(f"cpu baseline: prefill sample of {len(pos)} positions in {dt1:.1f}s", quiet)
        res["prefill_sample"] = {
            "gflops": round(fl / dt1 / 1e9, 3), "seconds": round(dt1, 1),
            "sample": f"one no-cache call for {len(pos)} query positions of the last chunk ({pos[0]}..{pos[-1]}, "
                      f"every 512th), all keys up to each re-rotated from raw, {fl / 1e9:.1f} GFLOP of attention",
            "extrapolated_prefill_s": round(prefill_flops / (fl / dt1), 0),
            "extrapolation": "linear in attention flops from the sample to the full 18-chunk prefill"}
    return res


if __name__ == "__main__":
    main()
