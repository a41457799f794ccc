"""A fixed sequence of launches for counter runs that relate kernels to the chip's clock.

    python -m kv_cache_attention_kvcache_amd.ceilings.clock_run

runs, on cuda:0: the matrix-core ceiling loop three times with constant
operands and three times with random ones; the causal prefill
of the last 4096-token chunk of a 73,728-token context six times (64 q / 8 kv
heads, head_dim 128, bf16); and twenty batch-8 decodes at that context.
Under `rocprofv3 --kernel-trace --pmc GRBM_GUI_ACTIVE ...` each dispatch then
carries both its duration and its active cycles (summed over the 8 XCDs), so
its shader clock is cycles / 8 / duration, and SQ_VALU_MFMA_BUSY_CYCLES
(matrix-core work cycles summed over all SIMDs) over cycles / 8 x SIMDs is the
fraction of the time the matrix cores had work.  Inputs are N(0, 1) from a
seeded generator.
"""
from __future__ import annotations

import torch

import kv_cache_attention_kvcache_amd as kvc
from kv_cache_attention_kvcache_amd import ceilings


def main() -> None:
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    bf = torch.bfloat16
    hq, hkv, d, t_chunk, start = 64, 8, 128, 4096, 69632
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    for rnd in (False, True):
        for _ in range(3):
            ceilings.mfma_bf16(2500, 4, cus * 2, sink, random_operands=rnd)
    cache = kvc.KVCache.empty(1, 1, start + t_chunk, hkv, d, dtype=bf, device=dev)
    cache.k.normal_(generator=gen)
    cache.v.normal_(generator=gen)
    cache.seqlens.fill_(start)
    q = torch.randn((1, t_chunk, hq, d), generator=gen, device=dev).to(bf)
    out = torch.empty_like(q)
    for _ in range(6):
        kvc.kvc_attn_prefill(cache, 0, q, out=out)
    del cache, q, out
    rows, ctx = 8, start + t_chunk
    c8 = kvc.KVCache.empty(1, rows, ctx + 1, hkv, d, dtype=bf, device=dev)
    c8.k.normal_(generator=gen)
    c8.v.normal_(generator=gen)
    c8.seqlens.fill_(ctx)
    q8 = torch.randn((rows, 1, hq, d), generator=gen, device=dev).to(bf)
    ws = torch.empty(kvc.kvc_decode_workspace_bytes(c8, hq), dtype=torch.uint8, device=dev)
    for _ in range(20):
        kvc.kvc_attn_decode(c8, 0, q8, workspace=ws)
    torch.cuda.synchronize()
    print("clock_run: done", flush=True)


if __name__ == "__main__":
    main()
