"""The five workloads end to end on the GPU, against the no-cache oracle (GPU).

Each test runs the HIP library at the workload's real shapes -- the RoPE +
append, prefill, decode and clone calls in the order a caller makes them --
and compares with the CPU oracle recomputing attention from scratch over the
same raw inputs.  Where the oracle would take minutes at full size, it checks
sampled query rows, layers and steps; the GPU still runs the whole workload.

Projections, norms, MLP and logits of the two tiny fp32 models are torch
float32 ops around the library calls: they are the model the pages run, not
part of the attention path.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import attention as oatt
from oracle import model as omodel
from oracle import numerics, rope
from tests import gates
from tests.gpu_util import bits, dev, host64, rope_error_ok, rope_excess_ratio

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _exact_fp32():
    """Full float32 GEMMs in the tiny models' torch glue (no reduced-precision modes)."""
    old = torch.backends.cuda.matmul.allow_tf32
    torch.backends.cuda.matmul.allow_tf32 = False
    yield
    torch.backends.cuda.matmul.allow_tf32 = old


def _t(x, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(x)).to(dtype).cuda()


# ---------------------------------------------------------------- tiny layer (fp32)

def test_tiny_layer_cached_equals_nocache_every_step(kvc):
    """Single fp32 attention layer: 8-token prompt, then 248 cached decode steps; every
    step's output equals the no-cache rerun over the whole history (Tiny-GPT post,
    "The Cache, in Code": the cache changes nothing)."""
    w = synth.TINY_LAYER
    c, hq, d = w.extra["d_model"], w.n_q_heads, w.head_dim
    n_prompt, n_steps = w.extra["prompt"], w.extra["steps"]
    w_qkv, w_out = synth.tiny_layer_weights(w)
    x = synth.tiny_layer_inputs(w)[0]  # (256, C)
    wq, wo = _t(w_qkv), _t(w_out)
    cache = kvc.KVCache.empty(1, 1, w.max_seq, w.n_kv_heads, d, dtype=torch.float32)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")

    def layer(xs):  # xs: (T, C) -> (T, C)
        t = xs.shape[0]
        qkv = _t(xs) @ wq
        q, k, v = (qkv[:, i * c:(i + 1) * c].reshape(1, t, hq, d).contiguous() for i in range(3))
        q_rot = kvc.kvc_rope_append(cache, 0, q, k, v, dev_err=err)
        o = kvc.kvc_attn_prefill(cache, 0, q_rot, dev_err=err) if t > 1 else \
            kvc.kvc_attn_decode(cache, 0, q_rot, dev_err=err)
        cache.seqlens += t
        return (o.reshape(t, c) @ wo).cpu().numpy().astype(np.float64)

    outs = [layer(x[:n_prompt])]
    for s in range(n_steps):
        outs.append(layer(x[n_prompt + s:n_prompt + s + 1]))
    torch.cuda.synchronize()
    assert err.item() == 0
    got = np.concatenate(outs)
    ref = omodel.tiny_layer_nocache(x, w_qkv, w_out, hq, context=w.max_seq)
    # the causal rerun's row p is the no-cache output at step p: check every position
    gates.check(got, ref, "f32", "tiny layer, all 256 positions")
    # and literally rerun from scratch for a few steps
    for p in (8, 9, 100, 255):
        step_ref = omodel.tiny_layer_nocache(x[:p + 1], w_qkv, w_out, hq, context=w.max_seq)[-1]
        gates.check(got[p], step_ref, "f32", f"tiny layer, step at position {p}")


# ---------------------------------------------------------------- tiny GPT (fp32, B=16)

class _GpuTinyGPT:
    """The six-layer tiny GPT on the GPU: torch float32 glue, attention in the library."""

    def __init__(self, kvc, weights, w):
        self.kvc, self.w = kvc, w
        self.c, self.hq, self.d = w.extra["d_model"], w.n_q_heads, w.head_dim
        self.n_layers, self.eps = w.extra["n_layers"], w.extra["rms_eps"]
        self.wt = {k: _t(v) for k, v in weights.items()}
        self.cache = kvc.KVCache.empty(self.n_layers, w.extra["batch"], w.max_seq, w.n_kv_heads, self.d,
                                       dtype=torch.float32)
        self.err = torch.zeros(1, dtype=torch.int32, device="cuda")

    def _norm(self, x):
        return x * torch.rsqrt((x * x).mean(-1, keepdim=True) + self.eps)

    def step(self, tokens):
        """tokens (B, T) int64 -> last-position logits (B, vocab), float32."""
        kvc, c, hq, d = self.kvc, self.c, self.hq, self.d
        b, t = tokens.shape
        x = self.wt["emb"][tokens]
        for layer in range(self.n_layers):
            qkv = self._norm(x) @ self.wt[f"qkv{layer}"]
            q, k, v = (qkv[..., i * c:(i + 1) * c].reshape(b, t, hq, d).contiguous() for i in range(3))
            q_rot = kvc.kvc_rope_append(self.cache, layer, q, k, v, dev_err=self.err)
            o = kvc.kvc_attn_prefill(self.cache, layer, q_rot, dev_err=self.err) if t > 1 else \
                kvc.kvc_attn_decode(self.cache, layer, q_rot, dev_err=self.err)
            x = x + o.reshape(b, t, c) @ self.wt[f"out{layer}"]
            hmid = torch.nn.functional.gelu(self._norm(x) @ self.wt[f"fc1{layer}"], approximate="none")
            x = x + hmid @ self.wt[f"fc2{layer}"]
        self.cache.seqlens += t  # after every layer of the step (nanochat post)
        return self._norm(x[:, -1]) @ self.wt["emb"].T


def test_tiny_gpt_b16_greedy_matches_nocache_logits(kvc):
    """Six fp32 layers, batch 16, 8-token prompts, 248 greedy steps through the cache.
    At sampled steps every row's logits equal the oracle's full no-cache rerun of that
    row's token history, and the greedy pick agrees except within the pages' near-tie
    margin (top-2 gap below 1e-4)."""
    w = synth.TINY_GPT6
    weights = synth.tiny_gpt_weights(w)
    prompts = synth.tiny_gpt_prompt(w)  # (16, 8)
    gpt = _GpuTinyGPT(kvc, weights, w)
    hist = prompts.copy()
    logits = gpt.step(torch.from_numpy(prompts).cuda())
    check_steps = {0, 1, 7, 60, 150, w.extra["steps"] - 1}
    for s in range(w.extra["steps"]):
        lg = logits.float().cpu().numpy().astype(np.float64)
        nxt = lg.argmax(axis=1)
        if s in check_steps:
            for b in range(hist.shape[0]):
                ref = omodel.tiny_gpt_logits_nocache(hist[b], weights, w.extra["n_layers"], w.n_q_heads,
                                                     context=w.max_seq, eps=w.extra["rms_eps"])
                gates.check(lg[b], ref, "f32", f"tiny GPT logits, step {s} row {b}")
                if nxt[b] != omodel.greedy(ref):
                    assert omodel.top2_gap(ref) < 1e-4, f"greedy disagreement at step {s} row {b}"
        hist = np.concatenate([hist, nxt[:, None]], axis=1)
        if s + 1 < w.extra["steps"]:
            logits = gpt.step(torch.from_numpy(nxt[:, None]).cuda())
    torch.cuda.synchronize()
    assert gpt.err.item() == 0
    assert gpt.cache.seqlens.cpu().tolist() == [8 + w.extra["steps"] - 1] * 16


# ---------------------------------------------------------------- GQA prompt + clone (bf16)

def test_gqa_prompt_prefill_clone_and_diverging_rows(kvc):
    """One 2000-token prompt prefilled at batch 1 (16 q / 4 kv heads, head_dim 128), cloned
    into 8 rows, then 256 decode steps with distinct per-row tokens (nanochat post, "The
    prefill trick, 12 lines"): prefill rows, the clone (bit-exact) and every row's decode
    outputs match the oracle's no-cache recompute of that row's own history."""
    w = synth.GQA_CLONE
    n_prompt, n_rows, n_steps = w.extra["prompt"], w.extra["n_rows"], w.extra["steps"]
    hq, hkv, d = w.n_q_heads, w.n_kv_heads, w.head_dim
    bf = torch.bfloat16
    q, k, v = synth.prompt_qkv(w, n_prompt)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    one = kvc.KVCache.empty(1, 1, w.max_seq, hkv, d, dtype=bf)
    q_rot = kvc.kvc_rope_append(one, 0, dev(q[None], "bf16"), dev(k[None], "bf16"), dev(v[None], "bf16"), dev_err=err)
    pre = kvc.kvc_attn_prefill(one, 0, q_rot, dev_err=err)
    one.seqlens += n_prompt
    rows_chk = np.array([0, 1, 63, 64, 1000, 1998, 1999])
    ref = oatt.nocache_outputs(q, k, v, rows_chk, "bf16")
    gates.check(host64(pre)[0, rows_chk], ref, "bf16", "2000-token prefill")

    many = kvc.KVCache.empty(1, n_rows, w.max_seq, hkv, d, dtype=bf)
    kvc.kvc_prefill_clone(one, n_prompt, many, dev_err=err)
    torch.cuda.synchronize()
    assert many.seqlens.cpu().tolist() == [n_prompt] * n_rows
    sk, sv = bits(one.k[:, 0, :n_prompt]), bits(one.v[:, 0, :n_prompt])
    for r in range(n_rows):
        assert np.array_equal(bits(many.k[:, r, :n_prompt]), sk) and np.array_equal(bits(many.v[:, r, :n_prompt]), sv)

    hist_q = [[] for _ in range(n_rows)]
    hist_k = [[] for _ in range(n_rows)]
    hist_v = [[] for _ in range(n_rows)]
    check_steps = {0, 1, 100, n_steps - 1}
    solo = kvc.KVCache.empty(1, 1, w.max_seq, hkv, d, dtype=bf)  # row 3 alone, for clone == independent
    kvc.kvc_prefill_clone(one, n_prompt, solo, dev_err=err)
    for s in range(n_steps):
        qs, ks, vs = synth.decode_qkv_batch(w, s, n_rows)
        for r in range(n_rows):
            hist_q[r].append(qs[r, 0]); hist_k[r].append(ks[r, 0]); hist_v[r].append(vs[r, 0])
        q_rot = kvc.kvc_rope_append(many, 0, dev(qs, "bf16"), dev(ks, "bf16"), dev(vs, "bf16"), dev_err=err)
        out = kvc.kvc_attn_decode(many, 0, q_rot, dev_err=err)
        q_solo = kvc.kvc_rope_append(solo, 0, dev(qs[3:4], "bf16"), dev(ks[3:4], "bf16"), dev(vs[3:4], "bf16"),
                                     dev_err=err)
        out_solo = kvc.kvc_attn_decode(solo, 0, q_solo, dev_err=err)
        if s in check_steps:
            o = host64(out)[:, 0]
            for r in range(n_rows):
                qa = np.concatenate([q, np.stack(hist_q[r])])
                ka = np.concatenate([k, np.stack(hist_k[r])])
                va = np.concatenate([v, np.stack(hist_v[r])])
                ref = oatt.nocache_outputs(qa, ka, va, [n_prompt + s], "bf16")[0]
                gates.check(o[r], ref, "bf16", f"decode step {s} row {r}")
            gates.check(host64(out_solo)[0, 0], o[3], "bf16", f"row 3 alone vs in the batch, step {s}")
        many.seqlens += 1
        solo.seqlens += 1
    torch.cuda.synchronize()
    assert err.item() == 0


# ---------------------------------------------------------------- ragged batch-64 decode (bf16)

def test_ragged_b64_decode_over_streamed_layers(kvc):
    """Batch 64 (64 q / 8 kv heads, head_dim 128), cached lengths uniform in [1, 32768],
    one new token per row with RoPE at its own offset, 80 logical layers streamed over
    the physical cache slices.  Logical layers 0 and 1 are checked on all 64 rows and every
    later one on two rows, against the oracle's decode over the row's cached prefix."""
    w = synth.RAGGED_DECODE
    b_sz, hq, hkv, d = w.extra["batch"], w.n_q_heads, w.n_kv_heads, w.head_dim
    n_phys, n_logical = w.extra["physical_layers"], w.extra["logical_layers"]
    lengths = synth.ragged_lengths(w)
    pool = synth.ragged_pool(w)
    offs = synth.ragged_offsets(w)
    cache = kvc.KVCache.empty(n_phys, b_sz, w.max_seq, hkv, d, dtype=torch.bfloat16)
    pool_dev = torch.from_numpy(pool).cuda()
    for layer in range(n_phys):
        for b in range(b_sz):
            n = int(lengths[b]) * hkv * d
            for which, t in ((0, cache.k), (1, cache.v)):
                o = int(offs[layer, b, which])
                t[layer, b, :lengths[b]] = pool_dev[o:o + n].view(int(lengths[b]), hkv, d).to(torch.bfloat16)
    del pool_dev
    cache.seqlens.copy_(torch.from_numpy(lengths))
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.empty(kvc.kvc_decode_workspace_bytes(cache, hq), dtype=torch.uint8, device="cuda")
    pool_r = numerics.round_to(pool, "bf16")  # what the cache holds, rounded once by the oracle's own RNE
    # two logical layers (two physical slices) on every row; every other logical layer on
    # eight rows spread over the batch (a different eight each layer), so each of the 80
    # layers is checked and every row is checked on many layers
    checks = {0: range(b_sz), 1: range(b_sz)}
    for ell in range(2, n_logical):
        checks[ell] = sorted({(ell + j * (b_sz // 8)) % b_sz for j in range(8)})
    for ell in range(n_logical):
        q, k, v = synth.ragged_new_qkv(w, ell)
        q_rot = kvc.kvc_rope_append(cache, ell % n_phys, dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), dev_err=err)
        out = kvc.kvc_attn_decode(cache, ell % n_phys, q_rot, workspace=ws, dev_err=err)
        rows = checks.get(ell, [])
        if rows:
            o = host64(out)[:, 0]
            layer = ell % n_phys
            for b in rows:
                p = int(lengths[b])
                kc = pool_r[offs[layer, b, 0]:offs[layer, b, 0] + p * hkv * d].reshape(p, hkv, d)
                vc = pool_r[offs[layer, b, 1]:offs[layer, b, 1] + p * hkv * d].reshape(p, hkv, d)
                ref = oatt.decode_over_existing(kc, vc, q[b, 0], k[b, 0], v[b, 0], "bf16")
                gates.check(o[b], ref, "bf16", f"logical layer {ell} row {b} (length {p})")
    torch.cuda.synchronize()
    assert err.item() == 0
    assert cache.seqlens.cpu().numpy().tolist() == lengths.tolist()  # the library never advances it


# ---------------------------------------------------------------- long context (bf16)

def test_long_context_chunked_prefill_clone_and_decode(kvc):
    """A 73,728-token sequence (64 q / 8 kv heads, head_dim 128) prefilled in 18 chunks of
    4096 (Cake paper, Section 3 "Chunk Prefill"), cloned to 8 rows, then decoded at batch 1
    and batch 8.  Sampled prefill rows (chunk edges, interior, the last rows) and the
    decode outputs match the oracle; every cached slot is checked against the oracle's append."""
    w = synth.LONG_CONTEXT
    ctx, chunk, rows = w.extra["context"], w.extra["chunk"], w.extra["clone_rows"]
    hq, hkv, d = w.n_q_heads, w.n_kv_heads, w.head_dim
    n_chunks = ctx // chunk
    bf = torch.bfloat16
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    one = kvc.KVCache.empty(1, 1, w.max_seq, hkv, d, dtype=bf)
    one.k.fill_(float("nan"))  # canary: no kernel may read or write a slot it was not given
    one.v.fill_(float("nan"))
    ks, vs, sampled_q, sampled_out, sampled_pos = [], [], [], [], []
    for c in range(n_chunks):
        q, k, v = synth.chunk_qkv(w, c, chunk)
        ks.append(k); vs.append(v)
        q_rot = kvc.kvc_rope_append(one, 0, dev(q[None], "bf16"), dev(k[None], "bf16"), dev(v[None], "bf16"),
                                    dev_err=err)
        out = kvc.kvc_attn_prefill(one, 0, q_rot, dev_err=err)
        one.seqlens += chunk
        # every 64th position, both sides of every chunk boundary, and the last chunk's
        # final 256 rows in full
        local = np.unique(np.concatenate([np.arange(0, chunk, 64), [1, chunk // 2 + 1, chunk - 2, chunk - 1]]))
        if c == n_chunks - 1:
            local = np.unique(np.concatenate([local, np.arange(chunk - 256, chunk)]))
        sampled_q.append(q[local]); sampled_pos.append(c * chunk + local)
        sampled_out.append(host64(out[0].index_select(0, torch.as_tensor(local, device=out.device))))
    torch.cuda.synchronize()
    assert err.item() == 0
    k_all, v_all = np.concatenate(ks), np.concatenate(vs)
    del ks, vs
    # the oracle's own rotated history, built once from the raw keys
    _, k_hat, v_r = oatt.rebuild_row(None, k_all, v_all, "bf16")
    pos = np.concatenate(sampled_pos)
    q_hat = rope.rotate_round(numerics.round_to(np.concatenate(sampled_q), "bf16"), pos, "bf16")
    got_rows = np.concatenate(sampled_out)
    for lo in range(0, len(pos), 128):  # the oracle in slices of 128 query rows (bounded memory)
        sl = slice(lo, lo + 128)
        ref = oatt.attend(q_hat[sl], k_hat[:pos[sl].max() + 1], v_r[:pos[sl].max() + 1], pos[sl])
        gates.check(got_rows[sl], ref, "bf16", f"chunked prefill, sampled rows at positions {pos[sl][0]}..")
    # every cached slot: the values bit for bit, the rotated keys within the error of a
    # float32 rotation (one bfloat16 ulp, or 2^-20 of the pair's length where x c - y s cancels)
    k_raw = numerics.round_to(k_all, "bf16")
    worst, n_over = 0.0, 0
    for lo in range(0, ctx, 8192):
        hi = min(ctx, lo + 8192)
        assert np.array_equal(host64(one.v[0, 0, lo:hi]), v_r[lo:hi]), f"V slots {lo}..{hi}"
        k_got = host64(one.k[0, 0, lo:hi])
        assert rope_error_ok(k_got, k_hat[lo:hi], k_raw[lo:hi], "bf16"), f"K slots {lo}..{hi}"
        r, n = rope_excess_ratio(k_got, k_hat[lo:hi], k_raw[lo:hi], "bf16")
        worst, n_over = max(worst, r), n_over + n
    # how close the keys come to the allowance: elements more than one bfloat16 ulp off, and
    # their largest error relative to the pair length (the gate allows 2^-20)
    print(f"K slots more than 1 ulp off: {n_over} of {k_raw.size}; largest error / |pair| = "
          f"{worst:.3e} = 2^{np.log2(worst) if worst else float('-inf'):.2f} (allowed 2^-20)")
    # slots past the context keep their NaN canary: nothing outside the appended slots is written
    assert bool(torch.isnan(one.k[0, 0, ctx:].float()).all()) and bool(torch.isnan(one.v[0, 0, ctx:].float()).all())
    assert np.array_equal(host64(one.k[0, 0, 0]), k_hat[0])  # position 0 rotates by the identity

    many = kvc.KVCache.empty(1, rows, w.max_seq, hkv, d, dtype=bf)
    kvc.kvc_prefill_clone(one, ctx, many, dev_err=err)
    n_steps, hist = 16, {r: ([], [], []) for r in range(rows)}
    for s in range(n_steps):
        q8, k8, v8 = synth.decode_qkv_batch(w, s, rows)
        for r in range(rows):
            for i, a in enumerate((q8, k8, v8)):
                hist[r][i].append(a[r, 0])
        out1 = kvc.kvc_attn_decode(one, 0, kvc.kvc_rope_append(one, 0, dev(q8[:1], "bf16"), dev(k8[:1], "bf16"),
                                                               dev(v8[:1], "bf16"), dev_err=err), dev_err=err)
        out8 = kvc.kvc_attn_decode(many, 0, kvc.kvc_rope_append(many, 0, dev(q8, "bf16"), dev(k8, "bf16"),
                                                                dev(v8, "bf16"), dev_err=err), dev_err=err)
        if s in (0, n_steps - 1):
            o8, o1 = host64(out8)[:, 0], host64(out1)[0, 0]
            for r in range(rows):
                hq_r, hk_r, hv_r = (np.stack(a) for a in hist[r])
                pos_new = np.arange(ctx, ctx + s + 1)
                k_new = rope.rotate_round(numerics.round_to(hk_r, "bf16"), pos_new, "bf16")
                q_new = rope.rotate_round(numerics.round_to(hq_r[-1:], "bf16"), [ctx + s], "bf16")
                ref = oatt.attend(q_new, np.concatenate([k_hat, k_new]),
                                  np.concatenate([v_r, numerics.round_to(hv_r, "bf16")]), [ctx + s])[0]
                gates.check(o8[r], ref, "bf16", f"batch-8 decode step {s} row {r}")
                if r == 0:
                    gates.check(o1, ref, "bf16", f"batch-1 decode step {s}")
        one.seqlens += 1
        many.seqlens += 1
    torch.cuda.synchronize()
    assert err.item() == 0
