"""Pins of the oracle's sliding-window attention (CPU only)."""
import numpy as np

from oracle import attention as oatt
from oracle import brute, model


def test_window_covering_history_is_plain_attention():
    g = np.random.default_rng(20)
    n, hq, hkv, d = 40, 4, 2, 16
    q, k, v = g.standard_normal((n, hq, d)), g.standard_normal((n, hkv, d)), g.standard_normal((n, hkv, d))
    pos = [0, 7, 39]
    a = oatt.window_outputs(q, k, v, pos, window=64, dtype="f32")
    b = oatt.nocache_outputs(q, k, v, pos, "f32")
    assert np.allclose(a, b, rtol=0, atol=1e-14)


def test_window_equals_rerun_at_relative_positions():
    """Scores depend only on query-key distance (Tiny-GPT, "Does the Cache Change the Output?"):
    the window at absolute positions equals the trimmed history rerun from position 0, up to the
    float32 rounding of the rotated vectors; a wrong window start or offset fails by far more."""
    g = np.random.default_rng(21)
    n, w, hq, hkv, d = 300, 64, 4, 2, 32
    q, k, v = g.standard_normal((n, hq, d)), g.standard_normal((n, hkv, d)), g.standard_normal((n, hkv, d))
    for p in (63, 64, 65, 200, 299):
        got = oatt.window_outputs(q, k, v, [p], window=w, dtype="f32")[0]
        lo = p + 1 - w
        rel = oatt.nocache_outputs(q[lo:p + 1], k[lo:p + 1], v[lo:p + 1], [w - 1], "f32")[0]
        assert np.max(np.abs(got - rel)) < 1e-5
        if lo >= 1:
            shifted = oatt.nocache_outputs(q[lo - 1:p], k[lo - 1:p], v[lo - 1:p], [w - 1], "f32")[0]
            assert np.max(np.abs(got - shifted)) > 1e-2  # a window one position off is visible


def test_window_matches_brute_force():
    g = np.random.default_rng(22)
    n, w, hq, hkv, d = 12, 5, 2, 1, 8
    q, k, v = (g.standard_normal((n, h, d)).astype(np.float32) for h in (hq, hkv, hkv))
    for p in (2, 4, 5, 11):
        got = oatt.window_outputs(q, k, v, [p], window=w, dtype="bf16")[0]
        lo = max(0, p + 1 - w)
        st = lambda vec: [brute.to_storage(float(x), "bf16") for x in vec]
        k_hat = [[brute.rope_vec(st(k[j][gg]), j, 10000.0, "bf16") for gg in range(hkv)] for j in range(lo, p + 1)]
        vv = [[st(v[j][gg]) for gg in range(hkv)] for j in range(lo, p + 1)]
        q_hat = [[brute.rope_vec(st(q[p][h]), p, 10000.0, "bf16") for h in range(hq)]]
        ref = brute.attention_row(q_hat, k_hat, vv, [p - lo], 1.0 / np.sqrt(d))
        assert np.allclose(got, np.asarray(ref[0]), rtol=0, atol=1e-12)


def test_tiny_layer_window_equals_per_step_trimmed_rerun():
    """The single attention layer's trimmed rerun (the page's uncached loop) equals window attention
    over its projections: one layer carries no context from evicted tokens."""
    g = np.random.default_rng(23)
    c, hq, ctx = 64, 2, 16
    w_qkv, w_out = g.standard_normal((c, 3 * c)) * 0.1, g.standard_normal((c, c)) * 0.1
    x = g.standard_normal((40, c))
    qkv = x @ w_qkv
    d = c // hq
    q, k, v = (qkv[:, i * c:(i + 1) * c].reshape(40, hq, d) for i in range(3))
    for p in (10, 15, 16, 39):
        rerun = model.tiny_layer_nocache(x[:p + 1], w_qkv, w_out, hq, context=ctx)[-1]
        win = oatt.window_outputs(q, k, v, [p], window=ctx, dtype="f32")[0].reshape(c) @ w_out
        assert np.max(np.abs(rerun - win)) < 1e-5
