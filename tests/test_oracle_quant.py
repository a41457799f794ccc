"""Pins of the oracle's 8-bit KV quantizer (CPU only).

The quantizer is tied to hand-worked values, to a pure-Python brute force
that evaluates the definition element by element, to torch's float32
division and half-to-even rounding, and to the error bound the definition
implies.
"""
import struct

import numpy as np
import torch

from oracle import numerics, quant


def _f32(x: float) -> float:
    """Round a Python float (double) to the nearest float32."""
    return struct.unpack("f", struct.pack("f", x))[0]


def _brute(vec):
    """The definition, one element at a time in Python floats.

    A single float32 division computed in double and rounded once to float32 is
    the correctly rounded float32 quotient (53 >= 2 * 24 + 2 bits), and Python's
    round() sends halves to the even integer.
    """
    amax = max(abs(float(v)) for v in vec)
    s = _f32(amax / 127.0)
    if s == 0.0:
        return [0] * len(vec), 0.0
    return [max(-127, min(127, round(_f32(float(v) / s)))) for v in vec], s


def test_hand_worked_scale_one():
    # amax 127 gives scale exactly 1: codes are x rounded half to even.
    x = np.array([127.0, -63.5, 0.5, 1.5, 2.5, -127.0, 3.25, -0.5], dtype=np.float32)
    codes, scale = quant.quantize_int8(x)
    assert scale == np.float32(1.0)
    assert codes.tolist() == [127, -64, 0, 2, 2, -127, 3, 0]
    assert np.array_equal(quant.dequantize_int8(codes, scale), codes.astype(np.float64))


def test_zero_vector_and_extremes():
    codes, scale = quant.quantize_int8(np.zeros((3, 64), dtype=np.float32))
    assert np.all(scale == 0) and np.all(codes == 0)
    assert np.all(quant.dequantize_int8(codes, scale) == 0)
    g = np.random.default_rng(1)
    x = numerics.round_bf16(g.standard_normal((50, 128)) * 3.0)
    codes, scale = quant.quantize_int8(x)
    i = np.argmax(np.abs(x), axis=-1)
    # the largest magnitude of each vector maps to +-127 exactly
    assert np.array_equal(np.abs(codes[np.arange(50), i]), np.full(50, 127))
    assert np.array_equal(np.sign(codes[np.arange(50), i]), np.sign(x[np.arange(50), i]))


def test_matches_brute_force():
    g = np.random.default_rng(2)
    x = numerics.round_bf16(np.concatenate([
        g.standard_normal((40, 64)),
        g.standard_normal((20, 64)) * 1e-3,
        g.standard_normal((20, 64)) * 300.0,
        np.round(g.standard_normal((20, 64)) * 40.0) / 2.0,  # many exact halves of the grid
    ]))
    codes, scale = quant.quantize_int8(x)
    for r in range(x.shape[0]):
        bc, bs = _brute(x[r])
        assert np.float32(bs) == scale[r]
        assert codes[r].tolist() == bc


def test_matches_torch_float32_round_half_even():
    g = np.random.default_rng(3)
    x = numerics.round_bf16(g.standard_normal((200, 128)) * 2.0).astype(np.float32)
    codes, scale = quant.quantize_int8(x)
    xt = torch.from_numpy(x)
    st = xt.abs().amax(dim=-1) / torch.tensor(127.0, dtype=torch.float32)
    ct = torch.clamp(torch.round(xt / st[:, None]), -127, 127).to(torch.int8)  # torch.round: half to even
    assert np.array_equal(st.numpy(), scale)
    assert np.array_equal(ct.numpy(), codes)


def test_error_bound_and_scale_invariance():
    g = np.random.default_rng(4)
    x = numerics.round_bf16(g.standard_normal((100, 128)))
    codes, scale = quant.quantize_int8(x)
    err = np.abs(quant.dequantize_int8(codes, scale) - x)
    # half a step, plus the float32 rounding of the quotient x / s (|x / s| <= 127,
    # so at most 127 * 2^-24 of a step)
    assert np.all(err <= scale[:, None].astype(np.float64) * (0.5 + 127 * 2.0 ** -24))
    assert np.max(err / scale[:, None]) > 0.49  # and the bound is nearly reached
    # doubling a vector (exact in float32) doubles the scale and keeps every code
    codes2, scale2 = quant.quantize_int8(2.0 * x)
    assert np.array_equal(codes2, codes) and np.array_equal(scale2, 2 * scale)


def test_int8_decode_is_bf16_decode_on_dequantized_values():
    """decode_over_int8 equals the bfloat16 decode oracle run on the dequantized history and on
    the dequantized new key/value; and it differs from the unquantized decode by no more than
    the quantization moves the values (a loose sanity bound)."""
    from oracle import attention as oatt
    from oracle import rope
    g = np.random.default_rng(5)
    p, hkv, hq, d = 37, 2, 4, 64
    hist_k = numerics.round_bf16(g.standard_normal((p, hkv, d)))
    hist_v = numerics.round_bf16(g.standard_normal((p, hkv, d)))
    kc, ks = quant.quantize_int8(hist_k)
    vc, vs = quant.quantize_int8(hist_v)
    q, k, v = (g.standard_normal((n, d)).astype(np.float32) for n in (hq, hkv, hkv))
    got = quant.decode_over_int8(kc, ks, vc, vs, q, k, v)
    k_new = rope.rotate_round(numerics.round_bf16(k[None]), [p], "bf16")
    nkc, nks = quant.quantize_int8(k_new)
    nvc, nvs = quant.quantize_int8(numerics.round_bf16(v[None]))
    k_all = np.concatenate([quant.dequantize_int8(kc, ks), quant.dequantize_int8(nkc, nks)])
    v_all = np.concatenate([quant.dequantize_int8(vc, vs), quant.dequantize_int8(nvc, nvs)])
    q_hat = rope.rotate_round(numerics.round_bf16(q[None]), [p], "bf16")
    ref = oatt.attend(q_hat, k_all, v_all, [p])[0]
    assert np.allclose(got, ref, rtol=0, atol=1e-13)
    plain = oatt.decode_over_existing(hist_k, hist_v, q, k, v, "bf16")
    assert 0 < np.max(np.abs(got - plain)) < 0.05
