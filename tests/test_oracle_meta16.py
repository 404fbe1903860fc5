"""Pins of the oracle's compressed group metadata: an fp16 scale rounded
toward +inf, packed with the int16 zero-point into one 32-bit word.

The affine map itself is the pgsm.cn KV-cache quantization article's
X_Q = round(X / S) - Z (section 2.1); only the storage of S changes: the
smallest fp16 value >= the fp32 scale, so the group's range still fits the
2^b levels.
"""
import numpy as np
import pytest

from oracle import (META_F16, QuantizedKVCache, attention_call_bytes, dequantize, quantize_groups,
                    round_up_to_fp16)


def _groups(n, G, seed):
    g = np.random.default_rng(seed)
    x = g.standard_normal((n, G)) * g.choice([1e-4, 0.01, 1.0, 30.0], size=(n, 1))
    x += g.choice([0.0, 0.0, 5.0, -700.0], size=(n, 1))
    return x.astype(np.float16)


def test_round_up_to_fp16_is_the_smallest_fp16_above():
    g = np.random.default_rng(1)
    s = np.abs(g.standard_normal(20000) * g.choice([1e-6, 1e-3, 1.0, 1e3], size=20000)).astype(np.float32) + 1e-7
    up = round_up_to_fp16(s)
    h = up.astype(np.float16)
    assert np.array_equal(h.astype(np.float32), up)                     # exactly representable
    assert np.all(up >= s)
    below = np.nextafter(h, np.float16(0)).astype(np.float32)          # the fp16 just below
    assert np.all(below < s)


@pytest.mark.parametrize("bits", [2, 4])
def test_on_grid_lattices_with_fp16_scales_are_exact(bits):
    qmax = (1 << bits) - 1
    g = np.random.default_rng(10 + bits)
    for _ in range(200):
        s = np.float32(2.0 ** int(g.integers(-8, 5)))
        z = int(g.integers(-30, 30))
        k = g.integers(0, qmax + 1, size=32)
        k[0], k[1] = 0, qmax
        x = (s * (z + k)).astype(np.float16)
        c, S, Z = quantize_groups(x[None], bits, f16_scale=True)
        assert S[0] == s and int(Z[0]) == z and np.array_equal(c[0], k.astype(np.uint8))


@pytest.mark.parametrize("bits", [2, 4])
def test_codes_are_nearest_level_with_the_rounded_scale(bits):
    qmax = (1 << bits) - 1
    x = _groups(3000, 32, 5 + bits)
    c, S, Z = quantize_groups(x, bits, f16_scale=True)
    c32, S32, _ = quantize_groups(x, bits)
    assert np.all(S >= S32) and np.array_equal(S, round_up_to_fp16(S32))
    xf = x.astype(np.float32)
    levels = (S[:, None] * (np.arange(qmax + 1, dtype=np.float32)[None, :] + Z[:, None].astype(np.float32)))
    best = np.abs(xf[..., None] - levels[:, None, :]).min(-1)
    got = np.abs(xf - dequantize(c, S, Z))
    assert np.all(got <= best * (1 + 1e-6) + 1e-30)
    assert np.all(got <= S[:, None] / 2 * (1 + 1e-5) + 1e-30)


def test_packed_words_decode_to_scale_and_zero():
    g = np.random.default_rng(3)
    k = (g.standard_normal((1, 2, 200, 128)) * 3 + 1).astype(np.float16)
    v = g.standard_normal((1, 2, 200, 128)).astype(np.float16)
    c = QuantizedKVCache(2, 32, 64, 1, 2, 128, meta=META_F16)
    c.prefill(k, v)
    buf = c.buffers(256)
    assert buf["k_scale"].dtype == np.uint32 and buf["k_zero"].size == 0 and buf["v_zero"].size == 0
    nq = c.nq_k
    w = buf["k_scale"][:, :, :nq // 32]
    S = (w & 0xFFFF).astype(np.uint16).view(np.float16).astype(np.float32)
    Z = (w >> 16).astype(np.uint16).view(np.int16)
    assert np.array_equal(S, c.kq_scale) and np.array_equal(Z, c.kq_zero)
    wv = buf["v_scale"][:, :, :nq]
    assert np.array_equal((wv & 0xFFFF).astype(np.uint16).view(np.float16).astype(np.float32), c.vq_scale)


def test_call_bytes_drop_by_a_third_of_the_metadata():
    a = attention_call_bytes(16, 32, 32, 128, 2, 32, 4097, 4096, 4096)
    b = attention_call_bytes(16, 32, 32, 128, 2, 32, 4097, 4096, 4096, META_F16)
    meta6 = 2 * 16 * 32 * 4096 * 4 * 6     # K and V metadata, 6 bytes per group
    assert a - b == meta6 // 3
    assert round(b / 1e6, 1) == 202.0
