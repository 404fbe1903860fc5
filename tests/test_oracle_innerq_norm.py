"""Pins of the oracle's one-time per-channel key normalization of the
InnerQ-style cache (euno.news InnerQ summary, methodology 4: keys scaled once
per channel at prefill, the scale folded into the query).  Reading: the scale
of channel c is the smallest power of two >= max(1, max over the prompt of
|k[c]|), which normalizes the prompt's keys into [-1, 1] (the per-channel
[-1, 1] normalization of the KVQuant part of the juejin.cn page) while keeping
the division and the fold exact."""
import math

import numpy as np
import pytest

import oracle
from oracle import InnerQCache, key_channel_normalizer, normalize_keys, quantize_groups_hybrid

D = 128


def _keys(shape, seed, outliers=4, gain=10.0):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal(shape).astype(np.float32)
    for b in range(shape[0]):
        for h in range(shape[1]):
            ch = rng.choice(shape[3], outliers, replace=False)
            k[b, h, :, ch] *= gain
    return k.astype(np.float16)


def test_scale_is_the_smallest_power_of_two_at_least_max_abs():
    rng = np.random.default_rng(1)
    k = (rng.standard_normal((2, 3, 50, D)) * rng.choice([0.01, 0.5, 1, 3, 100, 3000], (2, 3, 1, D))).astype(np.float16)
    k[0, 0, :, 5] = np.float16(0.25)
    k[0, 0, 7, 5] = 8.0                     # an exact power of two
    k[0, 0, :, 6] = 0.0                     # a silent channel
    k[1, 2, 3, 9] = np.float16(65504.0)     # the fp16 maximum
    k[1, 1, :, 10] = np.float16(2.0 ** -24)  # subnormals only
    lam = key_channel_normalizer(k)
    assert lam.dtype == np.float32 and lam.shape == (2, 3, D)
    amax = np.abs(k.astype(np.float64)).max(axis=2)
    for idx in np.ndindex(*amax.shape):
        target = max(1.0, amax[idx])
        want = next(2.0 ** j for j in range(0, 18) if 2.0 ** j >= target)
        assert lam[idx] == want, (idx, amax[idx], lam[idx])
    assert lam[0, 0, 5] == 8.0 and lam[0, 0, 6] == 1.0 and lam[1, 2, 9] == 65536.0 and lam[1, 1, 10] == 1.0


def test_empty_prompt_gives_unit_scales():
    assert np.array_equal(key_channel_normalizer(np.zeros((1, 2, 0, D), np.float16)), np.ones((1, 2, D), np.float32))


def test_prompt_keys_land_in_the_unit_range():
    k = _keys((1, 2, 300, D), 2)
    lam = key_channel_normalizer(k)
    kn = normalize_keys(k, lam[:, :, None, :]).astype(np.float64)
    assert np.abs(kn).max() <= 1.0
    # each normalized value is the fp16 rounding of an exact quotient
    exact = k.astype(np.float64) / lam[:, :, None, :]
    assert np.array_equal(kn, exact.astype(np.float32).astype(np.float16).astype(np.float64))
    # values in the fp16 normal range divide exactly
    big = np.abs(exact) >= 2.0 ** -14
    assert np.array_equal(kn[big], exact[big])


def _cache(k, v, key_norm, bits=4, G=64, R=16, S=4):
    c = InnerQCache(bits, G, R, S, k.shape[0], k.shape[1], D, key_norm=key_norm)
    c.prefill(k, v)
    return c


def test_scales_are_fixed_at_prefill_and_used_for_every_pop():
    k = _keys((1, 2, 100, D), 3)
    v = np.random.default_rng(4).standard_normal((1, 2, 100, D)).astype(np.float16)
    c = _cache(k, v, True)
    lam = c.k_norm.copy()
    rng = np.random.default_rng(5)
    for i in range(40):
        kn = (rng.standard_normal((1, 2, D)) * 50).astype(np.float16)   # beyond the prompt's range
        window_oldest = c.rk[:, :, 0].copy()
        c.append(kn, rng.standard_normal((1, 2, D)).astype(np.float16))
        assert np.array_equal(c.k_norm, lam), "appends must not change the scales"
        row = normalize_keys(window_oldest, lam)[:, :, None, :]
        codes, s, z = quantize_groups_hybrid(row.reshape(1, 2, 1, D // 64, 64), 4)
        assert np.array_equal(c.qk[:, :, -1:], codes.reshape(1, 2, 1, D))
        assert np.array_equal(c.qk_s[:, :, -1:], s) and np.array_equal(c.qk_z[:, :, -1:], z)


def test_keys_within_the_unit_range_give_the_plain_cache():
    rng = np.random.default_rng(6)
    k = np.clip(rng.standard_normal((2, 2, 90, D)) * 0.3, -1, 1).astype(np.float16)
    v = rng.standard_normal((2, 2, 90, D)).astype(np.float16)
    a, b = _cache(k, v, True), _cache(k, v, False)
    assert np.array_equal(a.k_norm, np.ones_like(a.k_norm))
    ba, bb = a.buffers(128), b.buffers(128)
    for name in bb:
        assert np.array_equal(ba[name], bb[name]), name
    for x, y in zip(a.dequantized(), b.dequantized()):
        assert np.array_equal(x, y)


def test_a_common_power_of_two_scale_is_exact():
    """Every channel's prompt max-abs in (4, 8]: all scales are 8, the
    normalized keys are the keys / 8 exactly, so the codes, zero-points and
    mode choices equal the plain cache's, the key scales are exactly 1/8 of
    them, and the dequantized cache and attention are bit-identical."""
    rng = np.random.default_rng(7)
    k = rng.standard_normal((1, 2, 120, D)).astype(np.float32)
    k = np.where(np.abs(k) < 2.0 ** -10, 0.0, k)           # no fp16 subnormals after / 8
    k[:, :, 0, :] = 7.5                                        # max-abs of every channel in (4, 8]
    k = np.clip(k, -7.5, 7.5).astype(np.float16)
    v = rng.standard_normal((1, 2, 120, D)).astype(np.float16)
    a, b = _cache(k, v, True), _cache(k, v, False)
    assert np.all(a.k_norm == 8.0)
    assert np.array_equal(a.qk, b.qk) and np.array_equal(a.qk_z, b.qk_z)
    assert np.array_equal(a.qk_s * 8, b.qk_s)
    Ka, Va = a.dequantized()
    Kb, Vb = b.dequantized()
    assert np.array_equal(Ka, Kb) and np.array_equal(Va, Vb)
    q = rng.standard_normal((1, 2, D)).astype(np.float16)
    assert np.array_equal(oracle.attention(q, Ka, Va, 1 / math.sqrt(D)), oracle.attention(q, Kb, Vb, 1 / math.sqrt(D)))


def test_folding_the_scale_into_the_query_equals_dequantize_then_scale():
    k = _keys((1, 1, 200, D), 8)
    v = np.random.default_rng(9).standard_normal((1, 1, 200, D)).astype(np.float16)
    c = _cache(k, v, True)
    q = np.random.default_rng(10).standard_normal((1, 1, D)).astype(np.float16)
    scale = 1 / math.sqrt(D)
    want = oracle.attention(q, *c.dequantized(), scale)
    # folded form: quantized tokens scored with q * lambda against the
    # normalized dequantized keys, fp16 tokens with the plain query
    G, m = c.G, c.qk.shape[2]
    kq = oracle.dequantize(c.qk.reshape(1, 1, m, D // G, G), c.qk_s, c.qk_z).reshape(m, D).astype(np.float64)
    q64 = q[0, 0].astype(np.float64)
    s_q = kq @ (q64 * c.k_norm[0, 0].astype(np.float64))
    fp16 = np.concatenate([c.sink_k[0, 0], c.rk[0, 0]]).astype(np.float64)
    s_f = fp16 @ q64
    s = np.concatenate([s_f[:c.sink_k.shape[2]], s_q, s_f[c.sink_k.shape[2]:]]) * scale
    p = np.exp(s - s.max())
    p /= p.sum()
    got = p @ c.dequantized()[1][0, 0].astype(np.float64)
    assert np.abs(got - want[0, 0]).max() <= 1e-13


def test_reconstruction_error_is_bounded_by_the_scaled_step():
    k = _keys((1, 2, 150, D), 11)
    v = np.zeros((1, 2, 150, D), np.float16)
    c = _cache(k, v, True, bits=4, G=64, R=16, S=4)
    K, _ = c.dequantized()
    m = c.qk.shape[2]
    kq = K[:, :, 4:4 + m].astype(np.float64).reshape(1, 2, m, 2, 64)
    orig = k[:, :, 4:4 + m].astype(np.float64).reshape(1, 2, m, 2, 64)
    lam = c.k_norm.astype(np.float64).reshape(1, 2, 1, 2, 64)
    step = c.qk_s.astype(np.float64)[..., None]           # S of each (token, group), normalized units
    err = np.abs(kq - orig)
    # S/2 from rounding plus the fp16 rounding of tiny normalized values
    assert np.all(err <= lam * (step / 2 + 2.0 ** -25) * (1 + 1e-6))


def test_normalization_lowers_the_key_error_on_outlier_channels():
    """The purpose of the scaling: with a few large fixed channels the
    hidden-dim groups are dominated by them; scaling channels first lowers
    the error of the other channels' keys and of the scores."""
    k = _keys((1, 4, 600, D), 12)
    v = np.zeros((1, 4, 600, D), np.float16)
    a, b = _cache(k, v, True), _cache(k, v, False)
    m = a.qk.shape[2]
    orig = k[:, :, 4:4 + m].astype(np.float64)
    ea = np.abs(a.dequantized()[0][:, :, 4:4 + m] - orig).mean()
    eb = np.abs(b.dequantized()[0][:, :, 4:4 + m] - orig).mean()
    assert ea < 0.8 * eb, (ea, eb)
