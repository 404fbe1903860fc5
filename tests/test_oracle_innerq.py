"""Pins of the oracle's InnerQ-style variant: the hybrid group quantizer and
the cache with attention sinks and a recent fp16 window.

Source: euno.news, "【论文】InnerQ：硬件感知免调优KV缓存量化用于大语言模型",
methodology 1 (groups along the hidden dimension), 2 (per-group statistics;
symmetric quantization for zero-centred groups, asymmetric otherwise), 4
(sink tokens and a recent window kept in fp16); symmetric quantization as in
the pgsm.cn KV-cache quantization article, section 2.1.  Reading used here
for "centred on zero": |mean| < 0.1 * std (population std).
"""
import math

import numpy as np
import pytest
import torch

from oracle import (InnerQCache, attention, dequantize, hybrid_is_symmetric,
                    innerq_attention_call_bytes, quantize_groups, quantize_groups_hybrid,
                    quantize_groups_symmetric)


def _mixed_groups(n, G, seed):
    g = np.random.default_rng(seed)
    x = g.standard_normal((n, G)) + g.uniform(-0.3, 0.3, (n, 1))
    x *= g.choice([0.01, 1.0, 30.0], size=(n, 1))
    return x.astype(np.float16)


# ------------------------------------------------------------ mode choice
@pytest.mark.parametrize("G", [32, 64, 128])
def test_mode_choice_agrees_with_numpy_statistics(G):
    x = _mixed_groups(4000, G, 11 + G)
    xf = x.astype(np.float64)
    mean = xf.mean(axis=-1)
    std = xf.std(axis=-1)
    ratio = np.abs(mean) / std
    clear = np.abs(ratio - 0.1) > 1e-9
    sym = hybrid_is_symmetric(x)
    assert np.array_equal(sym[clear], (ratio < 0.1)[clear])
    assert 0.2 < sym.mean() < 0.8, "the workload should exercise both modes"


def test_mode_choice_on_constructed_groups():
    sym_group = np.array([1, -1] * 16, np.float16)                # mean 0
    off_group = np.array([5, 6] * 16, np.float16)                 # mean 5.5, std 0.5
    zero_group = np.zeros(32, np.float16)                         # 0 < 0 is false
    out = hybrid_is_symmetric(np.stack([sym_group, off_group, zero_group]))
    assert out.tolist() == [True, False, False]


# ------------------------------------------------------------ symmetric quantizer
@pytest.mark.parametrize("bits", [2, 4])
def test_symmetric_on_grid_values_are_recovered_exactly(bits):
    """x = s*k with s a power of two, signed k in [-qm, qm] and |k| = qm
    present: S = s, stored code k + 2^(b-1), Z = -2^(b-1), exact round trip."""
    qm = (1 << (bits - 1)) - 1
    g = np.random.default_rng(3 + bits)
    for _ in range(200):
        s = np.float32(2.0 ** int(g.integers(-8, 6)))
        k = g.integers(-qm, qm + 1, size=64)
        k[int(g.integers(0, 64))] = qm * int(g.choice([-1, 1]))
        x = (s * k).astype(np.float16)
        u, S, Z = quantize_groups_symmetric(x[None], bits)
        assert S[0] == s and int(Z[0]) == -(1 << (bits - 1))
        assert np.array_equal(u[0].astype(np.int64) - (1 << (bits - 1)), k)
        assert np.array_equal(dequantize(u, S, Z)[0], x.astype(np.float32))


@pytest.mark.parametrize("bits", [2, 4])
def test_symmetric_codes_are_nearest_level_and_never_use_code_zero(bits):
    """Brute force over the 2^b - 1 symmetric levels S*k, k in [-qm, qm]."""
    qm = (1 << (bits - 1)) - 1
    x = _mixed_groups(500, 32, 5)
    u, S, Z = quantize_groups_symmetric(x, bits)
    assert u.min() >= 1 and u.max() <= 2 * qm + 1
    xf = x.astype(np.float32)
    levels = S[:, None, None] * np.arange(-qm, qm + 1, dtype=np.float32)[None, None, :]
    dist = np.abs(xf[..., None] - levels)
    best = dist.min(axis=-1)
    got = np.abs(xf - dequantize(u, S, Z))
    assert np.all(got <= best * (1 + 1e-6) + 1e-30)
    assert np.all(got <= S[:, None] / 2 * (1 + 1e-6))


def test_symmetric_all_zero_group():
    u, S, Z = quantize_groups_symmetric(np.zeros((1, 32), np.float16), 2)
    assert S[0] == 1.0 and np.all(dequantize(u, S, Z) == 0)


# ------------------------------------------------------------ hybrid quantizer
@pytest.mark.parametrize("bits", [2, 4])
def test_hybrid_takes_each_groups_own_mode(bits):
    x = _mixed_groups(2000, 64, 9)
    sym = hybrid_is_symmetric(x)
    c, s, z = quantize_groups_hybrid(x, bits)
    ca, sa, za = quantize_groups(x, bits)
    cs, ss, zs = quantize_groups_symmetric(x, bits)
    assert np.array_equal(c[~sym], ca[~sym]) and np.array_equal(s[~sym], sa[~sym])
    assert np.array_equal(z[~sym], za[~sym])
    assert np.array_equal(c[sym], cs[sym]) and np.array_equal(s[sym], ss[sym])
    assert np.all(z[sym] == -(1 << (bits - 1)))
    err = np.abs(dequantize(c, s, z) - x.astype(np.float32))
    assert np.all(err <= s[:, None] / 2 * (1 + 1e-6) + 1e-30)


def test_zero_centred_2bit_group_uses_three_levels():
    """A zero-centred 2-bit group has the 3 levels {-S, 0, S} with S = max|x|:
    values round to the nearest of them, so the error is at most S / 2."""
    x = np.array([[-4, -2, 0, 2, 4, 1, -1, 0] * 4], np.float16)
    assert hybrid_is_symmetric(x)[0]
    c, s, z = quantize_groups_hybrid(x, 2)
    assert s[0] == 4.0
    assert np.max(np.abs(dequantize(c, s, z) - x.astype(np.float32))) <= 2.0


# ------------------------------------------------------------ cache
def _kv(B, H, L, d, seed):
    g = np.random.default_rng(seed)
    k = g.standard_normal((B, H, L, d)) + g.uniform(-0.3, 0.3, (B, H, 1, d))
    v = g.standard_normal((B, H, L, d))
    return k.astype(np.float16), v.astype(np.float16)


def _steps(B, H, m, d, seed):
    g = np.random.default_rng(seed)
    return (g.standard_normal((m, B, H, d)).astype(np.float16),
            g.standard_normal((m, B, H, d)).astype(np.float16))


def _buffers_equal(a, b, cap):
    A, Bb = a.buffers(cap), b.buffers(cap)
    for key in A:
        assert np.array_equal(A[key], Bb[key]), key


@pytest.mark.parametrize("S,R,L", [(4, 32, 300), (4, 32, 10), (0, 16, 100), (4, 8, 2), (2, 32, 0)])
def test_window_and_sinks_invariants(S, R, L):
    B, H, d = 1, 2, 128
    k, v = _kv(B, H, L, d, 1)
    kn, vn = _steps(B, H, 60, d, 2)
    c = InnerQCache(4, 64, R, S, B, H, d)
    c.prefill(k, v)
    for i in range(61):
        n = c.n
        assert c.sink_k.shape[2] == min(n, S)
        window = c.rk.shape[2]
        assert window == (min(R, n - S) if n > S else 0)
        assert c.nq == (n if n <= S else n - window)
        assert c.qk.shape[2] == max(0, c.nq - S)
        if i < 60:
            c.append(kn[i], vn[i])
    allk = np.concatenate([k] + [kn[i][:, :, None] for i in range(60)], axis=2)
    assert np.array_equal(c.sink_k, allk[:, :, :min(S, c.n)])
    assert np.array_equal(c.rk, allk[:, :, c.nq:c.n] if c.n > S else allk[:, :, :0])


@pytest.mark.parametrize("bits,G,S,R", [(4, 64, 4, 32), (2, 32, 4, 16), (2, 128, 0, 8)])
def test_prefill_plus_appends_equals_longer_prefill(bits, G, S, R):
    B, H, d, L, m = 2, 2, 128, 50, 40
    k, v = _kv(B, H, L + m, d, 3)
    a = InnerQCache(bits, G, R, S, B, H, d)
    a.prefill(k[:, :, :L], v[:, :, :L])
    for i in range(m):
        a.append(k[:, :, L + i], v[:, :, L + i])
    b = InnerQCache(bits, G, R, S, B, H, d)
    b.prefill(k, v)
    assert (a.n, a.nq) == (b.n, b.nq)
    _buffers_equal(a, b, L + m)


def test_quantized_rows_are_per_token_hybrid_groups():
    B, H, d, G = 1, 2, 128, 64
    k, v = _kv(B, H, 200, d, 4)
    c = InnerQCache(4, G, 32, 4, B, H, d)
    c.prefill(k, v)
    rows = k[:, :, 4:c.nq]
    codes, s, z = quantize_groups_hybrid(rows.reshape(B, H, -1, d // G, G), 4)
    assert np.array_equal(c.qk, codes.reshape(c.qk.shape))
    assert np.array_equal(c.qk_s, s) and np.array_equal(c.qk_z, z)
    K, V = c.dequantized()
    assert np.array_equal(K[:, :, :4], k[:, :, :4].astype(np.float32))
    assert np.array_equal(K[:, :, c.nq:], k[:, :, c.nq:].astype(np.float32))
    err = np.abs(K[:, :, 4:c.nq] - rows.astype(np.float32)).reshape(B, H, -1, d // G, G)
    assert np.all(err <= c.qk_s[..., None] / 2 * (1 + 1e-6) + 1e-30)


def test_all_fp16_cache_is_plain_attention():
    """With n <= sinks + R nothing is quantized: attention equals torch's
    float64 SDPA on the fp16 inputs."""
    B, Hq, H, d = 2, 4, 2, 128
    k, v = _kv(B, H, 30, d, 5)
    c = InnerQCache(2, 32, 32, 4, B, H, d)
    c.prefill(k, v)
    assert c.qk.shape[2] == 0
    K, V = c.dequantized()
    q = np.random.default_rng(6).standard_normal((B, Hq, d)).astype(np.float16)
    got = attention(q, K, V, 1 / math.sqrt(d))
    qt = torch.from_numpy(q.astype(np.float64))[:, :, None]
    Kt = torch.from_numpy(k.astype(np.float64)).repeat_interleave(Hq // H, dim=1)
    Vt = torch.from_numpy(v.astype(np.float64)).repeat_interleave(Hq // H, dim=1)
    want = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, scale=1 / math.sqrt(d))
    np.testing.assert_allclose(got, want[:, :, 0].numpy(), atol=1e-12, rtol=0)


def test_buffers_place_window_in_ring_slots():
    B, H, d, S, R = 1, 1, 128, 4, 16
    k, v = _kv(B, H, 70, d, 7)
    c = InnerQCache(2, 32, R, S, B, H, d)
    c.prefill(k, v)
    kn, vn = _steps(B, H, 9, d, 8)
    for i in range(9):
        c.append(kn[i], vn[i])
    buf = c.buffers(96)
    allk = np.concatenate([k] + [kn[i][:, :, None] for i in range(9)], axis=2)
    for t in range(c.nq, c.n):
        assert np.array_equal(buf["k_resid"][:, :, t % R], allk[:, :, t])
    assert np.array_equal(buf["k_sink"], allk[:, :, :S])
    assert not buf["k_codes"][:, :, :S].any() and not buf["k_codes"][:, :, c.nq:].any()


def test_errors():
    c = InnerQCache(2, 32, 16, 4, 1, 1, 128)
    with pytest.raises(RuntimeError):
        c.append(np.zeros((1, 1, 128), np.float16), np.zeros((1, 1, 128), np.float16))
    with pytest.raises(ValueError):
        InnerQCache(2, 48, 16, 4, 1, 1, 128)
    with pytest.raises(ValueError):
        InnerQCache(2, 32, 0, 4, 1, 1, 128)


def test_call_bytes_match_the_buffers_read():
    """Bytes of one call = the slices of the device buffers it must read
    (quantized rows, sinks, live window slots) plus q and out."""
    B, Hq, H, d, S, R = 2, 4, 2, 128, 4, 32
    for bits, G, L in [(2, 32, 300), (4, 64, 20), (4, 128, 36)]:
        k, v = _kv(B, H, L, d, 9)
        c = InnerQCache(bits, G, R, S, B, H, d)
        c.prefill(k, v)
        buf = c.buffers(L)
        m = max(0, c.nq - S) if c.n > S else 0
        rows = slice(S, S + m)
        total = sum(buf[n][:, :, rows].nbytes for n in
                    ("k_codes", "k_scale", "k_zero", "v_codes", "v_scale", "v_zero"))
        total += buf["k_sink"][:, :, :min(S, L)].nbytes * 2
        total += buf["k_resid"][:, :, :c.rk.shape[2]].nbytes * 2
        total += B * Hq * d * (2 + 4)
        assert innerq_attention_call_bytes(B, Hq, H, d, bits, G, c.n, c.nq, S) == total
