"""Pins of the oracle's cache state machine, attention and byte accounting.

Cache rules come from the KIVI section of the juejin.cn page
"大模型量化技术原理：KIVI、IntactKV、KVQuant" (how it works: grouped part plus a
full-precision remainder with l - r divisible by G, the key flush at R tokens
with R divisible by G, the value queue) and from the pgsm.cn KV-cache
quantization article (3.1 fixed-size fp16 residual cache; 3.2 bytes per token).
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import (CHUNK, FIFO, QuantizedKVCache, attention, attention_call_bytes,
                    kv_code_bytes_per_token, dequantize, quantize_groups)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _kv(B, H, L, d, seed):
    g = np.random.default_rng(seed)
    k = g.standard_normal((B, H, L, d)).astype(np.float32)
    k[..., 3] *= 10.0
    v = g.standard_normal((B, H, L, d)).astype(np.float32)
    return k.astype(np.float16), v.astype(np.float16)


def _steps(B, H, m, d, seed):
    g = np.random.default_rng(seed)
    k = g.standard_normal((m, B, H, d)).astype(np.float16)
    v = g.standard_normal((m, B, H, d)).astype(np.float16)
    return k, v


# --------------------------------------------------------------- byte accounting
def test_llama2_7b_bytes_per_token_table():
    with open(os.path.join(GOLDEN, "llama2_7b_kv_bytes.json")) as f:
        gold = json.load(f)
    shp = gold["model_shape"]
    for bits, want in gold["bytes_per_token"].items():
        got = kv_code_bytes_per_token(shp["layers"], shp["kv_heads"], shp["head_dim"], int(bits))
        assert got == want
    for bits, gb in gold["gb_for_10k_tokens_approx"].items():
        got = 10_000 * kv_code_bytes_per_token(32, 32, 128, int(bits)) / 1e9
        assert abs(got - gb) / gb < 0.06


def test_attention_call_bytes_breakdown():
    """Llama-2-7B layer shape, 2-bit, G=32, right after the first append (n=4097)."""
    B, H, d, G, n, nq = 16, 32, 128, 32, 4097, 4096
    units = B * H
    k_codes = units * nq * d * 2 // 8
    k_meta = units * (nq // G) * d * (4 + 2)
    v_codes = units * nq * d * 2 // 8
    v_meta = units * nq * (d // G) * (4 + 2)
    resid = units * 2 * 1 * d * 2
    qo = B * H * d * (2 + 4)
    assert k_codes == 67_108_864 and k_meta == 50_331_648
    total = attention_call_bytes(B, H, H, d, 2, G, n, nq, nq)
    assert total == k_codes + k_meta + v_codes + v_meta + resid + qo == 235_536_384


# --------------------------------------------------------------- split / flush rules
@pytest.mark.parametrize("policy", [CHUNK, FIFO])
@pytest.mark.parametrize("L", [0, 1, 31, 32, 33, 64, 100, 128])
def test_split_invariants_and_flush_count(policy, L):
    B, H, d, G, R = 1, 2, 128, 32, 64
    c = QuantizedKVCache(2, G, R, B, H, d, policy)
    k, v = _kv(B, H, L, d, 5)
    c.prefill(k, v)
    assert c.nq_k % G == 0 and (c.n - c.nq_k) < R
    ks, vs = _steps(B, H, 3 * R, d, 6)
    f0 = c.flushes
    for i in range(3 * R):
        c.append(ks[i], vs[i])
        assert c.nq_k % G == 0, "grouped part must hold whole groups"
        assert 0 <= c.n - c.nq_k < R
        if policy == CHUNK:
            assert c.nq_v == c.nq_k
        else:
            assert c.n - c.nq_v == min(c.n, R)
    assert c.flushes - f0 == 3, "exactly one key flush per R appends"
    assert c.n == L + 3 * R


@pytest.mark.parametrize("policy", [CHUNK, FIFO])
@pytest.mark.parametrize("bits,G,R", [(2, 32, 32), (4, 64, 128), (2, 32, 96)])
def test_prefill_plus_appends_equals_longer_prefill(policy, bits, G, R):
    B, H, d = 2, 2, 128
    L, m = 70, 2 * R + 5
    k, v = _kv(B, H, L + m, d, 11)
    a = QuantizedKVCache(bits, G, R, B, H, d, policy)
    a.prefill(k[:, :, :L], v[:, :, :L])
    for i in range(m):
        a.append(k[:, :, L + i], v[:, :, L + i])
    b = QuantizedKVCache(bits, G, R, B, H, d, policy)
    b.prefill(k, v)
    cap = ((L + m + R - 1) // R) * R + R
    ba, bb = a.buffers(cap), b.buffers(cap)
    for key in ("k_codes", "k_scale", "k_zero", "v_codes", "v_scale", "v_zero"):
        assert np.array_equal(ba[key], bb[key]), key
    ka, va = a.live_resid_slots()
    assert (ka, va) == b.live_resid_slots()
    assert np.array_equal(ba["k_resid"][:, :, ka], bb["k_resid"][:, :, ka])
    assert np.array_equal(ba["v_resid"][:, :, va], bb["v_resid"][:, :, va])
    Ka, Va = a.dequantized()
    Kb, Vb = b.dequantized()
    assert np.array_equal(Ka, Kb) and np.array_equal(Va, Vb)


def test_fifo_and_chunk_value_codes_agree_per_token():
    B, H, d, G, R = 1, 3, 128, 32, 32
    k, v = _kv(B, H, 200, d, 21)
    a = QuantizedKVCache(2, G, R, B, H, d, CHUNK)
    b = QuantizedKVCache(2, G, R, B, H, d, FIFO)
    a.prefill(k[:, :, :50], v[:, :, :50])
    b.prefill(k[:, :, :50], v[:, :, :50])
    for t in range(50, 200):
        a.append(k[:, :, t], v[:, :, t])
        b.append(k[:, :, t], v[:, :, t])
    m = min(a.nq_v, b.nq_v)
    assert m > 100
    assert np.array_equal(a.vq_codes[:, :, :m], b.vq_codes[:, :, :m])
    assert np.array_equal(a.vq_scale[:, :, :m], b.vq_scale[:, :, :m])
    assert np.array_equal(a.kq_codes, b.kq_codes)
    # every token is present exactly once, quantized or fp16
    Ka, Va = a.dequantized()
    Kb, Vb = b.dequantized()
    assert Ka.shape == Kb.shape == (B, H, 200, d) and Va.shape == Vb.shape


def test_quantized_rows_match_direct_group_quantization():
    """Keys: each (token group, channel) is one group of G tokens; values: each
    (token, channel group) is one group of G channels."""
    B, H, d, G, R = 1, 1, 128, 32, 64
    k, v = _kv(B, H, 128, d, 31)
    c = QuantizedKVCache(2, G, R, B, H, d)
    c.prefill(k, v)
    codes, s, z = quantize_groups(k[0, 0, 32:64, 5], 2)      # group 1, channel 5
    assert np.array_equal(c.kq_codes[0, 0, 32:64, 5], codes)
    assert c.kq_scale[0, 0, 1, 5] == s and c.kq_zero[0, 0, 1, 5] == z
    codes, s, z = quantize_groups(v[0, 0, 77, 64:96], 2)      # token 77, channel group 2
    assert np.array_equal(c.vq_codes[0, 0, 77, 64:96], codes)
    assert c.vq_scale[0, 0, 77, 2] == s and c.vq_zero[0, 0, 77, 2] == z


def test_errors():
    with pytest.raises(ValueError):
        QuantizedKVCache(3, 32, 64, 1, 1, 128)
    with pytest.raises(ValueError):
        QuantizedKVCache(2, 32, 48, 1, 1, 128)
    c = QuantizedKVCache(2, 32, 64, 1, 1, 128)
    with pytest.raises(RuntimeError):
        c.append(np.zeros((1, 1, 128), np.float16), np.zeros((1, 1, 128), np.float16))
    c.prefill(*_kv(1, 1, 4, 128, 1))
    with pytest.raises(RuntimeError):
        c.prefill(*_kv(1, 1, 4, 128, 1))


# --------------------------------------------------------------- attention
def _sdpa64(q, K, V, scale, Hq):
    qt = torch.from_numpy(np.asarray(q, np.float64))[:, :, None, :]
    Kt = torch.from_numpy(np.asarray(K, np.float64))
    Vt = torch.from_numpy(np.asarray(V, np.float64))
    rep = Hq // Kt.shape[1]
    Kt = Kt.repeat_interleave(rep, dim=1)
    Vt = Vt.repeat_interleave(rep, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, scale=scale)
    return o[:, :, 0, :].numpy()


def test_residual_only_cache_is_plain_attention():
    """R > n: nothing is quantized and attention reduces to textbook attention
    on the fp16 inputs (checked with torch's float64 SDPA)."""
    B, H, d, G, R = 2, 4, 128, 32, 256
    k, v = _kv(B, H, 100, d, 41)
    c = QuantizedKVCache(2, G, R, B, H, d)
    c.prefill(k, v)
    K, V = c.dequantized()
    assert c.nq_k == 0 and np.array_equal(K, k.astype(np.float32))
    q = np.random.default_rng(3).standard_normal((B, H, d)).astype(np.float16)
    scale = 1.0 / np.sqrt(d)
    np.testing.assert_allclose(attention(q, K, V, scale), _sdpa64(q, K, V, scale, H), rtol=0, atol=1e-12)


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 2), (4, 1)])
def test_attention_matches_sdpa_on_dequantized_cache(Hq, Hkv):
    B, d, G, R = 2, 128, 32, 64
    k, v = _kv(B, Hkv, 300, d, 51)
    c = QuantizedKVCache(2, G, R, B, Hkv, d)
    c.prefill(k, v)
    K, V = c.dequantized()
    q = np.random.default_rng(4).standard_normal((B, Hq, d)).astype(np.float16)
    scale = 1.0 / np.sqrt(d)
    np.testing.assert_allclose(attention(q, K, V, scale), _sdpa64(q, K, V, scale, Hq), rtol=0, atol=1e-12)


def test_attention_special_cases():
    B, H, d = 1, 2, 128
    g = np.random.default_rng(8)
    K = g.standard_normal((B, H, 37, d)).astype(np.float32)
    V = g.standard_normal((B, H, 37, d)).astype(np.float32)
    out = attention(np.zeros((B, H, d), np.float16), K, V, 0.1)
    np.testing.assert_allclose(out, V.astype(np.float64).mean(axis=2), atol=1e-14)
    out = attention(g.standard_normal((B, H, d)).astype(np.float16), K[:, :, :1], V[:, :, :1], 0.1)
    np.testing.assert_allclose(out, V[:, :, 0].astype(np.float64), atol=0)


def test_attention_brute_force_loops():
    """Scalar loops: scores, max-subtracted exponentials, weighted sum."""
    import math
    B, Hq, Hkv, n, d = 1, 2, 1, 5, 8
    g = np.random.default_rng(9)
    q = g.standard_normal((B, Hq, d)).astype(np.float16)
    K = g.standard_normal((B, Hkv, n, d)).astype(np.float32)
    V = g.standard_normal((B, Hkv, n, d)).astype(np.float32)
    sc = 0.3
    got = attention(q, K, V, sc)
    for h in range(Hq):
        s = [sc * sum(float(q[0, h, c]) * float(K[0, 0, t, c]) for c in range(d)) for t in range(n)]
        mx = max(s)
        e = [math.exp(x - mx) for x in s]
        tot = sum(e)
        for c in range(d):
            o = sum(e[t] * float(V[0, 0, t, c]) for t in range(n)) / tot
            assert abs(o - got[0, h, c]) < 1e-12


def test_dequantized_cache_error_is_bounded_by_half_scale():
    B, H, d, G, R = 1, 2, 128, 32, 64
    k, v = _kv(B, H, 256, d, 61)
    c = QuantizedKVCache(2, G, R, B, H, d)
    c.prefill(k, v)
    K, V = c.dequantized()
    ek = np.abs(K[:, :, :256] - k.astype(np.float32))
    sk = np.repeat(c.kq_scale, G, axis=2)
    assert np.all(ek <= sk * 0.5001 + 1e-6)
    ev = np.abs(V - v.astype(np.float32))
    sv = np.repeat(c.vq_scale, G, axis=3)
    assert np.all(ev <= sv * 0.5001 + 1e-6)
