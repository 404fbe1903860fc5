"""Pins of the oracle's KIVI cache with fp16 sink tokens.

Source: the juejin.cn page "大模型量化技术原理：KIVI、IntactKV、KVQuant", KVQuant part,
section 五 (attention-sink-aware quantization: the first tokens stay fp16);
the KIVI state machine itself is pinned in test_oracle_cache.py.
"""
import math

import numpy as np
import pytest
import torch

from oracle import CHUNK, FIFO, KiviSinkCache, QuantizedKVCache, attention


def _kv(B, H, L, d, seed):
    g = np.random.default_rng(seed)
    k = g.standard_normal((B, H, L, d)).astype(np.float32)
    k[..., 5] *= 8.0
    return k.astype(np.float16), g.standard_normal((B, H, L, d)).astype(np.float16)


@pytest.mark.parametrize("policy", [CHUNK, FIFO])
@pytest.mark.parametrize("S,L", [(4, 300), (4, 2), (1, 64), (8, 8)])
def test_sinks_exact_and_rest_is_a_plain_cache(policy, S, L):
    B, H, d, G, R = 1, 2, 128, 32, 64
    k, v = _kv(B, H, L + 40, d, 3)
    c = KiviSinkCache(2, G, R, S, B, H, d, policy)
    c.prefill(k[:, :, :L], v[:, :, :L])
    for i in range(40):
        c.append(k[:, :, L + i], v[:, :, L + i])
    n = L + 40
    assert c.n == n
    assert np.array_equal(c.sink_k, k[:, :, :S]) and np.array_equal(c.sink_v, v[:, :, :S])
    # the tokens after the sinks behave exactly like a plain cache fed that stream
    ref = QuantizedKVCache(2, G, R, B, H, d, policy)
    ref.prefill(k[:, :, S:max(L, S)], v[:, :, S:max(L, S)])
    for t in range(max(L, S), n):
        ref.append(k[:, :, t], v[:, :, t])
    A, Bb = c.buffers(512), ref.buffers(512)
    for name in ("k_codes", "k_scale", "k_zero", "v_codes", "v_scale", "v_zero"):
        assert np.array_equal(A[name], Bb[name]), name
    assert (c.nq_k, c.nq_v) == (S + ref.nq_k, S + ref.nq_v)
    K, V = c.dequantized()
    Kr, Vr = ref.dequantized()
    assert np.array_equal(K[:, :, S:], Kr) and np.array_equal(V[:, :, S:], Vr)
    assert np.array_equal(K[:, :, :S], k[:, :, :S].astype(np.float32))


def test_prefill_plus_appends_equals_longer_prefill_across_the_sink_boundary():
    B, H, d, S = 2, 2, 128, 6
    k, v = _kv(B, H, 200, d, 4)
    for L in (0, 3, 6, 7, 100):
        a = KiviSinkCache(4, 64, 128, S, B, H, d)
        a.prefill(k[:, :, :L], v[:, :, :L])
        for t in range(L, 200):
            a.append(k[:, :, t], v[:, :, t])
        b = KiviSinkCache(4, 64, 128, S, B, H, d)
        b.prefill(k, v)
        assert (a.n, a.nq_k, a.nq_v) == (b.n, b.nq_k, b.nq_v)
        A, Bb = a.buffers(256), b.buffers(256)
        for name in A:
            assert np.array_equal(A[name], Bb[name]), (L, name)


def test_counters_while_filling_the_sinks():
    c = KiviSinkCache(2, 32, 32, 4, 1, 1, 128)
    k, v = _kv(1, 1, 10, 128, 5)
    c.prefill(k[:, :, :1], v[:, :, :1])
    seen = [(c.n, c.nq_k)]
    for t in range(1, 10):
        c.append(k[:, :, t], v[:, :, t])
        seen.append((c.n, c.nq_k))
    assert seen[:4] == [(1, 1), (2, 2), (3, 3), (4, 4)]
    assert all(nq == 4 for n, nq in seen[4:])   # nothing after the sinks is quantized yet (R = 32)


def test_all_fp16_sink_cache_is_plain_attention():
    B, Hq, H, d = 1, 4, 2, 128
    k, v = _kv(B, H, 20, d, 6)
    c = KiviSinkCache(2, 32, 32, 4, B, H, d)
    c.prefill(k, v)
    K, V = c.dequantized()
    q = np.random.default_rng(7).standard_normal((B, Hq, d)).astype(np.float16)
    got = attention(q, K, V, 1 / math.sqrt(d))
    qt = torch.from_numpy(q.astype(np.float64))[:, :, None]
    Kt = torch.from_numpy(k.astype(np.float64)).repeat_interleave(Hq // H, dim=1)
    Vt = torch.from_numpy(v.astype(np.float64)).repeat_interleave(Hq // H, dim=1)
    want = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, scale=1 / math.sqrt(d))
    np.testing.assert_allclose(got, want[:, :, 0].numpy(), atol=1e-12, rtol=0)
