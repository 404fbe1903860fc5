"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.  Cache bytes (codes, scales, zero-points, residual) must be
bit-exact; attention within 2e-3 max abs of the float64 oracle."""
import math

import numpy as np
import pytest
import torch

import decode_attention_token_amd as kvq
import oracle
from workloads import Workload, gen_new_tokens, gen_prefill, gen_queries, TINY
from gpu_helpers import (split_tol, ATOL, compare_all_buffers, host, make_cache, max_err, oracle_attention,
                         queue_schedule)

pytestmark = pytest.mark.gpu

CHUNK, FIFO = kvq.KVQ_V_CHUNK, kvq.KVQ_V_FIFO


def _w(cid, B, Hq, Hkv, L, bits, G, R, steps, policy=CHUNK, outl=3, gain=8.0):
    return Workload(f"case{cid}", cid, B, Hq, Hkv, 128, L, bits, G, R, outl, gain, steps, 1, policy)


# (workload, steps at which attention is checked)
CASES = [
    (TINY, [1]),
    (_w(101, 2, 4, 4, 300, 2, 32, 64, 70), [1, 19, 20, 21, 70]),          # flush at step 20
    (_w(102, 2, 2, 2, 777, 4, 64, 128, 140), [1, 6, 7, 140]),             # 4-bit, flush at 7
    (_w(103, 1, 8, 2, 500, 2, 64, 128, 30, FIFO), [1, 12, 13, 30]),       # GQA 4, FIFO values
    (_w(104, 2, 4, 2, 129, 4, 32, 64, 65, FIFO), [1, 63, 64, 65]),        # GQA 2, FIFO
    (_w(105, 1, 2, 2, 1000, 2, 128, 128, 5), [1, 5]),                     # G = 128
    (_w(106, 1, 1, 1, 700, 4, 128, 256, 300, FIFO), [1, 68, 69, 300]),    # R = 256
    (_w(107, 3, 3, 3, 64, 2, 32, 64, 3), [1, 3]),                         # L multiple of R
    (_w(108, 1, 4, 1, 40, 2, 32, 128, 4), [1, 4]),                        # L < R: all fp16
]


@pytest.mark.parametrize("w,checks", CASES, ids=[c[0].name for c in CASES])
def test_prefill_append_attention_parity(w, checks):
    print(f"case {w.name}", flush=True)
    dev = "cuda"
    k, v = gen_prefill(w, 0, dev)
    kn, vn = gen_new_tokens(w, 0, dev)
    qs = gen_queries(w, 0, dev)
    cfg, cache = make_cache(w.bits, w.group, w.residual, w.batch, w.num_q_heads, w.num_kv_heads,
                            w.max_tokens, w.v_policy)
    ref = oracle.QuantizedKVCache(w.bits, w.group, w.residual, w.batch, w.num_kv_heads, 128, w.v_policy)
    cache.prefill(k, v)
    ref.prefill(host(k), host(v))
    torch.cuda.synchronize()
    compare_all_buffers(cache, ref)
    scale = 1.0 / math.sqrt(128)
    ws = cache.workspace()
    for step in range(1, w.steps + 1):
        cache.append(kn[step - 1].contiguous(), vn[step - 1].contiguous())
        ref.append(host(kn[step - 1]), host(vn[step - 1]))
        assert (cache.n_tokens, cache.nq_k, cache.nq_v, cache.flushes) == (ref.n, ref.nq_k, ref.nq_v, ref.flushes)
        if step in checks:
            q = qs[step - 1].contiguous()
            out = cache.attention(q, scale, workspace=ws)
            torch.cuda.synchronize()
            compare_all_buffers(cache, ref)
            err = max_err(out, oracle_attention(ref, host(q), scale))
            print(f"  step {step}: n={ref.n} nq_k={ref.nq_k} nq_v={ref.nq_v} err={err:.2e}", flush=True)
            assert err <= ATOL


@pytest.mark.parametrize("bits,G,hpg", [(2, 32, 1), (4, 64, 1), (2, 32, 4), (4, 32, 2)])
def test_split_count_invariance_and_determinism(bits, G, hpg):
    w = _w(110 + bits + hpg, 2, 2 * hpg, 2, 3000, bits, G, 128, 1)
    print(f"case {w.name}", flush=True)
    k, v = gen_prefill(w, 0, "cuda")
    kn, vn = gen_new_tokens(w, 0, "cuda")
    q = gen_queries(w, 0, "cuda")[0].contiguous()
    cfg, cache = make_cache(bits, G, 128, 2, 2 * hpg, 2, w.max_tokens)
    cache.prefill(k, v)
    cache.append(kn[0].contiguous(), vn[0].contiguous())
    ref = oracle.QuantizedKVCache(bits, G, 128, 2, 2, 128)
    ref.prefill(host(k), host(v))
    ref.append(host(kn[0]), host(vn[0]))
    want = oracle_attention(ref, host(q), 1 / math.sqrt(128))
    outs = []
    for s in (1, 2, 3, 7, 16, 64, 0):
        ws = cache.workspace(splits=s)
        o = cache.attention(q, workspace=ws, splits=s)
        torch.cuda.synchronize()
        assert max_err(o, want) <= ATOL, s
        outs.append(host(o))
    for o in outs[1:]:
        assert float(np.abs(o - outs[0]).max()) <= split_tol(hpg)
    again = host(cache.attention(q, splits=0))
    twice = host(cache.attention(q, splits=0))
    assert np.array_equal(again, twice), "reruns must be bit-identical"
    assert np.array_equal(again, outs[-1]), "reruns must be bit-identical"
    with queue_schedule(cache):
        dyn = host(cache.attention(q, splits=0))
    assert float(np.abs(dyn - again).max()) <= split_tol(hpg)


def test_empty_prefill_then_single_token():
    """prefill(0) is allowed; after one append the output is that token's value."""
    w = _w(120, 2, 2, 2, 0, 2, 32, 32, 3)
    kn, vn = gen_new_tokens(w, 0, "cuda")
    qs = gen_queries(w, 0, "cuda")
    cfg, cache = make_cache(2, 32, 32, 2, 2, 2, 64)
    cache.prefill(None, None)
    ref = oracle.QuantizedKVCache(2, 32, 32, 2, 2, 128)
    ref.prefill(np.zeros((2, 2, 0, 128), np.float16), np.zeros((2, 2, 0, 128), np.float16))
    assert cache.n_tokens == 0
    with pytest.raises(kvq.KVQError):
        cache.attention(qs[0].contiguous())
    for step in range(3):
        cache.append(kn[step].contiguous(), vn[step].contiguous())
        ref.append(host(kn[step]), host(vn[step]))
        out = cache.attention(qs[step].contiguous())
        torch.cuda.synchronize()
        want = oracle_attention(ref, host(qs[step]), 1 / math.sqrt(128))
        assert max_err(out, want) <= ATOL
        if step == 0:
            np.testing.assert_allclose(host(out), host(vn[0]).astype(np.float32), atol=1e-6)
    compare_all_buffers(cache, ref)


def test_capacity_edge_fills_the_cache_exactly():
    w = _w(121, 1, 1, 1, 100, 2, 32, 32, 28)
    k, v = gen_prefill(w, 0, "cuda")
    kn, vn = gen_new_tokens(w, 0, "cuda")
    cfg, cache = make_cache(2, 32, 32, 1, 1, 1, 128)
    cache.prefill(k, v)
    for i in range(28):
        cache.append(kn[i].contiguous(), vn[i].contiguous())
    assert cache.n_tokens == 128 and cache.nq_k == 128 and cache.nq_v == 128
    with pytest.raises(kvq.KVQError) as e:
        cache.append(kn[0].contiguous(), vn[0].contiguous())
    assert e.value.status == kvq.KVQ_ERR_CAPACITY
    ref = oracle.QuantizedKVCache(2, 32, 32, 1, 1, 128)
    ref.prefill(host(k), host(v))
    for i in range(28):
        ref.append(host(kn[i]), host(vn[i]))
    torch.cuda.synchronize()
    compare_all_buffers(cache, ref)
    q = gen_queries(w, 0, "cuda")[0].contiguous()
    assert max_err(cache.attention(q), oracle_attention(ref, host(q), 1 / math.sqrt(128))) <= ATOL


def test_prefill_leaves_inputs_untouched():
    w = _w(122, 2, 2, 2, 200, 4, 64, 64, 1)
    k, v = gen_prefill(w, 0, "cuda")
    k0, v0 = k.clone(), v.clone()
    cfg, cache = make_cache(4, 64, 64, 2, 2, 2, 256)
    cache.prefill(k, v)
    torch.cuda.synchronize()
    assert torch.equal(k, k0) and torch.equal(v, v0)


@pytest.mark.parametrize("policy", [CHUNK, FIFO])
def test_decode_step_matches_append_then_attention(policy):
    """kvq_decode_step (fused when no flush is due) gives the same cache bytes
    and bit-identical outputs as kvq_append_token + kvq_decode_attention, and
    stays within the oracle tolerance across flushes."""
    w = _w(130 + policy, 2, 4, 2, 190, 2, 32, 64, 80, policy)
    print(f"case {w.name}", flush=True)
    k, v = gen_prefill(w, 0, "cuda")
    kn, vn = gen_new_tokens(w, 0, "cuda")
    qs = gen_queries(w, 0, "cuda")
    cfg_a, fused = make_cache(2, 32, 64, 2, 4, 2, w.max_tokens, policy)
    cfg_b, plain = make_cache(2, 32, 64, 2, 4, 2, w.max_tokens, policy)
    ref = oracle.QuantizedKVCache(2, 32, 64, 2, 2, 128, policy)
    fused.prefill(k, v)
    plain.prefill(k, v)
    ref.prefill(host(k), host(v))
    ws_a, ws_b = fused.workspace(), plain.workspace()
    for i in range(w.steps):
        q = qs[i].contiguous()
        oa = fused.step(kn[i].contiguous(), vn[i].contiguous(), q, workspace=ws_a)
        plain.append(kn[i].contiguous(), vn[i].contiguous())
        ob = plain.attention(q, workspace=ws_b)
        ref.append(host(kn[i]), host(vn[i]))
        assert (fused.n_tokens, fused.nq_k, fused.nq_v) == (ref.n, ref.nq_k, ref.nq_v)
        torch.cuda.synchronize()
        assert torch.equal(oa, ob), f"step {i}"
        if i % 16 == 15 or i == w.steps - 1:
            assert max_err(oa, oracle_attention(ref, host(q), 1 / math.sqrt(128))) <= ATOL
    compare_all_buffers(fused, ref)


@pytest.mark.parametrize("sinks", [0, 4])
def test_fifo_steps_and_appends_interleaved(sinks):
    """KIVI with a FIFO value queue: fused steps, plain appends and attention
    calls in a seeded random order across key flushes.  A step after which
    the queue is full quantizes its oldest value ahead; the next step or
    append must use that row, and every state matches the oracle."""
    from gpu_helpers import compare_sink_unit
    w = _w(150 + sinks, 2, 4, 2, 100, 2, 32, 64, 150, FIFO)
    print(f"case {w.name} sinks {sinks}", flush=True)
    k, v = gen_prefill(w, 0, "cuda")
    kn, vn = gen_new_tokens(w, 0, "cuda")
    qs = gen_queries(w, 0, "cuda")
    cfg = kvq.make_config(2, 32, 64, 2, 4, 2, 128, 320, FIFO, kvq.KVQ_SCHEME_KIVI, sinks)
    cache = kvq.KVCache(cfg, "cuda")
    ref = oracle.KiviSinkCache(2, 32, 64, sinks, 2, 2, 128, FIFO)
    cache.prefill(k, v)
    ref.prefill(host(k), host(v))
    ws = cache.workspace()
    scale = 1 / math.sqrt(128)
    order = np.random.default_rng(150 + sinks).integers(0, 3, size=w.steps)
    ahead = 0
    for i in range(w.steps):
        q = qs[i].contiguous()
        if order[i] == 0:
            out = cache.step(kn[i].contiguous(), vn[i].contiguous(), q, workspace=ws)
            ahead += cache.c.prequant != 0
        else:
            cache.append(kn[i].contiguous(), vn[i].contiguous())
            out = cache.attention(q, workspace=ws) if order[i] == 1 else None
        ref.append(host(kn[i]), host(vn[i]))
        assert (cache.n_tokens, cache.nq_k, cache.nq_v) == (ref.n, ref.nq_k, ref.nq_v), i
        if out is not None:
            torch.cuda.synchronize()
            assert max_err(out, oracle_attention(ref, host(q), scale)) <= ATOL, i
        if i % 25 == 24 or i == w.steps - 1:
            for b in range(2):
                for h in range(2):
                    compare_sink_unit(cache, ref, b, h)
    assert ahead > 10


# KIVI with fp16 sink tokens: (workload, sinks, steps at which attention is checked)
SINK_CASES = [
    (_w(140, 2, 4, 4, 300, 2, 32, 64, 70), 4, [1, 20, 21, 70]),            # flush at step 20
    (_w(141, 2, 4, 2, 129, 4, 32, 64, 65, FIFO), 4, [1, 64, 65]),          # GQA 2, FIFO values
    (_w(142, 1, 8, 2, 2, 2, 64, 128, 140), 8, [1, 6, 7, 8, 140]),          # L < sinks, GQA 4
    (_w(143, 1, 2, 2, 3, 4, 64, 64, 5), 8, [1, 5]),                       # only sinks
]


@pytest.mark.parametrize("w,S,checks", SINK_CASES, ids=[c[0].name for c in SINK_CASES])
def test_kivi_sink_tokens_parity(w, S, checks):
    from gpu_helpers import compare_sink_unit
    print(f"case {w.name} sinks {S}", flush=True)
    k, v = gen_prefill(w, 0, "cuda")
    kn, vn = gen_new_tokens(w, 0, "cuda")
    qs = gen_queries(w, 0, "cuda")
    cfg = kvq.make_config(w.bits, w.group, w.residual, w.batch, w.num_q_heads, w.num_kv_heads, 128,
                          w.max_tokens + w.residual, w.v_policy, kvq.KVQ_SCHEME_KIVI, S)
    cache = kvq.KVCache(cfg, "cuda")
    ref = oracle.KiviSinkCache(w.bits, w.group, w.residual, S, w.batch, w.num_kv_heads, 128, w.v_policy)
    cache.prefill(k, v)
    ref.prefill(host(k), host(v))
    scale = 1.0 / math.sqrt(128)
    ws = cache.workspace()
    for step in range(1, w.steps + 1):
        cache.append(kn[step - 1].contiguous(), vn[step - 1].contiguous())
        ref.append(host(kn[step - 1]), host(vn[step - 1]))
        assert (cache.n_tokens, cache.nq_k, cache.nq_v) == (ref.n, ref.nq_k, ref.nq_v)
        if step in checks:
            q = qs[step - 1].contiguous()
            out = cache.attention(q, scale, workspace=ws)
            torch.cuda.synchronize()
            for b in range(w.batch):
                for h in range(w.num_kv_heads):
                    compare_sink_unit(cache, ref, b, h)
            err = max_err(out, oracle_attention(ref, host(q), scale))
            print(f"  step {step}: n={ref.n} nq_k={ref.nq_k} nq_v={ref.nq_v} err={err:.2e}", flush=True)
            assert err <= ATOL


@pytest.mark.parametrize("policy", [CHUNK, FIFO])
def test_kivi_sink_decode_step_matches_append_then_attention(policy):
    """The first steps fill the sink tokens (two calls), the later ones take
    the fused path (one launch, or the value pop and one launch for FIFO)."""
    from gpu_helpers import compare_sink_unit
    w = _w(144, 2, 4, 2, 2, 2, 32, 64, 80, policy)
    S = 4
    print(f"case {w.name} sinks {S}", flush=True)
    kn, vn = gen_new_tokens(w, 0, "cuda")
    k, v = gen_prefill(w, 0, "cuda")
    qs = gen_queries(w, 0, "cuda")
    mk = lambda: kvq.KVCache(kvq.make_config(2, 32, 64, 2, 4, 2, 128, 192, policy, kvq.KVQ_SCHEME_KIVI, S), "cuda")
    fused, plain = mk(), mk()
    ref = oracle.KiviSinkCache(2, 32, 64, S, 2, 2, 128, policy)
    fused.prefill(k, v)
    plain.prefill(k, v)
    ref.prefill(host(k), host(v))
    wa, wb = fused.workspace(), plain.workspace()
    for i in range(w.steps):
        q = qs[i].contiguous()
        oa = fused.step(kn[i].contiguous(), vn[i].contiguous(), q, workspace=wa)
        plain.append(kn[i].contiguous(), vn[i].contiguous())
        ob = plain.attention(q, workspace=wb)
        ref.append(host(kn[i]), host(vn[i]))
        assert (fused.n_tokens, fused.nq_k, fused.nq_v) == (ref.n, ref.nq_k, ref.nq_v)
        torch.cuda.synchronize()
        assert torch.equal(oa, ob), i
    assert max_err(oa, oracle_attention(ref, host(q), 1 / math.sqrt(128))) <= ATOL
    for b in range(2):
        for h in range(2):
            compare_sink_unit(fused, ref, b, h)


@pytest.mark.parametrize("bits,G,L", [(4, 64, 9000), (2, 32, 17000)])
def test_wave_orders_agree(bits, G, L):
    """One split per unit spans more than 32 KiB of key codes per wave, so its
    waves take every eighth key group; with 4 or 16 splits each wave keeps a
    contiguous range.  Both orders match the oracle and each other."""
    w = _w(130 + bits, 1, 2, 2, L, bits, G, 128, 1)
    print(f"case {w.name}", flush=True)
    k, v = gen_prefill(w, 0, "cuda")
    kn, vn = gen_new_tokens(w, 0, "cuda")
    q = gen_queries(w, 0, "cuda")[0].contiguous()
    cfg, cache = make_cache(bits, G, 128, 1, 2, 2, w.max_tokens)
    cache.prefill(k, v)
    cache.append(kn[0].contiguous(), vn[0].contiguous())
    ref = oracle.QuantizedKVCache(bits, G, 128, 1, 2, 128)
    ref.prefill(host(k), host(v))
    ref.append(host(kn[0]), host(vn[0]))
    want = oracle_attention(ref, host(q), 1 / math.sqrt(128))
    outs = {}
    for s in (1, 4, 16):
        o = cache.attention(q, workspace=cache.workspace(splits=s), splits=s)
        torch.cuda.synchronize()
        err = max_err(o, want)
        print(f"  splits {s}: err {err:.2e}", flush=True)
        assert err <= ATOL
        outs[s] = host(o)
    assert float(np.abs(outs[1] - outs[4]).max()) <= split_tol(1)
    assert float(np.abs(outs[1] - outs[16]).max()) <= split_tol(1)


def test_two_threads_two_streams():
    """Two host threads each drive their own cache on their own stream at the
    same time (prefill, then decode steps across a flush, FIFO and chunked
    values, the matrix-core and vector kernels): every output equals the same
    sequence run alone, bit for bit.  The library keeps no per-call global
    state besides the thread-local error text."""
    import threading
    cases = [(_w(160, 2, 4, 2, 300, 2, 32, 64, 80, FIFO), kvq.KVQ_V_FIFO),
             (_w(161, 2, 8, 2, 250, 4, 64, 64, 80), kvq.KVQ_V_CHUNK)]
    print("two threads, two streams", flush=True)

    def run(w, policy, stream, outs):
        k, v = gen_prefill(w, 0, "cuda")
        kn, vn = gen_new_tokens(w, 0, "cuda")
        qs = gen_queries(w, 0, "cuda")
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            cfg, cache = make_cache(w.bits, w.group, w.residual, w.batch, w.num_q_heads, w.num_kv_heads,
                                    w.max_tokens, policy)
            ws = cache.workspace()
            cache.prefill(k, v, stream)
            for i in range(w.steps):
                outs.append(cache.step(kn[i].contiguous(), vn[i].contiguous(), qs[i].contiguous(), workspace=ws,
                                       stream=stream).clone())
        stream.synchronize()

    alone = []
    for w, p in cases:
        o = []
        run(w, p, torch.cuda.Stream(), o)
        alone.append(o)
    together = [[], []]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    ts = [threading.Thread(target=run, args=(w, p, s, o)) for (w, p), s, o in zip(cases, streams, together)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    torch.cuda.synchronize()
    for a, b in zip(alone, together):
        assert len(a) == len(b) == 80
        for i, (x, y) in enumerate(zip(a, b)):
            assert torch.equal(x, y), i
