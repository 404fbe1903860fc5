"""GPU parity of the compressed group metadata (fp16 scale rounded up to the
next representable value and the int16 zero-point packed into one 32-bit
word): the HIP path against the oracle's META_F16 caches.  The packed words,
codes and residual bytes must be bit-exact; attention within 2e-3 of the
float64 oracle over the dequantized values it defines."""
import math

import numpy as np
import pytest
import torch

import decode_attention_token_amd as kvq
import oracle
from workloads import Workload, gen_new_tokens, gen_prefill, gen_queries
from gpu_helpers import (split_tol, ATOL, compare_all_buffers, compare_sink_unit, host, make_cache, max_err,
                         oracle_attention)

pytestmark = pytest.mark.gpu

CHUNK, FIFO = kvq.KVQ_V_CHUNK, kvq.KVQ_V_FIFO
F16 = kvq.KVQ_META_F16


def _w(cid, B, Hq, Hkv, L, bits, G, R, steps, policy=CHUNK, sinks=0):
    return Workload(f"m16-{cid}", cid, B, Hq, Hkv, 128, L, bits, G, R, 3, 8.0, steps, 1, policy,
                    sinks=sinks, meta=1)


# (workload, steps at which attention is checked)
CASES = [
    (_w(301, 2, 4, 4, 300, 2, 32, 64, 70), [1, 20, 21, 70]),            # flush at step 20
    (_w(302, 2, 2, 2, 777, 4, 64, 128, 10), [1, 6, 7, 10]),             # 4-bit, flush at 7
    (_w(303, 1, 8, 2, 500, 2, 64, 128, 30, FIFO), [1, 12, 13, 30]),     # GQA 4, FIFO values
    (_w(304, 2, 4, 2, 129, 4, 32, 64, 65, FIFO), [1, 63, 64, 65]),      # GQA 2, 4-bit FIFO
    (_w(305, 1, 2, 2, 3000, 2, 128, 128, 2), [1, 2]),                   # G = 128, several splits
    (_w(306, 2, 4, 2, 300, 2, 32, 64, 70, CHUNK, 4), [1, 20, 21, 70]),  # 4 sink tokens
    (_w(307, 1, 2, 2, 40, 4, 32, 128, 4), [1, 4]),                      # L < R: all fp16
]


def _ref(w):
    if w.sinks:
        return oracle.KiviSinkCache(w.bits, w.group, w.residual, w.sinks, w.batch, w.num_kv_heads, 128,
                                    w.v_policy, oracle.META_F16)
    return oracle.QuantizedKVCache(w.bits, w.group, w.residual, w.batch, w.num_kv_heads, 128, w.v_policy,
                                   oracle.META_F16)


def _compare(cache, ref, w):
    if w.sinks:
        for b in range(w.batch):
            for h in range(w.num_kv_heads):
                compare_sink_unit(cache, ref, b, h)
    else:
        compare_all_buffers(cache, ref)


@pytest.mark.parametrize("w,checks", CASES, ids=[c[0].name for c in CASES])
def test_meta16_prefill_append_attention_parity(w, checks):
    print(f"case {w.name}", flush=True)
    k, v = gen_prefill(w, 0, "cuda")
    kn, vn = gen_new_tokens(w, 0, "cuda")
    qs = gen_queries(w, 0, "cuda")
    cfg, cache = make_cache(w.bits, w.group, w.residual, w.batch, w.num_q_heads, w.num_kv_heads,
                            w.max_tokens + w.residual, w.v_policy, sinks=w.sinks, meta=F16)
    assert cache.tensors["k_scale"].dtype == torch.int32 and cache.tensors["k_zero"].numel() == 0
    ref = _ref(w)
    cache.prefill(k, v)
    ref.prefill(host(k), host(v))
    torch.cuda.synchronize()
    _compare(cache, ref, w)
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
            _compare(cache, ref, w)
            err = max_err(out, oracle_attention(ref, host(q), scale))
            print(f"  step {step}: n={ref.n} nq_k={ref.nq_k} nq_v={ref.nq_v} err={err:.2e}", flush=True)
            assert err <= ATOL


@pytest.mark.parametrize("bits,G,hpg", [(2, 32, 1), (4, 64, 1), (2, 32, 4)])
def test_meta16_split_count_invariance(bits, G, hpg):
    w = _w(310 + bits + hpg, 2, 2 * hpg, 2, 3000, bits, G, 128, 1)
    print(f"case {w.name}", flush=True)
    k, v = gen_prefill(w, 0, "cuda")
    kn, vn = gen_new_tokens(w, 0, "cuda")
    q = gen_queries(w, 0, "cuda")[0].contiguous()
    _, cache = make_cache(bits, G, 128, 2, 2 * hpg, 2, w.max_tokens, meta=F16)
    cache.prefill(k, v)
    cache.append(kn[0].contiguous(), vn[0].contiguous())
    ref = _ref(w)
    ref.prefill(host(k), host(v))
    ref.append(host(kn[0]), host(vn[0]))
    want = oracle_attention(ref, host(q), 1 / math.sqrt(128))
    outs = []
    for s in (1, 3, 16, 0):
        o = cache.attention(q, workspace=cache.workspace(splits=s), splits=s)
        torch.cuda.synchronize()
        assert max_err(o, want) <= ATOL, s
        outs.append(host(o))
    for o in outs[1:]:
        assert float(np.abs(o - outs[0]).max()) <= split_tol(hpg)


def test_meta16_fused_step_matches_append_then_attention():
    w = _w(320, 2, 4, 2, 100, 2, 32, 64, 40)
    k, v = gen_prefill(w, 0, "cuda")
    kn, vn = gen_new_tokens(w, 0, "cuda")
    qs = gen_queries(w, 0, "cuda")
    _, a = make_cache(2, 32, 64, 2, 4, 2, w.max_tokens, meta=F16)
    _, b = make_cache(2, 32, 64, 2, 4, 2, w.max_tokens, meta=F16)
    ref = _ref(w)
    a.prefill(k, v)
    b.prefill(k, v)
    ref.prefill(host(k), host(v))
    for i in range(w.steps):
        q = qs[i].contiguous()
        oa = a.step(kn[i].contiguous(), vn[i].contiguous(), q)
        b.append(kn[i].contiguous(), vn[i].contiguous())
        ob = b.attention(q)
        ref.append(host(kn[i]), host(vn[i]))
        torch.cuda.synchronize()
        assert torch.equal(oa, ob), i
    compare_all_buffers(a, ref)
    assert max_err(oa, oracle_attention(ref, host(q), 1 / math.sqrt(128))) <= ATOL


def test_meta16_scales_round_up():
    """The packed scale is never below the exact one and the two caches'
    attention outputs differ only by the scale rounding."""
    w = _w(330, 1, 4, 4, 1024, 2, 32, 128, 1)
    k, v = gen_prefill(w, 0, "cuda")
    q = gen_queries(w, 0, "cuda")[0].contiguous()
    _, c32 = make_cache(2, 32, 128, 1, 4, 4, 1152)
    _, c16 = make_cache(2, 32, 128, 1, 4, 4, 1152, meta=F16)
    c32.prefill(k, v)
    c16.prefill(k, v)
    torch.cuda.synchronize()
    for t in ("k", "v"):
        s32 = host(c32.tensors[t + "_scale"]).astype(np.float64)
        w16 = host(c16.tensors[t + "_scale"]).view(np.uint32)
        s16 = (w16 & 0xFFFF).astype(np.uint16).view(np.float16).astype(np.float64)
        z16 = (w16 >> 16).astype(np.uint16).view(np.int16)
        live = s32 > 0
        assert np.all(s16[live] >= s32[live]), t
        assert np.all(s16[live] <= s32[live] * (1 + 2.0 ** -9)), t
        assert z16.shape == s16.shape
    o32, o16 = c32.attention(q), c16.attention(q)
    torch.cuda.synchronize()
    assert float((o32 - o16).abs().max()) < 0.1
