"""GPU parity at the full workload sizes, in the launch configuration the bench
times (automatic split count): sampled units are checked bit-exact against the
oracle run on just those units, and their query heads' outputs within 2e-3."""
import math

import numpy as np
import pytest
import torch

import decode_attention_token_amd as kvq
import oracle
from workloads import GQA_LONG, LLAMA7B_2BIT, LLAMA7B_4BIT, LONG_4BIT, gen_new_tokens, gen_prefill, gen_queries
from gpu_helpers import ATOL, compare_innerq_unit, compare_unit_buffers, host

pytestmark = pytest.mark.gpu


def _sample_units(w, k=6, seed=0):
    U = w.units
    rng = np.random.default_rng(seed + w.config_id)
    picks = {0, U - 1} | set(int(x) for x in rng.integers(0, U, size=k))
    return sorted(picks)


@pytest.mark.parametrize("w,key_norm", [(LLAMA7B_2BIT, 0), (LLAMA7B_4BIT, 0), (GQA_LONG, 0), (LONG_4BIT, 0),
                                        (LONG_4BIT, 1)],
                         ids=lambda x: x.name if hasattr(x, "name") else ("key-norm" if x else "plain"))
def test_fullsize_sampled_parity(w, key_norm):
    print(f"workload {w.name} key_norm={key_norm}", flush=True)
    k, v = gen_prefill(w, 0, "cuda")
    kn, vn = gen_new_tokens(w, 0, "cuda", steps=1)
    q = gen_queries(w, 0, "cuda", steps=1)[0].contiguous()
    cfg = kvq.make_config(w.bits, w.group, w.residual, w.batch, w.num_q_heads, w.num_kv_heads,
                          w.head_dim, w.max_tokens, w.v_policy, w.scheme, w.sinks, key_norm=key_norm)
    cache = kvq.KVCache(cfg, "cuda")
    cache.prefill(k, v)
    cache.append(kn[0].contiguous(), vn[0].contiguous())
    scale = 1.0 / math.sqrt(w.head_dim)
    out = cache.attention(q, scale)
    torch.cuda.synchronize()
    hpg = w.num_q_heads // w.num_kv_heads
    worst = 0.0
    for u in _sample_units(w):
        b, h = divmod(u, w.num_kv_heads)
        if w.scheme == kvq.KVQ_SCHEME_INNERQ:
            ref = oracle.InnerQCache(w.bits, w.group, w.residual, w.sinks, 1, 1, w.head_dim, key_norm=bool(key_norm))
        else:
            ref = oracle.QuantizedKVCache(w.bits, w.group, w.residual, 1, 1, w.head_dim, w.v_policy)
        ref.prefill(host(k[b:b + 1, h:h + 1]), host(v[b:b + 1, h:h + 1]))
        ref.append(host(kn[0][b:b + 1, h:h + 1]), host(vn[0][b:b + 1, h:h + 1]))
        if w.scheme == kvq.KVQ_SCHEME_INNERQ:
            compare_innerq_unit(cache, ref, b, h, 0, 0)
        else:
            compare_unit_buffers(cache, ref, b, h, 0, 0)
        K, V = ref.dequantized()
        qh = host(q[b:b + 1, h * hpg:(h + 1) * hpg])
        want = oracle.attention(qh, K, V, scale)
        got = host(out[b:b + 1, h * hpg:(h + 1) * hpg]).astype(np.float64)
        err = float(np.abs(got - want).max())
        worst = max(worst, err)
        assert err <= ATOL, (u, err)
    print(f"  sampled units ok, worst attention err {worst:.2e}", flush=True)
    del k, v, cache
    torch.cuda.empty_cache()


@pytest.mark.parametrize("w", [LLAMA7B_4BIT, GQA_LONG, LONG_4BIT], ids=lambda x: x.name)
def test_fullsize_decode_steps(w):
    """The launch the bench times on these workloads: kvq_decode_step, one
    launch per step (the new token from k_new / v_new; for the InnerQ window,
    full after the prompt, the leaving token quantized one step ahead).  Three
    steps, then sampled units bit-exact and their heads' outputs within 2e-3
    of the oracle."""
    print(f"workload {w.name}: 3 decode steps", flush=True)
    k, v = gen_prefill(w, 0, "cuda")
    kn, vn = gen_new_tokens(w, 0, "cuda", steps=3)
    qs = gen_queries(w, 0, "cuda", steps=3)
    cfg = kvq.make_config(w.bits, w.group, w.residual, w.batch, w.num_q_heads, w.num_kv_heads,
                          w.head_dim, w.max_tokens, w.v_policy, w.scheme, w.sinks)
    cache = kvq.KVCache(cfg, "cuda")
    cache.prefill(k, v)
    scale = 1.0 / math.sqrt(w.head_dim)
    ws = cache.workspace()
    for i in range(3):
        out = cache.step(kn[i].contiguous(), vn[i].contiguous(), qs[i].contiguous(), scale, workspace=ws)
    torch.cuda.synchronize()
    if w.scheme == kvq.KVQ_SCHEME_INNERQ:
        assert cache.c.prequant == cache.nq_k + 1, "full window: the next leaving token is quantized ahead"
    hpg = w.num_q_heads // w.num_kv_heads
    worst = 0.0
    for u in _sample_units(w, seed=1):
        b, h = divmod(u, w.num_kv_heads)
        if w.scheme == kvq.KVQ_SCHEME_INNERQ:
            ref = oracle.InnerQCache(w.bits, w.group, w.residual, w.sinks, 1, 1, w.head_dim)
        else:
            ref = oracle.QuantizedKVCache(w.bits, w.group, w.residual, 1, 1, w.head_dim, w.v_policy)
        ref.prefill(host(k[b:b + 1, h:h + 1]), host(v[b:b + 1, h:h + 1]))
        for i in range(3):
            ref.append(host(kn[i][b:b + 1, h:h + 1]), host(vn[i][b:b + 1, h:h + 1]))
        if w.scheme == kvq.KVQ_SCHEME_INNERQ:
            compare_innerq_unit(cache, ref, b, h, 0, 0)
        else:
            compare_unit_buffers(cache, ref, b, h, 0, 0)
        K, V = ref.dequantized()
        qh = host(qs[2][b:b + 1, h * hpg:(h + 1) * hpg])
        want = oracle.attention(qh, K, V, scale)
        got = host(out[b:b + 1, h * hpg:(h + 1) * hpg]).astype(np.float64)
        err = float(np.abs(got - want).max())
        worst = max(worst, err)
        assert err <= ATOL, (u, err)
    print(f"  sampled units ok, worst attention err {worst:.2e}", flush=True)
    del k, v, cache
    torch.cuda.empty_cache()


# The bench's variant rows at full size: the value queue, packed metadata, the
# work-queue schedule, the vector-ALU kernel on the grouped-query shape, and
# per-channel key scales.  Same check as above after three decode steps.
VARIANTS = [
    ("llama2-7b-fifo", LLAMA7B_2BIT, dict(v_policy=kvq.KVQ_V_FIFO)),
    ("llama2-7b-meta16", LLAMA7B_2BIT, dict(meta=kvq.KVQ_META_F16)),
    ("b64-4bit-meta16", LLAMA7B_4BIT, dict(meta=kvq.KVQ_META_F16)),
    ("gqa-queue", GQA_LONG, dict(schedule=kvq.KVQ_SCHED_QUEUE)),
    ("gqa-valu", GQA_LONG, dict(kernel=kvq.KVQ_KERNEL_VALU)),
    ("gqa-fifo", GQA_LONG, dict(v_policy=kvq.KVQ_V_FIFO)),
    ("innerq-keynorm", LONG_4BIT, dict(key_norm=kvq.KVQ_KEYNORM_PROMPT)),
]


@pytest.mark.parametrize("name,w,opts", VARIANTS, ids=[v[0] for v in VARIANTS])
def test_fullsize_bench_variants(name, w, opts):
    print(f"workload {w.name} variant {name}: 3 decode steps", flush=True)
    policy = opts.get("v_policy", w.v_policy)
    meta = opts.get("meta", kvq.KVQ_META_F32)
    key_norm = opts.get("key_norm", kvq.KVQ_KEYNORM_NONE)
    k, v = gen_prefill(w, 0, "cuda")
    kn, vn = gen_new_tokens(w, 0, "cuda", steps=3)
    qs = gen_queries(w, 0, "cuda", steps=3)
    cfg = kvq.make_config(w.bits, w.group, w.residual, w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim,
                          w.max_tokens, policy, w.scheme, w.sinks, meta, opts.get("schedule", kvq.KVQ_SCHED_FIXED),
                          opts.get("kernel", kvq.KVQ_KERNEL_AUTO), key_norm)
    cache = kvq.KVCache(cfg, "cuda")
    cache.prefill(k, v)
    scale = 1.0 / math.sqrt(w.head_dim)
    ws = cache.workspace()
    for i in range(3):
        out = cache.step(kn[i].contiguous(), vn[i].contiguous(), qs[i].contiguous(), scale, workspace=ws)
    torch.cuda.synchronize()
    hpg = w.num_q_heads // w.num_kv_heads
    worst = 0.0
    for u in _sample_units(w, seed=2):
        b, h = divmod(u, w.num_kv_heads)
        if w.scheme == kvq.KVQ_SCHEME_INNERQ:
            ref = oracle.InnerQCache(w.bits, w.group, w.residual, w.sinks, 1, 1, w.head_dim, key_norm=bool(key_norm))
        else:
            ref = oracle.QuantizedKVCache(w.bits, w.group, w.residual, 1, 1, w.head_dim, policy,
                                          oracle.META_F16 if meta == kvq.KVQ_META_F16 else oracle.META_F32)
        ref.prefill(host(k[b:b + 1, h:h + 1]), host(v[b:b + 1, h:h + 1]))
        for i in range(3):
            ref.append(host(kn[i][b:b + 1, h:h + 1]), host(vn[i][b:b + 1, h:h + 1]))
        if w.scheme == kvq.KVQ_SCHEME_INNERQ:
            compare_innerq_unit(cache, ref, b, h, 0, 0)
        else:
            compare_unit_buffers(cache, ref, b, h, 0, 0)
        K, V = ref.dequantized()
        qh = host(qs[2][b:b + 1, h * hpg:(h + 1) * hpg])
        want = oracle.attention(qh, K, V, scale)
        got = host(out[b:b + 1, h * hpg:(h + 1) * hpg]).astype(np.float64)
        err = float(np.abs(got - want).max())
        worst = max(worst, err)
        assert err <= ATOL, (u, err)
    print(f"  sampled units ok, worst attention err {worst:.2e}", flush=True)
    del k, v, cache
    torch.cuda.empty_cache()
