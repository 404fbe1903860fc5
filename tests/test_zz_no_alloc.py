"""GPU test of kvq_decode_attention_static, the attention entry point that
allocates nothing (its scratch is the library's static device array): its
output must equal kvq_decode_attention's with a caller workspace and the
fixed schedule bit for bit, and stay within 2e-3 of the float64 oracle, on
two calls in a row with the second on a smaller input (the array then holds
the larger call's leftovers), for the matrix-core kernel (several splits, the
in-launch merge), the vector-ALU kernel with a merge launch, and the InnerQ
kernel; a call needing more scratch than the array holds is refused."""
import math

import numpy as np
import pytest
import torch

import decode_attention_token_amd as kvq
import oracle
from workloads import Workload, gen_new_tokens, gen_prefill, gen_queries
from gpu_helpers import ATOL, host, max_err, oracle_attention

pytestmark = pytest.mark.gpu


def _setup(w, scheme=kvq.KVQ_SCHEME_KIVI, schedule=kvq.KVQ_SCHED_FIXED):
    k, v = gen_prefill(w, 0, "cuda")
    kn, vn = gen_new_tokens(w, 0, "cuda", steps=1)
    q = gen_queries(w, 0, "cuda", steps=1)[0].contiguous()
    if scheme == kvq.KVQ_SCHEME_INNERQ:
        cfg = kvq.make_innerq_config(w.bits, w.group, w.residual, w.sinks, w.batch, w.num_q_heads,
                                     w.num_kv_heads, 128, w.context + 8)
        ref = oracle.InnerQCache(w.bits, w.group, w.residual, w.sinks, w.batch, w.num_kv_heads, 128)
    else:
        cap = ((w.context + 1 + w.residual - 1) // w.residual + 1) * w.residual
        cfg = kvq.make_config(w.bits, w.group, w.residual, w.batch, w.num_q_heads, w.num_kv_heads, 128, cap,
                              schedule=schedule)
        ref = oracle.QuantizedKVCache(w.bits, w.group, w.residual, w.batch, w.num_kv_heads, 128)
    cache = kvq.KVCache(cfg, "cuda")
    cache.prefill(k, v)
    cache.append(kn[0].contiguous(), vn[0].contiguous())
    ref.prefill(host(k), host(v))
    ref.append(host(kn[0]), host(vn[0]))
    return cache, ref, q


def _check(cache, ref, q, splits):
    scale = 1.0 / math.sqrt(128)
    fixed = kvq.KVQ_SCHED_FIXED
    old = cache.cfg.schedule
    cache.cfg.schedule = fixed
    try:
        want_ws = cache.attention(q, scale, workspace=cache.workspace(splits=splits), splits=splits)
    finally:
        cache.cfg.schedule = old
    got = cache.attention_static(q, scale, splits=splits)
    torch.cuda.synchronize()
    assert torch.equal(got, want_ws), "static scratch must give the workspace call's bits"
    err = max_err(got, oracle_attention(ref, host(q), scale))
    assert err <= ATOL, err
    return err


def _w(cid, B, Hq, Hkv, L, bits=2, G=32, R=128, sinks=0):
    return Workload(f"static{cid}", cid, B, Hq, Hkv, 128, L, bits, G, R, 4, 10.0, 1, 1, 0, 0, sinks)


@pytest.mark.parametrize("splits", [0, 5])
def test_static_scratch_two_calls_second_smaller(splits):
    print(f"static scratch, splits {splits}", flush=True)
    # matrix-core kernel: four query heads per kv head, several splits
    big = _setup(_w(601, 4, 32, 8, 3000))
    small = _setup(_w(602, 1, 8, 2, 900))
    # the work-queue schedule in the config is ignored: fixed order here
    queued = _setup(_w(603, 2, 8, 2, 1500), schedule=kvq.KVQ_SCHED_QUEUE)
    for cache, ref, q in (big, small, queued):
        print(f"  gqa n={cache.n_tokens} err {_check(cache, ref, q, splits):.2e}", flush=True)
    # vector-ALU kernel with split records and the merge launch
    mha_big = _setup(_w(604, 2, 8, 8, 4000))
    mha_small = _setup(_w(605, 1, 2, 2, 700))
    for cache, ref, q in (mha_big, mha_small):
        print(f"  mha n={cache.n_tokens} err {_check(cache, ref, q, splits or 7):.2e}", flush=True)
    # InnerQ kernel: the unit's last workgroup merges
    iq_big = _setup(_w(606, 2, 8, 8, 5000, 4, 64, 32, 4), kvq.KVQ_SCHEME_INNERQ)
    iq_small = _setup(_w(607, 1, 4, 4, 1200, 4, 64, 32, 4), kvq.KVQ_SCHEME_INNERQ)
    for cache, ref, q in (iq_big, iq_small):
        print(f"  innerq n={cache.n_tokens} err {_check(cache, ref, q, splits or 3):.2e}", flush=True)


def test_static_scratch_refuses_calls_above_its_size():
    w = _w(610, 64, 128, 32, 64, R=64)
    cache, ref, q = _setup(w)
    need = kvq.kvq_workspace_bytes(cache.cfg, cache.n_tokens, 64)
    assert need > kvq.KVQ_STATIC_SCRATCH_BYTES
    out = torch.full((w.batch, w.num_q_heads, 128), 7.0, device="cuda")
    with pytest.raises(kvq.KVQError) as e:
        cache.attention_static(q, out=out, splits=64)
    assert e.value.status == kvq.KVQ_ERR_CAPACITY
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()), "a refused call enqueues nothing"
    # the same cache within the limit still works
    assert max_err(cache.attention_static(q), oracle_attention(ref, host(q), 1 / math.sqrt(128))) <= ATOL
