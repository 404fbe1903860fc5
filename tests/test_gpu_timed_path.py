"""GPU parity of the launch the headline benchmark times: the Llama-2-7B layer
shape, 2-bit (batch 16, 32 query and 32 kv heads, context 4096, G = 32,
R = 128), driven through KVCache.step (kvq_decode_step) for 130 steps, so the
residual grows from 1 to 127 tokens in the fused append + attention launch
(one split per unit, the new token read from k_new / v_new and stored into
its ring slot), step 128 fills the residual and takes the flush branch
(flush launch, then attention), and steps 129-130 are fused again.

A second cache of the same shape runs kvq_append_token + kvq_decode_attention
on the same inputs: every step's output must be bit-identical to the fused
one.  At steps 1, 64, 127, 128, 129 and 130 sampled units' cache bytes are
compared bit-exact with the oracle run on just those units, and their query
heads' outputs within 2e-3 of the float64 oracle.
"""
import math

import numpy as np
import pytest
import torch

import decode_attention_token_amd as kvq
import oracle
from workloads import LLAMA7B_2BIT, gen_new_tokens, gen_prefill, gen_queries
from gpu_helpers import ATOL, compare_unit_buffers, host

pytestmark = pytest.mark.gpu

STEPS = 130
CHECKS = (1, 64, 127, 128, 129, 130)


def _sample_units(w, k=6, seed=11):
    rng = np.random.default_rng(seed)
    return sorted({0, w.units - 1} | set(int(x) for x in rng.integers(0, w.units, size=k)))


def test_llama2_7b_2bit_fused_steps_across_the_flush():
    w = LLAMA7B_2BIT
    print(f"workload {w.name}: {STEPS} decode steps through kvq_decode_step", flush=True)
    cap = ((w.context + STEPS + w.residual - 1) // w.residual) * w.residual
    cfg = kvq.make_config(w.bits, w.group, w.residual, w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, cap)
    k, v = gen_prefill(w, 0, "cuda")
    kn, vn = gen_new_tokens(w, 0, "cuda", steps=STEPS)
    qs = gen_queries(w, 0, "cuda", steps=STEPS)
    fused, split = kvq.KVCache(cfg, "cuda"), kvq.KVCache(cfg, "cuda")
    fused.prefill(k, v)
    split.prefill(k, v)
    assert kvq.kvq_auto_splits(cfg, w.context + 1) == 1, "the timed launch runs one split per unit"
    units = _sample_units(w)
    refs = {}
    for u in units:
        b, h = divmod(u, w.num_kv_heads)
        ref = oracle.QuantizedKVCache(w.bits, w.group, w.residual, 1, 1, w.head_dim)
        ref.prefill(host(k[b:b + 1, h:h + 1]), host(v[b:b + 1, h:h + 1]))
        refs[u] = ref
    knh, vnh, qh = host(kn), host(vn), host(qs)
    del k, v
    scale = 1.0 / math.sqrt(w.head_dim)
    ws_f, ws_s = fused.workspace(), split.workspace()
    out_f = torch.empty(w.batch, w.num_q_heads, w.head_dim, dtype=torch.float32, device="cuda")
    out_s = torch.empty_like(out_f)
    worst = 0.0
    for step in range(1, STEPS + 1):
        i = step - 1
        flushes = fused.flushes
        fused.step(kn[i], vn[i], qs[i], scale, out_f, ws_f)
        split.append(kn[i], vn[i])
        split.attention(qs[i], scale, out_s, ws_s)
        torch.cuda.synchronize()
        assert torch.equal(out_f, out_s), f"step {step}: fused step differs from append + attention"
        assert fused.flushes == flushes + (1 if step == 128 else 0)
        for u, ref in refs.items():
            b, h = divmod(u, w.num_kv_heads)
            ref.append(knh[i][b:b + 1, h:h + 1], vnh[i][b:b + 1, h:h + 1])
        if step not in CHECKS:
            continue
        for cache in (fused, split):
            assert (cache.n_tokens, cache.nq_k, cache.nq_v) == (w.context + step,) + (
                (w.context + (128 if step >= 128 else 0),) * 2)
        for u, ref in refs.items():
            b, h = divmod(u, w.num_kv_heads)
            compare_unit_buffers(fused, ref, b, h, 0, 0)
            K, V = ref.dequantized()
            want = oracle.attention(qh[i][b:b + 1, h:h + 1], K, V, scale)
            err = float(np.abs(host(out_f[b:b + 1, h:h + 1]).astype(np.float64) - want).max())
            worst = max(worst, err)
            assert err <= ATOL, (step, u, err)
        print(f"  step {step}: n={fused.n_tokens} nq={fused.nq_k} cache bit-exact, worst err {worst:.2e}",
              flush=True)
