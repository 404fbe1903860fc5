"""GPU parity of the InnerQ-style cache: the HIP path (through the C ABI)
against the oracle's InnerQCache on the same seeded inputs.  Quantized rows,
sink rows and window slots must be bit-exact; attention within 2e-3 max abs
of the float64 oracle."""
import math

import numpy as np
import pytest
import torch

import decode_attention_token_amd as kvq
import oracle
from workloads import Workload, gen_new_tokens, gen_prefill, gen_queries
from gpu_helpers import ATOL, compare_innerq_buffers, host, make_innerq_cache, max_err, oracle_attention

pytestmark = pytest.mark.gpu


def _w(cid, B, Hq, Hkv, L, bits, G, R, S, steps, outl=4, gain=10.0):
    return Workload(f"iq{cid}", cid, B, Hq, Hkv, 128, L, bits, G, R, outl, gain, steps, 1,
                    v_policy=1, scheme=1, sinks=S)


# (workload, steps at which attention is checked)
CASES = [
    (_w(201, 2, 4, 4, 300, 4, 64, 32, 4, 40), [1, 2, 40]),           # window full: a pop per step
    (_w(202, 1, 8, 2, 500, 2, 32, 32, 4, 20), [1, 20]),              # GQA 4, 2-bit
    (_w(203, 2, 4, 2, 100, 4, 128, 16, 0, 30), [1, 15, 30]),         # GQA 2, no sinks, G = 128
    (_w(204, 1, 2, 2, 2, 2, 32, 8, 4, 20), [1, 2, 3, 10, 11, 20]),   # L < sinks: sinks fill, then window
    (_w(205, 2, 2, 2, 36, 4, 64, 32, 4, 3), [1, 3]),                 # L = sinks + R: nothing quantized yet
    (_w(206, 1, 4, 4, 1000, 2, 64, 512, 8, 5), [1, 5]),              # R = 512, 8 sinks
    (_w(207, 3, 3, 3, 777, 4, 32, 20, 5, 25), [1, 7, 25]),           # window not a multiple of G or 16
    (_w(208, 1, 1, 1, 4000, 4, 64, 32, 4, 2), [1, 2]),               # several 512-token splits
]


def _cache_and_ref(w, key_norm=0):
    cfg, cache = make_innerq_cache(w.bits, w.group, w.residual, w.sinks, w.batch, w.num_q_heads,
                                   w.num_kv_heads, w.max_tokens, key_norm=key_norm)
    ref = oracle.InnerQCache(w.bits, w.group, w.residual, w.sinks, w.batch, w.num_kv_heads, 128,
                             key_norm=bool(key_norm))
    return cfg, cache, ref


@pytest.mark.parametrize("w,checks", CASES, ids=[c[0].name for c in CASES])
def test_innerq_prefill_append_attention_parity(w, checks):
    print(f"case {w.name}", flush=True)
    k, v = gen_prefill(w, 0, "cuda")
    kn, vn = gen_new_tokens(w, 0, "cuda")
    qs = gen_queries(w, 0, "cuda")
    cfg, cache, ref = _cache_and_ref(w)
    cache.prefill(k, v)
    ref.prefill(host(k), host(v))
    torch.cuda.synchronize()
    compare_innerq_buffers(cache, ref)
    scale = 1.0 / math.sqrt(128)
    ws = cache.workspace()
    for step in range(1, w.steps + 1):
        cache.append(kn[step - 1].contiguous(), vn[step - 1].contiguous())
        ref.append(host(kn[step - 1]), host(vn[step - 1]))
        assert (cache.n_tokens, cache.nq_k) == (ref.n, ref.nq)
        if step in checks:
            q = qs[step - 1].contiguous()
            out = cache.attention(q, scale, workspace=ws)
            torch.cuda.synchronize()
            compare_innerq_buffers(cache, ref)
            err = max_err(out, oracle_attention(ref, host(q), scale))
            print(f"  step {step}: n={ref.n} nq={ref.nq} window={ref.rk.shape[2]} err={err:.2e}", flush=True)
            assert err <= ATOL


def test_innerq_modes_both_occur_on_the_workload():
    """The synthetic inputs exercise both the symmetric and asymmetric map."""
    w = CASES[0][0]
    k, v = gen_prefill(w, 0, "cuda")
    cfg, cache, ref = _cache_and_ref(w)
    cache.prefill(k, v)
    torch.cuda.synchronize()
    half = -(1 << (w.bits - 1))
    for name in ("k_zero", "v_zero"):
        z = host(cache.tensors[name][:, :, w.sinks:cache.nq_k])
        frac = float(np.mean(z == half))
        print(f"  {name}: symmetric fraction {frac:.2f}", flush=True)
        assert 0.05 < frac < 0.95


@pytest.mark.parametrize("hpg", [1, 4])
def test_innerq_split_count_invariance_and_determinism(hpg):
    w = _w(210 + hpg, 2, 2 * hpg, 2, 3000, 4, 64, 32, 4, 1)
    print(f"case {w.name}", flush=True)
    k, v = gen_prefill(w, 0, "cuda")
    kn, vn = gen_new_tokens(w, 0, "cuda")
    q = gen_queries(w, 0, "cuda")[0].contiguous()
    cfg, cache, ref = _cache_and_ref(w)
    cache.prefill(k, v)
    cache.append(kn[0].contiguous(), vn[0].contiguous())
    ref.prefill(host(k), host(v))
    ref.append(host(kn[0]), host(vn[0]))
    want = oracle_attention(ref, host(q), 1 / math.sqrt(128))
    outs = []
    for s in (1, 2, 5, 16, 64, 0):
        ws = cache.workspace(splits=s)
        o = cache.attention(q, workspace=ws, splits=s)
        torch.cuda.synchronize()
        assert max_err(o, want) <= ATOL, s
        outs.append(host(o))
    for o in outs[1:]:
        assert float(np.abs(o - outs[0]).max()) <= 1e-5
    again = host(cache.attention(q, splits=0))
    assert np.array_equal(again, outs[-1]), "reruns must be bit-identical"


def test_innerq_empty_prefill_single_token_and_capacity():
    w = _w(220, 1, 2, 2, 0, 2, 32, 8, 4, 16)
    kn, vn = gen_new_tokens(w, 0, "cuda")
    qs = gen_queries(w, 0, "cuda")
    cfg, cache = make_innerq_cache(2, 32, 8, 4, 1, 2, 2, 16)
    ref = oracle.InnerQCache(2, 32, 8, 4, 1, 2, 128)
    cache.prefill(None, None)
    ref.prefill(np.zeros((1, 2, 0, 128), np.float16), np.zeros((1, 2, 0, 128), np.float16))
    with pytest.raises(kvq.KVQError):
        cache.attention(qs[0].contiguous())
    for step in range(16):
        cache.append(kn[step].contiguous(), vn[step].contiguous())
        ref.append(host(kn[step]), host(vn[step]))
        out = cache.attention(qs[step].contiguous())
        torch.cuda.synchronize()
        assert max_err(out, oracle_attention(ref, host(qs[step]), 1 / math.sqrt(128))) <= ATOL, step
        if step == 0:
            np.testing.assert_allclose(host(out), host(vn[0]).astype(np.float32), atol=1e-6)
    compare_innerq_buffers(cache, ref)
    assert cache.n_tokens == 16 and cache.nq_k == 8
    with pytest.raises(kvq.KVQError) as e:
        cache.append(kn[0].contiguous(), vn[0].contiguous())
    assert e.value.status == kvq.KVQ_ERR_CAPACITY


@pytest.mark.parametrize("key_norm", [0, 1], ids=["plain", "key-norm"])
def test_innerq_decode_step_matches_append_then_attention(key_norm):
    """The window is full after the prompt, so every step pops: the first one
    with a small quantize launch, later ones from the rows the previous
    step's attention launch quantized ahead."""
    w = _w(230, 2, 4, 2, 100, 4, 64, 32, 4, 20)
    print(f"case {w.name} key_norm={key_norm}", flush=True)
    k, v = gen_prefill(w, 0, "cuda")
    kn, vn = gen_new_tokens(w, 0, "cuda")
    qs = gen_queries(w, 0, "cuda")
    _, a, ref = _cache_and_ref(w, key_norm)
    _, b, _ = _cache_and_ref(w, key_norm)
    a.prefill(k, v)
    b.prefill(k, v)
    ref.prefill(host(k), host(v))
    wa, wb = a.workspace(), b.workspace()
    for i in range(w.steps):
        q = qs[i].contiguous()
        oa = a.step(kn[i].contiguous(), vn[i].contiguous(), q, workspace=wa)
        b.append(kn[i].contiguous(), vn[i].contiguous())
        ob = b.attention(q, workspace=wb)
        ref.append(host(kn[i]), host(vn[i]))
        assert (a.n_tokens, a.nq_k) == (ref.n, ref.nq)
        assert a.c.prequant == ref.nq + 1, "a full window: its oldest token is quantized ahead"
        torch.cuda.synchronize()
        assert torch.equal(oa, ob), i
    assert max_err(oa, oracle_attention(ref, host(q), 1 / math.sqrt(128))) <= ATOL
    compare_innerq_buffers(a, ref)


def test_innerq_steps_and_appends_interleaved():
    """Fused steps, plain appends and attention calls in a seeded random
    order, from a prompt shorter than the window (the window fills during the
    run): the rows quantized ahead by a step are used by the next append or
    step, and every state matches the oracle."""
    w = _w(231, 1, 2, 2, 20, 2, 32, 16, 2, 60)
    k, v = gen_prefill(w, 0, "cuda")
    kn, vn = gen_new_tokens(w, 0, "cuda")
    qs = gen_queries(w, 0, "cuda")
    _, cache, ref = _cache_and_ref(w)
    cache.prefill(k, v)
    ref.prefill(host(k), host(v))
    ws = cache.workspace()
    scale = 1 / math.sqrt(128)
    order = np.random.default_rng(231).integers(0, 3, size=w.steps)
    for i in range(w.steps):
        q = qs[i].contiguous()
        if order[i] == 0:
            out = cache.step(kn[i].contiguous(), vn[i].contiguous(), q, workspace=ws)
        else:
            cache.append(kn[i].contiguous(), vn[i].contiguous())
            out = cache.attention(q, workspace=ws) if order[i] == 1 else None
        ref.append(host(kn[i]), host(vn[i]))
        assert (cache.n_tokens, cache.nq_k) == (ref.n, ref.nq), i
        if out is not None:
            torch.cuda.synchronize()
            assert max_err(out, oracle_attention(ref, host(q), scale)) <= ATOL, i
        if i % 10 == 9:
            compare_innerq_buffers(cache, ref)
    compare_innerq_buffers(cache, ref)


# One-time per-channel key scales (KVQ_KEYNORM_PROMPT): the scales, the
# normalized quantized keys and the window are bit-exact, attention within
# 2e-3.  Case 204 takes its scales from a 2-token prompt and quantizes later
# keys with them; 209 appends keys 50x beyond the prompt's range.
NORM_CASES = [
    (CASES[0][0], [1, 2, 40]),
    (CASES[1][0], [1, 20]),
    (CASES[3][0], [1, 2, 3, 10, 11, 20]),
    (CASES[7][0], [1, 2]),
    (_w(209, 2, 4, 4, 300, 4, 64, 32, 4, 40, 4, 3.0), [1, 40]),
]


@pytest.mark.parametrize("w,checks", NORM_CASES, ids=[c[0].name + "-norm" for c in NORM_CASES])
def test_innerq_key_norm_parity(w, checks):
    print(f"case {w.name} with key scales", flush=True)
    k, v = gen_prefill(w, 0, "cuda")
    kn, vn = gen_new_tokens(w, 0, "cuda")
    if w.config_id == 209:
        kn = (kn.float() * 50).clamp(-60000, 60000).half()
    qs = gen_queries(w, 0, "cuda")
    cfg, cache = make_innerq_cache(w.bits, w.group, w.residual, w.sinks, w.batch, w.num_q_heads, w.num_kv_heads,
                                   w.max_tokens, key_norm=kvq.KVQ_KEYNORM_PROMPT)
    ref = oracle.InnerQCache(w.bits, w.group, w.residual, w.sinks, w.batch, w.num_kv_heads, 128, key_norm=True)
    cache.prefill(k, v)
    ref.prefill(host(k), host(v))
    torch.cuda.synchronize()
    compare_innerq_buffers(cache, ref)
    assert float(ref.k_norm.max()) > 1.0 or w.context <= w.sinks, "the scales must matter on this input"
    scale = 1.0 / math.sqrt(128)
    ws = cache.workspace()
    for step in range(1, w.steps + 1):
        cache.append(kn[step - 1].contiguous(), vn[step - 1].contiguous())
        ref.append(host(kn[step - 1]), host(vn[step - 1]))
        if step in checks:
            q = qs[step - 1].contiguous()
            out = cache.attention(q, scale, workspace=ws)
            torch.cuda.synchronize()
            compare_innerq_buffers(cache, ref)
            err = max_err(out, oracle_attention(ref, host(q), scale))
            print(f"  step {step}: n={ref.n} nq={ref.nq} err={err:.2e}", flush=True)
            assert err <= ATOL


@pytest.mark.parametrize("splits", [1, 4, 0])
def test_innerq_wave_orders_agree(splits):
    """9000 tokens: with one split a wave's contiguous share would span more
    than 32 KiB of key codes, so its waves take every eighth step; with four
    splits each wave keeps a contiguous range.  Both orders match the oracle
    and each other within the split tolerance."""
    w = _w(240, 1, 4, 4, 9000, 4, 64, 32, 4, 1)
    print(f"case {w.name} splits {splits}", flush=True)
    k, v = gen_prefill(w, 0, "cuda")
    kn, vn = gen_new_tokens(w, 0, "cuda")
    q = gen_queries(w, 0, "cuda")[0].contiguous()
    _, cache, ref = _cache_and_ref(w)
    cache.prefill(k, v)
    cache.append(kn[0].contiguous(), vn[0].contiguous())
    ref.prefill(host(k), host(v))
    ref.append(host(kn[0]), host(vn[0]))
    want = oracle_attention(ref, host(q), 1 / math.sqrt(128))
    out = cache.attention(q, workspace=cache.workspace(splits=splits), splits=splits)
    torch.cuda.synchronize()
    assert max_err(out, want) <= ATOL
    compare_innerq_buffers(cache, ref)
