"""GPU parity of the matrix-core kernel for four query heads per kv head
(KIVI layout): bf16 MFMA tiles with two-limb operands against the float64
oracle, across bit widths, group sizes, value policies, sink tokens,
metadata formats, split counts and both work schedules; and against the
vector-ALU kernel (config kernel = KVQ_KERNEL_VALU) on the same cache."""
import math

import numpy as np
import pytest
import torch

import decode_attention_token_amd as kvq
import oracle
from workloads import Workload, gen_new_tokens, gen_prefill, gen_queries
from gpu_helpers import (ATOL, SPLIT_TOL_MFMA, compare_all_buffers, compare_sink_unit, config_fields, host, max_err, oracle_attention,
                         queue_schedule)

pytestmark = pytest.mark.gpu

CHUNK, FIFO = kvq.KVQ_V_CHUNK, kvq.KVQ_V_FIFO


def _w(cid, B, L, bits, G, R, steps, policy=CHUNK, sinks=0, meta=0, hkv=2):
    return Workload(f"mfma{cid}", cid, B, 4 * hkv, hkv, 128, L, bits, G, R, 4, 10.0, steps, 1, policy,
                    sinks=sinks, meta=meta)


# (workload, steps at which attention is checked)
CASES = [
    (_w(401, 2, 1000, 2, 32, 128, 30), [1, 24, 25, 30]),                     # flush at 25
    (_w(402, 1, 700, 4, 32, 64, 6), [1, 4, 5, 6]),                           # 4-bit
    (_w(403, 2, 900, 2, 64, 128, 5, FIFO), [1, 5]),                          # G = 64, FIFO tail part
    (_w(404, 1, 1500, 4, 128, 128, 3, CHUNK, 0, 1), [1, 3]),                  # G = 128, packed metadata
    (_w(405, 2, 500, 2, 32, 64, 13, CHUNK, 4, 1), [1, 12, 13]),               # sinks + packed metadata
    (_w(406, 1, 800, 4, 64, 128, 2, FIFO, 4), [1, 2]),                       # sinks + FIFO: three kinds of parts
    (_w(407, 3, 97, 2, 32, 32, 40), [1, 31, 32, 40]),                        # a few groups only
    (_w(408, 1, 5000, 2, 32, 128, 1, CHUNK, 0, 0, 8), [1]),                  # 8 kv heads, ragged split ranges
    (_w(409, 1, 3000, 2, 128, 512, 3, FIFO, 512), [1, 3]),                   # largest fp16 list: 512 sinks + 639
    (_w(410, 2, 1200, 4, 64, 128, 4, FIFO, 8, 1), [1, 4]),                   # 4-bit FIFO, sinks, packed metadata
]


def _ref(w):
    if w.sinks:
        return oracle.KiviSinkCache(w.bits, w.group, w.residual, w.sinks, w.batch, w.num_kv_heads, 128,
                                    w.v_policy, w.meta)
    return oracle.QuantizedKVCache(w.bits, w.group, w.residual, w.batch, w.num_kv_heads, 128, w.v_policy, w.meta)


def _cache(w):
    cfg = kvq.make_config(w.bits, w.group, w.residual, w.batch, w.num_q_heads, w.num_kv_heads, 128,
                          w.max_tokens + w.residual, w.v_policy, kvq.KVQ_SCHEME_KIVI, w.sinks, w.meta)
    return kvq.KVCache(cfg, "cuda")


def _attention(cache, q, path, **kw):
    kernel = kvq.KVQ_KERNEL_VALU if path == "valu" else kvq.KVQ_KERNEL_AUTO
    with config_fields(cache, kernel=kernel):
        out = cache.attention(q, **kw)
        torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("w,checks", CASES, ids=[c[0].name for c in CASES])
def test_gqa_mfma_parity(w, checks):
    print(f"case {w.name} bits={w.bits} G={w.group} R={w.residual} policy={w.v_policy} sinks={w.sinks} "
          f"meta={w.meta} L={w.context}", flush=True)
    k, v = gen_prefill(w, 0, "cuda")
    kn, vn = gen_new_tokens(w, 0, "cuda")
    qs = gen_queries(w, 0, "cuda")
    cache, ref = _cache(w), _ref(w)
    cache.prefill(k, v)
    ref.prefill(host(k), host(v))
    scale = 1.0 / math.sqrt(128)
    for step in range(1, w.steps + 1):
        cache.append(kn[step - 1].contiguous(), vn[step - 1].contiguous())
        ref.append(host(kn[step - 1]), host(vn[step - 1]))
        if step in checks:
            q = qs[step - 1].contiguous()
            want = oracle_attention(ref, host(q), scale)
            out_m = _attention(cache, q, "mfma")
            out_v = _attention(cache, q, "valu")
            em, ev = max_err(out_m, want), max_err(out_v, want)
            print(f"  step {step}: n={ref.n} nq_k={ref.nq_k} nq_v={ref.nq_v} err mfma={em:.2e} valu={ev:.2e}",
                  flush=True)
            assert em <= ATOL and ev <= ATOL
            if w.sinks:
                for b in range(w.batch):
                    for h in range(w.num_kv_heads):
                        compare_sink_unit(cache, ref, b, h)


@pytest.mark.parametrize("policy,sinks", [(CHUNK, 0), (FIFO, 6)], ids=["chunk", "fifo-sinks"])
def test_gqa_mfma_fp16_shares_on_leading_splits(policy, sinks):
    """80 units: a launch of 8 or 16 splits per unit has its first 3 splits
    in the first dispatch round (256 compute units), and only those take the
    unit's fp16 tokens (sinks, the residual, the fused token).  Checked against
    the oracle and the vector-ALU kernel at several split counts, and through
    the fused step."""
    w = _w(450 + sinks, 40, 700, 2, 32, 128, 2, policy, sinks, 0, 2)
    print(f"case {w.name} units {w.units} policy {policy} sinks {sinks}", flush=True)
    k, v = gen_prefill(w, 0, "cuda")
    kn, vn = gen_new_tokens(w, 0, "cuda")
    qs = gen_queries(w, 0, "cuda")
    cache, ref = _cache(w), _ref(w)
    cache.prefill(k, v)
    ref.prefill(host(k), host(v))
    scale = 1.0 / math.sqrt(128)
    cache.append(kn[0].contiguous(), vn[0].contiguous())
    ref.append(host(kn[0]), host(vn[0]))
    q = qs[0].contiguous()
    want = oracle_attention(ref, host(q), scale)
    for s in (8, 16, 0):
        o = _attention(cache, q, "mfma", workspace=cache.workspace(splits=s), splits=s)
        err = max_err(o, want)
        print(f"  splits {s}: n={ref.n} rest={ref.n - (ref.nq_k // 32) * 32} err {err:.2e}", flush=True)
        assert err <= ATOL, s
    assert max_err(_attention(cache, q, "valu"), want) <= ATOL
    # the fused step takes the same path
    q = qs[1].contiguous()
    out = cache.step(kn[1].contiguous(), vn[1].contiguous(), q, scale, workspace=cache.workspace(splits=8),
                     splits=8)
    ref.append(host(kn[1]), host(vn[1]))
    torch.cuda.synchronize()
    assert max_err(out, oracle_attention(ref, host(q), scale)) <= ATOL


@pytest.mark.parametrize("bits,G", [(2, 32), (4, 64)])
def test_gqa_mfma_split_counts_and_reruns(bits, G):
    w = _w(420 + bits, 2, 4000, bits, G, 128, 1)
    print(f"case {w.name}", flush=True)
    k, v = gen_prefill(w, 0, "cuda")
    kn, vn = gen_new_tokens(w, 0, "cuda")
    q = gen_queries(w, 0, "cuda")[0].contiguous()
    cache, ref = _cache(w), _ref(w)
    cache.prefill(k, v)
    cache.append(kn[0].contiguous(), vn[0].contiguous())
    ref.prefill(host(k), host(v))
    ref.append(host(kn[0]), host(vn[0]))
    want = oracle_attention(ref, host(q), 1 / math.sqrt(128))
    outs = []
    for s in (1, 2, 7, 31, 64, 0):
        o = _attention(cache, q, "mfma", workspace=cache.workspace(splits=s), splits=s)
        err = max_err(o, want)
        print(f"  splits {s}: err {err:.2e}", flush=True)
        assert err <= ATOL, s
        outs.append(host(o))
    for o in outs[1:]:
        assert float(np.abs(o - outs[0]).max()) <= SPLIT_TOL_MFMA
    # The default fixed schedule gives bit-identical reruns.  With one split
    # (four waves over 31 super-chunks) the work-queue schedule runs mostly
    # from the queue, whose hand-out order varies between runs: its results
    # agree with the fixed order to fp32 reordering.
    for s in (1, 0):
        a = host(_attention(cache, q, "mfma", splits=s))
        b = host(_attention(cache, q, "mfma", splits=s))
        assert np.array_equal(a, b), f"splits {s}: reruns must be bit-identical"
        assert float(np.abs(a.astype(np.float64) - want).max()) <= ATOL
        with queue_schedule(cache):
            for _ in range(3):
                dyn = host(_attention(cache, q, "mfma", splits=s))
                assert float(np.abs(dyn - a).max()) <= SPLIT_TOL_MFMA
                assert float(np.abs(dyn.astype(np.float64) - want).max()) <= ATOL


@pytest.mark.parametrize("policy,sinks", [(CHUNK, 0), (FIFO, 0), (FIFO, 4)], ids=["chunk", "fifo", "fifo-sinks"])
def test_gqa_mfma_fused_step_matches_append_then_attention(policy, sinks):
    w = _w(430, 2, 300, 2, 32, 64, 40, policy, sinks)
    print(f"case {w.name} policy {policy} sinks {sinks}", flush=True)
    k, v = gen_prefill(w, 0, "cuda")
    kn, vn = gen_new_tokens(w, 0, "cuda")
    qs = gen_queries(w, 0, "cuda")
    a, b, ref = _cache(w), _cache(w), _ref(w)
    a.prefill(k, v)
    b.prefill(k, v)
    ref.prefill(host(k), host(v))
    for i in range(w.steps):
        q = qs[i].contiguous()
        oa = a.step(kn[i].contiguous(), vn[i].contiguous(), q)
        b.append(kn[i].contiguous(), vn[i].contiguous())
        ob = b.attention(q)
        ref.append(host(kn[i]), host(vn[i]))
        assert (a.n_tokens, a.nq_k, a.nq_v) == (ref.n, ref.nq_k, ref.nq_v)
        torch.cuda.synchronize()
        assert torch.equal(oa, ob), i
    assert max_err(oa, oracle_attention(ref, host(q), 1 / math.sqrt(128))) <= ATOL
    if sinks:
        for bb in range(w.batch):
            for h in range(w.num_kv_heads):
                compare_sink_unit(a, ref, bb, h)
    else:
        compare_all_buffers(a, ref)


def test_gqa_mfma_large_magnitudes():
    """Keys and queries scaled up 64x: the bf16 limbs keep fp32 range, so the
    result still matches the oracle to the same bound."""
    w = _w(440, 1, 600, 2, 32, 128, 1)
    k, v = gen_prefill(w, 0, "cuda")
    kn, vn = gen_new_tokens(w, 0, "cuda")
    q = gen_queries(w, 0, "cuda")[0].contiguous()
    k, kn0, q = (k.float() * 64).half(), (kn[0].float() * 64).half(), (q.float() / 8).half()
    cache, ref = _cache(w), _ref(w)
    cache.prefill(k, v)
    cache.append(kn0.contiguous(), vn[0].contiguous())
    ref.prefill(host(k), host(v))
    ref.append(host(kn0), host(vn[0]))
    err = max_err(_attention(cache, q, "mfma"), oracle_attention(ref, host(q), 1 / math.sqrt(128)))
    print(f"  err {err:.2e}", flush=True)
    assert err <= ATOL


def test_gqa_mfma_work_queue_counters():
    """The per-unit counters at the start of the workspace (ticket, pad, and a
    64-bit election word tagged with the launch) are zero after every call.
    A ticket that did not start at zero makes that unit's output NaN under the
    work-queue schedule (some super-chunks would be skipped) instead of a
    wrong number; the call returns it to zero and the next call is right.  An
    election word left over from another launch is ignored: the call is
    right, with one split or several, and the word is zero afterwards."""
    w = _w(450, 2, 4000, 2, 32, 128, 1)
    k, v = gen_prefill(w, 0, "cuda")
    kn, vn = gen_new_tokens(w, 0, "cuda")
    q = gen_queries(w, 0, "cuda")[0].contiguous()
    cache, ref = _cache(w), _ref(w)
    cache.prefill(k, v)
    cache.append(kn[0].contiguous(), vn[0].contiguous())
    ref.prefill(host(k), host(v))
    ref.append(host(kn[0]), host(vn[0]))
    want = oracle_attention(ref, host(q), 1 / math.sqrt(128))
    units = w.batch * w.num_kv_heads
    u = units - 1                         # unit (batch 1, kv head 1): query heads 4..7 of batch 1
    b, h = divmod(u, w.num_kv_heads)
    keep = np.ones(want.shape[:2], bool)
    keep[b, 4 * h:4 * h + 4] = False
    for schedule in (kvq.KVQ_SCHED_FIXED, kvq.KVQ_SCHED_QUEUE):
        with config_fields(cache, schedule=schedule):
            for splits in (1, 2, 5):
                print(f"  schedule {schedule} splits {splits}", flush=True)
                ws = cache.workspace(splits=splits)
                ctr = ws.view(torch.int32)[: 4 * units]
                out = _attention(cache, q, "mfma", workspace=ws, splits=splits)
                assert max_err(out, want) <= ATOL
                assert int(ctr.abs().sum()) == 0, host(ctr)
                # a stale election word: another launch's tag, some workgroups counted
                # (epochs 0 and near 2^32 are never those of a launch in this process)
                for stale in ((0xFFFFFFF0 << 32) | (1 << 24) | 7, (1 << 24), (0xFFFFFFFF << 32) | (3 << 24)):
                    ctr.view(torch.int64)[2 * u + 1] = int(np.array(stale, np.uint64).view(np.int64))
                    out = _attention(cache, q, "mfma", workspace=ws, splits=splits)
                    assert max_err(out, want) <= ATOL, (schedule, splits, stale)
                    assert int(ctr.abs().sum()) == 0, host(ctr)
                if schedule == kvq.KVQ_SCHED_QUEUE:
                    # each of the 4 * splits waves takes its first two super-chunks
                    # (four key groups each) by index; the ticket is read only
                    # when more super-chunks remain
                    nsc = -(-(min(ref.nq_k, ref.nq_v) // 32) // 4)
                    queued = 2 * 4 * splits < nsc
                    ctr[4 * u] = 5                # a ticket that did not start at zero
                    got = host(_attention(cache, q, "mfma", workspace=ws, splits=splits))
                    if queued:
                        assert np.isnan(got[b, 4 * h:4 * h + 4]).all(), "a miscounted unit must come out NaN"
                        assert float(np.abs(got[keep].astype(np.float64) - want[keep]).max()) <= ATOL
                    else:
                        assert float(np.abs(got.astype(np.float64) - want).max()) <= ATOL
                    assert int(ctr.abs().sum()) == 0, host(ctr)
                    assert max_err(_attention(cache, q, "mfma", workspace=ws, splits=splits), want) <= ATOL
