"""CPU pins of the bench's algorithmic byte formulas.

The bench divides these byte counts by measured kernel times, so each formula
is checked two ways against the oracle: against the oracle's own per-call
byte functions, and against the byte sizes of the oracle cache's buffer
slices that a call reads or writes (serialized in the library's device layout
by oracle buffers()).  The bench's timed loop itself never imports the oracle.
"""
import itertools

import numpy as np
import pytest

import bench
import decode_attention_token_amd as kvq
import oracle
from workloads import Workload

D = 128


def _w(bits, G, R, B=2, Hq=2, Hkv=2, policy=0, scheme=0, sinks=0, meta=0, L=300):
    return Workload("bytes", 900, B, Hq, Hkv, D, L, bits, G, R, 2, 8.0, 1, 1, policy, scheme, sinks, meta)


def _ref(w):
    if w.scheme == kvq.KVQ_SCHEME_INNERQ:
        return oracle.InnerQCache(w.bits, w.group, w.residual, w.sinks, w.batch, w.num_kv_heads, D)
    if w.sinks:
        return oracle.KiviSinkCache(w.bits, w.group, w.residual, w.sinks, w.batch, w.num_kv_heads, D,
                                    w.v_policy, w.meta)
    return oracle.QuantizedKVCache(w.bits, w.group, w.residual, w.batch, w.num_kv_heads, D, w.v_policy, w.meta)


def _tokens(w, n, seed):
    rng = np.random.default_rng(seed)
    shape = (w.batch, w.num_kv_heads, n, D)
    return rng.standard_normal(shape).astype(np.float16), rng.standard_normal(shape).astype(np.float16)


def _quantized_bytes(ref, cap):
    """Per-unit bytes of the quantized slices (codes + metadata) held by the
    oracle cache, read off its serialized buffers."""
    bufs = ref.buffers(cap)
    units = ref.B * ref.H
    if isinstance(ref, oracle.InnerQCache):
        rows = slice(ref.S, ref.nq) if ref.n > ref.S else slice(0, 0)
        names = ("k_codes", "k_scale", "k_zero", "v_codes", "v_scale", "v_zero")
        return sum(bufs[n][:, :, rows].nbytes for n in names) // units
    inner = ref.inner if isinstance(ref, oracle.KiviSinkCache) else ref
    G = inner.G
    total = (bufs["k_codes"][:, :, :inner.nq_k].nbytes + bufs["k_scale"][:, :, :inner.nq_k // G].nbytes
             + bufs["k_zero"][:, :, :inner.nq_k // G].nbytes + bufs["v_codes"][:, :, :inner.nq_v].nbytes
             + bufs["v_scale"][:, :, :inner.nq_v].nbytes + bufs["v_zero"][:, :, :inner.nq_v].nbytes)
    return total // units


def _fp16_bytes(ref):
    """Per-unit bytes of the live fp16 rows: residual ring or window slots and sinks."""
    ks, vs = ref.live_resid_slots()
    ns = min(ref.n, getattr(ref, "S", 0))
    return (len(ks) + len(vs) + 2 * ns) * D * 2


KIVI_CASES = [dict(bits=b, G=G, R=R, policy=p, sinks=s, meta=m)
              for (b, G), R, p, s, m in itertools.product([(2, 32), (4, 64)], [64, 128], [0, 1], [0, 4], [0, 1])]


@pytest.mark.parametrize("case", KIVI_CASES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_kivi_attention_bytes_match_oracle(case):
    w = _w(case["bits"], case["G"], case["R"], Hq=4, policy=case["policy"], sinks=case["sinks"], meta=case["meta"])
    ref = _ref(w)
    k, v = _tokens(w, 300, 1)
    ref.prefill(k, v)
    kn, vn = _tokens(w, 150, 2)
    cap = 640
    for i in range(150):
        ref.append(kn[:, :, i], vn[:, :, i])
        if i % 37 and i not in (0, 1, 149):
            continue
        got = bench.attn_bytes(w, ref.n, ref.nq_k, ref.nq_v)
        ns = min(ref.n, w.sinks)
        # the oracle's call-byte function counts quantized tokens only
        want = oracle.attention_call_bytes(w.batch, w.num_q_heads, w.num_kv_heads, D, w.bits, w.group, ref.n,
                                           ref.nq_k - ns, ref.nq_v - ns, w.meta)
        assert got == want
        slices = w.units * (_quantized_bytes(ref, cap) + _fp16_bytes(ref)) + w.batch * w.num_q_heads * D * 6
        assert got == slices


@pytest.mark.parametrize("bits,G,R,S", [(4, 64, 32, 4), (2, 32, 16, 0), (4, 128, 8, 5)])
def test_innerq_attention_bytes_match_oracle(bits, G, R, S):
    w = _w(bits, G, R, Hq=4, policy=1, scheme=1, sinks=S)
    ref = _ref(w)
    k, v = _tokens(w, 3, 3)
    ref.prefill(k, v)
    kn, vn = _tokens(w, 80, 4)
    for i in range(80):
        ref.append(kn[:, :, i], vn[:, :, i])
        got = bench.attn_bytes(w, ref.n, ref.nq, ref.nq)
        want = oracle.innerq_attention_call_bytes(w.batch, w.num_q_heads, w.num_kv_heads, D, bits, G, ref.n,
                                                  ref.nq, S)
        assert got == want
        slices = w.units * (_quantized_bytes(ref, 128) + _fp16_bytes(ref)) + w.batch * w.num_q_heads * D * 6
        assert got == slices


PREFILL_CASES = [(0, 0, 0), (1, 0, 0), (0, 4, 0), (1, 4, 1), (0, 0, 1)]


@pytest.mark.parametrize("policy,sinks,meta", PREFILL_CASES)
@pytest.mark.parametrize("L", [0, 3, 64, 200, 256])
def test_kivi_prefill_bytes_match_oracle(policy, sinks, meta, L):
    w = _w(2, 32, 64, policy=policy, sinks=sinks, meta=meta, L=L)
    ref = _ref(w)
    ref.prefill(*_tokens(w, L, 5))
    want = w.units * (L * D * 2 * 2 + _quantized_bytes(ref, 320) + _fp16_bytes(ref))
    assert bench.prefill_bytes(w, L) == want


@pytest.mark.parametrize("L", [0, 2, 20, 100])
def test_innerq_prefill_bytes_match_oracle(L):
    w = _w(4, 64, 32, policy=1, scheme=1, sinks=4, L=L)
    ref = _ref(w)
    ref.prefill(*_tokens(w, L, 6))
    want = w.units * (L * D * 2 * 2 + _quantized_bytes(ref, 128) + _fp16_bytes(ref))
    assert bench.prefill_bytes(w, L) == want


@pytest.mark.parametrize("policy", [0, 1])
@pytest.mark.parametrize("meta", [0, 1])
@pytest.mark.parametrize("bits,G,R", [(2, 32, 128), (4, 64, 128), (2, 32, 64)])
def test_kivi_flush_bytes_match_oracle(policy, meta, bits, G, R):
    """The append that flushes: quantized slices it adds, plus the fp16 rows it
    reads (R keys; chunked: R values; FIFO: the popped value and the new one)
    and, with FIFO values, the new value's ring store."""
    w = _w(bits, G, R, policy=policy, meta=meta, L=2 * R)
    ref = _ref(w)
    ref.prefill(*_tokens(w, 2 * R, 7))
    kn, vn = _tokens(w, R, 8)
    for i in range(R - 1):
        ref.append(kn[:, :, i], vn[:, :, i])
    before = _quantized_bytes(ref, 4 * R)
    f0 = ref.flushes
    ref.append(kn[:, :, R - 1], vn[:, :, R - 1])
    assert ref.flushes == f0 + 1
    written = _quantized_bytes(ref, 4 * R) - before
    fp16_moved = R * D * 2 + (R * D * 2 if policy == 0 else 3 * D * 2)
    assert bench.flush_bytes(w) == w.units * (written + fp16_moved)


def test_innerq_flush_bytes_match_oracle():
    """An InnerQ append whose window is full: the leaving token's codes and
    metadata out, its fp16 row and the new token in, the new token's ring
    slot out."""
    w = _w(4, 64, 32, policy=1, scheme=1, sinks=4, L=100)
    ref = _ref(w)
    ref.prefill(*_tokens(w, 100, 9))
    kn, vn = _tokens(w, 1, 10)
    before = _quantized_bytes(ref, 128)
    nq0 = ref.nq
    ref.append(kn[:, :, 0], vn[:, :, 0])
    assert ref.nq == nq0 + 1
    written = _quantized_bytes(ref, 128) - before
    assert bench.flush_bytes(w) == w.units * (written + 3 * 2 * D * 2)
