"""Host-only checks of the C ABI: the library loads, exports every function the
header declares, sizes buffers by the documented layout and rejects invalid
calls with a status code before touching the device."""
import ctypes
import os
import re

import pytest

import decode_attention_token_amd as kvq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kvq.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return kvq.load_library()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z_]+)\s*\(", text)))


def test_header_declares_the_binding_surface():
    assert _declared() == sorted(kvq.EXPORTED)


def test_every_declared_symbol_is_exported(lib):
    for name in _declared():
        assert hasattr(lib, name), name


def cfg(**kw):
    base = dict(bits=2, group=32, residual=128, batch=16, num_q_heads=32, num_kv_heads=32,
                head_dim=128, max_tokens=4224, v_policy=0)
    base.update(kw)
    return kvq.make_config(**base)


def test_layout_bytes_follow_the_documented_layout(lib):
    c = cfg()
    lay = kvq.kvq_layout_bytes(c)
    units, cap, d, G, R = 16 * 32, 4224, 128, 32, 128
    assert lay.k_codes == units * cap * (d * 2 // 32) * 4
    assert lay.k_scale == units * (cap // G) * d * 4
    assert lay.k_zero == units * (cap // G) * d * 2
    assert lay.v_codes == lay.k_codes
    assert lay.v_scale == units * cap * (d // G) * 4
    assert lay.v_zero == units * cap * (d // G) * 2
    assert lay.k_resid == lay.v_resid == units * R * d * 2
    lay4 = kvq.kvq_layout_bytes(cfg(bits=4, group=64))
    assert lay4.k_codes == units * cap * (d * 4 // 32) * 4


@pytest.mark.parametrize("bad,status", [
    (dict(bits=3), kvq.KVQ_ERR_ARG),
    (dict(bits=8), kvq.KVQ_ERR_ARG),
    (dict(residual=48), kvq.KVQ_ERR_ARG),          # R % G != 0
    (dict(residual=0), kvq.KVQ_ERR_ARG),
    (dict(group=48, residual=96), kvq.KVQ_ERR_ARG),  # d % G != 0
    (dict(group=8, residual=128), kvq.KVQ_ERR_ARG),  # G*bits % 32 != 0
    (dict(num_q_heads=30), kvq.KVQ_ERR_ARG),        # Hq % Hkv != 0
    (dict(max_tokens=4100), kvq.KVQ_ERR_ARG),       # capacity not a multiple of R
    (dict(v_policy=7), kvq.KVQ_ERR_ARG),
    (dict(head_dim=64, group=32), kvq.KVQ_ERR_UNSUPPORTED),
    (dict(group=16, residual=128), kvq.KVQ_ERR_UNSUPPORTED),
    (dict(num_q_heads=256), kvq.KVQ_ERR_UNSUPPORTED),   # 8 query heads per kv head
    (dict(residual=1024, max_tokens=8192), kvq.KVQ_ERR_UNSUPPORTED),
])
def test_invalid_configs_are_rejected(lib, bad, status):
    c = cfg(**bad)
    out = kvq.kvq_layout()
    assert lib.kvq_layout_bytes(ctypes.byref(c), ctypes.byref(out)) == status
    assert lib.kvq_last_error().decode() != ""
    assert lib.kvq_workspace_bytes(ctypes.byref(c), 4096, 0) == 0


def _fake_cache(started=0, n=0):
    c = kvq.kvq_cache()
    for i, name in enumerate(("k_codes", "k_scale", "k_zero", "v_codes", "v_scale", "v_zero",
                              "k_resid", "v_resid")):
        setattr(c, name, 0x1000 * (i + 1))        # never dereferenced: calls below fail validation
    c.started, c.n_tokens = started, n
    return c


def _snapshot(c):
    return (c.n_tokens, c.nq_k, c.nq_v, c.started, c.flushes)


def test_state_and_argument_errors_leave_counters_unchanged(lib):
    c = cfg()
    P = ctypes.byref
    cache = _fake_cache()
    before = _snapshot(cache)
    # append / attention before prefill
    assert lib.kvq_append_token(P(c), P(cache), 1, 1, None) == kvq.KVQ_ERR_STATE
    assert lib.kvq_decode_attention(P(c), P(cache), 1, 0.1, 1, 1, 1 << 30, 0, None) == kvq.KVQ_ERR_STATE
    # prefill longer than the capacity, negative, or with null inputs
    assert lib.kvq_quantize_prefill(P(c), P(cache), 1, 1, 5000, None) == kvq.KVQ_ERR_CAPACITY
    assert lib.kvq_quantize_prefill(P(c), P(cache), 1, 1, -1, None) == kvq.KVQ_ERR_ARG
    assert lib.kvq_quantize_prefill(P(c), P(cache), None, 1, 10, None) == kvq.KVQ_ERR_ARG
    # null cache buffers
    empty = kvq.kvq_cache()
    assert lib.kvq_quantize_prefill(P(c), P(empty), 1, 1, 10, None) == kvq.KVQ_ERR_ARG
    assert lib.kvq_quantize_prefill(P(c), None, 1, 1, 10, None) == kvq.KVQ_ERR_ARG
    assert _snapshot(cache) == before
    # a started cache refuses a second prefill; a full one refuses appends
    started = _fake_cache(started=1, n=4224)
    before = _snapshot(started)
    assert lib.kvq_quantize_prefill(P(c), P(started), 1, 1, 10, None) == kvq.KVQ_ERR_STATE
    assert lib.kvq_append_token(P(c), P(started), 1, 1, None) == kvq.KVQ_ERR_CAPACITY
    assert lib.kvq_append_token(P(c), P(_fake_cache(1, 10)), None, 1, None) == kvq.KVQ_ERR_ARG
    assert _snapshot(started) == before
    # attention argument checks
    s1 = _fake_cache(started=1, n=100)
    assert lib.kvq_decode_attention(P(c), P(s1), None, 0.1, 1, 1, 1 << 30, 0, None) == kvq.KVQ_ERR_ARG
    assert lib.kvq_decode_attention(P(c), P(s1), 1, 0.1, 1, 1, 1 << 30, 65, None) == kvq.KVQ_ERR_ARG
    assert lib.kvq_decode_attention(P(c), P(s1), 1, float("inf"), 1, 1, 1 << 30, 0, None) == kvq.KVQ_ERR_ARG
    assert lib.kvq_decode_attention(P(c), P(s1), 1, 0.1, 1, 1, 16, 0, None) == kvq.KVQ_ERR_CAPACITY
    # fused step: same checks as append + attention, nothing changes on failure
    st = _fake_cache(started=1, n=100)
    before = _snapshot(st)
    assert lib.kvq_decode_step(P(c), P(st), None, 1, 1, 0.1, 1, 1, 1 << 30, 0, None) == kvq.KVQ_ERR_ARG
    assert lib.kvq_decode_step(P(c), P(st), 1, 1, None, 0.1, 1, 1, 1 << 30, 0, None) == kvq.KVQ_ERR_ARG
    assert lib.kvq_decode_step(P(c), P(st), 1, 1, 1, 0.1, 1, 1, 16, 0, None) == kvq.KVQ_ERR_CAPACITY
    assert lib.kvq_decode_step(P(c), P(_fake_cache(1, 4224)), 1, 1, 1, 0.1, 1, 1, 1 << 30, 0, None) == kvq.KVQ_ERR_CAPACITY
    assert lib.kvq_decode_step(P(c), P(_fake_cache(0, 0)), 1, 1, 1, 0.1, 1, 1, 1 << 30, 0, None) == kvq.KVQ_ERR_STATE
    assert _snapshot(st) == before
    s0 = _fake_cache(started=1, n=0)
    assert lib.kvq_decode_attention(P(c), P(s0), 1, 0.1, 1, 1, 1 << 30, 0, None) == kvq.KVQ_ERR_STATE
    assert lib.kvq_status_string(kvq.KVQ_ERR_CAPACITY) == b"capacity exceeded"


def test_workspace_and_split_sizing(lib):
    c = cfg()
    s = kvq.kvq_auto_splits(c, 4097)
    assert 1 <= s <= 64
    assert kvq.kvq_workspace_bytes(c, 4097, 0) == 16 * 32 * (s + 1) * 132 * 4
    assert kvq.kvq_workspace_bytes(c, 4097, 3) == 16 * 32 * 4 * 132 * 4
    assert kvq.kvq_workspace_bytes(c, 4097, 65) == 0
    # more tokens never needs fewer splits, so sizing for capacity is enough
    prev = 0
    for n in range(0, 4224, 97):
        cur = kvq.kvq_auto_splits(c, n)
        assert cur >= prev
        prev = cur
