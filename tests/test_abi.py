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


def test_static_scratch_size_matches_the_header():
    m = re.search(r"#define\s+KVQ_STATIC_SCRATCH_BYTES\s+\((\d+)u\s*<<\s*(\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == kvq.KVQ_STATIC_SCRATCH_BYTES


def test_every_declared_symbol_is_exported(lib):
    for name in _declared():
        assert hasattr(lib, name), name


def cfg(**kw):
    base = dict(bits=2, group=32, residual=128, batch=16, num_q_heads=32, num_kv_heads=32,
                head_dim=128, max_tokens=4224, v_policy=0)
    base.update(kw)
    return kvq.make_config(**base)


def iq_cfg(**kw):
    base = dict(bits=4, group=64, residual=32, batch=4, num_q_heads=32, num_kv_heads=32,
                head_dim=128, max_tokens=1000, v_policy=kvq.KVQ_V_FIFO, scheme=kvq.KVQ_SCHEME_INNERQ,
                sink_tokens=4)
    base.update(kw)
    return kvq.make_config(**base)


_STRUCT_PROBE = r"""
#include <stdio.h>
#include <stddef.h>
#include "kvq.h"
#define F(T, m) printf(#T "." #m " %zu %zu\n", offsetof(T, m), sizeof(((T *)0)->m));
int main(void) {
  printf("kvq_config %zu\nkvq_layout %zu\nkvq_cache %zu\n", sizeof(kvq_config), sizeof(kvq_layout),
         sizeof(kvq_cache));
  F(kvq_config, scheme) F(kvq_config, sink_tokens) F(kvq_layout, k_sink) F(kvq_layout, v_sink)
  F(kvq_config, meta_format) F(kvq_config, schedule) F(kvq_config, kernel) F(kvq_config, key_norm)
  F(kvq_layout, k_norm) F(kvq_cache, k_norm) F(kvq_cache, prequant)
  F(kvq_cache, k_sink) F(kvq_cache, v_sink) F(kvq_cache, n_tokens) F(kvq_cache, flushes)
  return 0;
}
"""


def test_ctypes_structs_match_the_c_header(tmp_path):
    """Compiles a probe against include/kvq.h with the host C compiler and
    compares struct sizes and field offsets with the binding's ctypes view."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    src = tmp_path / "probe.c"
    src.write_text(_STRUCT_PROBE)
    exe = tmp_path / "probe"
    subprocess.run([cc, "-std=c11", "-D__HIP_PLATFORM_AMD__", "-I", os.path.dirname(HEADER),
                    "-I", "/opt/rocm/include", str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    got = {}
    for line in filter(None, out):
        parts = line.split()
        got[parts[0]] = tuple(int(x) for x in parts[1:])
    T = {"kvq_config": kvq.kvq_config, "kvq_layout": kvq.kvq_layout, "kvq_cache": kvq.kvq_cache}
    for name, ty in T.items():
        assert got[name] == (ctypes.sizeof(ty),), name
    for key, (off, size) in ((k, v) for k, v in got.items() if "." in k):
        tname, field = key.split(".")
        desc = getattr(T[tname], field)
        assert (desc.offset, desc.size) == (off, size), key


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


def test_packed_metadata_layout_bytes(lib):
    """Compressed metadata: one 32-bit word per group in the scale buffers,
    no zero-point buffers; codes and residual unchanged."""
    base, lay = kvq.kvq_layout_bytes(cfg()), kvq.kvq_layout_bytes(cfg(meta_format=kvq.KVQ_META_F16))
    units, cap, d, G = 16 * 32, 4224, 128, 32
    assert lay.k_scale == units * (cap // G) * d * 4 and lay.v_scale == units * cap * (d // G) * 4
    assert lay.k_zero == lay.v_zero == 0
    for name in ("k_codes", "v_codes", "k_resid", "v_resid", "k_sink", "v_sink"):
        assert getattr(lay, name) == getattr(base, name), name


@pytest.mark.parametrize("bad,status", [
    (cfg(meta_format=2), kvq.KVQ_ERR_ARG),
    (cfg(meta_format=-1), kvq.KVQ_ERR_ARG),
    (iq_cfg(meta_format=kvq.KVQ_META_F16), kvq.KVQ_ERR_UNSUPPORTED),
])
def test_invalid_metadata_formats_are_rejected(lib, bad, status):
    out = kvq.kvq_layout()
    assert lib.kvq_layout_bytes(ctypes.byref(bad), ctypes.byref(out)) == status
    assert "meta" in lib.kvq_last_error().decode()


@pytest.mark.parametrize("bad", [cfg(schedule=2), cfg(schedule=-1), cfg(kernel=2), cfg(kernel=-1)])
def test_invalid_launch_choices_are_rejected(lib, bad):
    out = kvq.kvq_layout()
    assert lib.kvq_layout_bytes(ctypes.byref(bad), ctypes.byref(out)) == kvq.KVQ_ERR_ARG
    err = lib.kvq_last_error().decode()
    assert "schedule" in err or "kernel" in err


def test_launch_choices_do_not_change_sizes(lib):
    base = kvq.kvq_layout_bytes(cfg(num_q_heads=128))
    for kw in (dict(schedule=kvq.KVQ_SCHED_QUEUE), dict(kernel=kvq.KVQ_KERNEL_VALU)):
        lay = kvq.kvq_layout_bytes(cfg(num_q_heads=128, **kw))
        assert all(getattr(lay, f) == getattr(base, f) for f, _ in kvq.kvq_layout._fields_), kw
        assert kvq.kvq_workspace_bytes(cfg(num_q_heads=128, **kw), 4224) == \
            kvq.kvq_workspace_bytes(cfg(num_q_heads=128), 4224)


def test_packed_metadata_needs_no_zero_buffers(lib):
    """With packed metadata the zero-point pointers may be null: validation
    passes them and stops at the next check (here the missing inputs)."""
    c = cfg(meta_format=kvq.KVQ_META_F16)
    cache = _fake_cache()
    cache.k_zero = cache.v_zero = None
    assert lib.kvq_quantize_prefill(ctypes.byref(c), ctypes.byref(cache), None, None, 10, None) == kvq.KVQ_ERR_ARG
    assert "zero" not in lib.kvq_last_error().decode()
    c32 = cfg()
    assert lib.kvq_quantize_prefill(ctypes.byref(c32), ctypes.byref(cache), None, None, 10, None) == kvq.KVQ_ERR_ARG


def test_innerq_layout_bytes(lib):
    c = iq_cfg()
    lay = kvq.kvq_layout_bytes(c)
    units, cap, d, G, R, S = 4 * 32, 1000, 128, 64, 32, 4
    assert lay.k_codes == lay.v_codes == units * cap * (d * 4 // 32) * 4
    assert lay.k_scale == lay.v_scale == units * cap * (d // G) * 4
    assert lay.k_zero == lay.v_zero == units * cap * (d // G) * 2
    assert lay.k_resid == lay.v_resid == units * R * d * 2
    assert lay.k_sink == lay.v_sink == units * S * d * 2
    assert kvq.kvq_layout_bytes(cfg()).k_sink == 0


@pytest.mark.parametrize("bad,status", [
    (dict(v_policy=kvq.KVQ_V_CHUNK), kvq.KVQ_ERR_ARG),
    (dict(sink_tokens=-1), kvq.KVQ_ERR_ARG),
    (dict(residual=0), kvq.KVQ_ERR_ARG),
    (dict(scheme=2), kvq.KVQ_ERR_ARG),
    (dict(group=48), kvq.KVQ_ERR_ARG),
    (dict(sink_tokens=513), kvq.KVQ_ERR_UNSUPPORTED),
    (dict(max_tokens=(1 << 25) + 1), kvq.KVQ_ERR_UNSUPPORTED),
    (dict(residual=513), kvq.KVQ_ERR_UNSUPPORTED),
])
def test_invalid_innerq_configs_are_rejected(lib, bad, status):
    c = iq_cfg(**bad)
    out = kvq.kvq_layout()
    assert lib.kvq_layout_bytes(ctypes.byref(c), ctypes.byref(out)) == status
    assert lib.kvq_last_error().decode() != ""


def test_innerq_relaxes_the_kivi_multiples(lib):
    # window not a multiple of G, capacity not a multiple of the window
    for kw in (dict(residual=20), dict(max_tokens=1001), dict(sink_tokens=0), dict(bits=2, group=32)):
        out = kvq.kvq_layout()
        assert lib.kvq_layout_bytes(ctypes.byref(iq_cfg(**kw)), ctypes.byref(out)) == kvq.KVQ_OK, kw
    # the KIVI scheme takes sinks too, and sizes their buffers
    out = kvq.kvq_layout()
    assert lib.kvq_layout_bytes(ctypes.byref(cfg(sink_tokens=4)), ctypes.byref(out)) == kvq.KVQ_OK
    assert out.k_sink == out.v_sink == 16 * 32 * 4 * 128 * 2
    assert lib.kvq_layout_bytes(ctypes.byref(cfg(sink_tokens=513)), ctypes.byref(out)) == kvq.KVQ_ERR_UNSUPPORTED


def test_innerq_null_sink_buffers_are_rejected(lib):
    c = iq_cfg()
    cache = _fake_cache()
    assert lib.kvq_quantize_prefill(ctypes.byref(c), ctypes.byref(cache), 1, 1, 10, None) == kvq.KVQ_ERR_ARG
    assert "sink" in lib.kvq_last_error().decode()
    assert cache.started == 0


def test_innerq_split_sizing_is_monotone(lib):
    c = iq_cfg(max_tokens=200000)
    prev = 0
    for n in list(range(0, 5000, 37)) + [131072, 199999]:
        cur = kvq.kvq_auto_splits(c, n)
        assert 1 <= cur <= 64 and cur >= prev
        prev = cur
    assert kvq.kvq_auto_splits(c, 131072) == 4   # 128 units: two 8-wave workgroups per CU


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
    # per-unit counters (four u32 per (batch, kv head): ticket, pad and a
    # 64-bit election word; padded to 256 bytes), then one record of 132
    # floats per query head and split
    ctr = 16 * 32 * 16
    assert kvq.kvq_workspace_bytes(c, 4097, 0) == ctr + 16 * 32 * s * 132 * 4
    assert kvq.kvq_workspace_bytes(c, 4097, 3) == ctr + 16 * 32 * 3 * 132 * 4
    assert kvq.kvq_workspace_bytes(c, 4097, 65) == 0
    # more tokens never needs fewer splits, so sizing for capacity is enough
    prev = 0
    for n in range(0, 4224, 97):
        cur = kvq.kvq_auto_splits(c, n)
        assert cur >= prev
        prev = cur


def test_stream_read_probe_rejects_bad_arguments_on_the_host(lib):
    """Measurement probe: null pointers, a size that is not a non-zero
    multiple of 16 and a misaligned buffer fail before any device work."""
    P = ctypes.c_void_p
    assert lib.kvq_stream_read_probe(None, 1024, P(64), None) == kvq.KVQ_ERR_ARG
    assert lib.kvq_stream_read_probe(P(64), 1024, None, None) == kvq.KVQ_ERR_ARG
    assert lib.kvq_stream_read_probe(P(64), 0, P(64), None) == kvq.KVQ_ERR_ARG
    assert lib.kvq_stream_read_probe(P(64), 1000, P(64), None) == kvq.KVQ_ERR_ARG
    assert lib.kvq_stream_read_probe(P(72), 1024, P(64), None) == kvq.KVQ_ERR_ARG
    assert b"16" in lib.kvq_last_error()
