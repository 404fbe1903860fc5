"""Shared helpers of the GPU parity tests: run the HIP path and the oracle on the
same seeded fp16 bits and compare buffers (bit-exact) and outputs (2e-3)."""
import contextlib

import numpy as np
import torch

import decode_attention_token_amd as kvq
import oracle

ATOL = 2e-3   # attention max-abs bound versus the float64 oracle
# Bound on the difference between split counts of one call.  fp32 paths only
# reorder fp32 sums (1e-5).  The matrix-core path for four query heads per kv
# head rounds its real operands to two bf16 limbs (about 17 bits) relative to
# each part's running maximum, so differently split calls round differently:
# up to 2^-17 of a weight times |score| up to ~30 (log2 units, outlier channels)
# moves an output by a few 1e-5; 1e-4 leaves margin and is still 20x below ATOL.
SPLIT_TOL = 1e-5
SPLIT_TOL_MFMA = 1e-4


@contextlib.contextmanager
def config_fields(cache, **fields):
    """Sets launch-choice fields of the cache's own kvq_config (schedule,
    kernel) for the calls inside, then restores them."""
    old = {k: getattr(cache.cfg, k) for k in fields}
    for k, v in fields.items():
        setattr(cache.cfg, k, v)
    try:
        yield
    finally:
        for k, v in old.items():
            setattr(cache.cfg, k, v)


def queue_schedule(cache):
    """The matrix-core kernel's work-queue schedule for the calls inside
    (the default is the fixed order with bit-identical reruns)."""
    return config_fields(cache, schedule=kvq.KVQ_SCHED_QUEUE)


def split_tol(heads_per_kv):
    return SPLIT_TOL_MFMA if heads_per_kv == 4 else SPLIT_TOL


def gpu_available():
    return torch.cuda.is_available()


def host(t):
    return t.detach().cpu().numpy()


def make_cache(bits, G, R, B, Hq, Hkv, cap, policy=kvq.KVQ_V_CHUNK, d=128, sinks=0, meta=kvq.KVQ_META_F32):
    cfg = kvq.make_config(bits, G, R, B, Hq, Hkv, d, cap, policy, kvq.KVQ_SCHEME_KIVI, sinks, meta)
    return cfg, kvq.KVCache(cfg, "cuda")


def make_innerq_cache(bits, G, R, S, B, Hq, Hkv, cap, d=128, key_norm=kvq.KVQ_KEYNORM_NONE):
    cfg = kvq.make_innerq_config(bits, G, R, S, B, Hq, Hkv, d, cap, key_norm)
    return cfg, kvq.KVCache(cfg, "cuda")


def _bits(x):
    """Host array with integer words viewed unsigned (packed metadata words are
    held in int32 tensors on the GPU and as uint32 in the oracle)."""
    return x.view(np.uint32) if x.dtype == np.int32 else x


def compare_innerq_unit(cache, ref, b, h, rb=None, rh=None):
    """Bit-exact comparison of one unit's live bytes of an InnerQ-style cache:
    quantized rows [sinks, nq), the sink rows present and the window slots."""
    rb = b if rb is None else rb
    rh = h if rh is None else rh
    bufs = ref.buffers(cache.cfg.max_tokens)
    assert (cache.n_tokens, cache.nq_k, cache.nq_v) == (ref.n, ref.nq, ref.nq)
    T = cache.tensors
    rows = np.s_[ref.S:ref.nq] if ref.n > ref.S else np.s_[0:0]
    for name in ("k_codes", "k_scale", "k_zero", "v_codes", "v_scale", "v_zero"):
        got = host(T[name][b, h][rows])
        if name.endswith("codes"):
            got = got.view(np.uint32)
        want = bufs[name][rb, rh][rows]
        if not np.array_equal(got, want):
            bad = np.argwhere(got != want)
            raise AssertionError(f"{name} unit ({b},{h}) differs at {bad[:5].tolist()} ({len(bad)} entries)")
    ns = min(ref.n, ref.S)
    for name in ("k_sink", "v_sink"):
        got = host(T[name][b, h][:ns]).view(np.uint16)
        assert np.array_equal(got, bufs[name][rb, rh][:ns].view(np.uint16)), name
    slots, _ = ref.live_resid_slots()
    for name in ("k_resid", "v_resid"):
        if slots:
            got = host(T[name][b, h][slots]).view(np.uint16)
            assert np.array_equal(got, bufs[name][rb, rh][slots].view(np.uint16)), name
    if "k_norm" in bufs:
        got = host(T["k_norm"][b, h])
        assert np.array_equal(got, bufs["k_norm"][rb, rh]), f"k_norm unit ({b},{h}): {got} vs {bufs['k_norm'][rb, rh]}"


def compare_innerq_buffers(cache, ref):
    for b in range(ref.B):
        for h in range(ref.H):
            compare_innerq_unit(cache, ref, b, h)


def compare_unit_buffers(cache, ref, b, h, rb=None, rh=None):
    """Bit-exact comparison of one unit's live cache bytes.

    (b, h) index the GPU cache; (rb, rh) the oracle cache (defaults: same)."""
    rb = b if rb is None else rb
    rh = h if rh is None else rh
    G = ref.G
    bufs = ref.buffers(cache.cfg.max_tokens)
    nq_k, nq_v = ref.nq_k, ref.nq_v
    assert (cache.n_tokens, cache.nq_k, cache.nq_v) == (ref.n, nq_k, nq_v)
    T = cache.tensors
    pairs = [
        ("k_codes", np.s_[:nq_k], lambda x: x.view(np.uint32)),
        ("k_scale", np.s_[:nq_k // G], None),
        ("k_zero", np.s_[:nq_k // G], None),
        ("v_codes", np.s_[:nq_v], lambda x: x.view(np.uint32)),
        ("v_scale", np.s_[:nq_v], None),
        ("v_zero", np.s_[:nq_v], None),
    ]
    for name, sl, conv in pairs:
        got = _bits(host(T[name][b, h][sl]))
        if conv:
            got = conv(got)
        want = bufs[name][rb, rh][sl]
        if not np.array_equal(got, want):
            bad = np.argwhere(got != want)
            raise AssertionError(f"{name} unit ({b},{h}) differs at {bad[:5].tolist()} "
                                 f"({len(bad)} entries)")
    ks, vs = ref.live_resid_slots()
    for name, slots in (("k_resid", ks), ("v_resid", vs)):
        if slots:
            got = host(T[name][b, h][slots])
            want = bufs[name][rb, rh][slots]
            assert np.array_equal(got.view(np.uint16), want.view(np.uint16)), name


def compare_sink_unit(cache, ref, b, h):
    """Bit-exact comparison of one unit of a KIVI cache with sink tokens
    (oracle.KiviSinkCache): the inner rows and ring slots, and the sink rows."""
    inner = ref.inner
    bufs = ref.buffers(cache.cfg.max_tokens)
    assert (cache.n_tokens, cache.nq_k, cache.nq_v) == (ref.n, ref.nq_k, ref.nq_v)
    T = cache.tensors
    G = ref.G
    for name, sl in (("k_codes", np.s_[:inner.nq_k]), ("k_scale", np.s_[:inner.nq_k // G]),
                     ("k_zero", np.s_[:inner.nq_k // G]), ("v_codes", np.s_[:inner.nq_v]),
                     ("v_scale", np.s_[:inner.nq_v]), ("v_zero", np.s_[:inner.nq_v])):
        got = _bits(host(T[name][b, h][sl]))
        if name.endswith("codes"):
            got = got.view(np.uint32)
        assert np.array_equal(got, bufs[name][b, h][sl]), name
    ns = min(ref.n, ref.S)
    for name in ("k_sink", "v_sink"):
        assert np.array_equal(host(T[name][b, h][:ns]).view(np.uint16), bufs[name][b, h][:ns].view(np.uint16)), name
    ks, vs = ref.live_resid_slots()
    for name, slots in (("k_resid", ks), ("v_resid", vs)):
        if slots:
            got = host(T[name][b, h][slots]).view(np.uint16)
            assert np.array_equal(got, bufs[name][b, h][slots].view(np.uint16)), name


def compare_all_buffers(cache, ref):
    for b in range(ref.B):
        for h in range(ref.H):
            compare_unit_buffers(cache, ref, b, h)


def oracle_attention(ref, q_np, scale):
    K, V = ref.dequantized()
    return oracle.attention(q_np, K, V, scale)


def max_err(out, want):
    return float(np.abs(host(out).astype(np.float64) - want).max())
