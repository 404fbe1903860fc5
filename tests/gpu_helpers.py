"""Shared helpers of the GPU parity tests: run the HIP path and the oracle on the
same seeded fp16 bits and compare buffers (bit-exact) and outputs (2e-3)."""
import numpy as np
import torch

import decode_attention_token_amd as kvq
import oracle

ATOL = 2e-3   # attention max-abs bound versus the float64 oracle


def gpu_available():
    return torch.cuda.is_available()


def host(t):
    return t.detach().cpu().numpy()


def make_cache(bits, G, R, B, Hq, Hkv, cap, policy=kvq.KVQ_V_CHUNK, d=128):
    cfg = kvq.make_config(bits, G, R, B, Hq, Hkv, d, cap, policy)
    return cfg, kvq.KVCache(cfg, "cuda")


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
        got = host(T[name][b, h][sl])
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


def compare_all_buffers(cache, ref):
    for b in range(ref.B):
        for h in range(ref.H):
            compare_unit_buffers(cache, ref, b, h)


def oracle_attention(ref, q_np, scale):
    K, V = ref.dequantized()
    return oracle.attention(q_np, K, V, scale)


def max_err(out, want):
    return float(np.abs(host(out).astype(np.float64) - want).max())
