"""GPU parity of the quantizers on the groups where an affine quantizer is
most easily wrong: constant groups (S = |min|, codes 0), all-zero groups
(S = 1), +0 / -0 mixes, two-value groups one fp16 step apart just above a
negative power of two (|Z| reaches (2^b - 1) * 2^11: 6144 for 2 bits, 30720
for 4 bits, the int16 worst case), the fp16 extremes +-65504, subnormals,
exact .5 ties of x / S, and a lone outlier.  The patterns are planted in
key groups (G tokens of one channel) and value groups (G channels of one
token), then run through every GPU path that quantizes: prefill, the chunked
flush append, the FIFO value pop with its key flush, both metadata formats,
and the InnerQ-style prefill and window pop, each through kvq_append_token
and through kvq_decode_step (whose attention launch quantizes the next
leaving FIFO value or window token ahead; for KIVI values with a one-wave
routine of its own).
Every cache byte must match the oracle bit for bit.
"""
import numpy as np
import pytest
import torch

import decode_attention_token_amd as kvq
import oracle
from gpu_helpers import compare_innerq_buffers, compare_all_buffers

pytestmark = pytest.mark.gpu

D = 128
F16 = np.float16


def _patterns(G, bits, rng):
    """Edge-case groups of G fp16 values (each a numpy array)."""
    L = (1 << bits) - 1

    def mix(a, b):
        x = rng.choice(np.array([a, b], F16), size=G)
        x[0], x[1] = F16(a), F16(b)          # both values present
        return x

    ties_pos = np.concatenate([[0.0, float(L)], np.arange(L) + 0.5])          # S = 1, x/S at .5
    ties_neg = -ties_pos
    pats = [
        np.full(G, 1.5, F16),
        np.full(G, -3.0, F16),
        np.full(G, 65504.0, F16),
        np.full(G, -65504.0, F16),
        np.zeros(G, F16),
        np.where(np.arange(G) % 2 == 0, F16(0.0), F16(-0.0)).astype(F16),
        mix(-2048.0, -2047.0),                  # |Z| = L * 2048
        mix(-0.5, -0.5 + 2.0 ** -12),           # the same one binade lower
        mix(-65504.0, 65504.0),
        rng.choice(np.array([0.0, 2.0 ** -24, 3 * 2.0 ** -24, -(2.0 ** -23)], F16), size=G),
        np.resize(ties_pos, G).astype(F16),
        np.resize(ties_neg, G).astype(F16),
        np.where(np.arange(G) == G // 3, F16(60000.0), F16(0.0)).astype(F16),
        rng.standard_normal(G).astype(F16),
    ]
    for p in pats:
        assert p.shape == (G,) and p.dtype == F16
    return pats


def _planted(bits, G, H, T, seed, keys_per_channel):
    """fp16 [1][H][T][128]: keys_per_channel plants a pattern in every group of
    G tokens of one channel (KIVI keys); otherwise in every group of G
    channels of one token (KIVI values, InnerQ keys and values)."""
    rng = np.random.default_rng(seed)
    pats = _patterns(G, bits, rng)
    x = np.zeros((1, H, T, D), F16)
    for h in range(H):
        if keys_per_channel:
            for g in range(T // G):
                for c in range(D):
                    x[0, h, g * G:(g + 1) * G, c] = pats[(7 * g + 3 * c + h) % len(pats)]
            rest = T - (T // G) * G
            if rest:
                x[0, h, T - rest:] = rng.standard_normal((rest, D)).astype(F16)
        else:
            for t in range(T):
                for j in range(D // G):
                    x[0, h, t, j * G:(j + 1) * G] = pats[(5 * t + 3 * j + h) % len(pats)]
    return x


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


KIVI_CASES = [(bits, G, policy, meta) for bits, G in ((2, 32), (4, 64)) for policy in (0, 1) for meta in (0, 1)]


def _push(cache, k, v, via):
    if via == "append":
        cache.append(k, v)
    else:
        H = cache.cfg.num_q_heads
        q = torch.ones(1, H, D, dtype=torch.float16, device="cuda")
        cache.step(k, v, q)


@pytest.mark.parametrize("via", ["append", "step"])
@pytest.mark.parametrize("bits,G,policy,meta", KIVI_CASES)
def test_kivi_quantizer_edge_groups(bits, G, policy, meta, via):
    H, R, L, A = 2, 64, 256, 2 * 64 + 3
    print(f"case KIVI bits={bits} G={G} policy={policy} meta={meta} via {via}", flush=True)
    T = L + A
    K = _planted(bits, G, H, T + G, 100 + bits, True)[:, :, :T]
    V = _planted(bits, G, H, T, 200 + bits, False)
    cap = ((T + R - 1) // R + 1) * R
    cfg = kvq.make_config(bits, G, R, 1, H, H, D, cap, policy, kvq.KVQ_SCHEME_KIVI, 0, meta)
    cache = kvq.KVCache(cfg, "cuda")
    ref = oracle.QuantizedKVCache(bits, G, R, 1, H, D, policy, meta)
    cache.prefill(_dev(K[:, :, :L]), _dev(V[:, :, :L]))
    ref.prefill(K[:, :, :L], V[:, :, :L])
    torch.cuda.synchronize()
    compare_all_buffers(cache, ref)
    for i in range(L, T):
        f0 = ref.flushes
        _push(cache, _dev(K[:, :, i]), _dev(V[:, :, i]), via)
        ref.append(K[:, :, i], V[:, :, i])
        if ref.flushes != f0 or policy == 1 or i == T - 1:
            torch.cuda.synchronize()
            compare_all_buffers(cache, ref)
    zmax = max(int(np.abs(ref.kq_zero).max()), int(np.abs(ref.vq_zero).max()))
    worst = ((1 << bits) - 1) * 2048
    # packed metadata rounds S up to fp16 first, which shrinks |Z| slightly
    assert zmax == worst if meta == 0 else worst * 0.99 < zmax <= worst, (zmax, worst)
    assert ref.flushes == 2


@pytest.mark.parametrize("via", ["append", "step"])
@pytest.mark.parametrize("key_norm", [0, 1])
@pytest.mark.parametrize("bits,G", [(4, 64), (2, 32)])
def test_innerq_quantizer_edge_groups(bits, G, key_norm, via):
    H, S, R, L, A = 2, 4, 16, 100, 40
    print(f"case InnerQ bits={bits} G={G} key_norm={key_norm} via {via}", flush=True)
    T = L + A
    K = _planted(bits, G, H, T, 300 + bits, False)
    V = _planted(bits, G, H, T, 400 + bits, False)
    cfg = kvq.make_innerq_config(bits, G, R, S, 1, H, H, D, T + 8, key_norm)
    cache = kvq.KVCache(cfg, "cuda")
    ref = oracle.InnerQCache(bits, G, R, S, 1, H, D, key_norm=bool(key_norm))
    cache.prefill(_dev(K[:, :, :L]), _dev(V[:, :, :L]))
    ref.prefill(K[:, :, :L], V[:, :, :L])
    torch.cuda.synchronize()
    compare_innerq_buffers(cache, ref)
    for i in range(L, T):
        _push(cache, _dev(K[:, :, i]), _dev(V[:, :, i]), via)
        ref.append(K[:, :, i], V[:, :, i])
        torch.cuda.synchronize()
        compare_innerq_buffers(cache, ref)
