"""GPU parity of the quantizers on values whose quotient x / S is a tie.

The kernels code a value from the product x * RN(1/S) and fall back to the
correctly rounded quotient RN(x / S) when the product lies close to a
half-integer.  Random data rarely reaches the cases where the two roundings
really differ, so these inputs are built for it: for seeded group ranges
[a, b] every fp16 value x in the range is scanned and those with
rint(x * RN(1/S)) != rint(RN(x / S)) in fp32 are kept (they sit on or next to
a half-integer quotient, where ties to even decide).  Key groups (per channel
over G tokens) and value groups (per token over G channels) are filled with
a, b and those values; the cache bytes after a prefill must equal the
oracle's bit for bit, for both metadata formats."""
import numpy as np
import pytest
import torch

import decode_attention_token_amd as kvq
import oracle
from gpu_helpers import compare_all_buffers, compare_innerq_buffers, host, make_cache

pytestmark = pytest.mark.gpu

_ALL_F16 = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float32)
_ALL_F16 = np.unique(np.concatenate([_ALL_F16, -_ALL_F16]))


def _round_up_fp16(s):
    h = np.float16(s)
    if np.float32(h) < s:
        h = np.nextafter(h, np.float16(np.inf))
    return np.float32(h)


def _tie_pairs(bits, meta16, seed, want=48, trials=20000):
    """[(a, b, xs)] with xs the fp16 values in [a, b] whose fast and correctly
    rounded quotients round to different integers."""
    rng = np.random.default_rng(seed)
    qmax = np.float32(2 ** bits - 1)
    out = []
    for _ in range(trials):
        scale = np.float32(rng.choice([0.01, 1.0, 30.0]))
        a, b = np.sort(np.float16(rng.normal(size=2) * scale).astype(np.float32))
        if not a < b:
            continue
        s = np.float32(np.float32(b - a) / qmax)
        if meta16:
            s = _round_up_fp16(s)
        r = np.float32(np.float32(1.0) / s)
        x = _ALL_F16[np.searchsorted(_ALL_F16, a):np.searchsorted(_ALL_F16, b, side="right")]
        xs = x[np.rint(x / s) != np.rint(x * r)]
        if len(xs):
            out.append((a, b, xs))
            if len(out) == want:
                break
    return out


def _fill(pairs, n_groups, G):
    """n_groups groups of G fp16 values: a, b, then the pair's tie values cycled."""
    g = np.empty((n_groups, G), np.float32)
    for i in range(n_groups):
        a, b, xs = pairs[i % len(pairs)]
        g[i, 0], g[i, 1] = a, b
        g[i, 2:] = xs[np.arange(G - 2) % len(xs)]
    return g.astype(np.float16)


@pytest.mark.parametrize("bits,G,meta", [(2, 32, kvq.KVQ_META_F32), (4, 64, kvq.KVQ_META_F32),
                                         (4, 32, kvq.KVQ_META_F16), (2, 128, kvq.KVQ_META_F16)])
def test_quantizer_ties_bit_exact(bits, G, meta):
    print(f"case bits={bits} G={G} meta={meta}", flush=True)
    meta16 = meta == kvq.KVQ_META_F16
    pairs = _tie_pairs(bits, meta16, seed=7000 + 10 * bits + G + meta)
    assert len(pairs) >= 8, "no tie inputs found"
    R, L, B, H, d = 128, 300, 2, 2, 128
    rng = np.random.default_rng(11)
    # keys: group (unit, token group, channel) runs over G tokens
    kg = _fill(pairs, B * H * (L // G + 1) * d, G)
    rng.shuffle(kg)
    k = kg.reshape(B, H, L // G + 1, d, G).transpose(0, 1, 2, 4, 3).reshape(B, H, -1, d)[:, :, :L]
    # values: group (unit, token, channel group) runs over G channels
    vg = _fill(pairs, B * H * L * (d // G), G)
    rng.shuffle(vg)
    v = vg.reshape(B, H, L, d)
    k, v = np.ascontiguousarray(k), np.ascontiguousarray(v)

    cfg, cache = make_cache(bits, G, R, B, H, H, 512, kvq.KVQ_V_FIFO, meta=meta)
    ref = oracle.QuantizedKVCache(bits, G, R, B, H, d, oracle.FIFO, oracle.META_F16 if meta16 else oracle.META_F32)
    cache.prefill(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda())
    ref.prefill(k, v)
    torch.cuda.synchronize()
    assert ref.nq_k > 0 and ref.nq_v > 0
    compare_all_buffers(cache, ref)
    # one appended token moves one value row out of the FIFO into the codes
    kn = torch.from_numpy(k[:, :, :1].reshape(B, H, d).copy()).cuda()
    vn = torch.from_numpy(v[:, :, -1].copy()).cuda()
    cache.append(kn, vn)
    ref.append(host(kn), host(vn))
    torch.cuda.synchronize()
    compare_all_buffers(cache, ref)


def _sym_tie_groups(bits, seed, want=48, trials=20000):
    """[(amax, xs)] with xs in (0, amax] whose fast and correctly rounded
    quotients by S = amax / (2^(b-1) - 1) round to different integers."""
    rng = np.random.default_rng(seed)
    qm = np.float32(2 ** (bits - 1) - 1)
    out = []
    for _ in range(trials):
        amax = np.float32(np.float16(abs(rng.normal()) * rng.choice([0.01, 1.0, 30.0])))
        if not amax > 0:
            continue
        s = np.float32(amax / qm)
        r = np.float32(np.float32(1.0) / s)
        x = _ALL_F16[np.searchsorted(_ALL_F16, 0, side="right"):np.searchsorted(_ALL_F16, amax, side="right")]
        xs = x[np.rint(x / s) != np.rint(x * r)]
        if len(xs):
            out.append((amax, xs))
            if len(out) == want:
                break
    return out


@pytest.mark.parametrize("bits,G", [(2, 32), (4, 64), (4, 128)])
def test_innerq_quantizer_ties_bit_exact(bits, G):
    """Per-token groups of the InnerQ-style cache: zero-centred groups
    (amax, -amax and +-x pairs: mean exactly 0, so symmetric) and offset
    groups (a, b and tie values), for keys and values."""
    print(f"case innerq bits={bits} G={G}", flush=True)
    sym = _sym_tie_groups(bits, seed=8000 + 10 * bits + G)
    asym = _tie_pairs(bits, False, seed=8500 + 10 * bits + G)
    # with 2 bits S = max|x| and the quotients stay within [-1, 1], where the
    # two roundings agree: zero-centred groups of random values stand in
    assert (len(sym) >= 8 or bits == 2) and len(asym) >= 8, "no tie inputs found"
    if not sym:
        rng0 = np.random.default_rng(8000 + G)
        sym = [(np.float32(1.0), np.abs(np.float16(rng0.normal(size=64) * 0.4)).astype(np.float32).clip(0, 1))]
    B, H, d, L, R, S = 2, 2, 128, 200, 16, 4
    n = B * H * L * (d // G)
    groups = np.empty((n, G), np.float32)
    for i in range(n):
        if i % 2 == 0:
            amax, xs = sym[(i // 2) % len(sym)]
            half = xs[np.arange(G // 2 - 1) % len(xs)]
            groups[i] = np.concatenate([[amax], half, [-amax], -half])
        else:
            a, b, xs = asym[(i // 2) % len(asym)]
            groups[i, 0], groups[i, 1] = a, b
            groups[i, 2:] = xs[np.arange(G - 2) % len(xs)]
    rng = np.random.default_rng(13)
    kg = groups.astype(np.float16)
    rng.shuffle(kg)
    vg = groups.astype(np.float16)[::-1].copy()
    k = np.ascontiguousarray(kg.reshape(B, H, L, d))
    v = np.ascontiguousarray(vg.reshape(B, H, L, d))
    ref = oracle.InnerQCache(bits, G, R, S, B, H, d)
    assert oracle.hybrid_is_symmetric(kg[:64]).any() and not oracle.hybrid_is_symmetric(kg[:64]).all()
    cfg = kvq.make_innerq_config(bits, G, R, S, B, H, H, d, 256)
    cache = kvq.KVCache(cfg, "cuda")
    cache.prefill(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda())
    ref.prefill(k, v)
    torch.cuda.synchronize()
    assert ref.nq > S
    compare_innerq_buffers(cache, ref)
