"""Plain NumPy oracle for KIVI-style quantized-KV decode attention.

TEST INFRASTRUCTURE ONLY: used by tests/, by the smoke check and by the bench's
CPU-baseline leg; never by the library.  Shares no code with the HIP path.

Sources (web pages, cited by title and section):
  [KIVI]  juejin.cn, "大模型量化技术原理：KIVI、IntactKV、KVQuant", part KIVI,
          sections 背景 (background), 为什么键和值缓存应该沿着不同的维度进行量化
          (why K and V are quantized along different axes) and 工作原理
          (how it works: grouped part + full-precision residual, the R-token
          key flush, the value queue, prefill).
  [HFQ]   pgsm.cn news 20017, KV-cache quantization article, section 2.1
          (affine quantization X_Q = round(X/S) - Z with scale S and zero-point
          offset Z, symmetric vs asymmetric), 2.2 (keys per channel, values per
          token), 3.1 (fixed-size fp16 residual cache, batch-quantized into the
          main cache when full), 3.2 (bytes per token for Llama-2-7B), 4.1
          (knobs nbits / group_size / residual_length).

Precision: the quantizer runs in float32 on fp16 inputs (every step is one
correctly rounded IEEE float32 operation, rounding half to even); attention is
accumulated in float64 on the float32 dequantized cache.

Parity status of each function (pins live in tests/test_oracle_*.py):
  quantize_groups        pinned: on-grid exactness (recovers S, Z, codes of a
                         lattice exactly), code(min) == 0, code(max) in
                         {2^b-2, 2^b-1}, monotone codes, |x - x_hat| <= S/2 + eps,
                         nearest-level brute force, constant groups exact.
  quantize_groups(f16_scale=True)
                         pinned: S is the smallest fp16 >= the fp32 scale
                         (neighbour enumeration), on-grid lattices with fp16
                         scales recovered exactly, nearest-level brute force,
                         |x - x_hat| <= S/2, packed words decode to S and Z.
  dequantize             pinned with quantize_groups (round trip).
  pack_rows/unpack_rows  pinned: literal words from the layout definition,
                         brute-force enumeration of all codes in a word.
  QuantizedKVCache       pinned: (l - r) % G == 0 after every call, one flush
                         per R appends, prefill(L)+appends == prefill(L+m),
                         FIFO and chunked value codes agree per token, cache
                         with R > n reduces to plain fp16 attention.
  attention              pinned: torch float64 SDPA on the same operands,
                         q == 0 gives the mean of V, n == 1 gives v_0,
                         brute-force scalar loops on tiny inputs.
  byte accounting        pinned: the per-token byte table for Llama-2-7B
                         (524,288 / 262,144 / 131,072 / 65,536 bytes) and the
                         ~5 GB for 10k fp16 tokens in [HFQ] 1 and 3.2.
  hybrid_is_symmetric    pinned: agrees with |mean| < 0.1 * std computed by
                         numpy away from the threshold; zero-centred groups
                         choose symmetric, offset groups asymmetric.
  quantize_groups_symmetric / _hybrid
                         pinned: on-grid exactness (x = s*k recovers S = s and
                         the signed codes), |x - x_hat| <= S/2, asymmetric
                         groups equal quantize_groups.
  KiviSinkCache          pinned: sinks stay exact fp16, the tokens after them
                         match a plain cache fed the same stream, prefill(L)
                         + appends == prefill(L+m) across the sink boundary,
                         all-fp16 reduces to plain attention.
  InnerQCache            pinned: sinks stay exact fp16, window holds
                         min(R, n - sinks) tokens, prefill(L)+appends ==
                         prefill(L+m), all-fp16 cache reduces to plain
                         attention.
  key_channel_normalizer / normalize_keys / InnerQCache(key_norm=True)
                         pinned: scales are the smallest powers of two >=
                         max(1, max-abs) (brute-force scan of powers of two),
                         prompt keys land in [-1, 1], scales never change on
                         append, keys all within [-1, 1] give the plain cache
                         byte for byte, a common power-of-two scale leaves
                         codes and attention bit-identical to the plain cache,
                         the fold-into-query form equals dequantize-then-scale,
                         |k - k_hat| <= lambda * S / 2.

Sources for the InnerQ-style variant:
  [InnerQ] euno.news, "【论文】InnerQ：硬件感知免调优KV缓存量化用于大语言模型",
           methodology 1 (groups along the inner / hidden dimension), 2 (per
           group statistics min, max, mean, variance; symmetric quantization
           when the group is centred on zero, asymmetric otherwise, one
           shared scale per group), 4 (recent and attention-sink tokens kept
           in fp16; keys scaled once per channel at prefill, the scale folded
           into the query).
  [HFQ] 2.1 defines symmetric quantization as a range symmetric about zero.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "quantize_groups", "dequantize", "pack_rows", "unpack_rows", "QuantizedKVCache",
    "attention", "kv_code_bytes_per_token", "attention_call_bytes",
    "CHUNK", "FIFO", "META_F32", "META_F16", "round_up_to_fp16", "hybrid_is_symmetric", "quantize_groups_symmetric", "quantize_groups_hybrid",
    "InnerQCache", "innerq_attention_call_bytes", "KiviSinkCache", "key_channel_normalizer", "normalize_keys",
]

CHUNK = 0   # value residual flushed as a block of R tokens, like the keys ([HFQ] 3.1)
FIFO = 1    # value residual kept as a queue of the R most recent tokens ([KIVI] 工作原理)

META_F32 = 0   # group metadata: fp32 scale + int16 zero-point (6 bytes)
META_F16 = 1   # group metadata: fp16 scale rounded up + int16 zero-point in one 32-bit word

_F32 = np.float32


# --------------------------------------------------------------------------- quantizer
def round_up_to_fp16(s):
    """Smallest fp16 value >= s, returned as float32 (s positive float32)."""
    s = np.asarray(s, _F32)
    h = s.astype(np.float16)                       # round to nearest even
    low = h.astype(_F32) < s
    h = np.where(low, np.nextafter(h, np.float16(np.inf)), h)
    return h.astype(_F32)


def quantize_groups(x, bits: int, f16_scale: bool = False):
    """Asymmetric affine quantization of each group along the last axis.

    [HFQ] 2.1 writes the quantizer as X_Q = round(X / S) - Z with scale S and
    zero-point offset Z; the asymmetric form maps each group's own [min, max]
    range onto the 2^b integer levels ([KIVI] 背景: 2-bit asymmetric).

      S      = (max - min) / (2^b - 1)       (float32, one rounding each)
               a constant group (max == min) takes S = |min|, or 1 when min == 0,
               so it reconstructs exactly
      Z      = rint(min / S)                 (integer, stored as int16)
      code_i = clamp(rint(x_i / S) - Z, 0, 2^b - 1)

    With f16_scale (compressed metadata) S is replaced by the smallest fp16
    value >= S before Z and the codes are computed, so it stores exactly in
    fp16 and the group's range still fits the 2^b levels.

    x: float16 array, groups along the last axis.
    Returns (codes uint8 same shape, S float32 [...], Z int16 [...]).
    """
    if bits not in (2, 4, 8):
        raise ValueError("bits must be 2, 4 or 8")
    xf = np.asarray(x, dtype=np.float16).astype(_F32)
    qmax = _F32((1 << bits) - 1)
    mn = xf.min(axis=-1)
    mx = xf.max(axis=-1)
    span = (mx - mn).astype(_F32)
    with np.errstate(divide="ignore", invalid="ignore"):
        s_range = (span / qmax).astype(_F32)
    s_const = np.where(mn != 0, np.abs(mn), _F32(1.0)).astype(_F32)
    scale = np.where(mx > mn, s_range, s_const).astype(_F32)
    if f16_scale:
        scale = round_up_to_fp16(scale)
    zero = np.rint((mn / scale).astype(_F32)).astype(_F32)
    q = np.rint((xf / scale[..., None]).astype(_F32)).astype(_F32) - zero[..., None]
    codes = np.clip(q, _F32(0), qmax).astype(np.uint8)
    if np.any(np.abs(zero) > 32767):
        raise OverflowError("zero-point does not fit int16")
    return codes, scale, zero.astype(np.int16)


def dequantize(codes, scale, zero):
    """x_hat = S * (code + Z), float32: the inverse of the [HFQ] 2.1 map.

    codes [..., G]; scale and zero broadcast over the last axis.
    """
    c = np.asarray(codes).astype(_F32)
    z = np.asarray(zero).astype(_F32)[..., None]
    s = np.asarray(scale, dtype=_F32)[..., None]
    return ((c + z) * s).astype(_F32)


# --------------------------------------------------------------------------- packing
def pack_rows(codes, bits: int):
    """Pack the d codes of each token row into d*bits/32 little-endian words.

    Channel c of a row sits at bits [(c*bits) % 32, +bits) of word (c*bits)//32.
    codes uint8 [..., d]  ->  uint32 [..., d*bits//32].
    """
    codes = np.asarray(codes, dtype=np.uint32)
    per = 32 // bits
    d = codes.shape[-1]
    assert d % per == 0
    grouped = codes.reshape(codes.shape[:-1] + (d // per, per))
    shifts = (np.arange(per, dtype=np.uint32) * np.uint32(bits))
    return np.bitwise_or.reduce(grouped << shifts, axis=-1).astype(np.uint32)


def unpack_rows(words, bits: int, d: int):
    """Inverse of :func:`pack_rows`."""
    words = np.asarray(words, dtype=np.uint32)
    per = 32 // bits
    shifts = (np.arange(per, dtype=np.uint32) * np.uint32(bits))
    mask = np.uint32((1 << bits) - 1)
    out = (words[..., None] >> shifts) & mask
    return out.reshape(words.shape[:-1] + (d,)).astype(np.uint8)


# --------------------------------------------------------------------------- cache
class QuantizedKVCache:
    """One layer's KV cache for every (batch, kv-head) unit; all units share n.

    Keys ([KIVI] 工作原理): the token axis is split into a grouped part
    X_Kg = X_K[:l-r], kept only as per-channel group quantizations over G
    tokens, and a full-precision remainder X_Kr = X_K[l-r:], with l - r
    divisible by G.  A new key joins X_Kr; when X_Kr holds R tokens it is
    quantized, appended to the grouped part and emptied (R % G == 0).

    Values: quantized per token over groups of G channels ([HFQ] 2.2).  The
    chunked policy treats the value residual exactly like the key residual,
    which is the fixed-size fp16 residual cache of [HFQ] 3.1.  The FIFO policy
    follows the queue of [KIVI] 工作原理: a new value is pushed and, once the
    queue would exceed R entries, the oldest one is popped, quantized and
    appended.

    Prefill ([KIVI] 工作原理, prefill paragraph) stores only the quantized part
    plus the residual; it never changes the fp16 inputs.
    """

    def __init__(self, bits, group, residual, batch, kv_heads, head_dim, v_policy=CHUNK, meta=META_F32):
        if bits not in (2, 4):
            raise ValueError("bits must be 2 or 4")
        if meta not in (META_F32, META_F16):
            raise ValueError("unknown metadata format")
        self.meta = meta
        if residual <= 0 or residual % group:
            raise ValueError("R must be a positive multiple of G")
        if head_dim % group:
            raise ValueError("head_dim must be a multiple of G")
        self.bits, self.G, self.R = bits, group, residual
        self.B, self.H, self.d = batch, kv_heads, head_dim
        self.v_policy = v_policy
        B, H, d, G = batch, kv_heads, head_dim, group
        self.kq_codes = np.zeros((B, H, 0, d), np.uint8)
        self.kq_scale = np.zeros((B, H, 0, d), _F32)   # [.., group, channel]
        self.kq_zero = np.zeros((B, H, 0, d), np.int16)
        self.kr = np.zeros((B, H, 0, d), np.float16)    # X_Kr, token order
        self.vq_codes = np.zeros((B, H, 0, d), np.uint8)
        self.vq_scale = np.zeros((B, H, 0, d // G), _F32)  # [.., token, channel group]
        self.vq_zero = np.zeros((B, H, 0, d // G), np.int16)
        self.vr = np.zeros((B, H, 0, d), np.float16)    # value residual / queue
        self.n = 0
        self.flushes = 0
        self.started = False

    # counters -----------------------------------------------------------------
    @property
    def nq_k(self):
        return self.kq_codes.shape[2]

    @property
    def nq_v(self):
        return self.vq_codes.shape[2]

    # quantization of token blocks ----------------------------------------------
    def _quantize_keys(self, k):
        """k fp16 [B,H,m,d], m % G == 0 -> per-channel groups of G tokens."""
        B, H, m, d = k.shape
        G = self.G
        assert m % G == 0
        grp = k.reshape(B, H, m // G, G, d).transpose(0, 1, 2, 4, 3)   # [.., g, c, t]
        codes, s, z = quantize_groups(grp, self.bits, self.meta == META_F16)
        codes = codes.transpose(0, 1, 2, 4, 3).reshape(B, H, m, d)
        return codes, s, z                                            # s,z [.., g, c]

    def _quantize_values(self, v):
        """v fp16 [B,H,m,d] -> per-token groups of G channels."""
        B, H, m, d = v.shape
        G = self.G
        grp = v.reshape(B, H, m, d // G, G)
        codes, s, z = quantize_groups(grp, self.bits, self.meta == META_F16)
        return codes.reshape(B, H, m, d), s, z                        # s,z [.., t, j]

    def _append_keys(self, k):
        c, s, z = self._quantize_keys(k)
        self.kq_codes = np.concatenate([self.kq_codes, c], axis=2)
        self.kq_scale = np.concatenate([self.kq_scale, s], axis=2)
        self.kq_zero = np.concatenate([self.kq_zero, z], axis=2)

    def _append_values(self, v):
        c, s, z = self._quantize_values(v)
        self.vq_codes = np.concatenate([self.vq_codes, c], axis=2)
        self.vq_scale = np.concatenate([self.vq_scale, s], axis=2)
        self.vq_zero = np.concatenate([self.vq_zero, z], axis=2)

    # public state transitions --------------------------------------------------
    def prefill(self, k, v):
        """k, v fp16 [B,H,L,d]; only allowed on an empty cache."""
        if self.started:
            raise RuntimeError("prefill on a non-empty cache")
        k = np.asarray(k, np.float16)
        v = np.asarray(v, np.float16)
        L = k.shape[2]
        r = L % self.R                      # residual count; l - r divisible by R (hence G)
        nq = L - r
        self._append_keys(k[:, :, :nq])
        self.kr = k[:, :, nq:].copy()
        if self.v_policy == CHUNK:
            nv = nq
        else:
            nv = max(0, L - self.R)         # the queue keeps the R most recent values
        self._append_values(v[:, :, :nv])
        self.vr = v[:, :, nv:].copy()
        self.n = L
        self.started = True

    def append(self, k_new, v_new):
        """k_new, v_new fp16 [B,H,d]: one decode step's new key and value."""
        if not self.started:
            raise RuntimeError("append before prefill")
        k_new = np.asarray(k_new, np.float16)[:, :, None, :]
        v_new = np.asarray(v_new, np.float16)[:, :, None, :]
        self.kr = np.concatenate([self.kr, k_new], axis=2)
        flushed = False
        if self.kr.shape[2] == self.R:      # X_Kr reached R: quantize, append, reset
            self._append_keys(self.kr)
            self.kr = self.kr[:, :, :0]
            flushed = True
        self.vr = np.concatenate([self.vr, v_new], axis=2)
        if self.v_policy == CHUNK:
            if self.vr.shape[2] == self.R:
                self._append_values(self.vr)
                self.vr = self.vr[:, :, :0]
        else:
            if self.vr.shape[2] > self.R:   # pop the oldest value and quantize it
                self._append_values(self.vr[:, :, :1])
                self.vr = self.vr[:, :, 1:]
        self.flushes += int(flushed)
        self.n += 1

    # views ------------------------------------------------------------------------
    def dequantized(self):
        """(K_hat, V_hat) float32 [B,H,n,d] in token order."""
        B, H, d, G = self.B, self.H, self.d, self.G
        nqk, nqv = self.nq_k, self.nq_v
        kc = self.kq_codes.reshape(B, H, nqk // G, G, d).transpose(0, 1, 2, 4, 3)
        kh = dequantize(kc, self.kq_scale, self.kq_zero)                  # [.., g, c, t]
        kh = kh.transpose(0, 1, 2, 4, 3).reshape(B, H, nqk, d)
        vc = self.vq_codes.reshape(B, H, nqv, d // G, G)
        vh = dequantize(vc, self.vq_scale, self.vq_zero).reshape(B, H, nqv, d)
        K = np.concatenate([kh, self.kr.astype(_F32)], axis=2)
        V = np.concatenate([vh, self.vr.astype(_F32)], axis=2)
        return K, V

    def buffers(self, max_tokens):
        """The cache serialized in the library's device layout.

        k_codes u32 [B,H,cap,d*b/32]   token rows of packed per-channel codes
        k_scale f32 [B,H,cap/G,d]      one scale per (token group, channel)
        k_zero  i16 [B,H,cap/G,d]
        v_codes u32 [B,H,cap,d*b/32]
        v_scale f32 [B,H,cap,d/G]      one scale per (token, channel group)
        v_zero  i16 [B,H,cap,d/G]
        k_resid, v_resid f16 [B,H,R,d] token t at slot t mod R (live slots only;
                                       the others hold whatever was there)
        With META_F16, k_scale / v_scale hold u32 words (fp16 S | Z << 16) of
        the same shapes and k_zero / v_zero are empty.
        """
        B, H, d, G, R, b = self.B, self.H, self.d, self.G, self.R, self.bits
        cap = max_tokens
        W = d * b // 32
        out = {
            "k_codes": np.zeros((B, H, cap, W), np.uint32),
            "k_scale": np.zeros((B, H, cap // G, d), _F32),
            "k_zero": np.zeros((B, H, cap // G, d), np.int16),
            "v_codes": np.zeros((B, H, cap, W), np.uint32),
            "v_scale": np.zeros((B, H, cap, d // G), _F32),
            "v_zero": np.zeros((B, H, cap, d // G), np.int16),
            "k_resid": np.zeros((B, H, R, d), np.float16),
            "v_resid": np.zeros((B, H, R, d), np.float16),
        }
        nqk, nqv = self.nq_k, self.nq_v
        out["k_codes"][:, :, :nqk] = pack_rows(self.kq_codes, b)
        out["k_scale"][:, :, :nqk // G] = self.kq_scale
        out["k_zero"][:, :, :nqk // G] = self.kq_zero
        out["v_codes"][:, :, :nqv] = pack_rows(self.vq_codes, b)
        out["v_scale"][:, :, :nqv] = self.vq_scale
        out["v_zero"][:, :, :nqv] = self.vq_zero
        for i in range(self.kr.shape[2]):
            out["k_resid"][:, :, (nqk + i) % R] = self.kr[:, :, i]
        for i in range(self.vr.shape[2]):
            out["v_resid"][:, :, (nqv + i) % R] = self.vr[:, :, i]
        if self.meta == META_F16:
            # one 32-bit word per group: fp16 bits of S in the low half, Z in the high half
            for t in ("k", "v"):
                sc, zr = out[t + "_scale"], out[t + "_zero"]
                bits16 = sc.astype(np.float16).view(np.uint16).astype(np.uint32)
                out[t + "_scale"] = bits16 | (zr.view(np.uint16).astype(np.uint32) << np.uint32(16))
                out[t + "_zero"] = np.zeros(zr.shape[:2] + (0,) + zr.shape[3:], np.int16)
        return out

    def live_resid_slots(self):
        """Ring slots that hold live residual tokens: (k_slots, v_slots)."""
        R = self.R
        ks = [(self.nq_k + i) % R for i in range(self.kr.shape[2])]
        vs = [(self.nq_v + i) % R for i in range(self.vr.shape[2])]
        return ks, vs


# --------------------------------------------------------------------------- KIVI with sinks
class KiviSinkCache:
    """KIVI-style cache whose first `sinks` tokens stay fp16 for the life of
    the cache (attention-sink-aware quantization: the juejin.cn KIVI/IntactKV/
    KVQuant page, KVQuant part, section 五 -- models put large attention on
    the first tokens, so their quantization error matters most).

    The KIVI state machine of QuantizedKVCache runs unchanged on the token
    stream after the sinks: token t >= sinks is token t - sinks of the inner
    cache.  Counters are reported for the whole stream: n, and nq_k / nq_v =
    end of the quantized key / value tokens, i.e. sinks + the inner counts
    (== n while n <= sinks).
    """

    def __init__(self, bits, group, residual, sinks, batch, kv_heads, head_dim, v_policy=CHUNK, meta=META_F32):
        if sinks < 0:
            raise ValueError("sinks must be non-negative")
        self.S = sinks
        self.inner = QuantizedKVCache(bits, group, residual, batch, kv_heads, head_dim, v_policy, meta)
        self.bits, self.G, self.R = bits, group, residual
        self.B, self.H, self.d = batch, kv_heads, head_dim
        self.sink_k = np.zeros((batch, kv_heads, 0, head_dim), np.float16)
        self.sink_v = np.zeros((batch, kv_heads, 0, head_dim), np.float16)

    @property
    def n(self):
        return self.sink_k.shape[2] + self.inner.n

    @property
    def nq_k(self):
        return self.n if self.n <= self.S else self.S + self.inner.nq_k

    @property
    def nq_v(self):
        return self.n if self.n <= self.S else self.S + self.inner.nq_v

    @property
    def flushes(self):
        return self.inner.flushes

    def prefill(self, k, v):
        k = np.asarray(k, np.float16)
        v = np.asarray(v, np.float16)
        ns = min(k.shape[2], self.S)
        self.inner.prefill(k[:, :, ns:], v[:, :, ns:])
        self.sink_k, self.sink_v = k[:, :, :ns].copy(), v[:, :, :ns].copy()

    def append(self, k_new, v_new):
        if not self.inner.started:
            raise RuntimeError("append before prefill")
        if self.n < self.S:
            self.sink_k = np.concatenate([self.sink_k, np.asarray(k_new, np.float16)[:, :, None]], axis=2)
            self.sink_v = np.concatenate([self.sink_v, np.asarray(v_new, np.float16)[:, :, None]], axis=2)
        else:
            self.inner.append(k_new, v_new)

    def dequantized(self):
        K, V = self.inner.dequantized()
        return (np.concatenate([self.sink_k.astype(_F32), K], axis=2),
                np.concatenate([self.sink_v.astype(_F32), V], axis=2))

    def buffers(self, max_tokens):
        """Device layout: the inner cache's buffers (token t >= sinks at row /
        ring slot of inner token t - sinks) plus k_sink / v_sink f16
        [B,H,sinks,d] holding sink t at row t."""
        out = self.inner.buffers(max_tokens)
        ks = np.zeros((self.B, self.H, self.S, self.d), np.float16)
        vs = np.zeros_like(ks)
        ns = self.sink_k.shape[2]
        ks[:, :, :ns], vs[:, :, :ns] = self.sink_k, self.sink_v
        out["k_sink"], out["v_sink"] = ks, vs
        return out

    def live_resid_slots(self):
        return self.inner.live_resid_slots()


# --------------------------------------------------------------------------- InnerQ-style
def hybrid_is_symmetric(x):
    """Per-group mode choice: symmetric when the group is centred on zero.

    [InnerQ] methodology 2 picks symmetric quantization for zero-centred
    groups from the group statistics.  Reading: centred means
    |mean| < 0.1 * std with the population standard deviation, which is
    exactly 101 * s1^2 < n * s2 for s1 = sum x, s2 = sum x^2.  Both sums run
    in index order in float64, so any implementation taking the same steps
    makes the same choice.  x: float16 [..., n]  ->  bool [...].
    """
    xf = np.asarray(x, dtype=np.float16).astype(np.float64)
    n = xf.shape[-1]
    s1 = np.zeros(xf.shape[:-1], np.float64)
    s2 = np.zeros(xf.shape[:-1], np.float64)
    for i in range(n):
        s1 = s1 + xf[..., i]
        s2 = s2 + xf[..., i] * xf[..., i]
    return 101.0 * (s1 * s1) < float(n) * s2


def quantize_groups_symmetric(x, bits: int):
    """Symmetric quantization about zero ([HFQ] 2.1): S = max|x| / (2^(b-1) - 1),
    signed code k = clamp(rint(x / S), -(2^(b-1) - 1), 2^(b-1) - 1).

    Storage: the code is kept offset-binary, u = k + 2^(b-1), and the group's
    zero-point is recorded as Z = -2^(b-1), so S * (u + Z) = S * k and the
    same dequantization serves both modes.  An all-zero group takes S = 1.
    Returns (u uint8, S float32, Z int16).
    """
    xf = np.asarray(x, dtype=np.float16).astype(_F32)
    half = 1 << (bits - 1)
    qm = _F32(half - 1)
    amax = np.abs(xf).max(axis=-1)
    with np.errstate(divide="ignore", invalid="ignore"):
        s_sym = (amax / qm).astype(_F32)
    scale = np.where(amax > 0, s_sym, _F32(1.0)).astype(_F32)
    k = np.clip(np.rint((xf / scale[..., None]).astype(_F32)), -qm, qm)
    u = (k + _F32(half)).astype(np.uint8)
    zero = np.full(scale.shape, -half, np.int16)
    return u, scale, zero


def quantize_groups_hybrid(x, bits: int):
    """[InnerQ] methodology 2: per group, symmetric when centred on zero
    (hybrid_is_symmetric), else the asymmetric map of quantize_groups."""
    sym = hybrid_is_symmetric(x)
    ca, sa, za = quantize_groups(x, bits)
    cs, ss, zs = quantize_groups_symmetric(x, bits)
    codes = np.where(sym[..., None], cs, ca).astype(np.uint8)
    return codes, np.where(sym, ss, sa).astype(_F32), np.where(sym, zs, za).astype(np.int16)


def key_channel_normalizer(k):
    """[InnerQ] methodology 4: one scale per key channel, computed once from
    the prompt's keys.  Reading: the per-channel normalization into [-1, 1]
    (as the KVQuant part of the juejin.cn page normalizes each channel),
    with the scale rounded up to a power of two and at least 1:
        lambda_c = smallest power of two >= max(1, max_t |k[t, c]|)
    so dividing a key by it and multiplying the query by it are exact.
    k: float16 [B, H, L, d] (L may be 0)  ->  float32 [B, H, d]."""
    k = np.asarray(k, np.float16).astype(np.float64)
    B, H, L, d = k.shape
    amax = np.abs(k).max(axis=2) if L else np.zeros((B, H, d))
    m, e = np.frexp(amax)                      # amax = m * 2^e, m in [0.5, 1)
    lam = np.where(m == 0.5, amax, np.ldexp(1.0, e))
    return np.where(amax <= 1.0, 1.0, lam).astype(_F32)


def normalize_keys(k, lam):
    """Keys divided by their channel scale (a power of two, exact in float32),
    rounded to float16 (round to nearest even; only values that fall below the
    float16 normal range round).  k [..., d] float16, lam broadcastable."""
    return (np.asarray(k, np.float16).astype(_F32) / np.asarray(lam, _F32)).astype(np.float16)


class InnerQCache:
    """InnerQ-style cache: keys and values both grouped along the hidden
    dimension (per token, groups of G channels, [InnerQ] methodology 1) with
    the hybrid per-group mode; the first `sinks` tokens and the most recent
    `window` tokens stay fp16 ([InnerQ] methodology 4).

    Token t < sinks is a sink.  Later tokens enter a FIFO window; once a push
    makes the window exceed `window` tokens, the oldest one is quantized and
    appended to the quantized part [sinks, nq).

    key_norm ([InnerQ] methodology 4, per-channel key scaling at prefill):
    the prompt's keys give one scale per (unit, channel) (key_channel_normalizer),
    fixed for the life of the cache; every key that is quantized, at prefill
    or when it leaves the window, is divided by it first (normalize_keys).
    The fp16 sinks and window keep the original keys.  Dequantized keys are
    returned in the original units (lambda * S * (code + Z)), which equals
    folding lambda into the query.
    """

    def __init__(self, bits, group, window, sinks, batch, kv_heads, head_dim, key_norm=False):
        if head_dim % group:
            raise ValueError("head_dim must be a multiple of G")
        if window <= 0 or sinks < 0:
            raise ValueError("window must be positive and sinks non-negative")
        self.bits, self.G, self.R, self.S = bits, group, window, sinks
        self.B, self.H, self.d = batch, kv_heads, head_dim
        B, H, d, G = batch, kv_heads, head_dim, group
        self.sink_k = np.zeros((B, H, 0, d), np.float16)
        self.sink_v = np.zeros((B, H, 0, d), np.float16)
        self.qk = np.zeros((B, H, 0, d), np.uint8)
        self.qk_s = np.zeros((B, H, 0, d // G), _F32)
        self.qk_z = np.zeros((B, H, 0, d // G), np.int16)
        self.qv = np.zeros((B, H, 0, d), np.uint8)
        self.qv_s = np.zeros((B, H, 0, d // G), _F32)
        self.qv_z = np.zeros((B, H, 0, d // G), np.int16)
        self.rk = np.zeros((B, H, 0, d), np.float16)
        self.rv = np.zeros((B, H, 0, d), np.float16)
        self.key_norm = bool(key_norm)
        self.k_norm = np.ones((B, H, d), _F32)
        self.n = 0
        self.started = False

    @property
    def nq(self):
        """End of the quantized part: tokens [sinks, nq) are quantized."""
        return self.n if self.n <= self.S else self.S + self.qk.shape[2]

    def _quantize_rows(self, rows):
        B, H, m, d = rows.shape
        G = self.G
        c, s, z = quantize_groups_hybrid(rows.reshape(B, H, m, d // G, G), self.bits)
        return c.reshape(B, H, m, d), s, z

    def _push_quantized(self, k, v):
        if self.key_norm:
            k = normalize_keys(k, self.k_norm[:, :, None, :])
        c, s, z = self._quantize_rows(k)
        self.qk = np.concatenate([self.qk, c], axis=2)
        self.qk_s = np.concatenate([self.qk_s, s], axis=2)
        self.qk_z = np.concatenate([self.qk_z, z], axis=2)
        c, s, z = self._quantize_rows(v)
        self.qv = np.concatenate([self.qv, c], axis=2)
        self.qv_s = np.concatenate([self.qv_s, s], axis=2)
        self.qv_z = np.concatenate([self.qv_z, z], axis=2)

    def prefill(self, k, v):
        if self.started:
            raise RuntimeError("prefill on a non-empty cache")
        k = np.asarray(k, np.float16)
        v = np.asarray(v, np.float16)
        L = k.shape[2]
        if self.key_norm:
            self.k_norm = key_channel_normalizer(k)
        ns = min(L, self.S)
        self.sink_k, self.sink_v = k[:, :, :ns].copy(), v[:, :, :ns].copy()
        if L > self.S:
            r = min(self.R, L - self.S)
            self._push_quantized(k[:, :, self.S:L - r], v[:, :, self.S:L - r])
            self.rk, self.rv = k[:, :, L - r:].copy(), v[:, :, L - r:].copy()
        self.n = L
        self.started = True

    def append(self, k_new, v_new):
        if not self.started:
            raise RuntimeError("append before prefill")
        k_new = np.asarray(k_new, np.float16)[:, :, None, :]
        v_new = np.asarray(v_new, np.float16)[:, :, None, :]
        if self.n < self.S:
            self.sink_k = np.concatenate([self.sink_k, k_new], axis=2)
            self.sink_v = np.concatenate([self.sink_v, v_new], axis=2)
        else:
            self.rk = np.concatenate([self.rk, k_new], axis=2)
            self.rv = np.concatenate([self.rv, v_new], axis=2)
            if self.rk.shape[2] > self.R:          # pop the oldest and quantize it
                self._push_quantized(self.rk[:, :, :1], self.rv[:, :, :1])
                self.rk, self.rv = self.rk[:, :, 1:], self.rv[:, :, 1:]
        self.n += 1

    def dequantized(self):
        B, H, d, G = self.B, self.H, self.d, self.G
        m = self.qk.shape[2]
        kh = dequantize(self.qk.reshape(B, H, m, d // G, G), self.qk_s, self.qk_z).reshape(B, H, m, d)
        kh = (kh * self.k_norm[:, :, None, :]).astype(_F32)   # exact: powers of two
        vh = dequantize(self.qv.reshape(B, H, m, d // G, G), self.qv_s, self.qv_z).reshape(B, H, m, d)
        K = np.concatenate([self.sink_k.astype(_F32), kh, self.rk.astype(_F32)], axis=2)
        V = np.concatenate([self.sink_v.astype(_F32), vh, self.rv.astype(_F32)], axis=2)
        return K, V

    def buffers(self, max_tokens):
        """Device layout: quantized token t (sinks <= t < nq) at row t of
        k_codes/v_codes u32 [B,H,cap,d*b/32] and of k_scale/k_zero/v_scale/
        v_zero [B,H,cap,d/G]; window token t at ring slot t mod R of
        k_resid/v_resid f16 [B,H,R,d]; sink t at row t of k_sink/v_sink f16
        [B,H,sinks,d]."""
        B, H, d, G, R, b, S = self.B, self.H, self.d, self.G, self.R, self.bits, self.S
        cap = max_tokens
        W = d * b // 32
        out = {
            "k_codes": np.zeros((B, H, cap, W), np.uint32),
            "k_scale": np.zeros((B, H, cap, d // G), _F32),
            "k_zero": np.zeros((B, H, cap, d // G), np.int16),
            "v_codes": np.zeros((B, H, cap, W), np.uint32),
            "v_scale": np.zeros((B, H, cap, d // G), _F32),
            "v_zero": np.zeros((B, H, cap, d // G), np.int16),
            "k_resid": np.zeros((B, H, R, d), np.float16),
            "v_resid": np.zeros((B, H, R, d), np.float16),
            "k_sink": np.zeros((B, H, S, d), np.float16),
            "v_sink": np.zeros((B, H, S, d), np.float16),
        }
        m = self.qk.shape[2]
        rows = slice(S, S + m)
        out["k_codes"][:, :, rows] = pack_rows(self.qk, b)
        out["v_codes"][:, :, rows] = pack_rows(self.qv, b)
        out["k_scale"][:, :, rows], out["k_zero"][:, :, rows] = self.qk_s, self.qk_z
        out["v_scale"][:, :, rows], out["v_zero"][:, :, rows] = self.qv_s, self.qv_z
        ns = self.sink_k.shape[2]
        out["k_sink"][:, :, :ns], out["v_sink"][:, :, :ns] = self.sink_k, self.sink_v
        nq = self.nq
        for i in range(self.rk.shape[2]):
            out["k_resid"][:, :, (nq + i) % R] = self.rk[:, :, i]
            out["v_resid"][:, :, (nq + i) % R] = self.rv[:, :, i]
        if self.key_norm:
            out["k_norm"] = self.k_norm.copy()     # f32 [B,H,d], channel scales
        return out

    def live_resid_slots(self):
        nq = self.nq
        slots = [(nq + i) % self.R for i in range(self.rk.shape[2])]
        return slots, slots


def innerq_attention_call_bytes(batch, q_heads, kv_heads, head_dim, bits, group, n, nq, sinks):
    """Algorithmic bytes of one decode-attention call over an InnerQ-style
    cache: per quantized token, key and value codes plus one fp32 scale and
    int16 zero per group each; fp16 sinks and window; fp16 q, fp32 out."""
    d, b, G = head_dim, bits, group
    m = max(0, nq - sinks) if n > sinks else 0
    fp16_tokens = n - m
    per_unit = m * 2 * (d * b // 8 + (d // G) * 6) + fp16_tokens * d * 2 * 2
    return batch * kv_heads * per_unit + batch * q_heads * d * (2 + 4)


# --------------------------------------------------------------------------- attention
def attention(q, K, V, softmax_scale):
    """Decode attention of one query per head over the whole cache, float64.

    out = softmax(scale * q K^T) V with no mask (the new token is part of the
    cache and attends to every cached token, itself included).  Query head h
    reads kv head h // (Hq / Hkv).

    q fp16/float [B,Hq,d]; K, V float32 [B,Hkv,n,d]  ->  float64 [B,Hq,d].
    """
    q = np.asarray(q).astype(np.float64)
    K = np.asarray(K).astype(np.float64)
    V = np.asarray(V).astype(np.float64)
    B, Hq, d = q.shape
    Hkv = K.shape[1]
    rep = Hq // Hkv
    Kx = np.repeat(K, rep, axis=1)                  # [B,Hq,n,d]
    Vx = np.repeat(V, rep, axis=1)
    s = np.einsum("bhd,bhnd->bhn", q, Kx) * float(softmax_scale)
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=-1, keepdims=True)
    return np.einsum("bhn,bhnd->bhd", p, Vx)


# --------------------------------------------------------------------------- bytes
def kv_code_bytes_per_token(layers, kv_heads, head_dim, bits):
    """Cache bytes one token adds for a whole model, codes only ([HFQ] 3.2)."""
    return layers * 2 * kv_heads * head_dim * bits // 8


def attention_call_bytes(batch, q_heads, kv_heads, head_dim, bits, group, n, nq_k, nq_v, meta=META_F32):
    """Algorithmic bytes one decode-attention call must move.

    Per unit: key codes + key metadata (scale + int16 zero per (group,
    channel): 6 bytes, or 4 with META_F16) + value codes + value metadata (per
    (token, channel group)) + the fp16 residual keys and values; plus the
    fp16 query and the fp32 output of every query head.
    """
    d, b, G = head_dim, bits, group
    mb = 6 if meta == META_F32 else 4
    per_unit = (nq_k * d * b // 8 + (nq_k // G) * d * mb
                + nq_v * d * b // 8 + nq_v * (d // G) * mb
                + ((n - nq_k) + (n - nq_v)) * d * 2)
    return batch * kv_heads * per_unit + batch * q_heads * d * (2 + 4)
