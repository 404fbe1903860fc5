"""Seeded synthetic workloads shared by the tests, the bench and the smoke check.

This module only draws inputs: shapes, seeds and value distributions.  It holds
none of the method's arithmetic (no quantizer, no packing, no attention), so both
the CPU oracle and the HIP path can consume the very same fp16 bits without
sharing any code that computes a result.

Value laws follow the KIVI observations on the juejin.cn page "大模型量化技术原理：
KIVI、IntactKV、KVQuant" (KIVI, section on why keys and values are quantized
along different axes): a few fixed key channels carry very large magnitudes for
every token, while values show no outliers.  Values are drawn N(0, 1) in fp32,
the chosen key channels are multiplied by a fixed factor, and the result is
rounded to fp16 (round to nearest even).  The shapes are those of the
Llama-2-7B KV cache (32 layers, 32 heads, head_dim 128) used on the pgsm.cn page
on KV-cache quantization (section 3.2, memory example).

Seed for a tensor = 1000 * config_id + 10 * layer + tensor_id, with tensor ids
0 K, 1 V, 2 q (all decode steps), 3 k_new, 4 v_new, 5 outlier-channel pick.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

T_K, T_V, T_Q, T_KNEW, T_VNEW, T_OUTLIER = 0, 1, 2, 3, 4, 5


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic decode-attention workload."""

    name: str
    config_id: int
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    context: int          # tokens present after prefill
    bits: int
    group: int            # G
    residual: int         # R
    outlier_channels: int  # fixed key channels per kv head that are scaled
    outlier_scale: float
    steps: int            # decode steps the workload runs
    layers: int           # distinct layer caches the workload cycles through
    v_policy: int = 0     # 0 chunked residual, 1 FIFO value queue
    scheme: int = 0       # 0 KIVI-style, 1 InnerQ-style (R is then the recent window)
    sinks: int = 0        # leading tokens kept fp16
    meta: int = 0         # 0 fp32 scale + int16 zero; 1 packed fp16 scale | zero word

    @property
    def units(self) -> int:
        return self.batch * self.num_kv_heads

    @property
    def max_tokens(self) -> int:
        """Cache capacity: context plus the decode steps, rounded up to R."""
        need = self.context + self.steps
        r = self.residual
        return ((need + r - 1) // r) * r

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads: a tiny one the oracle finishes in well under a second,
# the Llama-2-7B-layer-shaped 2-bit decode, a 4-bit variant, a grouped-query
# long-context case and a long-context 4-bit InnerQ-style case (groups of 64
# channels per token for keys and values, 4 sink and 32 recent fp16 tokens,
# as in the euno.news InnerQ summary, methodology 1 and 4).
TINY = Workload("tiny-b1-h1-L256-2bit-G32-R32", 1, 1, 1, 1, 128, 256, 2, 32, 32, 4, 10.0, 1, 1)
LLAMA7B_2BIT = Workload("llama2-7b-layer-b16-h32-L4096-2bit-G32-R128", 2, 16, 32, 32, 128, 4096,
                        2, 32, 128, 3, 8.0, 64, 32)
LLAMA7B_4BIT = Workload("b64-h32-L8192-4bit-G64-R128", 3, 64, 32, 32, 128, 8192, 4, 64, 128,
                        3, 8.0, 128, 1)
GQA_LONG = Workload("gqa-b8-q32-kv8-L32768-2bit-G32-R128", 4, 8, 32, 8, 128, 32768, 2, 32, 128,
                    4, 10.0, 1, 8)
LONG_4BIT = Workload("innerq-b4-h32-L131072-4bit-G64-S4-W32", 5, 4, 32, 32, 128, 131072, 4, 64, 32,
                     4, 10.0, 1, 1, v_policy=1, scheme=1, sinks=4)

WORKLOADS = {w.config_id: w for w in (TINY, LLAMA7B_2BIT, LLAMA7B_4BIT, GQA_LONG, LONG_4BIT)}


def seed_of(w: Workload, layer: int, tensor: int) -> int:
    return 1000 * w.config_id + 10 * layer + tensor


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def outlier_channels(w: Workload, layer: int = 0) -> torch.Tensor:
    """Fixed outlier key channels, int64 [num_kv_heads][outlier_channels]."""
    g = _gen("cpu", seed_of(w, layer, T_OUTLIER))
    picks = [torch.randperm(w.head_dim, generator=g)[: w.outlier_channels]
             for _ in range(w.num_kv_heads)]
    if w.outlier_channels == 0:
        return torch.zeros(w.num_kv_heads, 0, dtype=torch.int64)
    return torch.stack(picks)


def _channel_gain(w: Workload, layer: int, device) -> torch.Tensor:
    gain = torch.ones(w.num_kv_heads, w.head_dim, dtype=torch.float32)
    ch = outlier_channels(w, layer)
    for h in range(w.num_kv_heads):
        gain[h, ch[h]] = w.outlier_scale
    return gain.to(device)


def _randn(shape, device, seed: int) -> torch.Tensor:
    return torch.randn(*shape, generator=_gen(device, seed), device=device, dtype=torch.float32)


def gen_prefill(w: Workload, layer: int = 0, device="cpu", context: Optional[int] = None):
    """K, V fp16 [B][Hkv][L][d] for the prompt."""
    L = w.context if context is None else context
    shape = (w.batch, w.num_kv_heads, L, w.head_dim)
    k = _randn(shape, device, seed_of(w, layer, T_K))
    k.mul_(_channel_gain(w, layer, device)[None, :, None, :])
    v = _randn(shape, device, seed_of(w, layer, T_V))
    return k.half(), v.half()


def gen_queries(w: Workload, layer: int = 0, device="cpu", steps: Optional[int] = None):
    """q fp16 [steps][B][Hq][d]."""
    s = w.steps if steps is None else steps
    q = _randn((s, w.batch, w.num_q_heads, w.head_dim), device, seed_of(w, layer, T_Q))
    return q.half()


def gen_new_tokens(w: Workload, layer: int = 0, device="cpu", steps: Optional[int] = None):
    """k_new, v_new fp16 [steps][B][Hkv][d]; the keys keep the same outlier channels."""
    s = w.steps if steps is None else steps
    shape = (s, w.batch, w.num_kv_heads, w.head_dim)
    k = _randn(shape, device, seed_of(w, layer, T_KNEW))
    k.mul_(_channel_gain(w, layer, device)[None, None, :, :])
    v = _randn(shape, device, seed_of(w, layer, T_VNEW))
    return k.half(), v.half()
