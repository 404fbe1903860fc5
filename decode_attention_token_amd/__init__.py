"""Python binding of libkvq: quantized KV cache + decode attention on MI355X.

Argument marshalling only: every step of the hot path runs in the HIP kernels
behind the C ABI declared in include/kvq.h.  PyTorch supplies device memory
and the current HIP stream.  There is no CPU fallback: if libkvq.so is not
built, importing the library raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkvq.so")

KVQ_OK, KVQ_ERR_ARG, KVQ_ERR_CAPACITY, KVQ_ERR_STATE, KVQ_ERR_DEVICE, KVQ_ERR_UNSUPPORTED = range(6)
KVQ_V_CHUNK, KVQ_V_FIFO = 0, 1
KVQ_SCHEME_KIVI, KVQ_SCHEME_INNERQ = 0, 1
KVQ_META_F32, KVQ_META_F16 = 0, 1
KVQ_SCHED_FIXED, KVQ_SCHED_QUEUE = 0, 1
KVQ_KERNEL_AUTO, KVQ_KERNEL_VALU = 0, 1
KVQ_KEYNORM_NONE, KVQ_KEYNORM_PROMPT = 0, 1

EXPORTED = [
    "kvq_layout_bytes", "kvq_auto_splits", "kvq_workspace_bytes", "kvq_quantize_prefill",
    "kvq_append_token", "kvq_decode_attention", "kvq_decode_attention_static", "kvq_decode_step",
    "kvq_stream_read_probe", "kvq_status_string", "kvq_last_error",
]
KVQ_STATIC_SCRATCH_BYTES = 16 << 20


class kvq_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "bits", "group", "residual", "batch", "num_q_heads", "num_kv_heads", "head_dim",
        "max_tokens", "v_policy", "scheme", "sink_tokens", "meta_format", "schedule", "kernel", "key_norm")]


class kvq_layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in (
        "k_codes", "k_scale", "k_zero", "v_codes", "v_scale", "v_zero", "k_resid", "v_resid", "k_sink",
        "v_sink", "k_norm")]


class kvq_cache(ctypes.Structure):
    _fields_ = [
        ("k_codes", ctypes.c_void_p), ("k_scale", ctypes.c_void_p), ("k_zero", ctypes.c_void_p),
        ("v_codes", ctypes.c_void_p), ("v_scale", ctypes.c_void_p), ("v_zero", ctypes.c_void_p),
        ("k_resid", ctypes.c_void_p), ("v_resid", ctypes.c_void_p),
        ("k_sink", ctypes.c_void_p), ("v_sink", ctypes.c_void_p),
        ("n_tokens", ctypes.c_int64), ("nq_k", ctypes.c_int64), ("nq_v", ctypes.c_int64),
        ("started", ctypes.c_int32), ("flushes", ctypes.c_int32), ("k_norm", ctypes.c_void_p),
        ("prequant", ctypes.c_int64),
    ]


class KVQError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"kvq status {status}: {msg}")
        self.status = status


_lib_handle = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Loads libkvq.so (built in-tree) and declares its signatures."""
    global _lib_handle
    if _lib_handle is not None:
        return _lib_handle
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing; build it with __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    vp = ctypes.c_void_p
    lib.kvq_layout_bytes.argtypes = [P(kvq_config), P(kvq_layout)]
    lib.kvq_layout_bytes.restype = ctypes.c_int
    lib.kvq_auto_splits.argtypes = [P(kvq_config), ctypes.c_int64]
    lib.kvq_auto_splits.restype = ctypes.c_int32
    lib.kvq_workspace_bytes.argtypes = [P(kvq_config), ctypes.c_int64, ctypes.c_int32]
    lib.kvq_workspace_bytes.restype = ctypes.c_size_t
    lib.kvq_quantize_prefill.argtypes = [P(kvq_config), P(kvq_cache), vp, vp, ctypes.c_int64, vp]
    lib.kvq_quantize_prefill.restype = ctypes.c_int
    lib.kvq_append_token.argtypes = [P(kvq_config), P(kvq_cache), vp, vp, vp]
    lib.kvq_append_token.restype = ctypes.c_int
    lib.kvq_decode_attention.argtypes = [P(kvq_config), P(kvq_cache), vp, ctypes.c_float, vp, vp,
                                         ctypes.c_size_t, ctypes.c_int32, vp]
    lib.kvq_decode_attention.restype = ctypes.c_int
    lib.kvq_decode_attention_static.argtypes = [P(kvq_config), P(kvq_cache), vp, ctypes.c_float, vp,
                                                ctypes.c_int32, vp]
    lib.kvq_decode_attention_static.restype = ctypes.c_int
    lib.kvq_decode_step.argtypes = [P(kvq_config), P(kvq_cache), vp, vp, vp, ctypes.c_float, vp, vp,
                                    ctypes.c_size_t, ctypes.c_int32, vp]
    lib.kvq_decode_step.restype = ctypes.c_int
    lib.kvq_stream_read_probe.argtypes = [vp, ctypes.c_size_t, vp, vp]
    lib.kvq_stream_read_probe.restype = ctypes.c_int
    lib.kvq_status_string.argtypes = [ctypes.c_int]
    lib.kvq_status_string.restype = ctypes.c_char_p
    lib.kvq_last_error.argtypes = []
    lib.kvq_last_error.restype = ctypes.c_char_p
    _lib_handle = lib
    return lib


def _check(status: int):
    if status != KVQ_OK:
        lib = load_library()
        raise KVQError(status, lib.kvq_last_error().decode() or lib.kvq_status_string(status).decode())


def make_config(bits, group, residual, batch, num_q_heads, num_kv_heads, head_dim, max_tokens,
                v_policy=KVQ_V_CHUNK, scheme=KVQ_SCHEME_KIVI, sink_tokens=0, meta_format=KVQ_META_F32,
                schedule=KVQ_SCHED_FIXED, kernel=KVQ_KERNEL_AUTO, key_norm=KVQ_KEYNORM_NONE) -> kvq_config:
    return kvq_config(bits, group, residual, batch, num_q_heads, num_kv_heads, head_dim, max_tokens,
                      v_policy, scheme, sink_tokens, meta_format, schedule, kernel, key_norm)


def make_innerq_config(bits, group, window, sink_tokens, batch, num_q_heads, num_kv_heads, head_dim,
                       max_tokens, key_norm=KVQ_KEYNORM_NONE) -> kvq_config:
    """InnerQ-style cache: hybrid groups of `group` channels per token for keys
    and values, `sink_tokens` leading and `window` recent tokens in fp16;
    key_norm=KVQ_KEYNORM_PROMPT scales keys once per channel at prefill."""
    return make_config(bits, group, window, batch, num_q_heads, num_kv_heads, head_dim, max_tokens,
                       KVQ_V_FIFO, KVQ_SCHEME_INNERQ, sink_tokens, key_norm=key_norm)


def kvq_layout_bytes(cfg: kvq_config) -> kvq_layout:
    out = kvq_layout()
    _check(load_library().kvq_layout_bytes(ctypes.byref(cfg), ctypes.byref(out)))
    return out


def kvq_auto_splits(cfg: kvq_config, n_tokens: int) -> int:
    return int(load_library().kvq_auto_splits(ctypes.byref(cfg), int(n_tokens)))


def kvq_workspace_bytes(cfg: kvq_config, n_tokens: int, splits: int = 0) -> int:
    return int(load_library().kvq_workspace_bytes(ctypes.byref(cfg), int(n_tokens), int(splits)))


def _stream_ptr(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


def _f16_ptr(t: Optional[torch.Tensor], shape, name) -> int:
    if t is None:
        return 0
    if t.dtype != torch.float16 or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous fp16 CUDA tensor")
    if t.shape != shape:
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr()


class KVCache:
    """One layer's quantized KV cache in caller-owned (torch) device memory."""

    _DT = {"k_codes": torch.int32, "k_scale": torch.float32, "k_zero": torch.int16,
           "v_codes": torch.int32, "v_scale": torch.float32, "v_zero": torch.int16,
           "k_resid": torch.float16, "v_resid": torch.float16, "k_sink": torch.float16,
           "v_sink": torch.float16, "k_norm": torch.float32}

    def __init__(self, cfg: kvq_config, device="cuda"):
        self.cfg = cfg
        lay = kvq_layout_bytes(cfg)
        B, H, d, cap, G, R, S = (cfg.batch, cfg.num_kv_heads, cfg.head_dim, cfg.max_tokens,
                                 cfg.group, cfg.residual, cfg.sink_tokens)
        W = d * cfg.bits // 32
        innerq = cfg.scheme == KVQ_SCHEME_INNERQ
        packed = cfg.meta_format == KVQ_META_F16   # (S, Z) words in *_scale, no *_zero
        kmeta = (B, H, cap, d // G) if innerq else (B, H, cap // G, d)
        vmeta = (B, H, cap, d // G)
        none = lambda shp: shp[:2] + (0,) + shp[3:]
        shapes = {"k_codes": (B, H, cap, W), "k_scale": kmeta, "k_zero": none(kmeta) if packed else kmeta,
                  "v_codes": (B, H, cap, W), "v_scale": vmeta, "v_zero": none(vmeta) if packed else vmeta,
                  "k_resid": (B, H, R, d), "v_resid": (B, H, R, d),
                  "k_sink": (B, H, S, d), "v_sink": (B, H, S, d),
                  "k_norm": (B, H, d if cfg.key_norm else 0)}
        self.tensors = {}
        for name, shp in shapes.items():
            dt = torch.int32 if packed and name in ("k_scale", "v_scale") else self._DT[name]
            t = torch.zeros(shp, dtype=dt, device=device)
            assert t.numel() * t.element_size() == getattr(lay, name), name
            self.tensors[name] = t
        self.c = kvq_cache()
        for name, t in self.tensors.items():
            setattr(self.c, name, t.data_ptr() if t.numel() else None)
        # per-call marshalling state, built once
        self._cfg_ref = ctypes.byref(cfg)
        self._c_ref = ctypes.byref(self.c)
        self._q_shape = torch.Size((cfg.batch, cfg.num_q_heads, cfg.head_dim))
        self._kv_shape = torch.Size((cfg.batch, cfg.num_kv_heads, cfg.head_dim))

    # counters
    @property
    def n_tokens(self):
        return self.c.n_tokens

    @property
    def nq_k(self):
        return self.c.nq_k

    @property
    def nq_v(self):
        return self.c.nq_v

    @property
    def flushes(self):
        return self.c.flushes

    def prefill(self, k: torch.Tensor, v: torch.Tensor, stream=None):
        kvq_quantize_prefill(self.cfg, self, k, v, stream)

    def append(self, k_new: torch.Tensor, v_new: torch.Tensor, stream=None):
        kvq_append_token(self.cfg, self, k_new, v_new, stream)

    def workspace(self, n_tokens=None, splits=0) -> torch.Tensor:
        n = self.cfg.max_tokens if n_tokens is None else n_tokens
        nbytes = kvq_workspace_bytes(self.cfg, n, splits)
        # zero-filled: the leading work-queue counters must start at zero
        # (every call leaves them at zero)
        return torch.zeros(max(nbytes, 4) // 4, dtype=torch.float32, device=self.tensors["k_codes"].device)

    def step(self, k_new, v_new, q, softmax_scale=None, out=None, workspace=None, splits=0, stream=None):
        """Append one token and attend (one launch when no flush is due)."""
        cfg = self.cfg
        if softmax_scale is None:
            softmax_scale = 1.0 / math.sqrt(cfg.head_dim)
        if out is None:
            out = torch.empty(cfg.batch, cfg.num_q_heads, cfg.head_dim, dtype=torch.float32, device=q.device)
        if workspace is None:
            workspace = self.workspace(self.n_tokens + 1, splits)
        kvq_decode_step(cfg, self, k_new, v_new, q, softmax_scale, out, workspace, splits, stream)
        return out

    def attention_static(self, q, softmax_scale=None, out=None, splits=0, stream=None):
        """Attention without a workspace: the library's static device scratch."""
        cfg = self.cfg
        if softmax_scale is None:
            softmax_scale = 1.0 / math.sqrt(cfg.head_dim)
        if out is None:
            out = torch.empty(cfg.batch, cfg.num_q_heads, cfg.head_dim, dtype=torch.float32, device=q.device)
        kvq_decode_attention_static(cfg, self, q, softmax_scale, out, splits, stream)
        return out

    def attention(self, q, softmax_scale=None, out=None, workspace=None, splits=0, stream=None):
        cfg = self.cfg
        if softmax_scale is None:
            softmax_scale = 1.0 / math.sqrt(cfg.head_dim)
        if out is None:
            out = torch.empty(cfg.batch, cfg.num_q_heads, cfg.head_dim, dtype=torch.float32, device=q.device)
        if workspace is None:
            workspace = self.workspace(self.n_tokens, splits)
        kvq_decode_attention(cfg, self, q, softmax_scale, out, workspace, splits, stream)
        return out


def kvq_quantize_prefill(cfg, cache: KVCache, k, v, stream=None):
    L = 0 if k is None else int(k.shape[2])
    shape = (cfg.batch, cfg.num_kv_heads, L, cfg.head_dim)
    kp = _f16_ptr(k, shape, "k") if L else 0
    vp = _f16_ptr(v, shape, "v") if L else 0
    _check(load_library().kvq_quantize_prefill(ctypes.byref(cfg), ctypes.byref(cache.c), kp, vp, L,
                                               _stream_ptr(stream)))


def kvq_append_token(cfg, cache: KVCache, k_new, v_new, stream=None):
    if cfg is not cache.cfg:
        raise ValueError("cfg must be the cache's own config")
    shape = cache._kv_shape
    _check(_lib_handle.kvq_append_token(cache._cfg_ref, cache._c_ref, _f16_ptr(k_new, shape, "k_new"),
                                        _f16_ptr(v_new, shape, "v_new"), _stream_ptr(stream)))


def kvq_decode_attention(cfg, cache: KVCache, q, softmax_scale, out, workspace, splits=0, stream=None):
    if cfg is not cache.cfg:
        raise ValueError("cfg must be the cache's own config")
    qp = _f16_ptr(q, cache._q_shape, "q")
    if out.dtype != torch.float32 or not out.is_cuda or not out.is_contiguous() or out.shape != cache._q_shape:
        raise ValueError("out must be a contiguous fp32 CUDA tensor [batch][num_q_heads][head_dim]")
    if not workspace.is_cuda:
        raise ValueError("workspace must be device memory")
    nbytes = workspace.numel() * workspace.element_size()
    _check(_lib_handle.kvq_decode_attention(cache._cfg_ref, cache._c_ref, qp, softmax_scale, out.data_ptr(),
                                            workspace.data_ptr(), nbytes, splits, _stream_ptr(stream)))


def kvq_decode_attention_static(cfg, cache: KVCache, q, softmax_scale, out, splits=0, stream=None):
    """kvq_decode_attention with the library's static device scratch in place
    of a workspace (for callers that cannot allocate)."""
    if cfg is not cache.cfg:
        raise ValueError("cfg must be the cache's own config")
    qp = _f16_ptr(q, cache._q_shape, "q")
    if out.dtype != torch.float32 or not out.is_cuda or not out.is_contiguous() or out.shape != cache._q_shape:
        raise ValueError("out must be a contiguous fp32 CUDA tensor [batch][num_q_heads][head_dim]")
    _check(load_library().kvq_decode_attention_static(cache._cfg_ref, cache._c_ref, qp, softmax_scale,
                                                      out.data_ptr(), splits, _stream_ptr(stream)))


def kvq_decode_step(cfg, cache: KVCache, k_new, v_new, q, softmax_scale, out, workspace, splits=0, stream=None):
    if cfg is not cache.cfg:
        raise ValueError("cfg must be the cache's own config")
    kv = cache._kv_shape
    qp = _f16_ptr(q, cache._q_shape, "q")
    kp = _f16_ptr(k_new, kv, "k_new")
    vp = _f16_ptr(v_new, kv, "v_new")
    if out.dtype != torch.float32 or not out.is_cuda or not out.is_contiguous() or out.shape != cache._q_shape:
        raise ValueError("out must be a contiguous fp32 CUDA tensor [batch][num_q_heads][head_dim]")
    if not workspace.is_cuda:
        raise ValueError("workspace must be device memory")
    nbytes = workspace.numel() * workspace.element_size()
    _check(_lib_handle.kvq_decode_step(cache._cfg_ref, cache._c_ref, kp, vp, qp, softmax_scale, out.data_ptr(),
                                       workspace.data_ptr(), nbytes, splits, _stream_ptr(stream)))


def kvq_stream_read_probe(buf: torch.Tensor, out: torch.Tensor, stream=None):
    """Streaming-read probe over a device buffer (measurement only): reads
    every byte of `buf` once; `out` is a device int32 scratch word."""
    if not buf.is_cuda or not out.is_cuda:
        raise ValueError("buf and out must be device tensors")
    nbytes = buf.numel() * buf.element_size()
    _check(load_library().kvq_stream_read_probe(buf.data_ptr(), nbytes, out.data_ptr(), _stream_ptr(stream)))
