"""Decode-attention benchmark on one MI355X.

A step is one decode step of the whole batch through every layer of the
workload: per layer, kvq_decode_step = kvq_append_token (residual write, eager
flush when due) + kvq_decode_attention, one kernel launch when no flush is
due.  Caches are prefilled before timing; inputs for every step are resident
in HBM when timing starts.

Prints one JSON line:
  value        effective KV GB/s of the whole timed loop (algorithmic bytes of
               every attention call / loop time)
  tokens_per_s batch * steps / loop time
  roofline     the decode kernel as the timed loop launches it (the fused
               append + attention step): algorithmic bytes per launch / its
               average duration, from HIP events on the library's stream
               around the timed loop, against 8 TB/s
  attention_only  the same kernel launched by kvq_decode_attention alone
               (back-to-back passes over the layers, HIP events)
  fp16_equivalent  bytes an fp16 cache of the same tokens would move per
               call / the attention-only call time (labelled; not a roofline
               fraction)
  stream_ceiling  GB/s of the library's plain streaming-read probe over
               4 GiB (median of 3 timed batches after 0.5 s of untimed
               reads), and the roofline's achieved rate as a fraction of it
  prefill, flush  HIP-event timings of one prefill and one flushing append
  tiny         latency of one decode step on the tiny workload
  cpu_baseline the NumPy oracle on sampled units, timed on this host: one
               thread and a process pool over the host cores, scaled to the
               same byte formula; plus one oracle prefill and one flush
  source       content digests of the sources that produced the numbers
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import decode_attention_token_amd as kvq  # noqa: E402
from workloads import WORKLOADS, LLAMA7B_2BIT, gen_new_tokens, gen_prefill, gen_queries  # noqa: E402

HBM_PEAK_GBS = 8000.0
METRIC = "decode-attn effective KV GB/s (% HBM peak) + tokens/s, Llama-2-7B shape 2-bit"


def attn_bytes(w, n, nq_k, nq_v):
    """Algorithmic bytes of one decode-attention call (codes, fp32 scale + int16
    zero per group, fp16 residual / sinks / window, fp16 q, fp32 out)."""
    d, b, G = w.head_dim, w.bits, w.group
    if w.scheme == kvq.KVQ_SCHEME_INNERQ:
        m = nq_k - min(n, w.sinks)   # quantized tokens
        per_unit = m * 2 * (d * b // 8 + (d // G) * 6) + (n - m) * d * 2 * 2
    else:
        ns = min(n, w.sinks)            # fp16 sink tokens; nq_k / nq_v count them
        qk, qv = nq_k - ns, nq_v - ns   # quantized key / value tokens
        mb = 4 if w.meta else 6         # metadata bytes per group
        per_unit = (qk * d * b // 8 + (qk // G) * d * mb + qv * d * b // 8 + qv * (d // G) * mb
                    + ((n - qk) + (n - qv)) * d * 2)
    return w.batch * w.num_kv_heads * per_unit + w.batch * w.num_q_heads * d * 6


def stream_ceiling(dev, stream, reps=5, settle_s=0.5, batches=3):
    """GB/s of kvq_stream_read_probe over a 4 GiB buffer (16x the MALL),
    timed with HIP events on the given stream: the median of `batches`
    batches of `reps` reads, after settle_s seconds of untimed reads.  For
    up to 0.6 s after large device buffers are returned to the driver, reads
    run about 6% slower; the bench returns none before its timings, and the
    settle is a second guard."""
    buf = torch.ones(4 << 30, dtype=torch.uint8, device=dev)
    out = torch.zeros(1, dtype=torch.int32, device=dev)
    sp = stream.cuda_stream
    t0 = time.perf_counter()
    while True:
        for _ in range(4):
            kvq.kvq_stream_read_probe(buf, out, sp)
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= settle_s:
            break
    rates = []
    for _ in range(batches):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            kvq.kvq_stream_read_probe(buf, out, sp)
        e1.record(stream)
        torch.cuda.synchronize()
        rates.append(buf.numel() * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del buf, out
    torch.cuda.empty_cache()
    return sorted(rates)[len(rates) // 2]


KEY_NORM = {"on": False}   # --key-norm: InnerQ caches scale keys per channel at prefill


def make_cfg(w, max_tokens, schedule=kvq.KVQ_SCHED_FIXED, kernel=kvq.KVQ_KERNEL_AUTO):
    key_norm = kvq.KVQ_KEYNORM_PROMPT if KEY_NORM["on"] and w.scheme == kvq.KVQ_SCHEME_INNERQ else 0
    return kvq.make_config(w.bits, w.group, w.residual, w.batch, w.num_q_heads, w.num_kv_heads,
                           w.head_dim, max_tokens, w.v_policy, w.scheme, w.sinks, w.meta, schedule, kernel, key_norm)


def build_caches(w, layers, max_tokens, dev, schedule=kvq.KVQ_SCHED_FIXED, kernel=kvq.KVQ_KERNEL_AUTO):
    cfg = make_cfg(w, max_tokens, schedule, kernel)
    caches = []
    for layer in range(layers):
        k, v = gen_prefill(w, layer, dev)
        c = kvq.KVCache(cfg, dev)
        c.prefill(k, v)
        torch.cuda.synchronize()
        del k, v
        caches.append(c)
    # (no torch.cuda.empty_cache(): returning the prefill temporaries to the
    # driver slows every read of the device by about 6% for up to 0.6 s)
    return cfg, caches


def sample_units(w, host_bytes=512 << 20, seed=7):
    """A seeded sample of (batch, kv head) units for the oracle, as many as
    fit about host_bytes of fp16 prompt (at least 4, at most 64)."""
    per_unit = w.context * w.head_dim * 2 * 2
    count = max(4, min(64, host_bytes // max(per_unit, 1), w.units))
    return [int(u) for u in np.random.default_rng(seed).permutation(w.units)[:count]]


# decode kernel and its source files per kind
KERNELS = {
    0: ("decode_attn_kernel", ("kvq_attn.hip", "kvq_attn_common.h", "kvq_quant_common.h", "kvq_internal.h")),
    1: ("innerq_attn_kernel", ("kvq_innerq.hip", "kvq_attn_common.h", "kvq_quant_common.h", "kvq_internal.h")),
    "gqa4": ("gqa_mfma_kernel", ("kvq_attn_gqa.hip", "kvq_attn_common.h", "kvq_quant_common.h", "kvq_internal.h")),
}


def kernel_key(w, kernel=kvq.KVQ_KERNEL_AUTO):
    """Which decode kernel dominates the workload: the matrix-core kernel for
    four query heads per kv head (KIVI layout, unless the config selects the
    vector-ALU kernel), else the scheme's vector-ALU kernel."""
    if (w.scheme == kvq.KVQ_SCHEME_KIVI and w.num_q_heads == 4 * w.num_kv_heads
            and kernel == kvq.KVQ_KERNEL_AUTO):
        return "gqa4"
    return w.scheme


def kernel_source_digest(scheme=0):
    import hashlib
    h = hashlib.sha256()
    for name in KERNELS[scheme][1]:
        with open(os.path.join(ROOT, "decode_attention_token_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(w, kernel=kvq.KVQ_KERNEL_AUTO):
    """HBM bytes per launch of the decode kernel from the committed counter
    summaries (profiles/*_traffic.txt) for this workload, or None when none
    exists or it was taken on a different kernel source."""
    key = kernel_key(w, kernel)
    pdir = os.path.join(ROOT, "profiles")
    try:
        names = sorted(f for f in os.listdir(pdir) if f.endswith("_traffic.txt"))
    except OSError:
        return None
    for name in names:
        with open(os.path.join(pdir, name)) as f:
            kv = dict(line.split(":", 1) for line in f if ":" in line and not line.startswith("#"))
        kv = {k.strip(): v.strip() for k, v in kv.items()}
        if kv.get("workload") != w.name or not kv.get("kernel", "").startswith(KERNELS[key][0]):
            continue
        if kv.get("kernel_source_digest") != kernel_source_digest(key):
            return None
        try:
            return int(float(kv["hbm_bytes_per_launch"]))
        except (KeyError, ValueError):
            return None
    return None


def host_sample(w, units, dev):
    """Host copies of the sampled units' layer-0 inputs (the same fp16 bits
    the GPU caches use): prompt K, V, R new tokens and the first query."""
    k, v = gen_prefill(w, 0, dev)
    kn, vn = gen_new_tokens(w, 0, dev, steps=w.residual)
    q = gen_queries(w, 0, dev, steps=1)[0]
    hpg = w.num_q_heads // w.num_kv_heads
    out = []
    for u in units:
        b, h = divmod(u, w.num_kv_heads)
        out.append((k[b:b + 1, h:h + 1].cpu().numpy(), v[b:b + 1, h:h + 1].cpu().numpy(),
                    kn[:, b:b + 1, h:h + 1].cpu().numpy(), vn[:, b:b + 1, h:h + 1].cpu().numpy(),
                    q[b:b + 1, h * hpg:(h + 1) * hpg].cpu().numpy()))
    del k, v, kn, vn
    return out


def _oracle_unit_cache(w, key_norm=False):
    import oracle
    if w.scheme == kvq.KVQ_SCHEME_INNERQ:
        return oracle.InnerQCache(w.bits, w.group, w.residual, w.sinks, 1, 1, w.head_dim, key_norm=key_norm)
    if w.sinks:
        return oracle.KiviSinkCache(w.bits, w.group, w.residual, w.sinks, 1, 1, w.head_dim, w.v_policy, w.meta)
    return oracle.QuantizedKVCache(w.bits, w.group, w.residual, 1, 1, w.head_dim, w.v_policy, w.meta)


def _unit_attn_bytes(w, ref):
    hpg = w.num_q_heads // w.num_kv_heads
    unit_w = w.scaled(batch=1, num_kv_heads=1, num_q_heads=hpg)
    if w.scheme == kvq.KVQ_SCHEME_INNERQ:
        return attn_bytes(unit_w, ref.n, ref.nq, ref.nq)
    return attn_bytes(unit_w, ref.n, ref.nq_k, ref.nq_v)


def _oracle_attention_worker(w, items, budget_s, key_norm=False):
    """Oracle decode-attention calls (dequantize + float64 attention) on the
    given units, one thread (BLAS included), swept until budget_s seconds of
    timed work: (bytes, seconds, calls)."""
    import oracle
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        refs = []
        for k, v, kn, vn, q in items:
            ref = _oracle_unit_cache(w, key_norm)
            ref.prefill(k, v)
            ref.append(kn[0], vn[0])
            refs.append((ref, q, _unit_attn_bytes(w, ref)))
        t_total, done, nbytes = 0.0, 0, 0
        while t_total < budget_s:
            for ref, q, nb in refs:
                t0 = time.perf_counter()
                K, V = ref.dequantized()
                oracle.attention(q, K, V, 1.0 / math.sqrt(w.head_dim))
                t_total += time.perf_counter() - t0
                done += 1
                nbytes += nb
                if t_total >= budget_s:
                    break
    return nbytes, t_total, done


def host_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def host_cores(limit=16):
    """Cores this process may run on, capped at the host share of one GPU."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, limit))


def cpu_baseline(w, sample, budget_s=10.0, pool_budget_s=6.0):
    """The oracle timed on this host, on sampled units of the workload:
    decode-attention calls (dequantize + float64 attention) on one thread and
    in a process pool over the host cores (one BLAS thread per worker), each
    scaled by the algorithmic byte formula; and one oracle prefill and one
    flushing append per sampled unit (one thread), scaled to all units."""
    import multiprocessing as mp
    from threadpoolctl import threadpool_limits
    import oracle  # noqa: F401  (the oracle is the baseline being timed)

    key_norm = KEY_NORM["on"] and w.scheme == kvq.KVQ_SCHEME_INNERQ
    one = _oracle_attention_worker(w, sample, budget_s, key_norm)
    cores = min(host_cores(), len(sample))
    shards = [sample[i::cores] for i in range(cores)]
    with mp.get_context("spawn").Pool(cores) as pool:
        res = pool.starmap(_oracle_attention_worker, [(w, sh, pool_budget_s, key_norm) for sh in shards])
    pool_bytes = sum(r[0] for r in res)
    pool_s = max(r[1] for r in res)
    pool_calls = sum(r[2] for r in res)

    # one prefill and one flushing append per sampled unit, one thread
    nunits = min(len(sample), 8)
    t_pre = t_fl = 0.0
    with threadpool_limits(limits=1):
        for k, v, kn, vn, q in sample[:nunits]:
            ref = _oracle_unit_cache(w, key_norm)
            t0 = time.perf_counter()
            ref.prefill(k, v)
            t_pre += time.perf_counter() - t0
            # bring the residual to R - 1 tokens, then time the append that quantizes
            if w.scheme == kvq.KVQ_SCHEME_INNERQ:
                need = 0
            else:
                need = (w.residual - 1) - (ref.n - ref.nq_k)
            for i in range(need):
                ref.append(kn[i], vn[i])
            q0 = ref.nq if w.scheme == kvq.KVQ_SCHEME_INNERQ else ref.nq_k
            t0 = time.perf_counter()
            ref.append(kn[-1], vn[-1])
            t_fl += time.perf_counter() - t0
            assert (ref.nq if w.scheme == kvq.KVQ_SCHEME_INNERQ else ref.nq_k) > q0
    pre_s = t_pre / nunits * w.units
    fl_s = t_fl / nunits * w.units
    pb, fb = prefill_bytes(w, w.context), flush_bytes(w)
    return {"value": round(pool_bytes / pool_s / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "host": host_model(),
            "sample": f"decode-attention calls (dequantize + float64 attention) of the NumPy oracle on {len(sample)} "
                      f"of {w.units} (batch, kv head) units at n={w.context + 1}, same fp16 inputs as the GPU "
                      f"caches: {pool_calls} unit-calls in a pool of {cores} processes (one BLAS thread each) "
                      f"over {pool_s:.1f} s, scaled by the algorithmic byte formula",
            "single_thread": {"value": round(one[0] / one[1] / 1e9, 4), "unit": "GB/s", "cores": 1,
                              "calls": one[2], "seconds": round(one[1], 2),
                              "seconds_per_call_extrapolated": round(one[1] / one[2] * w.units, 3)},
            "pool_seconds_per_call_extrapolated": round(pool_s / pool_calls * cores * w.units / cores, 3),
            "prefill": {"seconds_extrapolated": round(pre_s, 3), "bytes": pb,
                        "GB/s": round(pb / pre_s / 1e9, 4), "cores": 1,
                        "sample": f"oracle prefill of {w.context} tokens on {nunits} units, scaled to {w.units}"},
            "flush": {"seconds_extrapolated": round(fl_s, 4), "bytes": fb, "GB/s": round(fb / fl_s / 1e9, 4),
                      "cores": 1,
                      "sample": f"oracle append that quantizes, on {nunits} units, scaled to {w.units}"}}


def one_launch_step(w, c):
    """Whether kvq_decode_step on cache c (before the step) is one launch:
    the new token is not a sink, no key group is quantized (KIVI), the
    chunked residual's rings are aligned, and a token leaving a FIFO value
    queue or the InnerQ window was quantized ahead by the previous step."""
    st = c.c
    n1, R = st.n_tokens + 1, w.residual
    iq = w.scheme == kvq.KVQ_SCHEME_INNERQ
    fifo = iq or w.v_policy == kvq.KVQ_V_FIFO
    if st.n_tokens < w.sinks:
        return False
    if not iq and (n1 - st.nq_k >= R or (not fifo and st.nq_k != st.nq_v)):
        return False
    return not (fifo and n1 - st.nq_v > R and st.prequant != st.nq_v + 1)


def ahead_bytes(w):
    """Bytes of quantizing one leaving token ahead, all units: the fp16 row(s)
    read, codes and metadata written (KIVI: the value row; InnerQ: key and
    value rows)."""
    d, b, G = w.head_dim, w.bits, w.group
    mb = 4 if w.meta else 6
    per_row = d * 2 + d * b // 8 + (d // G) * mb
    return w.units * per_row * (2 if w.scheme == kvq.KVQ_SCHEME_INNERQ else 1)


def prefill_bytes(w, L):
    """Bytes a prefill of L tokens must move: fp16 K and V in; codes,
    metadata and the fp16 rows kept (sinks, residual or window) out."""
    d, b, G, R = w.head_dim, w.bits, w.group, w.residual
    if w.scheme == kvq.KVQ_SCHEME_INNERQ:
        m = max(0, L - w.sinks - R)
        out = m * 2 * (d * b // 8 + (d // G) * 6) + (L - m) * d * 2 * 2
    else:
        ns = min(L, w.sinks)
        inner = L - ns
        nq_k = inner - inner % R                                   # quantized keys after the sinks
        nq_v = nq_k if w.v_policy == kvq.KVQ_V_CHUNK else max(0, inner - R)
        mb = 4 if w.meta else 6
        out = (nq_k * d * b // 8 + (nq_k // G) * d * mb + nq_v * d * b // 8 + nq_v * (d // G) * mb
               + ((L - nq_k) + (L - nq_v)) * d * 2)
    return w.units * (L * d * 2 * 2 + out)


def flush_bytes(w):
    """Bytes of the append that quantizes (the bench times it with the key
    residual at R - 1 tokens).  KIVI, chunked values: the R keys and values
    (R - 1 ring slots and the new token) in, their codes and metadata out;
    no ring slot is written.  KIVI, FIFO values: the R keys and the popped
    value row in, their codes and metadata out, the new value into its ring
    slot (the new key is one of the R).  InnerQ: the token leaving the window
    and the new token in, the old one's codes and metadata and the new one's
    ring slot out."""
    d, b, G, R = w.head_dim, w.bits, w.group, w.residual
    if w.scheme == kvq.KVQ_SCHEME_INNERQ:
        return w.units * (2 * d * 2 + 2 * (d * b // 8 + (d // G) * 6) + 2 * d * 2 + 2 * d * 2)
    mb = 4 if w.meta else 6
    keys = R * d * 2 + R * d * b // 8 + (R // G) * d * mb
    if w.v_policy == kvq.KVQ_V_CHUNK:
        return w.units * (keys + R * d * 2 + R * d * b // 8 + R * (d // G) * mb)
    return w.units * (keys + d * 2 + d * b // 8 + (d // G) * mb + d * 2 + d * 2)


def time_prefill_and_flush(w, dev, stream, reps=5):
    """HIP-event timing of one prefill (layer-0 prompt) and of one append that
    flushes the residual, on a scratch cache of the same shape."""
    L = w.context
    k, v = gen_prefill(w, 0, dev)
    cap = ((L + 2 * w.residual) // w.residual) * w.residual
    c = kvq.KVCache(make_cfg(w, cap), dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    times = []
    for _ in range(reps + 1):
        c.c.started, c.c.n_tokens, c.c.nq_k, c.c.nq_v = 0, 0, 0, 0
        e0.record(stream)
        c.prefill(k, v, stream.cuda_stream)
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3)
    pre_us = sorted(times[1:])[len(times[1:]) // 2]
    # bring the residual to R - 1 tokens, then time the append that flushes
    # (InnerQ: the window is full after a long prefill, every append quantizes)
    kn, vn = gen_new_tokens(w, 0, dev, steps=w.residual)
    need = 0 if w.scheme == kvq.KVQ_SCHEME_INNERQ else (w.residual - 1) - (c.n_tokens - c.nq_k)
    for i in range(need):
        c.append(kn[i], vn[i], stream.cuda_stream)
    # (the rewind restores every host field, the quantize-ahead record too)
    state = (c.c.n_tokens, c.c.nq_k, c.c.nq_v, c.c.flushes, c.c.prequant)
    times = []
    for _ in range(reps + 1):
        c.c.n_tokens, c.c.nq_k, c.c.nq_v, c.c.flushes, c.c.prequant = state
        e0.record(stream)
        c.append(kn[-1], vn[-1], stream.cuda_stream)
        e1.record(stream)
        torch.cuda.synchronize()
        assert c.flushes == state[3] + 1
        times.append(e0.elapsed_time(e1) * 1e3)
    fl_us = sorted(times[1:])[len(times[1:]) // 2]
    pb, fb = prefill_bytes(w, L), flush_bytes(w)
    del k, v, c   # kept in torch's cache: freeing them would slow the reads timed next
    return {"prefill": {"us": round(pre_us, 1), "bytes": pb, "GB/s": round(pb / pre_us / 1e3, 1),
                        "frac": round(pb / pre_us / 1e3 / HBM_PEAK_GBS, 4), "tokens": L},
            "flush": {"us": round(fl_us, 2), "bytes": fb, "GB/s": round(fb / fl_us / 1e3, 1),
                      "frac": round(fb / fl_us / 1e3 / HBM_PEAK_GBS, 4),
                      "per_appended_token_us": round(fl_us / (1 if w.scheme else w.residual), 3)}}


def source_digest():
    """Content digests of the sources behind the numbers: one sha256 over the
    library, binding, bench and workload sources, and the git blob id (sha1 of
    "blob <size>\\0" + content) of each kernel source, which matches
    `git ls-tree` of the commit the tree came from."""
    import hashlib
    names = []
    for sub in ("decode_attention_token_amd/csrc", "include"):
        d = os.path.join(ROOT, sub)
        names += [os.path.join(sub, f) for f in sorted(os.listdir(d)) if not f.startswith(".")]
    names += ["decode_attention_token_amd/__init__.py", "bench.py", "workloads/__init__.py"]
    h = hashlib.sha256()
    blobs = {}
    for n in names:
        with open(os.path.join(ROOT, n), "rb") as f:
            data = f.read()
        h.update(n.encode() + b"\0" + data)
        if n.startswith("decode_attention_token_amd/csrc"):
            blobs[os.path.basename(n)] = hashlib.sha1(b"blob %d\0" % len(data) + data).hexdigest()
    sha = None
    try:
        import subprocess
        sha = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True, text=True,
                             timeout=10).stdout.strip() or None
    except Exception:
        sha = None
    return {"sha256": h.hexdigest()[:16], "git_head": sha, "kernel_blobs": blobs}


def tiny_latency(dev, stream, steps=20):
    """Per-step latency of the tiny workload (batch 1, one head, context 256):
    decode steps timed one at a time with HIP events; launch-bound, so it is
    reported as a latency, not against a roofline."""
    from workloads import TINY
    w = TINY
    cap = ((w.context + steps + 2 + w.residual - 1) // w.residual) * w.residual
    cfg = make_cfg(w, cap)
    k, v = gen_prefill(w, 0, dev)
    kn, vn = gen_new_tokens(w, 0, dev, steps=steps + 2)
    q = gen_queries(w, 0, dev, steps=steps + 2)
    c = kvq.KVCache(cfg, dev)
    c.prefill(k, v, stream.cuda_stream)
    ws = c.workspace(cap)
    out = torch.empty(w.batch, w.num_q_heads, w.head_dim, dtype=torch.float32, device=dev)
    sp = stream.cuda_stream
    scale = 1.0 / math.sqrt(w.head_dim)
    times = []
    for i in range(steps + 2):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        c.step(kn[i], vn[i], q[i], scale, out, ws, 0, sp)
        e1.record(stream)
        torch.cuda.synchronize()
        if i >= 2:
            times.append(e0.elapsed_time(e1) * 1e3)
    times.sort()
    return {"workload": w.name, "us_per_step_median": round(times[len(times) // 2], 2),
            "us_per_step_min": round(times[0], 2), "steps": steps,
            "note": "one kvq_decode_step per step (append + attention), HIP events around each step"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=LLAMA7B_2BIT.config_id,
                    help="workload id (2 = Llama-2-7B layer shape, 2-bit)")
    ap.add_argument("--layers", type=int, default=None)
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--reps", type=int, default=4, help="attention-only passes for kernel timing")
    ap.add_argument("--settle", type=float, default=0.5,
                    help="seconds of untimed back-to-back attention calls before timing")
    ap.add_argument("--no-side", action="store_true", help="skip the prefill, flush and tiny-workload timings")
    ap.add_argument("--v-policy", choices=("chunk", "fifo"), default=None,
                    help="override the workload's value-residual policy (KIVI scheme)")
    ap.add_argument("--sinks", type=int, default=None, help="override the workload's fp16 sink tokens")
    ap.add_argument("--meta", choices=("f32", "f16"), default=None,
                    help="group metadata: fp32 scale + int16 zero, or a packed fp16 scale | zero word (KIVI)")
    ap.add_argument("--schedule", choices=("fixed", "queue"), default="fixed",
                    help="matrix-core kernel work order: fixed (bit-identical reruns) or the work queue")
    ap.add_argument("--kernel", choices=("auto", "valu"), default="auto",
                    help="four query heads per kv head: matrix cores (auto) or the vector-ALU kernel")
    ap.add_argument("--key-norm", action="store_true",
                    help="InnerQ scheme: scale keys once per channel at prefill, folded into the query")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 256 MiB device copy (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(2)
    w = WORKLOADS[args.workload]
    if args.v_policy is not None:
        w = w.scaled(v_policy=0 if args.v_policy == "chunk" else 1)
    if args.sinks is not None:
        w = w.scaled(sinks=args.sinks)
    if args.meta is not None:
        w = w.scaled(meta=0 if args.meta == "f32" else 1, name=w.name + ("-meta16" if args.meta == "f16" else ""))
    if args.key_norm and w.scheme == kvq.KVQ_SCHEME_INNERQ:
        KEY_NORM["on"] = True
        w = w.scaled(name=w.name + "-keynorm")
    schedule = kvq.KVQ_SCHED_QUEUE if args.schedule == "queue" else kvq.KVQ_SCHED_FIXED
    kernel = kvq.KVQ_KERNEL_VALU if args.kernel == "valu" else kvq.KVQ_KERNEL_AUTO
    steps = w.steps if args.steps is None else args.steps
    layers = w.layers if args.layers is None else args.layers
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    need = w.context + args.warmup + steps
    max_tokens = ((need + w.residual - 1) // w.residual) * w.residual
    sample = None
    if not args.no_cpu:
        sample = host_sample(w, sample_units(w), dev)
    print(f"# workload {w.name}: prefill {layers} layer caches", file=sys.stderr, flush=True)
    cfg, caches = build_caches(w, layers, max_tokens, dev, schedule, kernel)
    total = args.warmup + steps
    news = [gen_new_tokens(w, layer, dev, steps=total) for layer in range(layers)]
    qs = [gen_queries(w, layer, dev, steps=total) for layer in range(layers)]
    outs = [torch.empty(w.batch, w.num_q_heads, w.head_dim, dtype=torch.float32, device=dev)
            for _ in range(layers)]
    ws = caches[0].workspace(max_tokens, args.splits)
    scale = 1.0 / math.sqrt(w.head_dim)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def step(i, count_bytes):
        nb = 0
        for layer in range(layers):
            c = caches[layer]
            kn, vn = news[layer]
            c.step(kn[i], vn[i], qs[layer][i], scale, outs[layer], ws, args.splits, sp)
            if count_bytes:
                nb += attn_bytes(w, c.n_tokens, c.nq_k, c.nq_v)
        return nb

    # Steady state: the device's clocks ramp under sustained load (and for up
    # to 0.6 s after large buffers are returned to the driver, which the bench
    # avoids, reads run about 6% slower), so before anything is timed the
    # attention kernel runs back to back (untimed) for at least settle_s.
    last = total - 1

    def attention_pass():
        calls, cb, fb = 0, 0, 0
        for layer in range(layers):
            c = caches[layer]
            c.attention(qs[layer][last], scale, outs[layer], ws, args.splits, sp)
            calls += 1
            cb += attn_bytes(w, c.n_tokens, c.nq_k, c.nq_v)
            fb += w.units * c.n_tokens * w.head_dim * 2 * 2 + w.batch * w.num_q_heads * w.head_dim * 6
        return calls, cb, fb

    print("# settle", file=sys.stderr, flush=True)
    t_settle = time.perf_counter()
    settle_calls = 0
    while time.perf_counter() - t_settle < args.settle:
        settle_calls += attention_pass()[0]
        torch.cuda.synchronize()
    settle_s = time.perf_counter() - t_settle

    def timed_attention(reps):
        """Attention-only passes over the layers, HIP events on the library's stream."""
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        calls, cb, fb = 0, 0, 0
        ev0.record(stream)
        for _ in range(reps):
            c_, b_, f_ = attention_pass()
            calls, cb, fb = calls + c_, cb + b_, fb + f_
        ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) * 1e3 / calls, cb / calls, fb / calls, calls

    print("# kernel timing", file=sys.stderr, flush=True)
    n_before = caches[0].n_tokens
    call_us, call_bytes, fp16_bytes, calls = timed_attention(args.reps)

    print("# warmup", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    print("# timed loop", file=sys.stderr, flush=True)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    flushed, single, ahead, step_bytes = [], [], [], []
    t0 = time.perf_counter()
    nbytes = 0
    for k, i in enumerate(range(args.warmup, total)):
        evs[k].record(stream)
        f0 = caches[0].flushes
        single.append(one_launch_step(w, caches[0]))
        nb = step(i, True)
        nbytes += nb
        step_bytes.append(nb)
        flushed.append(caches[0].flushes != f0)
        ahead.append(caches[0].c.prequant != 0)
    evs[steps].record(stream)
    t_enq = time.perf_counter() - t0   # host time to enqueue the loop
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    step_us = [evs[k].elapsed_time(evs[k + 1]) * 1e3 for k in range(steps)]
    plain = [k for k in range(steps) if single[k]]
    # the timed loop's launches: one fused append + attention launch per layer
    # and step when no key group is quantized; its bytes add the new token's
    # ring stores and, when the step quantizes the next leaving token ahead,
    # that row's read and quantized write
    fused_us = sum(step_us[k] for k in plain) / (len(plain) * layers) if plain else None
    fused_bytes = (sum(step_bytes[k] + layers * ahead_bytes(w) * ahead[k] for k in plain) / (len(plain) * layers)
                   + w.units * w.head_dim * 2 * 2 if plain else None)

    # the same attention-only passes again after the loop (drift check)
    after_us, after_bytes, _, _ = timed_attention(args.reps)
    att_gbs = call_bytes / (call_us * 1e-6) / 1e9

    side = time_prefill_and_flush(w, dev, stream) if not args.no_side else None
    tiny = tiny_latency(dev, stream) if not args.no_side else None
    ceiling = stream_ceiling(dev, stream)

    if args.copy_probe:
        # a plain elementwise kernel of known traffic: reads and writes 256 MiB
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    # a decode step is one launch unless it quantizes a key group (or the
    # token that leaves the queue or window was not quantized ahead)
    one_launch = bool(plain) and len(plain) == steps
    if fused_us is not None:
        roof_us, roof_bytes, roof_launch = fused_us, fused_bytes, "fused decode step (kvq_decode_step)"
    else:
        roof_us, roof_bytes, roof_launch = call_us, call_bytes, "attention only (kvq_decode_attention)"
    achieved = roof_bytes / (roof_us * 1e-6) / 1e9
    splits_used = args.splits or kvq.kvq_auto_splits(cfg, caches[0].n_tokens)
    res = {
        "metric": METRIC,
        "value": round(nbytes / dt / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(dt / steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "tokens_per_s": round(w.batch * steps / dt, 1),
        "hbm_peak_frac": round(nbytes / dt / 1e9 / HBM_PEAK_GBS, 4),
        "config": {"workload": w.name, "batch": w.batch, "q_heads": w.num_q_heads,
                   "kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "context": w.context,
                   "bits": w.bits, "group": w.group, "residual": w.residual, "layers": layers,
                   "splits": splits_used, "codes": f"u{w.bits}", "v_policy": "chunk" if w.v_policy == 0 else "fifo",
                   "scheme": "innerq" if w.scheme == kvq.KVQ_SCHEME_INNERQ else "kivi", "sinks": w.sinks,
                   "meta": "f16-packed" if w.meta else "f32+i16", "schedule": args.schedule,
                   "key_norm": bool(KEY_NORM["on"]),
                   "kernel": KERNELS[kernel_key(w, kernel)][0]},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(w, kernel),
                     "kernel": KERNELS[kernel_key(w, kernel)][0], "launch": roof_launch,
                     "avg_launch_us": round(roof_us, 2), "bytes_per_launch": int(roof_bytes),
                     "launches": (len(plain) * layers) if roof_us is fused_us else calls},
        "attention_only": {"avg_call_us": round(call_us, 2), "bytes_per_call": int(call_bytes),
                           "GB/s": round(att_gbs, 1), "frac": round(att_gbs / HBM_PEAK_GBS, 4), "calls": calls,
                           "n_tokens": n_before,
                           "after_loop": {"avg_call_us": round(after_us, 2), "bytes_per_call": int(after_bytes),
                                          "n_tokens": caches[0].n_tokens}},
        "settle": {"seconds": round(settle_s, 3), "attention_calls": settle_calls,
                   "note": "untimed back-to-back attention calls before any timing (clocks reach steady state)"},
        "host_enqueue_us_per_launch": round(t_enq / (steps * layers) * 1e6, 2),
        "loop_steps_with_flush": int(sum(flushed)),
        "loop_steps_single_launch": len(plain),
        "loop_step_us": {"median": round(sorted(step_us)[len(step_us) // 2], 1), "min": round(min(step_us), 1),
                         "max": round(max(step_us), 1), "first": [round(t, 1) for t in step_us[:8]],
                         "launches_per_step": layers if one_launch else None},
        # what an fp16 cache of the same tokens would move per call, over the
        # same call time: a compression view, not a roofline fraction
        "fp16_equivalent": {"GB/s": round(fp16_bytes / (call_us * 1e-6) / 1e9, 1),
                            "bytes_per_call": int(fp16_bytes)},
        # the library's plain streaming-read kernel over 4 GiB on this device:
        # the achievable read rate, for context beside the 8 TB/s peak
        "stream_ceiling": {"GB/s": round(ceiling, 1), "frac_of_peak": round(ceiling / HBM_PEAK_GBS, 4),
                           "roofline_frac_of_ceiling": round(achieved / ceiling, 4)},
        "source": source_digest(),
    }
    if side is not None:
        res.update(side)
        res["tiny"] = tiny
    if not args.no_cpu:
        print("# cpu baseline (oracle)", file=sys.stderr, flush=True)
        del caches, news, qs
        torch.cuda.empty_cache()
        res["cpu_baseline"] = cpu_baseline(w, sample)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
