"""Decode-attention benchmark on one MI355X.

A step is one decode step of the whole batch through every layer of the
workload: per layer, kvq_decode_step = kvq_append_token (residual write, eager
flush when due) + kvq_decode_attention, one kernel launch when no flush is due.  Caches are prefilled before
timing; inputs for every step are resident in HBM when timing starts.

Prints one JSON line:
  value        effective KV GB/s of the whole timed loop (algorithmic bytes of
               every attention call / loop time)
  tokens_per_s batch * steps / loop time
  roofline     split-kernel bytes per launch / its average duration (HIP
               events on the library's stream), against 8 TB/s
  fp16_equivalent  bytes an fp16 cache of the same tokens would move per
               call / the same call time (labelled; not a roofline fraction)
  stream_ceiling  GB/s of the library's plain streaming-read probe over
               4 GiB, and the roofline's achieved rate as a fraction of it
  cpu_baseline the NumPy oracle's decode-attention call on a sample of units,
               timed on this host, scaled to the same byte formula
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


def stream_ceiling(dev, stream, reps=5):
    """GB/s of kvq_stream_read_probe over a 4 GiB buffer (16x the MALL),
    timed with HIP events on the given stream."""
    buf = torch.ones(4 << 30, dtype=torch.uint8, device=dev)
    out = torch.zeros(1, dtype=torch.int32, device=dev)
    sp = stream.cuda_stream
    for _ in range(2):
        kvq.kvq_stream_read_probe(buf, out, sp)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        kvq.kvq_stream_read_probe(buf, out, sp)
    e1.record(stream)
    torch.cuda.synchronize()
    gbs = buf.numel() * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del buf, out
    torch.cuda.empty_cache()
    return gbs


def make_cfg(w, max_tokens):
    return kvq.make_config(w.bits, w.group, w.residual, w.batch, w.num_q_heads, w.num_kv_heads,
                           w.head_dim, max_tokens, w.v_policy, w.scheme, w.sinks, w.meta)


def build_caches(w, layers, max_tokens, dev):
    cfg = make_cfg(w, max_tokens)
    caches = []
    for layer in range(layers):
        k, v = gen_prefill(w, layer, dev)
        c = kvq.KVCache(cfg, dev)
        c.prefill(k, v)
        torch.cuda.synchronize()
        del k, v
        caches.append(c)
    torch.cuda.empty_cache()
    return cfg, caches


def sample_units(w, count=512, seed=7):
    return [int(u) for u in np.random.default_rng(seed).permutation(w.units)[:count]]


# decode kernel, its source files and its committed counter summary per scheme
KERNELS = {
    0: ("decode_attn_kernel", ("kvq_attn.hip", "kvq_attn_common.h", "kvq_internal.h"),
        "decode_attn_llama2_7b_2bit_traffic.txt"),
    1: ("innerq_attn_kernel", ("kvq_innerq.hip", "kvq_attn_common.h", "kvq_internal.h"),
        "innerq_attn_b4_h32_L131072_4bit_traffic.txt"),
    "gqa4": ("gqa_mfma_kernel", ("kvq_attn_gqa.hip", "kvq_attn_common.h", "kvq_internal.h"),
             "gqa_mfma_b8_q32_kv8_L32768_2bit_traffic.txt"),
}


def kernel_key(w):
    """Which decode kernel dominates the workload: the matrix-core kernel for
    four query heads per kv head (KIVI layout, unless KVQ_GQA_PATH=valu),
    else the scheme's vector-ALU kernel."""
    if (w.scheme == kvq.KVQ_SCHEME_KIVI and w.num_q_heads == 4 * w.num_kv_heads
            and os.environ.get("KVQ_GQA_PATH") != "valu"):
        return "gqa4"
    return w.scheme


def kernel_source_digest(scheme=0):
    import hashlib
    h = hashlib.sha256()
    for name in KERNELS[scheme][1]:
        with open(os.path.join(ROOT, "decode_attention_token_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(w):
    """HBM bytes per launch of the decode kernel from the committed counter
    summary, or None when it is missing, for another workload, or taken on a
    different kernel source."""
    try:
        with open(os.path.join(ROOT, "profiles", KERNELS[kernel_key(w)][2])) as f:
            kv = dict(line.split(":", 1) for line in f if ":" in line and not line.startswith("#"))
    except OSError:
        return None
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    if kv.get("kernel_source_digest") != kernel_source_digest(kernel_key(w)) or kv.get("workload") != w.name:
        return None
    try:
        return int(float(kv["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def host_sample(w, units, dev):
    """Host copies of the sampled units' layer-0 inputs (the same fp16 bits the GPU caches use)."""
    k, v = gen_prefill(w, 0, dev)
    kn, vn = gen_new_tokens(w, 0, dev, steps=1)
    q = gen_queries(w, 0, dev, steps=1)[0]
    hpg = w.num_q_heads // w.num_kv_heads
    out = []
    for u in units:
        b, h = divmod(u, w.num_kv_heads)
        out.append((k[b:b + 1, h:h + 1].cpu().numpy(), v[b:b + 1, h:h + 1].cpu().numpy(),
                    kn[0][b:b + 1, h:h + 1].cpu().numpy(), vn[0][b:b + 1, h:h + 1].cpu().numpy(),
                    q[b:b + 1, h * hpg:(h + 1) * hpg].cpu().numpy()))
    del k, v
    return out


def cpu_baseline(w, sample, budget_s=12.0):
    """The oracle's decode-attention call (dequantize + float64 attention) on
    sampled units, one host thread, scaled by the algorithmic byte formula.
    The sampled units are swept repeatedly until about budget_s seconds of
    timed oracle work have accumulated."""
    import oracle
    hpg = w.num_q_heads // w.num_kv_heads
    unit_w = w.scaled(batch=1, num_kv_heads=1, num_q_heads=hpg)
    refs = []
    for k, v, kn, vn, q in sample:
        if w.scheme == kvq.KVQ_SCHEME_INNERQ:
            ref = oracle.InnerQCache(w.bits, w.group, w.residual, w.sinks, 1, 1, w.head_dim)
        elif w.sinks:
            ref = oracle.KiviSinkCache(w.bits, w.group, w.residual, w.sinks, 1, 1, w.head_dim, w.v_policy, w.meta)
        else:
            ref = oracle.QuantizedKVCache(w.bits, w.group, w.residual, 1, 1, w.head_dim, w.v_policy, w.meta)
        ref.prefill(k, v)
        ref.append(kn, vn)
        refs.append((ref, q))
    t_total, done, nbytes = 0.0, 0, 0
    while t_total < budget_s:
        for ref, q in refs:
            t0 = time.perf_counter()
            K, V = ref.dequantized()
            oracle.attention(q, K, V, 1.0 / math.sqrt(w.head_dim))
            t_total += time.perf_counter() - t0
            done += 1
            nq = ref.nq if w.scheme == kvq.KVQ_SCHEME_INNERQ else ref.nq_k
            nbytes += attn_bytes(unit_w, ref.n, nq, ref.nq if w.scheme == kvq.KVQ_SCHEME_INNERQ else ref.nq_v)
            if t_total >= budget_s:
                break
    return {"value": round(nbytes / t_total / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} unit-calls over {len(refs)} of {w.units} (batch, kv-head) units: one "
                      f"decode-attention call each (dequantize + float64 attention) at n={w.context + 1}, "
                      f"same fp16 inputs as the GPU caches; {t_total:.1f} s on one host thread",
            "seconds_per_call_extrapolated": round(t_total / done * w.units, 3)}


def prefill_bytes(w, L):
    """Bytes a prefill of L tokens must move: fp16 K and V in, codes +
    metadata + fp16 residual (or sinks and window) out."""
    d, b, G, R = w.head_dim, w.bits, w.group, w.residual
    if w.scheme == kvq.KVQ_SCHEME_INNERQ:
        m = max(0, L - w.sinks - R)
        out = m * 2 * (d * b // 8 + (d // G) * 6) + (L - m) * d * 2 * 2
    else:
        ns = min(L, w.sinks)
        nq = (L - ns) - (L - ns) % R    # quantized tokens after the sinks
        mb = 4 if w.meta else 6
        out = nq * d * b // 8 * 2 + (nq // G) * d * mb + nq * (d // G) * mb + (L - nq) * d * 2 * 2
    return w.units * (L * d * 2 * 2 + out)


def flush_bytes(w):
    """Bytes one quantizing append must move (the append's own token write
    included).  KIVI: R fp16 keys and values in, their codes and metadata
    out.  InnerQ: the token leaving the window in, its codes and metadata
    out."""
    d, b, G, R = w.head_dim, w.bits, w.group, w.residual
    if w.scheme == kvq.KVQ_SCHEME_INNERQ:
        return w.units * (d * 2 * 2 + 2 * (d * b // 8 + (d // G) * 6) + d * 2 * 2)
    mb = 4 if w.meta else 6
    return w.units * (R * d * 2 * 2 + R * d * b // 8 * 2 + (R // G) * d * mb + R * (d // G) * mb + d * 2 * 2)


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
    state = (c.c.n_tokens, c.c.nq_k, c.c.nq_v, c.c.flushes)
    times = []
    for _ in range(reps + 1):
        c.c.n_tokens, c.c.nq_k, c.c.nq_v, c.c.flushes = state
        e0.record(stream)
        c.append(kn[-1], vn[-1], stream.cuda_stream)
        e1.record(stream)
        torch.cuda.synchronize()
        assert c.flushes == state[3] + 1
        times.append(e0.elapsed_time(e1) * 1e3)
    fl_us = sorted(times[1:])[len(times[1:]) // 2]
    pb, fb = prefill_bytes(w, L), flush_bytes(w)
    del k, v, c
    torch.cuda.empty_cache()
    return {"prefill": {"us": round(pre_us, 1), "bytes": pb, "GB/s": round(pb / pre_us / 1e3, 1),
                        "frac": round(pb / pre_us / 1e3 / HBM_PEAK_GBS, 4), "tokens": L},
            "flush": {"us": round(fl_us, 2), "bytes": fb, "GB/s": round(fb / fl_us / 1e3, 1),
                      "frac": round(fb / fl_us / 1e3 / HBM_PEAK_GBS, 4),
                      "per_appended_token_us": round(fl_us / (1 if w.scheme else w.residual), 3)}}


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
    ap.add_argument("--no-side", action="store_true", help="skip the prefill and flush timings")
    ap.add_argument("--v-policy", choices=("chunk", "fifo"), default=None,
                    help="override the workload's value-residual policy (KIVI scheme)")
    ap.add_argument("--sinks", type=int, default=None, help="override the workload's fp16 sink tokens")
    ap.add_argument("--meta", choices=("f32", "f16"), default=None,
                    help="group metadata: fp32 scale + int16 zero, or a packed fp16 scale | zero word (KIVI)")
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
    cfg, caches = build_caches(w, layers, max_tokens, dev)
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

    print("# warmup", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    print("# timed loop", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    nbytes = 0
    for i in range(args.warmup, total):
        nbytes += step(i, True)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0

    # attention-only passes, timed with HIP events on the library's stream
    print("# kernel timing", file=sys.stderr, flush=True)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    last = total - 1
    calls, cb, fb = 0, 0, 0
    ev0.record(stream)
    for _ in range(args.reps):
        for layer in range(layers):
            c = caches[layer]
            c.attention(qs[layer][last], scale, outs[layer], ws, args.splits, sp)
            calls += 1
            cb += attn_bytes(w, c.n_tokens, c.nq_k, c.nq_v)
            fb += w.units * c.n_tokens * w.head_dim * 2 * 2 + w.batch * w.num_q_heads * w.head_dim * 6
    ev1.record(stream)
    torch.cuda.synchronize()
    call_us = ev0.elapsed_time(ev1) * 1e3 / calls
    call_bytes = cb / calls
    achieved = call_bytes / (call_us * 1e-6) / 1e9

    side = time_prefill_and_flush(w, dev, stream) if not args.no_side else None
    ceiling = stream_ceiling(dev, stream)

    if args.copy_probe:
        # a plain elementwise kernel of known traffic: reads and writes 256 MiB
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

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
                   "meta": "f16-packed" if w.meta else "f32+i16"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(w),
                     "kernel": KERNELS[kernel_key(w)][0], "avg_call_us": round(call_us, 2),
                     "bytes_per_call": int(call_bytes)},
        # what an fp16 cache of the same tokens would move per call, over the
        # same call time: a compression view, not a roofline fraction
        "fp16_equivalent": {"GB/s": round(fb / calls / (call_us * 1e-6) / 1e9, 1),
                            "bytes_per_call": int(fb / calls)},
        # the library's plain streaming-read kernel over 4 GiB on this device:
        # the achievable read rate, for context beside the 8 TB/s peak
        "stream_ceiling": {"GB/s": round(ceiling, 1), "frac_of_peak": round(ceiling / HBM_PEAK_GBS, 4),
                           "roofline_frac_of_ceiling": round(achieved / ceiling, 4)},
    }
    if side is not None:
        res.update(side)
    if not args.no_cpu:
        print("# cpu baseline (oracle)", file=sys.stderr, flush=True)
        del caches, news, qs
        torch.cuda.empty_cache()
        res["cpu_baseline"] = cpu_baseline(w, sample)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
