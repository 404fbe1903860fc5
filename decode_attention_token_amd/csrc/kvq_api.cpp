// Host side of libkvq: argument validation, buffer layout, host counters and
// stream-ordered kernel launches.  See include/kvq.h for the contract.
//
// KIVI cache state machine (KIVI part of the juejin.cn page "大模型量化技术原理：
// KIVI、IntactKV、KVQuant", how it works; pgsm.cn KV-cache quantization
// article, 3.1): the key cache is split into a grouped part of nq_k tokens
// (a multiple of G, here also of R) and an fp16 remainder of n - nq_k < R
// tokens; a new key joins the remainder, and when the remainder holds R
// tokens it is quantized, appended and emptied in the same call.  Values use
// the same chunked rule, or a FIFO queue of the R most recent tokens.  The
// InnerQ-style state machine is described at innerq_prefill below.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "../../include/kvq.h"
#include "kvq_internal.h"
#include "kvq_api_internal.h"

namespace {

thread_local char g_err[512] = "";

kvq_status fail(kvq_status s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

bool is_innerq(const kvq_config *c) { return c->scheme == KVQ_SCHEME_INNERQ; }

kvq_status check_config(const kvq_config *c) {
  if (!c) return fail(KVQ_ERR_ARG, "config is null");
  if (c->scheme != KVQ_SCHEME_KIVI && c->scheme != KVQ_SCHEME_INNERQ) return fail(KVQ_ERR_ARG, "unknown scheme");
  const bool iq = is_innerq(c);
  if (c->bits != 2 && c->bits != 4) return fail(KVQ_ERR_ARG, "bits must be 2 or 4 (got %d)", c->bits);
  if (c->group <= 0) return fail(KVQ_ERR_ARG, "group must be positive");
  if (c->residual <= 0) return fail(KVQ_ERR_ARG, "residual must be positive");
  if (!iq && c->residual % c->group)
    return fail(KVQ_ERR_ARG, "residual (%d) must be a positive multiple of group (%d)", c->residual, c->group);
  if (c->head_dim <= 0 || c->head_dim % c->group)
    return fail(KVQ_ERR_ARG, "head_dim (%d) must be a multiple of group (%d)", c->head_dim, c->group);
  if ((c->group * c->bits) % 32) return fail(KVQ_ERR_ARG, "group * bits must be a multiple of 32");
  if (c->batch <= 0 || c->num_kv_heads <= 0 || c->num_q_heads <= 0)
    return fail(KVQ_ERR_ARG, "batch and head counts must be positive");
  if (c->num_q_heads % c->num_kv_heads) return fail(KVQ_ERR_ARG, "num_q_heads must be a multiple of num_kv_heads");
  if (c->max_tokens <= 0) return fail(KVQ_ERR_ARG, "max_tokens must be positive");
  if (!iq && c->max_tokens % c->residual)
    return fail(KVQ_ERR_ARG, "max_tokens (%d) must be a positive multiple of residual (%d)", c->max_tokens,
                c->residual);
  if (c->v_policy != KVQ_V_CHUNK && c->v_policy != KVQ_V_FIFO) return fail(KVQ_ERR_ARG, "unknown v_policy");
  if (c->sink_tokens < 0) return fail(KVQ_ERR_ARG, "sink_tokens must be non-negative");
  if (c->meta_format != KVQ_META_F32 && c->meta_format != KVQ_META_F16) return fail(KVQ_ERR_ARG, "unknown meta_format");
  if (c->schedule != KVQ_SCHED_FIXED && c->schedule != KVQ_SCHED_QUEUE) return fail(KVQ_ERR_ARG, "unknown schedule");
  if (c->kernel != KVQ_KERNEL_AUTO && c->kernel != KVQ_KERNEL_VALU) return fail(KVQ_ERR_ARG, "unknown kernel");
  if (c->key_norm != KVQ_KEYNORM_NONE && c->key_norm != KVQ_KEYNORM_PROMPT) return fail(KVQ_ERR_ARG, "unknown key_norm");
  if (!iq && c->key_norm != KVQ_KEYNORM_NONE)
    return fail(KVQ_ERR_UNSUPPORTED, "key normalization is implemented for the InnerQ scheme only");
  if (iq && c->meta_format != KVQ_META_F32)
    return fail(KVQ_ERR_UNSUPPORTED, "compressed metadata is implemented for the KIVI scheme only");
  if (iq && c->v_policy != KVQ_V_FIFO) return fail(KVQ_ERR_ARG, "the InnerQ scheme keeps a FIFO window (v_policy 1)");
  if (c->sink_tokens > 512) return fail(KVQ_ERR_UNSUPPORTED, "more than 512 sink tokens is not implemented");
  if (c->max_tokens > kvq::kMaxTokens) return fail(KVQ_ERR_UNSUPPORTED, "max_tokens above 2^25 is not implemented");
  if (c->head_dim != kvq::kHeadDim) return fail(KVQ_ERR_UNSUPPORTED, "only head_dim 128 is implemented");
  if (c->group != 32 && c->group != 64 && c->group != 128)
    return fail(KVQ_ERR_UNSUPPORTED, "only group 32, 64 or 128 is implemented");
  const int hpg = c->num_q_heads / c->num_kv_heads;
  if (hpg != 1 && hpg != 2 && hpg != 4)
    return fail(KVQ_ERR_UNSUPPORTED, "only 1, 2 or 4 query heads per kv head are implemented");
  if (c->residual > 512) return fail(KVQ_ERR_UNSUPPORTED, "residual above 512 is not implemented");
  if ((int64_t)c->batch * c->num_kv_heads > 65535) return fail(KVQ_ERR_UNSUPPORTED, "more than 65535 units");
  if ((int64_t)c->batch * c->num_q_heads > 2147483647LL) return fail(KVQ_ERR_UNSUPPORTED, "too many query heads");
  return KVQ_OK;
}

kvq_status check_cache(const kvq_config *c, const kvq_cache *k) {
  if (!k) return fail(KVQ_ERR_ARG, "cache is null");
  const bool zeros = c->meta_format == KVQ_META_F32;   // separate zero-point buffers
  if (!k->k_codes || !k->k_scale || !k->v_codes || !k->v_scale || !k->k_resid || !k->v_resid ||
      (zeros && (!k->k_zero || !k->v_zero)))
    return fail(KVQ_ERR_ARG, "a cache buffer pointer is null");
  if (c->sink_tokens > 0 && (!k->k_sink || !k->v_sink)) return fail(KVQ_ERR_ARG, "a sink buffer pointer is null");
  if (c->key_norm != KVQ_KEYNORM_NONE && !k->k_norm) return fail(KVQ_ERR_ARG, "the k_norm buffer pointer is null");
  return KVQ_OK;
}

kvq::CacheView view_of(const kvq_config *c, const kvq_cache *k) {
  kvq::CacheView v;
  v.k_codes = k->k_codes;
  v.k_scale = k->k_scale;
  v.k_zero = k->k_zero;
  v.v_codes = k->v_codes;
  v.v_scale = k->v_scale;
  v.v_zero = k->v_zero;
  v.k_resid = k->k_resid;
  v.v_resid = k->v_resid;
  v.k_sink = k->k_sink;
  v.v_sink = k->v_sink;
  v.cap = c->max_tokens;
  v.bits = c->bits;
  v.group = c->group;
  v.residual = c->residual;
  v.sinks = c->sink_tokens;
  v.meta = c->meta_format;
  v.k_norm = c->key_norm != KVQ_KEYNORM_NONE ? k->k_norm : nullptr;
  return v;
}

kvq_status device_error(hipError_t e, const char *what) {
  return fail(KVQ_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

// Compute units of the current device (queried once per device).
hipError_t compute_units(int *out) {
  static std::atomic<int> cached[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < 64 && cached[dev].load() > 0) {
    *out = cached[dev].load();
    return hipSuccess;
  }
  int n = 0;
  e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (n < 1) n = 1;
  if (dev >= 0 && dev < 64) cached[dev].store(n);
  *out = n;
  return hipSuccess;
}

int64_t main_tokens(const kvq_config *c, const kvq_cache *k) {
  const int64_t m = k->nq_k < k->nq_v ? k->nq_k : k->nq_v;
  return (m / c->group) * c->group;
}

// Splits for `nq` quantized tokens per unit: aim for two 8-wave workgroups
// per compute unit of a 256-CU part, but keep at least 512 tokens (KIVI:
// sixteen key groups, two per wave) in every split.
int32_t auto_splits_for(const kvq_config *c, int64_t nq) {
  const int64_t units = (int64_t)c->batch * c->num_kv_heads;
  int64_t s = (512 + units - 1) / units;   // 512 workgroups: two per CU
  const int64_t by_work = is_innerq(c) ? nq / 512 : nq / c->group / 16;
  if (s > by_work) s = by_work;
  if (s < 1) s = 1;
  if (s > kvq::kMaxSplits) s = kvq::kMaxSplits;
  return (int32_t)s;
}

// Workspace: per-unit work-queue counters (zero between calls), then fp32
// partial (acc[128], max, sum) records, one per query head and split.
size_t workspace_for(const kvq_config *c, int32_t splits) {
  return kvq::counter_bytes((int64_t)c->batch * c->num_kv_heads) +
         (size_t)c->batch * c->num_q_heads * (size_t)splits * kvq::kPartialStride * sizeof(float);
}

// cfg->schedule: KVQ_SCHED_FIXED (default) makes the matrix-core kernel
// hand super-chunks to waves in a fixed order, so reruns are bit-identical;
// KVQ_SCHED_QUEUE lets waves take them from a work queue, which only changes
// the order of fp32 partial sums from run to run.
// Epoch of a launch: tags the per-unit election words, so a word an earlier
// launch left behind never counts toward this one (zero is never used).
uint32_t next_epoch() {
  static std::atomic<uint32_t> counter{0};
  uint32_t e;
  do {
    e = counter.fetch_add(1, std::memory_order_relaxed) + 1;
  } while (e == 0);
  return e;
}

void set_workspace(kvq::AttnArgs &a, const kvq_config *c, void *workspace) {
  a.epoch = next_epoch();
  a.dynamic = c->schedule == KVQ_SCHED_QUEUE ? 1 : 0;
  a.mfma = c->kernel == KVQ_KERNEL_AUTO ? 1 : 0;
  a.ctr = static_cast<uint32_t *>(workspace);
  a.partials = reinterpret_cast<float *>(static_cast<char *>(workspace) +
                                         kvq::counter_bytes((int64_t)c->batch * c->num_kv_heads));
}

// InnerQ-style state (euno.news InnerQ summary, methodology 4): tokens
// t < sinks are kept fp16 in the sink rows; later tokens enter a FIFO window
// of at most R fp16 tokens (ring slot t mod R) whose oldest token is
// quantized into row nq once a push would make it exceed R; tokens
// [sinks, nq) are quantized.  While n <= sinks, nq == n.
kvq_status innerq_prefill(const kvq_config *cfg, kvq_cache *cache, const uint16_t *k, const uint16_t *v,
                          int64_t len, hipStream_t stream) {
  const int R = cfg->residual, S = cfg->sink_tokens;
  const int units = cfg->batch * cfg->num_kv_heads;
  const kvq::CacheView cv = view_of(cfg, cache);
  const int64_t ns = len < S ? len : S;
  const int64_t r = len > S ? (len - S < R ? len - S : R) : 0;
  const int64_t nq = len - r;
  hipError_t e;
  if (cv.k_norm != nullptr) {
    // the per-channel key scales from every prompt token, before any key is quantized
    e = kvq::launch_key_norm(cache->k_norm, units, k, len, stream);
    if (e != hipSuccess) return device_error(e, "key channel scales");
  }
  e = kvq::launch_copy_rows(cv.k_sink, cv.v_sink, S, k, v, len, 0, (int)ns, 0, units, stream);
  if (e != hipSuccess) return device_error(e, "copy sink tokens");
  if (nq > ns) {
    e = kvq::launch_innerq_quantize(cv, units, k, v, len, ns, (int)(nq - ns), ns, stream);
    if (e != hipSuccess) return device_error(e, "quantize prompt");
  }
  e = kvq::launch_copy_rows(cv.k_resid, cv.v_resid, R, k, v, len, nq, (int)r, (int)(nq % R), units, stream);
  if (e != hipSuccess) return device_error(e, "copy window tokens");
  cache->n_tokens = len;
  cache->nq_k = cache->nq_v = nq;
  cache->started = 1;
  cache->flushes = 0;
  cache->prequant = 0;
  return KVQ_OK;
}

kvq_status innerq_append(const kvq_config *cfg, kvq_cache *cache, const uint16_t *k_new, const uint16_t *v_new,
                         hipStream_t stream) {
  const int R = cfg->residual, S = cfg->sink_tokens;
  const int units = cfg->batch * cfg->num_kv_heads;
  const int64_t n = cache->n_tokens, nq = cache->nq_k;
  const bool to_sink = n < S;
  const bool pop = !to_sink && n - nq == R;
  // a decode step may have quantized the leaving token's rows already
  const bool ready = cache->prequant == nq + 1;
  const hipError_t e = kvq::launch_innerq_append(view_of(cfg, cache), units, k_new, v_new,
                                                 (pop && !ready) ? nq : -1, to_sink, (int)(to_sink ? n : n % R),
                                                 stream);
  if (e != hipSuccess) return device_error(e, "append");
  cache->n_tokens = n + 1;
  cache->prequant = 0;
  if (to_sink) {
    cache->nq_k = cache->nq_v = n + 1;
  } else if (pop) {
    cache->nq_k = cache->nq_v = nq + 1;
    cache->flushes += 1;
  }
  return KVQ_OK;
}

}  // namespace

extern "C" {

kvq_status kvq_layout_bytes(const kvq_config *cfg, kvq_layout *out) {
  kvq_status s = check_config(cfg);
  if (s != KVQ_OK) return s;
  if (!out) return fail(KVQ_ERR_ARG, "layout output is null");
  const size_t units = (size_t)cfg->batch * cfg->num_kv_heads;
  const size_t cap = (size_t)cfg->max_tokens;
  const size_t d = (size_t)cfg->head_dim;
  const size_t words = d * cfg->bits / 32;
  const size_t G = (size_t)cfg->group;
  out->k_codes = units * cap * words * 4;
  if (is_innerq(cfg)) {
    out->k_scale = units * cap * (d / G) * 4;
    out->k_zero = units * cap * (d / G) * 2;
  } else {
    out->k_scale = units * (cap / G) * d * 4;
    out->k_zero = units * (cap / G) * d * 2;
  }
  out->v_codes = units * cap * words * 4;
  out->v_scale = units * cap * (d / G) * 4;
  out->v_zero = units * cap * (d / G) * 2;
  if (cfg->meta_format == KVQ_META_F16) out->k_zero = out->v_zero = 0;   // packed into *_scale
  out->k_resid = units * (size_t)cfg->residual * d * 2;
  out->v_resid = out->k_resid;
  out->k_sink = units * (size_t)cfg->sink_tokens * d * 2;
  out->v_sink = out->k_sink;
  out->k_norm = cfg->key_norm != KVQ_KEYNORM_NONE ? units * d * 4 : 0;
  g_err[0] = 0;
  return KVQ_OK;
}

int32_t kvq_auto_splits(const kvq_config *cfg, int64_t n_tokens) {
  if (check_config(cfg) != KVQ_OK || n_tokens < 0) return 0;
  // an upper bound of the quantized tokens keeps this a pure function of the
  // length: KIVI covers whole key groups of the grouped part, InnerQ the
  // tokens after the sinks
  const int64_t nq = is_innerq(cfg) ? (n_tokens > cfg->sink_tokens ? n_tokens - cfg->sink_tokens : 0)
                                    : n_tokens - (n_tokens % cfg->residual);
  return auto_splits_for(cfg, nq);
}

size_t kvq_workspace_bytes(const kvq_config *cfg, int64_t n_tokens, int32_t splits) {
  if (check_config(cfg) != KVQ_OK || splits < 0 || splits > kvq::kMaxSplits) return 0;
  if (splits == 0) splits = kvq_auto_splits(cfg, n_tokens);
  return workspace_for(cfg, splits);
}

kvq_status kvq_quantize_prefill(const kvq_config *cfg, kvq_cache *cache, const uint16_t *k, const uint16_t *v,
                                int64_t len, hipStream_t stream) {
  kvq_status s = check_config(cfg);
  if (s != KVQ_OK) return s;
  if ((s = check_cache(cfg, cache)) != KVQ_OK) return s;
  if (cache->started) return fail(KVQ_ERR_STATE, "prefill on a cache that already holds tokens");
  if (len < 0) return fail(KVQ_ERR_ARG, "negative length");
  if (len > cfg->max_tokens) return fail(KVQ_ERR_CAPACITY, "len %lld exceeds max_tokens %d", (long long)len,
                                         cfg->max_tokens);
  if (len > 0 && (!k || !v)) return fail(KVQ_ERR_ARG, "k or v is null");
  if (is_innerq(cfg)) {
    s = innerq_prefill(cfg, cache, k, v, len, stream);
    if (s == KVQ_OK) g_err[0] = 0;
    return s;
  }
  const int R = cfg->residual, G = cfg->group;
  const int units = cfg->batch * cfg->num_kv_heads;
  const kvq::CacheView cv = view_of(cfg, cache);
  // sink tokens [0, ns) stay fp16; the KIVI rules apply to the L tokens after
  // them (row and ring indices count from the first token after the sinks)
  const int64_t ns = len < cfg->sink_tokens ? len : cfg->sink_tokens;
  const int64_t L = len - ns;
  const int64_t nq_k = L - (L % R);
  const int64_t nq_v = (cfg->v_policy == KVQ_V_CHUNK) ? nq_k : (L > R ? L - R : 0);
  hipError_t e = kvq::launch_copy_rows(cv.k_sink, cv.v_sink, cfg->sink_tokens, k, v, len, 0, (int)ns, 0, units,
                                       stream);
  if (e != hipSuccess) return device_error(e, "copy sink tokens");
  if (nq_k > 0 || nq_v > 0) {
    e = kvq::launch_quantize_kv(cv, units, k, v, len, ns, (int)(nq_k / G), (int)nq_v, stream);
    if (e != hipSuccess) return device_error(e, "quantize keys and values");
  }
  if (L > nq_k) {
    e = kvq::launch_copy_to_residual(cv, units, k, nullptr, len, ns + nq_k, (int)(L - nq_k), (int)(nq_k % R), true,
                                     false, stream);
    if (e != hipSuccess) return device_error(e, "copy key residual");
  }
  if (L > nq_v) {
    e = kvq::launch_copy_to_residual(cv, units, nullptr, v, len, ns + nq_v, (int)(L - nq_v), (int)(nq_v % R), false,
                                     true, stream);
    if (e != hipSuccess) return device_error(e, "copy value residual");
  }
  cache->n_tokens = len;
  cache->nq_k = ns + nq_k;
  cache->nq_v = ns + nq_v;
  cache->started = 1;
  cache->flushes = 0;
  cache->prequant = 0;
  g_err[0] = 0;
  return KVQ_OK;
}

kvq_status kvq_append_token(const kvq_config *cfg, kvq_cache *cache, const uint16_t *k_new,
                            const uint16_t *v_new, hipStream_t stream) {
  kvq_status s = check_config(cfg);
  if (s != KVQ_OK) return s;
  if ((s = check_cache(cfg, cache)) != KVQ_OK) return s;
  if (!cache->started) return fail(KVQ_ERR_STATE, "append before prefill");
  if (!k_new || !v_new) return fail(KVQ_ERR_ARG, "k_new or v_new is null");
  if (cache->n_tokens >= cfg->max_tokens) return fail(KVQ_ERR_CAPACITY, "cache is full (%d tokens)", cfg->max_tokens);
  if (is_innerq(cfg)) {
    s = innerq_append(cfg, cache, k_new, v_new, stream);
    if (s == KVQ_OK) g_err[0] = 0;
    return s;
  }
  const int R = cfg->residual, G = cfg->group;
  const int units = cfg->batch * cfg->num_kv_heads;
  const kvq::CacheView cv = view_of(cfg, cache);
  const int S = cfg->sink_tokens;
  hipError_t e;
  if (cache->n_tokens < S) {
    // still filling the sink tokens
    e = kvq::launch_copy_rows(cv.k_sink, cv.v_sink, S, k_new, v_new, 1, 0, 1, (int)cache->n_tokens, units, stream);
    if (e != hipSuccess) return device_error(e, "append sink token");
    cache->n_tokens += 1;
    cache->nq_k = cache->nq_v = cache->n_tokens;
    g_err[0] = 0;
    return KVQ_OK;
  }
  // counters of the token stream after the sinks
  int64_t n = cache->n_tokens - S, nq_k = cache->nq_k - S, nq_v = cache->nq_v - S;
  int32_t flushes = cache->flushes;
  // FIFO: the value queue would exceed R, so quantize its oldest entry before
  // its ring slot (the same slot the new token takes) is overwritten
  if (cfg->v_policy == KVQ_V_FIFO && (n + 1) - nq_v > R) {
    // (unless a decode step has quantized that row already)
    if (cache->prequant != S + nq_v + 1) {
      e = kvq::launch_quantize_values(cv, units, cache->v_resid, R, nq_v % R, 1, nq_v, stream);
      if (e != hipSuccess) return device_error(e, "quantize popped value");
    }
    nq_v += 1;
  }
  cache->prequant = 0;
  if (cfg->v_policy == KVQ_V_CHUNK && (n + 1) - nq_k == R && nq_v == nq_k) {
    // both rings fill with this token: one launch quantizes them, reading the
    // new token from k_new / v_new; no ring slot is live afterwards
    e = kvq::launch_flush(cv, units, k_new, v_new, (int)(n % R), nq_k / G, nq_v, stream);
    if (e != hipSuccess) return device_error(e, "flush");
    cache->n_tokens = S + n + 1;
    cache->nq_k = cache->nq_v = S + n + 1;
    cache->flushes = flushes + 1;
    g_err[0] = 0;
    return KVQ_OK;
  }
  e = kvq::launch_copy_to_residual(cv, units, k_new, v_new, 1, 0, 1, (int)(n % R), true, true, stream);
  if (e != hipSuccess) return device_error(e, "append to residual");
  n += 1;
  if (n - nq_k == R) {
    // the key residual holds R tokens, slots 0..R-1 in token order
    e = kvq::launch_quantize_keys(cv, units, cache->k_resid, R, 0, R / G, nq_k / G, stream);
    if (e != hipSuccess) return device_error(e, "flush keys");
    nq_k += R;
    flushes += 1;
  }
  if (cfg->v_policy == KVQ_V_CHUNK && n - nq_v == R) {
    e = kvq::launch_quantize_values(cv, units, cache->v_resid, R, 0, R, nq_v, stream);
    if (e != hipSuccess) return device_error(e, "flush values");
    nq_v += R;
  }
  cache->n_tokens = S + n;
  cache->nq_k = S + nq_k;
  cache->nq_v = S + nq_v;
  cache->flushes = flushes;
  g_err[0] = 0;
  return KVQ_OK;
}

}  // extern "C"

namespace {

kvq_status check_attention_args(const kvq_config *cfg, const kvq_cache *cache, const uint16_t *q, float *out,
                                void *workspace, int32_t splits, float softmax_scale) {
  kvq_status s = check_config(cfg);
  if (s != KVQ_OK) return s;
  if ((s = check_cache(cfg, cache)) != KVQ_OK) return s;
  if (!cache->started) return fail(KVQ_ERR_STATE, "attention before prefill");
  if (!q || !out || !workspace) return fail(KVQ_ERR_ARG, "q, out or workspace is null");
  if (splits < 0 || splits > kvq::kMaxSplits) return fail(KVQ_ERR_ARG, "splits must be in [0, %d]", kvq::kMaxSplits);
  if (!std::isfinite(softmax_scale)) return fail(KVQ_ERR_ARG, "softmax_scale must be finite");
  return KVQ_OK;
}

// Enqueues attention over a cache of n_tokens tokens; with k_new/v_new the
// last token is taken from them and stored into its residual slot.
kvq_status launch_innerq_attention(const kvq_config *cfg, const kvq_cache *cache, const uint16_t *k_new,
                                   const uint16_t *v_new, const uint16_t *q, float softmax_scale, float *out,
                                   void *workspace, size_t workspace_bytes, int32_t splits, int64_t prequant,
                                   hipStream_t stream) {
  const int64_t n = cache->n_tokens;
  const int64_t first = n < cfg->sink_tokens ? n : cfg->sink_tokens;
  if (splits == 0) splits = auto_splits_for(cfg, cache->nq_k - first);
  const size_t need = workspace_for(cfg, splits);
  if (workspace_bytes < need)
    return fail(KVQ_ERR_CAPACITY, "workspace of %zu bytes is below the %zu needed", workspace_bytes, need);
  kvq::AttnArgs a;
  a.c = view_of(cfg, cache);
  a.q = q;
  a.out = out;
  set_workspace(a, cfg, workspace);
  a.batch = cfg->batch;
  a.hq = cfg->num_q_heads;
  a.hkv = cfg->num_kv_heads;
  a.n = n;
  a.nq_k = a.nq_v = cache->nq_k;
  a.n_main = cache->nq_k;
  a.splits = splits;
  // wave order, as for the KIVI kernel: every eighth 16-token step when a
  // wave's contiguous share would span more than 32 KiB of key codes (1%
  // faster on the 4-bit cache of 131072 tokens, 256 KiB per wave)
  const int64_t wave_bytes = (cache->nq_k - first) / splits / 8 * (cfg->head_dim * cfg->bits / 8);
  a.interleave = wave_bytes > 32 * 1024 ? 1 : 0;
  a.resid_main = 1;
  a.nparts = splits;
  a.qscale = softmax_scale * 1.4426950408889634f;
  a.k_new = k_new;
  a.v_new = v_new;
  a.prequant = prequant;
  a.early = splits;
  a.nsink = 0;   // the InnerQ kernel derives its sinks from n and the config
  const hipError_t e = kvq::launch_innerq_attention(a, stream);
  if (e != hipSuccess) return device_error(e, "decode attention");
  return KVQ_OK;
}

// prequant: token (whole-stream index) whose quantized row(s) the launch
// writes ahead of its pop, or -1.
kvq_status launch_attention(const kvq_config *cfg, const kvq_cache *cache, int64_t n_tokens, const uint16_t *k_new,
                            const uint16_t *v_new, const uint16_t *q, float softmax_scale, float *out,
                            void *workspace, size_t workspace_bytes, int32_t splits, int64_t prequant,
                            hipStream_t stream) {
  if (is_innerq(cfg))
    return launch_innerq_attention(cfg, cache, k_new, v_new, q, softmax_scale, out, workspace, workspace_bytes,
                                   splits, prequant, stream);
  // sink tokens [0, ns) are fp16; everything else is indexed from the first
  // token after them
  const int64_t ns = n_tokens < cfg->sink_tokens ? n_tokens : cfg->sink_tokens;
  const int64_t nq_k = cache->nq_k - ns, nq_v = cache->nq_v - ns;
  n_tokens -= ns;
  const int64_t m = nq_k < nq_v ? nq_k : nq_v;
  const int64_t n_main = (m / cfg->group) * cfg->group;
  if (splits == 0) splits = auto_splits_for(cfg, n_main);
  const size_t need = workspace_for(cfg, splits);
  if (workspace_bytes < need)
    return fail(KVQ_ERR_CAPACITY, "workspace of %zu bytes is below the %zu needed", workspace_bytes, need);
  kvq::AttnArgs a;
  a.c = view_of(cfg, cache);
  a.q = q;
  a.out = out;
  set_workspace(a, cfg, workspace);
  a.batch = cfg->batch;
  a.hq = cfg->num_q_heads;
  a.hkv = cfg->num_kv_heads;
  a.n = n_tokens;
  a.nq_k = nq_k;
  a.nq_v = nq_v;
  a.n_main = n_main;
  a.nsink = (int)ns;
  // tokens [n_main, n) and the sink tokens go to the last split, which reads
  // each token's key and value quantized or fp16 (a FIFO value queue leaves
  // keys quantized whose values are still fp16)
  const bool has_rest = n_tokens > n_main;
  a.resid_main = has_rest ? 1 : 0;
  a.splits = n_main > 0 ? splits : ((a.resid_main || ns > 0) ? 1 : 0);
  a.nparts = a.splits;
  // Wave order of the vector-ALU kernel: when a wave's contiguous share of
  // its split would span more than 32 KiB of key codes, its waves take
  // every eighth key group instead (measured: 3.6% faster on a 4-bit cache
  // of 8192 tokens, 64 KiB per wave; 1.5% slower on a 2-bit cache of 4096
  // tokens, 16 KiB per wave).
  const int64_t wave_span = (a.splits > 0 ? n_main / a.splits : 0) / 8 * (cfg->head_dim * cfg->bits / 8);
  a.interleave = wave_span > 32 * 1024 ? 1 : 0;
  a.qscale = softmax_scale * 1.4426950408889634f;
  a.k_new = k_new;
  a.v_new = v_new;
  a.prequant = prequant >= 0 ? prequant - ns : -1;
  int cus = 0;
  hipError_t e = compute_units(&cus);
  if (e != hipSuccess) return device_error(e, "device attributes");
  const int units = cfg->batch * cfg->num_kv_heads;
  a.early = cus / units;
  if (a.early < 1 || a.early > a.splits) a.early = a.splits;
  e = kvq::launch_decode_attention(a, stream);
  if (e != hipSuccess) return device_error(e, "decode attention");
  return KVQ_OK;
}

}  // namespace

namespace kvq {

kvq_status report(kvq_status s, const char *msg) { return fail(s, "%s", msg); }

kvq_status decode_attention_into(const kvq_config *cfg, const kvq_cache *cache, const uint16_t *q,
                                 float softmax_scale, float *out, void *workspace, size_t workspace_bytes,
                                 int32_t splits, hipStream_t stream) {
  kvq_status s = check_attention_args(cfg, cache, q, out, workspace, splits, softmax_scale);
  if (s != KVQ_OK) return s;
  if (cache->n_tokens < 1) return fail(KVQ_ERR_STATE, "attention over an empty cache");
  s = launch_attention(cfg, cache, cache->n_tokens, nullptr, nullptr, q, softmax_scale, out, workspace,
                       workspace_bytes, splits, -1, stream);
  if (s == KVQ_OK) g_err[0] = 0;
  return s;
}

}  // namespace kvq

extern "C" {

kvq_status kvq_decode_attention(const kvq_config *cfg, const kvq_cache *cache, const uint16_t *q,
                                float softmax_scale, float *out, void *workspace, size_t workspace_bytes,
                                int32_t splits, hipStream_t stream) {
  return kvq::decode_attention_into(cfg, cache, q, softmax_scale, out, workspace, workspace_bytes, splits, stream);
}

kvq_status kvq_decode_step(const kvq_config *cfg, kvq_cache *cache, const uint16_t *k_new, const uint16_t *v_new,
                           const uint16_t *q, float softmax_scale, float *out, void *workspace,
                           size_t workspace_bytes, int32_t splits, hipStream_t stream) {
  kvq_status s = check_attention_args(cfg, cache, q, out, workspace, splits, softmax_scale);
  if (s != KVQ_OK) return s;
  if (!k_new || !v_new) return fail(KVQ_ERR_ARG, "k_new or v_new is null");
  if (cache->n_tokens >= cfg->max_tokens) return fail(KVQ_ERR_CAPACITY, "cache is full (%d tokens)", cfg->max_tokens);
  const int R = cfg->residual, S = cfg->sink_tokens;
  const int64_t n1 = cache->n_tokens + 1;
  const size_t need = workspace_for(cfg, splits == 0 ? kvq_auto_splits(cfg, n1) : splits);
  if (workspace_bytes < need)
    return fail(KVQ_ERR_CAPACITY, "workspace of %zu bytes is below the %zu needed", workspace_bytes, need);
  // The attention launch also takes the new token from k_new / v_new and
  // stores it into its ring slots when the new token is not a sink and (KIVI)
  // the append quantizes no key group.  A token that leaves a FIFO value
  // queue or the InnerQ window is quantized ahead: the step that fills the
  // queue or window has its attention launch write the oldest token's
  // quantized rows (cache->prequant records which), so in steady state a
  // step is one launch.  Without that, one small launch quantizes it first.
  // Otherwise the two calls in sequence.
  const bool iq = is_innerq(cfg);
  const bool fifo = iq || cfg->v_policy == KVQ_V_FIFO;
  const bool fused = cache->n_tokens >= S &&
                     (iq || ((fifo || cache->nq_k == cache->nq_v) && n1 - cache->nq_k < R));
  if (!fused) {
    s = kvq_append_token(cfg, cache, k_new, v_new, stream);
    if (s != KVQ_OK) return s;
    return kvq_decode_attention(cfg, cache, q, softmax_scale, out, workspace, workspace_bytes, splits, stream);
  }
  const int units = cfg->batch * cfg->num_kv_heads;
  const kvq::CacheView cv = view_of(cfg, cache);
  int64_t nq_k = cache->nq_k, nq_v = cache->nq_v;
  int32_t flushes = cache->flushes;
  if (fifo && n1 - nq_v > R) {
    // the oldest fp16 value (InnerQ: token) leaves
    if (cache->prequant != nq_v + 1) {
      const hipError_t e = iq ? kvq::launch_innerq_append(cv, units, nullptr, nullptr, nq_v, false, 0, stream)
                              : kvq::launch_quantize_values(cv, units, cache->v_resid, R, (nq_v - S) % R, 1, nq_v - S,
                                                            stream);
      if (e != hipSuccess) return device_error(e, "quantize the token leaving the residual");
    }
    nq_v += 1;
    if (iq) {
      nq_k = nq_v;
      flushes += 1;
    }
  }
  // after this step the queue or window is full: its oldest token leaves at
  // the next append (the ring slot differs from the new token's, R >= 2)
  const int64_t pre = (fifo && R >= 2 && n1 - nq_v == R) ? nq_v : -1;
  kvq_cache next = *cache;
  next.n_tokens = n1;
  next.nq_k = nq_k;
  next.nq_v = nq_v;
  s = launch_attention(cfg, &next, n1, k_new, v_new, q, softmax_scale, out, workspace, workspace_bytes, splits, pre,
                       stream);
  if (s != KVQ_OK) return s;
  cache->nq_k = nq_k;
  cache->nq_v = nq_v;
  cache->flushes = flushes;
  cache->prequant = pre >= 0 ? pre + 1 : 0;
  cache->n_tokens = n1;
  g_err[0] = 0;
  return KVQ_OK;
}

kvq_status kvq_stream_read_probe(const void *buf, size_t bytes, uint32_t *out, hipStream_t stream) {
  if (!buf || !out) return fail(KVQ_ERR_ARG, "buf or out is null");
  if (bytes == 0 || bytes % 16 || reinterpret_cast<uintptr_t>(buf) % 16)
    return fail(KVQ_ERR_ARG, "probe buffer must be 16-byte aligned and a non-zero multiple of 16 bytes");
  const hipError_t e = kvq::launch_stream_read(buf, bytes, out, stream);
  if (e != hipSuccess) return device_error(e, "stream-read probe");
  g_err[0] = 0;
  return KVQ_OK;
}

const char *kvq_status_string(kvq_status s) {
  switch (s) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_ARG: return "invalid argument";
    case KVQ_ERR_CAPACITY: return "capacity exceeded";
    case KVQ_ERR_STATE: return "invalid cache state";
    case KVQ_ERR_DEVICE: return "device error";
    case KVQ_ERR_UNSUPPORTED: return "unsupported configuration";
  }
  return "unknown status";
}

const char *kvq_last_error(void) { return g_err; }

}  // extern "C"
