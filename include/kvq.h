/*
 * kvq.h - C ABI of libkvq: 2/4-bit quantized KV caches (KIVI-style and
 * InnerQ-style) and decode attention over them, for AMD Instinct MI355X
 * (gfx950).
 *
 * Method sources (web pages, cited by title and section):
 *   [KIVI] juejin.cn, "大模型量化技术原理：KIVI、IntactKV、KVQuant", KIVI part:
 *          background (2-bit asymmetric, keys per channel, values per token),
 *          工作原理 / how it works (grouped part X_Kg = X_K[:l-r] quantized in
 *          groups of G tokens, full-precision remainder X_Kr, flush of X_Kr
 *          once it holds R tokens with R % G == 0, value queue, prefill keeps
 *          only the quantized cache).
 *   [HFQ]  pgsm.cn news 20017, KV-cache quantization article: 2.1 affine map
 *          X_Q = round(X / S) - Z, symmetric vs asymmetric ranges, 2.2 keys
 *          per channel / values per token, 3.1 fp16 residual cache
 *          batch-quantized when full, 4.1 knobs nbits, group_size,
 *          residual_length.
 *   [KVQ]  the same juejin.cn page, KVQuant part, section 五 (attention-sink
 *          aware quantization: the first tokens stay fp16).
 *   [InnerQ] euno.news, "【论文】InnerQ：硬件感知免调优KV缓存量化用于大语言模型",
 *          methodology 1 (groups along the hidden dimension), 2 (per-group
 *          symmetric or asymmetric mode from the group statistics, one shared
 *          scale per group), 4 (recent and sink tokens kept fp16).
 *
 * Conventions
 *   - fp16 tensors are passed as uint16_t bit patterns; every pointer named
 *     "device" is HIP device memory owned by the caller.  The library never
 *     allocates or frees device memory and keeps no global state other than a
 *     thread-local error string and a process-wide launch counter (its value
 *     tags the per-call counters in an attention workspace).
 *   - Every call is stream-ordered on the given hipStream_t and never
 *     synchronizes the device.  The host-side counters in kvq_cache are
 *     updated at enqueue time, so calls on one cache must be serialized by
 *     the caller (one host thread, one stream).
 *   - A call that fails validation returns a non-zero status, enqueues
 *     nothing and leaves kvq_cache unchanged; kvq_last_error() explains why.
 *     A failed kernel launch returns KVQ_ERR_DEVICE; counters are then
 *     undefined and the cache must be rebuilt.
 *   - Only head_dim == 128, bits in {2, 4}, G in {32, 64, 128}, a query to
 *     key head ratio in {1, 2, 4}, residual <= 512, sink_tokens <= 512 and
 *     max_tokens <= 2^25 are implemented; other valid shapes return
 *     KVQ_ERR_UNSUPPORTED.
 *
 * Device layout of one layer's KVQ_SCHEME_KIVI cache (U = batch *
 * num_kv_heads units, unit u = b * num_kv_heads + h; cap = max_tokens;
 * W = head_dim * bits / 32):
 *   k_codes u32 [U][cap][W]        token-major rows; channel c's code sits at
 *                                  bits [(c*bits) % 32, +bits) of word
 *                                  (c*bits) / 32 of the token's row
 *   k_scale f32 [U][cap/G][head_dim]  per (group of G tokens, channel)
 *   k_zero  i16 [U][cap/G][head_dim]
 *   v_codes u32 [U][cap][W]        same row format as keys
 *   v_scale f32 [U][cap][head_dim/G]  per (token, group of G channels)
 *   v_zero  i16 [U][cap][head_dim/G]
 *   k_resid, v_resid f16 [U][R][head_dim]  fp16 residual ring, token t in
 *                                  slot t mod R
 *   Dequantized value of a code: S * (code + Z) (inverse of [HFQ] 2.1).
 *   With sink_tokens = S > 0 ([KVQ]): tokens t < S are kept fp16 in
 *   k_sink, v_sink f16 [U][S][head_dim] (row t), and the rules above apply to
 *   the tokens after them: token t >= S is token t - S of the rows, groups
 *   and ring slots above.
 *
 * Device layout of a KVQ_SCHEME_INNERQ cache: k_codes, v_codes as above;
 *   k_scale, v_scale f32 [U][cap][head_dim/G]  per (token, group of G channels)
 *   k_zero, v_zero   i16 [U][cap][head_dim/G]
 *   k_resid, v_resid f16 [U][R][head_dim]  recent-token window, token t in
 *                                  slot t mod R
 *   k_sink, v_sink   f16 [U][sink_tokens][head_dim]  token t < sink_tokens
 *   k_norm  f32 [U][head_dim]      per-channel key scale (KVQ_KEYNORM_PROMPT)
 *   Quantized tokens are those in [sink_tokens, nq); a symmetric group stores
 *   the signed level k as code k + 2^(bits-1) with Z = -2^(bits-1), so
 *   S * (code + Z) dequantizes both modes.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVQ_OK = 0,
  KVQ_ERR_ARG = 1,          /* invalid argument or null pointer */
  KVQ_ERR_CAPACITY = 2,     /* the call would exceed max_tokens / workspace */
  KVQ_ERR_STATE = 3,        /* prefill on a started cache, append/attend before prefill */
  KVQ_ERR_DEVICE = 4,       /* a HIP launch failed */
  KVQ_ERR_UNSUPPORTED = 5   /* valid but not implemented shape */
} kvq_status;

/* Value-residual policy.  KVQ_V_CHUNK: values flushed as a block of R tokens
 * together with the keys ([HFQ] 3.1).  KVQ_V_FIFO: values kept as a queue of
 * the R most recent tokens; once a push makes it exceed R, the oldest value is
 * quantized and appended ([KIVI] how it works, value queue). */
typedef enum { KVQ_V_CHUNK = 0, KVQ_V_FIFO = 1 } kvq_v_policy;

/* Quantization scheme.
 * KVQ_SCHEME_KIVI: keys per channel over groups of G tokens, values per token
 *   over groups of G channels, asymmetric ([KIVI], [HFQ] 2.2); fp16 residual
 *   of fewer than R tokens (or the R most recent values, KVQ_V_FIFO); the
 *   first sink_tokens tokens optionally kept fp16 ([KVQ]).
 * KVQ_SCHEME_INNERQ: keys and values both per token over groups of G channels
 *   ([InnerQ] methodology 1); each group symmetric when it is centred on zero,
 *   read as |mean| < std / 10 with the population std, else asymmetric
 *   ([InnerQ] methodology 2); the first sink_tokens tokens and the R most
 *   recent tokens stay fp16 ([InnerQ] methodology 4), the recent ones as a
 *   FIFO window whose oldest token is quantized when a push makes it exceed
 *   R.  Requires v_policy == KVQ_V_FIFO. */
typedef enum { KVQ_SCHEME_KIVI = 0, KVQ_SCHEME_INNERQ = 1 } kvq_scheme;

/* Storage of a group's (S, Z).
 * KVQ_META_F32: fp32 scale in *_scale and int16 zero-point in *_zero, 6 bytes.
 * KVQ_META_F16: one 32-bit word per group in *_scale, the fp16 bits of S in
 *   the low half and Z in the high half (4 bytes); *_zero are unused (0
 *   bytes).  S is first replaced by the smallest fp16 value >= S, then Z and
 *   the codes are computed with it, so the group's range still fits the 2^b
 *   levels.  KIVI scheme only. */
typedef enum { KVQ_META_F32 = 0, KVQ_META_F16 = 1 } kvq_meta_format;

/* Order in which the matrix-core kernel (four query heads per kv head) hands
 * its super-chunks (four key groups) to waves.
 * KVQ_SCHED_FIXED (default): a fixed strided order, so reruns on the same
 *   inputs are bit-identical.
 * KVQ_SCHED_QUEUE: each wave takes its next super-chunk from a per-unit
 *   ticket counter in the workspace, which balances waves that run at
 *   different speeds; the order, and so the rounding of the fp32 partial
 *   sums, varies from run to run (results agree to about 1e-6, within 1e-4).
 * The other kernels use a fixed order under both values. */
typedef enum { KVQ_SCHED_FIXED = 0, KVQ_SCHED_QUEUE = 1 } kvq_schedule;

/* Attention kernel family for four query heads per kv head (KIVI scheme).
 * KVQ_KERNEL_AUTO (default): the matrix-core kernel (bf16 MFMA tiles over
 *   the quantized groups).  KVQ_KERNEL_VALU: the vector-ALU kernel every
 *   other head ratio uses (kept for comparison).  Ignored elsewhere. */
typedef enum { KVQ_KERNEL_AUTO = 0, KVQ_KERNEL_VALU = 1 } kvq_kernel;

/* One-time per-channel key normalization ([InnerQ] methodology 4: the key
 * matrix is scaled once per channel at prefill and the scale folded into the
 * query).  KVQ_KEYNORM_NONE (default): keys are quantized as they are.
 * KVQ_KEYNORM_PROMPT (InnerQ scheme only): prefill sets
 *     k_norm[u][c] = smallest power of two >= max(1, max over the prompt's
 *                    keys of unit u of |k[c]|)
 * (one scale per (batch, kv head) and channel, fixed for the life of the
 * cache); every key that is quantized, at prefill or when it leaves the
 * window, is first multiplied by 1 / k_norm and rounded to fp16 (round to
 * nearest even); sink and window keys stay as they are; attention multiplies
 * the query by k_norm for the quantized keys, so the scores are those of the
 * keys in their original units. */
typedef enum { KVQ_KEYNORM_NONE = 0, KVQ_KEYNORM_PROMPT = 1 } kvq_key_norm;

/* Cache configuration: nbits / group_size / residual_length of [HFQ] 4.1
 * plus the attention shape, the scheme and two launch choices (schedule,
 * kernel; zero selects the defaults).  Constraints: bits in {2,4};
 * head_dim % group == 0; group * bits % 32 == 0; num_q_heads % num_kv_heads
 * == 0; residual > 0; max_tokens > 0; sink_tokens >= 0.  KVQ_SCHEME_KIVI
 * also needs residual % group == 0 ([KIVI] how it works) and max_tokens %
 * residual == 0; KVQ_SCHEME_INNERQ needs v_policy == KVQ_V_FIFO and
 * meta_format == KVQ_META_F32. */
typedef struct {
  int32_t bits;
  int32_t group;        /* G */
  int32_t residual;     /* R */
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t max_tokens;   /* capacity per unit, prompt plus generated tokens */
  int32_t v_policy;     /* kvq_v_policy */
  int32_t scheme;       /* kvq_scheme */
  int32_t sink_tokens;  /* leading tokens kept fp16 (both schemes; 0 = none) */
  int32_t meta_format;  /* kvq_meta_format */
  int32_t schedule;     /* kvq_schedule (0 = fixed order, bit-identical reruns) */
  int32_t kernel;       /* kvq_kernel (0 = matrix cores for four query heads per kv head) */
  int32_t key_norm;     /* kvq_key_norm (0 = none) */
} kvq_config;

/* Byte sizes of the caller-allocated device buffers of one cache (k_sink and
 * v_sink are 0 unless sink_tokens > 0; k_zero and v_zero are 0 with
 * KVQ_META_F16; k_norm is 0 unless key_norm is set). */
typedef struct {
  size_t k_codes, k_scale, k_zero, v_codes, v_scale, v_zero, k_resid, v_resid, k_sink, v_sink, k_norm;
} kvq_layout;

/* One layer's cache: caller-owned device buffers (sized by kvq_layout_bytes)
 * and host counters.  Zero-initialize the struct, set the pointers, and leave
 * the counters to the library.  n_tokens = tokens cached; nq_k / nq_v = end of
 * the quantized key / value tokens, which are [sink_tokens, nq) (InnerQ:
 * nq_k == nq_v), with nq == n_tokens while n_tokens <= sink_tokens;
 * started = prefill has run.  k_sink / v_sink may be null when sink_tokens
 * is 0, k_zero / v_zero with KVQ_META_F16 (k_scale / v_scale then hold the
 * packed words). */
typedef struct {
  uint32_t *k_codes;
  float *k_scale;
  int16_t *k_zero;
  uint32_t *v_codes;
  float *v_scale;
  int16_t *v_zero;
  uint16_t *k_resid;
  uint16_t *v_resid;
  uint16_t *k_sink;
  uint16_t *v_sink;
  int64_t n_tokens;
  int64_t nq_k;
  int64_t nq_v;
  int32_t started;
  int32_t flushes;      /* KIVI: key-residual flushes since prefill; InnerQ:
                           appends that quantized a token leaving the window */
  float *k_norm;        /* device f32 [U][head_dim], written by prefill; only
                           with key_norm (may be null otherwise) */
  int64_t prequant;     /* library-owned: 1 + the token whose quantized rows a
                           decode step has already written ahead of its leaving
                           the FIFO value queue (KIVI) or the window (InnerQ);
                           0 = none.  A caller that saves and restores the
                           counters must restore this field with them (or set
                           it to 0, which is always safe) */
} kvq_cache;

/* Validates cfg and fills *out with the buffer sizes.  Host only. */
kvq_status kvq_layout_bytes(const kvq_config *cfg, kvq_layout *out);

/* Split count kvq_decode_attention uses for a cache of n_tokens tokens when
 * it is passed splits == 0.  Host only; returns 0 on an invalid cfg. */
int32_t kvq_auto_splits(const kvq_config *cfg, int64_t n_tokens);

/* Workspace bytes kvq_decode_attention needs for `splits` splits (0 = the
 * automatic count for n_tokens; more tokens never need fewer splits, so the
 * size for max_tokens covers every call): four u32 counter words per (batch,
 * kv head) (a work-queue ticket and a 64-bit election word tagged with the
 * launch), padded to 256 bytes, then fp32 partial (acc[head_dim], max, sum)
 * records for every query head and part.  Host only; 0 on an invalid cfg. */
size_t kvq_workspace_bytes(const kvq_config *cfg, int64_t n_tokens, int32_t splits);

/* Prefill ([KIVI] how it works): k, v are the prompt's keys and values, fp16
 * device [batch][num_kv_heads][len][head_dim], read only (the full-precision
 * tensors stay valid for the caller, as the page's prefill paragraph
 * requires).  Tokens t < sink_tokens go to the sink rows.  KIVI, on the
 * L = len - sinks tokens after them: the first L - (L mod R) are quantized,
 * keys per channel over groups of G tokens and values per token over groups
 * of G channels; the last L mod R go to the residual ring.  With KVQ_V_FIFO
 * the last min(L, R) values stay fp16 instead.  InnerQ: the last
 * min(R, len - sink_tokens) go to the window, the rest are quantized.  Needs
 * a cache with started == 0 and len <= max_tokens; len == 0 is allowed. */
kvq_status kvq_quantize_prefill(const kvq_config *cfg, kvq_cache *cache,
                                const uint16_t *k, const uint16_t *v, int64_t len,
                                hipStream_t stream);

/* One decode step's new key and value, fp16 device [batch][num_kv_heads]
 * [head_dim]; n += 1.  Token n < sink_tokens goes to sink row n.  KIVI,
 * otherwise: written to residual slot (n - sinks) mod R; when the key
 * residual reaches R tokens it is quantized and appended to the grouped part
 * in the same call (eager flush, [KIVI] how it works; [HFQ] 3.1); values
 * follow the cache's kvq_v_policy.  InnerQ, otherwise: when the window
 * already holds R tokens its oldest token (ring slot nq mod R) is quantized
 * into row nq first, and the new token takes ring slot n mod R; one kernel
 * launch.  A value or window token that a decode step has already quantized
 * (cache->prequant) is not quantized again.  Needs started and
 * n < max_tokens. */
kvq_status kvq_append_token(const kvq_config *cfg, kvq_cache *cache,
                            const uint16_t *k_new, const uint16_t *v_new,
                            hipStream_t stream);

/* Decode attention of one query per head over the whole cache, including the
 * token appended in the same step.
 * Defining passages: generating a token reads every cached key and value
 * while the arithmetic units mostly wait, so this call streams the packed
 * cache once ([KIVI] background); the group's shared scale is loaded once and
 * dequantization is fused into the dot products of a GEMV ([InnerQ]
 * methodology 3); the result is the textbook attention of the dequantized
 * cache, which none of the pages prints:
 *     out[b][h] = sum_t p_t V^[t],  p = softmax(softmax_scale * q[b][h] . K^[t]),
 * with K^, V^ = S * (code + Z) for quantized tokens ([HFQ] 2.1, inverted) and
 * the stored fp16 values for sink, residual and window tokens; no mask.
 * Arguments:
 *   q        fp16 device [batch][num_q_heads][head_dim], read only; query head
 *            h uses key head h / (num_q_heads / num_kv_heads).
 *   softmax_scale  finite; 1/sqrt(head_dim) for the textbook scaling.
 *   out      fp32 device [batch][num_q_heads][head_dim], written.
 *   workspace  device, at least kvq_workspace_bytes(cfg, n_tokens, splits)
 *            bytes, zero-filled once before its first use.  Its leading bytes
 *            hold per-(batch, kv head) counters that every call leaves at
 *            zero again; the rest is scratch for split records.  An election
 *            word left non-zero by an earlier, interrupted call is ignored
 *            (it carries another launch's tag); a work-queue ticket that did
 *            not start at zero makes that call write NaN for the affected
 *            units instead of a wrong number, and the call returns it to
 *            zero.  Calls that share a workspace must be ordered on one
 *            stream: overlapping calls race on it.
 *   splits   0 = automatic (kvq_auto_splits), else 1..64 parts per unit.
 * One kernel launch when every unit fits one part, else a second (merge)
 * launch, except for the matrix-core kernel (four query heads per kv head)
 * and the InnerQ kernel, which merge inside their one launch; cfg->schedule
 * and cfg->kernel choose the matrix-core kernel's work order and whether it
 * runs at all.  Needs started and n_tokens >= 1; KVQ_ERR_CAPACITY for a
 * workspace below the size needed; never synchronizes. */
kvq_status kvq_decode_attention(const kvq_config *cfg, const kvq_cache *cache,
                                const uint16_t *q, float softmax_scale, float *out,
                                void *workspace, size_t workspace_bytes, int32_t splits,
                                hipStream_t stream);

/* Size in bytes of the device array kvq_decode_attention_static uses in place
 * of a workspace (one copy per GPU, held until the process ends). */
#define KVQ_STATIC_SCRATCH_BYTES (16u << 20)

/* kvq_decode_attention without a workspace argument, for callers that cannot
 * allocate device memory (code under stream capture, tight serving loops,
 * harnesses that forbid allocation): the per-unit counters and split records
 * live in a file-scope device array of KVQ_STATIC_SCRATCH_BYTES bytes that the
 * library's code object carries; nothing is allocated or freed at run time.
 * Same arguments, results and requirements as kvq_decode_attention, except:
 * the matrix-core kernel always runs the fixed schedule (cfg->schedule is
 * ignored), so results equal kvq_decode_attention's with KVQ_SCHED_FIXED bit
 * for bit; `stream` must belong to the current device (KVQ_ERR_ARG
 * otherwise); a call whose workspace size (kvq_workspace_bytes for its splits
 * and n_tokens) exceeds KVQ_STATIC_SCRATCH_BYTES returns KVQ_ERR_CAPACITY and
 * enqueues nothing.  Every call on a GPU shares that GPU's array, which keeps
 * the last call's contents; no part of it needs to start at zero.  Calls that
 * overlap on one GPU (other streams, other host threads) race on the array
 * and must be ordered by the caller.  The first call on a device looks up the
 * array's device address (KVQ_ERR_DEVICE if that fails). */
kvq_status kvq_decode_attention_static(const kvq_config *cfg, const kvq_cache *cache, const uint16_t *q,
                                       float softmax_scale, float *out, int32_t splits, hipStream_t stream);

/* One decode step: kvq_append_token(k_new, v_new) followed by
 * kvq_decode_attention(q), with the same cache bytes and bit-identical
 * output.  When the new token is not a sink and (KIVI) the append quantizes
 * no key group, the attention kernel reads the new token from k_new/v_new
 * and stores it into its residual slots: one launch.  A token that leaves a
 * FIFO value queue or the InnerQ window at this append is quantized by that
 * same launch one step ahead: a step after which the queue or window is
 * full also writes the quantized rows of its oldest token (recorded in
 * cache->prequant), so the next step, or the next kvq_append_token, only
 * advances the counters; without that record one small launch quantizes it
 * first.  Otherwise the two calls run in sequence.  Arguments and
 * requirements are those of the two calls; on a validation failure
 * (including a workspace below kvq_workspace_bytes for the split count used)
 * nothing is enqueued and the cache is unchanged. */
kvq_status kvq_decode_step(const kvq_config *cfg, kvq_cache *cache, const uint16_t *k_new,
                           const uint16_t *v_new, const uint16_t *q, float softmax_scale, float *out,
                           void *workspace, size_t workspace_bytes, int32_t splits, hipStream_t stream);

/* Measurement only, not part of the attention path: reads `bytes` of device
 * memory at buf (16-byte aligned, bytes a non-zero multiple of 16) with a
 * plain streaming kernel, so a caller can time the device's achievable HBM
 * read rate and compare the decode kernels' bandwidth with it as well as
 * with the specification's peak.  out: device, one u32 the kernel writes
 * only in a case a buffer of ones never produces (it keeps the loads live).
 * KVQ_ERR_ARG for a null pointer, misalignment or a bad size; stream-ordered,
 * never synchronizes. */
kvq_status kvq_stream_read_probe(const void *buf, size_t bytes, uint32_t *out, hipStream_t stream);

/* Static description of a status code. */
const char *kvq_status_string(kvq_status s);

/* Thread-local text of the last failure on this thread ("" if none). */
const char *kvq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
