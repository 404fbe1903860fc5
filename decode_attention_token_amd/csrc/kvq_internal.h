// Internal launch interface between the C ABI (kvq_api.cpp) and the HIP
// kernels (kvq_quant.hip, kvq_attn.hip).  Not part of the public ABI.
#pragma once

#include <stdint.h>
#include <hip/hip_runtime_api.h>

namespace kvq {

constexpr int kHeadDim = 128;
constexpr int kMaxSplits = 64;
// Largest accepted max_tokens.  With 4-bit codes a unit's code buffer is then
// 2^25 * 64 = 2^31 bytes, the largest buffer resource a kernel builds.
constexpr int kMaxTokens = 1 << 25;
constexpr int kPartialStride = kHeadDim + 4;   // acc[128], m, l, pad, pad (floats)
// Workspace: per-unit counters (kCtrWords u32 each: the work-queue ticket,
// a pad word and a 64-bit election word), padded to 256 bytes, then the
// partial records.
constexpr int kCtrWords = 4;
inline size_t counter_bytes(int64_t units) { return (size_t)((units * kCtrWords * 4 + 255) / 256 * 256); }

struct CacheView {
  uint32_t *k_codes;
  float *k_scale;
  int16_t *k_zero;
  uint32_t *v_codes;
  float *v_scale;
  int16_t *v_zero;
  uint16_t *k_resid;
  uint16_t *v_resid;
  uint16_t *k_sink;   // InnerQ-style layout: fp16 sink rows [unit][sinks][128]
  uint16_t *v_sink;
  int64_t cap;      // max_tokens
  int bits, group, residual;
  int sinks;        // sink tokens kept fp16 (0 = none)
  int meta;         // 0: fp32 scale + int16 zero; 1: packed fp16 scale | zero << 16 in *_scale
  const float *k_norm;   // InnerQ key channel scales [unit][128] (powers of two), or null
};

// Quantize `ngroups` key groups per unit.  Source rows: src + (unit * src_rows
// + src_row0 + i) * 128 for token i of the block; destination group index
// dst_group0 + g.
hipError_t launch_quantize_keys(const CacheView &c, int units, const uint16_t *src,
                                int64_t src_rows, int64_t src_row0, int ngroups,
                                int64_t dst_group0, hipStream_t s);

// Quantize `count` value rows per unit (source row src_row0 + i) into
// destination token rows dst_row0 + i.
// Chunked residual flush of both rings in one launch: the R ring slots in
// token order, ring slot `slot` read from k_new / v_new ([unit][128]) instead
// (the token the same append brings), keys into group dst_group0 and values
// into row dst_row0 of every unit.  The ring slots are left as they are.
hipError_t launch_flush(const CacheView &c, int units, const uint16_t *k_new, const uint16_t *v_new, int slot,
                        int64_t dst_group0, int64_t dst_row0, hipStream_t s);

hipError_t launch_quantize_values(const CacheView &c, int units, const uint16_t *src,
                                  int64_t src_rows, int64_t src_row0, int count,
                                  int64_t dst_row0, hipStream_t s);

// A prefill's quantization: `ngroups` key groups per unit (into groups 0 ..)
// and `count` value rows per unit (into rows 0 ..), both from source rows
// src_row0 + i of [unit][src_rows][128] fp16; one launch at G = 32, the two
// quantizer launches otherwise.
hipError_t launch_quantize_kv(const CacheView &c, int units, const uint16_t *ksrc, const uint16_t *vsrc,
                              int64_t src_rows, int64_t src_row0, int ngroups, int count, hipStream_t s);

// Copy rows [row0, row0 + count) of src ([unit][src_rows][128] fp16) into
// residual slots slot0 + i of both rings (keys from ksrc, values from vsrc).
hipError_t launch_copy_to_residual(const CacheView &c, int units, const uint16_t *ksrc,
                                   const uint16_t *vsrc, int64_t src_rows, int64_t row0,
                                   int count, int slot0, bool keys, bool values, hipStream_t s);

// Copy rows [row0, row0 + count) of ksrc / vsrc ([unit][src_rows][128] fp16)
// into rows (slot0 + i) mod dst_rows of kdst / vdst ([unit][dst_rows][128]);
// a null destination is skipped.
hipError_t launch_copy_rows(uint16_t *kdst, uint16_t *vdst, int dst_rows, const uint16_t *ksrc,
                            const uint16_t *vsrc, int64_t src_rows, int64_t row0, int count, int slot0,
                            int units, hipStream_t s);

// InnerQ-style layout: quantize `count` token rows per unit, keys from ksrc
// and values from vsrc (row src_row0 + i of [unit][src_rows][128]), into
// cache rows dst_row0 + i, hybrid groups of G channels.
hipError_t launch_innerq_quantize(const CacheView &c, int units, const uint16_t *ksrc, const uint16_t *vsrc,
                                  int64_t src_rows, int64_t src_row0, int count, int64_t dst_row0,
                                  hipStream_t s);

// Key channel scales of the prompt: norm[u][c] = smallest power of two
// >= max(1, max over rows [0, len) of |k[u][row][c]|) (two launches: a fill
// with 1, then an atomic maximum per (unit, channel) over row chunks).
hipError_t launch_key_norm(float *norm, int units, const uint16_t *k, int64_t len, hipStream_t s);

// InnerQ-style append: if pop_row >= 0, quantize ring slot pop_row mod R into
// cache row pop_row; then store k_new / v_new ([unit][128]) into row `slot`
// of the sink rows (to_sink) or of the ring.
hipError_t launch_innerq_append(const CacheView &c, int units, const uint16_t *k_new, const uint16_t *v_new,
                                int64_t pop_row, bool to_sink, int slot, hipStream_t s);

struct AttnArgs {
  CacheView c;
  const uint16_t *q;     // [B][Hq][128]
  float *out;            // [B][Hq][128]
  float *partials;       // [B][Hq][nparts][kPartialStride]
  uint32_t *ctr;         // [B*Hkv][kCtrWords] work-queue counters (zero between calls)
  uint32_t epoch;        // non-zero, different for consecutive launches: tags the election words
  int dynamic;           // 1: waves take super-chunks from the work queue; 0: fixed strided order
  int mfma;              // 1: four query heads per kv head run on the matrix-core kernel
  int batch, hq, hkv;
  int64_t n, nq_k, nq_v;
  int64_t n_main;        // tokens [0, n_main) covered by whole key and value groups
  int splits;            // workgroups per unit over [0, n_main) (>= 1 when resid_main or sinks)
  int interleave;        // vector-ALU kernels: waves take every eighth key group (KIVI) or
                         // 16-token step (InnerQ) of their split instead of a contiguous eighth
  int resid_main;        // 1: the last split takes tokens [n_main, n) (keys and values each
                         // quantized or fp16 per token)
  int nparts;            // parts per unit (== splits); 1 means the kernel writes out directly
  int nsink;             // KIVI: fp16 sink tokens present (rows of c.k_sink); counters above
                         // then count the tokens after them
  int early;             // matrix-core kernel: its leading splits whose workgroups all dispatch
                         // in the first round (one per compute unit), in [1, splits]; they end
                         // first, so the unit's fp16 tokens are shared among them
  float qscale;          // softmax_scale * log2(e)
  // Fused decode step: token n - 1 is read from k_new / v_new ([B*Hkv][128])
  // instead of the residual ring, and the last split writes it into its ring
  // slot.  Null when the token was appended beforehand.
  const uint16_t *k_new;
  const uint16_t *v_new;
  // Token whose quantized row(s) the launch writes ahead of its pop (same
  // counting as n), or -1: KIVI, the value of a full FIFO queue's oldest
  // token (ring slot prequant mod R); InnerQ, the key and value of a full
  // window's oldest token.  Nothing in the launch reads that row or writes
  // that ring slot.
  int64_t prequant;
};

hipError_t launch_decode_attention(const AttnArgs &a, hipStream_t s);

// Matrix-core kernel for four query heads per kv head (KIVI layout): the
// quantized groups [0, n_main) in a.splits parts, each part also taking its
// share of the sinks and tokens [n_main, n) (at most kGqaMaxRest of them);
// writes the normalized output when a.nparts == 1.
constexpr int kGqaMaxRest = 512 + 512 + 127;
hipError_t launch_gqa_mfma(const AttnArgs &a, hipStream_t s);

// InnerQ-style attention: quantized tokens [min(n, sinks), nq_k) split over
// `splits` workgroups per unit, fp16 sinks and window in the last split;
// nparts == splits.
hipError_t launch_innerq_attention(const AttnArgs &a, hipStream_t s);

// Second launch that merges the part records when nparts > 1 (no-op else).
hipError_t launch_merge(const AttnArgs &a, hipStream_t s);

// Streaming-read probe over `bytes` (a multiple of 16) of device memory.
hipError_t launch_stream_read(const void *buf, size_t bytes, uint32_t *out, hipStream_t s);

}  // namespace kvq
