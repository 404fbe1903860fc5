// Internal launch interface between the C ABI (kvq_api.cpp) and the HIP
// kernels (kvq_quant.hip, kvq_attn.hip).  Not part of the public ABI.
#pragma once

#include <stdint.h>
#include <hip/hip_runtime_api.h>

namespace kvq {

constexpr int kHeadDim = 128;
constexpr int kMaxSplits = 64;
constexpr int kPartialStride = kHeadDim + 4;   // acc[128], m, l, pad, pad (floats)

struct CacheView {
  uint32_t *k_codes;
  float *k_scale;
  int16_t *k_zero;
  uint32_t *v_codes;
  float *v_scale;
  int16_t *v_zero;
  uint16_t *k_resid;
  uint16_t *v_resid;
  int64_t cap;      // max_tokens
  int bits, group, residual;
};

// Quantize `ngroups` key groups per unit.  Source rows: src + (unit * src_rows
// + src_row0 + i) * 128 for token i of the block; destination group index
// dst_group0 + g.
hipError_t launch_quantize_keys(const CacheView &c, int units, const uint16_t *src,
                                int64_t src_rows, int64_t src_row0, int ngroups,
                                int64_t dst_group0, hipStream_t s);

// Quantize `count` value rows per unit (source row src_row0 + i) into
// destination token rows dst_row0 + i.
hipError_t launch_quantize_values(const CacheView &c, int units, const uint16_t *src,
                                  int64_t src_rows, int64_t src_row0, int count,
                                  int64_t dst_row0, hipStream_t s);

// Copy rows [row0, row0 + count) of src ([unit][src_rows][128] fp16) into
// residual slots slot0 + i of both rings (keys from ksrc, values from vsrc).
hipError_t launch_copy_to_residual(const CacheView &c, int units, const uint16_t *ksrc,
                                   const uint16_t *vsrc, int64_t src_rows, int64_t row0,
                                   int count, int slot0, bool keys, bool values, hipStream_t s);

struct AttnArgs {
  CacheView c;
  const uint16_t *q;     // [B][Hq][128]
  float *out;            // [B][Hq][128]
  float *partials;       // [B][Hq][nparts][kPartialStride]
  int batch, hq, hkv;
  int64_t n, nq_k, nq_v;
  int64_t n_main;        // tokens [0, n_main) covered by whole key and value groups
  int splits;            // workgroups per unit over [0, n_main) (>= 1 when resid_main)
  int tail_wg;           // 1: an extra workgroup per unit runs the mixed tail [n_main, n)
  int resid_main;        // 1: [n_main, n) is all-fp16 and the last split takes it
  int nparts;            // splits + tail_wg; 1 means the kernel writes out directly
  float qscale;          // softmax_scale * log2(e)
  // Fused decode step: token n - 1 is read from k_new / v_new ([B*Hkv][128])
  // instead of the residual ring, and the last split writes it into its ring
  // slot.  Null when the token was appended beforehand.
  const uint16_t *k_new;
  const uint16_t *v_new;
};

hipError_t launch_decode_attention(const AttnArgs &a, hipStream_t s);

}  // namespace kvq
