// Quantize / pack / residual kernels for gfx950.
//
// Keys are quantized per channel over groups of G tokens and values per token
// over groups of G channels, as the KIVI part of the juejin.cn page
// "大模型量化技术原理：KIVI、IntactKV、KVQuant" (how it works) and section 2.2
// of the pgsm.cn KV-cache quantization article describe.  The group map is
// the asymmetric form of X_Q = round(X / S) - Z (pgsm.cn article, 2.1).
//
// Bit-exactness: every arithmetic step is one IEEE fp32 operation with round
// to nearest even (sub, div, rint), so the codes, scales and zero-points equal
// those of any other correctly rounded fp32 implementation of the same steps.
// The build must not use fast-math or approximate division.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include "kvq_internal.h"
#include "kvq_quant_common.h"

namespace kvq {
namespace {

// One workgroup of 256 threads quantizes one key group (GS tokens x 128
// channels) of one unit.  Thread (pair, part) owns channels 2*pair, 2*pair+1
// and a quarter of the group's tokens, held in registers: it reduces min/max
// over its quarter (the quarters combine in LDS), codes its values into an LDS
// byte tile, and the tile is packed into token rows word by word with
// coalesced stores.
template <int BITS, int GS>
__global__ __launch_bounds__(256) void quantize_keys_kernel(CacheView c, const uint16_t *__restrict__ src,
                                                            int64_t src_rows, int64_t src_row0,
                                                            int64_t dst_group0) {
  constexpr int PER = 32 / BITS;              // codes per word
  constexpr int W = kHeadDim / PER;           // words per token row
  constexpr int TQ = GS / 4;                  // tokens per thread
  constexpr float QMAX = float((1 << BITS) - 1);
  const int g = blockIdx.x;
  const int unit = blockIdx.y;
  const int tid = threadIdx.x;
  const int pair = tid & 63, part = tid >> 6;
  const int ch = 2 * pair;
  __shared__ float s_mn[4][kHeadDim], s_mx[4][kHeadDim];
  __shared__ uint8_t s_code[GS][kHeadDim];

  const uint16_t *rows = src + ((int64_t)unit * src_rows + src_row0 + (int64_t)g * GS + part * TQ) * kHeadDim + ch;
  float xa[TQ], xb[TQ];
#pragma unroll
  for (int t = 0; t < TQ; ++t) {
    const uint32_t w = *reinterpret_cast<const uint32_t *>(rows + (int64_t)t * kHeadDim);
    xa[t] = h2f((uint16_t)(w & 0xffffu));
    xb[t] = h2f((uint16_t)(w >> 16));
  }
  float mn0 = INFINITY, mx0 = -INFINITY, mn1 = INFINITY, mx1 = -INFINITY;
#pragma unroll
  for (int t = 0; t < TQ; ++t) {
    mn0 = fminf(mn0, xa[t]);
    mx0 = fmaxf(mx0, xa[t]);
    mn1 = fminf(mn1, xb[t]);
    mx1 = fmaxf(mx1, xb[t]);
  }
  s_mn[part][ch] = mn0;
  s_mn[part][ch + 1] = mn1;
  s_mx[part][ch] = mx0;
  s_mx[part][ch + 1] = mx1;
  __syncthreads();
  mn0 = fminf(fminf(s_mn[0][ch], s_mn[1][ch]), fminf(s_mn[2][ch], s_mn[3][ch]));
  mx0 = fmaxf(fmaxf(s_mx[0][ch], s_mx[1][ch]), fmaxf(s_mx[2][ch], s_mx[3][ch]));
  mn1 = fminf(fminf(s_mn[0][ch + 1], s_mn[1][ch + 1]), fminf(s_mn[2][ch + 1], s_mn[3][ch + 1]));
  mx1 = fmaxf(fmaxf(s_mx[0][ch + 1], s_mx[1][ch + 1]), fmaxf(s_mx[2][ch + 1], s_mx[3][ch + 1]));
  const GroupParams p0 = group_params(mn0, mx0, QMAX, c.meta != 0);
  const GroupParams p1 = group_params(mn1, mx1, QMAX, c.meta != 0);
  if (part == 0) {
    const int64_t gidx = ((int64_t)unit * (c.cap / GS) + dst_group0 + g) * kHeadDim + ch;
    if (c.meta) {
      *reinterpret_cast<uint2 *>(c.k_scale + gidx) = make_uint2(pack_meta(p0.s, p0.z), pack_meta(p1.s, p1.z));
    } else {
      *reinterpret_cast<float2 *>(c.k_scale + gidx) = make_float2(p0.s, p1.s);
      *reinterpret_cast<uint32_t *>(c.k_zero + gidx) =
          (uint32_t)(uint16_t)(int16_t)p0.z | ((uint32_t)(uint16_t)(int16_t)p1.z << 16);
    }
  }
  uint32_t ca[TQ], cb[TQ];
  codes_of<TQ>(xa, p0, 0.0f, QMAX, ca);
  codes_of<TQ>(xb, p1, 0.0f, QMAX, cb);
#pragma unroll
  for (int t = 0; t < TQ; ++t)
    *reinterpret_cast<uint16_t *>(&s_code[part * TQ + t][ch]) = (uint16_t)(ca[t] | (cb[t] << 8));
  __syncthreads();
  uint32_t *dst = c.k_codes + ((int64_t)unit * c.cap + (dst_group0 + g) * (int64_t)GS) * W;
  for (int i = tid; i < GS * W; i += blockDim.x) {
    const int t = i / W, w = i % W;
    const uint8_t *b = &s_code[t][w * PER];
    uint32_t word = 0;
#pragma unroll
    for (int k = 0; k < PER; ++k) word |= (uint32_t)b[k] << (k * BITS);
    dst[i] = word;
  }
}

// One thread quantizes one value group (G channels of one token row) in
// chunks of 32 channels held in registers: a min/max pass, then a coding
// pass over the same 16-byte loads (served by the cache).
template <int BITS>
__global__ __launch_bounds__(256) void quantize_values_kernel(CacheView c, const uint16_t *__restrict__ src,
                                                              int64_t src_rows, int64_t src_row0, int count,
                                                              int64_t dst_row0, int units) {
  constexpr int PER = 32 / BITS;
  constexpr int W = kHeadDim / PER;
  constexpr float QMAX = float((1 << BITS) - 1);
  const int G = c.group;
  const int NG = kHeadDim / G;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)units * count * NG;
  if (idx >= total) return;
  const int j = (int)(idx % NG);
  const int64_t r = idx / NG;
  const int i = (int)(r % count);
  const int unit = (int)(r / count);

  const uint16_t *x = src + ((int64_t)unit * src_rows + src_row0 + i) * kHeadDim + j * G;
  float mn = INFINITY, mx = -INFINITY;
  for (int k0 = 0; k0 < G; k0 += 32) {
    float v[32];
#pragma unroll
    for (int q = 0; q < 4; ++q) load8(x + k0 + 8 * q, v + 8 * q);
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      mn = fminf(mn, v[k]);
      mx = fmaxf(mx, v[k]);
    }
  }
  const GroupParams p = group_params(mn, mx, QMAX, c.meta != 0);
  const int64_t row = (int64_t)unit * c.cap + dst_row0 + i;
  if (c.meta) {
    reinterpret_cast<uint32_t *>(c.v_scale)[row * NG + j] = pack_meta(p.s, p.z);
  } else {
    c.v_scale[row * NG + j] = p.s;
    c.v_zero[row * NG + j] = static_cast<int16_t>(p.z);
  }
  uint32_t *dst = c.v_codes + row * W + j * (G / PER);
  for (int k0 = 0; k0 < G; k0 += 32) {
    float v[32];
#pragma unroll
    for (int q = 0; q < 4; ++q) load8(x + k0 + 8 * q, v + 8 * q);
    uint32_t cd[32];
    codes_of<32>(v, p, 0.0f, QMAX, cd);
    uint32_t words[32 / PER];
#pragma unroll
    for (int w = 0; w < 32 / PER; ++w) {
      uint32_t word = 0;
#pragma unroll
      for (int k = 0; k < PER; ++k) word |= cd[w * PER + k] << (k * BITS);
      words[w] = word;
    }
    if constexpr (BITS == 2) {
      *reinterpret_cast<uint2 *>(dst + k0 / PER) = make_uint2(words[0], words[1]);
    } else {
      *reinterpret_cast<uint4 *>(dst + k0 / PER) = make_uint4(words[0], words[1], words[2], words[3]);
    }
  }
}

// Copies fp16 rows into ring-indexed destination rows (the residual rings or
// the sink rows), 16 bytes per thread; the second half of the grid (when both
// destinations are given) copies the value rows.
__global__ __launch_bounds__(256) void copy_rows_kernel(uint16_t *__restrict__ kring, uint16_t *__restrict__ vring,
                                                        int ring_rows, const uint16_t *__restrict__ ksrc,
                                                        const uint16_t *__restrict__ vsrc, int64_t src_rows,
                                                        int64_t row0, int count, int slot0, int units) {
  constexpr int CHUNKS = kHeadDim * 2 / 16;
  int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)units * count * CHUNKS;
  uint16_t *ring = kring;
  const uint16_t *src = ksrc;
  if (ring == nullptr || idx >= total) {
    if (ring != nullptr) idx -= total;
    ring = vring;
    src = vsrc;
  }
  if (ring == nullptr || idx >= total) return;
  const int ch = (int)(idx % CHUNKS);
  const int64_t r = idx / CHUNKS;
  const int i = (int)(r % count);
  const int unit = (int)(r / count);
  const int slot = (slot0 + i) % ring_rows;
  const uint4 *s = reinterpret_cast<const uint4 *>(src + ((int64_t)unit * src_rows + row0 + i) * kHeadDim);
  uint4 *d = reinterpret_cast<uint4 *>(ring + ((int64_t)unit * ring_rows + slot) * kHeadDim);
  d[ch] = s[ch];
}

}  // namespace

hipError_t launch_quantize_keys(const CacheView &c, int units, const uint16_t *src, int64_t src_rows,
                                int64_t src_row0, int ngroups, int64_t dst_group0, hipStream_t s) {
  if (ngroups <= 0 || units <= 0) return hipSuccess;
  dim3 grid(ngroups, units);
#define KVQ_QK(B, G)                                                                                     \
  hipLaunchKernelGGL((quantize_keys_kernel<B, G>), grid, dim3(256), 0, s, c, src, src_rows, src_row0, \
                     dst_group0)
  if (c.bits == 2) {
    if (c.group == 32) KVQ_QK(2, 32);
    else if (c.group == 64) KVQ_QK(2, 64);
    else KVQ_QK(2, 128);
  } else {
    if (c.group == 32) KVQ_QK(4, 32);
    else if (c.group == 64) KVQ_QK(4, 64);
    else KVQ_QK(4, 128);
  }
#undef KVQ_QK
  return hipGetLastError();
}

hipError_t launch_quantize_values(const CacheView &c, int units, const uint16_t *src, int64_t src_rows,
                                  int64_t src_row0, int count, int64_t dst_row0, hipStream_t s) {
  if (count <= 0 || units <= 0) return hipSuccess;
  const int64_t total = (int64_t)units * count * (kHeadDim / c.group);
  const int64_t blocks = (total + 255) / 256;
  if (c.bits == 2)
    hipLaunchKernelGGL(quantize_values_kernel<2>, dim3((unsigned)blocks), dim3(256), 0, s, c, src, src_rows,
                       src_row0, count, dst_row0, units);
  else
    hipLaunchKernelGGL(quantize_values_kernel<4>, dim3((unsigned)blocks), dim3(256), 0, s, c, src, src_rows,
                       src_row0, count, dst_row0, units);
  return hipGetLastError();
}

hipError_t launch_copy_rows(uint16_t *kdst, uint16_t *vdst, int dst_rows, const uint16_t *ksrc,
                            const uint16_t *vsrc, int64_t src_rows, int64_t row0, int count, int slot0,
                            int units, hipStream_t s) {
  if (count <= 0 || units <= 0) return hipSuccess;
  if (kdst == nullptr && vdst == nullptr) return hipSuccess;
  const int64_t total = (int64_t)units * count * (kHeadDim * 2 / 16) * ((kdst && vdst) ? 2 : 1);
  const unsigned blocks = (unsigned)((total + 255) / 256);
  hipLaunchKernelGGL(copy_rows_kernel, dim3(blocks), dim3(256), 0, s, kdst, vdst, dst_rows, ksrc, vsrc, src_rows,
                     row0, count, slot0, units);
  return hipGetLastError();
}

hipError_t launch_copy_to_residual(const CacheView &c, int units, const uint16_t *ksrc, const uint16_t *vsrc,
                                   int64_t src_rows, int64_t row0, int count, int slot0, bool keys, bool values,
                                   hipStream_t s) {
  return launch_copy_rows(keys ? c.k_resid : nullptr, values ? c.v_resid : nullptr, c.residual, ksrc, vsrc,
                          src_rows, row0, count, slot0, units, s);
}

}  // namespace kvq
