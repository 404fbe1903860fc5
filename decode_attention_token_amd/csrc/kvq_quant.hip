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

namespace kvq {
namespace {

__device__ __forceinline__ float h2f(uint16_t h) { return __half2float(__ushort_as_half(h)); }

struct GroupParams {
  float s, z;
};

// Scale and zero-point of one group from its minimum and maximum: S spreads
// the range over the 2^b - 1 steps and Z = rint(min / S), which maps the
// minimum to code 0.  A constant group takes S = |min| (1 for an all-zero
// group) and so reconstructs exactly.
__device__ __forceinline__ GroupParams group_params(float mn, float mx, float qmax) {
  float s;
  if (mx > mn) {
    s = (mx - mn) / qmax;
  } else {
    s = (mn != 0.0f) ? fabsf(mn) : 1.0f;
  }
  return {s, rintf(mn / s)};
}

__device__ __forceinline__ uint32_t code_of(float x, GroupParams p, float qmax) {
  float q = rintf(x / p.s) - p.z;
  q = fminf(fmaxf(q, 0.0f), qmax);
  return static_cast<uint32_t>(q);
}

// One workgroup of 128 threads quantizes one key group (G tokens x 128
// channels) of one unit.  Thread c reduces channel c over the G tokens; then
// the threads pack token rows word by word from the shared parameters.
template <int BITS>
__global__ __launch_bounds__(128) void quantize_keys_kernel(CacheView c, const uint16_t *__restrict__ src,
                                                            int64_t src_rows, int64_t src_row0,
                                                            int64_t dst_group0) {
  constexpr int PER = 32 / BITS;              // codes per word
  constexpr int W = kHeadDim / PER;           // words per token row
  constexpr float QMAX = float((1 << BITS) - 1);
  const int G = c.group;
  const int g = blockIdx.x;
  const int unit = blockIdx.y;
  const int tid = threadIdx.x;
  __shared__ float s_s[kHeadDim];
  __shared__ float s_z[kHeadDim];

  const uint16_t *rows = src + ((int64_t)unit * src_rows + src_row0 + (int64_t)g * G) * kHeadDim;
  float mn = INFINITY, mx = -INFINITY;
  for (int t = 0; t < G; ++t) {
    const float x = h2f(rows[(int64_t)t * kHeadDim + tid]);
    mn = fminf(mn, x);
    mx = fmaxf(mx, x);
  }
  const GroupParams p = group_params(mn, mx, QMAX);
  const int64_t gidx = (int64_t)unit * (c.cap / G) + dst_group0 + g;
  c.k_scale[gidx * kHeadDim + tid] = p.s;
  c.k_zero[gidx * kHeadDim + tid] = static_cast<int16_t>(p.z);
  s_s[tid] = p.s;
  s_z[tid] = p.z;
  __syncthreads();

  uint32_t *dst = c.k_codes + ((int64_t)unit * c.cap + (dst_group0 + g) * (int64_t)G) * W;
  for (int i = tid; i < G * W; i += blockDim.x) {
    const int t = i / W;
    const int w = i % W;
    const uint16_t *r = rows + (int64_t)t * kHeadDim + w * PER;
    uint32_t word = 0;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int ch = w * PER + k;
      word |= code_of(h2f(r[k]), GroupParams{s_s[ch], s_z[ch]}, QMAX) << (k * BITS);
    }
    dst[i] = word;
  }
}

// One thread quantizes one value group: G channels of one token row.
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
  for (int k = 0; k < G; ++k) {
    const float v = h2f(x[k]);
    mn = fminf(mn, v);
    mx = fmaxf(mx, v);
  }
  const GroupParams p = group_params(mn, mx, QMAX);
  const int64_t row = (int64_t)unit * c.cap + dst_row0 + i;
  c.v_scale[row * NG + j] = p.s;
  c.v_zero[row * NG + j] = static_cast<int16_t>(p.z);
  uint32_t *dst = c.v_codes + row * W + j * (G / PER);
  for (int w = 0; w < G / PER; ++w) {
    uint32_t word = 0;
#pragma unroll
    for (int k = 0; k < PER; ++k) word |= code_of(h2f(x[w * PER + k]), p, QMAX) << (k * BITS);
    dst[w] = word;
  }
}

// Copies fp16 rows into the residual rings, 16 bytes per thread; the second
// half of the grid (when both are given) copies the value rows.
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
  if (c.bits == 2)
    hipLaunchKernelGGL(quantize_keys_kernel<2>, grid, dim3(128), 0, s, c, src, src_rows, src_row0, dst_group0);
  else
    hipLaunchKernelGGL(quantize_keys_kernel<4>, grid, dim3(128), 0, s, c, src, src_rows, src_row0, dst_group0);
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

hipError_t launch_copy_to_residual(const CacheView &c, int units, const uint16_t *ksrc, const uint16_t *vsrc,
                                   int64_t src_rows, int64_t row0, int count, int slot0, bool keys, bool values,
                                   hipStream_t s) {
  if (count <= 0 || units <= 0) return hipSuccess;
  if (!keys && !values) return hipSuccess;
  const int64_t total = (int64_t)units * count * (kHeadDim * 2 / 16) * ((keys && values) ? 2 : 1);
  const unsigned blocks = (unsigned)((total + 255) / 256);
  hipLaunchKernelGGL(copy_rows_kernel, dim3(blocks), dim3(256), 0, s, keys ? c.k_resid : nullptr,
                     values ? c.v_resid : nullptr, c.residual, ksrc, vsrc, src_rows, row0, count, slot0, units);
  return hipGetLastError();
}

}  // namespace kvq
