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

// Packed fp16 minimum / maximum over lanes l, l ^ 16, l ^ 32 and l ^ 48.  A
// 16-lane row swap of a register with itself leaves lane l's and lane
// (l ^ 16)'s values in the two results at every lane; a 32-lane swap does the
// same for l ^ 32.  Both are plain VALU lane swaps (no LDS traffic).
__device__ __forceinline__ f16x2 min_over_rows(f16x2 x) {
  auto p = __builtin_amdgcn_permlane16_swap(as_u32(x), as_u32(x), false, false);
  x = hmin(as_h2(p[0]), as_h2(p[1]));
  p = __builtin_amdgcn_permlane32_swap(as_u32(x), as_u32(x), false, false);
  return hmin(as_h2(p[0]), as_h2(p[1]));
}
__device__ __forceinline__ f16x2 max_over_rows(f16x2 x) {
  auto p = __builtin_amdgcn_permlane16_swap(as_u32(x), as_u32(x), false, false);
  x = hmax(as_h2(p[0]), as_h2(p[1]));
  p = __builtin_amdgcn_permlane32_swap(as_u32(x), as_u32(x), false, false);
  return hmax(as_h2(p[0]), as_h2(p[1]));
}

// One wave quantizes one key group (GS tokens x 128 channels) of one unit.
// Lane l holds channels 8 (l % 16) .. + 7 of the group's token rows
// 4 i + l / 16 as 16-byte words (each load instruction reads 1 KB of
// consecutive rows).  Per-channel minimum and maximum reduce in packed fp16
// over the lane's rows, then across the four lanes that hold the same
// channels.  Each of those four lanes derives scale, zero-point and tie
// threshold for two of the eight channels (the divisions are spread over the
// wave) and hands them to the others through LDS, laid out so that each read
// instruction touches 16 consecutive entries.  Codes are packed into
// token rows in registers and stored as 256 contiguous bytes per instruction.
// Block `blk` of a grid of 4-wave blocks.  ovr (null: unused) supplies
// source row ovr_row of every unit ([unit][128] fp16) in place of the row in
// src: a flush reads the token appended by the same call from there.
template <int BITS, int GS>
__device__ __forceinline__ void quantize_keys_block(const CacheView &c, const uint16_t *__restrict__ src,
                                                    int64_t src_rows, int64_t src_row0, int64_t dst_group0,
                                                    int ngroups, int total, int blk,
                                                    const uint16_t *__restrict__ ovr, int64_t ovr_row) {
  constexpr int RL = GS / 4;                  // rows per lane
  constexpr int PER = 32 / BITS;              // codes per word
  constexpr int W = kHeadDim / PER;           // words per token row
  constexpr float QMAX = float((1 << BITS) - 1);
  __shared__ float4 s_par[4][8][16];          // [wave][channel % 8][channel / 8]: r, z, thr, s
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int gi = blk * 4 + wave;
  if (gi >= total) return;                    // wave-uniform
  const int unit = gi / ngroups, g = gi - unit * ngroups;
  const int cs = lane & 15, q = lane >> 4;

  const uint4 *in =
      reinterpret_cast<const uint4 *>(src + ((int64_t)unit * src_rows + src_row0 + (int64_t)g * GS + q) * kHeadDim) +
      cs;
  const int64_t srow = src_row0 + (int64_t)g * GS + q;   // source row of raw[0]
  const uint4 *ov = ovr ? reinterpret_cast<const uint4 *>(ovr + (int64_t)unit * kHeadDim) + cs : nullptr;
  uint4 raw[RL];
#pragma unroll
  for (int i = 0; i < RL; ++i) raw[i] = (ov && srow + 4 * i == ovr_row) ? *ov : in[i * 4 * (kHeadDim / 8)];

  f16x2 mn[4], mx[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) mn[e] = mx[e] = as_h2(word_of(raw[0], e));
#pragma unroll
  for (int i = 1; i < RL; ++i) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const f16x2 h = as_h2(word_of(raw[i], e));
      mn[e] = hmin(mn[e], h);
      mx[e] = hmax(mx[e], h);
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    mn[e] = min_over_rows(mn[e]);
    mx[e] = max_over_rows(mx[e]);
  }

  // lane (cs, q) derives the parameters of channels 8 cs + 2 q and 8 cs + 2 q + 1
  const f16x2 a = q == 0 ? mn[0] : q == 1 ? mn[1] : q == 2 ? mn[2] : mn[3];
  const f16x2 b = q == 0 ? mx[0] : q == 1 ? mx[1] : q == 2 ? mx[2] : mx[3];
  GroupParams p[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const float lo = (float)a[e], hi = (float)b[e];
    p[e] = group_params(lo, hi, QMAX, c.meta != 0);
    s_par[wave][2 * q + e][cs] = make_float4(p[e].r, p[e].z, tie_threshold(fmaxf(fabsf(lo), fabsf(hi)), p[e].r),
                                                  p[e].s);
  }
  const int64_t gidx = ((int64_t)unit * (c.cap / GS) + dst_group0 + g) * kHeadDim + 8 * cs + 2 * q;
  if (c.meta) {
    *reinterpret_cast<uint2 *>(c.k_scale + gidx) = make_uint2(pack_meta(p[0].s, p[0].z), pack_meta(p[1].s, p[1].z));
  } else {
    *reinterpret_cast<float2 *>(c.k_scale + gidx) = make_float2(p[0].s, p[1].s);
    *reinterpret_cast<uint32_t *>(c.k_zero + gidx) =
        (uint32_t)(uint16_t)(int16_t)p[0].z | ((uint32_t)(uint16_t)(int16_t)p[1].z << 16);
  }
  lds_wave_sync();
  float r[8], z[8], thr[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float4 v = s_par[wave][k][cs];
    r[k] = v.x;
    z[k] = v.y;
    thr[k] = v.z;
  }
  auto code_row = [&](const uint4 &v) {
    bool near = false;
    uint32_t u = code8_fast<BITS>(v, r, z, thr, 0.0f, near);
    if (__any(near)) {
      float sv[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) sv[k] = s_par[wave][k][cs].w;
      u = code8_exact<BITS>(v, sv, z, 0.0f);
    }
    return u;
  };

  uint32_t *dst = c.k_codes + ((int64_t)unit * c.cap + (dst_group0 + g) * (int64_t)GS + q) * W;
  if constexpr (BITS == 2) {
    const bool odd = cs & 1;
#pragma unroll
    for (int k = 0; k < RL / 2; ++k) {
      const uint32_t ua = code_row(raw[2 * k]), ub = code_row(raw[2 * k + 1]);
      dst[4 * (2 * k + (odd ? 1 : 0)) * W + (cs >> 1)] = pair_words(ua, ub, odd);
    }
  } else {
#pragma unroll
    for (int i = 0; i < RL; ++i) dst[4 * i * W + cs] = code_row(raw[i]);
  }
}

// One wave quantizes 32 consecutive token rows of the flattened (unit, token)
// range, one value group per row and G channels.  Lane l holds channels
// 8 (l % 16) .. + 7 of rows 4 i + l / 16 (16-byte loads, 1 KB of consecutive
// rows per load instruction where the rows are contiguous), so a group spans
// G / 8 neighbouring lanes: its minimum and maximum reduce with DPP moves as
// one packed (min, -max) fp16 pair.  The group's lanes split the rows for
// the parameter divisions and share the results through LDS; codes are
// packed and stored as for keys.
template <int BITS, int G>
__device__ __forceinline__ void quantize_values_block(const CacheView &c, const uint16_t *__restrict__ src,
                                                      int64_t src_rows, int64_t src_row0, int count,
                                                      int64_t dst_row0, int total_rows, int blk,
                                                      const uint16_t *__restrict__ ovr, int64_t ovr_row) {
  constexpr int NR = 8;                       // rows per lane
  constexpr int LPG = G / 8;                  // lanes per value group
  constexpr int NG = kHeadDim / G;            // value groups per row
  constexpr int NS = NR / LPG > 0 ? NR / LPG : 1;  // parameter rows per lane
  constexpr int PER = 32 / BITS;
  constexpr int W = kHeadDim / PER;
  constexpr float QMAX = float((1 << BITS) - 1);
  __shared__ float4 s_par[4][NR][4][NG];      // [wave][row][l / 16][group]: r, z, thr, s
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int cs = lane & 15, q = lane >> 4, j = cs / LPG, gl = cs % LPG;
  const int row0 = (blk * 4 + wave) * 4 * NR;
  if (row0 >= total_rows) return;             // wave-uniform
  // (unit, token) of the lane's row i, stepped from the block's first row
  // (one wave-uniform division per block)
  const int u0 = row0 / count, t0 = row0 - u0 * count;
  auto locate = [&](int i, int &u, int &t) {
    u = u0;
    t = t0 + 4 * i + q;
    while (t >= count) {
      t -= count;
      ++u;
    }
  };
  auto valid = [&](int i) { return row0 + 4 * i + q < total_rows; };

  uint4 raw[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    raw[i] = make_uint4(0u, 0u, 0u, 0u);
    if (valid(i)) {
      int u, t;
      locate(i, u, t);
      raw[i] = (ovr && src_row0 + t == ovr_row)
                   ? *(reinterpret_cast<const uint4 *>(ovr + (int64_t)u * kHeadDim) + cs)
                   : *(reinterpret_cast<const uint4 *>(src + ((int64_t)u * src_rows + src_row0 + t) * kHeadDim) + cs);
    }
  }

  float mnr[NR], mxr[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const f16x2 h0 = as_h2(raw[i].x), h1 = as_h2(raw[i].y), h2 = as_h2(raw[i].z), h3 = as_h2(raw[i].w);
    const f16x2 lo = hmin(hmin(h0, h1), hmin(h2, h3)), hi = hmax(hmax(h0, h1), hmax(h2, h3));
    const f16x2 lo2 = hmin(lo, lo.yx), hi2 = hmax(hi, hi.yx);
    f16x2 v = {lo2.x, -hi2.x};                // (min, -max): one packed minimum reduces both
    v = hmin(v, as_h2((uint32_t)__builtin_amdgcn_mov_dpp((int)as_u32(v), 0xB1, 0xF, 0xF, true)));   // lane ^ 1
    v = hmin(v, as_h2((uint32_t)__builtin_amdgcn_mov_dpp((int)as_u32(v), 0x4E, 0xF, 0xF, true)));   // lane ^ 2
    if constexpr (LPG >= 8)
      v = hmin(v, as_h2((uint32_t)__builtin_amdgcn_mov_dpp((int)as_u32(v), 0x141, 0xF, 0xF, true)));  // other quad of 8
    if constexpr (LPG >= 16)
      v = hmin(v, as_h2((uint32_t)__builtin_amdgcn_mov_dpp((int)as_u32(v), 0x140, 0xF, 0xF, true)));  // other half of 16
    mnr[i] = (float)v.x;
    mxr[i] = -(float)v.y;
  }

  // lane gl of a group derives the parameters of rows gl, gl + LPG, ...
#pragma unroll
  for (int sl = 0; sl < NS; ++sl) {
    const int i = gl + LPG * sl;
    float lo = mnr[0], hi = mxr[0];
#pragma unroll
    for (int ii = 1; ii < NR; ++ii) {
      lo = (i == ii) ? mnr[ii] : lo;
      hi = (i == ii) ? mxr[ii] : hi;
    }
    const GroupParams p = group_params(lo, hi, QMAX, c.meta != 0);
    if (i < NR) {
      s_par[wave][i][q][j] = make_float4(p.r, p.z, tie_threshold(fmaxf(fabsf(lo), fabsf(hi)), p.r), p.s);
      if (valid(i)) {
        int u, t;
        locate(i, u, t);
        const int64_t row = (int64_t)u * c.cap + dst_row0 + t;
        if (c.meta) {
          reinterpret_cast<uint32_t *>(c.v_scale)[row * NG + j] = pack_meta(p.s, p.z);
        } else {
          c.v_scale[row * NG + j] = p.s;
          c.v_zero[row * NG + j] = static_cast<int16_t>(p.z);
        }
      }
    }
  }
  lds_wave_sync();

  auto code_row = [&](int i) {
    const float4 pv = s_par[wave][i][q][j];
    float r[8], z[8], thr[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      r[k] = pv.x;
      z[k] = pv.y;
      thr[k] = pv.z;
    }
    bool near = false;
    uint32_t u = code8_fast<BITS>(raw[i], r, z, thr, 0.0f, near);
    if (__any(near)) {
      float sv[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) sv[k] = pv.w;
      u = code8_exact<BITS>(raw[i], sv, z, 0.0f);
    }
    return u;
  };
  auto store = [&](int i, uint32_t word, int w) {
    if (valid(i)) {
      int u, t;
      locate(i, u, t);
      c.v_codes[((int64_t)u * c.cap + dst_row0 + t) * W + w] = word;
    }
  };
  if constexpr (BITS == 2) {
    const bool odd = cs & 1;
#pragma unroll
    for (int k = 0; k < NR / 2; ++k) {
      const uint32_t ua = code_row(2 * k), ub = code_row(2 * k + 1);
      store(2 * k + (odd ? 1 : 0), pair_words(ua, ub, odd), cs >> 1);
    }
  } else {
#pragma unroll
    for (int i = 0; i < NR; ++i) store(i, code_row(i), cs);
  }
}

template <int BITS, int GS>
__global__ __launch_bounds__(256) void quantize_keys_kernel(CacheView c, const uint16_t *__restrict__ src,
                                                            int64_t src_rows, int64_t src_row0,
                                                            int64_t dst_group0, int ngroups, int total) {
  quantize_keys_block<BITS, GS>(c, src, src_rows, src_row0, dst_group0, ngroups, total, (int)blockIdx.x, nullptr, -1);
}

template <int BITS, int G>
__global__ __launch_bounds__(256) void quantize_values_kernel(CacheView c, const uint16_t *__restrict__ src,
                                                              int64_t src_rows, int64_t src_row0, int count,
                                                              int64_t dst_row0, int total_rows) {
  quantize_values_block<BITS, G>(c, src, src_rows, src_row0, count, dst_row0, total_rows, (int)blockIdx.x, nullptr,
                                 -1);
}

// Residual flush of both rings in one launch (the key groups, then the value
// rows, of the R ring slots in token order), with the token appended by the
// same call read from k_new / v_new at its ring slot `slot`.  The ring slot
// itself is not written: once flushed, no ring slot is live.
template <int BITS, int G>
__global__ __launch_bounds__(256) void flush_kernel(CacheView c, const uint16_t *__restrict__ k_new,
                                                    const uint16_t *__restrict__ v_new, int slot,
                                                    int64_t dst_group0, int64_t dst_row0, int units, int kblocks) {
  const int R = c.residual;
  if ((int)blockIdx.x < kblocks) {
    quantize_keys_block<BITS, G>(c, c.k_resid, R, 0, dst_group0, R / G, units * (R / G), (int)blockIdx.x, k_new,
                                 slot);
  } else {
    quantize_values_block<BITS, G>(c, c.v_resid, R, 0, R, dst_row0, units * R, (int)blockIdx.x - kblocks, v_new,
                                   slot);
  }
}

// A prefill's key groups and value rows in one launch: blocks below kblocks
// quantize key groups, the rest value rows (no gap between two launches, and
// value blocks fill the compute units the key blocks' tail leaves idle;
// 2-2.5% off a G = 32 prefill).
template <int BITS, int G>
__global__ __launch_bounds__(256) void quantize_kv_kernel(CacheView c, const uint16_t *__restrict__ ksrc,
                                                          const uint16_t *__restrict__ vsrc, int64_t src_rows,
                                                          int64_t src_row0, int ngroups, int ktotal, int count,
                                                          int vtotal, int kblocks) {
  if ((int)blockIdx.x < kblocks) {
    quantize_keys_block<BITS, G>(c, ksrc, src_rows, src_row0, 0, ngroups, ktotal, (int)blockIdx.x, nullptr, -1);
  } else {
    quantize_values_block<BITS, G>(c, vsrc, src_rows, src_row0, count, 0, vtotal, (int)blockIdx.x - kblocks,
                                   nullptr, -1);
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
  const int64_t total = (int64_t)units * ngroups;
  if (total > INT32_MAX - 4) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((total + 3) / 4));
#define KVQ_QK(B, G)                                                                                     \
  hipLaunchKernelGGL((quantize_keys_kernel<B, G>), grid, dim3(256), 0, s, c, src, src_rows, src_row0, \
                     dst_group0, ngroups, (int)total)
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
  const int64_t total = (int64_t)units * count;
  if (total > INT32_MAX - 256) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((total + 127) / 128));
#define KVQ_QV(B, G)                                                                                       \
  hipLaunchKernelGGL((quantize_values_kernel<B, G>), grid, dim3(256), 0, s, c, src, src_rows, src_row0, \
                     count, dst_row0, (int)total)
  if (c.bits == 2) {
    if (c.group == 32) KVQ_QV(2, 32);
    else if (c.group == 64) KVQ_QV(2, 64);
    else KVQ_QV(2, 128);
  } else {
    if (c.group == 32) KVQ_QV(4, 32);
    else if (c.group == 64) KVQ_QV(4, 64);
    else KVQ_QV(4, 128);
  }
#undef KVQ_QV
  return hipGetLastError();
}

hipError_t launch_quantize_kv(const CacheView &c, int units, const uint16_t *ksrc, const uint16_t *vsrc,
                              int64_t src_rows, int64_t src_row0, int ngroups, int count, hipStream_t s) {
  if (units <= 0 || (ngroups <= 0 && count <= 0)) return hipSuccess;
  if (c.group != 32) {
    // At G = 64 and 128 the key quantizer holds 112-176 VGPRs, and one launch
    // would run the value blocks at the key blocks' occupancy (half of
    // theirs): 2.4% slower on the 4-bit G = 64 workload.  Two launches there.
    hipError_t e = launch_quantize_keys(c, units, ksrc, src_rows, src_row0, ngroups, 0, s);
    if (e == hipSuccess) e = launch_quantize_values(c, units, vsrc, src_rows, src_row0, count, 0, s);
    return e;
  }
  const int64_t ktotal = (int64_t)units * (ngroups > 0 ? ngroups : 0);
  const int64_t vtotal = (int64_t)units * (count > 0 ? count : 0);
  if (ktotal > INT32_MAX - 4 || vtotal > INT32_MAX - 256) return hipErrorInvalidValue;
  const int64_t kblocks = (ktotal + 3) / 4, vblocks = (vtotal + 127) / 128;
  if (kblocks + vblocks > INT32_MAX) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(kblocks + vblocks));
  if (c.bits == 2) {
    hipLaunchKernelGGL((quantize_kv_kernel<2, 32>), grid, dim3(256), 0, s, c, ksrc, vsrc, src_rows, src_row0, ngroups,
                       (int)ktotal, count, (int)vtotal, (int)kblocks);
  } else {
    hipLaunchKernelGGL((quantize_kv_kernel<4, 32>), grid, dim3(256), 0, s, c, ksrc, vsrc, src_rows, src_row0, ngroups,
                       (int)ktotal, count, (int)vtotal, (int)kblocks);
  }
  return hipGetLastError();
}

hipError_t launch_flush(const CacheView &c, int units, const uint16_t *k_new, const uint16_t *v_new, int slot,
                        int64_t dst_group0, int64_t dst_row0, hipStream_t s) {
  if (units <= 0) return hipSuccess;
  const int64_t kwaves = (int64_t)units * (c.residual / c.group);   // one key group per wave
  const int64_t vrows = (int64_t)units * c.residual;                // 32 value rows per wave
  if (vrows > INT32_MAX - 256) return hipErrorInvalidValue;
  const int kblocks = (int)((kwaves + 3) / 4);
  const int vblocks = (int)((vrows + 127) / 128);
#define KVQ_FL(B, G)                                                                                          \
  hipLaunchKernelGGL((flush_kernel<B, G>), dim3(kblocks + vblocks), dim3(256), 0, s, c, k_new, v_new, slot, \
                     dst_group0, dst_row0, units, kblocks)
  if (c.bits == 2) {
    if (c.group == 32) KVQ_FL(2, 32);
    else if (c.group == 64) KVQ_FL(2, 64);
    else KVQ_FL(2, 128);
  } else {
    if (c.group == 32) KVQ_FL(4, 32);
    else if (c.group == 64) KVQ_FL(4, 64);
    else KVQ_FL(4, 128);
  }
#undef KVQ_FL
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
