// Device-side quantizer pieces shared by kvq_quant.hip (KIVI layout),
// kvq_innerq.hip (InnerQ-style layout) and the KIVI attention kernels (which
// quantize one value row ahead of a FIFO pop): group scale and zero-point,
// the exactly rounded code map with its fast path, 16-byte fp16 loads and
// the 8-channel tile coder.
// Private to the HIP sources.
//
// Bit-exactness: every arithmetic step is one IEEE fp32 operation with round
// to nearest even (sub, div, rint), so the codes, scales and zero-points equal
// those of any other correctly rounded fp32 implementation of the same steps.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include "kvq_device_util.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

struct GroupParams {
  float s, z;
  float r;   // RN(1 / s), for the fast quotient
};

// Smallest fp16 value >= s (s > 0), as a float: round to nearest, then one
// fp16 step up if that fell below.
__device__ __forceinline__ float round_up_fp16(float s) {
  __half h = __float2half_rn(s);
  if (__half2float(h) < s) h = __ushort_as_half((unsigned short)(__half_as_ushort(h) + 1));
  return __half2float(h);
}

// Compressed metadata word: fp16 bits of S (exactly representable) in the low
// half, the int16 zero-point in the high half.
__device__ __forceinline__ uint32_t pack_meta(float s, float z) {
  return (uint32_t)__half_as_ushort(__float2half_rn(s)) | ((uint32_t)(uint16_t)(int16_t)z << 16);
}

// Scale and zero-point of one group from its minimum and maximum: S spreads
// the range over the 2^b - 1 steps and Z = rint(min / S), which maps the
// minimum to code 0.  A constant group takes S = |min| (1 for an all-zero
// group) and so reconstructs exactly.  With compressed metadata S is first
// rounded up to fp16, so the range still fits the levels.
__device__ __forceinline__ GroupParams group_params(float mn, float mx, float qmax, bool f16_scale = false) {
  float s;
  if (mx > mn) {
    s = (mx - mn) / qmax;
  } else {
    s = (mn != 0.0f) ? fabsf(mn) : 1.0f;
  }
  if (f16_scale) s = round_up_fp16(s);
  return {s, rintf(mn / s), 1.0f / s};
}

// clamp(rint(x / S) - Z, lo, qmax) with the correctly rounded quotient.
// lo is 0 for the asymmetric map and 1 for the symmetric one, whose codes
// are the signed levels offset by 2^(b-1).
__device__ __forceinline__ uint32_t code_of(float x, GroupParams p, float lo, float qmax) {
  float q = rintf(x / p.s) - p.z;
  q = fminf(fmaxf(q, lo), qmax);
  return static_cast<uint32_t>(q);
}

// Codes of N values of one group.  rint(x / s) with x / s correctly rounded
// equals rint(x * r), r = RN(1/s), unless the quotient lies within 2^-21 |x/s|
// of a half-integer (x * r is that close to the correctly rounded quotient).
// The fast products are checked for that; if any lane of the wave meets such
// a value, the whole chunk is redone with IEEE divisions (a rare, uniform
// branch), so the codes stay exactly those of the correctly rounded map.
template <int N>
__device__ __forceinline__ void codes_of(const float *x, GroupParams p, float lo, float qmax, uint32_t *code) {
  bool near = false;
#pragma unroll
  for (int k = 0; k < N; ++k) {
    const float y = x[k] * p.r;
    const float mid = floorf(y) + 0.5f;
    near |= fabsf(y - mid) <= fmaxf(fabsf(y), 1.0f) * 0x1p-20f;
    code[k] = static_cast<uint32_t>(fminf(fmaxf(rintf(y) - p.z, lo), qmax));
  }
  if (__any(near)) {
#pragma unroll
    for (int k = 0; k < N; ++k) code[k] = code_of(x[k], p, lo, qmax);
  }
}

// Orders a wave's LDS writes before its later LDS reads of other lanes' data.
__device__ __forceinline__ void lds_wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Threshold of the tile coder's tie test for a group whose values are at most
// amax in magnitude: the fast quotient y = x * RN(1/S) can round differently
// from RN(x / S) only when y lies within 2^-20 max(|y|, 1) of a half-integer,
// i.e. when |y - rint(y)| >= 0.5 - 2^-20 max(|y|, 1).  |y| <= RN(amax * r)
// (rounding is monotonic), and subtracting twice that tolerance keeps the
// rounded threshold below the exact one (its rounding error is far smaller).
__device__ __forceinline__ float tie_threshold(float amax, float r) {
  return 0.5f - 2.0f * (fmaxf(amax * r, 1.0f) * 0x1p-20f);
}

// Unpacks 8 fp16 values (one 16-byte load) to fp32.
__device__ __forceinline__ void load8(const uint16_t *p, float *x) {
  const uint4 v = *reinterpret_cast<const uint4 *>(p);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = h2f((uint16_t)(w[i] & 0xffffu));
    x[2 * i + 1] = h2f((uint16_t)(w[i] >> 16));
  }
}

// ---------------------------------------------------------------- tile coder
// Pieces of the wave-per-tile quantizers: lanes hold 16-byte words of 8
// consecutive fp16 channels of one token row.
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f16x2 as_h2(uint32_t w) { return __builtin_bit_cast(f16x2, w); }
__device__ __forceinline__ uint32_t as_u32(f16x2 h) { return __builtin_bit_cast(uint32_t, h); }
__device__ __forceinline__ f16x2 hmin(f16x2 a, f16x2 b) { return __builtin_elementwise_minimum(a, b); }
__device__ __forceinline__ f16x2 hmax(f16x2 a, f16x2 b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ uint32_t word_of(const uint4 &v, int k) {
  return k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
}

// Packed codes of the 8 fp16 values of one 16-byte word (8 consecutive
// channels of one token row), value k coded with r[k] = RN(1/S), z[k] and the
// tie threshold thr[k], clamped to [lo, 2^b - 1] (lo = 1 for symmetric
// groups, 0 otherwise).  The code map is the fast quotient of codes_of: a
// product x * r (fp16 x read straight into the fused multiply), its rint, and
// the tie test |y - rint(y)| >= thr, which flags every value whose fast code
// could differ from the correctly rounded one (near is set, and the caller
// redoes the word with code8_exact).  Codes accumulate as exact small
// integers in fp32 (sum of code * 2^(BITS k) < 2^16 per half word).
// 2-bit: bits 0..15 hold the 8 codes; 4-bit: all 32 bits.
template <int BITS>
__device__ __forceinline__ uint32_t code8_fast(const uint4 &raw, const float *r, const float *z, const float *thr,
                                               float lo, bool &near) {
  constexpr float QMAX = float((1 << BITS) - 1);
  float acc[2] = {0.0f, 0.0f};
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const f16x2 h = as_h2(word_of(raw, k >> 1));
    const float y = __builtin_fmaf((float)h[k & 1], r[k], 0.0f);
    const float t = rintf(y);
    near |= fabsf(y - t) >= thr[k];
    const float code = __builtin_amdgcn_fmed3f(t - z[k], lo, QMAX);
    const int half = (BITS == 4 && k >= 4) ? 1 : 0;
    const int pos = (BITS == 4) ? (k & 3) : k;
    acc[half] = __builtin_fmaf(code, float(1u << (BITS * pos)), acc[half]);
  }
  if constexpr (BITS == 2) return (uint32_t)acc[0];
  return (uint32_t)acc[0] | ((uint32_t)acc[1] << 16);
}

// The same word through the correctly rounded quotient (code_of).
template <int BITS>
__device__ __forceinline__ uint32_t code8_exact(const uint4 &raw, const float *s, const float *z, float lo) {
  constexpr float QMAX = float((1 << BITS) - 1);
  uint32_t word = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t w = word_of(raw, k >> 1);
    const float x = h2f((uint16_t)((k & 1) ? (w >> 16) : (w & 0xffffu)));
    word |= code_of(x, GroupParams{s[k], z[k], 0.0f}, lo, QMAX) << (BITS * k);
  }
  return word;
}

// 2-bit rows: a lane's 8 codes fill half a word.  Lanes cs and cs ^ 1 hold the
// two halves of one word for the same rows, so for a pair of rows (a, b) the
// even lane assembles row a's word and the odd lane row b's, each taking the
// other half from its neighbour (a quad swap).  Returns the word of row
// a + (cs & 1).
__device__ __forceinline__ uint32_t pair_words(uint32_t ua, uint32_t ub, bool odd) {
  const uint32_t send = odd ? ua : ub;
  const uint32_t recv = (uint32_t)__builtin_amdgcn_mov_dpp((int)send, 0xB1, 0xF, 0xF, true);  // quad_perm 1,0,3,2
  return odd ? (recv | (ub << 16)) : (ua | (recv << 16));
}

// One value row of the KIVI layout (128 fp16 channels of one token at src)
// quantized into cache row `row` (unit * cap + token) by a whole wave, with
// the arithmetic of the value quantizer kernel: groups of G channels, the
// group minimum and maximum as one packed (min, -max) fp16 pair reduced over
// the group's lanes, group_params, and the tile coder with its exact
// fallback, so the codes and metadata are those the quantizer kernel writes
// for the same row.  Lane l takes channels 8 (l % 16) .. + 7; the four
// 16-lane rows of the wave repeat the work and the first one stores.  Every
// lane of the wave must call it (cross-lane moves and a wave vote).
template <int BITS, int G>
__device__ __forceinline__ void quantize_value_row(const CacheView &c, const uint16_t *__restrict__ src,
                                                   int64_t row) {
  constexpr int LPG = G / 8;                  // lanes per value group
  constexpr int NG = kHeadDim / G;
  constexpr int W = kHeadDim * BITS / 32;     // code words per row
  constexpr float QMAX = float((1 << BITS) - 1);
  const int lane = threadIdx.x & 63, cs = lane & 15, j = cs / LPG;
  const uint4 raw = reinterpret_cast<const uint4 *>(src)[cs];
  const f16x2 h0 = as_h2(raw.x), h1 = as_h2(raw.y), h2 = as_h2(raw.z), h3 = as_h2(raw.w);
  const f16x2 lo = hmin(hmin(h0, h1), hmin(h2, h3)), hi = hmax(hmax(h0, h1), hmax(h2, h3));
  const f16x2 lo2 = hmin(lo, lo.yx), hi2 = hmax(hi, hi.yx);
  f16x2 v = {lo2.x, -hi2.x};
  v = hmin(v, as_h2((uint32_t)__builtin_amdgcn_mov_dpp((int)as_u32(v), 0xB1, 0xF, 0xF, true)));   // lane ^ 1
  v = hmin(v, as_h2((uint32_t)__builtin_amdgcn_mov_dpp((int)as_u32(v), 0x4E, 0xF, 0xF, true)));   // lane ^ 2
  if constexpr (LPG >= 8)
    v = hmin(v, as_h2((uint32_t)__builtin_amdgcn_mov_dpp((int)as_u32(v), 0x141, 0xF, 0xF, true)));  // other quad of 8
  if constexpr (LPG >= 16)
    v = hmin(v, as_h2((uint32_t)__builtin_amdgcn_mov_dpp((int)as_u32(v), 0x140, 0xF, 0xF, true)));  // other half of 16
  const float mn = (float)v.x, mx = -(float)v.y;
  const GroupParams p = group_params(mn, mx, QMAX, c.meta != 0);
  const float thr1 = tie_threshold(fmaxf(fabsf(mn), fabsf(mx)), p.r);
  float r[8], z[8], thr[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    r[k] = p.r;
    z[k] = p.z;
    thr[k] = thr1;
  }
  bool near = false;
  uint32_t u = code8_fast<BITS>(raw, r, z, thr, 0.0f, near);
  if (__any(near)) {
    float sv[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) sv[k] = p.s;
    u = code8_exact<BITS>(raw, sv, z, 0.0f);
  }
  if (lane < 16 && cs % LPG == 0) {
    if (c.meta) {
      reinterpret_cast<uint32_t *>(c.v_scale)[row * NG + j] = pack_meta(p.s, p.z);
    } else {
      c.v_scale[row * NG + j] = p.s;
      c.v_zero[row * NG + j] = static_cast<int16_t>(p.z);
    }
  }
  if constexpr (BITS == 2) {
    // a word holds the 8 codes of an even lane and then those of the odd one
    const uint32_t odd = (uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0xB1, 0xF, 0xF, true);   // lane ^ 1
    if (lane < 16 && (cs & 1) == 0) c.v_codes[row * W + (cs >> 1)] = u | (odd << 16);
  } else {
    if (lane < 16) c.v_codes[row * W + cs] = u;
  }
}

}  // namespace
}  // namespace kvq
