// Device-side quantizer pieces shared by kvq_quant.hip (KIVI layout) and
// kvq_innerq.hip (InnerQ-style layout): group scale and zero-point, the
// exactly rounded code map with its fast path, and 16-byte fp16 loads.
// Private to the HIP sources.
//
// Bit-exactness: every arithmetic step is one IEEE fp32 operation with round
// to nearest even (sub, div, rint), so the codes, scales and zero-points equal
// those of any other correctly rounded fp32 implementation of the same steps.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include "kvq_device_util.h"

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

}  // namespace
}  // namespace kvq
