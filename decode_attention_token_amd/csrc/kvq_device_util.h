// Small device helpers shared by every HIP source of libkvq.  Private.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

namespace kvq {
namespace {

// fp16 bit pattern -> float (exact).
__device__ __forceinline__ float h2f(uint16_t h) { return __half2float(__ushort_as_half(h)); }

}  // namespace
}  // namespace kvq
