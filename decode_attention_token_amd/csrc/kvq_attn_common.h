// Device-side building blocks shared by the decode-attention kernels
// (kvq_attn.hip for the KIVI layout, kvq_innerq.hip for the InnerQ-style
// layout): cross-lane reductions, code unpacking, raw buffer loads, the
// per-lane online-softmax state, the fp16-token step and the combination of a
// workgroup's waves into one (max, sum, acc) result.  Private to the HIP
// sources; include after kvq_internal.h.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include "kvq_device_util.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kWave = 64;
constexpr int kWaves = 8;                         // waves per workgroup
constexpr int kThreads = kWave * kWaves;
constexpr int kParts = kThreads / 128;            // thread groups of 128 in the reductions
constexpr float kMargin = 8.0f;    // log2 units: weights stay below 2^8 between rescales

typedef float f2 __attribute__((ext_vector_type(2)));

// 2^x with the hardware instruction; arguments here are <= kMargin or -inf,
// and results below the fp32 normal range only ever weight negligible terms.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------- cross-lane
// DPP controls (gfx9): quad_perm [1,0,3,2] and [2,3,0,1] swap lanes xor 1 and
// xor 2; row_half_mirror / row_mirror reverse 8- and 16-lane blocks, which
// pairs equal-sum halves once the smaller blocks are reduced.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over aligned blocks of N lanes; every lane of a block gets the same bits.
template <int N>
__device__ __forceinline__ float block_sum(float v) {
  if constexpr (N >= 2) v += dpp<0xB1>(v);
  if constexpr (N >= 4) v += dpp<0x4E>(v);
  if constexpr (N >= 8) v += dpp<0x141>(v);
  if constexpr (N >= 16) v += dpp<0x140>(v);
  static_assert(N <= 16, "block wider than a DPP row");
  return v;
}

template <int N>
__device__ __forceinline__ float block_max(float v) {
  if constexpr (N >= 2) v = fmaxf(v, dpp<0xB1>(v));
  if constexpr (N >= 4) v = fmaxf(v, dpp<0x4E>(v));
  if constexpr (N >= 8) v = fmaxf(v, dpp<0x141>(v));
  if constexpr (N >= 16) v = fmaxf(v, dpp<0x140>(v));
  return v;
}

__device__ __forceinline__ float lane_of(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Whole-wave sum / max, returned uniformly to every lane.
__device__ __forceinline__ float wave_sum(float v) {
  v = block_sum<16>(v);
  return (lane_of(v, 0) + lane_of(v, 16)) + (lane_of(v, 32) + lane_of(v, 48));
}

__device__ __forceinline__ float wave_max(float v) {
  v = block_max<16>(v);
  return fmaxf(fmaxf(lane_of(v, 0), lane_of(v, 16)), fmaxf(lane_of(v, 32), lane_of(v, 48)));
}

// Issue priority from progress: the SIMD arbiter favours the oldest waves,
// so with equal shares of work the younger waves (and the second workgroup
// on a compute unit) would finish well after the older ones.  A wave with
// more of its steps left gets a higher priority, so all waves finish close
// together.  `left` and `total` are wave-uniform step counts.
__device__ __forceinline__ void progress_priority(int left, int total) {
  const int band = (4 * left) / (total + 1);
  if (band >= 3) __builtin_amdgcn_s_setprio(3);
  else if (band == 2) __builtin_amdgcn_s_setprio(2);
  else if (band == 1) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

// A wave-uniform value moved to a scalar register.
__device__ __forceinline__ float uniform(float v) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------- unpacking
// One 32-bit code word -> floats equal to code * scale, in channel order.
// 2-bit: a nibble 0b00cc read as an fp4 e2m1 number is exactly cc / 2, so the
// word is masked into nibbles and two nibbles convert per instruction
// (16 codes: 3 integer + 8 conversion instructions).
// 4-bit: a byte 0b0000cccc read as an fp8 e4m3 number is exactly cccc * 2^-9
// (subnormals 0..7, then the first binade), two bytes per instruction.
template <int BITS>
struct Unpack;

template <>
struct Unpack<2> {
  static constexpr float scale = 0.5f;
  __device__ static __forceinline__ void run(uint32_t w, float *out) {
    const uint32_t m0 = w & 0x33333333u;          // nibble k: code 2k
    const uint32_t m1 = (w >> 2) & 0x33333333u;   // nibble k: code 2k + 1
    f2 a0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(m0, 1.0f, 0);
    f2 b0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(m1, 1.0f, 0);
    f2 a1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(m0, 1.0f, 1);
    f2 b1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(m1, 1.0f, 1);
    f2 a2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(m0, 1.0f, 2);
    f2 b2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(m1, 1.0f, 2);
    f2 a3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(m0, 1.0f, 3);
    f2 b3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(m1, 1.0f, 3);
    out[0] = a0.x;  out[2] = a0.y;  out[1] = b0.x;  out[3] = b0.y;
    out[4] = a1.x;  out[6] = a1.y;  out[5] = b1.x;  out[7] = b1.y;
    out[8] = a2.x;  out[10] = a2.y; out[9] = b2.x;  out[11] = b2.y;
    out[12] = a3.x; out[14] = a3.y; out[13] = b3.x; out[15] = b3.y;
  }
};

template <>
struct Unpack<4> {
  static constexpr float scale = 1.0f / 512.0f;
  __device__ static __forceinline__ void run(uint32_t w, float *out) {
    const uint32_t m0 = w & 0x0F0F0F0Fu;          // byte k: code 2k
    const uint32_t m1 = (w >> 4) & 0x0F0F0F0Fu;   // byte k: code 2k + 1
    f2 a = __builtin_amdgcn_cvt_pk_f32_fp8(m0, false);
    f2 b = __builtin_amdgcn_cvt_pk_f32_fp8(m0, true);
    f2 c = __builtin_amdgcn_cvt_pk_f32_fp8(m1, false);
    f2 d = __builtin_amdgcn_cvt_pk_f32_fp8(m1, true);
    out[0] = a.x; out[2] = a.y; out[4] = b.x; out[6] = b.y;
    out[1] = c.x; out[3] = c.y; out[5] = d.x; out[7] = d.y;
  }
};

// Raw buffer loads: an SGPR resource per stream, a lane-constant VGPR byte
// offset and a uniform SGPR byte offset per step, so no vector ALU work goes
// into addressing; out-of-range offsets read zero instead of faulting.
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kStream = 2;   // cache policy: non-temporal (the cache is read once per call)

__device__ __forceinline__ Rsrc rsrc_of(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, kRsrcWord3);
}

template <int N>
__device__ __forceinline__ void bload_words(Rsrc r, uint32_t voff, uint32_t soff, uint32_t *w) {
  if constexpr (N == 4) {
    const uint4 v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kStream));
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  } else if constexpr (N == 2) {
    const uint2 v = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kStream));
    w[0] = v.x; w[1] = v.y;
  } else {
    static_assert(N == 1, "words per lane");
    w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, kStream);
  }
}

// Result staging shared by the main and tail paths: acc[HPG][128], (m, l)[HPG],
// per-wave (m, l)[kWaves][HPG].
struct Stage {
  float *acc, *ml, *wml;
};

template <int HPG>
__device__ __forceinline__ Stage stage_of(float *smem, int work) {
  Stage s;
  s.acc = smem + work;
  s.ml = s.acc + HPG * kHeadDim;
  s.wml = s.ml + 2 * HPG;
  return s;
}

// Writes this part's result: the normalized output when the unit has one
// part, else an unnormalized (acc, m, l) record for the merge kernel.
template <int HPG>
__device__ void finish_part(const AttnArgs &a, int unit, int part, const Stage &st) {
  const int tid = threadIdx.x;
  const int b = unit / a.hkv, hk = unit % a.hkv;
  const int nparts = a.nparts;
  if (nparts == 1) {
    for (int i = tid; i < HPG * kHeadDim; i += blockDim.x) {
      const int h = i / kHeadDim, c = i % kHeadDim;
      const int64_t bh = (int64_t)b * a.hq + hk * HPG + h;
      a.out[bh * kHeadDim + c] = st.acc[i] / st.ml[2 * h + 1];
    }
    return;
  }
  for (int i = tid; i < HPG * (kHeadDim + 2); i += blockDim.x) {
    const int h = i / (kHeadDim + 2), c = i % (kHeadDim + 2);
    const int64_t bh = (int64_t)b * a.hq + hk * HPG + h;
    float *rec = a.partials + (bh * nparts + part) * kPartialStride;
    rec[c] = c < kHeadDim ? st.acc[h * kHeadDim + c] : st.ml[2 * h + (c - kHeadDim)];
  }
}


// Merge of one query head's split records (nparts records of kPartialStride
// floats from p: acc[128], max, sum) for channel c: m = max m_i,
// l = sum l_i 2^(m_i - m), out = sum acc_i 2^(m_i - m) / l.  Records are read
// kMergeBatch at a time: every load of a batch is issued before any is used,
// so a batch costs one memory round trip.  The batches fold into a running
// (max, sum, acc) by the same rescaling rule the kernels use inside a split.
constexpr int kMergeBatch = 8;

struct PlainLoad {
  __device__ float operator()(const float *p) const { return *p; }
};

template <class Load = PlainLoad>
__device__ __forceinline__ float merge_records(const float *__restrict__ p, int nparts, int c, Load ld = Load()) {
  float M = -INFINITY, L = 0.0f, acc = 0.0f;
  for (int i0 = 0; i0 < nparts; i0 += kMergeBatch) {
    float mv[kMergeBatch], lv[kMergeBatch], av[kMergeBatch];
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      const bool in = i0 + j < nparts;
      const float *r = p + (int64_t)(in ? i0 + j : i0) * kPartialStride;
      mv[j] = in ? ld(r + kHeadDim) : -INFINITY;
      lv[j] = ld(r + kHeadDim + 1);
      av[j] = ld(r + c);
    }
    float bm = mv[0];
#pragma unroll
    for (int j = 1; j < kMergeBatch; ++j) bm = fmaxf(bm, mv[j]);
    if (bm == -INFINITY) continue;   // no tokens in this batch's records
    if (bm > M) {
      const float f = (M == -INFINITY) ? 0.0f : exp2f(M - bm);
      L *= f;
      acc *= f;
      M = bm;
    }
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      if (mv[j] == -INFINITY) continue;   // empty record (or past the last one)
      const float f = exp2f(mv[j] - M);
      L = fmaf(f, lv[j], L);
      acc = fmaf(f, av[j], acc);
    }
  }
  return acc / L;
}

// Agent-scope atomic load: reads what another XCD wrote with an agent-scope
// atomic store.
struct CoherentLoad {
  __device__ float operator()(const float *p) const {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
};

// Per-unit counters in the workspace (kCtrWords u32 per unit):
//   word 0     ticket: waves of the work-queue schedule take chunks of the
//              unit's tokens from it (queue_grab);
//   words 2-3  one 64-bit election word: the call's epoch in the high half
//              and, in the low half, the workgroups that finished (bits
//              24..31) and the chunks they took (bits 0..23).
__device__ __forceinline__ uint32_t queue_grab(uint32_t *ctr, int lane) {
  uint32_t v = 0;
  if (lane == 0) v = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return v;   // in lane 0; read it (readlane) a chunk later
}

// End of a part of a unit split over a.splits workgroups.
// s_flag: LDS, [NW] chunks taken per wave, then one word for the result.
// With several parts, the part's (acc, m, l) record goes out with
// agent-scope atomic stores (the records cross XCDs, whose L2 caches are not
// kept coherent for ordinary stores) and every wave waits for its own stores
// before the workgroup is counted in.  Counting is a compare-and-swap on the
// unit's election word: a word whose epoch is not this call's (a.epoch, new
// for every launch) counts as empty, so a word left over from an earlier
// call, interrupted or never zero-filled, cannot bring the count forward.
// Exactly one workgroup, the one whose swap completes the count, is the
// unit's last: it checks the chunk total (a total short of nchunks means the
// ticket did not start at zero, and its outputs are NaN instead of a wrong
// result), returns the ticket and the word to zero for the next call and
// merges every record of the unit; a single part writes the normalized
// output itself.  Ordering: each record store and the swap are agent-scope
// atomics, the stores are complete (s_waitcnt 0) before the barrier that
// precedes the swap, and the last workgroup reads the records only after
// its swap has returned, with agent-scope loads that go to the coherent
// level.
template <int HPG, int NW>
__device__ void queue_finish(const AttnArgs &a, int unit, int split, const Stage &st, uint32_t *s_flag,
                             uint32_t nchunks) {
  const int tid = threadIdx.x, nthreads = blockDim.x;
  const int b = unit / a.hkv, hk = unit % a.hkv;
  uint32_t *ctr = a.ctr + kCtrWords * unit;
  if (a.nparts > 1) {
    for (int i = tid; i < HPG * (kHeadDim + 2); i += nthreads) {
      const int h = i / (kHeadDim + 2), c = i % (kHeadDim + 2);
      const int64_t bh = (int64_t)b * a.hq + hk * HPG + h;
      float *rec = a.partials + (bh * a.nparts + split) * kPartialStride;
      __hip_atomic_store(rec + c, c < kHeadDim ? st.acc[h * kHeadDim + c] : st.ml[2 * h + (c - kHeadDim)],
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  if (tid == 0) {
    uint32_t took = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) took += s_flag[w];
    uint64_t *word = reinterpret_cast<uint64_t *>(ctr + 2);
    const uint64_t tag = (uint64_t)a.epoch << 32;
    // first guess: the word is clean (every call leaves it at zero)
    uint64_t seen = 0, base;
    for (;;) {
      base = (seen >> 32) == a.epoch ? (seen & 0xffffffffull) : 0ull;
      uint64_t expect = seen;
      if (__hip_atomic_compare_exchange_strong(word, &expect, tag | (base + ((1u << 24) | took)), __ATOMIC_RELAXED,
                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
        break;
      seen = expect;
    }
    uint32_t last = 0;
    if ((uint32_t)(base >> 24) + 1u == (uint32_t)a.splits) {
      last = ((uint32_t)(base & 0xffffffu) + took == nchunks) ? 1u : 2u;
      __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(word, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    s_flag[NW] = last;
  }
  __syncthreads();
  const uint32_t last = s_flag[NW];
  if (a.nparts == 1) {
    if (last == 2 && tid < HPG) st.ml[2 * tid + 1] = __builtin_nanf("");
    __syncthreads();
    finish_part<HPG>(a, unit, split, st);
    return;
  }
  if (last == 0) return;
  for (int i = tid; i < HPG * kHeadDim; i += nthreads) {
    const int h = i / kHeadDim, c = i % kHeadDim;
    const int64_t bh = (int64_t)b * a.hq + hk * HPG + h;
    a.out[bh * kHeadDim + c] =
        last == 2 ? __builtin_nanf("")
                  : merge_records(a.partials + bh * a.nparts * kPartialStride, a.nparts, c, CoherentLoad());
  }
}

// Occupancy target: four waves per SIMD (at most 128 VGPRs) for the MHA
// tilings, two for the grouped-query tiling that keeps 4 heads in registers.
template <int HPG>
constexpr int kWavesPerEU = HPG == 1 ? 4 : 2;

// Floats of the LDS area combine_waves uses: per wave and query head, one
// row of 128 channel sums for each of the wave's four 16-lane rows.
template <int HPG>
constexpr int kRedFloats = kWaves * HPG * 4 * kHeadDim;

// Floats of the Stage area after the work area.
template <int HPG>
constexpr int kStageFloats = HPG * kHeadDim + 2 * HPG + 2 * kWaves * HPG;

// Online-softmax state of one lane for HPG query heads: the wave-uniform
// running maximum m (log2 units), raised only when some score passes
// mthr = m + kMargin so the rescale branch is rare and uniform; the lane's
// share of the weight sum; the weighted code sums of its CPL channels; and
// the weighted zero-point terms of its NVG value groups.
template <int HPG, int CPL, int NVG>
struct Online {
  float m[HPG], mthr[HPG], lsum[HPG], acc[HPG][CPL], bias[HPG][NVG];

  __device__ __forceinline__ void init() {
#pragma unroll
    for (int h = 0; h < HPG; ++h) {
      m[h] = -INFINITY;
      mthr[h] = -INFINITY;
      lsum[h] = 0.0f;
#pragma unroll
      for (int i = 0; i < CPL; ++i) acc[h][i] = 0.0f;
#pragma unroll
      for (int k = 0; k < NVG; ++k) bias[h][k] = 0.0f;
    }
  }

  // Weight 2^(sv - m) of a score; rescales the state first when any lane of
  // the wave passes the threshold.  Every call site has at least one finite
  // score in the wave, so m is finite after the first call.
  __device__ __forceinline__ float weight(int h, float sv) {
    if (__any(sv > mthr[h])) {
      const float mn = fmaxf(m[h], wave_max(sv));
      const float f = fast_exp2(m[h] - mn);
      m[h] = uniform(mn);   // wave-uniform: kept in scalar registers
      mthr[h] = uniform(mn + kMargin);
      lsum[h] *= f;
#pragma unroll
      for (int i = 0; i < CPL; ++i) acc[h][i] *= f;
#pragma unroll
      for (int k = 0; k < NVG; ++k) bias[h][k] *= f;
    }
    const float p = fast_exp2(sv - m[h]);
    lsum[h] += p;
    return p;
  }
};

// CPL consecutive fp16 values (16 bytes at a time) as floats.
template <int CPL>
__device__ __forceinline__ void fp16_row(const uint16_t *row, float *x) {
  static_assert(CPL % 8 == 0, "fp16 rows are read 16 bytes at a time");
#pragma unroll
  for (int i = 0; i < CPL; i += 8) {
    const uint4 w = *reinterpret_cast<const uint4 *>(row + i);
    const uint32_t w4[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[i + 2 * e] = h2f((uint16_t)(w4[e] & 0xffffu));
      x[i + 2 * e + 1] = h2f((uint16_t)(w4[e] >> 16));
    }
  }
}

// One token per group of LPT lanes whose keys and values each lane holds as
// floats for its CPL channels: scores them against the plain query
// qf = q * qscale and adds weight * U * v, so that the 1/U scaling of the
// quantized codes applies to these tokens too.  Lanes of an invalid token
// score -inf.
// The weights, wt[h] = weight * U, of one token from its key floats.
template <int HPG, int CPL, int NVG, int LPT>
__device__ __forceinline__ void token_weights(Online<HPG, CPL, NVG> &o, const float (&qf)[HPG][CPL], const float *kf,
                                              bool valid, float U, float *wt) {
#pragma unroll
  for (int h = 0; h < HPG; ++h) {
    float d0 = 0.0f, d1 = 0.0f;
#pragma unroll
    for (int i = 0; i < CPL; i += 2) {
      d0 = fmaf(qf[h][i], kf[i], d0);
      d1 = fmaf(qf[h][i + 1], kf[i + 1], d1);
    }
    float sv = block_sum<LPT>(d0 + d1);
    sv = valid ? sv : -INFINITY;
    wt[h] = o.weight(h, sv) * U;
  }
}

template <int HPG, int CPL, int NVG>
__device__ __forceinline__ void token_values(Online<HPG, CPL, NVG> &o, const float *wt, const float *vf) {
#pragma unroll
  for (int h = 0; h < HPG; ++h) {
#pragma unroll
    for (int i = 0; i < CPL; ++i) o.acc[h][i] = fmaf(wt[h], vf[i], o.acc[h][i]);
  }
}

template <int HPG, int CPL, int NVG, int LPT>
__device__ __forceinline__ void token_update(Online<HPG, CPL, NVG> &o, const float (&qf)[HPG][CPL], const float *kf,
                                             const float *vf, bool valid, float U) {
  float wt[HPG];
  token_weights<HPG, CPL, NVG, LPT>(o, qf, kf, valid, U, wt);
  token_values<HPG, CPL, NVG>(o, wt, vf);
}

// One fp16 token per group of LPT lanes (rows krow, vrow: this lane's CPL
// channels).
template <int HPG, int CPL, int NVG, int LPT>
__device__ __forceinline__ void fp16_token(Online<HPG, CPL, NVG> &o, const float (&qf)[HPG][CPL],
                                           const uint16_t *krow, const uint16_t *vrow, bool valid, float U) {
  float kf[CPL], vf[CPL];
  fp16_row<CPL>(krow, kf);
  fp16_row<CPL>(vrow, vf);
  token_update<HPG, CPL, NVG, LPT>(o, qf, kf, vf, valid, U);
}

// Sum over the token lanes of one 16-lane row that share channel slice j
// (lanes tl * LPT + j): rotates by 8 (and 4) within the row.  Every lane of
// the row gets its slice's row total.
template <int LPT>
__device__ __forceinline__ float sum_row_token_lanes(float v) {
  static_assert(LPT == 4 || LPT == 8, "token lanes per row");
  v += dpp<0x128>(v);                       // row_ror:8
  if constexpr (LPT == 4) v += dpp<0x124>(v);   // row_ror:4
  return v;
}

// Combines the waves of a workgroup and the token lanes of each wave into
// st.acc[h][128] (unnormalized, relative to the workgroup maximum) and
// st.ml[h] = (max, sum).  o.acc holds sums of weight * code * U per channel
// and o.bias the zero-point terms per value group; inv_u = 1 / U.  Each wave
// sums over the token lanes of each 16-lane row in registers and stores four
// rows per head; after one barrier, four threads per channel merge the
// waves' rows with their 2^(m_w - M) factors and sum with a quad swap.  Ends
// with a barrier; smem must hold kRedFloats<HPG> floats before the Stage area.
template <int HPG, int LPT, int NVG>
__device__ __forceinline__ void combine_waves(const Online<HPG, kHeadDim / LPT, NVG> &o, float *smem,
                                              const Stage &st, int wave, int lane, float inv_u) {
  constexpr int CPL = kHeadDim / LPT;
  const int tid = threadIdx.x, j = lane % LPT;
  float *rows = smem;   // [kWaves][HPG][4][128]
  __syncthreads();      // every wave is done with the work area
#pragma unroll
  for (int h = 0; h < HPG; ++h) {
    const float lw = wave_sum(o.lsum[h]) * (1.0f / LPT);
    float *row = rows + ((wave * HPG + h) * 4 + lane / 16) * kHeadDim + j * CPL;
#pragma unroll
    for (int i = 0; i < CPL; i += 4) {
      const int k0 = (NVG > 1) ? (i / (CPL / NVG)) : 0;
      const float b = o.bias[h][k0];
      float4 v;
      v.x = sum_row_token_lanes<LPT>(fmaf(o.acc[h][i], inv_u, b));
      v.y = sum_row_token_lanes<LPT>(fmaf(o.acc[h][i + 1], inv_u, b));
      v.z = sum_row_token_lanes<LPT>(fmaf(o.acc[h][i + 2], inv_u, b));
      v.w = sum_row_token_lanes<LPT>(fmaf(o.acc[h][i + 3], inv_u, b));
      if (lane % 16 < LPT) *reinterpret_cast<float4 *>(row + i) = v;
    }
    if (lane == 0) {
      st.wml[(wave * HPG + h) * 2] = o.m[h];
      st.wml[(wave * HPG + h) * 2 + 1] = lw;
    }
  }
  __syncthreads();
  static_assert((HPG * kHeadDim * 4) % kThreads == 0, "whole merge passes");
  for (int i = tid; i < HPG * kHeadDim * 4; i += kThreads) {
    const int r = i % 4, c = (i / 4) % kHeadDim, h = i / (4 * kHeadDim);
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, st.wml[(w * HPG + h) * 2]);
    float acc = 0.0f, L = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = st.wml[(w * HPG + h) * 2];
      const float f = (mw == -INFINITY) ? 0.0f : fast_exp2(mw - M);
      L = fmaf(f, st.wml[(w * HPG + h) * 2 + 1], L);
      acc = fmaf(f, rows[((w * HPG + h) * 4 + r) * kHeadDim + c], acc);
    }
    acc = block_sum<4>(acc);   // the four rows of channel c sit in one quad
    if (r == 0) {
      st.acc[h * kHeadDim + c] = acc;
      if (c == 0) {
        st.ml[2 * h] = M;
        st.ml[2 * h + 1] = L;
      }
    }
  }
  __syncthreads();
}

}  // namespace
}  // namespace kvq
