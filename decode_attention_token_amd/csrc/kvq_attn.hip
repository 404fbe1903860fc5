// Split-K decode attention over the quantized KV cache, gfx950.
//
// Decoding one token must read the whole KV cache while the arithmetic units
// mostly wait (KIVI part of the juejin.cn page "大模型量化技术原理：KIVI、
// IntactKV、KVQuant", background section), so the kernel streams packed codes
// once and fuses dequantization into both products, in the spirit of the
// fused group-dequantize + GEMV kernel of the euno.news InnerQ summary
// (methodology 3 and 5: a group's shared scale is loaded once and reused for
// the whole group).
//
// Scores.  Keys carry one (S, Z) per (group of G tokens, channel), so for a
// group g the score of token t is
//     s_t = sum_c q_c S_gc (k_tc + Z_gc) = sum_c q'_c k_tc + beta_g,
//     q'_c = q_c S_gc,  beta_g = sum_c q'_c Z_gc,
// i.e. the group's scales are folded into the query once per group and the
// zero-points collapse into one bias; the inner loop is one FMA per code.
// Values carry (S, Z) per (token, group of G channels), so with softmax
// weight p_t the output accumulates w = p_t S_tj per token and group:
//     acc_c += w * v_tc,  bias_j += w * Z_tj,  out_c = (acc_c + bias_j) / l.
//
// Work split.  A workgroup of 8 waves handles one split of one unit (batch,
// kv head): a contiguous range of the unit's whole key groups.  The last
// split also takes the fp16 residual tokens when both their keys and values
// are fp16 (the chunked residual); otherwise (a FIFO value queue leaves keys
// quantized whose values are still fp16) one extra workgroup per unit runs a
// plain dequantize-then-dot tail path.  Within a wave, LPT lanes share a
// token and each owns 128 / LPT channels, so a wave step reads contiguous key
// and value rows with 8- or 16-byte loads; loads run two steps ahead of the
// arithmetic through a ring of three register buffers.  Each wave keeps its
// own online-softmax state with a wave-uniform running maximum that is raised
// only when a score exceeds it by more than a margin, so the rescale branch is
// rare and uniform.  A unit with one part writes its output directly;
// otherwise every part writes a (max, sum, acc) record and a second kernel
// merges them.  Softmax arithmetic is in log2 units.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kWave = 64;
constexpr int kWaves = 8;                         // waves per workgroup
constexpr int kThreads = kWave * kWaves;
constexpr int kParts = kThreads / 128;            // thread groups of 128 in the reductions
constexpr float kMargin = 8.0f;    // log2 units: weights stay below 2^8 between rescales
constexpr int kMaxTail = 512 + 127;  // residual <= 512, group <= 128

typedef float f2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float h2f(uint16_t h) { return __half2float(__ushort_as_half(h)); }

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

template <int N>
__device__ __forceinline__ void load_words(const uint32_t *p, uint32_t *w) {
  if constexpr (N == 4) {
    const uint4 v = *reinterpret_cast<const uint4 *>(p);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  } else if constexpr (N == 2) {
    const uint2 v = *reinterpret_cast<const uint2 *>(p);
    w[0] = v.x; w[1] = v.y;
  } else {
    static_assert(N == 1, "words per lane");
    w[0] = *p;
  }
}

// ---------------------------------------------------------------- geometry
template <int BITS, int GS, int HPG, int LPT>
struct Geo {
  static constexpr int CPL = kHeadDim / LPT;             // channels per lane
  static constexpr int TPS = kWave / LPT;                // tokens per wave step
  static constexpr int PER = 32 / BITS;                  // codes per word
  static constexpr int WPL = CPL / PER;                  // code words per lane per token
  static constexpr int W = kHeadDim / PER;               // words per token row
  static constexpr int NVG = CPL >= GS ? CPL / GS : 1;   // value groups per lane
  static constexpr int VGR = kHeadDim / GS;              // value groups per row
  static constexpr int SPG = GS / TPS;                   // wave steps per key group
  static constexpr int RS = kHeadDim + 4;                // padded reduction row (floats)
  static constexpr int RED = kWaves * TPS * RS + kParts * kHeadDim;
  static constexpr int QPW = HPG * (kHeadDim + 8);                // per wave: q'[HPG][128], beta[HPG][8]
  static constexpr int QP = kWaves * QPW;
  static constexpr int TAIL = HPG * kMaxTail + kParts * HPG * kHeadDim;
  static constexpr int WORK = RED > QP ? (RED > TAIL ? RED : TAIL) : (QP > TAIL ? QP : TAIL);
  static constexpr int RES = HPG * kHeadDim + 2 * HPG + 2 * kWaves * HPG;
  static constexpr int SMEM = WORK + RES;                // floats
};

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

// ---------------------------------------------------------------- tail path
// Tokens [n_main, n): keys and values may each be quantized or fp16 per token.
// Plain dequantize-then-dot: a wave per token for scores, a thread per
// channel for P.V.
template <int BITS, int HPG>
__device__ void decode_tail(const AttnArgs &a, int unit, float *smem, const Stage &st) {
  constexpr int PER = 32 / BITS;
  constexpr int W = kHeadDim / PER;
  constexpr uint32_t MASK = (1u << BITS) - 1u;
  const int G = a.c.group;
  const int VGR = kHeadDim / G;
  const int R = a.c.residual;
  const int64_t cap = a.c.cap;
  const int64_t t0 = a.n_main;
  const int nt = (int)(a.n - a.n_main);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = unit / a.hkv, hk = unit % a.hkv;
  float *s_sc = smem;                    // [HPG][nt] scores, then weights
  float *s_half = smem + HPG * nt;       // [kParts][HPG][128]

  float qa[HPG], qb[HPG];
#pragma unroll
  for (int h = 0; h < HPG; ++h) {
    const uint16_t *qp = a.q + ((int64_t)(b * a.hq + hk * HPG + h)) * kHeadDim + 2 * lane;
    qa[h] = h2f(qp[0]) * a.qscale;
    qb[h] = h2f(qp[1]) * a.qscale;
  }
  const int c0 = 2 * lane;
  for (int i = wave; i < nt; i += kWaves) {
    const int64_t t = t0 + i;
    float k0, k1;
    if (t < a.nq_k) {
      const int64_t g = t / G;
      const uint32_t word = a.c.k_codes[((int64_t)unit * cap + t) * W + c0 / PER];
      const int sh = (c0 % PER) * BITS;
      const float *S = a.c.k_scale + ((int64_t)unit * (cap / G) + g) * kHeadDim + c0;
      const int16_t *Z = a.c.k_zero + ((int64_t)unit * (cap / G) + g) * kHeadDim + c0;
      k0 = ((float)((word >> sh) & MASK) + (float)Z[0]) * S[0];
      k1 = ((float)((word >> (sh + BITS)) & MASK) + (float)Z[1]) * S[1];
    } else {
      const uint16_t *r = a.c.k_resid + ((int64_t)unit * R + (t % R)) * kHeadDim + c0;
      k0 = h2f(r[0]);
      k1 = h2f(r[1]);
    }
#pragma unroll
    for (int h = 0; h < HPG; ++h) {
      const float d = wave_sum(fmaf(qa[h], k0, qb[h] * k1));
      if (lane == 0) s_sc[h * nt + i] = d;
    }
  }
  __syncthreads();
  if (wave < HPG) {
    const int h = wave;
    float mx = -INFINITY;
    for (int i = lane; i < nt; i += kWave) mx = fmaxf(mx, s_sc[h * nt + i]);
    mx = wave_max(mx);
    float l = 0.0f;
    for (int i = lane; i < nt; i += kWave) {
      const float p = exp2f(s_sc[h * nt + i] - mx);
      s_sc[h * nt + i] = p;
      l += p;
    }
    l = wave_sum(l);
    if (lane == 0) {
      st.ml[2 * h] = nt > 0 ? mx : -INFINITY;
      st.ml[2 * h + 1] = l;
    }
  }
  __syncthreads();
  const int c = tid & (kHeadDim - 1);
  const int half = tid >> 7;
  float acc[HPG];
#pragma unroll
  for (int h = 0; h < HPG; ++h) acc[h] = 0.0f;
  for (int i = half; i < nt; i += kParts) {
    const int64_t t = t0 + i;
    float v;
    if (t < a.nq_v) {
      const uint32_t word = a.c.v_codes[((int64_t)unit * cap + t) * W + c / PER];
      const int64_t gi = ((int64_t)unit * cap + t) * VGR + c / G;
      v = ((float)((word >> ((c % PER) * BITS)) & MASK) + (float)a.c.v_zero[gi]) * a.c.v_scale[gi];
    } else {
      v = h2f(a.c.v_resid[((int64_t)unit * R + (t % R)) * kHeadDim + c]);
    }
#pragma unroll
    for (int h = 0; h < HPG; ++h) acc[h] = fmaf(s_sc[h * nt + i], v, acc[h]);
  }
#pragma unroll
  for (int h = 0; h < HPG; ++h) s_half[(half * HPG + h) * kHeadDim + c] = acc[h];
  __syncthreads();
  for (int i = tid; i < HPG * kHeadDim; i += blockDim.x) {
    float t = 0.0f;
#pragma unroll
    for (int p = 0; p < kParts; ++p) t += s_half[p * HPG * kHeadDim + i];
    st.acc[i] = t;
  }
  __syncthreads();
}

// ---------------------------------------------------------------- main path
template <int WPL, int NVG>
struct StepBuf {
  uint32_t kw[WPL];
  uint32_t vw[WPL];
  float vs[NVG];
  uint32_t vz;       // NVG int16 zero-points
  float2 ks;         // key scales of channels 2*lane, 2*lane+1 (this step's group)
  uint32_t kz;       // their int16 zero-points
};

// Occupancy target: four waves per SIMD (at most 128 VGPRs) for the MHA
// tilings, two for the grouped-query tiling that keeps 4 heads in registers.
template <int HPG>
constexpr int kWavesPerEU = HPG == 1 ? 4 : 2;

template <int BITS, int GS, int HPG, int LPT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWavesPerEU<HPG>, 8)))
void decode_attn_kernel(AttnArgs a) {
  using Gm = Geo<BITS, GS, HPG, LPT>;
  constexpr int CPL = Gm::CPL, TPS = Gm::TPS, PER = Gm::PER, WPL = Gm::WPL, W = Gm::W;
  constexpr int NVG = Gm::NVG, VGR = Gm::VGR, SPG = Gm::SPG;
  constexpr float U = Unpack<BITS>::scale;
  constexpr float INV_U = 1.0f / U;
  static_assert(GS % TPS == 0, "a wave step must stay inside one key group");
  static_assert(WPL >= 1, "lane slice must hold whole words");
  static_assert(CPL % 8 == 0, "fp16 residual rows are read 16 bytes at a time");
  using Buf = StepBuf<WPL, NVG>;

  __shared__ __attribute__((aligned(16))) float smem[Gm::SMEM];
  const Stage st = stage_of<HPG>(smem, Gm::WORK);

  const int units = a.batch * a.hkv;
  int blk = blockIdx.x;
  if (a.tail_wg) {
    if (blk < units) {
      decode_tail<BITS, HPG>(a, blk, smem, st);
      finish_part<HPG>(a, blk, a.splits, st);
      return;
    }
    blk -= units;
  }
  const int split = blk / units;
  const int unit = blk % units;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
  const int j = lane % LPT, tl = lane / LPT;
  const int b = unit / a.hkv, hk = unit % a.hkv;
  const int64_t cap = a.c.cap;
  const int ngroups = (int)(a.n_main / GS);
  const int g0 = (int)((int64_t)ngroups * split / a.splits);
  const int g1 = (int)((int64_t)ngroups * (split + 1) / a.splits);
  const int wg0 = g0 + (g1 - g0) * wave / kWaves;
  const int wg1 = g0 + (g1 - g0) * (wave + 1) / kWaves;
  const int nsteps = (wg1 - wg0) * SPG;

  // query (log2 units, divided by the unpack scale) for channels 2*lane,
  // 2*lane+1, used to fold key scales
  float qa[HPG], qb[HPG];
#pragma unroll
  for (int h = 0; h < HPG; ++h) {
    const uint16_t *qp = a.q + ((int64_t)(b * a.hq + hk * HPG + h)) * kHeadDim + 2 * lane;
    qa[h] = h2f(qp[0]) * (a.qscale * INV_U);
    qb[h] = h2f(qp[1]) * (a.qscale * INV_U);
  }

  // per-wave folded-query buffer: q'[h][128] then the slice biases beta[h][LPT]
  float *lds_qp = smem + wave * Gm::QPW;
  float *lds_beta = lds_qp + HPG * kHeadDim;
  constexpr int FOLD = CPL / 2;   // fold lanes (two channels each) per lane slice
  static_assert(FOLD <= 16 && (FOLD & (FOLD - 1)) == 0, "slice bias must reduce within a DPP row");
  float qf[HPG][CPL];
  float beta[HPG];   // zero-point bias of this lane's channel slice for the current key group
  float m[HPG], mthr[HPG], lsum[HPG], acc[HPG][CPL], bias[HPG][NVG];
#pragma unroll
  for (int h = 0; h < HPG; ++h) {
    m[h] = -INFINITY;
    mthr[h] = -INFINITY;
    lsum[h] = 0.0f;
    beta[h] = 0.0f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      acc[h][i] = 0.0f;
      qf[h][i] = 0.0f;
    }
#pragma unroll
    for (int k = 0; k < NVG; ++k) bias[h][k] = 0.0f;
  }

  // per-unit buffer resources (uniform); lane-constant byte offsets
  const int64_t ngr_cap = cap / GS;
  const Rsrc rkc = rsrc_of(a.c.k_codes + (int64_t)unit * cap * W, (uint32_t)(cap * W * 4));
  const Rsrc rvc = rsrc_of(a.c.v_codes + (int64_t)unit * cap * W, (uint32_t)(cap * W * 4));
  const Rsrc rvs = rsrc_of(a.c.v_scale + (int64_t)unit * cap * VGR, (uint32_t)(cap * VGR * 4));
  const Rsrc rvz = rsrc_of(a.c.v_zero + (int64_t)unit * cap * VGR, (uint32_t)(cap * VGR * 2));
  const Rsrc rks = rsrc_of(a.c.k_scale + (int64_t)unit * ngr_cap * kHeadDim, (uint32_t)(ngr_cap * kHeadDim * 4));
  const Rsrc rkz = rsrc_of(a.c.k_zero + (int64_t)unit * ngr_cap * kHeadDim, (uint32_t)(ngr_cap * kHeadDim * 2));
  const uint32_t code_lane = (uint32_t)(tl * W + j * WPL) * 4u;
  const uint32_t vmeta_lane = (uint32_t)(tl * VGR + (j * CPL) / GS);
  const uint32_t kmeta_lane = (uint32_t)(2 * lane);

  auto load = [&](Buf &bf, int s) {
    s = s < nsteps ? s : nsteps - 1;   // past the end: reload the last step (never processed)
    const uint32_t g = (uint32_t)(wg0 + s / SPG);
    const uint32_t tb = g * GS + (uint32_t)((s % SPG) * TPS);   // first token of the step (uniform)
    bload_words<WPL>(rkc, code_lane, tb * (W * 4), bf.kw);
    bload_words<WPL>(rvc, code_lane, tb * (W * 4), bf.vw);
    if constexpr (NVG == 2) {
      const float2 v2 = __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(rvs, vmeta_lane * 4, tb * (VGR * 4), kStream));
      bf.vs[0] = v2.x;
      bf.vs[1] = v2.y;
      bf.vz = __builtin_amdgcn_raw_buffer_load_b32(rvz, vmeta_lane * 2, tb * (VGR * 2), kStream);
    } else {
      static_assert(NVG == 1, "value groups per lane");
      bf.vs[0] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rvs, vmeta_lane * 4, tb * (VGR * 4), kStream));
      bf.vz = __builtin_amdgcn_raw_buffer_load_b16(rvz, vmeta_lane * 2, tb * (VGR * 2), kStream);
    }
    bf.ks = __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(rks, kmeta_lane * 4, g * (kHeadDim * 4), 0));
    bf.kz = __builtin_amdgcn_raw_buffer_load_b32(rkz, kmeta_lane * 2, g * (kHeadDim * 2), 0);
  };

  // online softmax with a lazily raised, wave-uniform maximum; returns p
  auto soft = [&](int h, float sv) -> float {
    if (__any(sv > mthr[h])) {
      const float mn = fmaxf(m[h], wave_max(sv));
      const float f = fast_exp2(m[h] - mn);
      m[h] = mn;
      mthr[h] = mn + kMargin;
      lsum[h] *= f;
#pragma unroll
      for (int i = 0; i < CPL; ++i) acc[h][i] *= f;
#pragma unroll
      for (int k = 0; k < NVG; ++k) bias[h][k] *= f;
    }
    const float p = fast_exp2(sv - m[h]);
    lsum[h] += p;
    return p;
  };

  auto process = [&](const Buf &bf, int s) {
    if (s % SPG == 0) {
      // new key group: fold its per-channel scales into the query; each block
      // of FOLD lanes holds one lane slice's channels and sums its share of
      // the zero-point bias
      const float z0 = (float)(int16_t)(bf.kz & 0xffffu);
      const float z1 = (float)(int16_t)(bf.kz >> 16);
#pragma unroll
      for (int h = 0; h < HPG; ++h) {
        const float p0 = qa[h] * bf.ks.x, p1 = qb[h] * bf.ks.y;   // q'/U
        const float part = block_sum<FOLD>(fmaf(p0, z0, p1 * z1));
        *reinterpret_cast<float2 *>(lds_qp + h * kHeadDim + 2 * lane) = make_float2(p0, p1);
        if (lane % FOLD == 0) lds_beta[h * 8 + lane / FOLD] = part * U;
      }
      wave_sync();
#pragma unroll
      for (int h = 0; h < HPG; ++h) {
#pragma unroll
        for (int i = 0; i < CPL; i += 4) {
          const float4 v = *reinterpret_cast<const float4 *>(lds_qp + h * kHeadDim + j * CPL + i);
          qf[h][i] = v.x;
          qf[h][i + 1] = v.y;
          qf[h][i + 2] = v.z;
          qf[h][i + 3] = v.w;
        }
        beta[h] = lds_beta[h * 8 + j];
      }
      wave_sync();
    }
    // scores
    float sc[HPG], d1[HPG];
#pragma unroll
    for (int h = 0; h < HPG; ++h) sc[h] = d1[h] = 0.0f;
#pragma unroll
    for (int w = 0; w < WPL; ++w) {
      float kf[PER];
      Unpack<BITS>::run(bf.kw[w], kf);
#pragma unroll
      for (int h = 0; h < HPG; ++h) {
#pragma unroll
        for (int i = 0; i < PER; i += 2) {
          sc[h] = fmaf(qf[h][w * PER + i], kf[i], sc[h]);
          d1[h] = fmaf(qf[h][w * PER + i + 1], kf[i + 1], d1[h]);
        }
      }
    }
    float p[HPG];
#pragma unroll
    for (int h = 0; h < HPG; ++h) p[h] = soft(h, block_sum<LPT>((sc[h] + d1[h]) + beta[h]));
    // values
    float vz[NVG];
    vz[0] = (float)(int16_t)(bf.vz & 0xffffu);
    if constexpr (NVG == 2) vz[1] = (float)(int16_t)(bf.vz >> 16);
#pragma unroll
    for (int h = 0; h < HPG; ++h) {
#pragma unroll
      for (int k = 0; k < NVG; ++k) bias[h][k] = fmaf(p[h] * bf.vs[k], vz[k], bias[h][k]);
    }
#pragma unroll
    for (int w = 0; w < WPL; ++w) {
      float vf[PER];
      Unpack<BITS>::run(bf.vw[w], vf);
      constexpr int SPAN = CPL / NVG;
      const int k = (w * PER) / SPAN;
#pragma unroll
      for (int h = 0; h < HPG; ++h) {
        const float wt = p[h] * bf.vs[k];
#pragma unroll
        for (int i = 0; i < PER; ++i) acc[h][w * PER + i] = fmaf(wt, vf[i], acc[h][w * PER + i]);
      }
    }
  };

  if (nsteps > 0) {
    Buf A, B, C;
    load(A, 0);
    load(B, 1);
    for (int s = 0; s < nsteps; s += 3) {
      load(C, s + 2);
      process(A, s);
      load(A, s + 3);
      if (s + 1 < nsteps) process(B, s + 1);
      load(B, s + 4);
      if (s + 2 < nsteps) process(C, s + 2);
    }
  }

  // fp16 residual tokens [n_main, n), all keys and values fp16: same lane
  // layout, plain query, weights p * U so the final 1/U scaling applies
  if (a.resid_main && split == a.splits - 1) {
    const int R = a.c.residual;
    const int rcount = (int)(a.n - a.n_main);
    const int rsteps = (rcount + TPS - 1) / TPS;
    const uint16_t *kr = a.c.k_resid + (int64_t)unit * R * kHeadDim + j * CPL;
    const uint16_t *vr = a.c.v_resid + (int64_t)unit * R * kHeadDim + j * CPL;
#pragma unroll
    for (int h = 0; h < HPG; ++h) {
      const uint16_t *qp = a.q + ((int64_t)(b * a.hq + hk * HPG + h)) * kHeadDim + j * CPL;
#pragma unroll
      for (int i = 0; i < CPL; ++i) qf[h][i] = h2f(qp[i]) * a.qscale;
    }
    if (a.k_new != nullptr && tid < 2 * (kHeadDim * 2 / 16)) {
      // fused step: store the new token into its ring slot
      constexpr int CH = kHeadDim * 2 / 16;
      const int which = tid / CH, ch = tid % CH;
      const uint4 *src = reinterpret_cast<const uint4 *>((which ? a.v_new : a.k_new) + (int64_t)unit * kHeadDim);
      uint4 *dst = reinterpret_cast<uint4 *>((which ? a.c.v_resid : a.c.k_resid) +
                                             ((int64_t)unit * R + (a.n - 1) % R) * kHeadDim);
      dst[ch] = src[ch];
    }
    for (int rs = wave; rs < rsteps; rs += kWaves) {
      const int64_t t = a.n_main + (int64_t)rs * TPS + tl;
      const bool valid = t < a.n;
      const int slot = (int)((valid ? t : a.n_main) % R);
      const bool fresh = a.k_new != nullptr && t == a.n - 1;   // not in the ring yet
      const uint16_t *krow = fresh ? a.k_new + (int64_t)unit * kHeadDim + j * CPL : kr + (int64_t)slot * kHeadDim;
      const uint16_t *vrow = fresh ? a.v_new + (int64_t)unit * kHeadDim + j * CPL : vr + (int64_t)slot * kHeadDim;
      float kf[CPL], vf[CPL];
#pragma unroll
      for (int i = 0; i < CPL; i += 8) {
        const uint4 kk = *reinterpret_cast<const uint4 *>(krow + i);
        const uint4 vv = *reinterpret_cast<const uint4 *>(vrow + i);
        const uint32_t kw4[4] = {kk.x, kk.y, kk.z, kk.w};
        const uint32_t vw4[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kf[i + 2 * e] = h2f((uint16_t)(kw4[e] & 0xffffu));
          kf[i + 2 * e + 1] = h2f((uint16_t)(kw4[e] >> 16));
          vf[i + 2 * e] = h2f((uint16_t)(vw4[e] & 0xffffu));
          vf[i + 2 * e + 1] = h2f((uint16_t)(vw4[e] >> 16));
        }
      }
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
        const float wt = soft(h, sv) * U;
#pragma unroll
        for (int i = 0; i < CPL; ++i) acc[h][i] = fmaf(wt, vf[i], acc[h][i]);
      }
    }
  }

  // ---- combine the waves and the TPS token lanes of each wave
  float lw[HPG];
#pragma unroll
  for (int h = 0; h < HPG; ++h) lw[h] = wave_sum(lsum[h]) * (1.0f / LPT);
  __syncthreads();   // every wave is done with its folded-query buffer
  float *s_red = smem;                              // [kWaves*TPS][RS]
  float *s_half = smem + kWaves * TPS * Gm::RS;     // [kParts][128]
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < HPG; ++h) {
      st.wml[(wave * HPG + h) * 2] = m[h];
      st.wml[(wave * HPG + h) * 2 + 1] = lw[h];
    }
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < HPG; ++h) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, st.wml[(w * HPG + h) * 2]);
    const float fw = (m[h] == -INFINITY) ? 0.0f : exp2f(m[h] - M);
    float *row = s_red + (wave * TPS + tl) * Gm::RS + j * CPL;
#pragma unroll
    for (int i = 0; i < CPL; i += 4) {
      const int k0 = (NVG > 1) ? (i / (CPL / NVG)) : 0;
      float4 v;
      v.x = fmaf(acc[h][i], INV_U, bias[h][k0]) * fw;
      v.y = fmaf(acc[h][i + 1], INV_U, bias[h][k0]) * fw;
      v.z = fmaf(acc[h][i + 2], INV_U, bias[h][k0]) * fw;
      v.w = fmaf(acc[h][i + 3], INV_U, bias[h][k0]) * fw;
      *reinterpret_cast<float4 *>(row + i) = v;
    }
    __syncthreads();
    {
      const int c = tid & (kHeadDim - 1), half = tid >> 7;
      float sum = 0.0f;
      for (int r = half; r < kWaves * TPS; r += kParts) sum += s_red[r * Gm::RS + c];
      s_half[half * kHeadDim + c] = sum;
    }
    __syncthreads();
    if (tid < kHeadDim) {
      float t = 0.0f;
#pragma unroll
      for (int p = 0; p < kParts; ++p) t += s_half[p * kHeadDim + tid];
      st.acc[h * kHeadDim + tid] = t;
      if (tid == 0) {
        float L = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          const float mw = st.wml[(w * HPG + h) * 2];
          if (mw != -INFINITY) L = fmaf(exp2f(mw - M), st.wml[(w * HPG + h) * 2 + 1], L);
        }
        st.ml[2 * h] = M;
        st.ml[2 * h + 1] = L;
      }
    }
    __syncthreads();
  }
  finish_part<HPG>(a, unit, split, st);
}

// Merge of the part records: m = max m_i, l = sum l_i 2^(m_i - m),
// out = sum acc_i 2^(m_i - m) / l.
__global__ __launch_bounds__(kHeadDim) void merge_kernel(const float *__restrict__ partials,
                                                         float *__restrict__ out, int nparts) {
  const int64_t bh = blockIdx.x;
  const int c = threadIdx.x;
  const float *p = partials + bh * nparts * kPartialStride;
  float M = -INFINITY;
  for (int i = 0; i < nparts; ++i) M = fmaxf(M, p[i * kPartialStride + kHeadDim]);
  float L = 0.0f, acc = 0.0f;
  for (int i = 0; i < nparts; ++i) {
    const float mi = p[i * kPartialStride + kHeadDim];
    if (mi == -INFINITY) continue;
    const float f = exp2f(mi - M);
    L = fmaf(f, p[i * kPartialStride + kHeadDim + 1], L);
    acc = fmaf(f, p[i * kPartialStride + c], acc);
  }
  out[bh * kHeadDim + c] = acc / L;
}

template <int BITS, int GS, int HPG>
hipError_t launch_kernel(const AttnArgs &a, hipStream_t s) {
  constexpr int LPT = (HPG == 1) ? 4 : (HPG == 2 ? 4 : 8);
  const int units = a.batch * a.hkv;
  hipLaunchKernelGGL((decode_attn_kernel<BITS, GS, HPG, LPT>), dim3(units * a.nparts), dim3(kThreads), 0,
                     s, a);
  return hipGetLastError();
}

template <int BITS, int GS>
hipError_t launch_by_heads(const AttnArgs &a, hipStream_t s) {
  switch (a.hq / a.hkv) {
    case 1: return launch_kernel<BITS, GS, 1>(a, s);
    case 2: return launch_kernel<BITS, GS, 2>(a, s);
    case 4: return launch_kernel<BITS, GS, 4>(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <int BITS>
hipError_t launch_by_group(const AttnArgs &a, hipStream_t s) {
  switch (a.c.group) {
    case 32: return launch_by_heads<BITS, 32>(a, s);
    case 64: return launch_by_heads<BITS, 64>(a, s);
    case 128: return launch_by_heads<BITS, 128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode_attention(const AttnArgs &a, hipStream_t s) {
  hipError_t e = (a.c.bits == 2) ? launch_by_group<2>(a, s) : launch_by_group<4>(a, s);
  if (e != hipSuccess || a.nparts == 1) return e;
  hipLaunchKernelGGL(merge_kernel, dim3(a.batch * a.hq), dim3(kHeadDim), 0, s, a.partials, a.out, a.nparts);
  return hipGetLastError();
}

}  // namespace kvq
