// InnerQ-style cache for gfx950: quantizer, append and decode attention.
//
// Layout (euno.news, "【论文】InnerQ：硬件感知免调优KV缓存量化用于大语言模型",
// methodology 1, 2 and 4): keys and values are both grouped per token along
// the hidden dimension, G channels per group, each group with one shared
// scale; a group whose values are centred on zero is quantized symmetrically,
// any other asymmetrically; the first `sinks` tokens and the most recent
// `residual` tokens (a FIFO window) stay fp16.
//
// Symmetric groups store the signed level k in [-(2^(b-1)-1), 2^(b-1)-1] as
// the code k + 2^(b-1) with zero-point Z = -2^(b-1), so S * (code + Z) is the
// dequantized value in both modes and the attention kernel needs no mode bit.
//
// Attention.  Grouping along the reduction dimension means a lane's channel
// slice (32 or 16 channels) lies inside one key group, so a token's score is
//     s_t = sum_g S_tg (sum_{c in g} q_c k_tc + Z_tg sum_{c in g} q_c)
// and each lane multiplies its partial dot product by its group's scale once
// (methodology 3: the scale is loaded once per group and reused for the
// group's products).  Values follow the same per-(token, group) rule as the
// KIVI value path.  The lane layout, load pipeline, online softmax and wave
// combination are those of the KIVI kernel (kvq_attn.hip).
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include "kvq_internal.h"
#include "kvq_attn_common.h"
#include "kvq_quant_common.h"

namespace kvq {
namespace {

// ---------------------------------------------------------------- quantizer
// Quantizes the G fp16 values at x (one group of one token row).  Mode:
// symmetric when 101 * s1^2 < G * s2 with s1 = sum x and s2 = sum x^2 taken in
// float64 in channel order (|mean| < std / 10, population std).  Symmetric:
// S = max|x| / (2^(b-1) - 1) (1 for an all-zero group), Z = -2^(b-1), codes
// clamp(rint(x / S) - Z, 1, 2^b - 1).  Asymmetric: the KIVI group map.
// A key divided by its channel scale and rounded to fp16 (round to nearest
// even), returned as a float.  The scale is a power of two 2^e, so the
// quotient is the exact product with 2^-e, whose bits are those of the scale
// subtracted from 0x7F000000 (biased exponent 254 - (e + 127)).
__device__ __forceinline__ float normalized_key(float x, float lam) {
  return __half2float(__float2half_rn(x * __uint_as_float(0x7F000000u - __float_as_uint(lam))));
}

// lam: the G channels' key scales, or null (no normalization).
template <int BITS>
__device__ __forceinline__ void quantize_group_hybrid(const uint16_t *x, int G, uint32_t *codes, float *scale,
                                                      int16_t *zero, const float *lam) {
  constexpr int PER = 32 / BITS;
  constexpr float QMAX = float((1 << BITS) - 1);
  constexpr float QM = float((1 << (BITS - 1)) - 1);
  constexpr float HALF = float(1 << (BITS - 1));
  float mn = INFINITY, mx = -INFINITY, amax = 0.0f;
  double s1 = 0.0, s2 = 0.0;
  for (int k0 = 0; k0 < G; k0 += 32) {
    float v[32];
#pragma unroll
    for (int q = 0; q < 4; ++q) load8(x + k0 + 8 * q, v + 8 * q);
    if (lam != nullptr) {
#pragma unroll
      for (int k = 0; k < 32; ++k) v[k] = normalized_key(v[k], lam[k0 + k]);
    }
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      mn = fminf(mn, v[k]);
      mx = fmaxf(mx, v[k]);
      amax = fmaxf(amax, fabsf(v[k]));
      const double xd = (double)v[k];
      s1 += xd;
      s2 += xd * xd;   // exact product of an fp16 value, so contraction is harmless
    }
  }
  const bool sym = 101.0 * (s1 * s1) < (double)G * s2;
  GroupParams p;
  float lo;
  if (sym) {
    const float s = amax > 0.0f ? amax / QM : 1.0f;
    p = {s, -HALF, 1.0f / s};
    lo = 1.0f;
  } else {
    p = group_params(mn, mx, QMAX);
    lo = 0.0f;
  }
  *scale = p.s;
  *zero = static_cast<int16_t>(p.z);
  for (int k0 = 0; k0 < G; k0 += 32) {
    float v[32];
#pragma unroll
    for (int q = 0; q < 4; ++q) load8(x + k0 + 8 * q, v + 8 * q);
    if (lam != nullptr) {
#pragma unroll
      for (int k = 0; k < 32; ++k) v[k] = normalized_key(v[k], lam[k0 + k]);
    }
    uint32_t cd[32];
    codes_of<32>(v, p, lo, QMAX, cd);
    uint32_t words[32 / PER];
#pragma unroll
    for (int w = 0; w < 32 / PER; ++w) {
      uint32_t word = 0;
#pragma unroll
      for (int k = 0; k < PER; ++k) word |= cd[w * PER + k] << (k * BITS);
      words[w] = word;
    }
    if constexpr (BITS == 2) {
      *reinterpret_cast<uint2 *>(codes + k0 / PER) = make_uint2(words[0], words[1]);
    } else {
      *reinterpret_cast<uint4 *>(codes + k0 / PER) = make_uint4(words[0], words[1], words[2], words[3]);
    }
  }
}

// Destination of group j of token row `row` (absolute, unit * cap + t).
template <int BITS>
__device__ __forceinline__ void quantize_into(const CacheView &c, bool values, const uint16_t *x, int64_t row,
                                              int j) {
  constexpr int PER = 32 / BITS;
  constexpr int W = kHeadDim / PER;
  const int G = c.group, NG = kHeadDim / G;
  uint32_t *codes = (values ? c.v_codes : c.k_codes) + row * W + j * (G / PER);
  float *scale = (values ? c.v_scale : c.k_scale) + row * NG + j;
  int16_t *zero = (values ? c.v_zero : c.k_zero) + row * NG + j;
  const float *lam = (!values && c.k_norm != nullptr) ? c.k_norm + (row / c.cap) * kHeadDim + j * G : nullptr;
  quantize_group_hybrid<BITS>(x, G, codes, scale, zero, lam);
}

// One wave quantizes a block of 32 consecutive rows of the flattened
// (unit, row) range of one tensor: key blocks in the first half of the grid,
// value blocks in the second.  Source row src_row0 + i of [unit][src_rows]
// [128] goes to cache row dst_row0 + i.  Lane l loads channels 8 (l % 16) ..
// + 7 of rows 4 i + l / 16 with 16-byte loads (1 KB of consecutive rows per
// instruction) and stages them in a per-wave LDS tile.  The group statistics
// (the index-order float64 sums of the mode test, minimum, maximum) then run
// one lane per (row, group), reading the group from the tile; the lane
// writes the group's scale and zero-point and leaves r = RN(1/S), Z, the tie
// threshold and the lower code bound in LDS.  Finally every lane codes its
// own 8 values per row from registers with the tile coder (the same codes as
// quantize_group_hybrid) and stores packed words.
template <int BITS, int G>
__global__ __launch_bounds__(256) void innerq_quantize_kernel(CacheView c, const uint16_t *__restrict__ ksrc,
                                                              const uint16_t *__restrict__ vsrc, int64_t src_rows,
                                                              int64_t src_row0, int count, int64_t dst_row0,
                                                              int units, int nblocks) {
  constexpr int NR = 8, BR = 4 * NR;          // rows per lane, rows per block
  constexpr int LPG = G / 8, NG = kHeadDim / G;
  constexpr int PER = 32 / BITS, W = kHeadDim / PER;
  constexpr float QMAX = float((1 << BITS) - 1);
  constexpr float QM = float((1 << (BITS - 1)) - 1);
  constexpr float HALF = float(1 << (BITS - 1));
  constexpr int TS = kHeadDim + 8;            // tile row stride (halves): rows 4 banks apart
  static_assert(BR * NG * 20 <= BR * TS * 2, "parameters reuse the tile");
  __shared__ __attribute__((aligned(16))) uint16_t s_tile[4][BR * TS];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int cs = lane & 15, q = lane >> 4, j = cs / LPG;
  const int wb = (int)blockIdx.x * 4 + wave;
  if (wb >= 2 * nblocks) return;
  const bool values = wb >= nblocks;
  const int row0 = (values ? wb - nblocks : wb) * BR;
  const int total_rows = units * count;
  const uint16_t *src = values ? vsrc : ksrc;
  uint32_t *codes = values ? c.v_codes : c.k_codes;
  float *scale = values ? c.v_scale : c.k_scale;
  int16_t *zero = values ? c.v_zero : c.k_zero;

  // (unit, row) of block row r, stepped from the block's first row (one
  // wave-uniform division per block)
  const int ub = row0 / count, tb = row0 - ub * count;
  auto locate = [&](int r, int &u, int &t) {
    u = ub;
    t = tb + r;
    while (t >= count) {
      t -= count;
      ++u;
    }
  };
  auto valid = [&](int r) { return row0 + r < total_rows; };

  uint4 raw[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    raw[i] = make_uint4(0u, 0u, 0u, 0u);
    const int r = 4 * i + q;
    if (valid(r)) {
      int u, t;
      locate(r, u, t);
      raw[i] = *(reinterpret_cast<const uint4 *>(src + ((int64_t)u * src_rows + src_row0 + t) * kHeadDim) + cs);
      if (!values && c.k_norm != nullptr) {
        // keys of normalized caches: times 1 / scale of their channels (a
        // power of two, exact in fp16 down to 2^-16; its bits as in
        // normalized_key), one fp16 rounding
        const float4 l0 = reinterpret_cast<const float4 *>(c.k_norm + (int64_t)u * kHeadDim + 8 * cs)[0];
        const float4 l1 = reinterpret_cast<const float4 *>(c.k_norm + (int64_t)u * kHeadDim + 8 * cs)[1];
        auto inv = [](float l) { return (_Float16)__uint_as_float(0x7F000000u - __float_as_uint(l)); };
        const f16x2 f0 = {inv(l0.x), inv(l0.y)};
        const f16x2 f1 = {inv(l0.z), inv(l0.w)};
        const f16x2 f2 = {inv(l1.x), inv(l1.y)};
        const f16x2 f3 = {inv(l1.z), inv(l1.w)};
        raw[i] = make_uint4(as_u32(as_h2(raw[i].x) * f0), as_u32(as_h2(raw[i].y) * f1), as_u32(as_h2(raw[i].z) * f2),
                            as_u32(as_h2(raw[i].w) * f3));
      }
    }
  }
  uint16_t *tile = s_tile[wave];
#pragma unroll
  for (int i = 0; i < NR; ++i) *reinterpret_cast<uint4 *>(tile + (4 * i + q) * TS + 8 * cs) = raw[i];
  lds_wave_sync();

  // group statistics and parameters, one lane per (row, group)
  float4 par[(BR * NG + 63) / 64];
  float sc[(BR * NG + 63) / 64];
#pragma unroll
  for (int k = 0; k < (BR * NG + 63) / 64; ++k) {
    const int gg = lane + 64 * k;
    const int r = gg / NG, jj = gg % NG;
    double s1 = 0.0, s2 = 0.0;
    f16x2 mn2 = as_h2(0x7C007C00u), mx2 = as_h2(0xFC00FC00u);   // +inf, -inf
    if (gg < BR * NG) {
      const uint16_t *x = tile + r * TS + jj * G;
      for (int k0 = 0; k0 < G; k0 += 8) {
        const uint4 w = *reinterpret_cast<const uint4 *>(x + k0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const f16x2 h = as_h2(word_of(w, e));
          mn2 = hmin(mn2, h);
          mx2 = hmax(mx2, h);
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const double xd = (double)(float)h[hh];
            s1 = s1 + xd;
            s2 = __builtin_fma(xd, xd, s2);   // x^2 is exact, so this is s2 + x * x rounded once
          }
        }
      }
    }
    const float mn = fminf((float)mn2[0], (float)mn2[1]), mx = fmaxf((float)mx2[0], (float)mx2[1]);
    const float amax = fmaxf(fabsf(mn), fabsf(mx));
    const bool sym = 101.0 * (s1 * s1) < (double)G * s2;
    GroupParams p;
    float lo;
    if (sym) {
      const float sv = amax > 0.0f ? amax / QM : 1.0f;
      p = {sv, -HALF, 1.0f / sv};
      lo = 1.0f;
    } else {
      p = group_params(mn, mx, QMAX);
      lo = 0.0f;
    }
    par[k] = make_float4(p.r, p.z, tie_threshold(amax, p.r), lo);
    sc[k] = p.s;
    if (gg < BR * NG && valid(r)) {
      int u, t;
      locate(r, u, t);
      const int64_t row = (int64_t)u * c.cap + dst_row0 + t;
      scale[row * NG + jj] = p.s;
      zero[row * NG + jj] = static_cast<int16_t>(p.z);
    }
  }
  // the parameter tables reuse the start of the tile: [row][group] float4,
  // then [row][group] S
  lds_wave_sync();
  float4 *s_par = reinterpret_cast<float4 *>(tile);
  float *s_s = reinterpret_cast<float *>(tile) + 4 * BR * NG;
#pragma unroll
  for (int k = 0; k < (BR * NG + 63) / 64; ++k) {
    const int gg = lane + 64 * k;
    if (gg < BR * NG) {
      s_par[gg] = par[k];
      s_s[gg] = sc[k];
    }
  }
  lds_wave_sync();

  auto code_row = [&](int i) {
    const int r = 4 * i + q;
    const float4 pv = s_par[r * NG + j];
    float rr[8], z[8], thr[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      rr[k] = pv.x;
      z[k] = pv.y;
      thr[k] = pv.z;
    }
    bool near = false;
    uint32_t u = code8_fast<BITS>(raw[i], rr, z, thr, pv.w, near);
    if (__any(near)) {
      float sv[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) sv[k] = s_s[r * NG + j];
      u = code8_exact<BITS>(raw[i], sv, z, pv.w);
    }
    return u;
  };
  auto store = [&](int i, uint32_t word, int w) {
    const int r = 4 * i + q;
    if (valid(r)) {
      int u, t;
      locate(r, u, t);
      codes[((int64_t)u * c.cap + dst_row0 + t) * W + w] = word;
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

// Key channel scales.  norm is first filled with 1; then each workgroup
// takes kNormRows rows of one unit's prompt keys: thread t owns channels
// 8 (t % 16) .. + 7 of rows t / 16 + 16 i and keeps their largest magnitude
// as an fp16 bit pattern (the order of non-negative fp16 patterns is that of
// their values), the 16 row-threads of a channel combine through LDS, and
// the channel's scale, the smallest power of two >= max(1, max-abs), goes to
// norm with an atomic maximum on its bit pattern (an order-preserving map for
// positive floats), so the chunks of a unit combine in any order.
constexpr int kNormRows = 1024;

__global__ __launch_bounds__(256) void fill_ones_kernel(float *p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 1.0f;
}

__global__ __launch_bounds__(256) void key_norm_kernel(float *__restrict__ norm, const uint16_t *__restrict__ k,
                                                       int64_t len) {
  __shared__ uint32_t s_max[16][kHeadDim];
  const int u = blockIdx.y, ch = blockIdx.x;
  const int t = threadIdx.x, cs = t & 15, r0 = t >> 4;
  const int64_t rb = (int64_t)ch * kNormRows;
  const int64_t re = len < rb + kNormRows ? len : rb + kNormRows;
  const uint16_t *base = k + (int64_t)u * len * kHeadDim + 8 * cs;
  uint32_t m[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
  for (int64_t r = rb + r0; r < re; r += 16) {
    const uint4 w = *reinterpret_cast<const uint4 *>(base + r * kHeadDim);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t lo = ws[e] & 0x7fffu, hi = (ws[e] >> 16) & 0x7fffu;
      m[2 * e] = m[2 * e] > lo ? m[2 * e] : lo;
      m[2 * e + 1] = m[2 * e + 1] > hi ? m[2 * e + 1] : hi;
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) s_max[r0][8 * cs + e] = m[e];
  __syncthreads();
  if (t < kHeadDim) {
    uint32_t mb = 0;
#pragma unroll
    for (int r = 0; r < 16; ++r) mb = mb > s_max[r][t] ? mb : s_max[r][t];
    const float amax = h2f((uint16_t)mb);
    float lam = 1.0f;
    if (amax > 1.0f) {
      const uint32_t bits = __float_as_uint(amax);
      lam = (bits & 0x7fffffu) == 0 ? amax : __uint_as_float((bits & 0x7f800000u) + 0x00800000u);
    }
    atomicMax(reinterpret_cast<unsigned int *>(norm) + (int64_t)u * kHeadDim + t, __float_as_uint(lam));
  }
}

// One workgroup (one wave) per unit.  When pop_row >= 0 the window is full:
// the oldest window token (ring slot pop_row mod R) is quantized into cache
// row pop_row first.  Then the new key and value rows, unless k_new is null
// (a fused step's attention launch stores them), are written into row
// `slot` of the sink rows (to_sink) or of the ring.
template <int BITS>
__global__ __launch_bounds__(64) void innerq_append_kernel(CacheView c, const uint16_t *__restrict__ k_new,
                                                           const uint16_t *__restrict__ v_new, int64_t pop_row,
                                                           int to_sink, int slot) {
  const int unit = blockIdx.x, tid = threadIdx.x;
  const int R = c.residual, NG = kHeadDim / c.group;
  if (pop_row >= 0) {
    if (tid < 2 * NG) {
      const bool values = tid >= NG;
      const int j = tid % NG;
      const uint16_t *ring = values ? c.v_resid : c.k_resid;
      const uint16_t *x = ring + ((int64_t)unit * R + pop_row % R) * kHeadDim + j * c.group;
      quantize_into<BITS>(c, values, x, (int64_t)unit * c.cap + pop_row, j);
    }
    __syncthreads();   // the popped slot is read before the new token overwrites it
  }
  constexpr int CH = kHeadDim * 2 / 16;   // 16-byte chunks per row
  if (k_new != nullptr && tid < 2 * CH) {
    const bool values = tid >= CH;
    const int ch = tid % CH;
    const uint4 *src = reinterpret_cast<const uint4 *>((values ? v_new : k_new) + (int64_t)unit * kHeadDim);
    uint16_t *base = to_sink ? (values ? c.v_sink : c.k_sink) + ((int64_t)unit * c.sinks + slot) * kHeadDim
                             : (values ? c.v_resid : c.k_resid) + ((int64_t)unit * R + slot) * kHeadDim;
    reinterpret_cast<uint4 *>(base)[ch] = src[ch];
  }
}

// ---------------------------------------------------------------- attention
template <int WPL>
struct IqBuf {
  uint32_t kw[WPL];
  uint32_t vw[WPL];
  float ks, vs;       // this lane's key / value group scales
  uint32_t kz, vz;    // their int16 zero-points (low half)
};

// One workgroup of 8 waves per (split, unit).  The quantized tokens
// [t0, nq) (t0 = number of sink tokens present) are covered by steps of TPS
// tokens that start on multiples of TPS, so every step's metadata read is a
// whole aligned run of cache lines; each split takes a contiguous range of
// steps and each wave a contiguous sub-range.  Lanes of a token outside
// [t0, nq) score -inf.  The last split also takes the fp16 tokens: the sinks
// and the window [nq, n).
template <int BITS, int GS, int HPG, int LPT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWavesPerEU<HPG>, 8)))
void innerq_attn_kernel(AttnArgs a) {
  constexpr int CPL = kHeadDim / LPT, TPS = kWave / LPT, PER = 32 / BITS, WPL = CPL / PER;
  constexpr int W = kHeadDim / PER;
  constexpr int NG = kHeadDim / GS;
  constexpr float U = Unpack<BITS>::scale;
  constexpr float INV_U = 1.0f / U;
  static_assert(CPL <= GS, "a lane's channel slice must lie inside one group");
  static_assert(WPL >= 1, "lane slice must hold whole words");
  using Buf = IqBuf<WPL>;

  __shared__ __attribute__((aligned(16))) float smem[kRedFloats<HPG> + kStageFloats<HPG>];
  __shared__ uint32_t s_done[kWaves + 1];   // no work queue here (zeros); then the last-part flag
  const Stage st = stage_of<HPG>(smem, kRedFloats<HPG>);

  const int units = a.batch * a.hkv;
  const int split = blockIdx.x / units;
  const int unit = blockIdx.x % units;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane % LPT, tl = lane / LPT;
  const int b = unit / a.hkv, hk = unit % a.hkv;
  const int64_t cap = a.c.cap;
  const int S = a.c.sinks;
  const int64_t nsink = a.n < S ? a.n : S;   // sink tokens present
  const int64_t t0 = nsink;                  // first quantized token
  const int64_t nq = a.nq_k;                 // end of the quantized tokens
  const int64_t tb0 = t0 - t0 % TPS;         // first step start, aligned
  const int tsteps = nq > t0 ? (int)((nq - tb0 + TPS - 1) / TPS) : 0;
  const int t0i = (int)t0, tb0i = (int)tb0, nqi = (int)nq;
  const int s0 = (int)((int64_t)tsteps * split / a.splits);
  const int s1 = (int)((int64_t)tsteps * (split + 1) / a.splits);
  // a wave's steps: a contiguous eighth of the split, or (a.interleave,
  // chosen on the host for long splits) every eighth step, so the
  // workgroup's waves read neighbouring steps at any one time
  const int ws0 = a.interleave ? s0 + wave : s0 + (s1 - s0) * wave / kWaves;
  const int wstride = a.interleave ? kWaves : 1;
  const int nsteps = a.interleave ? (s1 - s0 - wave + kWaves - 1) / kWaves
                                  : s0 + (s1 - s0) * (wave + 1) / kWaves - ws0;

  // query slice of this lane, in log2 units and divided by the unpack scale,
  // and its plain sum (the zero-point term of the lane's group)
  // With key scales (normalized keys) the query carries them: q_c * lambda_c
  // (powers of two, so exact), for the quantized keys only.
  float qf[HPG][CPL], qsum[HPG];
  float lam[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) lam[i] = 1.0f;
  if (a.c.k_norm != nullptr) {
#pragma unroll
    for (int i = 0; i < CPL; i += 4) {
      const float4 l4 = *reinterpret_cast<const float4 *>(a.c.k_norm + (int64_t)unit * kHeadDim + j * CPL + i);
      lam[i] = l4.x;
      lam[i + 1] = l4.y;
      lam[i + 2] = l4.z;
      lam[i + 3] = l4.w;
    }
  }
#pragma unroll
  for (int h = 0; h < HPG; ++h) {
    const uint16_t *qp = a.q + ((int64_t)(b * a.hq + hk * HPG + h)) * kHeadDim + j * CPL;
    qsum[h] = 0.0f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const float qv = h2f(qp[i]) * a.qscale * lam[i];
      qsum[h] += qv;
      qf[h][i] = qv * INV_U;
    }
  }
  Online<HPG, CPL, 1> o;
  o.init();

  // per-unit buffer resources; the step's token offset goes into the vector
  // offset so the hardware range check turns reads past the capacity into
  // zeros (those lanes are masked)
  const Rsrc rkc = rsrc_of(a.c.k_codes + (int64_t)unit * cap * W, (uint32_t)(cap * W * 4));
  const Rsrc rvc = rsrc_of(a.c.v_codes + (int64_t)unit * cap * W, (uint32_t)(cap * W * 4));
  const Rsrc rks = rsrc_of(a.c.k_scale + (int64_t)unit * cap * NG, (uint32_t)(cap * NG * 4));
  const Rsrc rkz = rsrc_of(a.c.k_zero + (int64_t)unit * cap * NG, (uint32_t)(cap * NG * 2));
  const Rsrc rvs = rsrc_of(a.c.v_scale + (int64_t)unit * cap * NG, (uint32_t)(cap * NG * 4));
  const Rsrc rvz = rsrc_of(a.c.v_zero + (int64_t)unit * cap * NG, (uint32_t)(cap * NG * 2));
  const uint32_t code_lane = (uint32_t)(tl * W + j * WPL) * 4u;
  const uint32_t meta_lane = (uint32_t)(tl * NG + (j * CPL) / GS);

  auto load = [&](Buf &bf, int s) {
    s = s < nsteps ? s : nsteps - 1;   // past the end: reload the last step (never processed)
    const uint32_t tb = (uint32_t)(tb0 + (int64_t)(ws0 + wstride * s) * TPS);   // first token of the step
    const uint32_t vc = code_lane + tb * (W * 4);
    const uint32_t vm = meta_lane + tb * NG;
    bload_words<WPL>(rkc, vc, 0, bf.kw);
    bload_words<WPL>(rvc, vc, 0, bf.vw);
    bf.ks = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rks, vm * 4, 0, kStream));
    bf.vs = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rvs, vm * 4, 0, kStream));
    // a step's zero-points fill half a cache line; the next step reads the
    // other half, so these loads keep the default caching
    bf.kz = __builtin_amdgcn_raw_buffer_load_b16(rkz, vm * 2, 0, 0);
    bf.vz = __builtin_amdgcn_raw_buffer_load_b16(rvz, vm * 2, 0, 0);
  };

  auto process = [&](const Buf &bf, int s) {
    const int tok = tb0i + (ws0 + wstride * s) * TPS + tl;   // token indices fit 32 bits (capacity <= 2^25)
    const bool valid = tok >= t0i && tok < nqi;  // rows outside may hold any bits
    const float kz = (float)(int16_t)(bf.kz & 0xffffu);
    const float vz = (float)(int16_t)(bf.vz & 0xffffu);
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
    for (int h = 0; h < HPG; ++h) {
      const float sv = block_sum<LPT>(bf.ks * fmaf(kz, qsum[h], sc[h] + d1[h]));
      p[h] = o.weight(h, valid ? sv : -INFINITY);
    }
    const float vs = valid ? bf.vs : 0.0f;
#pragma unroll
    for (int h = 0; h < HPG; ++h) o.bias[h][0] = fmaf(p[h] * vs, vz, o.bias[h][0]);
#pragma unroll
    for (int w = 0; w < WPL; ++w) {
      float vf[PER];
      Unpack<BITS>::run(bf.vw[w], vf);
#pragma unroll
      for (int h = 0; h < HPG; ++h) {
        const float wt = p[h] * vs;
#pragma unroll
        for (int i = 0; i < PER; ++i) o.acc[h][w * PER + i] = fmaf(wt, vf[i], o.acc[h][w * PER + i]);
      }
    }
  };

  if (nsteps > 0) {
    Buf A, B, C;
    // the two prologue batches must be issued in order: the compiler's wait
    // counts are merged over the loop entry, and interleaved prologue loads
    // would make every step wait for the step after it as well
    load(A, 0);
    asm volatile("" ::: "memory");
    load(B, 1);
    asm volatile("" ::: "memory");
    for (int s = 0; s < nsteps; s += 3) {
      progress_priority(nsteps - s, nsteps);
      load(C, s + 2);
      process(A, s);
      load(A, s + 3);
      if (s + 1 < nsteps) process(B, s + 1);
      load(B, s + 4);
      if (s + 2 < nsteps) process(C, s + 2);
    }
  }

  if (lane == 0) s_done[wave] = 0;

  // fp16 tokens: sinks [0, nsink) from the sink rows, then the window
  // [nq, n) from ring slots t mod R
  if (split == a.splits - 1) {
    const int R = a.c.residual;
    const int nf = (int)(nsink + (a.n - nq));
#pragma unroll
    for (int h = 0; h < HPG; ++h) {
      // plain query: the fp16 keys keep their original units
      const uint16_t *qp = a.q + ((int64_t)(b * a.hq + hk * HPG + h)) * kHeadDim + j * CPL;
#pragma unroll
      for (int i = 0; i < CPL; ++i) qf[h][i] = h2f(qp[i]) * a.qscale;
    }
    for (int rs = wave; rs * TPS < nf; rs += kWaves) {
      const int i = rs * TPS + tl;
      const bool valid = i < nf;
      const int ii = valid ? i : 0;
      const uint16_t *krow, *vrow;
      if (ii < nsink) {
        const int64_t off = ((int64_t)unit * S + ii) * kHeadDim + j * CPL;
        krow = a.c.k_sink + off;
        vrow = a.c.v_sink + off;
      } else if (a.k_new != nullptr && nq + (ii - nsink) == a.n - 1) {
        // fused step: the new token, not in the ring yet
        const int64_t off = (int64_t)unit * kHeadDim + j * CPL;
        krow = a.k_new + off;
        vrow = a.v_new + off;
      } else {
        const int64_t off = ((int64_t)unit * R + (nq + (ii - nsink)) % R) * kHeadDim + j * CPL;
        krow = a.c.k_resid + off;
        vrow = a.c.v_resid + off;
      }
      fp16_token<HPG, CPL, 1, LPT>(o, qf, krow, vrow, valid, U);
    }
    if (a.k_new != nullptr && tid < 2 * (kHeadDim * 2 / 16)) {
      // fused step: the new token goes into its window slot, the slot of the
      // token that left the window (read quantized by this launch)
      constexpr int CH = kHeadDim * 2 / 16;
      const int which = tid / CH, ch = tid % CH;
      const uint4 *src = reinterpret_cast<const uint4 *>((which ? a.v_new : a.k_new) + (int64_t)unit * kHeadDim);
      uint4 *dst = reinterpret_cast<uint4 *>((which ? a.c.v_resid : a.c.k_resid) +
                                             ((int64_t)unit * R + (a.n - 1) % R) * kHeadDim);
      dst[ch] = src[ch];
    }
  }
  if (a.prequant >= 0 && split == 0 && wave == 0 && lane < 2 * NG) {
    // a full window: its oldest token's key and value rows are quantized
    // now, ahead of the next append's pop (one lane per group)
    const bool values = lane >= NG;
    const int g = lane % NG;
    const uint16_t *ring = values ? a.c.v_resid : a.c.k_resid;
    const uint16_t *x = ring + ((int64_t)unit * a.c.residual + a.prequant % a.c.residual) * kHeadDim + g * GS;
    quantize_into<BITS>(a.c, values, x, (int64_t)unit * cap + a.prequant, g);
  }

  combine_waves<HPG, LPT, 1>(o, smem, st, wave, lane, INV_U);
  // each wave keeps its contiguous step range (the kernel streams HBM near
  // its ceiling, and scattered chunks lost more than balancing gained); the
  // unit's last workgroup merges the split records
  queue_finish<HPG, kWaves>(a, unit, split, st, s_done, 0u);
}

template <int BITS, int GS, int HPG>
hipError_t launch_iq_kernel(const AttnArgs &a, hipStream_t s) {
  constexpr int LPT = (HPG == 4) ? 8 : 4;
  hipLaunchKernelGGL((innerq_attn_kernel<BITS, GS, HPG, LPT>), dim3(a.batch * a.hkv * a.nparts), dim3(kThreads),
                     0, s, a);
  return hipGetLastError();
}

template <int BITS, int GS>
hipError_t launch_iq_by_heads(const AttnArgs &a, hipStream_t s) {
  switch (a.hq / a.hkv) {
    case 1: return launch_iq_kernel<BITS, GS, 1>(a, s);
    case 2: return launch_iq_kernel<BITS, GS, 2>(a, s);
    case 4: return launch_iq_kernel<BITS, GS, 4>(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <int BITS>
hipError_t launch_iq_by_group(const AttnArgs &a, hipStream_t s) {
  switch (a.c.group) {
    case 32: return launch_iq_by_heads<BITS, 32>(a, s);
    case 64: return launch_iq_by_heads<BITS, 64>(a, s);
    case 128: return launch_iq_by_heads<BITS, 128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_innerq_quantize(const CacheView &c, int units, const uint16_t *ksrc, const uint16_t *vsrc,
                                  int64_t src_rows, int64_t src_row0, int count, int64_t dst_row0, hipStream_t s) {
  if (count <= 0 || units <= 0) return hipSuccess;
  const int64_t total = (int64_t)units * count;
  if (total > INT32_MAX / 2) return hipErrorInvalidValue;
  const int nblocks = (int)((total + 31) / 32);   // 32 rows per wave, per tensor
  const dim3 grid((unsigned)((2 * (int64_t)nblocks + 3) / 4));
#define KVQ_IQQ(B, G)                                                                                        \
  hipLaunchKernelGGL((innerq_quantize_kernel<B, G>), grid, dim3(256), 0, s, c, ksrc, vsrc, src_rows, src_row0, \
                     count, dst_row0, units, nblocks)
  if (c.bits == 2) {
    if (c.group == 32) KVQ_IQQ(2, 32);
    else if (c.group == 64) KVQ_IQQ(2, 64);
    else KVQ_IQQ(2, 128);
  } else {
    if (c.group == 32) KVQ_IQQ(4, 32);
    else if (c.group == 64) KVQ_IQQ(4, 64);
    else KVQ_IQQ(4, 128);
  }
#undef KVQ_IQQ
  return hipGetLastError();
}

hipError_t launch_key_norm(float *norm, int units, const uint16_t *k, int64_t len, hipStream_t s) {
  const int n = units * kHeadDim;
  hipLaunchKernelGGL(fill_ones_kernel, dim3((n + 255) / 256), dim3(256), 0, s, norm, n);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || len == 0) return e;
  const int chunks = (int)((len + kNormRows - 1) / kNormRows);
  hipLaunchKernelGGL(key_norm_kernel, dim3(chunks, units), dim3(256), 0, s, norm, k, len);
  return hipGetLastError();
}

hipError_t launch_innerq_append(const CacheView &c, int units, const uint16_t *k_new, const uint16_t *v_new,
                                int64_t pop_row, bool to_sink, int slot, hipStream_t s) {
  if (c.bits == 2)
    hipLaunchKernelGGL(innerq_append_kernel<2>, dim3(units), dim3(64), 0, s, c, k_new, v_new, pop_row,
                       to_sink ? 1 : 0, slot);
  else
    hipLaunchKernelGGL(innerq_append_kernel<4>, dim3(units), dim3(64), 0, s, c, k_new, v_new, pop_row,
                       to_sink ? 1 : 0, slot);
  return hipGetLastError();
}

hipError_t launch_innerq_attention(const AttnArgs &a, hipStream_t s) {
  // the unit's last workgroup merges the split records itself
  return (a.c.bits == 2) ? launch_iq_by_group<2>(a, s) : launch_iq_by_group<4>(a, s);
}

}  // namespace kvq
