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
// Work split.  One workgroup = 4 waves = one unit (batch, kv head) and one
// split of its grouped tokens.  Within a wave, LPT lanes share a token and
// each owns 128 / LPT channels: one 16-byte (or smaller) slice of the key row
// and of the value row, so a wave step reads whole contiguous rows.  Every
// wave keeps its own online-softmax state with a wave-uniform running maximum
// that is only raised when a score exceeds it by more than a margin, so the
// rescale branch is rare and uniform.  Partial (max, sum, acc) records of all
// splits, plus one record for the tokens not covered by whole key and value
// groups (fp16 residual, FIFO queue), are merged by a second kernel.
// All softmax arithmetic is in log2 units (scores pre-multiplied by log2 e).
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kWave = 64;
constexpr int kWaves = 4;
constexpr float kMargin = 8.0f;    // log2 units: weights stay below 2^8 between rescales

typedef float f2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float h2f(uint16_t h) { return __half2float(__ushort_as_half(h)); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Unpacking of one 32-bit code word into floats equal to code * scale.
// 2-bit: a nibble 0b00cc read as an fp4 e2m1 number is exactly cc / 2, so
// masking the word into nibbles and converting two nibbles per instruction
// unpacks 16 codes in 3 integer + 8 conversion instructions.
// 4-bit: a byte 0b0000cccc read as an fp8 e4m3 number is exactly cccc * 2^-9
// (subnormals 0..7, then the first binade), two bytes per instruction.
template <int BITS>
struct Unpack;

template <>
struct Unpack<2> {
  static constexpr float scale = 0.5f;
  __device__ static __forceinline__ void run(uint32_t w, float *out) {
#ifdef KVQ_PLAIN_UNPACK
#pragma unroll
    for (int i = 0; i < 16; ++i) out[i] = 0.5f * (float)((w >> (2 * i)) & 3u);
#else
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
#endif
  }
};

template <>
struct Unpack<4> {
  static constexpr float scale = 1.0f / 512.0f;
  __device__ static __forceinline__ void run(uint32_t w, float *out) {
#ifdef KVQ_PLAIN_UNPACK
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = (1.0f / 512.0f) * (float)((w >> (4 * i)) & 15u);
#else
    const uint32_t m0 = w & 0x0F0F0F0Fu;          // byte k: code 2k
    const uint32_t m1 = (w >> 4) & 0x0F0F0F0Fu;   // byte k: code 2k + 1
    f2 a = __builtin_amdgcn_cvt_pk_f32_fp8(m0, false);
    f2 b = __builtin_amdgcn_cvt_pk_f32_fp8(m0, true);
    f2 c = __builtin_amdgcn_cvt_pk_f32_fp8(m1, false);
    f2 d = __builtin_amdgcn_cvt_pk_f32_fp8(m1, true);
    out[0] = a.x; out[2] = a.y; out[4] = b.x; out[6] = b.y;
    out[1] = c.x; out[3] = c.y; out[5] = d.x; out[7] = d.y;
#endif
  }
};

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

// Shared-memory footprint of the split kernel (floats).
template <int BITS, int HPG, int LPT>
struct SplitSmem {
  static constexpr int TPS = kWave / LPT;
  static constexpr int RS = kHeadDim + 4;                         // padded row
  static constexpr int RED = kWaves * TPS * RS + 2 * kHeadDim;    // reduction rows + halves
  static constexpr int QP = kWaves * HPG * kHeadDim;              // per-wave folded queries
  static constexpr int MAIN = (RED > QP ? RED : QP) + 4 * kWaves * HPG;
};

// Tail: tokens [n_main, n), where keys and values may each be quantized or
// fp16 per token.  One workgroup per unit, plain dequantize-then-dot.
template <int BITS, int HPG>
__device__ void decode_tail(const AttnArgs &a, int unit, float *smem, int smem_floats) {
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
  float *s_sc = smem;                       // [HPG][nt] scores, then weights
  float *s_half = smem + HPG * nt;          // [2][HPG][128]
  float *s_ml = s_half + 2 * HPG * kHeadDim;  // [HPG][2]
  (void)smem_floats;

  float qa[HPG], qb[HPG];
#pragma unroll
  for (int h = 0; h < HPG; ++h) {
    const uint16_t *qp = a.q + ((int64_t)(b * a.hq + hk * HPG + h)) * kHeadDim + 2 * lane;
    qa[h] = h2f(qp[0]);
    qb[h] = h2f(qp[1]);
  }
  // scores: one wave per token, two channels per lane
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
      const float d = wave_sum(qa[h] * k0 + qb[h] * k1);
      if (lane == 0) s_sc[h * nt + i] = d * a.qscale;
    }
  }
  __syncthreads();
  // softmax statistics: wave h handles head h (HPG <= kWaves)
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
      s_ml[2 * h] = mx;
      s_ml[2 * h + 1] = l;
    }
  }
  __syncthreads();
  // P.V: thread owns one channel and half of the tokens
  const int c = tid & (kHeadDim - 1);
  const int part = tid >> 7;
  float acc[HPG];
#pragma unroll
  for (int h = 0; h < HPG; ++h) acc[h] = 0.0f;
  for (int i = part; i < nt; i += 2) {
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
  for (int h = 0; h < HPG; ++h) s_half[(part * HPG + h) * kHeadDim + c] = acc[h];
  __syncthreads();
  if (tid < kHeadDim) {
    const int nparts = a.splits + 1;
#pragma unroll
    for (int h = 0; h < HPG; ++h) {
      const int64_t bh = (int64_t)b * a.hq + hk * HPG + h;
      float *rec = a.partials + (bh * nparts + a.splits) * kPartialStride;
      rec[tid] = s_half[h * kHeadDim + tid] + s_half[(HPG + h) * kHeadDim + tid];
      if (tid == 0) {
        rec[kHeadDim] = nt > 0 ? s_ml[2 * h] : -INFINITY;
        rec[kHeadDim + 1] = nt > 0 ? s_ml[2 * h + 1] : 0.0f;
      }
    }
  }
}

template <int BITS, int GS, int HPG, int LPT>
__global__ __launch_bounds__(kWave *kWaves) void decode_split_kernel(AttnArgs a) {
  constexpr int CPL = kHeadDim / LPT;       // channels per lane
  constexpr int TPS = kWave / LPT;          // tokens per wave step
  constexpr int PER = 32 / BITS;            // codes per word
  constexpr int WPL = CPL / PER;            // code words per lane per token
  constexpr int W = kHeadDim / PER;         // words per token row
  constexpr int NVG = CPL >= GS ? CPL / GS : 1;   // value groups per lane
  constexpr int VGR = kHeadDim / GS;        // value groups per row
  constexpr int SPG = GS / TPS;             // wave steps per key group
  constexpr float U = Unpack<BITS>::scale;
  constexpr float INV_U = 1.0f / U;
  using SM = SplitSmem<BITS, HPG, LPT>;
  static_assert(GS % TPS == 0, "a wave step must stay inside one key group");
  static_assert(WPL >= 1, "lane slice must hold whole words");

  __shared__ __attribute__((aligned(16))) float smem[SM::MAIN];

  const int unit = blockIdx.x;
  const int split = blockIdx.y;
  if (split == a.splits) {
    decode_tail<BITS, HPG>(a, unit, smem, SM::MAIN);
    return;
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = lane % LPT, tl = lane / LPT;
  const int b = unit / a.hkv, hk = unit % a.hkv;
  const int64_t cap = a.c.cap;
  const int64_t ngroups = a.n_main / GS;
  const int64_t g0 = ngroups * split / a.splits;
  const int64_t g1 = ngroups * (split + 1) / a.splits;
  const int64_t wg0 = g0 + (g1 - g0) * wave / kWaves;
  const int64_t wg1 = g0 + (g1 - g0) * (wave + 1) / kWaves;

  // query (log2 units) for channels 2*lane, 2*lane+1, used to fold key scales
  float qa[HPG], qb[HPG];
#pragma unroll
  for (int h = 0; h < HPG; ++h) {
    const uint16_t *qp = a.q + ((int64_t)(b * a.hq + hk * HPG + h)) * kHeadDim + 2 * lane;
    qa[h] = h2f(qp[0]) * a.qscale;
    qb[h] = h2f(qp[1]) * a.qscale;
  }

  float *lds_qp = smem + wave * (HPG * kHeadDim);
  float qf[HPG][CPL];
  float beta[HPG];
  float m[HPG], lsum[HPG], acc[HPG][CPL], bias[HPG][NVG];
#pragma unroll
  for (int h = 0; h < HPG; ++h) {
    m[h] = -INFINITY;
    lsum[h] = 0.0f;
    beta[h] = 0.0f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) acc[h][i] = 0.0f;
#pragma unroll
    for (int k = 0; k < NVG; ++k) bias[h][k] = 0.0f;
  }

  const uint32_t *kc = a.c.k_codes + (int64_t)unit * cap * W + j * WPL;
  const uint32_t *vc = a.c.v_codes + (int64_t)unit * cap * W + j * WPL;
  const float *vsp = a.c.v_scale + (int64_t)unit * cap * VGR + (j * CPL) / GS;
  const int16_t *vzp = a.c.v_zero + (int64_t)unit * cap * VGR + (j * CPL) / GS;
  const float *ksp = a.c.k_scale + (int64_t)unit * (cap / GS) * kHeadDim + 2 * lane;
  const int16_t *kzp = a.c.k_zero + (int64_t)unit * (cap / GS) * kHeadDim + 2 * lane;

  const int64_t nsteps = (wg1 - wg0) * SPG;
  for (int64_t st = 0; st < nsteps; ++st) {
    const int64_t g = wg0 + st / SPG;
    const int sub = (int)(st % SPG);
    if (sub == 0) {
      // fold this key group's per-channel scales into the query
      const float2 S = *reinterpret_cast<const float2 *>(ksp + g * kHeadDim);
      const uint32_t zw = *reinterpret_cast<const uint32_t *>(kzp + g * kHeadDim);
      const float z0 = (float)(int16_t)(zw & 0xffffu);
      const float z1 = (float)(int16_t)(zw >> 16);
#pragma unroll
      for (int h = 0; h < HPG; ++h) {
        const float p0 = qa[h] * S.x, p1 = qb[h] * S.y;
        beta[h] = wave_sum(fmaf(p0, z0, p1 * z1));
        *reinterpret_cast<float2 *>(lds_qp + h * kHeadDim + 2 * lane) = make_float2(p0 * INV_U, p1 * INV_U);
      }
      wave_sync();
#pragma unroll
      for (int h = 0; h < HPG; ++h) {
#pragma unroll
        for (int i = 0; i < CPL; i += 4) {
          const float4 v = *reinterpret_cast<const float4 *>(lds_qp + h * kHeadDim + j * CPL + i);
          qf[h][i] = v.x; qf[h][i + 1] = v.y; qf[h][i + 2] = v.z; qf[h][i + 3] = v.w;
        }
      }
      wave_sync();
    }
    const int64_t t = g * GS + (int64_t)sub * TPS + tl;
    uint32_t kw[WPL], vw[WPL];
    load_words<WPL>(kc + t * W, kw);
    load_words<WPL>(vc + t * W, vw);
    float vs[NVG], vz[NVG];
#pragma unroll
    for (int k = 0; k < NVG; ++k) {
      vs[k] = vsp[t * VGR + k];
      vz[k] = (float)vzp[t * VGR + k];
    }

    // scores
    float kf[CPL];
#pragma unroll
    for (int w = 0; w < WPL; ++w) Unpack<BITS>::run(kw[w], kf + w * PER);
    float s[HPG];
#pragma unroll
    for (int h = 0; h < HPG; ++h) {
      float d0 = 0.f, d1 = 0.f, d2 = 0.f, d3 = 0.f;
#pragma unroll
      for (int i = 0; i < CPL; i += 4) {
        d0 = fmaf(qf[h][i], kf[i], d0);
        d1 = fmaf(qf[h][i + 1], kf[i + 1], d1);
        d2 = fmaf(qf[h][i + 2], kf[i + 2], d2);
        d3 = fmaf(qf[h][i + 3], kf[i + 3], d3);
      }
      float d = (d0 + d1) + (d2 + d3);
#pragma unroll
      for (int o = 1; o < LPT; o <<= 1) d += __shfl_xor(d, o);
      s[h] = d + beta[h];
    }
    // online softmax with a lazily raised, wave-uniform maximum
    float p[HPG];
#pragma unroll
    for (int h = 0; h < HPG; ++h) {
      if (__any(s[h] > m[h] + kMargin)) {
        const float mn = fmaxf(m[h], wave_max(s[h]));
        const float f = exp2f(m[h] - mn);
        m[h] = mn;
        lsum[h] *= f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) acc[h][i] *= f;
#pragma unroll
        for (int k = 0; k < NVG; ++k) bias[h][k] *= f;
      }
      p[h] = exp2f(s[h] - m[h]);
      lsum[h] += p[h];
    }
    // values
    float vf[CPL];
#pragma unroll
    for (int w = 0; w < WPL; ++w) Unpack<BITS>::run(vw[w], vf + w * PER);
#pragma unroll
    for (int h = 0; h < HPG; ++h) {
#pragma unroll
      for (int k = 0; k < NVG; ++k) {
        const float wt = p[h] * vs[k];
        bias[h][k] = fmaf(wt, vz[k], bias[h][k]);
        constexpr int SPAN = CPL / NVG;
#pragma unroll
        for (int i = 0; i < SPAN; ++i) acc[h][k * SPAN + i] = fmaf(wt, vf[k * SPAN + i], acc[h][k * SPAN + i]);
      }
    }
  }

  // ---- combine the 4 waves and the TPS token lanes of each wave
  float lw[HPG];
#pragma unroll
  for (int h = 0; h < HPG; ++h) lw[h] = wave_sum(lsum[h]) * (1.0f / LPT);
  __syncthreads();   // every wave is done with its folded-query buffer
  float *s_ml = smem + (SM::MAIN - 4 * kWaves * HPG);   // [wave][h][m, l]
  float *s_red = smem;                                  // [kWaves*TPS][RS]
  float *s_half = smem + kWaves * TPS * SM::RS;         // [2][128]
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < HPG; ++h) {
      s_ml[(wave * HPG + h) * 2] = m[h];
      s_ml[(wave * HPG + h) * 2 + 1] = lw[h];
    }
  }
  __syncthreads();
  const int nparts = a.splits + 1;
#pragma unroll
  for (int h = 0; h < HPG; ++h) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_ml[(w * HPG + h) * 2]);
    const float fw = (m[h] == -INFINITY) ? 0.0f : exp2f(m[h] - M);
    float *row = s_red + (wave * TPS + tl) * SM::RS + j * CPL;
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
      const int c = tid & (kHeadDim - 1), part = tid >> 7;
      float sum = 0.0f;
      for (int r = part; r < kWaves * TPS; r += 2) sum += s_red[r * SM::RS + c];
      s_half[part * kHeadDim + c] = sum;
    }
    __syncthreads();
    if (tid < kHeadDim) {
      const int64_t bh = (int64_t)b * a.hq + hk * HPG + h;
      float *rec = a.partials + (bh * nparts + split) * kPartialStride;
      rec[tid] = s_half[tid] + s_half[kHeadDim + tid];
      if (tid == 0) {
        float L = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          const float mw = s_ml[(w * HPG + h) * 2];
          if (mw != -INFINITY) L += exp2f(mw - M) * s_ml[(w * HPG + h) * 2 + 1];
        }
        rec[kHeadDim] = M;
        rec[kHeadDim + 1] = L;
      }
    }
    __syncthreads();
  }
}

// Merge of the split records: m = max m_i, l = sum l_i 2^(m_i - m),
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
hipError_t launch_split(const AttnArgs &a, hipStream_t s) {
  constexpr int LPT = (HPG == 1) ? (BITS == 2 ? 2 : 4) : (HPG == 2 ? 4 : 8);
  dim3 grid(a.batch * a.hkv, a.splits + 1);
  hipLaunchKernelGGL((decode_split_kernel<BITS, GS, HPG, LPT>), grid, dim3(kWave * kWaves), 0, s, a);
  return hipGetLastError();
}

template <int BITS, int GS>
hipError_t launch_by_heads(const AttnArgs &a, hipStream_t s) {
  switch (a.hq / a.hkv) {
    case 1: return launch_split<BITS, GS, 1>(a, s);
    case 2: return launch_split<BITS, GS, 2>(a, s);
    case 4: return launch_split<BITS, GS, 4>(a, s);
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
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(merge_kernel, dim3(a.batch * a.hq), dim3(kHeadDim), 0, s, a.partials, a.out,
                     a.splits + 1);
  return hipGetLastError();
}

}  // namespace kvq
