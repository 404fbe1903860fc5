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
// split also takes the tokens after the whole groups and the sink tokens,
// reading each token's key and value either dequantized or fp16 (with a FIFO
// value queue, keys may be quantized while their values are still fp16).
// Within a wave, LPT lanes share a
// token and each owns 128 / LPT channels, so a wave step reads contiguous key
// and value rows with 8- or 16-byte loads; loads run one step ahead of the
// arithmetic through a ring of two register buffers.  Each wave keeps its
// own online-softmax state with a wave-uniform running maximum that is raised
// only when a score exceeds it by more than a margin, so the rescale branch is
// rare and uniform.  A unit with one part writes its output directly;
// otherwise every part writes a (max, sum, acc) record and a second kernel
// merges them.  Softmax arithmetic is in log2 units.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include "kvq_internal.h"
#include "kvq_attn_common.h"
#include "kvq_quant_common.h"

namespace kvq {
namespace {

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
  static constexpr int RED = kRedFloats<HPG>;
  static constexpr int QPW = HPG * (kHeadDim + 8);                // per wave: q'[HPG][128], beta[HPG][8]
  static constexpr int QP = kWaves * QPW;
  static constexpr int WORK = RED > QP ? RED : QP;
  static constexpr int SMEM = WORK + kStageFloats<HPG>;  // floats
};

// One group's (S, Z) at index idx of a scale / zero-point pair of arrays, in
// either metadata format.
template <int META>
__device__ __forceinline__ void group_meta(const float *scale, const int16_t *zero, int64_t idx, float &S, float &Z) {
  if constexpr (META) {
    const uint32_t w = reinterpret_cast<const uint32_t *>(scale)[idx];
    S = h2f((uint16_t)(w & 0xffffu));
    Z = (float)(int16_t)(w >> 16);
  } else {
    S = scale[idx];
    Z = (float)zero[idx];
  }
}

// ---------------------------------------------------------------- rest tokens
// Channels c0 .. c0 + CPL - 1 of one token row of the cache, dequantized:
// x = S * (code + Z) with the (S, Z) of the channel's group.  Keys carry one
// (S, Z) per (group of GS tokens, channel), values one per (token, group of
// GS channels).
template <int BITS, int GS, int CPL, int META>
__device__ __forceinline__ void dequant_row(const CacheView &c, bool values, int unit, int64_t t, int c0, float *x) {
  constexpr int PER = 32 / BITS, W = kHeadDim / PER, VGR = kHeadDim / GS;
  constexpr uint32_t MASK = (1u << BITS) - 1u;
  const int64_t cap = c.cap;
  const uint32_t *row = (values ? c.v_codes : c.k_codes) + ((int64_t)unit * cap + t) * W + c0 / PER;
#pragma unroll
  for (int w = 0; w < CPL / PER; ++w) {
    const uint32_t word = row[w];
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int ch = c0 + w * PER + e;
      const int64_t idx = values ? ((int64_t)unit * cap + t) * VGR + ch / GS
                                 : ((int64_t)unit * (cap / GS) + t / GS) * kHeadDim + ch;
      float S, Z;
      group_meta<META>(values ? c.v_scale : c.k_scale, values ? c.v_zero : c.k_zero, idx, S, Z);
      x[w * PER + e] = S * ((float)((word >> (e * BITS)) & MASK) + Z);
    }
  }
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

// META = 1: group metadata as packed words (fp16 S | Z << 16) in *_scale.
// MIXED = 1: some of the tokens after the whole key groups have a quantized
// key or value (a FIFO value queue), so the rest phase can dequantize rows;
// the instance without it keeps the registers of the all-fp16 rest phase.
template <int BITS, int GS, int HPG, int LPT, int META, int MIXED>
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
  const int split = (int)blockIdx.x / units;
  const int unit = (int)blockIdx.x % units;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
  const int j = lane % LPT, tl = lane / LPT;
  const int b = unit / a.hkv, hk = unit % a.hkv;
  const int64_t cap = a.c.cap;
  const int ngroups = (int)(a.n_main / GS);
  const int g0 = (int)((int64_t)ngroups * split / a.splits);
  const int g1 = (int)((int64_t)ngroups * (split + 1) / a.splits);
  // a wave's key groups: a contiguous eighth of the split, or (a.interleave,
  // chosen on the host for long splits) every eighth group, so the
  // workgroup's waves read neighbouring groups at any one time
  const int wg0 = a.interleave ? g0 + wave : g0 + (g1 - g0) * wave / kWaves;
  const int wstride = a.interleave ? kWaves : 1;
  const int wgroups = a.interleave ? (g1 - g0 - wave + kWaves - 1) / kWaves
                                   : (g1 - g0) * (wave + 1) / kWaves - (g1 - g0) * wave / kWaves;
  const int nsteps = wgroups * SPG;

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
#pragma unroll
  for (int h = 0; h < HPG; ++h) {
    beta[h] = 0.0f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) qf[h][i] = 0.0f;
  }
  Online<HPG, CPL, NVG> o;
  o.init();

  // per-unit buffer resources (uniform); lane-constant byte offsets
  const int64_t ngr_cap = cap / GS;
  const Rsrc rkc = rsrc_of(a.c.k_codes + (int64_t)unit * cap * W, (uint32_t)(cap * W * 4));
  const Rsrc rvc = rsrc_of(a.c.v_codes + (int64_t)unit * cap * W, (uint32_t)(cap * W * 4));
  const Rsrc rvs = rsrc_of(a.c.v_scale + (int64_t)unit * cap * VGR, (uint32_t)(cap * VGR * 4));
  const Rsrc rks = rsrc_of(a.c.k_scale + (int64_t)unit * ngr_cap * kHeadDim, (uint32_t)(ngr_cap * kHeadDim * 4));
  // separate zero-point arrays only with fp32 metadata (null otherwise)
  const Rsrc rvz = META ? rvs : rsrc_of(a.c.v_zero + (int64_t)unit * cap * VGR, (uint32_t)(cap * VGR * 2));
  const Rsrc rkz = META ? rks : rsrc_of(a.c.k_zero + (int64_t)unit * ngr_cap * kHeadDim, (uint32_t)(ngr_cap * kHeadDim * 2));
  const uint32_t code_lane = (uint32_t)(tl * W + j * WPL) * 4u;
  const uint32_t vmeta_lane = (uint32_t)(tl * VGR + (j * CPL) / GS);
  const uint32_t kmeta_lane = (uint32_t)(2 * lane);

  auto load = [&](Buf &bf, int s) {
    s = s < nsteps ? s : nsteps - 1;   // past the end: reload the last step (never processed)
    const uint32_t g = (uint32_t)(wg0 + wstride * (s / SPG));
    const uint32_t tb = g * GS + (uint32_t)((s % SPG) * TPS);   // first token of the step (uniform)
    bload_words<WPL>(rkc, code_lane, tb * (W * 4), bf.kw);
    bload_words<WPL>(rvc, code_lane, tb * (W * 4), bf.vw);
    if constexpr (META) {
      // packed words: vs[] carries the raw words, decoded in process()
      if constexpr (NVG == 2) {
        const float2 v2 = __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(rvs, vmeta_lane * 4, tb * (VGR * 4), kStream));
        bf.vs[0] = v2.x;
        bf.vs[1] = v2.y;
      } else {
        bf.vs[0] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rvs, vmeta_lane * 4, tb * (VGR * 4), kStream));
      }
      bf.vz = 0;
    } else if constexpr (NVG == 2) {
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
    if constexpr (META) {
      bf.kz = 0;   // the zero-points are in the high halves of ks
    } else {
      bf.kz = __builtin_amdgcn_raw_buffer_load_b32(rkz, kmeta_lane * 2, g * (kHeadDim * 2), 0);
    }
  };

  auto process = [&](const Buf &bf, int s) {
    if (s % SPG == 0) {
      // new key group: fold its per-channel scales into the query; each block
      // of FOLD lanes holds one lane slice's channels and sums its share of
      // the zero-point bias
      float ks0, ks1, z0, z1;
      if constexpr (META) {
        const uint32_t w0 = __float_as_uint(bf.ks.x), w1 = __float_as_uint(bf.ks.y);
        ks0 = h2f((uint16_t)(w0 & 0xffffu));
        ks1 = h2f((uint16_t)(w1 & 0xffffu));
        z0 = (float)(int16_t)(w0 >> 16);
        z1 = (float)(int16_t)(w1 >> 16);
      } else {
        ks0 = bf.ks.x;
        ks1 = bf.ks.y;
        z0 = (float)(int16_t)(bf.kz & 0xffffu);
        z1 = (float)(int16_t)(bf.kz >> 16);
      }
#pragma unroll
      for (int h = 0; h < HPG; ++h) {
        const float p0 = qa[h] * ks0, p1 = qb[h] * ks1;   // q'/U
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
    for (int h = 0; h < HPG; ++h) p[h] = o.weight(h, block_sum<LPT>((sc[h] + d1[h]) + beta[h]));
    // values
    float vs[NVG], vz[NVG];
    if constexpr (META) {
#pragma unroll
      for (int k = 0; k < NVG; ++k) {
        const uint32_t w = __float_as_uint(bf.vs[k]);
        vs[k] = h2f((uint16_t)(w & 0xffffu));
        vz[k] = (float)(int16_t)(w >> 16);
      }
    } else {
#pragma unroll
      for (int k = 0; k < NVG; ++k) vs[k] = bf.vs[k];
      vz[0] = (float)(int16_t)(bf.vz & 0xffffu);
      if constexpr (NVG == 2) vz[1] = (float)(int16_t)(bf.vz >> 16);
    }
#pragma unroll
    for (int h = 0; h < HPG; ++h) {
#pragma unroll
      for (int k = 0; k < NVG; ++k) o.bias[h][k] = fmaf(p[h] * vs[k], vz[k], o.bias[h][k]);
    }
#pragma unroll
    for (int w = 0; w < WPL; ++w) {
      float vf[PER];
      Unpack<BITS>::run(bf.vw[w], vf);
      constexpr int SPAN = CPL / NVG;
      const int k = (w * PER) / SPAN;
#pragma unroll
      for (int h = 0; h < HPG; ++h) {
        const float wt = p[h] * vs[k];
#pragma unroll
        for (int i = 0; i < PER; ++i) o.acc[h][w * PER + i] = fmaf(wt, vf[i], o.acc[h][w * PER + i]);
      }
    }
  };

  if (nsteps > 0) {
    // Loads run one step ahead (a two-buffer ring).  Two steps ahead put
    // about 58 KB per compute unit in flight, past the point where a plain
    // streaming read loses bandwidth on this part (a read probe peaks near
    // 32 KB per compute unit); one step ahead measured 2.5-3% faster on the
    // 2-bit and 4-bit MHA workloads.
    Buf A, B;
    load(A, 0);
    asm volatile("" ::: "memory");
    for (int s = 0; s < nsteps; s += 2) {
      progress_priority(nsteps - s, nsteps);
      load(B, s + 1);
      process(A, s);
      load(A, s + 2);
      if (s + 1 < nsteps) process(B, s + 1);
    }
  }

  // The rest of the tokens, in the last split: the sink tokens (rows of
  // k_sink) and tokens [n_main, n) after the whole key groups, whose keys and
  // values are each quantized (t < nq_k, t < nq_v: a FIFO value queue leaves
  // keys quantized whose values are still fp16) or fp16 in the ring.  Same
  // lane layout, plain query, the keys and values of each token dequantized
  // or read as fp16, weights p * U so the final 1/U scaling applies.
  const int rcount = a.resid_main ? (int)(a.n - a.n_main) : 0;
  const int nf = a.nsink + rcount;
  if (nf > 0 && split == a.splits - 1) {
    const int R = a.c.residual, S = a.c.sinks;
    const uint16_t *kr = a.c.k_resid + (int64_t)unit * R * kHeadDim + j * CPL;
    const uint16_t *vr = a.c.v_resid + (int64_t)unit * R * kHeadDim + j * CPL;
#pragma unroll
    for (int h = 0; h < HPG; ++h) {
      const uint16_t *qp = a.q + ((int64_t)(b * a.hq + hk * HPG + h)) * kHeadDim + j * CPL;
#pragma unroll
      for (int i = 0; i < CPL; ++i) qf[h][i] = h2f(qp[i]) * a.qscale;
    }
    if (rcount > 0 && a.k_new != nullptr && tid < 2 * (kHeadDim * 2 / 16)) {
      // fused step: store the new token into its ring slot
      constexpr int CH = kHeadDim * 2 / 16;
      const int which = tid / CH, ch = tid % CH;
      const uint4 *src = reinterpret_cast<const uint4 *>((which ? a.v_new : a.k_new) + (int64_t)unit * kHeadDim);
      uint4 *dst = reinterpret_cast<uint4 *>((which ? a.c.v_resid : a.c.k_resid) +
                                             ((int64_t)unit * R + (a.n - 1) % R) * kHeadDim);
      dst[ch] = src[ch];
    }
    for (int rs = wave; rs * TPS < nf; rs += kWaves) {
      const int i = rs * TPS + tl;
      const bool valid = i < nf;
      const int ii = valid ? i : 0;
      const bool sink = ii < a.nsink;
      const int64_t t = a.n_main + (ii - a.nsink);             // when not a sink
      const bool fresh = !sink && a.k_new != nullptr && t == a.n - 1;   // not in the ring yet
      const int64_t sink_off = ((int64_t)unit * S + ii) * kHeadDim + j * CPL;
      const int64_t slot = sink ? 0 : t % R;
      if constexpr (!MIXED) {
        // all fp16: both rows load together
        const uint16_t *krow = sink ? a.c.k_sink + sink_off
                                    : (fresh ? a.k_new + (int64_t)unit * kHeadDim + j * CPL : kr + slot * kHeadDim);
        const uint16_t *vrow = sink ? a.c.v_sink + sink_off
                                    : (fresh ? a.v_new + (int64_t)unit * kHeadDim + j * CPL : vr + slot * kHeadDim);
        fp16_token<HPG, CPL, NVG, LPT>(o, qf, krow, vrow, valid, U);
        continue;
      }
      // keys first, then values, so only one of the rows is live at a time
      float wt[HPG];
      {
        float kf[CPL];
        if (sink) {
          fp16_row<CPL>(a.c.k_sink + sink_off, kf);
        } else if (MIXED && t < a.nq_k) {
          dequant_row<BITS, GS, CPL, META>(a.c, false, unit, t, j * CPL, kf);
        } else {
          fp16_row<CPL>(fresh ? a.k_new + (int64_t)unit * kHeadDim + j * CPL : kr + slot * kHeadDim, kf);
        }
        token_weights<HPG, CPL, NVG, LPT>(o, qf, kf, valid, U, wt);
      }
      asm volatile("" ::: "memory");
      {
        float vf[CPL];
        if (sink) {
          fp16_row<CPL>(a.c.v_sink + sink_off, vf);
        } else if (MIXED && t < a.nq_v) {
          dequant_row<BITS, GS, CPL, META>(a.c, true, unit, t, j * CPL, vf);
        } else {
          fp16_row<CPL>(fresh ? a.v_new + (int64_t)unit * kHeadDim + j * CPL : vr + slot * kHeadDim, vf);
        }
        token_values<HPG, CPL, NVG>(o, wt, vf);
      }
    }
  }

  combine_waves<HPG, LPT, NVG>(o, smem, st, wave, lane, INV_U);
  finish_part<HPG>(a, unit, split, st);
  if (a.prequant >= 0 && split == 0 && wave == kWaves - 1) {
    // a full FIFO queue: its oldest value row is quantized now, ahead of the
    // next append's pop
    const int R = a.c.residual;
    quantize_value_row<BITS, GS>(a.c, a.c.v_resid + ((int64_t)unit * R + a.prequant % R) * kHeadDim,
                                 (int64_t)unit * cap + a.prequant);
  }
}

// Merge of the part records (one workgroup per query head, one thread per
// channel).
__global__ __launch_bounds__(kHeadDim) void merge_kernel(const float *__restrict__ partials,
                                                         float *__restrict__ out, int nparts) {
  const int64_t bh = blockIdx.x;
  const int c = threadIdx.x;
  out[bh * kHeadDim + c] = merge_records(partials + bh * nparts * kPartialStride, nparts, c);
}

template <int BITS, int GS, int HPG, int META>
hipError_t launch_kernel(const AttnArgs &a, hipStream_t s) {
  constexpr int LPT = (HPG == 1) ? 4 : (HPG == 2 ? 4 : 8);
  const int units = a.batch * a.hkv;
  // tokens after the whole key groups with a quantized key or value
  const bool mixed = a.resid_main && (a.nq_k > a.n_main || a.nq_v > a.n_main);
  if (mixed) {
    hipLaunchKernelGGL((decode_attn_kernel<BITS, GS, HPG, LPT, META, 1>), dim3(units * a.splits), dim3(kThreads), 0,
                       s, a);
  } else {
    hipLaunchKernelGGL((decode_attn_kernel<BITS, GS, HPG, LPT, META, 0>), dim3(units * a.splits), dim3(kThreads), 0,
                       s, a);
  }
  return hipGetLastError();
}

template <int BITS, int GS, int META>
hipError_t launch_by_heads(const AttnArgs &a, hipStream_t s) {
  switch (a.hq / a.hkv) {
    case 1: return launch_kernel<BITS, GS, 1, META>(a, s);
    case 2: return launch_kernel<BITS, GS, 2, META>(a, s);
    case 4: return launch_kernel<BITS, GS, 4, META>(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <int BITS, int META>
hipError_t launch_by_group(const AttnArgs &a, hipStream_t s) {
  switch (a.c.group) {
    case 32: return launch_by_heads<BITS, 32, META>(a, s);
    case 64: return launch_by_heads<BITS, 64, META>(a, s);
    case 128: return launch_by_heads<BITS, 128, META>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_merge(const AttnArgs &a, hipStream_t s) {
  if (a.nparts == 1) return hipSuccess;
  hipLaunchKernelGGL(merge_kernel, dim3(a.batch * a.hq), dim3(kHeadDim), 0, s, a.partials, a.out, a.nparts);
  return hipGetLastError();
}

namespace {

hipError_t launch_valu(const AttnArgs &a, hipStream_t s) {
  if (a.c.meta) return (a.c.bits == 2) ? launch_by_group<2, 1>(a, s) : launch_by_group<4, 1>(a, s);
  return (a.c.bits == 2) ? launch_by_group<2, 0>(a, s) : launch_by_group<4, 0>(a, s);
}

}  // namespace

hipError_t launch_decode_attention(const AttnArgs &a, hipStream_t s) {
  hipError_t e;
  // four query heads per kv head: the matrix-core kernel; each split also
  // takes a share of the sinks and tokens [n_main, n)
  const int64_t rest_tokens = a.nsink + (a.n - a.n_main);
  if (a.hq == 4 * a.hkv && a.n_main >= a.c.group && a.splits >= 1 && rest_tokens <= kGqaMaxRest &&
      a.mfma) {
    AttnArgs m = a;
    m.resid_main = 0;
    m.nparts = m.splits;
    // the unit's last workgroup merges the split records itself
    return launch_gqa_mfma(m, s);
  }
  if ((e = launch_valu(a, s)) != hipSuccess) return e;
  return launch_merge(a, s);
}

}  // namespace kvq
