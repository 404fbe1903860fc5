// Grouped-query decode attention on the matrix cores, gfx950: four query
// heads share each kv head, KIVI layout (keys quantized per channel over
// groups of G tokens, values per token over groups of G channels).
//
// Decoding reads the whole quantized cache once (KIVI part of the juejin.cn
// page "大模型量化技术原理：KIVI、IntactKV、KVQuant"); with four query heads
// per kv head each code feeds four products, and doing them one fused
// multiply-add at a time leaves the kernel limited by vector ALU issue rather
// than by HBM.  Both products are dense contractions, so this kernel runs
// them as 16x16 bf16 MFMA tiles with fp32 accumulation, keeping the
// group-dequantize-inside-the-product structure of the fused kernel in the
// euno.news InnerQ summary (methodology 3 and 5) and the scale folding of
// the vector-ALU kernel:
//
//   scores  s[t][h] = sum_c code[t][c] * q'[h][c] + beta[h]   (per key group)
//           q'[h][c] = q[h][c] S[g][c],  beta[h] = sum_c q'[h][c] Z[g][c]
//   values  o[h][c] += sum_t w[h][t][j] * code[t][c],  bias[h][j] += sum_t w[h][t][j] Z[t][j]
//           w[h][t][j] = p[h][t] S[t][j]   (j = value group of channel c)
//
// The codes are small integers, exact in bf16.  The real-valued operands q'
// and w are split into two bf16 limbs (high: the value rounded to bf16; low:
// the exact remainder rounded to bf16), so each product is two MFMAs on the
// same accumulator and its operand carries about 17 significant bits instead
// of 8.
//
// Tiles (one wave, 32 tokens per step = two 16-token blocks):
//  * key MFMA (16x16x32): A = codes, rows = 16 tokens, K = 32 channels per
//    pass (4 passes); B = q' limbs, columns = (head h, key group slot g') for
//    the four groups of a "super-chunk", so one preparation of q' serves 4G
//    tokens.  Output lane (column n, row block r) holds 4 tokens' scores for
//    column n; only columns of the step's own group slot are used.
//  * value codes are transposed to tokens-along-K through LDS: each wave
//    writes its step's codes as token rows and reads them back with a gfx950
//    transposing LDS read, so lane (channel, r) holds the codes of tokens
//    4r..4r+3 of each block -- exactly the token set whose scores the same
//    lane index holds in the key output.  The codes travel as 4-bit fields
//    (2-bit codes) or bytes (4-bit codes), a quarter or half of the bytes of
//    bf16, and are converted to bf16 after the read.
//  * value MFMA (16x16x32): A = w limbs, rows = (head, 32-channel slice),
//    K = the 32 tokens; B = transposed codes, columns = 16 channels.  The
//    weights move from the key output lanes to the A lanes with one quad
//    broadcast (same 16-lane row, lane g' of each quad).
// Key metadata of the next super-chunk and value metadata of the current step
// arrive with the step's loads (coalesced) and are staged through a per-wave
// LDS area into the lanes that need them.  The online softmax (log2 units,
// wave-uniform per-head maximum raised only past a margin) follows the
// vector-ALU kernel.  Work split: a unit's key groups form super-chunks of
// four; a unit has `splits` workgroups of four waves, rotated across the
// XCDs, and each wave takes super-chunks in a fixed strided order or, with
// the work-queue schedule, its first two by index and the rest from a
// per-unit ticket counter.  After its quantized groups every workgroup takes
// its share of the unit's fp16 tokens (sinks, the residual ring, the token of
// a fused step, the FIFO tail whose values are still fp16) with a plain
// dequantize-then-dot routine (gqa_fp16_part).  The unit's last workgroup, by
// a finished-workgroup counter, merges the split records inside the same
// launch (queue_finish).
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <utility>

#include "kvq_internal.h"
#include "kvq_attn_common.h"
#include "kvq_quant_common.h"

namespace kvq {
namespace {

typedef __bf16 bf8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));
typedef float fx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

constexpr int kHpg = 4;   // query heads per kv head on this path
// Tokens the fp16 part can take: sinks (<= 512), the residual (<= 512) and a
// partial key group (< 128).
constexpr int kMaxRest = kGqaMaxRest;

// Lane byte offset past every buffer this kernel reads, so a load that uses
// it returns zero and touches no memory.  The largest resource is a unit's
// 4-bit code buffer at the largest capacity, 2^25 tokens * 64 bytes = 2^31
// bytes; the loads that take this offset add at most 32 rows of 64 bytes of
// uniform offset (plus a 16-byte step), and the sum stays below 2^32, so the
// offset neither lands inside a resource nor wraps around.
constexpr uint32_t kOutOfRange = 0xFFFFF000u;
static_assert((uint64_t)kMaxTokens * (kHeadDim * 4 / 8) <= 0x80000000ull, "largest code resource");
static_assert((uint64_t)kOutOfRange >= 0x80000000ull + 4096, "sentinel above every resource");
static_assert((uint64_t)kOutOfRange + 32 * 64 + 16 < 0x100000000ull, "sentinel plus step offset fits 32 bits");
// Four waves per workgroup, two waves per SIMD (up to 256 VGPRs: the
// accumulators, both q' limb sets and a three-step load ring stay in
// registers; at three waves per SIMD the kernel spills and runs slower).
constexpr int kGqaWaves = 4;
constexpr int kGqaThreads = kGqaWaves * kWave;
constexpr int kGqaWavesPerEU = 2;


__device__ __forceinline__ fx4 mma_x32(u32x4 a, u32x4 b, fx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8_t, a), __builtin_bit_cast(bf8_t, b), c, 0,
                                                 0, 0);
}

// bf16 pair (lo = a, hi = b), each rounded to nearest even.
__device__ __forceinline__ uint32_t rne_pair(float a, float b) {
  const bf2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Two-limb split of a pair: hi = the values rounded to bf16, lo = the exact
// remainders (at most half a bf16 ulp) rounded to bf16, so hi + lo carries
// about 17 significant bits.
__device__ __forceinline__ void limbs(float a, float b, uint32_t &hi, uint32_t &lo) {
  hi = rne_pair(a, b);
  const float ha = __uint_as_float(hi << 16), hb = __uint_as_float(hi & 0xffff0000u);
  lo = rne_pair(a - ha, b - hb);
}

// A lane's 32 codes (channels 32 kq .. 32 kq + 31 of one token) as 16 words of
// exact bf16 pairs, produced one word at a time from the raw code words w[].
// Word 4p + r holds channels 8p + {0,2}, {1,3}, {4,6}, {5,7} for r = 0..3
// (the order the converts produce; the key preparation arranges q' the same
// way).  J is a compile-time index: the converts take a literal byte select.
template <int BITS>
struct CodesBf16;

template <>
struct CodesBf16<2> {
  static constexpr int WPL = 2;   // code words per lane per token
  template <int J>
  __device__ static __forceinline__ uint32_t word(const uint32_t *w) {
    constexpr int k = J / 8, b = (J % 8) / 2;
    // nibble i of m holds code 2i (even J) or 2i + 1 (odd J); fp4 nibble c is
    // worth c / 2, so scale 2 gives the code itself
    const uint32_t m = ((J & 1) ? (w[k] >> 2) : w[k]) & 0x33333333u;
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(m, 2.0f, b));
  }
};

template <>
struct CodesBf16<4> {
  static constexpr int WPL = 4;
  template <int J>
  __device__ static __forceinline__ uint32_t word(const uint32_t *w) {
    constexpr int k = J / 4, r = J % 4;
    // byte i of m holds code 2i (r even) or 2i + 1 (r odd); fp8 e4m3 byte c
    // (c < 16) is worth c / 512, so scale 512 gives the code itself
    const uint32_t m = ((r & 1) ? (w[k] >> 4) : w[k]) & 0x0F0F0F0Fu;
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(m, 512.0f, r >= 2));
  }
};

// Calls f(std::integral_constant<int, I>) for I = 0 .. N-1.
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Value codes are transposed through a per-wave LDS tile.  2-bit codes go
// through it as 4-bit fields: a token row
// is 64 bytes (rows kNRow bytes apart), and the step's second 16-token block
// starts kNBlk bytes after the first.  With 80-byte rows and the second block
// 64 bytes further on, the sixteen 8-byte rows one 16-lane group of a
// transposing read takes (tokens 4 kq + e and 16 + 4 kq + e, two 16-channel
// chunks) cover all 32 four-byte banks once, and the eight 16-byte row
// pieces a group of lanes writes fall in different bank quads.
constexpr int kNRow = 80;
constexpr int kNBlk = 16 * kNRow + 64;
// 4-bit codes go through it as bytes: a token row is 128 bytes (rows kBRow
// bytes apart, the second block kBBlk bytes after the first).  With 144-byte
// rows and the second block 64 bytes further on, the eight 16-byte row pieces
// one 16-lane group of a transposing 8-bit read takes (tokens 4 kq + e and
// 16 + 4 kq + e, one 16-channel chunk) fall in different bank quads, and so do
// the eight row pieces a group of lanes writes.
constexpr int kBRow = 144;
constexpr int kBBlk = 16 * kBRow + 64;
// Bytes of the tile area: the byte tile's extent, which holds the 4-bit one.
constexpr int kTileBytes = kBBlk + 16 * kBRow;
static_assert(kNBlk + 16 * kNRow <= kTileBytes && kTileBytes % 16 == 0, "tile area");
// Row length (floats) of the per-wave key-metadata staging, [4 groups][kKmRow].
constexpr int kKmRow = kHeadDim + 4;

// Channel offset (within 8) of element e of word r of a pass: 0,2 | 1,3 | 4,6 | 5,7.
__device__ __host__ constexpr int pass_chan(int r, int e) { return (r >> 1) * 4 + (r & 1) + 2 * e; }

// Channel (within 16) of 4-bit field f of a tile chunk: even channels in the
// first word, odd ones in the second.
__device__ __host__ constexpr int nib_chan(int f) { return f < 8 ? 2 * f : 2 * f - 15; }

// Fields 2B and 2B + 1 of a word of 2-bit codes held as 4-bit fields, as a
// bf16 pair (fp4 field c is worth c / 2, so scale 2 gives the code itself).
template <int B>
__device__ __forceinline__ uint32_t nib_bf16(uint32_t f) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(f, 2.0f, B));
}

// Channel (within 16) of byte p of a byte-tile chunk: the even codes of a
// code word, then its odd codes, for two code words.
__device__ __host__ constexpr int byte_chan(int p) { return 8 * (p >> 3) + 2 * (p & 3) + ((p >> 2) & 1); }

// Bytes 2H and 2H + 1 of a word of 4-bit codes held as bytes, as a bf16 pair
// (an fp8 e4m3 byte c < 16 is worth c / 512, so scale 512 gives the code).
template <int H>
__device__ __forceinline__ uint32_t byte_bf16(uint32_t f) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(f, 512.0f, H == 1));
}

template <int GS>
struct GqaGeo {
  static constexpr int SPG = GS / 32;                 // 32-token steps per key group
  static constexpr int SPC = 4 * SPG;                 // steps per super-chunk (4 groups)
  static constexpr int VGR = kHeadDim / GS;           // value groups per token
  static constexpr int EPS = 128 / SPG;               // metadata entries per step (keys and values alike)
  static constexpr int E = SPG == 1 ? 2 : 1;          // entries per lane per step
  static constexpr int SH = SPG == 1 ? 0 : (SPG == 2 ? 1 : 2);   // 32-channel slice -> value group shift
  // per-wave LDS staging (floats): key S and Z of a super-chunk [4][kKmRow]
  // (rows padded by 4 so the four groups' rows start on different banks),
  // value S and Z of a step [VGR][32]
  static constexpr int KM = 4 * kKmRow;
  static constexpr int VM = VGR * 32;
  // value codes of a step (the tile area, in floats)
  static constexpr int VT = kTileBytes / 4;
  static constexpr int PER_WAVE = 2 * KM + 2 * VM + VT;
  static constexpr int ROWS = kGqaWaves * kHpg * kHeadDim;   // combine rows [wave][h][128]
  static constexpr int STAGING = kGqaWaves * PER_WAVE;
  static constexpr int COMBINE = ROWS + 2 * kGqaWaves * kHpg;
  static constexpr int REST = kHpg * kMaxRest + kGqaWaves * kHpg * kHeadDim;   // fp16-part scores + wave sums
  static constexpr int WORK = STAGING > COMBINE ? (STAGING > REST ? STAGING : REST) : (COMBINE > REST ? COMBINE : REST);
  static constexpr int QS = kHpg * kHeadDim;                  // scaled query [h][128]
  static constexpr int STAGE2 = kStageFloats<kHpg>;                // second result: the fp16 share
  static constexpr int SMEM = WORK + QS + kStageFloats<kHpg> + kHpg * kHeadDim + 2 * kHpg;
};

template <int BITS, int GS>
struct GqaBuf {
  static constexpr int WPL = CodesBf16<BITS>::WPL;
  static constexpr int E = GqaGeo<GS>::E;
  uint32_t kw[2 * WPL];   // key code words, block 0 then block 1
  uint32_t vw[2 * WPL];
  uint32_t vs[E];         // value metadata of this step (S, or packed S | Z)
  uint32_t vz;            // int16 zero-points (fp32 metadata only)
};

// Key metadata of one super-chunk (4 groups x 128 channels = 512 entries),
// entries 8 lane .. 8 lane + 7: raw S (or packed S | Z) words and int16 Z.
struct GqaKMeta {
  uint4 s0, s1, z;
};

// Lane L of each quad to all four lanes of the quad.
template <int L>
__device__ __forceinline__ float quad_bcast(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), L * 0x55, 0xF, 0xF, true));
}

__device__ __forceinline__ float sel4(int i, float a, float b, float c, float d) {
  return i == 0 ? a : (i == 1 ? b : (i == 2 ? c : d));
}

__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m); }

// One (S, Z) metadata entry from its raw word(s).
template <int META>
__device__ __forceinline__ void decode_meta(uint32_t s_word, uint32_t zhalf, float &S, float &Z) {
  if constexpr (META) {
    S = h2f((uint16_t)(s_word & 0xffffu));
    Z = (float)(int16_t)(s_word >> 16);
  } else {
    S = __uint_as_float(s_word);
    Z = (float)(int16_t)zhalf;
  }
}

// A share of the unit's fp16 list -- sink rows [0, nsink), then tokens
// [n_main, n), whose keys and values are each quantized (rows below nq_k /
// nq_v) or fp16 (ring slot t mod R, or k_new / v_new for token n - 1 of a
// fused step): entries [ib, ie).  Plain dequantize-then-dot.  Scores: 16
// lanes per token (8 channels each), four tokens per wave at a time.
// Softmax: one wave per head.  P.V: 16 token slots x 16 channel octets.  Row
// loads of kRestBatch rounds (16 tokens each) are issued before any of them
// is used.  Two rounds cover the usual share (a split's part of a residual
// of at most R tokens); eight made this rarely run code so long that a fused
// decode step on the 2-bit GQA workload took 2.2 us longer (its instructions
// are fetched cold once per call).
// Leaves the share's (acc, max, sum) in out_acc / out_ml.
constexpr int kRestBatch = 2;

// 8 channels (8 c .. 8 c + 7) of token i of the fp16 part, as raw fp16 pairs
// (fp16 rows) or dequantized (quantized rows, via `quant`).
struct RestRow {
  const uint16_t *row;   // fp16 row, or null for a quantized one
  int t;                 // token index when quantized (below 2^25)
};

// (Index arithmetic with the compile-time group size and 32-bit token
// indices: this code runs once per call, and its length is fetched cold.)
template <int BITS, int GS, int META>
__device__ __forceinline__ void dequant8(const uint32_t *codes, const float *scale, const int16_t *zero, int unit,
                                         int64_t cap, int t, int c8, bool keys, float *out) {
  constexpr int PER = 32 / BITS;
  constexpr int W = kHeadDim / PER;
  constexpr uint32_t MASK = (1u << BITS) - 1u;
  const int64_t row = (int64_t)unit * cap + t;
  const uint32_t w = codes[row * W + (8 * c8) / PER];
  const int sh = ((8 * c8) % PER) * BITS;
  // keys: (S, Z) per (group of GS tokens, channel); values: per (token, group
  // of GS channels) -- the 8 channels share one value group since GS >= 32
  const int64_t mi = keys ? ((int64_t)unit * (cap / GS) + t / GS) * kHeadDim + 8 * c8
                          : row * (kHeadDim / GS) + (8 * c8) / GS;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float Sc, Z;
    const int64_t m = keys ? mi + e : mi;
    if constexpr (META) {
      decode_meta<1>(reinterpret_cast<const uint32_t *>(scale)[m], 0, Sc, Z);
    } else {
      decode_meta<0>(__float_as_uint(scale[m]), (uint16_t)zero[m], Sc, Z);
    }
    out[e] = ((float)((w >> (sh + e * BITS)) & MASK) + Z) * Sc;
  }
}

__device__ __forceinline__ void fp16x8(uint4 v, float *out) {
  const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    out[2 * e] = h2f((uint16_t)(w4[e] & 0xffffu));
    out[2 * e + 1] = h2f((uint16_t)(w4[e] >> 16));
  }
}

static_assert(kGqaWaves == kHpg, "the fp16 part runs one wave per head in its softmax");

template <int BITS, int GS, int META>
__device__ void gqa_fp16_part(const AttnArgs &a, int unit, float *smem, const float *qsm, float *out_acc,
                              float *out_ml, int ib, int ie) {
  const int R = a.c.residual, S = a.c.sinks;
  const int64_t cap = a.c.cap;
  const int ns = a.nsink;
  const int nt = ie - ib;                     // tokens [ib, ie) of the unit's fp16 list
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float *s_sc = smem;                         // [kHpg][nt] scores, then weights
  float *s_red = smem + kHpg * kMaxRest;      // [kGqaWaves][kHpg][128]
  // row of local token li (list entry ib + li) for keys (k = true) or values
  // token counts stay below 2^25, so 32-bit indices (and one 32-bit
  // remainder) do here
  const int n_main = (int)a.n_main, n_last = (int)a.n - 1, nqk = (int)a.nq_k, nqv = (int)a.nq_v;
  auto row_of = [&](int li, bool k) -> RestRow {
    const int i = ib + li;
    if (i < ns) return {(k ? a.c.k_sink : a.c.v_sink) + ((int64_t)unit * S + i) * kHeadDim, 0};
    const int t = n_main + (i - ns);
    if (t < (k ? nqk : nqv)) return {nullptr, t};
    if ((k ? a.k_new : a.v_new) != nullptr && t == n_last)
      return {(k ? a.k_new : a.v_new) + (int64_t)unit * kHeadDim, 0};
    return {(k ? a.c.k_resid : a.c.v_resid) + ((int64_t)unit * R + (int)((uint32_t)t % (uint32_t)R)) * kHeadDim, 0};
  };

  // ---- scores: lane j of token group sub takes channels 8j .. 8j + 7
  {
    const int j = lane & 15, sub = lane >> 4;
    float qv[kHpg][8];
#pragma unroll
    for (int h = 0; h < kHpg; ++h) {
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[h][e] = qsm[h * kHeadDim + 8 * j + e];
    }
    constexpr int STRIDE = kGqaWaves * 4;   // tokens per round
    for (int i0 = wave * 4 + sub; i0 < nt; i0 += STRIDE * kRestBatch) {
      uint4 raw[kRestBatch];
      RestRow rr[kRestBatch];
#pragma unroll
      for (int r = 0; r < kRestBatch; ++r) {
        const int i = i0 + r * STRIDE;
        rr[r] = i < nt ? row_of(i, true) : RestRow{nullptr, -1};
        raw[r] = rr[r].row != nullptr ? *reinterpret_cast<const uint4 *>(rr[r].row + 8 * j) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < kRestBatch; ++r) {
        const int i = i0 + r * STRIDE;
        float kf[8];
        if (rr[r].row != nullptr || rr[r].t < 0) {
          fp16x8(raw[r], kf);
        } else {
          dequant8<BITS, GS, META>(a.c.k_codes, a.c.k_scale, a.c.k_zero, unit, cap, rr[r].t, j, true, kf);
        }
#pragma unroll
        for (int h = 0; h < kHpg; ++h) {
          float d = 0.0f;
#pragma unroll
          for (int e = 0; e < 8; ++e) d = fmaf(qv[h][e], kf[e], d);
          d = block_sum<16>(d);
          if (j == 0 && i < nt) s_sc[h * nt + i] = d;
        }
      }
    }
  }
  __syncthreads();
  {
    const int h = wave;   // one wave per head
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
      out_ml[2 * h] = nt > 0 ? mx : -INFINITY;
      out_ml[2 * h + 1] = l;
    }
  }
  __syncthreads();
  // ---- P.V: thread (token slot ts, channel octet c8)
  {
    const int c8 = tid & 15, ts = tid >> 4;
    float acc[kHpg][8];
#pragma unroll
    for (int h = 0; h < kHpg; ++h) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] = 0.0f;
    }
    constexpr int SLOTS = kGqaThreads / 16;
    for (int i0 = ts; i0 < nt; i0 += SLOTS * kRestBatch) {
      uint4 raw[kRestBatch];
      RestRow rr[kRestBatch];
#pragma unroll
      for (int r = 0; r < kRestBatch; ++r) {
        const int i = i0 + r * SLOTS;
        rr[r] = i < nt ? row_of(i, false) : RestRow{nullptr, -1};
        raw[r] = rr[r].row != nullptr ? *reinterpret_cast<const uint4 *>(rr[r].row + 8 * c8) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < kRestBatch; ++r) {
        const int i = i0 + r * SLOTS;
        if (i >= nt) continue;
        float vf[8];
        if (rr[r].row != nullptr) {
          fp16x8(raw[r], vf);
        } else {
          dequant8<BITS, GS, META>(a.c.v_codes, a.c.v_scale, a.c.v_zero, unit, cap, rr[r].t, c8, false, vf);
        }
#pragma unroll
        for (int h = 0; h < kHpg; ++h) {
          const float p = s_sc[h * nt + i];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(p, vf[e], acc[h][e]);
        }
      }
    }
    // sum the four token slots of each wave (lanes xor 16, xor 32), then the waves
#pragma unroll
    for (int h = 0; h < kHpg; ++h) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float v = acc[h][e];
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        acc[h][e] = v;
      }
    }
    if (lane < 16) {
#pragma unroll
      for (int h = 0; h < kHpg; ++h) {
#pragma unroll
        for (int e = 0; e < 8; ++e) s_red[(wave * kHpg + h) * kHeadDim + 8 * c8 + e] = acc[h][e];
      }
    }
  }
  __syncthreads();
  for (int idx = tid; idx < kHpg * kHeadDim; idx += kGqaThreads) {
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < kGqaWaves; ++w) v += s_red[w * kHpg * kHeadDim + idx];
    out_acc[idx] = v;
  }
  __syncthreads();
}

template <int BITS, int GS, int META>
__global__ __launch_bounds__(kGqaThreads) __attribute__((amdgpu_waves_per_eu(kGqaWavesPerEU, kGqaWavesPerEU)))
void gqa_mfma_kernel(AttnArgs a) {
  using Gm = GqaGeo<GS>;
  using Buf = GqaBuf<BITS, GS>;
  constexpr int WPL = Buf::WPL, E = Gm::E, SPG = Gm::SPG, SPC = Gm::SPC, VGR = Gm::VGR, EPS = Gm::EPS;
  constexpr int W = kHeadDim * BITS / 32;   // code words per token row
  constexpr int LOG_SPG = SPG == 1 ? 0 : (SPG == 2 ? 1 : 2);
  // Steps whose loads are in flight ahead of the one processed: three for
  // 2-bit codes (a four-buffer ring, 2% faster on the 2-bit GQA workload),
  // two for 4-bit, whose larger buffers would not fit a fourth one.
  constexpr int LA = BITS == 2 ? 3 : 2;

  __shared__ __attribute__((aligned(16))) float smem[Gm::SMEM];
  __shared__ uint32_t s_took[kGqaWaves + 1];   // super-chunks per wave; then the last-part flag
  const Stage st = stage_of<kHpg>(smem, Gm::WORK + Gm::QS);
  float *qsm = smem + Gm::WORK;   // scaled query [h][128], shared by the workgroup's waves

  const int units = a.batch * a.hkv;
  const int split = (int)blockIdx.x / units;
  // Workgroups are dealt to the XCDs round-robin, and the first 256 take one
  // slot per CU before the rest fill the second.  Rotating the unit by the
  // split puts a unit's workgroups on different XCDs and in both rounds, so
  // the shared work queue below can even out slower XCDs and the younger
  // workgroup of each CU.
  const int unit = ((int)blockIdx.x % units + split) % units;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i16 = lane & 15, kq = lane >> 4;
  const int hk_lane = i16 >> 2;   // head of key-output / value-A lanes
  const int b = unit / a.hkv, hk = unit % a.hkv;
  const int64_t cap = a.c.cap;
  const int ngroups = (int)(a.n_main / GS);
  // Work queue.  The unit's key groups form super-chunks of four (the last
  // one possibly shorter).  Each wave of the unit takes its first two
  // super-chunks by its index among the unit's nw waves (slot, nw + slot),
  // then one at a time from the unit's ticket counter (super-chunk
  // 2 nw + ticket), grabbed a whole super-chunk before its loads are issued.
  // With a.dynamic == 0 the sequence stays strided (slot + k nw): the same
  // partial sums on every run.
  // Ids only grow along a wave's sequence, so the first id past the end ends
  // the wave.  At its end every workgroup adds (1 << 24) | (super-chunks its
  // waves took) to the unit's second counter; the unit's last workgroup
  // checks that the count is complete (else its output is NaN: the counters
  // did not start at zero), returns both counters to zero for the next call
  // and merges the unit's split records.
  const int nsc = (ngroups + 3) / 4;
  const int nw = a.splits * kGqaWaves;
  const int slot = split * kGqaWaves + wave;
  uint32_t *const ticket = a.ctr + kCtrWords * unit;
  auto grab = [&]() { return queue_grab(ticket, lane); };   // read at the next super-chunk
  auto live_steps = [&](uint32_t id) { return (ngroups - 4 * (int)id < 4 ? ngroups - 4 * (int)id : 4) * SPG; };
  // ids compare unsigned, so any value past the end (however large) ends the wave
  uint32_t idL = slot, idL1 = nw + slot;   // super-chunk of the load cursor, and the next one
  int nsteps = 0x7fffffff;                 // known once the next super-chunk is past the end
  uint32_t pend = 0;                       // ticket grabbed for the super-chunk after idL1
  if (idL >= (uint32_t)nsc) {
    nsteps = 0;
  } else if (idL1 >= (uint32_t)nsc) {
    nsteps = live_steps(idL);
  } else if (a.dynamic) {
    pend = grab();
  }

  float *kmS = smem + wave * Gm::PER_WAVE;
  float *kmZ = kmS + Gm::KM;
  float *lvS = kmZ + Gm::KM;
  float *lvZ = lvS + Gm::VM;
  uint8_t *const nt = reinterpret_cast<uint8_t *>(lvZ + Gm::VM);   // value-code tile (4-bit fields or bytes)

  // scaled query of the unit's four heads
  for (int i = tid; i < kHpg * kHeadDim; i += kGqaThreads)
    qsm[i] = h2f(a.q[((int64_t)(b * a.hq + hk * kHpg)) * kHeadDim + i]) * a.qscale;
  __syncthreads();

  // 2-bit codes: lane (token i16 of block k, kq) writes its 32 codes as 4-bit
  // fields at row i16 of block k, bytes 16 kq ..: chunk 2 kq + x (8 bytes)
  // holds channels 16 (2 kq + x) + {0, 2, .., 14} in its first word and
  // + {1, 3, .., 15} in its second, so field f of a chunk is channel
  // 16 chunk + nib_chan(f).  A transposing 4-bit read returns to lane i of a
  // 16-lane group field i of the 8-byte row each lane j of the group points
  // at, in lane order; lane j points at token 4 kq + (j mod 4) of block
  // (j / 4) mod 2, chunk 2 u + j / 8.  So lane (column i16, kq) receives, in
  // its first word, the codes of channel 16 (2u) + nib_chan(i16) for tokens
  // 4 kq + e and 16 + 4 kq + e (e = 0..3, in that order: the key-output token
  // order), and the same for chunk 2u + 1 in its second word.
  uint8_t *const nt_w = nt + i16 * kNRow + 16 * kq;
  const uint8_t *const nt_r = nt + ((i16 >> 2) & 1) * kNBlk + (4 * kq + (i16 & 3)) * kNRow + 8 * (i16 >> 3);
  // 4-bit codes: lane (token i16 of block k, kq) writes its 32 codes as bytes
  // at row i16 of block k, bytes 32 kq ..: chunk 2 kq + x (16 bytes) holds
  // the even and then the odd codes of code words 2x and 2x + 1, so byte p of
  // a chunk is channel 16 chunk + byte_chan(p).  A transposing 8-bit read
  // returns to lane i of a 16-lane group, as its byte e, byte i mod 8 of the
  // 8-byte piece lane 2e + i / 8 points at; lane j points at token
  // 4 kq + (e mod 4) of block e / 4 (e = j / 2), bytes 8 (j mod 2) of the
  // chunk.  So lane (column i16, kq) receives the codes of channel
  // 16 chunk + byte_chan(i16) for tokens 4 kq + e and 16 + 4 kq + e (e = 0..3,
  // the key-output token order), one chunk per read.
  uint8_t *const bt_w = nt + i16 * kBRow + 32 * kq;
  const uint8_t *const bt_r = nt + ((i16 >> 3) & 1) * kBBlk + (4 * kq + ((i16 >> 1) & 3)) * kBRow + 8 * (i16 & 1);

  // online-softmax state
  float m[kHpg], mthr[kHpg];
#pragma unroll
  for (int h = 0; h < kHpg; ++h) m[h] = mthr[h] = -INFINITY;
  float m_lane = -INFINITY, mthr_lane = -INFINITY;   // for head hk_lane
  float lsum = 0.0f;    // key-output lanes: weights of head hk_lane (own group slot only)
  float vbias = 0.0f;   // value-A lanes: zero-point term of (head hk_lane, slice i16 & 3)
  fx4 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = fx4{0.0f, 0.0f, 0.0f, 0.0f};

  // q' limbs of the current super-chunk, per pass p and word r
  uint32_t bhi[4][4], blo[4][4];
  float beta = 0.0f;

  const int64_t ngr_cap = cap / GS;
  const Rsrc rkc = rsrc_of(a.c.k_codes + (int64_t)unit * cap * W, (uint32_t)(cap * W * 4));
  const Rsrc rvc = rsrc_of(a.c.v_codes + (int64_t)unit * cap * W, (uint32_t)(cap * W * 4));
  const Rsrc rvs = rsrc_of(a.c.v_scale + (int64_t)unit * cap * VGR, (uint32_t)(cap * VGR * 4));
  const Rsrc rks = rsrc_of(a.c.k_scale + (int64_t)unit * ngr_cap * kHeadDim, (uint32_t)(ngr_cap * kHeadDim * 4));
  const Rsrc rvz = META ? rvs : rsrc_of(a.c.v_zero + (int64_t)unit * cap * VGR, (uint32_t)(cap * VGR * 2));
  const Rsrc rkz = META ? rks
                        : rsrc_of(a.c.k_zero + (int64_t)unit * ngr_cap * kHeadDim, (uint32_t)(ngr_cap * kHeadDim * 2));
  const uint32_t code_lane = (uint32_t)(i16 * W + WPL * kq) * 4u;
  // metadata entry of this lane within a step's block of EPS entries
  const uint32_t mflat = (uint32_t)(SPG == 4 ? (lane & 31) : lane * E);

  // key metadata of the super-chunk starting at group gfirst, in two or three
  // 16-byte loads per lane; entries of groups past the wave's range get an
  // out-of-range lane offset, so they read zero without touching memory
  auto load_kmeta = [&](GqaKMeta &km, uint32_t gfirst) {
    const bool kneed = gfirst + (uint32_t)(lane >> 4) < (uint32_t)ngroups;
    const uint32_t koff = gfirst * kHeadDim + 8u * (uint32_t)lane;
    const uint32_t so = kneed ? koff * 4 : kOutOfRange;
    km.s0 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rks, so, 0, kStream));
    km.s1 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rks, kneed ? so + 16 : kOutOfRange, 0, kStream));
    if constexpr (!META) {
      km.z = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rkz, kneed ? koff * 2 : kOutOfRange, 0, kStream));
    } else {
      km.z = make_uint4(0, 0, 0, 0);
    }
  };
  auto stage_kmeta = [&](const GqaKMeta &km) {
    const uint32_t sw[8] = {km.s0.x, km.s0.y, km.s0.z, km.s0.w, km.s1.x, km.s1.y, km.s1.z, km.s1.w};
    const uint32_t zw[4] = {km.z.x, km.z.y, km.z.z, km.z.w};
    float S[8], Z[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) decode_meta<META>(sw[e], (zw[e / 2] >> (16 * (e & 1))) & 0xffffu, S[e], Z[e]);
    const int km_at = (lane >> 4) * kKmRow + 8 * (lane & 15);   // group lane / 16, channels 8 (lane mod 16) ..
    *reinterpret_cast<float4 *>(kmS + km_at) = make_float4(S[0], S[1], S[2], S[3]);
    *reinterpret_cast<float4 *>(kmS + km_at + 4) = make_float4(S[4], S[5], S[6], S[7]);
    *reinterpret_cast<float4 *>(kmZ + km_at) = make_float4(Z[0], Z[1], Z[2], Z[3]);
    *reinterpret_cast<float4 *>(kmZ + km_at + 4) = make_float4(Z[4], Z[5], Z[6], Z[7]);
  };
  GqaKMeta kmr;   // key metadata of the next super-chunk, loaded at its predecessor's first step

  auto load = [&](Buf &bf, int s) {
    // key metadata of the next super-chunk with the loads of a super-chunk's
    // first step; staged into LDS, after the preparation, at the first step
    // (three steps loaded ahead) or the second (two ahead), before the load
    // of the next super-chunk's first step overwrites it
    if (s < nsteps && s % SPC == 0) {
      if (s > 0) {   // the load cursor enters the next super-chunk
        idL = idL1;
        idL1 = a.dynamic ? 2u * nw + (uint32_t)__builtin_amdgcn_readlane(pend, 0) : idL1 + nw;
        if (idL1 < (uint32_t)nsc) {
          if (a.dynamic) pend = grab();
        } else {
          nsteps = s + live_steps(idL);
        }
      }
      if (idL1 < (uint32_t)nsc) load_kmeta(kmr, 4u * idL1);
    }
    // past the end (never processed): out-of-range lane offsets, so the
    // ring's last loads read zero instead of fetching data again
    const bool live = s < nsteps;
    const uint32_t g = 4u * idL + (uint32_t)((s % SPC) >> LOG_SPG);
    const uint32_t t0 = live ? g * GS + (uint32_t)((s & (SPG - 1)) * 32) : 0u;
    const uint32_t cl = live ? code_lane : kOutOfRange;
    const uint32_t ml4 = live ? mflat * 4 : kOutOfRange, ml2 = live ? mflat * 2 : kOutOfRange;
    bload_words<WPL>(rkc, cl, t0 * (W * 4), bf.kw);
    bload_words<WPL>(rkc, cl, (t0 + 16) * (W * 4), bf.kw + WPL);
    bload_words<WPL>(rvc, cl, t0 * (W * 4), bf.vw);
    bload_words<WPL>(rvc, cl, (t0 + 16) * (W * 4), bf.vw + WPL);
    bload_words<E>(rvs, ml4, t0 * (VGR * 4), bf.vs);
    if constexpr (!META) {
      if constexpr (E == 2) {
        bf.vz = __builtin_amdgcn_raw_buffer_load_b32(rvz, ml2, t0 * (VGR * 2), kStream);
      } else {
        bf.vz = __builtin_amdgcn_raw_buffer_load_b16(rvz, ml2, t0 * (VGR * 2), kStream);
      }
    } else {
      bf.vz = 0;
    }
  };

  // stage one step's value metadata entries (raw words) into LDS as
  // [group][token] floats
  auto stage_vmeta = [&](const uint32_t *sw, uint32_t zw) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float S, Z;
      decode_meta<META>(sw[e], (zw >> (16 * e)) & 0xffffu, S, Z);
      const uint32_t f = mflat + e;
      const uint32_t idx = (f % VGR) * 32 + f / VGR;
      lvS[idx] = S;
      lvZ[idx] = Z;
    }
  };

  // q' limbs and bias of the super-chunk whose metadata is in kmS / kmZ
  auto prep = [&]() {
    const float *sS = kmS + (i16 & 3) * kKmRow + 32 * kq;
    const float *sZ = kmZ + (i16 & 3) * kKmRow + 32 * kq;
    const float *sq = qsm + hk_lane * kHeadDim + 32 * kq;
    float qp[32];
    float bp = 0.0f;
#pragma unroll
    for (int c = 0; c < 32; c += 4) {
      const float4 S4 = *reinterpret_cast<const float4 *>(sS + c);
      const float4 Z4 = *reinterpret_cast<const float4 *>(sZ + c);
      const float4 Q4 = *reinterpret_cast<const float4 *>(sq + c);
      qp[c] = Q4.x * S4.x;
      qp[c + 1] = Q4.y * S4.y;
      qp[c + 2] = Q4.z * S4.z;
      qp[c + 3] = Q4.w * S4.w;
      bp = fmaf(qp[c], Z4.x, bp);
      bp = fmaf(qp[c + 1], Z4.y, bp);
      bp = fmaf(qp[c + 2], Z4.z, bp);
      bp = fmaf(qp[c + 3], Z4.w, bp);
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
#pragma unroll
      for (int r = 0; r < 4; ++r) limbs(qp[8 * p + pass_chan(r, 0)], qp[8 * p + pass_chan(r, 1)], bhi[p][r], blo[p][r]);
    }
    bp += shfl_xor_f(bp, 16);
    bp += shfl_xor_f(bp, 32);
    beta = bp;
  };

  // raise the per-head maxima past the new scores (uniform branch)
  auto rescale = [&](float mx_valid) {
    float hm = block_max<4>(mx_valid);   // the quad of a head's group slots
    hm = fmaxf(hm, shfl_xor_f(hm, 16));
    hm = fmaxf(hm, shfl_xor_f(hm, 32));
    float f[kHpg];
#pragma unroll
    for (int h = 0; h < kHpg; ++h) {
      const float mn = fmaxf(m[h], lane_of(hm, 4 * h));
      f[h] = (mn == m[h]) ? 1.0f : fast_exp2(m[h] - mn);
      m[h] = uniform(mn);
      mthr[h] = uniform(mn + kMargin);
    }
    m_lane = sel4(hk_lane, m[0], m[1], m[2], m[3]);
    mthr_lane = sel4(hk_lane, mthr[0], mthr[1], mthr[2], mthr[3]);
    const float fk = sel4(hk_lane, f[0], f[1], f[2], f[3]);
    const float fv = sel4(kq, f[0], f[1], f[2], f[3]);
    lsum *= fk;
    vbias *= fk;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] *= fv;
  };

  auto process = [&](const Buf &bf, int s) {
    const int gq = (s >> LOG_SPG) & 3;   // group slot of this step in its super-chunk
    const int kk = s % SPC;
    if (kk == 0) prep();
    // key scores of both blocks; the high and low limb products accumulate
    // separately so four MFMA chains interleave
    fx4 sc[2], sl2[2];
    sc[0] = sc[1] = fx4{beta, beta, beta, beta};
    sl2[0] = sl2[1] = fx4{0.0f, 0.0f, 0.0f, 0.0f};
    static_for<4>([&](auto pc) {
      constexpr int p = decltype(pc)::value;
      using C = CodesBf16<BITS>;
      const u32x4 bh = {bhi[p][0], bhi[p][1], bhi[p][2], bhi[p][3]};
      const u32x4 bl = {blo[p][0], blo[p][1], blo[p][2], blo[p][3]};
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const uint32_t *w = bf.kw + k * WPL;
        const u32x4 ak = {C::template word<4 * p>(w), C::template word<4 * p + 1>(w), C::template word<4 * p + 2>(w),
                          C::template word<4 * p + 3>(w)};
        sc[k] = mma_x32(ak, bh, sc[k]);
        sl2[k] = mma_x32(ak, bl, sl2[k]);
      }
    });
    // staging while the key products run: metadata and the value tile
    wave_sync();
    // the next super-chunk's key metadata (loaded with the current one's first
    // step, LA steps ahead; its first step is at least SPC away)
    if (kk == (LA == 3 ? 0 : 1)) stage_kmeta(kmr);
    stage_vmeta(bf.vs, bf.vz);
    // value codes of both blocks into the tile: 4-bit fields (2-bit codes)
    // or bytes (4-bit codes)
    static_for<2>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      const uint32_t *w = bf.vw + k * WPL;
      if constexpr (BITS == 2) {
        *reinterpret_cast<uint4 *>(nt_w + k * kNBlk) =
            make_uint4(w[0] & 0x33333333u, (w[0] >> 2) & 0x33333333u, w[1] & 0x33333333u, (w[1] >> 2) & 0x33333333u);
      } else {
        *reinterpret_cast<uint4 *>(bt_w + k * kBBlk) =
            make_uint4(w[0] & 0x0F0F0F0Fu, (w[0] >> 4) & 0x0F0F0F0Fu, w[1] & 0x0F0F0F0Fu, (w[1] >> 4) & 0x0F0F0F0Fu);
        *reinterpret_cast<uint4 *>(bt_w + k * kBBlk + 16) =
            make_uint4(w[2] & 0x0F0F0F0Fu, (w[2] >> 4) & 0x0F0F0F0Fu, w[3] & 0x0F0F0F0Fu, (w[3] >> 4) & 0x0F0F0F0Fu);
      }
    });
    wave_sync();
    sc[0] += sl2[0];
    sc[1] += sl2[1];

    // softmax weights (valid in the lanes of this step's group slot)
    const bool valid = (i16 & 3) == gq;
    bool over = false;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
#pragma unroll
      for (int r = 0; r < 4; ++r) over |= sc[k][r] > mthr_lane;
    }
    if (__any(over && valid)) {
      float mx = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                       fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
      rescale(valid ? mx : -INFINITY);
    }
    float pw[8];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
#pragma unroll
      for (int r = 0; r < 4; ++r) pw[4 * k + r] = fast_exp2(sc[k][r] - m_lane);
    }
    const float psum = ((pw[0] + pw[1]) + (pw[2] + pw[3])) + ((pw[4] + pw[5]) + (pw[6] + pw[7]));
    lsum += valid ? psum : 0.0f;

    // value metadata of this lane's 8 tokens (value-A role)
    float sv[8], zv[8];
    {
      const int gcv = (i16 & 3) >> Gm::SH;
      const float *pS = lvS + gcv * 32 + 4 * kq;
      const float *pZ = lvZ + gcv * 32 + 4 * kq;
      const float4 s0 = *reinterpret_cast<const float4 *>(pS);
      const float4 s1 = *reinterpret_cast<const float4 *>(pS + 16);
      const float4 z0 = *reinterpret_cast<const float4 *>(pZ);
      const float4 z1 = *reinterpret_cast<const float4 *>(pZ + 16);
      sv[0] = s0.x; sv[1] = s0.y; sv[2] = s0.z; sv[3] = s0.w;
      sv[4] = s1.x; sv[5] = s1.y; sv[6] = s1.z; sv[7] = s1.w;
      zv[0] = z0.x; zv[1] = z0.y; zv[2] = z0.z; zv[3] = z0.w;
      zv[4] = z1.x; zv[5] = z1.y; zv[6] = z1.z; zv[7] = z1.w;
    }

    // weights of the step's group slot to every lane of the quad
    float pb[8];
    if (gq == 0) {
#pragma unroll
      for (int j = 0; j < 8; ++j) pb[j] = quad_bcast<0>(pw[j]);
    } else if (gq == 1) {
#pragma unroll
      for (int j = 0; j < 8; ++j) pb[j] = quad_bcast<1>(pw[j]);
    } else if (gq == 2) {
#pragma unroll
      for (int j = 0; j < 8; ++j) pb[j] = quad_bcast<2>(pw[j]);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) pb[j] = quad_bcast<3>(pw[j]);
    }
    u32x4 ahi, alo;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float w0 = pb[2 * q] * sv[2 * q], w1 = pb[2 * q + 1] * sv[2 * q + 1];
      vbias = fmaf(w0, zv[2 * q], vbias);
      vbias = fmaf(w1, zv[2 * q + 1], vbias);
      uint32_t h, l;
      limbs(w0, w1, h, l);
      ahi[q] = h;
      alo[q] = l;
    }

    // values: 16 channel positions at a time, transposed by the LDS reads
    if constexpr (BITS == 2) {
      // one 4-bit transposing read per pair of 16-channel chunks; fields 2q,
      // 2q + 1 of a word are the tokens of bf16 word q of the operand
      static_for<4>([&](auto uc) {
        constexpr int u = decltype(uc)::value;
        const i32x2 r = __builtin_amdgcn_ds_read_tr4_b64_v2i32((lds_i32x2 *)(nt_r + 16 * u));
        static_for<2>([&](auto xc) {
          constexpr int x = decltype(xc)::value, cb = 2 * u + x;
          const uint32_t f = (uint32_t)r[x];
          const u32x4 bv = {nib_bf16<0>(f), nib_bf16<1>(f), nib_bf16<2>(f), nib_bf16<3>(f)};
          acc[cb] = mma_x32(ahi, bv, acc[cb]);
          acc[cb] = mma_x32(alo, bv, acc[cb]);
        });
      });
    } else {
      // one 8-bit transposing read per 16-channel chunk; bytes 2q, 2q + 1 of
      // the pair of words are the tokens of bf16 word q of the operand
      static_for<8>([&](auto cc) {
        constexpr int cb = decltype(cc)::value;
        const i32x2 r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2 *)(bt_r + 16 * cb));
        const u32x4 bv = {byte_bf16<0>((uint32_t)r[0]), byte_bf16<1>((uint32_t)r[0]), byte_bf16<0>((uint32_t)r[1]),
                          byte_bf16<1>((uint32_t)r[1])};
        acc[cb] = mma_x32(ahi, bv, acc[cb]);
        acc[cb] = mma_x32(alo, bv, acc[cb]);
      });
    }
  };

  if (nsteps > 0) {
    // metadata of the first super-chunk
    {
      GqaKMeta km0;
      load_kmeta(km0, 4u * idL);
      stage_kmeta(km0);
    }
    if constexpr (LA == 3) {
      Buf A, B, C, D;
      asm volatile("" ::: "memory");
      load(A, 0);
      asm volatile("" ::: "memory");
      load(B, 1);
      asm volatile("" ::: "memory");
      load(C, 2);
      asm volatile("" ::: "memory");
      wave_sync();
      for (int s = 0; s < nsteps; s += 4) {
        load(D, s + 3);
        process(A, s);
        load(A, s + 4);
        if (s + 1 < nsteps) process(B, s + 1);
        load(B, s + 5);
        if (s + 2 < nsteps) process(C, s + 2);
        load(C, s + 6);
        if (s + 3 < nsteps) process(D, s + 3);
      }
    } else {
      Buf A, B, C;
      asm volatile("" ::: "memory");
      load(A, 0);
      asm volatile("" ::: "memory");
      load(B, 1);
      asm volatile("" ::: "memory");
      wave_sync();
      for (int s = 0; s < nsteps; s += 3) {
        load(C, s + 2);
        process(A, s);
        load(A, s + 3);
        if (s + 1 < nsteps) process(B, s + 1);
        load(B, s + 4);
        if (s + 2 < nsteps) process(C, s + 2);
      }
    }
  }
  // every grab of this wave has been read: the super-chunks it took
  if (lane == 0) s_took[wave] = (uint32_t)((nsteps + SPC - 1) / SPC);

  // ---- combine: per-wave rows [h][128] in LDS, then across waves
  float L = block_sum<4>(lsum);
  L += shfl_xor_f(L, 16);
  L += shfl_xor_f(L, 32);            // weight sum of head hk_lane
  float vb = vbias + shfl_xor_f(vbias, 16);
  vb += shfl_xor_f(vb, 32);          // bias of (head hk_lane, slice i16 & 3)
  float vbs[4];                      // bias of (head kq, slice s)
#pragma unroll
  for (int sl = 0; sl < 4; ++sl) vbs[sl] = __shfl(vb, 4 * kq + sl);
  __syncthreads();                   // every wave is done with its staging area
  float *rows = smem;                // [kGqaWaves][kHpg][128]
  float *wml = smem + Gm::ROWS;      // [kGqaWaves][kHpg][2]
  {
    // column i16 of block cb holds tile position 16 cb + i16, i.e. channel
    // 32 (cb / 2) + 8 p + pass_chan(r, e) with 16 (cb mod 2) + i16 = 8 p + 2 r + e;
    // its 32-channel slice is cb / 2, the accumulator row to keep
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) {
      const int ch = 16 * cb + (BITS == 2 ? nib_chan(i16) : byte_chan(i16));
      rows[(wave * kHpg + kq) * kHeadDim + ch] = acc[cb][cb >> 1] + vbs[cb >> 1];
    }
  }
  if (lane < kHpg) {
    const float mh = sel4(lane, m[0], m[1], m[2], m[3]);
    wml[(wave * kHpg + lane) * 2] = mh;
  }
  if (kq == 0 && (i16 & 3) == 0) wml[(wave * kHpg + hk_lane) * 2 + 1] = L;
  __syncthreads();
  static_assert((kHpg * kHeadDim) % kGqaThreads == 0, "whole merge passes");
  for (int i = tid; i < kHpg * kHeadDim; i += kGqaThreads) {
    const int h = i / kHeadDim, c = i % kHeadDim;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kGqaWaves; ++w) M = fmaxf(M, wml[(w * kHpg + h) * 2]);
    float accv = 0.0f, Lt = 0.0f;
#pragma unroll
    for (int w = 0; w < kGqaWaves; ++w) {
      const float mw = wml[(w * kHpg + h) * 2];
      const float f = (mw == -INFINITY) ? 0.0f : fast_exp2(mw - M);
      Lt = fmaf(f, wml[(w * kHpg + h) * 2 + 1], Lt);
      accv = fmaf(f, rows[(w * kHpg + h) * kHeadDim + c], accv);
    }
    st.acc[h * kHeadDim + c] = accv;
    if (c == 0) {
      st.ml[2 * h] = M;
      st.ml[2 * h + 1] = Lt;
    }
  }
  __syncthreads();

  // this split's share of the unit's fp16 tokens (sinks, then [n_main, n)),
  // merged into the part's result
  const int nrest = a.nsink + (int)(a.n - a.n_main);
  if (split == 0 && a.k_new != nullptr && tid < 2 * (kHeadDim * 2 / 16)) {
    // fused step: the new token goes into its ring slot (the shares read it from k_new / v_new)
    constexpr int CH = kHeadDim * 2 / 16;
    const int which = tid / CH, ch = tid % CH;
    const uint4 *src = reinterpret_cast<const uint4 *>((which ? a.v_new : a.k_new) + (int64_t)unit * kHeadDim);
    uint4 *dst = reinterpret_cast<uint4 *>((which ? a.c.v_resid : a.c.k_resid) +
                                           ((int64_t)unit * a.c.residual + (a.n - 1) % a.c.residual) * kHeadDim);
    dst[ch] = src[ch];
  }
  // The shares go to the leading a.early splits, whose workgroups all
  // dispatch in the first round: they end a few microseconds before the
  // second round's, which then no longer wait for the shares (3.6% off a
  // fused decode step on the 2-bit GQA workload).
  const int ib = split < a.early ? (int)((int64_t)nrest * split / a.early) : 0;
  const int ie = split < a.early ? (int)((int64_t)nrest * (split + 1) / a.early) : 0;
  if (ie > ib) {
    float *acc2 = st.acc + Gm::STAGE2;   // [kHpg][128], then (max, sum)[kHpg]
    float *ml2 = acc2 + kHpg * kHeadDim;
    gqa_fp16_part<BITS, GS, META>(a, unit, smem, qsm, acc2, ml2, ib, ie);
    float f1[kHpg], f2[kHpg], mn[kHpg];
#pragma unroll
    for (int h = 0; h < kHpg; ++h) {
      const float M = st.ml[2 * h], m2 = ml2[2 * h];
      mn[h] = fmaxf(M, m2);
      f1[h] = M == -INFINITY ? 0.0f : fast_exp2(M - mn[h]);
      f2[h] = m2 == -INFINITY ? 0.0f : fast_exp2(m2 - mn[h]);
    }
    for (int idx = tid; idx < kHpg * kHeadDim; idx += kGqaThreads) {
      const int h = idx / kHeadDim;
      st.acc[idx] = st.acc[idx] * f1[h] + acc2[idx] * f2[h];
    }
    __syncthreads();
    if (tid < kHpg) {
      const int h = tid;
      const float L = st.ml[2 * h + 1] * f1[h] + ml2[2 * h + 1] * f2[h];
      st.ml[2 * h] = mn[h];
      st.ml[2 * h + 1] = L;
    }
    __syncthreads();
  }
  if (a.prequant >= 0 && split == a.splits - 1 && wave == 0) {
    // a full FIFO queue: its oldest value row is quantized now, ahead of the
    // next append's pop
    const int R = a.c.residual;
    quantize_value_row<BITS, GS>(a.c, a.c.v_resid + ((int64_t)unit * R + a.prequant % R) * kHeadDim,
                                 (int64_t)unit * cap + a.prequant);
  }
  queue_finish<kHpg, kGqaWaves>(a, unit, split, st, s_took, (uint32_t)nsc);
}

template <int BITS, int GS, int META>
hipError_t launch_gqa(const AttnArgs &a, int splits, hipStream_t s) {
  const int units = a.batch * a.hkv;
  hipLaunchKernelGGL((gqa_mfma_kernel<BITS, GS, META>), dim3(units * splits), dim3(kGqaThreads), 0, s, a);
  return hipGetLastError();
}

template <int BITS, int META>
hipError_t launch_gqa_by_group(const AttnArgs &a, int splits, hipStream_t s) {
  switch (a.c.group) {
    case 32: return launch_gqa<BITS, 32, META>(a, splits, s);
    case 64: return launch_gqa<BITS, 64, META>(a, splits, s);
    case 128: return launch_gqa<BITS, 128, META>(a, splits, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_gqa_mfma(const AttnArgs &a, hipStream_t s) {
  if (a.hq != kHpg * a.hkv) return hipErrorInvalidValue;
  const int splits = a.splits;
  if (a.c.meta)
    return (a.c.bits == 2) ? launch_gqa_by_group<2, 1>(a, splits, s) : launch_gqa_by_group<4, 1>(a, splits, s);
  return (a.c.bits == 2) ? launch_gqa_by_group<2, 0>(a, splits, s) : launch_gqa_by_group<4, 0>(a, splits, s);
}

}  // namespace kvq
