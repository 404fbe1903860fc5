// Host-side check of the C ABI (decode_attention_token_amd/csrc/kvq_api.cpp),
// built with g++ under AddressSanitizer and UndefinedBehaviorSanitizer and
// linked against this file instead of the HIP kernels.
//
// Every kvq::launch_* entry point is replaced by a stub that launches
// nothing: it checks, from the launch arguments and the indexing of the
// kernel it stands for, that every element the kernel would read or write
// lies inside the buffer the caller sized with kvq_layout_bytes (or the
// prompt, new-token, query, output and workspace buffers), that the
// kernel's 32-bit offsets cannot wrap, and that the fp16 tokens an
// attention launch reads from the residual ring are still live there.
// Buffers are fake address ranges registered by size (nothing is ever
// dereferenced), so the sweep reaches max_tokens = 2^25.
//
// The main program runs (1) the validation paths of every entry point, checking
// the status, that kvq_last_error explains it and that the cache struct is
// left unchanged, and (2) seeded sequences of prefill, append, attention and
// decode steps over a sweep of the supported shapes: bits, group size,
// query heads per kv head, both value policies, both metadata formats, the
// InnerQ scheme with and without key scales, residual lengths up to 512,
// sink counts up to 512 and capacities up to 2^25 tokens.  It also checks
// that a decode step in steady state is a single launch.
//
// Exit status 0 when every check passes; a failed check prints its reason
// and aborts.
#include <cinttypes>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "kvq.h"
#include "kvq_internal.h"

// ---------------------------------------------------------------- registry
namespace {

struct Region {
  uintptr_t base;
  size_t size;
  const char *name;
};
std::vector<Region> g_regions;
uintptr_t g_next = (uintptr_t)1 << 44;   // fake device addresses, never dereferenced
int g_launches = 0;
const char *g_context = "";
const char *g_shrink = nullptr;   // name of a buffer registered 16 bytes short (a planted mistake)

[[noreturn]] void die(const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  fprintf(stderr, "CHECK FAILED (%s): ", g_context);
  vfprintf(stderr, fmt, ap);
  fprintf(stderr, "\n");
  va_end(ap);
  abort();
}

void *fake_alloc(size_t size, const char *name) {
  if (size == 0) return nullptr;
  if (g_shrink && strcmp(g_shrink, name) == 0 && size > 16) size -= 16;
  const uintptr_t base = g_next;
  g_next += (size + ((uintptr_t)1 << 24) + 4095) & ~(uintptr_t)4095;   // a gap after every region
  g_regions.push_back({base, size, name});
  return reinterpret_cast<void *>(base);
}

void reset_regions() {
  g_regions.clear();
  g_next = (uintptr_t)1 << 44;
}

// Bytes [first, end) past p must lie inside one registered region.
void need(const void *p, int64_t first, int64_t end, const char *what) {
  if (end <= first) return;   // nothing accessed
  if (p == nullptr) die("%s: null pointer for bytes [%" PRId64 ", %" PRId64 ")", what, first, end);
  if (first < 0) die("%s: negative offset %" PRId64, what, first);
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  for (const Region &r : g_regions) {
    if (a >= r.base && a < r.base + r.size) {
      const uint64_t off = a - r.base;
      if (off + (uint64_t)end > r.size)
        die("%s: bytes [%" PRId64 ", %" PRId64 ") at offset %" PRIu64 " overrun %s (%zu bytes)", what, first, end,
            off, r.name, r.size);
      return;
    }
  }
  die("%s: pointer outside every buffer", what);
}

void expect(bool ok, const char *fmt, ...) {
  if (ok) return;
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  die("%s", buf);
}

int words_per_row(const kvq::CacheView &c) { return kvq::kHeadDim * c.bits / 32; }

// Writes of quantized key groups [g0, g0 + ng) of every unit (KIVI layout).
void need_key_groups(const kvq::CacheView &c, int units, int64_t g0, int64_t ng, const char *what) {
  const int G = c.group, W = words_per_row(c);
  const int64_t ngc = c.cap / G;
  expect(g0 >= 0 && (g0 + ng) * G <= c.cap, "%s: key groups [%" PRId64 ", +%" PRId64 ") past capacity", what, g0, ng);
  need(c.k_codes, g0 * G * W * 4, ((int64_t)(units - 1) * c.cap + (g0 + ng) * G) * W * 4, what);
  need(c.k_scale, g0 * kvq::kHeadDim * 4, ((int64_t)(units - 1) * ngc + g0 + ng) * kvq::kHeadDim * 4, what);
  if (!c.meta) need(c.k_zero, g0 * kvq::kHeadDim * 2, ((int64_t)(units - 1) * ngc + g0 + ng) * kvq::kHeadDim * 2, what);
}

// Quantized rows [r0, r0 + count) of every unit, per-token metadata (KIVI
// values; InnerQ keys and values).
void need_rows(const kvq::CacheView &c, bool values, int units, int64_t r0, int64_t count, const char *what) {
  const int W = words_per_row(c), NG = kvq::kHeadDim / c.group;
  expect(r0 >= 0 && r0 + count <= c.cap, "%s: rows [%" PRId64 ", +%" PRId64 ") past capacity", what, r0, count);
  const int64_t last = (int64_t)(units - 1) * c.cap + r0 + count;
  need(values ? c.v_codes : c.k_codes, r0 * W * 4, last * W * 4, what);
  need(values ? c.v_scale : c.k_scale, r0 * NG * 4, last * NG * 4, what);
  if (!c.meta) need(values ? c.v_zero : c.k_zero, r0 * NG * 2, last * NG * 2, what);
}

// fp16 rows [r0, r0 + count) of a [units][rows][128] tensor.
void need_fp16(const void *p, int units, int64_t rows, int64_t r0, int64_t count, const char *what) {
  expect(r0 >= 0 && r0 + count <= rows, "%s: rows [%" PRId64 ", +%" PRId64 ") outside %" PRId64, what, r0, count,
         rows);
  need(p, r0 * 256, ((int64_t)(units - 1) * rows + r0 + count) * 256, what);
}

// 32-bit buffer-resource sizes and offsets the kernels build per unit.
void check_resources(const kvq::CacheView &c) {
  const uint64_t code_bytes = (uint64_t)c.cap * words_per_row(c) * 4;
  expect(code_bytes <= 0x80000000ull, "code resource of %" PRIu64 " bytes", code_bytes);
  expect((uint64_t)c.cap * kvq::kHeadDim * 4 / c.group < 0x100000000ull, "key metadata resource");
}

}  // namespace

extern "C" const char *hipGetErrorString(hipError_t) { return "stubbed launch"; }
extern "C" hipError_t hipGetDevice(int *dev) {
  *dev = 0;
  return hipSuccess;
}
extern "C" hipError_t hipDeviceGetAttribute(int *value, hipDeviceAttribute_t attr, int) {
  *value = attr == hipDeviceAttributeMultiprocessorCount ? 256 : 0;
  return hipSuccess;
}

// ---------------------------------------------------------------- stubs
namespace kvq {

hipError_t launch_quantize_keys(const CacheView &c, int units, const uint16_t *src, int64_t src_rows,
                                int64_t src_row0, int ngroups, int64_t dst_group0, hipStream_t) {
  if (ngroups <= 0 || units <= 0) return hipSuccess;
  ++g_launches;
  expect((int64_t)units * ngroups <= INT32_MAX - 4, "key quantizer grid");
  need_fp16(src, units, src_rows, src_row0, (int64_t)ngroups * c.group, "quantize keys: source");
  need_key_groups(c, units, dst_group0, ngroups, "quantize keys: cache");
  return hipSuccess;
}

hipError_t launch_quantize_values(const CacheView &c, int units, const uint16_t *src, int64_t src_rows,
                                  int64_t src_row0, int count, int64_t dst_row0, hipStream_t) {
  if (count <= 0 || units <= 0) return hipSuccess;
  ++g_launches;
  expect((int64_t)units * count <= INT32_MAX - 256, "value quantizer grid");
  need_fp16(src, units, src_rows, src_row0, count, "quantize values: source");
  need_rows(c, true, units, dst_row0, count, "quantize values: cache");
  return hipSuccess;
}

hipError_t launch_quantize_kv(const CacheView &c, int units, const uint16_t *ksrc, const uint16_t *vsrc,
                              int64_t src_rows, int64_t src_row0, int ngroups, int count, hipStream_t) {
  if (units <= 0 || (ngroups <= 0 && count <= 0)) return hipSuccess;
  ++g_launches;
  const int64_t kblocks = ngroups > 0 ? ((int64_t)units * ngroups + 3) / 4 : 0;
  const int64_t vblocks = count > 0 ? ((int64_t)units * count + 127) / 128 : 0;
  expect((int64_t)units * (ngroups > 0 ? ngroups : 0) <= INT32_MAX - 4, "prefill key grid");
  expect((int64_t)units * (count > 0 ? count : 0) <= INT32_MAX - 256, "prefill value grid");
  expect(kblocks + vblocks <= INT32_MAX, "prefill grid");
  if (ngroups > 0) {
    need_fp16(ksrc, units, src_rows, src_row0, (int64_t)ngroups * c.group, "prefill keys: source");
    need_key_groups(c, units, 0, ngroups, "prefill keys: cache");
  }
  if (count > 0) {
    need_fp16(vsrc, units, src_rows, src_row0, count, "prefill values: source");
    need_rows(c, true, units, 0, count, "prefill values: cache");
  }
  return hipSuccess;
}

hipError_t launch_flush(const CacheView &c, int units, const uint16_t *k_new, const uint16_t *v_new, int slot,
                        int64_t dst_group0, int64_t dst_row0, hipStream_t) {
  if (units <= 0) return hipSuccess;
  ++g_launches;
  const int R = c.residual;
  expect(slot >= 0 && slot < R, "flush: slot %d", slot);
  need_fp16(c.k_resid, units, R, 0, R, "flush: key ring");
  need_fp16(c.v_resid, units, R, 0, R, "flush: value ring");
  need_fp16(k_new, units, 1, 0, 1, "flush: k_new");
  need_fp16(v_new, units, 1, 0, 1, "flush: v_new");
  need_key_groups(c, units, dst_group0, R / c.group, "flush: keys");
  need_rows(c, true, units, dst_row0, R, "flush: values");
  return hipSuccess;
}

hipError_t launch_copy_rows(uint16_t *kdst, uint16_t *vdst, int dst_rows, const uint16_t *ksrc, const uint16_t *vsrc,
                            int64_t src_rows, int64_t row0, int count, int slot0, int units, hipStream_t) {
  if (count <= 0 || units <= 0) return hipSuccess;
  if (kdst == nullptr && vdst == nullptr) return hipSuccess;
  ++g_launches;
  expect(count <= dst_rows && slot0 >= 0, "copy rows: %d rows into %d slots from slot %d", count, dst_rows, slot0);
  if (kdst) {
    need_fp16(ksrc, units, src_rows, row0, count, "copy rows: key source");
    need_fp16(kdst, units, dst_rows, 0, dst_rows, "copy rows: key destination");
  }
  if (vdst) {
    need_fp16(vsrc, units, src_rows, row0, count, "copy rows: value source");
    need_fp16(vdst, units, dst_rows, 0, dst_rows, "copy rows: value destination");
  }
  return hipSuccess;
}

hipError_t launch_copy_to_residual(const CacheView &c, int units, const uint16_t *ksrc, const uint16_t *vsrc,
                                   int64_t src_rows, int64_t row0, int count, int slot0, bool keys, bool values,
                                   hipStream_t s) {
  return launch_copy_rows(keys ? c.k_resid : nullptr, values ? c.v_resid : nullptr, c.residual, ksrc, vsrc, src_rows,
                          row0, count, slot0, units, s);
}

hipError_t launch_innerq_quantize(const CacheView &c, int units, const uint16_t *ksrc, const uint16_t *vsrc,
                                  int64_t src_rows, int64_t src_row0, int count, int64_t dst_row0, hipStream_t) {
  if (count <= 0 || units <= 0) return hipSuccess;
  ++g_launches;
  expect((int64_t)units * count <= INT32_MAX / 2, "InnerQ quantizer grid");
  need_fp16(ksrc, units, src_rows, src_row0, count, "InnerQ quantize: keys");
  need_fp16(vsrc, units, src_rows, src_row0, count, "InnerQ quantize: values");
  need_rows(c, false, units, dst_row0, count, "InnerQ quantize: key rows");
  need_rows(c, true, units, dst_row0, count, "InnerQ quantize: value rows");
  if (c.k_norm) need(c.k_norm, 0, (int64_t)units * kHeadDim * 4, "InnerQ quantize: key scales");
  return hipSuccess;
}

hipError_t launch_key_norm(float *norm, int units, const uint16_t *k, int64_t len, hipStream_t) {
  ++g_launches;
  need(norm, 0, (int64_t)units * kHeadDim * 4, "key scales");
  if (len > 0) {
    ++g_launches;
    need_fp16(k, units, len, 0, len, "key scales: prompt");
  }
  return hipSuccess;
}

hipError_t launch_innerq_append(const CacheView &c, int units, const uint16_t *k_new, const uint16_t *v_new,
                                int64_t pop_row, bool to_sink, int slot, hipStream_t) {
  ++g_launches;
  const int R = c.residual;
  if (pop_row >= 0) {
    need_fp16(c.k_resid, units, R, pop_row % R, 1, "InnerQ append: leaving key");
    need_fp16(c.v_resid, units, R, pop_row % R, 1, "InnerQ append: leaving value");
    need_rows(c, false, units, pop_row, 1, "InnerQ append: key row");
    need_rows(c, true, units, pop_row, 1, "InnerQ append: value row");
    if (c.k_norm) need(c.k_norm, 0, (int64_t)units * kHeadDim * 4, "InnerQ append: key scales");
  }
  if (k_new != nullptr) {
    need_fp16(k_new, units, 1, 0, 1, "InnerQ append: k_new");
    need_fp16(v_new, units, 1, 0, 1, "InnerQ append: v_new");
    if (to_sink) {
      need_fp16(c.k_sink, units, c.sinks, slot, 1, "InnerQ append: key sink");
      need_fp16(c.v_sink, units, c.sinks, slot, 1, "InnerQ append: value sink");
    } else {
      need_fp16(c.k_resid, units, R, slot, 1, "InnerQ append: key slot");
      need_fp16(c.v_resid, units, R, slot, 1, "InnerQ append: value slot");
    }
  }
  return hipSuccess;
}

namespace {

// Query, output, workspace and fused-token buffers of an attention launch.
void need_io(const AttnArgs &a) {
  const int units = a.batch * a.hkv;
  expect(a.splits >= 1 && a.splits <= kMaxSplits && a.nparts == a.splits, "splits %d, parts %d", a.splits, a.nparts);
  expect((int64_t)units * a.splits <= INT32_MAX, "attention grid");
  need(a.q, 0, (int64_t)a.batch * a.hq * kHeadDim * 2, "attention: q");
  need(a.out, 0, (int64_t)a.batch * a.hq * kHeadDim * 4, "attention: out");
  need(a.ctr, 0, (int64_t)units * kCtrWords * 4, "attention: counters");
  need(a.partials, 0, (int64_t)a.batch * a.hq * a.nparts * kPartialStride * 4, "attention: partial records");
  expect(a.epoch != 0, "launch epoch 0");
  if (a.k_new) {
    need_fp16(a.k_new, units, 1, 0, 1, "attention: k_new");
    need_fp16(a.v_new, units, 1, 0, 1, "attention: v_new");
  }
}

}  // namespace

hipError_t launch_decode_attention(const AttnArgs &a, hipStream_t) {
  ++g_launches;
  const CacheView &c = a.c;
  const int units = a.batch * a.hkv, G = c.group, R = c.residual;
  check_resources(c);
  need_io(a);
  // counters (relative to the sink tokens) and the whole groups
  expect(a.n_main % G == 0 && a.n_main >= 0 && a.n_main <= a.nq_k && a.n_main <= a.nq_v,
         "n_main %" PRId64 " against nq_k %" PRId64 ", nq_v %" PRId64, a.n_main, a.nq_k, a.nq_v);
  expect(a.nq_k <= a.n && a.nq_v <= a.n && a.nq_k % G == 0, "counters n %" PRId64 " nq_k %" PRId64 " nq_v %" PRId64,
         a.n, a.nq_k, a.nq_v);
  expect(a.n + a.nsink <= c.cap && a.nsink <= c.sinks, "n %" PRId64 " + sinks %d past capacity", a.n, a.nsink);
  // the fp16 tokens of [nq, n) must all still be in the ring
  expect(a.n - a.nq_k <= R && a.n - a.nq_v <= R, "ring holds at most %d tokens", R);
  if (a.n_main > 0) need_key_groups(c, units, 0, a.n_main / G, "attention: key groups");
  const int64_t nk = a.nq_k > a.n_main ? a.nq_k : a.n_main, nv = a.nq_v > a.n_main ? a.nq_v : a.n_main;
  if (nk > 0) need_key_groups(c, units, 0, nk / G, "attention: quantized keys");
  if (nv > 0) need_rows(c, true, units, 0, nv, "attention: quantized values");
  if (a.n > a.nq_k || a.n > a.nq_v) {
    need_fp16(c.k_resid, units, R, 0, R, "attention: key ring");
    need_fp16(c.v_resid, units, R, 0, R, "attention: value ring");
  }
  if (a.nsink > 0) {
    need_fp16(c.k_sink, units, c.sinks, 0, a.nsink, "attention: key sinks");
    need_fp16(c.v_sink, units, c.sinks, 0, a.nsink, "attention: value sinks");
  }
  expect(a.k_new == nullptr || a.n > a.nq_k, "fused token must be an fp16 token");
  expect(a.early >= 1 && a.early <= a.splits, "early splits %d of %d", a.early, a.splits);
  if (a.prequant >= 0) {
    // its value is in the ring, not the fused token's slot, and not yet quantized
    expect(a.prequant >= a.nq_v && a.prequant < a.n - 1 && a.n - a.prequant == R,
           "quantize-ahead token %" PRId64 " (n %" PRId64 ", nq_v %" PRId64 ")", a.prequant, a.n, a.nq_v);
    need_rows(c, true, units, a.prequant, 1, "attention: quantize-ahead row");
  }
  return hipSuccess;
}

hipError_t launch_innerq_attention(const AttnArgs &a, hipStream_t) {
  ++g_launches;
  const CacheView &c = a.c;
  const int units = a.batch * a.hkv, R = c.residual;
  check_resources(c);
  need_io(a);
  const int64_t nsink = a.n < c.sinks ? a.n : c.sinks;
  expect(a.nq_k == a.nq_v && a.nq_k >= nsink && a.nq_k <= a.n && a.n <= c.cap,
         "counters n %" PRId64 " nq %" PRId64, a.n, a.nq_k);
  expect(a.n - a.nq_k <= R, "window holds at most %d tokens", R);
  if (a.nq_k > nsink) {
    need_rows(c, false, units, 0, a.nq_k, "InnerQ attention: key rows");
    need_rows(c, true, units, 0, a.nq_k, "InnerQ attention: value rows");
  }
  if (nsink > 0) {
    need_fp16(c.k_sink, units, c.sinks, 0, nsink, "InnerQ attention: key sinks");
    need_fp16(c.v_sink, units, c.sinks, 0, nsink, "InnerQ attention: value sinks");
  }
  if (a.n > a.nq_k) {
    need_fp16(c.k_resid, units, R, 0, R, "InnerQ attention: key window");
    need_fp16(c.v_resid, units, R, 0, R, "InnerQ attention: value window");
  }
  if (c.k_norm) need(c.k_norm, 0, (int64_t)units * kHeadDim * 4, "InnerQ attention: key scales");
  if (a.prequant >= 0) {
    expect(a.prequant == a.nq_k && a.prequant < a.n - 1 && a.n - a.prequant == R,
           "quantize-ahead token %" PRId64 " (n %" PRId64 ", nq %" PRId64 ")", a.prequant, a.n, a.nq_k);
    need_rows(c, false, units, a.prequant, 1, "InnerQ attention: quantize-ahead key row");
    need_rows(c, true, units, a.prequant, 1, "InnerQ attention: quantize-ahead value row");
  }
  return hipSuccess;
}

hipError_t launch_stream_read(const void *buf, size_t bytes, uint32_t *out, hipStream_t) {
  ++g_launches;
  need(buf, 0, (int64_t)bytes, "stream probe: buffer");
  need(out, 0, 4, "stream probe: out");
  return hipSuccess;
}

}  // namespace kvq

// ---------------------------------------------------------------- main program
namespace {

struct Setup {
  kvq_config cfg;
  kvq_cache cache;
  uint16_t *k, *v, *kn, *vn, *q;
  float *out;
  void *ws;
  size_t ws_bytes;
  int64_t prompt_rows;
};

void alloc_cache(Setup &s, int64_t prompt_rows) {
  reset_regions();
  kvq_layout L;
  expect(kvq_layout_bytes(&s.cfg, &L) == KVQ_OK, "layout: %s", kvq_last_error());
  memset(&s.cache, 0, sizeof(s.cache));
  s.cache.k_codes = (uint32_t *)fake_alloc(L.k_codes, "k_codes");
  s.cache.k_scale = (float *)fake_alloc(L.k_scale, "k_scale");
  s.cache.k_zero = (int16_t *)fake_alloc(L.k_zero, "k_zero");
  s.cache.v_codes = (uint32_t *)fake_alloc(L.v_codes, "v_codes");
  s.cache.v_scale = (float *)fake_alloc(L.v_scale, "v_scale");
  s.cache.v_zero = (int16_t *)fake_alloc(L.v_zero, "v_zero");
  s.cache.k_resid = (uint16_t *)fake_alloc(L.k_resid, "k_resid");
  s.cache.v_resid = (uint16_t *)fake_alloc(L.v_resid, "v_resid");
  s.cache.k_sink = (uint16_t *)fake_alloc(L.k_sink, "k_sink");
  s.cache.v_sink = (uint16_t *)fake_alloc(L.v_sink, "v_sink");
  s.cache.k_norm = (float *)fake_alloc(L.k_norm, "k_norm");
  const int64_t units = (int64_t)s.cfg.batch * s.cfg.num_kv_heads;
  s.prompt_rows = prompt_rows;
  s.k = (uint16_t *)fake_alloc((size_t)(units * prompt_rows * 256), "prompt keys");
  s.v = (uint16_t *)fake_alloc((size_t)(units * prompt_rows * 256), "prompt values");
  s.kn = (uint16_t *)fake_alloc((size_t)(units * 256), "k_new");
  s.vn = (uint16_t *)fake_alloc((size_t)(units * 256), "v_new");
  s.q = (uint16_t *)fake_alloc((size_t)s.cfg.batch * s.cfg.num_q_heads * 256, "q");
  s.out = (float *)fake_alloc((size_t)s.cfg.batch * s.cfg.num_q_heads * 512, "out");
  s.ws_bytes = kvq_workspace_bytes(&s.cfg, s.cfg.max_tokens, 0);
  for (int sp : {1, 7, kvq::kMaxSplits}) {
    const size_t b = kvq_workspace_bytes(&s.cfg, s.cfg.max_tokens, sp);
    if (b > s.ws_bytes) s.ws_bytes = b;
  }
  s.ws = fake_alloc(s.ws_bytes, "workspace");
}

kvq_config base_config() {
  kvq_config c;
  memset(&c, 0, sizeof(c));
  c.bits = 2;
  c.group = 32;
  c.residual = 128;
  c.batch = 2;
  c.num_q_heads = 4;
  c.num_kv_heads = 2;
  c.head_dim = 128;
  c.max_tokens = 1024;
  return c;
}

// ---- (1) validation paths
void expect_status(kvq_status got, kvq_status want, const kvq_cache *before, const kvq_cache *after,
                   const char *what) {
  expect(got == want, "%s: status %d, expected %d (%s)", what, (int)got, (int)want, kvq_last_error());
  expect(kvq_last_error()[0] != 0, "%s: no error text", what);
  if (before) expect(memcmp(before, after, sizeof(kvq_cache)) == 0, "%s: cache changed on failure", what);
}

void validation_cases() {
  g_context = "validation";
  kvq_layout L;
  expect_status(kvq_layout_bytes(nullptr, &L), KVQ_ERR_ARG, nullptr, nullptr, "null config");
  struct Bad {
    const char *what;
    void (*edit)(kvq_config &);
    kvq_status want;
  };
  const Bad bad[] = {
      {"bits 3", [](kvq_config &c) { c.bits = 3; }, KVQ_ERR_ARG},
      {"group 0", [](kvq_config &c) { c.group = 0; }, KVQ_ERR_ARG},
      {"group 16", [](kvq_config &c) { c.group = 16; }, KVQ_ERR_UNSUPPORTED},
      {"group 96", [](kvq_config &c) { c.group = 96; c.residual = 96; c.max_tokens = 960; c.head_dim = 96; }, KVQ_ERR_UNSUPPORTED},
      {"residual not a multiple", [](kvq_config &c) { c.residual = 100; }, KVQ_ERR_ARG},
      {"residual 0", [](kvq_config &c) { c.residual = 0; }, KVQ_ERR_ARG},
      {"residual 1024", [](kvq_config &c) { c.residual = 1024; c.max_tokens = 2048; }, KVQ_ERR_UNSUPPORTED},
      {"head_dim 64", [](kvq_config &c) { c.head_dim = 64; }, KVQ_ERR_UNSUPPORTED},
      {"3 query heads per kv head", [](kvq_config &c) { c.num_q_heads = 6; }, KVQ_ERR_UNSUPPORTED},
      {"heads not a multiple", [](kvq_config &c) { c.num_q_heads = 5; }, KVQ_ERR_ARG},
      {"batch 0", [](kvq_config &c) { c.batch = 0; }, KVQ_ERR_ARG},
      {"max_tokens 0", [](kvq_config &c) { c.max_tokens = 0; }, KVQ_ERR_ARG},
      {"max_tokens not a multiple of R", [](kvq_config &c) { c.max_tokens = 1000; }, KVQ_ERR_ARG},
      {"max_tokens 2^26", [](kvq_config &c) { c.max_tokens = 1 << 26; }, KVQ_ERR_UNSUPPORTED},
      {"sinks 513", [](kvq_config &c) { c.sink_tokens = 513; }, KVQ_ERR_UNSUPPORTED},
      {"sinks -1", [](kvq_config &c) { c.sink_tokens = -1; }, KVQ_ERR_ARG},
      {"v_policy 2", [](kvq_config &c) { c.v_policy = (kvq_v_policy)2; }, KVQ_ERR_ARG},
      {"scheme 2", [](kvq_config &c) { c.scheme = (kvq_scheme)2; }, KVQ_ERR_ARG},
      {"meta 2", [](kvq_config &c) { c.meta_format = (kvq_meta_format)2; }, KVQ_ERR_ARG},
      {"schedule 2", [](kvq_config &c) { c.schedule = (kvq_schedule)2; }, KVQ_ERR_ARG},
      {"kernel 2", [](kvq_config &c) { c.kernel = (kvq_kernel)2; }, KVQ_ERR_ARG},
      {"key scales on KIVI", [](kvq_config &c) { c.key_norm = KVQ_KEYNORM_PROMPT; }, KVQ_ERR_UNSUPPORTED},
      {"key_norm 2", [](kvq_config &c) { c.key_norm = (kvq_key_norm)2; }, KVQ_ERR_ARG},
      {"InnerQ chunked", [](kvq_config &c) { c.scheme = KVQ_SCHEME_INNERQ; }, KVQ_ERR_ARG},
      {"InnerQ packed metadata",
       [](kvq_config &c) { c.scheme = KVQ_SCHEME_INNERQ; c.v_policy = KVQ_V_FIFO; c.meta_format = KVQ_META_F16; },
       KVQ_ERR_UNSUPPORTED},
      {"too many units", [](kvq_config &c) { c.batch = 40000; }, KVQ_ERR_UNSUPPORTED},
  };
  for (const Bad &b : bad) {
    kvq_config c = base_config();
    b.edit(c);
    expect_status(kvq_layout_bytes(&c, &L), b.want, nullptr, nullptr, b.what);
    expect(kvq_workspace_bytes(&c, 100, 0) == 0 && kvq_auto_splits(&c, 100) == 0, "%s: sizes of a bad config", b.what);
  }

  Setup s;
  s.cfg = base_config();
  alloc_cache(s, 1024);
  kvq_cache before;
  const float scale = 0.088f;
  // buffer pointers
  {
    const size_t offs[] = {offsetof(kvq_cache, k_codes), offsetof(kvq_cache, k_scale), offsetof(kvq_cache, k_zero),
                           offsetof(kvq_cache, v_codes), offsetof(kvq_cache, v_scale), offsetof(kvq_cache, v_zero),
                           offsetof(kvq_cache, k_resid), offsetof(kvq_cache, v_resid)};
    for (size_t off : offs) {
      kvq_cache c = s.cache;
      memset(reinterpret_cast<char *>(&c) + off, 0, sizeof(void *));
      before = c;
      expect_status(kvq_quantize_prefill(&s.cfg, &c, s.k, s.v, 10, nullptr), KVQ_ERR_ARG, &before, &c,
                    "null cache buffer");
    }
  }
  before = s.cache;
  expect_status(kvq_append_token(&s.cfg, &s.cache, s.kn, s.vn, nullptr), KVQ_ERR_STATE, &before, &s.cache,
                "append before prefill");
  expect_status(kvq_decode_attention(&s.cfg, &s.cache, s.q, scale, s.out, s.ws, s.ws_bytes, 0, nullptr),
                KVQ_ERR_STATE, &before, &s.cache, "attention before prefill");
  expect_status(kvq_quantize_prefill(&s.cfg, &s.cache, s.k, s.v, 2000, nullptr), KVQ_ERR_CAPACITY, &before, &s.cache,
                "prefill past capacity");
  expect_status(kvq_quantize_prefill(&s.cfg, &s.cache, s.k, s.v, -1, nullptr), KVQ_ERR_ARG, &before, &s.cache,
                "negative prompt length");
  expect_status(kvq_quantize_prefill(&s.cfg, &s.cache, nullptr, s.v, 10, nullptr), KVQ_ERR_ARG, &before, &s.cache,
                "null prompt");
  expect(kvq_quantize_prefill(&s.cfg, &s.cache, s.k, s.v, 1000, nullptr) == KVQ_OK, "prefill: %s", kvq_last_error());
  before = s.cache;
  expect_status(kvq_quantize_prefill(&s.cfg, &s.cache, s.k, s.v, 10, nullptr), KVQ_ERR_STATE, &before, &s.cache,
                "second prefill");
  expect_status(kvq_append_token(&s.cfg, &s.cache, nullptr, s.vn, nullptr), KVQ_ERR_ARG, &before, &s.cache,
                "null k_new");
  expect_status(kvq_decode_attention(&s.cfg, &s.cache, nullptr, scale, s.out, s.ws, s.ws_bytes, 0, nullptr),
                KVQ_ERR_ARG, &before, &s.cache, "null q");
  expect_status(kvq_decode_attention(&s.cfg, &s.cache, s.q, scale, nullptr, s.ws, s.ws_bytes, 0, nullptr),
                KVQ_ERR_ARG, &before, &s.cache, "null out");
  expect_status(kvq_decode_attention(&s.cfg, &s.cache, s.q, scale, s.out, nullptr, s.ws_bytes, 0, nullptr),
                KVQ_ERR_ARG, &before, &s.cache, "null workspace");
  expect_status(kvq_decode_attention(&s.cfg, &s.cache, s.q, scale, s.out, s.ws, s.ws_bytes, -1, nullptr),
                KVQ_ERR_ARG, &before, &s.cache, "splits -1");
  expect_status(kvq_decode_attention(&s.cfg, &s.cache, s.q, scale, s.out, s.ws, s.ws_bytes, kvq::kMaxSplits + 1,
                                     nullptr),
                KVQ_ERR_ARG, &before, &s.cache, "splits past the maximum");
  expect_status(kvq_decode_attention(&s.cfg, &s.cache, s.q, NAN, s.out, s.ws, s.ws_bytes, 0, nullptr), KVQ_ERR_ARG,
                &before, &s.cache, "NaN scale");
  expect_status(kvq_decode_attention(&s.cfg, &s.cache, s.q, scale, s.out, s.ws, 16, 0, nullptr), KVQ_ERR_CAPACITY,
                &before, &s.cache, "small workspace");
  expect_status(kvq_decode_step(&s.cfg, &s.cache, s.kn, s.vn, s.q, scale, s.out, s.ws, 16, 0, nullptr),
                KVQ_ERR_CAPACITY, &before, &s.cache, "small workspace (step)");
  expect_status(kvq_decode_step(&s.cfg, &s.cache, s.kn, nullptr, s.q, scale, s.out, s.ws, s.ws_bytes, 0, nullptr),
                KVQ_ERR_ARG, &before, &s.cache, "null v_new (step)");
  for (int i = 0; i < 24; ++i)
    expect(kvq_append_token(&s.cfg, &s.cache, s.kn, s.vn, nullptr) == KVQ_OK, "append: %s", kvq_last_error());
  before = s.cache;
  expect_status(kvq_append_token(&s.cfg, &s.cache, s.kn, s.vn, nullptr), KVQ_ERR_CAPACITY, &before, &s.cache,
                "append to a full cache");
  expect_status(kvq_decode_step(&s.cfg, &s.cache, s.kn, s.vn, s.q, scale, s.out, s.ws, s.ws_bytes, 0, nullptr),
                KVQ_ERR_CAPACITY, &before, &s.cache, "step on a full cache");
  expect_status(kvq_stream_read_probe(s.ws, 17, (uint32_t *)s.out, nullptr), KVQ_ERR_ARG, nullptr, nullptr,
                "probe size");
  expect(kvq_stream_read_probe(s.ws, 256, (uint32_t *)s.out, nullptr) == KVQ_OK, "probe");
  expect(strcmp(kvq_status_string(KVQ_OK), "") != 0, "status text");
}

// ---- (2) sequences over the supported shapes
struct Shape {
  int bits, group, hpg, residual, sinks, max_tokens;
  kvq_v_policy policy;
  kvq_scheme scheme;
  kvq_meta_format meta;
  kvq_key_norm norm;
};

void run_sequence(const Shape &sh, uint64_t seed) {
  char ctx[256];
  snprintf(ctx, sizeof(ctx), "bits %d G %d hpg %d R %d sinks %d cap %d policy %d scheme %d meta %d norm %d", sh.bits,
           sh.group, sh.hpg, sh.residual, sh.sinks, sh.max_tokens, (int)sh.policy, (int)sh.scheme, (int)sh.meta,
           (int)sh.norm);
  g_context = ctx;
  Setup s;
  s.cfg = base_config();
  s.cfg.bits = sh.bits;
  s.cfg.group = sh.group;
  s.cfg.residual = sh.residual;
  s.cfg.batch = 2;
  s.cfg.num_kv_heads = 2;
  s.cfg.num_q_heads = 2 * sh.hpg;
  s.cfg.max_tokens = sh.max_tokens;
  s.cfg.v_policy = sh.policy;
  s.cfg.scheme = sh.scheme;
  s.cfg.meta_format = sh.meta;
  s.cfg.sink_tokens = sh.sinks;
  s.cfg.key_norm = sh.norm;
  s.cfg.kernel = (seed & 1) ? KVQ_KERNEL_AUTO : KVQ_KERNEL_VALU;
  s.cfg.schedule = (seed & 2) ? KVQ_SCHED_QUEUE : KVQ_SCHED_FIXED;
  std::mt19937_64 rng(seed);
  // prompt lengths: empty, short, around the sinks and a ring, and near capacity
  const int64_t R = sh.residual, S = sh.sinks, cap = sh.max_tokens;
  const int64_t room = 3 * R + 40;
  int64_t lens[] = {0, 1, S, S + 1, S + R - 1, S + R, S + 2 * R + 5, cap - room};
  const int64_t len = lens[rng() % 8];
  if (len < 0 || len + room > cap) return;
  alloc_cache(s, len > 0 ? len : 1);
  expect(kvq_quantize_prefill(&s.cfg, &s.cache, s.k, s.v, len, nullptr) == KVQ_OK, "prefill %" PRId64 ": %s", len,
         kvq_last_error());
  const float scale = 0.088f;
  int steps_checked = 0;
  for (int64_t i = 0; i < room && s.cache.n_tokens < cap; ++i) {
    const int op = (int)(rng() % 4);
    const int32_t splits = (rng() % 3 == 0) ? (int32_t)(1 + rng() % kvq::kMaxSplits) : 0;
    const kvq_cache before = s.cache;
    g_launches = 0;
    if (op == 0) {
      expect(kvq_append_token(&s.cfg, &s.cache, s.kn, s.vn, nullptr) == KVQ_OK, "append: %s", kvq_last_error());
    } else if (op == 1) {
      expect(kvq_append_token(&s.cfg, &s.cache, s.kn, s.vn, nullptr) == KVQ_OK, "append: %s", kvq_last_error());
      expect(kvq_decode_attention(&s.cfg, &s.cache, s.q, scale, s.out, s.ws, s.ws_bytes, splits, nullptr) == KVQ_OK,
             "attention: %s", kvq_last_error());
    } else {
      expect(kvq_decode_step(&s.cfg, &s.cache, s.kn, s.vn, s.q, scale, s.out, s.ws, s.ws_bytes, splits, nullptr) ==
                 KVQ_OK,
             "step: %s", kvq_last_error());
      // steady state: a step is one launch (plus the merge of split records
      // on the vector-ALU path) unless a key group is quantized, the token is
      // a sink, or nothing was quantized ahead for a token that leaves
      const bool iq = sh.scheme == KVQ_SCHEME_INNERQ;
      const bool fifo = iq || sh.policy == KVQ_V_FIFO;
      const bool sink = before.n_tokens < S;
      const int64_t n1 = before.n_tokens + 1;
      const bool key_flush = !iq && n1 - before.nq_k >= R;
      const bool chunk_lag = !iq && !fifo && before.nq_k != before.nq_v;
      const bool pops = fifo && n1 - before.nq_v > R;
      const bool ready = !pops || before.prequant == before.nq_v + 1;
      if (!sink && !key_flush && !chunk_lag && ready) {
        expect(g_launches == 1, "a steady-state step took %d launches", g_launches);
        ++steps_checked;
      }
      if (fifo && R >= 2 && !sink && !key_flush && n1 - s.cache.nq_v == R)
        expect(s.cache.prequant == s.cache.nq_v + 1, "full queue after a step, nothing quantized ahead");
    }
    expect(s.cache.n_tokens == before.n_tokens + 1, "token count");
    expect(s.cache.nq_k <= s.cache.n_tokens && s.cache.nq_v <= s.cache.n_tokens, "counters past n");
    expect(s.cache.n_tokens - s.cache.nq_k <= R && s.cache.n_tokens - s.cache.nq_v <= R, "ring overfull");
  }
  (void)steps_checked;
}

void shape_sweep() {
  int runs = 0;
  uint64_t seed = 1;
  for (int bits : {2, 4})
    for (int G : {32, 64, 128})
      for (int hpg : {1, 2, 4})
        for (int scheme = 0; scheme < 2; ++scheme)
          for (int variant = 0; variant < 4; ++variant)
            for (int R : {1, 32, 128, 512})
              for (int S : {0, 5, 512})
                for (int cap : {4096, 1 << 25}) {
                  Shape sh;
                  sh.bits = bits;
                  sh.group = G;
                  sh.hpg = hpg;
                  sh.residual = R;
                  sh.sinks = S;
                  sh.scheme = scheme ? KVQ_SCHEME_INNERQ : KVQ_SCHEME_KIVI;
                  if (scheme == 0) {
                    if (R % G) continue;
                    sh.policy = (variant & 1) ? KVQ_V_FIFO : KVQ_V_CHUNK;
                    sh.meta = (variant & 2) ? KVQ_META_F16 : KVQ_META_F32;
                    sh.norm = KVQ_KEYNORM_NONE;
                  } else {
                    if (variant >= 2) continue;
                    sh.policy = KVQ_V_FIFO;
                    sh.meta = KVQ_META_F32;
                    sh.norm = variant ? KVQ_KEYNORM_PROMPT : KVQ_KEYNORM_NONE;
                  }
                  sh.max_tokens = cap - cap % R;
                  for (int rep = 0; rep < 2; ++rep) run_sequence(sh, seed++);
                  ++runs;
                }
  printf("shape sweep: %d shapes, %d sequences\n", runs, (int)(seed - 1));
}

}  // namespace

// Usage: kvq_launch_check [--shrink BUFFER]
// --shrink registers the named buffer (k_codes, v_scale, k_resid, workspace,
// ...) 16 bytes shorter than kvq_layout_bytes says, a planted mistake the
// checks must catch (the run then aborts).
int main(int argc, char **argv) {
  if (argc == 3 && strcmp(argv[1], "--shrink") == 0) {
    g_shrink = argv[2];
    shape_sweep();
    return 0;
  }
  validation_cases();
  printf("validation cases: ok\n");
  shape_sweep();
  g_context = "done";
  printf("all checks passed\n");
  return 0;
}
