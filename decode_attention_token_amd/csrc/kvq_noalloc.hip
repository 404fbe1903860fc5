// kvq_decode_attention_static: decode attention whose scratch (the per-unit
// counters and the split records of the workspace) is a fixed-size array in
// device memory that the library's code object carries, so the caller passes
// no workspace and nothing is allocated at run time.  For callers that cannot
// allocate device memory.
//
// The array is a file-scope __device__ variable: every GPU the library runs
// on holds its own copy until the process ends.  In host code its name is
// only a stand-in, so its device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and only that address is
// ever passed to kernels.
//
// Nothing in the array has to start at zero: the matrix-core kernel runs its
// fixed schedule here (the work-queue ticket is not read), the split records
// are written before the unit's last workgroup or the merge kernel reads them
// in the same call, and the election words carry the launch's epoch, so a
// word left by an earlier call counts as empty.  Calls that overlap on one
// GPU share the array and race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/kvq.h"
#include "kvq_internal.h"
#include "kvq_api_internal.h"

namespace {

static_assert(KVQ_STATIC_SCRATCH_BYTES % 256 == 0, "scratch size");
__device__ __align__(256) unsigned char scratch[KVQ_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch[kMaxDevices];   // device address of `scratch` per device, once looked up

// Device address of this device's copy of the array; nullptr (with the
// error text set) on failure.
void *scratch_of(int dev, kvq_status &st) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      st = kvq::report(KVQ_ERR_DEVICE, "hipGetSymbolAddress of the static scratch array failed");
      return nullptr;
    }
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" kvq_status kvq_decode_attention_static(const kvq_config *cfg, const kvq_cache *cache, const uint16_t *q,
                                                  float softmax_scale, float *out, int32_t splits,
                                                  hipStream_t stream) {
  if (!cfg || !cache) return kvq::report(KVQ_ERR_ARG, "config or cache is null");
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return kvq::report(KVQ_ERR_DEVICE, "no current HIP device");
  if (stream != nullptr) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess)
      return kvq::report(KVQ_ERR_ARG, "the stream's device could not be determined");
    if ((int)sdev != dev)
      return kvq::report(KVQ_ERR_ARG, "the stream belongs to another device than the current one");
  }
  kvq_config c = *cfg;
  c.schedule = KVQ_SCHED_FIXED;   // the ticket counters would have to start at zero
  const size_t need = kvq_workspace_bytes(&c, cache->n_tokens, splits);
  if (need == 0) {
    kvq_layout lay;
    const kvq_status s = kvq_layout_bytes(&c, &lay);   // the reason of an invalid config
    return s != KVQ_OK ? s : kvq::report(KVQ_ERR_ARG, "splits must be in [0, 64]");
  }
  if (need > KVQ_STATIC_SCRATCH_BYTES)
    return kvq::report(KVQ_ERR_CAPACITY,
                       "the call needs more scratch than the static maximum (KVQ_STATIC_SCRATCH_BYTES, "
                       "16 MiB): fewer splits, batch or query heads, or kvq_decode_attention with a workspace");
  kvq_status st = KVQ_OK;
  void *ptr = scratch_of(dev, st);
  if (ptr == nullptr) return st;
  return kvq::decode_attention_into(&c, cache, q, softmax_scale, out, ptr, KVQ_STATIC_SCRATCH_BYTES, splits, stream);
}
