// Host-side helpers shared by the C ABI sources (kvq_api.cpp and
// kvq_noalloc.hip).  Not part of the public ABI.
#pragma once

#include "../../include/kvq.h"

namespace kvq {

// Sets the thread-local error text and returns s.
kvq_status report(kvq_status s, const char *msg);

// kvq_decode_attention with its arguments validated and its launches
// enqueued, into the given workspace.
kvq_status decode_attention_into(const kvq_config *cfg, const kvq_cache *cache, const uint16_t *q,
                                 float softmax_scale, float *out, void *workspace, size_t workspace_bytes,
                                 int32_t splits, hipStream_t stream);

}  // namespace kvq
