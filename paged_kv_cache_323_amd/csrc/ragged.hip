// Ragged mixed prefill + decode attention (selective batching). Placeholder until the kernel
// lands: the entry points validate nothing and report an unsupported shape.
#include <hip/hip_runtime.h>
#include "../../include/pagedkv.h"

extern "C" {
size_t pkv_ragged_workspace_bytes(int32_t, int32_t, int32_t, int32_t, int32_t, const pkv_cache_desc*) { return 0; }
int32_t pkv_paged_attention_ragged(void*, int32_t, const void*, const int32_t*, const int32_t*, const void*,
                                   const void*, const int32_t*, int32_t, int32_t, int32_t, int32_t, float,
                                   int32_t, int32_t, const pkv_cache_desc*, void*, size_t, void*) {
  return PKV_ESHAPE;
}
}
