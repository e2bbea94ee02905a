// Paged decode attention that allocates nothing: the split-context partials live in a
// file-scope device array instead of a caller's workspace.
//
// For callers that cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc). The array is `scratch`, PKV_NOALLOC_SCRATCH_BYTES
// bytes; every GPU the library runs on holds its own copy until the process ends. Host code
// never passes the array's name to a kernel (on the host it is only a stand-in for the device
// symbol): the first call on each device asks the runtime for that device's address of the
// array, with the device current, and every later call on the device uses the kept address.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/pagedkv.h"
#include "internal.hpp"

namespace {

static __device__ __align__(256) unsigned char scratch[PKV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// The current device's address of `scratch`, looked up once per device.
int32_t scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    pkv::set_last_launch_error(e);
    return PKV_ELAUNCH;
  }
  if (dev < 0 || dev >= kMaxDevices) return PKV_EINVAL;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      pkv::set_last_launch_error(e != hipSuccess ? e : hipErrorInvalidSymbol);
      return PKV_ELAUNCH;
    }
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return PKV_OK;
}

}  // namespace

extern "C" int32_t pkv_paged_attention_decode_noalloc(void* out, int32_t out_dtype, const void* q,
                                                      const void* k_cache, const void* v_cache,
                                                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                                                      const int32_t* context_lens, int32_t num_seqs,
                                                      int32_t num_q_heads, float scale, int32_t max_context_len,
                                                      const pkv_cache_desc* cache, void* stream) {
  // Size first, on the host only: the partials this call needs at the automatic partition size.
  const int32_t p = pkv_decode_partition_size(num_seqs, num_q_heads, max_context_len, cache);
  if (p < 0) {
    // An invalid cache, head count, count or length: the workspace entry point's validation
    // names it (with no workspace it stops at that check, before any device call).
    return pkv_paged_attention_decode_ex(out, out_dtype, q, k_cache, v_cache, block_tables, max_blocks_per_seq,
                                         context_lens, num_seqs, num_q_heads, scale, max_context_len, cache, 0,
                                         nullptr, 0, stream);
  }
  const size_t need = pkv_decode_workspace_bytes_ex(num_seqs, num_q_heads, max_context_len, cache, p);
  if (need > PKV_NOALLOC_SCRATCH_BYTES) return PKV_EWORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    const int32_t st = scratch_ptr(&ws);
    if (st != PKV_OK) return st;
  }
  // The same kernels as pkv_paged_attention_decode at the same partition size; they need no
  // initialised workspace, so nothing is cleared.
  return pkv_paged_attention_decode_ex(out, out_dtype, q, k_cache, v_cache, block_tables, max_blocks_per_seq,
                                       context_lens, num_seqs, num_q_heads, scale, max_context_len, cache, p, ws,
                                       need > 0 ? (size_t)PKV_NOALLOC_SCRATCH_BYTES : 0, stream);
}
