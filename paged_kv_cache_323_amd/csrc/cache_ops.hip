// Cache write and copy-on-write block copy: plain HBM streaming kernels.
//
// Both move whole 16-byte chunks; rows of every supported (dtype, head_dim) are multiples of
// 16 bytes, so the element type never matters here and the result is a bit copy.
#include "common.hpp"
#include "internal.hpp"

namespace pkv {

PKV_DEBUG_UNIT(cache_ops)

// pool[slot[t]] <- (k[t], v[t]): one thread per 16-byte chunk of one (token, kv head) row.
// A slot addresses block slot/B, offset slot%B; the device layout is [N][H][B][D].
__global__ __launch_bounds__(256) void kv_cache_write_kernel(
    const char* __restrict__ k, const char* __restrict__ v, char* __restrict__ kc,
    char* __restrict__ vc, const int32_t* __restrict__ slots, uint32_t total_chunks,
    uint32_t chunks_per_token, uint32_t chunks_per_row, int64_t k_stride_b, int64_t v_stride_b,
    int num_kv_heads, int block_size, int log2_block, int row_bytes, int64_t num_slots) {
  const uint32_t step = gridDim.x * blockDim.x;
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < total_chunks; i += step) {
    const uint32_t t = i / chunks_per_token;
    const uint32_t rem = i - t * chunks_per_token;
    const uint32_t h = rem / chunks_per_row;
    const uint32_t ch = rem - h * chunks_per_row;
    const int32_t slot = slots[t];
    if (slot < 0) continue;
    if (kDebugChecks && slot >= num_slots) {
      debug_flag(DBG_SLOT);
      continue;
    }
    const int64_t blk = slot >> log2_block;
    const int64_t off = slot & (block_size - 1);
    const int64_t dst = ((blk * num_kv_heads + h) * block_size + off) * row_bytes + ch * 16;
    const int64_t src_in_row = (int64_t)h * row_bytes + ch * 16;
    const u32x4 kk = *reinterpret_cast<const u32x4*>(k + t * k_stride_b + src_in_row);
    const u32x4 vv = *reinterpret_cast<const u32x4*>(v + t * v_stride_b + src_in_row);
    *reinterpret_cast<u32x4*>(kc + dst) = kk;
    *reinterpret_cast<u32x4*>(vc + dst) = vv;
  }
}

// Whole-block copies: block dst <- block src for K and V. A block of the head-major layout is one
// contiguous region, so each pair is two flat copies. Copy-on-write copies within one pool; swap
// copies between a GPU pool and a host swap pool (device-addressable pinned memory).
__global__ __launch_bounds__(256) void copy_blocks_kernel(char* __restrict__ dk, char* __restrict__ dv,
                                                          const char* __restrict__ sk, const char* __restrict__ sv,
                                                          const int32_t* __restrict__ pairs, int64_t block_bytes,
                                                          int src_blocks, int dst_blocks) {
  const int p = blockIdx.y;
  const int32_t si = pairs[2 * p], di = pairs[2 * p + 1];
  if (kDebugChecks &&
      (si < 0 || di < 0 || (src_blocks > 0 && si >= src_blocks) || (dst_blocks > 0 && di >= dst_blocks))) {
    if (blockIdx.x == 0 && threadIdx.x == 0) debug_flag(DBG_PAIR);
    return;  // uniform over the workgroup
  }
  const int64_t src = (int64_t)si * block_bytes;
  const int64_t dst = (int64_t)di * block_bytes;
  const int64_t step = (int64_t)gridDim.x * blockDim.x * 16;
  for (int64_t off = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 16; off < block_bytes; off += step) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(sk + src + off);
    const u32x4 b = *reinterpret_cast<const u32x4*>(sv + src + off);
    *reinterpret_cast<u32x4*>(dk + dst + off) = a;
    *reinterpret_cast<u32x4*>(dv + dst + off) = b;
  }
}

hipError_t launch_kv_cache_write(const void* k, const void* v, void* kc, void* vc, const int32_t* slots,
                                 int num_tokens, int64_t k_stride_b, int64_t v_stride_b, int num_kv_heads,
                                 int block_size, int head_dim, int elem_bytes, int num_blocks, hipStream_t stream) {
  const int row_bytes = head_dim * elem_bytes;
  const uint32_t cpr = row_bytes / 16;
  const uint32_t cpt = cpr * num_kv_heads;
  const uint64_t total = (uint64_t)cpt * num_tokens;
  if (total == 0) return hipSuccess;
  if (total > 0xffffffffull) return hipErrorInvalidConfiguration;
  const uint64_t want = (total + 255) / 256;
  const unsigned grid = (unsigned)(want < 65536 ? want : 65536);
  return launch_kernel(kv_cache_write_kernel, dim3(grid), dim3(256), stream, static_cast<const char*>(k),
                       static_cast<const char*>(v), static_cast<char*>(kc), static_cast<char*>(vc), slots,
                       (uint32_t)total, cpt, cpr, k_stride_b, v_stride_b, num_kv_heads, block_size,
                       ilog2(block_size), row_bytes, (int64_t)num_blocks * block_size);
}

hipError_t launch_copy_between(void* dk, void* dv, const void* sk, const void* sv, const int32_t* pairs, int num_pairs,
                               int64_t block_bytes, int src_blocks, int dst_blocks, hipStream_t stream) {
  int64_t gx = (block_bytes + 256 * 16 * 4 - 1) / (256 * 16 * 4);  // ~4 chunks per thread
  if (gx < 1) gx = 1;
  if (gx > 256) gx = 256;
  for (int first = 0; first < num_pairs; first += 65535) {  // grid.y limit
    const int n = num_pairs - first < 65535 ? num_pairs - first : 65535;
    const hipError_t e =
        launch_kernel(copy_blocks_kernel, dim3((unsigned)gx, (unsigned)n), dim3(256), stream, static_cast<char*>(dk),
                      static_cast<char*>(dv), static_cast<const char*>(sk), static_cast<const char*>(sv),
                      pairs + 2 * (int64_t)first, block_bytes, src_blocks, dst_blocks);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_copy_blocks(void* kc, void* vc, const int32_t* pairs, int num_pairs, int64_t block_bytes,
                              int num_blocks, hipStream_t stream) {
  return launch_copy_between(kc, vc, kc, vc, pairs, num_pairs, block_bytes, num_blocks, num_blocks, stream);
}

}  // namespace pkv
