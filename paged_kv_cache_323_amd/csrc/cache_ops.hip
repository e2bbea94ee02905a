// Cache write and copy-on-write block copy: plain HBM streaming kernels.
//
// Both move whole 16-byte chunks; rows of every supported (dtype, head_dim) are multiples of
// 16 bytes, so the element type never matters here and the result is a bit copy.
#include "common.hpp"
#include "internal.hpp"

namespace pkv {

PKV_DEBUG_UNIT(cache_ops)

// Tuning knobs, chosen by sweeping on the GPU against a plain streaming-copy probe:
//   PKV_COPY_UNROLL  chunks in flight per thread per pool (a group of 256 x U chunks per
//                    workgroup and iteration, all loads of a group issued before its stores);
//   PKV_COPY_NT      cache policy of the loads (bit 0) and stores (bit 1): non-temporal, since
//                    neither kernel re-reads what it moves (the cache write of a 9.4 k-token step
//                    from cold caches: 4.9 against 3.8 TB/s);
//   PKV_COPY_GRID    largest grid; workgroups stride over the remaining groups.
// With one chunk per pool in flight (two loads per thread) and up to 65536 workgroups, the
// 4096-pair copy of sequentially placed blocks reaches 97-98 % of the probe's contiguous copy
// (6.1 of 6.24 TB/s); randomly placed blocks cost about 13 % (5.3 TB/s), which every variant
// swept (1-8 in flight, 4096-65536 workgroups) shares.
#ifndef PKV_COPY_UNROLL
#define PKV_COPY_UNROLL 1
#endif
#ifndef PKV_COPY_NT
#define PKV_COPY_NT 3
#endif
#ifndef PKV_COPY_GRID
#define PKV_COPY_GRID 65536
#endif
constexpr int kCopyGrid = PKV_COPY_GRID;
constexpr int kCopyU = PKV_COPY_UNROLL;
static_assert(kCopyU >= 1 && kCopyU <= 8, "chunk counts leave room for one group of 256 x 8");
constexpr int kCopyNT = PKV_COPY_NT;

__device__ __forceinline__ u32x4 load16(const char* p) {
  if (kCopyNT & 1) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ void store16(char* p, const u32x4& v) {
  if (kCopyNT & 2)
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
  else
    *reinterpret_cast<u32x4*>(p) = v;
}

// pool[slot[t]] <- (k[t], v[t]). Chunk i of the launch is 16-byte chunk i mod cpr of row
// i / cpr, and row r is (token r / H, kv head r mod H), so consecutive lanes move consecutive
// bytes of a row. A slot addresses block slot/B, offset slot%B; the device layout is [N][H][B][D].
__global__ __launch_bounds__(256) void kv_cache_write_kernel(
    const char* __restrict__ k, const char* __restrict__ v, char* __restrict__ kc,
    char* __restrict__ vc, const int32_t* __restrict__ slots, uint32_t total_chunks, int log2_cpr,
    int64_t k_stride_b, int64_t v_stride_b, int num_kv_heads, int block_size, int log2_block, int row_bytes,
    int64_t num_slots) {
  constexpr int U = kCopyU;
  const uint32_t groups = (total_chunks + 256u * U - 1) / (256u * U);
  for (uint32_t g = blockIdx.x; g < groups; g += gridDim.x) {
    u32x4 kk[U], vv[U];
    int64_t dst[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t i = g * (256u * U) + 256u * u + threadIdx.x;
      dst[u] = -1;
      if (i < total_chunks) {
        const uint32_t r = i >> log2_cpr;
        const uint32_t ch = i & ((1u << log2_cpr) - 1);
        const uint32_t t = r / (uint32_t)num_kv_heads;
        const uint32_t h = r - t * (uint32_t)num_kv_heads;
        const int32_t slot = slots[t];
        if (kDebugChecks && slot >= num_slots) debug_flag(DBG_SLOT);
        if (slot >= 0 && (!kDebugChecks || slot < num_slots)) {
          const int64_t blk = slot >> log2_block;
          const int64_t off = slot & (block_size - 1);
#ifdef PKV_TOKEN_MAJOR  // tuning variant: token-major pool [N][B][H][D]
          dst[u] = ((blk * block_size + off) * num_kv_heads + h) * row_bytes + ch * 16;
#else
          dst[u] = ((blk * num_kv_heads + h) * block_size + off) * row_bytes + ch * 16;
#endif
          const int64_t src_in_row = (int64_t)h * row_bytes + ch * 16;
          kk[u] = load16(k + t * k_stride_b + src_in_row);
          vv[u] = load16(v + t * v_stride_b + src_in_row);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (dst[u] >= 0) {
        store16(kc + dst[u], kk[u]);
        store16(vc + dst[u], vv[u]);
      }
    }
  }
}

// Whole-block copies: block dst <- block src for K and V. A block of the head-major layout is one
// contiguous region, so each pair is two flat copies. The launch's work items are (pair, group of
// 256 x U chunks), pair-major; each workgroup strides over them (a bounded grid of long-lived
// workgroups streams better than one short workgroup per item). Copy-on-write copies within one
// pool; swap copies between a GPU pool and a host swap pool (device-addressable pinned memory).
__global__ __launch_bounds__(256) void copy_blocks_kernel(char* __restrict__ dk, char* __restrict__ dv,
                                                          const char* __restrict__ sk, const char* __restrict__ sv,
                                                          const int32_t* __restrict__ pairs, int num_pairs,
                                                          int64_t block_bytes, int src_blocks, int dst_blocks) {
  constexpr int U = kCopyU;
  const int64_t chunks = block_bytes >> 4;
  const int64_t per_pair = (chunks + 256 * U - 1) / (256 * U);
  const int64_t items = per_pair * num_pairs;
  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    const int p = (int)(it / per_pair);
    const int64_t c0 = (it - (int64_t)p * per_pair) * 256 * U;
    const int32_t si = pairs[2 * p], di = pairs[2 * p + 1];
    if (kDebugChecks &&
        (si < 0 || di < 0 || (src_blocks > 0 && si >= src_blocks) || (dst_blocks > 0 && di >= dst_blocks))) {
      if (c0 == 0 && threadIdx.x == 0) debug_flag(DBG_PAIR);
      continue;  // uniform over the workgroup
    }
    const int64_t src = (int64_t)si * block_bytes;
    const int64_t dst = (int64_t)di * block_bytes;
    u32x4 a[U], b[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + 256 * u + threadIdx.x;
      if (c < chunks) {
        a[u] = load16(sk + src + 16 * c);
        b[u] = load16(sv + src + 16 * c);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + 256 * u + threadIdx.x;
      if (c < chunks) {
        store16(dk + dst + 16 * c, a[u]);
        store16(dv + dst + 16 * c, b[u]);
      }
    }
  }
}

hipError_t launch_kv_cache_write(const void* k, const void* v, void* kc, void* vc, const int32_t* slots,
                                 int num_tokens, int64_t k_stride_b, int64_t v_stride_b, int num_kv_heads,
                                 int block_size, int head_dim, int elem_bytes, int num_blocks, hipStream_t stream) {
  const int row_bytes = head_dim * elem_bytes;
  const uint32_t cpr = row_bytes / 16;  // 8, 16 or 32: a power of two
  const uint64_t total = (uint64_t)cpr * num_kv_heads * num_tokens;
  if (total == 0) return hipSuccess;
  if (total > 0xffffffffull - 2048) return hipErrorInvalidConfiguration;  // as validated by the caller
  const uint64_t want = (total + 256ull * kCopyU - 1) / (256ull * kCopyU);
  const unsigned grid = (unsigned)(want < (uint64_t)kCopyGrid ? want : (uint64_t)kCopyGrid);
  return launch_kernel(kv_cache_write_kernel, dim3(grid), dim3(256), stream, static_cast<const char*>(k),
                       static_cast<const char*>(v), static_cast<char*>(kc), static_cast<char*>(vc), slots,
                       (uint32_t)total, ilog2((int)cpr), k_stride_b, v_stride_b, num_kv_heads, block_size,
                       ilog2(block_size), row_bytes, (int64_t)num_blocks * block_size);
}

hipError_t launch_copy_between(void* dk, void* dv, const void* sk, const void* sv, const int32_t* pairs, int num_pairs,
                               int64_t block_bytes, int src_blocks, int dst_blocks, hipStream_t stream) {
  const int64_t per_pair = (block_bytes / 16 + 256 * kCopyU - 1) / (256 * kCopyU);
  const int64_t items = per_pair * num_pairs;
  if (items <= 0) return hipSuccess;
  const unsigned grid = (unsigned)(items < kCopyGrid ? items : kCopyGrid);
  return launch_kernel(copy_blocks_kernel, dim3(grid), dim3(256), stream, static_cast<char*>(dk),
                       static_cast<char*>(dv), static_cast<const char*>(sk), static_cast<const char*>(sv), pairs,
                       num_pairs, block_bytes, src_blocks, dst_blocks);
}

hipError_t launch_copy_blocks(void* kc, void* vc, const int32_t* pairs, int num_pairs, int64_t block_bytes,
                              int num_blocks, hipStream_t stream) {
  return launch_copy_between(kc, vc, kc, vc, pairs, num_pairs, block_bytes, num_blocks, num_blocks, stream);
}

}  // namespace pkv
