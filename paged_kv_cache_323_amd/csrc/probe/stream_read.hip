// Streaming-read probe (measurement only; not part of libpagedkv's interface).
//
// Reads a device buffer once with 16-byte non-temporal loads spread over a grid-stride loop
// and folds every word into a per-thread checksum. A single store happens only if the checksum
// equals a constant that a buffer filled with one repeated byte value cannot produce, so
// the launch moves `bytes` from HBM and writes nothing. The benchmark uses the achieved rate
// as the attainable HBM read bandwidth beside the 8 TB/s specification.
//
//   int32_t pkvprobe_stream_read(const void* buf, size_t bytes, uint32_t* sink, int32_t grid,
//                                void* stream)
// buf: device memory, 16-byte aligned, bytes a multiple of 16; sink: one device word;
// grid: workgroups of 256 threads (1..65535). Returns 0, -1 on bad arguments, or the
// hipError_t of the launch.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ p, size_t n,
                                                          uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * 256;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == 0x12345679u) sink[0] = acc;  // never true for a buffer of one repeated byte
}

extern "C" int32_t pkvprobe_stream_read(const void* buf, size_t bytes, uint32_t* sink, int32_t grid,
                                        void* stream) {
  if (!buf || !sink || bytes == 0 || bytes % 16 || (uintptr_t)buf % 16 || grid < 1 || grid > 65535) return -1;
  const u32x4* p = static_cast<const u32x4*>(buf);
  size_t n = bytes / 16;
  void* args[] = {&p, &n, &sink};
  return (int32_t)hipLaunchKernel(reinterpret_cast<const void*>(&stream_read_kernel), dim3(grid), dim3(256), args,
                                  0, (hipStream_t)stream);
}

// Tile-gather probe: the read pattern of the decode kernel without its arithmetic. Workgroup w
// takes list entries [w * per_wg, (w + 1) * per_wg) and reads each entry's whole tile from the K
// pool, then the same tiles from the V pool (as one decode workgroup reads a partition's K tiles,
// then its V tiles), 16 bytes per thread per 4 KiB with 8 loads in flight, folding every word
// into a checksum stored only if it equals a value that pools of one repeated byte cannot give.
//
//   int32_t pkvprobe_gather_read(const void* pool_k, const void* pool_v, const uint32_t* tiles,
//                                int32_t num_tiles, int32_t tile_bytes, int32_t per_wg,
//                                uint32_t* sink, void* stream)
// pool_k, pool_v: device memory, 16-byte aligned; tiles: device list of tile indices (tile i is
// bytes [i * tile_bytes, (i + 1) * tile_bytes) of each pool; the caller keeps every index inside
// both pools); tile_bytes: 1024, 2048 or a positive multiple of 4096; per_wg: list entries per
// workgroup.
// Returns 0, -1 on bad arguments, or the hipError_t of the launch.
__global__ __launch_bounds__(256) void gather_read_kernel(const u32x4* __restrict__ pk, const u32x4* __restrict__ pv,
                                                          const uint32_t* __restrict__ tiles, int32_t n,
                                                          int32_t per_wg, int32_t chunks, uint32_t* __restrict__ sink) {
  constexpr int U = 8;
  const long long i0 = (long long)blockIdx.x * per_wg * chunks;
  const long long i1 = min((long long)n, (long long)(blockIdx.x + 1) * per_wg) * chunks;
  uint32_t acc = 0;
  for (int pass = 0; pass < 2; ++pass) {
    const u32x4* pool = pass ? pv : pk;
    auto addr = [&](long long i) {  // chunk c of list entry t: 256 threads x 16 bytes
      const long long t = i / chunks, c = i - t * chunks;
      return pool + ((size_t)tiles[t] * chunks + c) * 256 + threadIdx.x;
    };
    long long i = i0;
    for (; i + U <= i1; i += U) {
      u32x4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(addr(i + u));
#pragma unroll
      for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    for (; i < i1; ++i) {
      const u32x4 v = __builtin_nontemporal_load(addr(i));
      acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
  }
  if (acc == 0x12345679u) sink[0] = acc;
}

// Tiles of 1 or 2 KiB (head_dim 64, or 8-token blocks, at 16 bits): every 256-thread step reads
// 4096 / tile_bytes consecutive list entries, tile_bytes / 16 threads per tile; the last step of a
// workgroup's range loads only the entries inside it.
__global__ __launch_bounds__(256) void gather_read_small_kernel(const u32x4* __restrict__ pk,
                                                                const u32x4* __restrict__ pv,
                                                                const uint32_t* __restrict__ tiles, int32_t n,
                                                                int32_t per_wg, int32_t lanes,
                                                                uint32_t* __restrict__ sink) {
  constexpr int U = 8;
  const int per_step = 256 / lanes;
  const long long t0 = (long long)blockIdx.x * per_wg;
  const long long t1 = min((long long)n, t0 + per_wg);
  const int sub = threadIdx.x / lanes, off = threadIdx.x % lanes;
  uint32_t acc = 0;
  for (int pass = 0; pass < 2; ++pass) {
    const u32x4* pool = pass ? pv : pk;
    long long t = t0;
    for (; t + (long long)U * per_step <= t1; t += (long long)U * per_step) {
      u32x4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        v[u] = __builtin_nontemporal_load(pool + (size_t)tiles[t + u * per_step + sub] * lanes + off);
#pragma unroll
      for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    for (; t < t1; t += per_step) {
      const long long e = t + sub;
      if (e < t1) {
        const u32x4 v = __builtin_nontemporal_load(pool + (size_t)tiles[e] * lanes + off);
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
      }
    }
  }
  if (acc == 0x12345679u) sink[0] = acc;
}

extern "C" int32_t pkvprobe_gather_read(const void* pool_k, const void* pool_v, const uint32_t* tiles,
                                        int32_t num_tiles, int32_t tile_bytes, int32_t per_wg, uint32_t* sink,
                                        void* stream) {
  if (!pool_k || !pool_v || !tiles || !sink || (uintptr_t)pool_k % 16 || (uintptr_t)pool_v % 16) return -1;
  const bool small = tile_bytes == 1024 || tile_bytes == 2048;
  if (num_tiles < 1 || per_wg < 1 || (!small && (tile_bytes < 4096 || tile_bytes % 4096))) return -1;
  const long long grid = ((long long)num_tiles + per_wg - 1) / per_wg;
  if (grid > 0x7fffffff) return -1;
  const u32x4* pk = static_cast<const u32x4*>(pool_k);
  const u32x4* pv = static_cast<const u32x4*>(pool_v);
  int32_t n = num_tiles;
  if (small) {
    int32_t lanes = tile_bytes / 16;
    void* args[] = {&pk, &pv, &tiles, &n, &per_wg, &lanes, &sink};
    return (int32_t)hipLaunchKernel(reinterpret_cast<const void*>(&gather_read_small_kernel), dim3((unsigned)grid),
                                    dim3(256), args, 0, (hipStream_t)stream);
  }
  int32_t chunks = tile_bytes / 4096;
  void* args[] = {&pk, &pv, &tiles, &n, &per_wg, &chunks, &sink};
  return (int32_t)hipLaunchKernel(reinterpret_cast<const void*>(&gather_read_kernel), dim3((unsigned)grid), dim3(256),
                                  args, 0, (hipStream_t)stream);
}

// Streaming-copy probe: dst <- src over `bytes`, 16 bytes per thread access, U accesses in
// flight per thread (all loads of a group issued before its stores), grid-stride over groups of
// U x 256 chunks per workgroup. `nt` selects non-temporal loads (bit 0) and stores (bit 1). The
// benchmark takes the best rate over a few grids and variants as the attainable copy bandwidth
// (bytes read + bytes written per second) that copy_blocks, the cache write and swap face.
//
//   int32_t pkvprobe_stream_copy(void* dst, const void* src, size_t bytes, int32_t grid,
//                                int32_t unroll, int32_t nt, void* stream)
// dst, src: device memory, 16-byte aligned, not overlapping; bytes: a multiple of 16 * 256 *
// unroll; unroll: 1, 2, 4 or 8; grid: workgroups of 256 threads (1..65535). Returns 0, -1 on bad
// arguments, or the hipError_t of the launch.
template <int U, int NT>
__global__ __launch_bounds__(256) void stream_copy_kernel(u32x4* __restrict__ d, const u32x4* __restrict__ s,
                                                          size_t groups) {
  for (size_t g = blockIdx.x; g < groups; g += gridDim.x) {
    const size_t base = g * (256 * U) + threadIdx.x;
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = (NT & 1) ? __builtin_nontemporal_load(s + base + 256 * u) : s[base + 256 * u];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (NT & 2)
        __builtin_nontemporal_store(v[u], d + base + 256 * u);
      else
        d[base + 256 * u] = v[u];
    }
  }
}

template <int U>
static const void* copy_kernel_for(int nt) {
  switch (nt) {
    case 0: return reinterpret_cast<const void*>(&stream_copy_kernel<U, 0>);
    case 1: return reinterpret_cast<const void*>(&stream_copy_kernel<U, 1>);
    case 2: return reinterpret_cast<const void*>(&stream_copy_kernel<U, 2>);
    default: return reinterpret_cast<const void*>(&stream_copy_kernel<U, 3>);
  }
}

extern "C" int32_t pkvprobe_stream_copy(void* dst, const void* src, size_t bytes, int32_t grid, int32_t unroll,
                                        int32_t nt, void* stream) {
  if (!dst || !src || (uintptr_t)dst % 16 || (uintptr_t)src % 16 || grid < 1 || grid > 65535) return -1;
  if ((unroll != 1 && unroll != 2 && unroll != 4 && unroll != 8) || nt < 0 || nt > 3) return -1;
  const size_t group_bytes = (size_t)16 * 256 * unroll;
  if (bytes == 0 || bytes % group_bytes) return -1;
  const char* s8 = static_cast<const char*>(src);
  const char* d8 = static_cast<const char*>(dst);
  if (!(d8 + bytes <= s8 || s8 + bytes <= d8)) return -1;  // overlapping ranges
  u32x4* d = static_cast<u32x4*>(dst);
  const u32x4* s = static_cast<const u32x4*>(src);
  size_t groups = bytes / group_bytes;
  void* args[] = {&d, &s, &groups};
  const void* k = unroll == 1 ? copy_kernel_for<1>(nt) : unroll == 2 ? copy_kernel_for<2>(nt)
                : unroll == 4 ? copy_kernel_for<4>(nt) : copy_kernel_for<8>(nt);
  return (int32_t)hipLaunchKernel(k, dim3(grid), dim3(256), args, 0, (hipStream_t)stream);
}

// Row-gather probe: like the tile-gather probe, but a tile is `rows` rows of `row_bytes` bytes,
// `row_stride` bytes apart, starting at tiles[t] * unit_bytes: the (block, kv head) tile of a
// head-major pool (rows D·e apart, contiguous) or of a token-major pool (rows H·D·e apart). One
// 16-byte load per thread per chunk, 8 in flight, K pool then V pool, checksum as above.
//
//   int32_t pkvprobe_gather_rows(const void* pool_k, const void* pool_v, const uint32_t* tiles,
//                                int32_t num_tiles, int64_t unit_bytes, int32_t rows,
//                                int32_t row_bytes, int64_t row_stride, int32_t per_wg,
//                                uint32_t* sink, void* stream)
// row_bytes: a multiple of 16, with rows * row_bytes a multiple of 4096;
// the caller keeps every row inside both pools. Returns 0, -1 on bad arguments, or the
// hipError_t of the launch.
__global__ __launch_bounds__(256) void gather_rows_kernel(const char* __restrict__ pk, const char* __restrict__ pv,
                                                          const uint32_t* __restrict__ tiles, int32_t n, int64_t unit,
                                                          int32_t cpr, int32_t chunks, int64_t stride,
                                                          int32_t per_wg, uint32_t* __restrict__ sink) {
  constexpr int U = 8;
  const long long i0 = (long long)blockIdx.x * per_wg * chunks;
  const long long i1 = min((long long)n, (long long)(blockIdx.x + 1) * per_wg) * chunks;
  uint32_t acc = 0;
  for (int pass = 0; pass < 2; ++pass) {
    const char* pool = pass ? pv : pk;
    auto addr = [&](long long i) {  // 4 KiB chunk c of entry t: 256 threads x 16 bytes
      const long long t = i / chunks, c = i - t * chunks;
      const long long e = c * 256 + threadIdx.x;  // 16-byte piece within the tile
      const long long row = e / cpr, col = e - row * cpr;
      return reinterpret_cast<const u32x4*>(pool + (long long)tiles[t] * unit + row * stride + col * 16);
    };
    long long i = i0;
    for (; i + U <= i1; i += U) {
      u32x4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(addr(i + u));
#pragma unroll
      for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    for (; i < i1; ++i) {
      const u32x4 v = __builtin_nontemporal_load(addr(i));
      acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
  }
  if (acc == 0x12345679u) sink[0] = acc;
}

extern "C" int32_t pkvprobe_gather_rows(const void* pool_k, const void* pool_v, const uint32_t* tiles,
                                        int32_t num_tiles, int64_t unit_bytes, int32_t rows, int32_t row_bytes,
                                        int64_t row_stride, int32_t per_wg, uint32_t* sink, void* stream) {
  if (!pool_k || !pool_v || !tiles || !sink || (uintptr_t)pool_k % 16 || (uintptr_t)pool_v % 16) return -1;
  if (num_tiles < 1 || rows < 1 || row_bytes < 16 || row_bytes % 16 || unit_bytes % 16 || row_stride % 16) return -1;
  if (((long long)rows * row_bytes) % 4096 || per_wg < 1) return -1;
  const long long grid = ((long long)num_tiles + per_wg - 1) / per_wg;
  if (grid > 0x7fffffff) return -1;
  const char* pk = static_cast<const char*>(pool_k);
  const char* pv = static_cast<const char*>(pool_v);
  int32_t n = num_tiles, cpr = row_bytes / 16, chunks = (int32_t)((long long)rows * row_bytes / 4096);
  int64_t unit = unit_bytes, stride = row_stride;
  void* args[] = {&pk, &pv, &tiles, &n, &unit, &cpr, &chunks, &stride, &per_wg, &sink};
  return (int32_t)hipLaunchKernel(reinterpret_cast<const void*>(&gather_rows_kernel), dim3((unsigned)grid), dim3(256),
                                  args, 0, (hipStream_t)stream);
}
