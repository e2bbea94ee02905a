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
