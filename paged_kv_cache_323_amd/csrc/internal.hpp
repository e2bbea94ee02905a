// Internal launch interface between the C ABI (api.cpp) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#ifndef PKV_SCORE_FLOATS
#define PKV_SCORE_FLOATS 8192
#endif
#ifndef PKV_DECODE_PREFETCH
#define PKV_DECODE_PREFETCH 3
#endif

// Query-head groupings (bit g set: g query heads per kv head) whose decode over 16-bit pools runs
// the one-pass kernel, at head_dim 128 and at head_dim 64; the others, and f32 pools, run the
// three-phase kernel. Chosen by measurement (bf16, block size 16, GQA lengths): the one-pass kernel
// is ahead at eight heads per kv head (both head sizes) and at four with head_dim 64, behind at
// four with head_dim 128 (-1 %) and at one or two (-2 to -4 %).
#ifndef PKV_DECODE_FLASH
#define PKV_DECODE_FLASH (1 << 8)
#endif
#ifndef PKV_DECODE_FLASH_D64
#define PKV_DECODE_FLASH_D64 ((1 << 8) | (1 << 4))
#endif
// Largest partition of the one-pass kernel (it holds no scores, so LDS does not bound it).
#ifndef PKV_FLASH_PARTITION
#define PKV_FLASH_PARTITION 4096
#endif

namespace pkv {

// Scores a three-phase decode workgroup holds in LDS: partition tokens x query heads per kv head
// (32 KiB, which keeps four 256-thread workgroups per CU for every head grouping).
constexpr int kScoreFloats = PKV_SCORE_FLOATS;
// Whether g query heads per kv head over a pool of element type dt (0 = f32, 1 = f16, 2 = bf16) and
// head_dim d run the one-pass decode kernel.
constexpr bool one_pass(int g, int dt, int d) {
  return dt != 0 && g >= 1 && g <= 16 && (((d == 64 ? PKV_DECODE_FLASH_D64 : PKV_DECODE_FLASH) >> g) & 1) != 0;
}
// Largest decode partition in tokens for that kernel choice.
constexpr int max_partition(int g, int dt, int d) { return one_pass(g, dt, d) ? PKV_FLASH_PARTITION : kScoreFloats / g; }

inline int ilog2(int x) {
  int r = 0;
  while ((1 << r) < x) ++r;
  return r;
}

// Records the HIP status that pkv_last_launch_error() reports (api.cpp).
void set_last_launch_error(hipError_t e);

template <class T> struct NonDeduced { using type = T; };

// Enqueue kernel<<<grid, block, 0, stream>>>(args...) and return the status of this launch
// alone: an error left behind by an earlier, unrelated HIP call on the thread does not leak in.
template <typename... P>
inline hipError_t launch_kernel(void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t stream,
                                typename NonDeduced<P>::type... args) {
  void* argv[] = {static_cast<void*>(&args)..., nullptr};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, 0, stream);
}

// Launchers return hipSuccess, the failed launch's hipError_t, or hipErrorInvalidConfiguration
// for a shape they do not handle.
// num_blocks: blocks of the pool (debug builds reject slots beyond it).
hipError_t launch_kv_cache_write(const void* k, const void* v, void* kc, void* vc, const int32_t* slots,
                                 int num_tokens, int64_t k_stride_b, int64_t v_stride_b, int num_kv_heads,
                                 int block_size, int head_dim, int elem_bytes, int num_blocks, hipStream_t stream);

hipError_t launch_copy_blocks(void* kc, void* vc, const int32_t* pairs, int num_pairs, int64_t block_bytes,
                              int num_blocks, hipStream_t stream);

// Whole-block copies from (src_k, src_v) to (dst_k, dst_v); either may be pinned host memory.
// src_blocks / dst_blocks bound the pair indices in debug builds (0: no upper bound known).
hipError_t launch_copy_between(void* dst_k, void* dst_v, const void* src_k, const void* src_v, const int32_t* pairs,
                               int num_pairs, int64_t block_bytes, int src_blocks, int dst_blocks,
                               hipStream_t stream);

// Debug builds: copy the translation unit's error words to out[DBG_WORDS] (after a device-wide
// wait) and clear them when clear is set. Release builds write zeros.
int debug_words_cache_ops(uint32_t* out, bool clear);
int debug_words_decode(uint32_t* out, bool clear);
int debug_words_ragged(uint32_t* out, bool clear);

struct DecodeLaunch {
  void* out;
  int out_dt;
  const void* q;
  const void* kc;
  const void* vc;
  const int32_t* tables;
  int max_blocks;
  const int32_t* ctx_lens;
  const int32_t* cu = nullptr;  // ragged batches: per-sequence query row offsets (decode rows only)
  int num_seqs;
  int num_q_heads;
  int num_kv_heads;
  int block_size;
  int head_dim;
  int dt;
  float scale;
  int partition;   // tokens per partition
  int max_parts;   // ceil(max_ctx / partition), >= 1
  float* ws_acc;   // [S][Hkv][max_parts][G][D]   (only when max_parts > 1)
  float* ws_ml;    // [S][Hkv][max_parts][G][2]
  int stage;       // 0: partitions then merge; 1: partitions only; 2: merge only
  int num_blocks;  // pool blocks (debug builds check table entries against it)
  int num_rows;    // rows of q / out (debug builds check ragged row offsets against it)
  const int32_t* items = nullptr;  // optional work list of (seq | part << 16) for the partition launch
  int num_items = 0;
  // 1: every query row of a ragged batch (cu set) is its own item and attends keys up to its own
  // position; partials are indexed by row (num_rows of them)
  int causal_rows = 0;
  // Optional: each sequence's new token, stored by the partition launch before it is attended
  // (k_new / v_new [num_seqs][Hkv][D], slot per sequence, < 0: none).
  const void* k_new = nullptr;
  const void* v_new = nullptr;
  const int32_t* new_slots = nullptr;
};

hipError_t launch_decode(const DecodeLaunch& a, hipStream_t stream);

struct PrefillLaunch {
  void* out;
  int out_dt;
  const void* q;
  const void* kc;
  const void* vc;
  const int32_t* tables;
  int max_blocks;
  const int32_t* cu;
  const int32_t* ctx_lens;
  int num_seqs;
  int num_tokens;
  int num_q_heads;
  int num_kv_heads;
  int block_size;
  int head_dim;
  int dt;
  float scale;
  int num_blocks;  // pool blocks (debug builds check table entries against it)
  int min_rows;    // sequences with at least this many query rows (1 or 2) get row tiles
};

// Causal attention of every sequence of a ragged batch with at least min_rows query rows (2:
// the prefill sequences; rows of single-row sequences are left untouched. 1: every sequence).
hipError_t launch_ragged_prefill(const PrefillLaunch& a, hipStream_t stream);

}  // namespace pkv
