// C ABI of libpagedkv.so: argument validation, launch sizing and workspace carving.
// The kernels live in cache_ops.hip, decode.hip and ragged.hip; the host block manager in
// block_manager.cpp.
#include <hip/hip_runtime.h>
#include <math.h>

#include <algorithm>
#include <vector>
#include <stdint.h>

#include "../../include/pagedkv.h"
#include "common.hpp"
#include "internal.hpp"

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int elem_bytes(int dt) { return dt == PKV_F32 ? 4 : (dt == PKV_F16 || dt == PKV_BF16) ? 2 : 0; }

// Validates the pool description; returns PKV_OK or the status to report.
int32_t check_cache(const pkv_cache_desc* c) {
  if (!c) return PKV_EINVAL;
  if (elem_bytes(c->dtype) == 0) return PKV_EDTYPE;
  if (c->block_size != 8 && c->block_size != 16 && c->block_size != 32) return PKV_ESHAPE;
  if (c->head_dim != 64 && c->head_dim != 128) return PKV_ESHAPE;
  if (c->num_blocks <= 0 || c->num_kv_heads <= 0) return PKV_EINVAL;
  if ((int64_t)c->num_blocks * c->block_size > INT32_MAX) return PKV_ESHAPE;
  return PKV_OK;
}

int32_t check_heads(int32_t hq, const pkv_cache_desc* c) {
  if (hq <= 0 || hq % c->num_kv_heads != 0) return PKV_ESHAPE;
  const int g = hq / c->num_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8) return PKV_ESHAPE;
  return PKV_OK;
}

int32_t check_out_dtype(int32_t out_dt, const pkv_cache_desc* c) {
  return (out_dt == PKV_F32 || out_dt == c->dtype) ? PKV_OK : PKV_EDTYPE;
}

// Automatic partition size. Contexts that fit the largest partition of the kernel that serves this
// head grouping, element type and head size (at most kMaxAutoPartition) take one partition (rounded up to 64
// tokens), longer ones partitions of that size. While the launch would then have fewer than kMinWorkgroups workgroups (sequences x
// kv heads x partitions of the longest context), the partition is halved, down to
// kMinAutoPartition tokens, so that a small batch of long contexts still spreads over the CUs.
constexpr int64_t kMinWorkgroups = 512;  // two per CU
constexpr int kMinAutoPartition = 256;
// Longer partitions than this leave a launch's tail to a few long contexts (one query head per
// kv head: 8192-token partitions measured 17 % slower than 4096 on lognormal lengths).
constexpr int kMaxAutoPartition = 4096;

// Largest partition the automatic size starts from for g query heads per kv head.
int auto_cap(int g, int dt, int d) { return std::min(pkv::max_partition(g, dt, d), kMaxAutoPartition); }

int auto_partition(int32_t num_seqs, int32_t hkv, int g, int dt, int d, int32_t max_ctx) {
  const int cap = auto_cap(g, dt, d);
  const int64_t ctx = max_ctx > 0 ? max_ctx : 1;
  int p = ctx <= cap ? (int)((ctx + 63) / 64 * 64) : cap;
  auto workgroups = [&](int part) { return (int64_t)num_seqs * hkv * ((ctx + part - 1) / part); };
  while (p > kMinAutoPartition && workgroups(p) < kMinWorkgroups)
    p = std::max(kMinAutoPartition, (p / 2 + 63) / 64 * 64);
  return p;
}

bool valid_partition(int p, int bs, int g, int dt, int d) {
  return p >= 64 && p <= pkv::max_partition(g, dt, d) && p % 64 == 0 && p % bs == 0;
}

struct DecodeWs {
  size_t acc, ml, total;
};

// Partial results of `items` (sequence, kv head, partition) triples, g query heads each.
DecodeWs decode_ws_items(size_t items, int g, int32_t head_dim) {
  DecodeWs w{0, 0, 0};
  if (items == 0) return w;
  w.acc = 0;
  w.ml = align_up(items * g * head_dim * sizeof(float));
  w.total = w.ml + align_up(items * g * 2 * sizeof(float));
  return w;
}

// Layout a launch indexes: dense over (sequence, kv head, partition < max_parts); none when every
// context fits one partition.
DecodeWs decode_ws_layout(int32_t S, int32_t hq, int32_t hkv, int32_t head_dim, int max_parts) {
  if (max_parts <= 1) return DecodeWs{0, 0, 0};
  return decode_ws_items((size_t)S * hkv * max_parts, hq / hkv, head_dim);
}

// Workspace bytes that cover every call at the automatic partition size with at most S sequences
// and a max_context_len of at most max_ctx (same heads and pool). A call whose partition was not
// halved has max(1, ceil(ctx / largest partition)) partitions, which grows with both arguments. A
// call whose partition was halved has fewer than 2 * kMinWorkgroups (sequence, kv head, partition)
// triples, since one halving at most doubles a count that was below kMinWorkgroups, and its
// partitions are at least kMinAutoPartition tokens long.
size_t decode_ws_auto_bound(int32_t S, int32_t hq, int32_t hkv, int32_t head_dim, int dt, int32_t max_ctx) {
  const int g = hq / hkv;
  const int cap = auto_cap(g, dt, head_dim);
  const int64_t ctx = max_ctx;
  size_t whole = 0;
  if (ctx > cap) whole = decode_ws_layout(S, hq, hkv, head_dim, (int)((ctx + cap - 1) / cap)).total;
  size_t halved = 0;
  if (ctx > kMinAutoPartition) {
    const int64_t most = (int64_t)S * hkv * ((ctx + kMinAutoPartition - 1) / kMinAutoPartition);
    halved = decode_ws_items((size_t)std::min<int64_t>(2 * kMinWorkgroups - 1, most), g, head_dim).total;
  }
  return std::max(whole, halved);
}

// HIP status of the most recent kernel launch made by an entry point on this thread.
thread_local hipError_t g_last_launch = hipSuccess;

int32_t launched(hipError_t e) {
  g_last_launch = e;
  return e == hipSuccess ? PKV_OK : PKV_ELAUNCH;
}

}  // namespace

namespace pkv {
void set_last_launch_error(hipError_t e) { g_last_launch = e; }
}  // namespace pkv

extern "C" {

const char* pkv_last_launch_error(void) { return hipGetErrorName(g_last_launch); }

int32_t pkv_debug_checks_enabled(void) { return pkv::kDebugChecks ? 1 : 0; }

int32_t pkv_debug_flags(uint32_t* flags, int32_t clear) {
  if (!flags) return PKV_EINVAL;
  uint32_t w[3][pkv::DBG_WORDS];
  if (pkv::debug_words_cache_ops(w[0], clear != 0) || pkv::debug_words_decode(w[1], clear != 0) ||
      pkv::debug_words_ragged(w[2], clear != 0))
    return PKV_ELAUNCH;
  uint32_t bits = 0;
  for (int u = 0; u < 3; ++u)
    for (int i = 0; i < pkv::DBG_WORDS; ++i)
      if (w[u][i]) bits |= 1u << i;
  *flags = bits;
  return PKV_OK;
}

const char* pkv_status_str(int32_t s) {
  switch (s) {
    case PKV_OK: return "ok";
    case PKV_EINVAL: return "invalid argument";
    case PKV_EDTYPE: return "unsupported dtype";
    case PKV_ESHAPE: return "unsupported shape";
    case PKV_EWORKSPACE: return "workspace missing or too small";
    case PKV_ELAUNCH: return "kernel launch failed";
    case PKV_ENOBLOCKS: return "no free blocks";
    case PKV_ENOSEQ: return "unknown sequence";
    case PKV_EEXIST: return "sequence exists";
    case PKV_ENOTRESIDENT: return "sequence not in the required pool (swapped out or resident)";
  }
  return "unknown status";
}

const char* pkv_version(void) { return "pagedkv 0.1 gfx950"; }

int32_t pkv_kv_cache_write(const void* k, const void* v, void* k_cache, void* v_cache,
                           const int32_t* slot_mapping, int32_t num_tokens, int64_t k_token_stride,
                           int64_t v_token_stride, const pkv_cache_desc* c, void* stream) {
  int32_t st = check_cache(c);
  if (st != PKV_OK) return st;
  if (num_tokens < 0) return PKV_EINVAL;
  if (num_tokens == 0) return PKV_OK;
  if (!k || !v || !k_cache || !v_cache || !slot_mapping) return PKV_EINVAL;
  const int64_t row = (int64_t)c->num_kv_heads * c->head_dim;
  if (k_token_stride < row || v_token_stride < row || k_token_stride % 8 || v_token_stride % 8)
    return PKV_EINVAL;
  const int es = elem_bytes(c->dtype);
  // 16-byte chunks are counted in 32 bits, with room for the launch's last group of 256 x 8
  if ((uint64_t)num_tokens * c->num_kv_heads * (c->head_dim * es / 16) > 0xffffffffull - 2048) return PKV_ESHAPE;
  return launched(pkv::launch_kv_cache_write(k, v, k_cache, v_cache, slot_mapping, num_tokens,
                                             k_token_stride * es, v_token_stride * es, c->num_kv_heads,
                                             c->block_size, c->head_dim, es, c->num_blocks, (hipStream_t)stream));
}

int32_t pkv_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int32_t num_pairs,
                        const pkv_cache_desc* c, void* stream) {
  int32_t st = check_cache(c);
  if (st != PKV_OK) return st;
  if (num_pairs < 0) return PKV_EINVAL;
  if (num_pairs == 0) return PKV_OK;
  if (!k_cache || !v_cache || !pairs) return PKV_EINVAL;
  const int64_t block_bytes = (int64_t)c->num_kv_heads * c->block_size * c->head_dim * elem_bytes(c->dtype);
  return launched(
      pkv::launch_copy_blocks(k_cache, v_cache, pairs, num_pairs, block_bytes, c->num_blocks, (hipStream_t)stream));
}

int32_t pkv_swap_blocks(void* dst_k, void* dst_v, const void* src_k, const void* src_v, const int32_t* pairs,
                        int32_t num_pairs, const pkv_cache_desc* c, void* stream) {
  int32_t st = check_cache(c);
  if (st != PKV_OK) return st;
  if (num_pairs < 0) return PKV_EINVAL;
  if (num_pairs == 0) return PKV_OK;
  if (!dst_k || !dst_v || !src_k || !src_v || !pairs) return PKV_EINVAL;
  const int64_t block_bytes = (int64_t)c->num_kv_heads * c->block_size * c->head_dim * elem_bytes(c->dtype);
  return launched(
      pkv::launch_copy_between(dst_k, dst_v, src_k, src_v, pairs, num_pairs, block_bytes, 0, 0, (hipStream_t)stream));
}

int32_t pkv_decode_max_partition(int32_t num_q_heads, const pkv_cache_desc* c) {
  if (check_cache(c) != PKV_OK || check_heads(num_q_heads, c) != PKV_OK) return PKV_EINVAL;
  return pkv::max_partition(num_q_heads / c->num_kv_heads, c->dtype, c->head_dim);
}

int32_t pkv_decode_partition_size(int32_t num_seqs, int32_t num_q_heads, int32_t max_ctx,
                                  const pkv_cache_desc* c) {
  if (check_cache(c) != PKV_OK || check_heads(num_q_heads, c) != PKV_OK || max_ctx < 0 || num_seqs < 0)
    return PKV_EINVAL;
  // a multiple of 64, hence of every block size
  return auto_partition(num_seqs, c->num_kv_heads, num_q_heads / c->num_kv_heads, c->dtype, c->head_dim, max_ctx);
}

size_t pkv_decode_workspace_bytes_ex(int32_t S, int32_t hq, int32_t max_ctx, const pkv_cache_desc* c,
                                     int32_t partition) {
  if (check_cache(c) != PKV_OK || check_heads(hq, c) != PKV_OK || S < 0 || max_ctx < 0) return 0;
  if (partition <= 0) return S > 0 ? decode_ws_auto_bound(S, hq, c->num_kv_heads, c->head_dim, c->dtype, max_ctx) : 0;
  if (!valid_partition(partition, c->block_size, hq / c->num_kv_heads, c->dtype, c->head_dim)) return 0;
  const int max_parts = max_ctx > 0 ? (max_ctx + partition - 1) / partition : 1;
  return decode_ws_layout(S, hq, c->num_kv_heads, c->head_dim, max_parts).total;
}

size_t pkv_decode_workspace_bytes(int32_t S, int32_t hq, int32_t max_ctx, const pkv_cache_desc* c) {
  return pkv_decode_workspace_bytes_ex(S, hq, max_ctx, c, 0);
}

static int32_t decode_common_cu(void* out, int32_t out_dtype, const void* q, const void* k_cache,
                                const void* v_cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                                const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads, float scale,
                                int32_t max_context_len, const pkv_cache_desc* c, int32_t partition_size,
                                void* workspace, size_t workspace_bytes, void* stream, const int32_t* cu,
                                int stage = 0, int32_t num_rows = -1, const int32_t* items = nullptr,
                                int32_t num_items = 0, bool causal_rows = false, const void* k_new = nullptr,
                                const void* v_new = nullptr, const int32_t* new_slots = nullptr) {
  int32_t st = check_cache(c);
  if (st != PKV_OK) return st;
  if ((st = check_heads(num_q_heads, c)) != PKV_OK) return st;
  if ((st = check_out_dtype(out_dtype, c)) != PKV_OK) return st;
  if (num_seqs < 0 || max_context_len < 0 || max_blocks_per_seq < 0) return PKV_EINVAL;
  if (num_seqs == 0) return PKV_OK;
  if (num_seqs > 65535) return PKV_ESHAPE;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens) return PKV_EINVAL;
  if ((int64_t)max_blocks_per_seq * c->block_size < max_context_len) return PKV_EINVAL;
  if (!(scale > 0.f) || !(scale < INFINITY)) return PKV_EINVAL;  // a positive, finite multiplier
  // Items of the launch: sequences, or in causal-rows mode the query rows of a ragged batch.
  if (causal_rows && (!cu || num_rows < 1)) return PKV_EINVAL;
  if (causal_rows && num_rows > 65535) return PKV_ESHAPE;
  const int32_t n_items = causal_rows ? num_rows : num_seqs;
  const int p = partition_size > 0 ? partition_size
                                   : pkv_decode_partition_size(n_items, num_q_heads, max_context_len, c);
  if (!valid_partition(p, c->block_size, num_q_heads / c->num_kv_heads, c->dtype, c->head_dim)) return PKV_EINVAL;
  const int max_parts = max_context_len > 0 ? (max_context_len + p - 1) / p : 1;
  if (max_parts > 65535) return PKV_ESHAPE;
  const DecodeWs ws = decode_ws_layout(n_items, num_q_heads, c->num_kv_heads, c->head_dim, max_parts);
  if (ws.total > 0 && (!workspace || workspace_bytes < ws.total || (uintptr_t)workspace % 16)) return PKV_EWORKSPACE;

  pkv::DecodeLaunch L;
  L.out = out;
  L.out_dt = out_dtype;
  L.q = q;
  L.kc = k_cache;
  L.vc = v_cache;
  L.tables = block_tables;
  L.max_blocks = max_blocks_per_seq;
  L.ctx_lens = context_lens;
  L.num_seqs = num_seqs;
  L.num_q_heads = num_q_heads;
  L.num_kv_heads = c->num_kv_heads;
  L.block_size = c->block_size;
  L.head_dim = c->head_dim;
  L.dt = c->dtype;
  L.scale = scale;
  L.partition = p;
  L.max_parts = max_parts;
  char* wb = static_cast<char*>(workspace);
  L.ws_acc = ws.total ? reinterpret_cast<float*>(wb + ws.acc) : nullptr;
  L.ws_ml = ws.total ? reinterpret_cast<float*>(wb + ws.ml) : nullptr;
  L.stage = stage;
  L.cu = cu;
  L.num_blocks = c->num_blocks;
  L.num_rows = num_rows >= 0 ? num_rows : num_seqs;
  L.items = items;
  L.num_items = num_items;
  L.causal_rows = causal_rows ? 1 : 0;
  L.k_new = k_new;
  L.v_new = v_new;
  L.new_slots = new_slots;
  return launched(pkv::launch_decode(L, (hipStream_t)stream));
}

static int32_t decode_common(void* out, int32_t out_dtype, const void* q, const void* k_cache,
                             const void* v_cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                             const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads, float scale,
                             int32_t max_context_len, const pkv_cache_desc* c, int32_t partition_size,
                             void* workspace, size_t workspace_bytes, void* stream, int stage) {
  return decode_common_cu(out, out_dtype, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                          num_seqs, num_q_heads, scale, max_context_len, c, partition_size, workspace,
                          workspace_bytes, stream, nullptr, stage);
}

int32_t pkv_paged_attention_decode_ex(void* out, int32_t out_dtype, const void* q, const void* k_cache,
                                      const void* v_cache, const int32_t* block_tables,
                                      int32_t max_blocks_per_seq, const int32_t* context_lens,
                                      int32_t num_seqs, int32_t num_q_heads, float scale,
                                      int32_t max_context_len, const pkv_cache_desc* c,
                                      int32_t partition_size, void* workspace, size_t workspace_bytes,
                                      void* stream) {
  return decode_common(out, out_dtype, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                       num_seqs, num_q_heads, scale, max_context_len, c, partition_size, workspace,
                       workspace_bytes, stream, 0);
}

int32_t pkv_paged_attention_decode_partitions(void* out, int32_t out_dtype, const void* q, const void* k_cache,
                                              const void* v_cache, const int32_t* block_tables,
                                              int32_t max_blocks_per_seq, const int32_t* context_lens,
                                              int32_t num_seqs, int32_t num_q_heads, float scale,
                                              int32_t max_context_len, const pkv_cache_desc* c,
                                              int32_t partition_size, void* workspace, size_t workspace_bytes,
                                              void* stream) {
  return decode_common(out, out_dtype, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                       num_seqs, num_q_heads, scale, max_context_len, c, partition_size, workspace,
                       workspace_bytes, stream, 1);
}

int32_t pkv_paged_attention_decode_partitions_items(void* out, int32_t out_dtype, const void* q,
                                                    const void* k_cache, const void* v_cache,
                                                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                                                    const int32_t* context_lens, int32_t num_seqs,
                                                    int32_t num_q_heads, float scale, int32_t max_context_len,
                                                    const pkv_cache_desc* c, int32_t partition_size,
                                                    const int32_t* items, int32_t num_items, void* workspace,
                                                    size_t workspace_bytes, void* stream) {
  if (partition_size <= 0 || num_items < 0 || (num_items > 0 && !items)) return PKV_EINVAL;
  if (c && (int64_t)num_items * (c->num_kv_heads > 0 ? c->num_kv_heads : 1) > 0x7fffffffLL) return PKV_ESHAPE;
  if (num_seqs > 65535) return PKV_ESHAPE;  // items carry 16-bit sequence indices; merge grid limit
  if (num_items == 0 && num_seqs > 0) {
    // Nothing to launch; still report argument errors like the other entry points.
    return decode_common_cu(out, out_dtype, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                            0, num_q_heads, scale, max_context_len, c, partition_size, workspace, workspace_bytes,
                            stream, nullptr, 1);
  }
  return decode_common_cu(out, out_dtype, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                          num_seqs, num_q_heads, scale, max_context_len, c, partition_size, workspace,
                          workspace_bytes, stream, nullptr, 1, -1, items, num_items);
}

int32_t pkv_paged_attention_decode_append(void* out, int32_t out_dtype, const void* q, const void* k_new,
                                          const void* v_new, const int32_t* slot_mapping, void* k_cache,
                                          void* v_cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                                          const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                                          float scale, int32_t max_context_len, const pkv_cache_desc* c,
                                          int32_t partition_size, const int32_t* items, int32_t num_items,
                                          void* workspace, size_t workspace_bytes, void* stream) {
  if (num_seqs > 0 && (!k_new || !v_new || !slot_mapping)) return PKV_EINVAL;
  if (items) {
    // work list: partitions of the listed items (with the stores), then the merge
    if (partition_size <= 0 || num_items < 0 || (num_seqs > 0 && num_items == 0)) return PKV_EINVAL;
    if (c && (int64_t)num_items * (c->num_kv_heads > 0 ? c->num_kv_heads : 1) > 0x7fffffffLL) return PKV_ESHAPE;
    if (num_seqs > 65535) return PKV_ESHAPE;
    int32_t st = decode_common_cu(out, out_dtype, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                                  num_items > 0 ? num_seqs : 0, num_q_heads, scale, max_context_len, c,
                                  partition_size, workspace, workspace_bytes, stream, nullptr, 1, -1, items,
                                  num_items, false, k_new, v_new, slot_mapping);
    if (st != PKV_OK) return st;
    return decode_common(out, out_dtype, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                         num_seqs, num_q_heads, scale, max_context_len, c, partition_size, workspace,
                         workspace_bytes, stream, 2);
  }
  if (num_items != 0) return PKV_EINVAL;
  return decode_common_cu(out, out_dtype, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                          num_seqs, num_q_heads, scale, max_context_len, c, partition_size, workspace,
                          workspace_bytes, stream, nullptr, 0, -1, nullptr, 0, false, k_new, v_new, slot_mapping);
}

int32_t pkv_decode_items(const int32_t* context_lens, int32_t num_seqs, int32_t partition_size, int32_t* items,
                         int32_t capacity) {
  if (!context_lens || num_seqs < 0 || partition_size <= 0 || partition_size % 64 || capacity < 0) return PKV_EINVAL;
  if (num_seqs > 65535) return PKV_ESHAPE;
  int64_t total = 0;
  int32_t max_parts = 0;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int32_t ctx = context_lens[s];
    const int32_t n = ctx > 0 ? (int32_t)(((int64_t)ctx + partition_size - 1) / partition_size) : 1;
    total += n;
    if (n > max_parts) max_parts = n;
  }
  if (max_parts > 65536 || total > 0x7fffffff) return PKV_ESHAPE;
  if (!items) return (int32_t)total;  // size query
  if (total > capacity) return PKV_EINVAL;
  int32_t k = 0;
  for (int32_t p = max_parts - 1; p >= 0; --p) {  // last partitions first, then sequence order
    for (int32_t s = 0; s < num_seqs; ++s) {
      const int32_t ctx = context_lens[s];
      const int32_t n = ctx > 0 ? (int32_t)(((int64_t)ctx + partition_size - 1) / partition_size) : 1;
      if (p < n) items[k++] = (int32_t)((uint32_t)s | ((uint32_t)p << 16));
    }
  }
  // Longest items first (ties keep the order above), so that the launch's tail holds the shortest
  // ones; an item's length is the token count of its partition as the kernel splits the context.
  // A counting sort on that length, stable by construction (a comparison sort when lengths
  // exceed 65536 tokens, to bound the buckets).
  auto tokens = [&](int32_t it) {
    const int32_t s = it & 0xffff, p = (int32_t)((uint32_t)it >> 16);
    const int32_t ctx = context_lens[s];
    if (ctx <= 0) return 0;
    const int32_t n = (int32_t)(((int64_t)ctx + partition_size - 1) / partition_size);
    const int32_t psz = std::min(partition_size, (((ctx + n - 1) / n) + 63) & ~63);
    return std::max(0, std::min(psz, ctx - p * psz));
  };
  thread_local std::vector<int32_t> keys, order, start;
  keys.resize(k);
  order.resize(k);
  int32_t longest = 0;
  for (int32_t i = 0; i < k; ++i) {
    keys[i] = tokens(items[i]);
    longest = std::max(longest, keys[i]);
  }
  if (longest > 65536) {
    for (int32_t i = 0; i < k; ++i) order[i] = i;
    std::stable_sort(order.begin(), order.end(), [&](int32_t x, int32_t y) { return keys[x] > keys[y]; });
    for (int32_t i = 0; i < k; ++i) order[i] = items[order[i]];
  } else {
    start.assign(longest + 2, 0);
    for (int32_t i = 0; i < k; ++i) ++start[longest - keys[i] + 1];  // ascending key = descending length
    for (int32_t v = 0; v <= longest; ++v) start[v + 1] += start[v];
    for (int32_t i = 0; i < k; ++i) order[start[longest - keys[i]]++] = items[i];
  }
  std::copy(order.begin(), order.end(), items);
  return k;
}

int32_t pkv_paged_attention_decode_merge(void* out, int32_t out_dtype, const void* q, const void* k_cache,
                                         const void* v_cache, const int32_t* block_tables,
                                         int32_t max_blocks_per_seq, const int32_t* context_lens,
                                         int32_t num_seqs, int32_t num_q_heads, float scale,
                                         int32_t max_context_len, const pkv_cache_desc* c,
                                         int32_t partition_size, void* workspace, size_t workspace_bytes,
                                         void* stream) {
  return decode_common(out, out_dtype, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                       num_seqs, num_q_heads, scale, max_context_len, c, partition_size, workspace,
                       workspace_bytes, stream, 2);
}

// Whether a ragged call runs every query row through the decode kernels (causal-rows mode): an
// fp32 pool with prefill rows (the prefill kernel is 16-bit MFMA), or short chunks only. The
// prefill kernel works per query head and so reads each kv head's keys and values g times; the
// decode kernels read them once per query row, so with max_q_len <= g they read no more (measured
// at g = 4: 188 against 424 us for 2-row chunks, 315 against 432 us for 4, 523 against 433 us for
// 8). Requires a valid cache and head count.
static bool ragged_rows_mode(int32_t num_tokens, int32_t num_q_heads, int32_t max_q_len, const pkv_cache_desc* c) {
  if (max_q_len <= 1) return false;
  if (c->dtype == PKV_F32) return true;
  return max_q_len <= num_q_heads / c->num_kv_heads && num_tokens <= 65535;
}

size_t pkv_ragged_workspace_bytes(int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads, int32_t max_q_len,
                                  int32_t max_context_len, const pkv_cache_desc* c) {
  if (check_cache(c) != PKV_OK || check_heads(num_q_heads, c) != PKV_OK) return 0;
  // one item per query row in causal-rows mode, else per sequence
  const int32_t items = ragged_rows_mode(num_tokens, num_q_heads, max_q_len, c) ? num_tokens : num_seqs;
  return pkv_decode_workspace_bytes_ex(items, num_q_heads, max_context_len, c, 0);
}

// The ragged step; decode rows through the dense partition grid (items == nullptr, partition_size
// 0: automatic) or through the caller's work list at partition_size.
static int32_t ragged_common(void* out, int32_t out_dtype, const void* q, const int32_t* cu_seqlens_q,
                             const int32_t* context_lens, const void* k_cache, const void* v_cache,
                             const int32_t* block_tables, int32_t max_blocks_per_seq, int32_t num_seqs,
                             int32_t num_tokens, int32_t num_q_heads, float scale, int32_t min_q_len,
                             int32_t max_q_len, int32_t max_context_len, const pkv_cache_desc* c,
                             int32_t partition_size, const int32_t* items, int32_t num_items, void* workspace,
                             size_t workspace_bytes, void* stream) {
  int32_t st = check_cache(c);
  if (st != PKV_OK) return st;
  if ((st = check_heads(num_q_heads, c)) != PKV_OK) return st;
  if ((st = check_out_dtype(out_dtype, c)) != PKV_OK) return st;
  if (num_seqs < 0 || num_tokens < 0 || max_q_len < 0 || max_context_len < 0 || max_blocks_per_seq < 0)
    return PKV_EINVAL;
  if (num_seqs == 0 || num_tokens == 0) return PKV_OK;
  if (max_q_len > max_context_len || max_q_len > num_tokens) return PKV_EINVAL;
  if (min_q_len < 1 || (min_q_len > 1 && min_q_len > max_q_len)) return PKV_EINVAL;
  if (!out || !q || !cu_seqlens_q || !context_lens || !k_cache || !v_cache || !block_tables) return PKV_EINVAL;
  // Every row through the decode kernels, one item per query row attending keys up to its own
  // position (fp32 throughout), when ragged_rows_mode says so; else decode rows there and
  // prefill chunks on the MFMA kernel.
  if (ragged_rows_mode(num_tokens, num_q_heads, max_q_len, c))
    return decode_common_cu(out, out_dtype, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                            num_seqs, num_q_heads, scale, max_context_len, c, 0, workspace, workspace_bytes, stream,
                            cu_seqlens_q, 0, num_tokens, nullptr, 0, true);
  // Decode rows (q_len == 1) through the decode kernels with row indirection, unless the caller
  // states that no sequence has a single row: then the two decode launches are skipped and any
  // single-row sequence there is after all gets a row tile of the prefill kernel.
  const bool decode_rows = min_q_len == 1;
  if (decode_rows) {
    st = decode_common_cu(out, out_dtype, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                          num_seqs, num_q_heads, scale, max_context_len, c, partition_size, workspace,
                          workspace_bytes, stream, cu_seqlens_q, 0, num_tokens, items, num_items);
    if (st != PKV_OK || max_q_len <= 1) return st;
  }
  pkv::PrefillLaunch P;
  P.out = out;
  P.out_dt = out_dtype;
  P.q = q;
  P.kc = k_cache;
  P.vc = v_cache;
  P.tables = block_tables;
  P.max_blocks = max_blocks_per_seq;
  P.cu = cu_seqlens_q;
  P.ctx_lens = context_lens;
  P.num_seqs = num_seqs;
  P.num_tokens = num_tokens;
  P.num_q_heads = num_q_heads;
  P.num_kv_heads = c->num_kv_heads;
  P.block_size = c->block_size;
  P.head_dim = c->head_dim;
  P.dt = c->dtype;
  P.scale = scale;
  P.num_blocks = c->num_blocks;
  P.min_rows = decode_rows ? 2 : 1;
  return launched(pkv::launch_ragged_prefill(P, (hipStream_t)stream));
}

int32_t pkv_paged_attention_ragged_ex(void* out, int32_t out_dtype, const void* q, const int32_t* cu_seqlens_q,
                                      const int32_t* context_lens, const void* k_cache, const void* v_cache,
                                      const int32_t* block_tables, int32_t max_blocks_per_seq, int32_t num_seqs,
                                      int32_t num_tokens, int32_t num_q_heads, float scale, int32_t min_q_len,
                                      int32_t max_q_len, int32_t max_context_len, const pkv_cache_desc* c,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  return ragged_common(out, out_dtype, q, cu_seqlens_q, context_lens, k_cache, v_cache, block_tables,
                       max_blocks_per_seq, num_seqs, num_tokens, num_q_heads, scale, min_q_len, max_q_len,
                       max_context_len, c, 0, nullptr, 0, workspace, workspace_bytes, stream);
}

int32_t pkv_paged_attention_ragged_items(void* out, int32_t out_dtype, const void* q, const int32_t* cu_seqlens_q,
                                         const int32_t* context_lens, const void* k_cache, const void* v_cache,
                                         const int32_t* block_tables, int32_t max_blocks_per_seq, int32_t num_seqs,
                                         int32_t num_tokens, int32_t num_q_heads, float scale, int32_t min_q_len,
                                         int32_t max_q_len, int32_t max_context_len, const pkv_cache_desc* c,
                                         int32_t partition_size, const int32_t* items, int32_t num_items,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  if (partition_size <= 0 || num_items < 0 || (num_items > 0 && !items)) return PKV_EINVAL;
  return ragged_common(out, out_dtype, q, cu_seqlens_q, context_lens, k_cache, v_cache, block_tables,
                       max_blocks_per_seq, num_seqs, num_tokens, num_q_heads, scale, min_q_len, max_q_len,
                       max_context_len, c, partition_size, items, num_items, workspace, workspace_bytes, stream);
}

int32_t pkv_paged_attention_ragged(void* out, int32_t out_dtype, const void* q, const int32_t* cu_seqlens_q,
                                   const int32_t* context_lens, const void* k_cache, const void* v_cache,
                                   const int32_t* block_tables, int32_t max_blocks_per_seq, int32_t num_seqs,
                                   int32_t num_tokens, int32_t num_q_heads, float scale, int32_t max_q_len,
                                   int32_t max_context_len, const pkv_cache_desc* c, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  return pkv_paged_attention_ragged_ex(out, out_dtype, q, cu_seqlens_q, context_lens, k_cache, v_cache, block_tables,
                                       max_blocks_per_seq, num_seqs, num_tokens, num_q_heads, scale,
                                       1, max_q_len, max_context_len, c, workspace,
                                       workspace_bytes, stream);
}

int32_t pkv_paged_attention_decode(void* out, int32_t out_dtype, const void* q, const void* k_cache,
                                   const void* v_cache, const int32_t* block_tables,
                                   int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                                   int32_t num_q_heads, float scale, int32_t max_context_len,
                                   const pkv_cache_desc* c, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  return decode_common(out, out_dtype, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                       num_seqs, num_q_heads, scale, max_context_len, c, 0, workspace, workspace_bytes, stream, 0);
}

}  // extern "C"
