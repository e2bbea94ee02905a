/*
 * pagedkv.h — C ABI of libpagedkv.so, paged-KV attention for AMD MI355X (gfx950).
 *
 * What the library computes (sources are the pages' titles and sections):
 *   - The KV cache is cut into fixed-size blocks of B token slots that live anywhere in a
 *     shared pool and are found through a per-sequence block table
 *     (「PagedAttention原理」 §从虚拟内存的启发, §实现一个虚拟内存).
 *   - Attention of a query row over its sequence's cached keys and values,
 *     o = softmax(scale · q Kᵀ) V, computed block by block
 *     (「PagedAttention原理」 §为什么会有 KV cache and the block-wise equation for A_ij and o_i
 *     in §实现一个虚拟内存).
 *   - Reference-counted copy-on-write of shared blocks (「PagedAttention原理」 §解决COW).
 *   - A ragged batch that mixes prefill chunks and decode rows, split per request only inside
 *     attention (「Paged Attention&Orca Paper笔记与解读」 §Orca的Solution, selective batching).
 *
 * Conventions for every entry point
 *   - Pointers documented as "device" are HIP device memory owned by the caller; the library
 *     never allocates, frees or retains device memory. "host" pointers are ordinary CPU memory.
 *   - Device work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the default
 *     stream). The return value only reports host-side validation and the launches themselves.
 *     After a validation error nothing has been enqueued. PKV_ELAUNCH means one launch failed;
 *     in an entry point that issues several (decode partitions then merge, ragged decode rows
 *     then prefill rows) the launches before it stay enqueued and their results are incomplete.
 *   - Device-resident indices (block ids, slots, lengths) are trusted: the caller guarantees
 *     they are in range. Host-visible scalars and shapes are validated.
 *   - Ordering between calls is the caller's job: on one stream, copy_blocks for an append's
 *     copy-on-write pairs, then kv_cache_write of the new tokens, then attention.
 *   - All integers are int32 unless stated; a pool may hold at most 2^31-1 slots.
 *
 * KV pool layout (the contract tests decode independently)
 *   K and V are two separate pools per layer with identical shape. With N = num_blocks,
 *   H = num_kv_heads, B = block_size, D = head_dim, the element for (block b, kv head h,
 *   slot o within the block, dim i) is at linear element index
 *         ((b * H + h) * B + o) * D + i
 *   i.e. [N][H][B][D], "head-major": one (block, kv head) tile of B×D elements is contiguous
 *   and a whole block (all heads) is one contiguous region of H·B·D elements.
 *   A slot number s addresses block s / B, offset s % B.
 *
 * Supported shapes: dtype f32 / f16 / bf16; B in {8, 16, 32}; D in {64, 128};
 * num_q_heads / num_kv_heads in {1, 2, 4, 8}.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { PKV_F32 = 0, PKV_F16 = 1, PKV_BF16 = 2 } pkv_dtype;

typedef enum {
  PKV_OK = 0,
  PKV_EINVAL = -1,      /* null pointer or out-of-range scalar argument */
  PKV_EDTYPE = -2,      /* unsupported element type (or out dtype)       */
  PKV_ESHAPE = -3,      /* unsupported block size, head dim or head ratio */
  PKV_EWORKSPACE = -4,  /* workspace missing, smaller than required or not 16-byte aligned */
  PKV_ELAUNCH = -5,     /* the HIP launch itself failed                   */
  PKV_ENOBLOCKS = -6,   /* block manager: pool exhausted (nothing changed) */
  PKV_ENOSEQ = -7,      /* block manager: unknown sequence id             */
  PKV_EEXIST = -8,      /* block manager: sequence id already present     */
  PKV_ENOTRESIDENT = -9 /* block manager: sequence is (or is not) swapped out as required */
} pkv_status;

/* Shape of one layer's K and V pools. */
typedef struct {
  int32_t num_blocks;
  int32_t block_size;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t dtype; /* a pkv_dtype */
} pkv_cache_desc;

/* Human-readable name of a status code (static storage). */
const char* pkv_status_str(int32_t status);

/* Library version string (static storage). */
const char* pkv_version(void);

/* Name of the HIP status ("hipSuccess", "hipErrorInvalidConfiguration", ...) of the most recent
 * kernel launch made by a device entry point on the calling thread; static storage. After an
 * entry point returns PKV_ELAUNCH it names the launch's own error, not one left behind by an
 * unrelated HIP call. */
const char* pkv_last_launch_error(void);

/*
 * Debug builds. Device-resident indices (slots, block-table entries, copy pairs, ragged row
 * offsets) are trusted by the release library. libpagedkv_debug.so, the same sources compiled
 * with PKV_DEBUG_CHECKS, checks each one in the kernel before using it:
 *   - a slot >= num_blocks * block_size is skipped                      (flag bit 0, PKV_DBG_SLOT)
 *   - a block-table entry outside [0, num_blocks) is read as block 0     (bit 1, PKV_DBG_BLOCK)
 *   - ragged row offsets that are negative, decreasing or past num_tokens make that sequence
 *     empty (and a decode row outside the batch is skipped)              (bit 2, PKV_DBG_RAGGED)
 *   - a copy pair with a negative index, or (copy_blocks) one >= num_blocks, is skipped;
 *     pkv_swap_blocks checks non-negativity only, as it does not know the host pool's size
 *                                                                        (bit 3, PKV_DBG_PAIR)
 * so a bad index yields wrong values instead of an out-of-bounds access. Results are otherwise
 * identical to the release build.
 *
 * pkv_debug_checks_enabled: 1 in a debug build, 0 in a release build.
 * pkv_debug_flags: waits for all work on the current device, writes the OR of the flag bits raised
 *   on it since the last clear into *flags, and clears them if clear != 0. Always 0 in a release
 *   build. Returns PKV_EINVAL for a null flags pointer, PKV_ELAUNCH if a HIP call fails.
 */
enum { PKV_DBG_SLOT = 1, PKV_DBG_BLOCK = 2, PKV_DBG_RAGGED = 4, PKV_DBG_PAIR = 8 };
int32_t pkv_debug_checks_enabled(void);
int32_t pkv_debug_flags(uint32_t* flags, int32_t clear);

/*
 * kv_cache_write — store new tokens' keys and values into their slots.
 *   k_cache[slot[t]] <- k[t], v_cache[slot[t]] <- v[t] for t < num_tokens, bit for bit.
 *   Each decode step stores the new token's K/V; a prefill stores the whole prompt's
 *   (「vllm」 §2.1 Prefill, §2.2 Decode).
 *   k, v        device, [num_tokens][H][D] rows in the pool dtype; row t starts at element
 *               t * k_token_stride (resp. v_token_stride); strides >= H*D, multiples of 8.
 *   k_cache, v_cache  device pools (layout above).
 *   slot_mapping      device int32 [num_tokens]; a negative slot means "skip this token".
 *   Two tokens must not name the same slot in one call.
 *   num_tokens == 0 is a no-op.
 */
int32_t pkv_kv_cache_write(const void* k, const void* v, void* k_cache, void* v_cache,
                           const int32_t* slot_mapping, int32_t num_tokens,
                           int64_t k_token_stride, int64_t v_token_stride,
                           const pkv_cache_desc* cache, void* stream);

/*
 * copy_blocks — step (2) of copy-on-write: copy each shared block into its new block
 *   (「PagedAttention原理」 §解决COW). For each pair i: the whole block dst_i <- block src_i,
 *   all B slots, all kv heads, K and V pools, bit for bit.
 *   block_pairs  device int32 [num_pairs][2] = (src, dst).
 *   No block may appear both as a source and as a destination in one call, and destinations
 *   must be distinct (the block manager's pair lists satisfy this). num_pairs == 0 is a no-op.
 */
int32_t pkv_copy_blocks(void* k_cache, void* v_cache, const int32_t* block_pairs,
                        int32_t num_pairs, const pkv_cache_desc* cache, void* stream);

/*
 * Workspace of the decode attention: per-partition partial results (running max, sum and
 * unnormalised output, fp32) of sequences whose context spans more than one partition.
 *   Returns bytes enough for a call at the automatic partition size with these arguments and
 *   for every such call with fewer sequences or a smaller max_context_len (same heads and pool),
 *   so one workspace sized for the largest batch serves every step; at most about 1024 (sequence,
 *   kv head, partition) partials beyond what the largest call itself needs. 0 means no such call
 *   needs a workspace (no context longer than 256 tokens, or num_seqs == 0) or the arguments
 *   are invalid. The contents need no initialisation and are scratch between calls; calls that
 *   share a workspace must not run concurrently.
 */
size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len,
                                  const pkv_cache_desc* cache);

/* Largest context partition, in tokens, the decode entry points accept for num_q_heads query
 * heads over this cache (g = num_q_heads / num_kv_heads query heads per kv head). Two kernels
 * serve decode. The one-pass kernel (16-bit pools with g = 8, and with g = 4 at head_dim 64)
 * keeps a running softmax per wave and no scores: 4096 tokens. The three-phase kernel (every other
 * case) keeps a score per token and query head in 32 KiB of LDS: 8192 / g tokens (8192, 4096,
 * 2048, 1024 for g = 1, 2, 4, 8). Returns PKV_EINVAL for an invalid cache or head count. */
int32_t pkv_decode_max_partition(int32_t num_q_heads, const pkv_cache_desc* cache);

/* Tokens per context partition the decode kernel uses for these arguments
 * (partition_size argument 0 of the _ex entry point). It starts from max_context_len rounded up
 * to a multiple of 64 when that fits min(4096, pkv_decode_max_partition), else that size; while
 * num_seqs x num_kv_heads x ceil(max_context_len / partition) is below 512 workgroups (two per
 * CU), it is halved (rounded up to a multiple of 64), down to 256, so a small batch of long
 * contexts still fills the GPU. The workspace and the launch must see the same arguments, since
 * the size depends on all of them. Returns PKV_EINVAL for an invalid cache, head count or
 * negative length or count. */
int32_t pkv_decode_partition_size(int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len,
                                  const pkv_cache_desc* cache);

/*
 * paged_attention_decode — one query row per sequence (the newest token, whose K/V were
 * already written) attending every cached token 0..context_lens[s]-1 of its sequence,
 * reached through its block table (「PagedAttention原理」 §实现一个虚拟内存).
 *   out[s][h][:] = softmax(scale · q[s][h] · K_sᵀ) V_s, K_s/V_s = kv head h / (Hq/Hkv).
 *   out           device [num_seqs][num_q_heads][D], element type out_dtype (PKV_F32 or the
 *                 pool dtype). Accumulation is in fp32.
 *   q             device [num_seqs][num_q_heads][D] in the pool dtype.
 *   block_tables  device int32 [num_seqs][max_blocks_per_seq]; entries past a sequence's
 *                 last block are never read.
 *   context_lens  device int32 [num_seqs], each in [0, max_context_len] and
 *                 <= max_blocks_per_seq * B. A length of 0 gives an all-zero output row. A length
 *                 outside that range is a caller error: the kernels clamp it to stay in bounds,
 *                 so the row is then computed over the clamped context.
 *   max_context_len  host upper bound of context_lens (sizes the split; not a limit check).
 *   scale         multiplier of q·k, positive and finite (1/sqrt(D) for standard attention).
 *   workspace     device, >= pkv_decode_workspace_bytes(...) bytes, 16-byte aligned (may be NULL
 *                 when that is 0).
 *   Long contexts are cut into partitions that are processed independently and merged with
 *   log-sum-exp weights; the result does not depend on which physical blocks hold the data.
 */
int32_t pkv_paged_attention_decode(void* out, int32_t out_dtype, const void* q,
                                   const void* k_cache, const void* v_cache,
                                   const int32_t* block_tables, int32_t max_blocks_per_seq,
                                   const int32_t* context_lens, int32_t num_seqs,
                                   int32_t num_q_heads, float scale, int32_t max_context_len,
                                   const pkv_cache_desc* cache, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* As pkv_paged_attention_decode with an explicit partition size in tokens (0 = automatic;
 * otherwise a multiple of 64 and of the block size, at most pkv_decode_max_partition). The
 * workspace must then be
 * sized with pkv_decode_workspace_bytes_ex. */
int32_t pkv_paged_attention_decode_ex(void* out, int32_t out_dtype, const void* q,
                                      const void* k_cache, const void* v_cache,
                                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                                      const int32_t* context_lens, int32_t num_seqs,
                                      int32_t num_q_heads, float scale, int32_t max_context_len,
                                      const pkv_cache_desc* cache, int32_t partition_size,
                                      void* workspace, size_t workspace_bytes, void* stream);

/* The two launches of pkv_paged_attention_decode_ex, for callers that time or schedule them
 * separately. _partitions processes every (kv head, sequence, partition): sequences whose
 * context fits one partition get their final output rows, the others leave partial results in
 * the workspace. _merge then combines those partials with log-sum-exp weights into their output
 * rows (it launches nothing when no context spans two partitions). Issued in that order on one
 * stream with identical arguments they equal one call of pkv_paged_attention_decode_ex. */
int32_t pkv_paged_attention_decode_partitions(void* out, int32_t out_dtype, const void* q,
                                              const void* k_cache, const void* v_cache,
                                              const int32_t* block_tables, int32_t max_blocks_per_seq,
                                              const int32_t* context_lens, int32_t num_seqs,
                                              int32_t num_q_heads, float scale,
                                              int32_t max_context_len, const pkv_cache_desc* cache,
                                              int32_t partition_size, void* workspace,
                                              size_t workspace_bytes, void* stream);
int32_t pkv_paged_attention_decode_merge(void* out, int32_t out_dtype, const void* q,
                                         const void* k_cache, const void* v_cache,
                                         const int32_t* block_tables, int32_t max_blocks_per_seq,
                                         const int32_t* context_lens, int32_t num_seqs,
                                         int32_t num_q_heads, float scale, int32_t max_context_len,
                                         const pkv_cache_desc* cache, int32_t partition_size,
                                         void* workspace, size_t workspace_bytes, void* stream);

/* Work-list form of pkv_paged_attention_decode_partitions, for callers that know the context
 * lengths on the host (a serving loop's block manager does). items: device int32 [num_items],
 * item = seq | (part << 16), part counted with the given partition_size (> 0, the size the
 * launch uses; see pkv_decode_partition_size). The launch has exactly one workgroup per (kv
 * head, item), so no workgroup is spent on partitions that do not exist, which the dense launch
 * sizes for max_context_len in every sequence. Items are independent, so their order only
 * steers scheduling: pkv_decode_items puts the longest items first. An item whose partition
 * does not exist for the device context length, or whose sequence index is >= num_seqs, does
 * nothing. With every item of every sequence listed, the result equals
 * pkv_paged_attention_decode_partitions, and pkv_paged_attention_decode_merge completes it.
 * num_seqs <= 65535 (as for every decode launch). Errors as pkv_paged_attention_decode_ex;
 * PKV_EINVAL also for partition_size <= 0 or a null items with num_items > 0. */
int32_t pkv_paged_attention_decode_partitions_items(void* out, int32_t out_dtype, const void* q,
                                                    const void* k_cache, const void* v_cache,
                                                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                                                    const int32_t* context_lens, int32_t num_seqs,
                                                    int32_t num_q_heads, float scale,
                                                    int32_t max_context_len, const pkv_cache_desc* cache,
                                                    int32_t partition_size, const int32_t* items,
                                                    int32_t num_items, void* workspace,
                                                    size_t workspace_bytes, void* stream);

/* Host helper (no device work): the decode work list for host context lengths
 * context_lens[0..num_seqs) and a partition size (a positive multiple of 64). Lists every
 * (s, p) with p < ceil(context_lens[s] / partition_size) (p = 0 alone for a length of 0) as
 * s | (p << 16). Longest items first: an item's length is the token count of its partition
 * (a context of n partitions is split into equal parts of ceil(ctx / n) rounded up to a multiple
 * of 64, at most partition_size, the last part taking the rest); ties in descending p, then
 * ascending s. Dispatching the longest partitions first leaves the shortest for the launch's
 * tail. With items == NULL returns the item count; otherwise writes the items (capacity must
 * hold them) and returns their count.
 * PKV_EINVAL for bad arguments or too small a capacity, PKV_ESHAPE beyond 65535 sequences or
 * 65536 partitions of one sequence. */
int32_t pkv_decode_items(const int32_t* context_lens, int32_t num_seqs, int32_t partition_size,
                         int32_t* items, int32_t capacity);

/* Workspace bytes for an explicit partition size: exactly what a call with these arguments
 * needs (which covers any call with fewer sequences or a smaller max_context_len at that
 * partition size); 0 when every context fits one partition or the arguments are invalid.
 * partition_size 0 gives pkv_decode_workspace_bytes. */
size_t pkv_decode_workspace_bytes_ex(int32_t num_seqs, int32_t num_q_heads,
                                     int32_t max_context_len, const pkv_cache_desc* cache,
                                     int32_t partition_size);

/*
 * paged_attention_decode_append — one decode step's cache write and attention in one pass: each
 *   sequence's new token is stored into its slot and then attended with the rest of its context
 *   (a decode step stores its token's K/V and attends over the cache: 「vllm」 §2.2 Decode;
 *   「PagedAttention原理」 §实现一个虚拟内存). Equal, bit for bit in outputs and pools, to
 *   pkv_kv_cache_write(k_new, v_new, ..., slot_mapping, num_seqs, ...) followed by
 *   pkv_paged_attention_decode_ex (items == NULL) or by the work-list partition launch and
 *   pkv_paged_attention_decode_merge (items != NULL), with the same arguments; one launch fewer.
 *   k_new, v_new  device [num_seqs][num_kv_heads][D] in the pool dtype (token stride Hkv·D).
 *   slot_mapping  device int32 [num_seqs]: the slot of position context_lens[s] - 1 of sequence s
 *                 (its newest token); < 0 stores nothing for that sequence. A slot elsewhere
 *                 breaks the contract (the token may be read before it is stored).
 *   k_cache, v_cache  device pools, written (the new rows) and read.
 *   partition_size 0: automatic (items == NULL only); items / num_items: as for
 *                 pkv_paged_attention_decode_partitions_items (every item of every sequence,
 *                 num_items >= 1 when num_seqs > 0), with partition_size > 0.
 *   The other arguments, the workspace and the errors are those of pkv_paged_attention_decode_ex;
 *   PKV_EINVAL also for a null k_new, v_new or slot_mapping with num_seqs > 0. Debug builds skip
 *   and flag a slot past the pool (PKV_DBG_SLOT).
 */
int32_t pkv_paged_attention_decode_append(void* out, int32_t out_dtype, const void* q,
                                          const void* k_new, const void* v_new,
                                          const int32_t* slot_mapping, void* k_cache, void* v_cache,
                                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                                          const int32_t* context_lens, int32_t num_seqs,
                                          int32_t num_q_heads, float scale, int32_t max_context_len,
                                          const pkv_cache_desc* cache, int32_t partition_size,
                                          const int32_t* items, int32_t num_items, void* workspace,
                                          size_t workspace_bytes, void* stream);

/*
 * paged_attention_decode_noalloc — pkv_paged_attention_decode without a caller workspace, for
 *   callers that cannot allocate device memory: code under HIP graph capture, tight serving
 *   loops, harnesses that forbid hipMalloc. Same arguments, layouts and results as
 *   pkv_paged_attention_decode (the same kernels at the same automatic partition size, so the
 *   outputs are bit-identical), minus workspace and workspace_bytes.
 *   The split-context partials go to a file-scope device array of PKV_NOALLOC_SCRATCH_BYTES
 *   bytes inside the library (64 MiB; each GPU the library runs on holds its own copy until the
 *   process ends). Nothing is allocated or freed, on the device or the host.
 *   A call whose partials would need more (pkv_decode_workspace_bytes_ex at the automatic
 *   partition size) returns PKV_EWORKSPACE before any device call; the other validation errors
 *   are those of pkv_paged_attention_decode. The first call on a device looks up that device's
 *   address of the array (PKV_ELAUNCH, with pkv_last_launch_error naming the cause, if the
 *   lookup fails).
 *   Every call on one GPU shares that GPU's array and leaves its partials there: calls that
 *   overlap on one GPU (several streams, or several host threads) race and must be ordered by
 *   the caller. The partials need no initial value, so no clearing is done between calls.
 */
#define PKV_NOALLOC_SCRATCH_BYTES (64u << 20)
int32_t pkv_paged_attention_decode_noalloc(void* out, int32_t out_dtype, const void* q,
                                           const void* k_cache, const void* v_cache,
                                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                                           const int32_t* context_lens, int32_t num_seqs,
                                           int32_t num_q_heads, float scale, int32_t max_context_len,
                                           const pkv_cache_desc* cache, void* stream);

/*
 * paged_attention_ragged — one selective-batching step: a flattened batch of query rows
 * from several sequences, some prefill chunks and some single decode rows
 * (「Paged Attention&Orca Paper笔记与解读」 §Orca的Solution).
 *   Sequence s owns query rows cu_seqlens_q[s] .. cu_seqlens_q[s+1]-1 (q_len_s rows). They
 *   are the last q_len_s positions of its context: row t sits at position
 *   context_lens[s] - q_len_s + t and attends keys 0..that position (causal), all read through
 *   the block table after this step's K/V were written. q_len_s == 1 is a decode row.
 *   out           device [num_tokens][num_q_heads][D], out_dtype PKV_F32 or the pool dtype.
 *   q             device [num_tokens][num_q_heads][D] in the pool dtype.
 *   cu_seqlens_q  device int32 [num_seqs+1], non-decreasing, cu[0] = 0,
 *                 cu[num_seqs] = num_tokens.
 *   context_lens  device int32 [num_seqs], context_lens[s] >= q_len_s.
 *   max_q_len, max_context_len  host upper bounds (launch sizing only).
 *   scale         multiplier of q·k, positive and finite.
 *   Every dtype serves every row. f16/bf16 prefill chunks (q_len > 1) run on MFMA, except when
 *   max_q_len <= num_q_heads / num_kv_heads (and num_tokens <= 65535): then, as always for an
 *   f32 pool with max_q_len > 1, every row runs through the decode kernels in fp32, one query
 *   row per item (an f32 pool's call takes at most 65535 rows, PKV_ESHAPE beyond).
 *   num_seqs is at most 65535 (PKV_ESHAPE beyond); the MFMA prefill launch itself has no row
 *   limit. Every validation error is returned before anything is enqueued.
 *   workspace     device, >= pkv_ragged_workspace_bytes(...) bytes, 16-byte aligned (NULL when
 *                 that is 0);
 *                 scratch between calls, as for decode.
 */
size_t pkv_ragged_workspace_bytes(int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                                  int32_t max_q_len, int32_t max_context_len,
                                  const pkv_cache_desc* cache);

int32_t pkv_paged_attention_ragged(void* out, int32_t out_dtype, const void* q,
                                   const int32_t* cu_seqlens_q, const int32_t* context_lens,
                                   const void* k_cache, const void* v_cache,
                                   const int32_t* block_tables, int32_t max_blocks_per_seq,
                                   int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                                   float scale, int32_t max_q_len, int32_t max_context_len,
                                   const pkv_cache_desc* cache, void* workspace,
                                   size_t workspace_bytes, void* stream);

/*
 * paged_attention_ragged_ex — pkv_paged_attention_ragged with a host lower bound min_q_len on
 *   every sequence's q_len beside the upper bound max_q_len (same step, same layouts). A batch of
 *   prefill chunks only (min_q_len >= 2) needs neither the decode-row launch nor its merge: both
 *   are skipped, and if a sequence has a single row after all it is computed by the prefill
 *   kernel, whose one-row tile attends the same keys, so a wrong bound costs time, not results.
 *   min_q_len == 1 is pkv_paged_attention_ragged exactly (bit-identical outputs). In causal-rows
 *   mode (see above) min_q_len has no effect.
 *   Errors: min_q_len < 1, or min_q_len > 1 and above max_q_len: PKV_EINVAL (nothing enqueued);
 *   otherwise as pkv_paged_attention_ragged. The workspace size is the same.
 */
int32_t pkv_paged_attention_ragged_ex(void* out, int32_t out_dtype, const void* q,
                                      const int32_t* cu_seqlens_q, const int32_t* context_lens,
                                      const void* k_cache, const void* v_cache,
                                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                                      int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                                      float scale, int32_t min_q_len, int32_t max_q_len,
                                      int32_t max_context_len, const pkv_cache_desc* cache,
                                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * paged_attention_ragged_items — pkv_paged_attention_ragged_ex with the decode rows run from a
 *   work list, for callers that know the context lengths on the host (a serving loop's block
 *   manager does; the selective-batching step of 「Paged Attention&Orca Paper笔记与解读」
 *   §Orca的Solution). The decode-row launch then has one workgroup per (kv head, item), in the
 *   items' order, instead of a grid sized for max_context_len in every sequence: with
 *   pkv_decode_items the longest partitions go first and the shortest fill the launch's tail.
 *   partition_size  > 0, the size the items were built with (a multiple of 64 and of the block
 *                 size, at most pkv_decode_max_partition); pkv_decode_partition_size gives the
 *                 automatic one.
 *   items, num_items  device int32 [num_items] as from pkv_decode_items over the host context
 *                 lengths: every partition of every decode-row (q_len == 1) sequence listed once.
 *                 Items of sequences with more than one row do nothing (those rows go to the
 *                 prefill kernel as always), so the list of every sequence serves. An item for
 *                 a partition that does not exist, or for a sequence >= num_seqs, does nothing.
 *                 num_items may be 0 when no sequence has a single row.
 *   workspace     at least pkv_ragged_workspace_bytes(...) and at least
 *                 pkv_decode_workspace_bytes_ex(num_seqs, num_q_heads, max_context_len, cache,
 *                 partition_size) bytes; 16-byte aligned.
 *   With every such item listed and partition_size the automatic size, the outputs equal those
 *   of pkv_paged_attention_ragged_ex bit for bit (the same partitions, merged the same way); at
 *   another size the decode rows are split at that size. In causal-rows mode (see
 *   pkv_paged_attention_ragged) and when min_q_len >= 2 the work list is not used and the call is
 *   pkv_paged_attention_ragged_ex.
 *   Errors: as pkv_paged_attention_ragged_ex; PKV_EINVAL also for partition_size <= 0,
 *   num_items < 0 or a null items with num_items > 0, and, when the work list is used, for a
 *   partition size the decode kernel does not take (all before anything is enqueued).
 */
int32_t pkv_paged_attention_ragged_items(void* out, int32_t out_dtype, const void* q,
                                         const int32_t* cu_seqlens_q, const int32_t* context_lens,
                                         const void* k_cache, const void* v_cache,
                                         const int32_t* block_tables, int32_t max_blocks_per_seq,
                                         int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                                         float scale, int32_t min_q_len, int32_t max_q_len,
                                         int32_t max_context_len, const pkv_cache_desc* cache,
                                         int32_t partition_size, const int32_t* items,
                                         int32_t num_items, void* workspace, size_t workspace_bytes,
                                         void* stream);

/*
 * swap_blocks — move whole blocks between a GPU pool and a host swap pool for preemption and
 *   restore (「PagedAttention原理」 §抢占与恢复 / §swap). For each pair i: block dst_i of
 *   (dst_k, dst_v) <- block src_i of (src_k, src_v), all B slots, all kv heads, bit for bit.
 *   Either side may be device memory or pinned host memory that the device can address (e.g.
 *   hipHostMalloc); both use the pool layout above with the same block shape (num_blocks of the
 *   descriptor is not used). The copy runs as a kernel on `stream`, so it is ordered with the
 *   attention and cache writes around it.
 *   block_pairs  device (or device-addressable) int32 [num_pairs][2] = (src, dst); destinations
 *                distinct. num_pairs == 0 is a no-op.
 */
int32_t pkv_swap_blocks(void* dst_k, void* dst_v, const void* src_k, const void* src_v,
                        const int32_t* block_pairs, int32_t num_pairs, const pkv_cache_desc* cache,
                        void* stream);

/* ------------------------------------------------------------------------------------------
 * Host block manager (CPU only; touches no device memory). Deterministic:
 *   - a sequence takes a new block only when its last block is full
 *     (「PagedAttention原理」 §从虚拟内存的启发);
 *   - the block table keeps the physical block of each logical block and the filled count
 *     (「PagedAttention原理」 §实现一个虚拟内存);
 *   - every physical block has a reference count; writing into a block with count 1 is in
 *     place, otherwise: allocate a new block, record (old, new) for copy_blocks, remap the
 *     logical block, drop the old count, and write into the new block
 *     (「PagedAttention原理」 §解决COW);
 *   - fork shares every block of the parent (count + 1 each); free drops counts and releases
 *     blocks at zero (「Paged Attention&Orca Paper笔记与解读」 §PagedAttention的方法);
 *   - an append is all-or-nothing: on PKV_ENOBLOCKS no state changes
 *     (「PagedAttention原理」 §all-or-nothing 调度).
 *   - preemption: a set of sequences is swapped to a host swap pool and back as a whole or not
 *     at all; while swapped out a sequence cannot be appended to, forked or attended
 *     (PKV_ENOTRESIDENT). A block also referenced by a sequence outside the set is copied
 *     (its count drops by the set's references) instead of moved, so the swap space never holds
 *     more blocks than the GPU pool (「PagedAttention原理」 §抢占与恢复, §swap;
 *     「Paged Attention&Orca Paper笔记与解读」 §PagedAttention的方法).
 * Tie-breaks: free blocks are taken from the head of the creation-time order and released
 * blocks join its tail in logical-block order; sequences of one append are served in the
 * order given, tokens in position order; swaps take destinations in first-reference order.
 * A pkv_bm object is not thread-safe.
 * ------------------------------------------------------------------------------------------ */
typedef struct pkv_bm pkv_bm;

/* free_order: host int32 [num_blocks], a permutation of 0..num_blocks-1 (NULL = identity).
 * Returns NULL on invalid arguments or allocation failure. */
pkv_bm* pkv_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order);
void pkv_bm_destroy(pkv_bm* bm);

/* An independent copy of a block manager's whole state (tables, lengths, reference counts, free
 * lists in order, host pool): later operations on either one leave the other unchanged. The
 * caller destroys it with pkv_bm_destroy. Returns NULL for a NULL argument or when memory runs
 * out. For callers that need to restart from a saved allocation state, e.g. repeated timing of
 * the same steps. */
pkv_bm* pkv_bm_clone(const pkv_bm* bm);

int32_t pkv_bm_add_seq(pkv_bm* bm, int64_t seq_id);
int32_t pkv_bm_fork(pkv_bm* bm, int64_t parent_id, int64_t child_id);
int32_t pkv_bm_free_seq(pkv_bm* bm, int64_t seq_id);

/* Number of new blocks (fresh or copy-on-write) an append of these tokens would take
 * (host arrays of n_seqs); negative status on error. */
int64_t pkv_bm_blocks_needed(const pkv_bm* bm, const int64_t* seq_ids, const int32_t* n_tokens,
                             int32_t n_seqs);

/*
 * Append n_tokens[i] positions to seq_ids[i] for i < n_seqs (host arrays).
 *   slots_out      host int32 [sum n_tokens]: slot of every new token, in the order given.
 *   cow_pairs_out  host int32 [2 * max_pairs]: (src, dst) per copy-on-write, in order.
 *   num_pairs_out  host int32: number of pairs written.
 *   max_pairs      capacity of cow_pairs_out in pairs; at most one pair per sequence per
 *                  append can occur, so n_seqs always suffices.
 * All or nothing: on any error status the manager is unchanged.
 */
int32_t pkv_bm_append(pkv_bm* bm, const int64_t* seq_ids, const int32_t* n_tokens, int32_t n_seqs,
                      int32_t* slots_out, int32_t* cow_pairs_out, int32_t max_pairs,
                      int32_t* num_pairs_out);

/* Block tables and context lengths of n resident sequences into host arrays:
 * tables_out [n][max_blocks] padded with -1; ctx_out [n] (may be NULL). */
int32_t pkv_bm_block_tables(const pkv_bm* bm, const int64_t* seq_ids, int32_t n, int32_t max_blocks,
                            int32_t* tables_out, int32_t* ctx_out);

/* As pkv_bm_block_tables, with pad == 0 writing only each row's first ceil(len / B) entries (the
 * ones a kernel reads for that context) and leaving the rest of the row as it was: a serving loop
 * that refills the same staging rows every step saves rewriting the padding. pad != 0 is
 * pkv_bm_block_tables. Errors and validation are the same (nothing is written on an error). */
int32_t pkv_bm_block_tables_ex(const pkv_bm* bm, const int64_t* seq_ids, int32_t n, int32_t max_blocks,
                               int32_t* tables_out, int32_t* ctx_out, int32_t pad);

/* Table of one sequence: writes up to cap entries, returns its length in blocks (or error). */
int32_t pkv_bm_seq_table(const pkv_bm* bm, int64_t seq_id, int32_t* table_out, int32_t cap);
int32_t pkv_bm_context_len(const pkv_bm* bm, int64_t seq_id);
int32_t pkv_bm_refcount(const pkv_bm* bm, int32_t block);
int32_t pkv_bm_num_free(const pkv_bm* bm);
/* Free list from head to tail into host out[cap]; returns its length. */
int32_t pkv_bm_free_list(const pkv_bm* bm, int32_t* out, int32_t cap);

/* Gives the manager a host swap pool of num_host_blocks blocks (ids 0..n-1; free_order a
 * permutation or NULL for the identity). Once per manager. */
int32_t pkv_bm_attach_host_pool(pkv_bm* bm, int32_t num_host_blocks, const int32_t* free_order);

/* Swap out (resp. in) the n sequences seq_ids (host array, distinct, all resident (resp. all
 * swapped out)). pairs_out receives (src, dst) block pairs to copy with pkv_swap_blocks BEFORE
 * any later write reuses a released block: (GPU block, host block) for swap_out, (host block,
 * GPU block) for swap_in; at most one pair per distinct block of the set, max_pairs is the
 * capacity. All or nothing: PKV_ENOBLOCKS (target pool short) leaves the manager unchanged. */
int32_t pkv_bm_swap_out(pkv_bm* bm, const int64_t* seq_ids, int32_t n, int32_t* pairs_out,
                        int32_t max_pairs, int32_t* num_pairs_out);
int32_t pkv_bm_swap_in(pkv_bm* bm, const int64_t* seq_ids, int32_t n, int32_t* pairs_out,
                       int32_t max_pairs, int32_t* num_pairs_out);
/* 1 if resident on the GPU, 0 if swapped out, negative status on error. */
int32_t pkv_bm_is_resident(const pkv_bm* bm, int64_t seq_id);
int32_t pkv_bm_host_refcount(const pkv_bm* bm, int32_t host_block);
int32_t pkv_bm_host_free_list(const pkv_bm* bm, int32_t* out, int32_t cap);

#ifdef __cplusplus
}
#endif
#endif /* PAGEDKV_H */
