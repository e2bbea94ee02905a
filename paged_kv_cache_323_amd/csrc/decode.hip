// Paged decode attention for gfx950.
//
// One workgroup (4 waves) per (kv head, sequence, context partition), or in causal-rows mode per
// (kv head, query row of a ragged batch, partition), the row attending its sequence's keys up to
// its own position. The g = Hq/Hkv query heads that share a kv head are served by the same
// workgroup, so every K/V tile is read from HBM once per item. Two kernels share this frame and
// its epilogue; which one serves a (g, element type, head_dim) is fixed at compile time.
//
// Three-phase kernel (f32 pools, and 16-bit pools with one or two query heads per kv head, or four
// at head_dim 128). The partition's tokens are walked through the block table in units of 8
// tokens (units never straddle a block, since B is a multiple of 8); unit u belongs to wave
// u mod 4, and each wave keeps PF units of loads in flight:
//   phase 1  scores: 8 lanes per token, each lane owns interleaved 16-byte chunks of the row;
//            packed dot2 (bf16/f16) or fma (f32) against the query slices held in registers;
//            an 8-lane DPP reduction (on MFMA instead at eight query heads per kv head); scores
//            (pre-multiplied by scale·log2 e) go to LDS.
//   softmax  per head over the partition: max, exp2, sum (one wave per head).
//   phase 2  values: 16 lanes per token, each lane owns D/16 contiguous elements of the row;
//            fp32 accumulators for all g heads; probabilities read from LDS.
//   merge    the four token rows of a wave are summed across lanes (permlane swaps), then the
//            waves through LDS (the score buffer's words, reused after a barrier).
// LDS holds a score per token and head, which bounds the partition at 8192 / g tokens.
//
// One-pass kernel (16-bit pools with eight query heads per kv head, or four at head_dim 64): each
// wave walks its 16-token units loading K and V together; S = K·Qᵀ and Oᵀ = Vᵀ·Pᵀ on MFMA with a
// running (online) softmax per wave, V staged through LDS for the transposing read; the four
// waves are combined with log-sum-exp weights. No scores are kept, so partitions of up to 4096
// tokens fit, and no barrier separates a K stream from a V stream.
//
// A sequence whose context fits one partition writes its normalised output directly. Longer
// contexts write (max, sum, unnormalised output) per partition to the workspace, and a second
// small kernel merges them with log-sum-exp weights. Any grouping of blocks gives the same
// softmax, which is what makes the partitioning exact: the block-wise attention equation of
// 「PagedAttention原理」 §实现一个虚拟内存 sums exponentials block by block against one common
// denominator. The merge runs as its own launch so that no workgroup has to publish data to
// another one inside a kernel (a device-scope fence per workgroup costs a full L2 write-back
// and invalidate on this chip).
#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

namespace pkv {

PKV_DEBUG_UNIT(decode)

constexpr int kDecThreads = 256;
constexpr int kDecWaves = 4;

struct DecodeArgs {
  void* out;
  const void* q;
  const void* kc;
  const void* vc;
  const int32_t* tables;
  const int32_t* ctx_lens;
  const int32_t* cu;  // ragged batches: query rows of sequence s are cu[s]..cu[s+1]-1 (else row s)
  float* ws_acc;
  float2* ws_ml;
  int out_dt;
  int max_blocks;
  int hq;
  int hkv;
  int bs;
  int log2_bs;
  float scale_log2;
  int partition;
  int max_parts;
  int num_blocks;  // pool blocks (debug builds check table entries)
  int num_rows;    // rows of q / out (debug builds check ragged row offsets)
  const uint32_t* items;  // work list: item i = seq | part << 16 (null: dense grid)
  int num_seqs;
  int causal_rows;  // 1: one item per query row of a ragged batch (every row, any q_len)
  const void* k_new;          // optional new token per sequence, stored before it is attended
  const void* v_new;
  const int32_t* new_slots;   // null: nothing to store
};

// Index of the sequence whose query rows cu[s]..cu[s+1]-1 hold `row` (cu non-decreasing, cu[0] =
// 0): the number of s in 1..num_seqs with cu[s] <= row. Every thread of the 256-thread workgroup
// calls it; it ends with a barrier. scratch: 4 ints of LDS.
__device__ __forceinline__ int seq_of_row(const int32_t* cu, int num_seqs, int row, int* scratch) {
  int c = 0;
  for (int j = (int)threadIdx.x + 1; j <= num_seqs; j += 256) c += cu[j] <= row ? 1 : 0;
  for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off);
  if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = c;
  __syncthreads();
  return scratch[0] + scratch[1] + scratch[2] + scratch[3];
}

// Raw words of one lane's slice of a V row (PV mapping): 8, 16 or 32 bytes.
template <int NWORDS> struct Words { uint32_t w[NWORDS]; };

// K/V tiles are read once per step: their loads are marked non-temporal so the stream does not
// displace reusable lines (measured +3-6% on the decode configurations).
#ifndef PKV_STREAM_LOADS
#define PKV_STREAM_LOADS 1
#endif
template <typename V> __device__ __forceinline__ V load_tile(const V* p) {
#if PKV_STREAM_LOADS
  return __builtin_nontemporal_load(p);
#else
  return *p;
#endif
}

template <int NWORDS> __device__ __forceinline__ Words<NWORDS> load_words(const void* p) {
  Words<NWORDS> r;
  if constexpr (NWORDS == 2) {
    const u32x2 x = load_tile(reinterpret_cast<const u32x2*>(p));
    r.w[0] = x[0]; r.w[1] = x[1];
  } else {
#pragma unroll
    for (int i = 0; i < NWORDS / 4; ++i) {
      const u32x4 x = load_tile(reinterpret_cast<const u32x4*>(p) + i);
      r.w[4 * i] = x[0]; r.w[4 * i + 1] = x[1]; r.w[4 * i + 2] = x[2]; r.w[4 * i + 3] = x[3];
    }
  }
  return r;
}

template <int DT, int NWORDS, int EPL> __device__ __forceinline__ void words_to_f32(const Words<NWORDS>& w, float (&f)[EPL]) {
  if constexpr (DT == DT_F32) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) f[i] = __uint_as_float(w.w[i]);
  } else {
#pragma unroll
    for (int i = 0; i < NWORDS; ++i) unpack2<DT>(w.w[i], f[2 * i], f[2 * i + 1]);
  }
}

#ifndef PKV_DECODE_MIN_WG
#define PKV_DECODE_MIN_WG 1
#endif

// S = K·Qᵀ and Oᵀ = Vᵀ·Pᵀ steps of the one-pass kernel: v_mfma_f32_16x16x32 on the pool's 16-bit
// type (16 rows of A by 16 columns of B, 32 deep).
typedef __bf16 dec_bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 dec_f16x8 __attribute__((ext_vector_type(8)));
typedef float dec_f32x4 __attribute__((ext_vector_type(4)));

template <int DT> __device__ __forceinline__ dec_f32x4 mfma16x32(const u32x4& a, const u32x4& b, const dec_f32x4& c) {
  if constexpr (DT == DT_BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(dec_bf16x8, a), __builtin_bit_cast(dec_bf16x8, b),
                                                   c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(dec_f16x8, a), __builtin_bit_cast(dec_f16x8, b), c,
                                                  0, 0, 0);
}

// Units of loads in flight per wave in the one-pass kernel (two measured 6-10 % slower: the
// second unit's registers cost a wave per SIMD at head_dim 128).
#ifndef PKV_DECODE_FLASH_PF
#define PKV_DECODE_FLASH_PF 1
#endif

// V reaches the A operand of Oᵀ = Vᵀ·Pᵀ through the wave's LDS staging tile and the transposing
// LDS read of gfx950 (ds_read_b64_tr_b16): within each group of 16 lanes, lane i receives element
// i % 4 of the 8-byte rows given by lanes 4j + i / 4, j = 0..3, which turns four staged token rows
// into four tokens of one head_dim column per lane.

template <int DT> __device__ __forceinline__ u32x2 lds_read_tr16(const unsigned char* p) {
  typedef __bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
  typedef __fp16 f16x4 __attribute__((__vector_size__(4 * sizeof(__fp16))));
  if constexpr (DT == DT_BF16)
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                                         (__attribute__((address_space(3))) bf16x4*)(const_cast<unsigned char*>(p))));
  else
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4f16(
                                         (__attribute__((address_space(3))) f16x4*)(const_cast<unsigned char*>(p))));
}

// Four probabilities as the B operand of a 32-deep MFMA: each rounded to the pool's 16-bit type,
// then the four rounded remainders x - round(x), round to nearest even both times. P thus enters
// with about 16 significant bits; one bf16 P alone (8 bits) can miss a 2e-3 error bound when a few
// tokens carry most of the weight.
template <int DT> __device__ __forceinline__ u32x4 p_operand(const dec_f32x4& p) {
  using H = typename std::conditional<DT == DT_BF16, __bf16, _Float16>::type;
  typedef H h8 __attribute__((ext_vector_type(8)));
  h8 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const H hi = (H)p[e];
    r[e] = hi;
    r[e + 4] = (H)(p[e] - (float)hi);
  }
  return __builtin_bit_cast(u32x4, r);
}

template <int DT, int D, int G, int PF>
__global__ __launch_bounds__(kDecThreads, one_pass(G, DT, D) ? 3 : PKV_DECODE_MIN_WG) void paged_decode_kernel(DecodeArgs a) {
  using T = typename Elem<DT>::T;
  constexpr int ES = sizeof(T);
  constexpr int VEC = 16 / ES;        // elements per 16-byte chunk
  constexpr int NCH = D / (8 * VEC);  // 16-byte chunks per lane per token row (score mapping)
  constexpr int EPL = D / 16;         // elements per lane per token row (value mapping)
  constexpr int NWORDS = EPL * ES / 4;
  static_assert(NCH >= 1 && EPL * ES % 8 == 0, "unsupported head dim");

  constexpr int kPart = max_partition(G, DT, D);
  constexpr int kScores = kPart * G + kWave;  // the tail absorbs discarded writes
  constexpr int kRed = kDecWaves * G * D;
  constexpr bool kFlash = one_pass(G, DT, D);                                                  // one pass
  constexpr int kSRow = D * ES + 32;  // staging row stride: four consecutive rows start 32 bytes apart in the banks
  constexpr int kStageBytes = kDecWaves * 16 * kSRow;
  constexpr int kBuf = kFlash ? (kStageBytes / 4 > kRed ? kStageBytes / 4 : kRed) : (kScores > kRed ? kScores : kRed);
  __shared__ int32_t s_tab[kPart / 8];
  // Three-phase kernel: [token][head] scaled scores, then probabilities. One-pass kernel: the
  // waves' V staging tiles. After the last of either is read, the same words hold the per-wave
  // partial outputs.
  __shared__ __align__(16) float s_buf[kBuf];
  __shared__ float s_wm[kFlash ? kDecWaves * G : 1];  // one-pass: per-wave running max and sum
  __shared__ float s_wl[kFlash ? kDecWaves * G : 1];
  unsigned char* const s_stage = reinterpret_cast<unsigned char*>(s_buf);
  float* const s_p = s_buf;
  float* const s_red = s_buf;
  __shared__ float s_m[G];
  __shared__ float s_l[G];
  __shared__ int s_cnt[kDecWaves];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  int kvh, s, part;
  int row = -1;  // query / output row; set here in causal-rows mode
  if (a.causal_rows) {
    // Causal rows: workgroup x serves kv head x mod Hkv of query row x / Hkv, which attends its
    // sequence's keys up to and including its own position.
    row = (int)(blockIdx.x / (uint32_t)a.hkv);
    kvh = (int)(blockIdx.x - (uint32_t)row * (uint32_t)a.hkv);
    part = (int)gridDim.z - 1 - (int)blockIdx.z;
    s = seq_of_row(a.cu, a.num_seqs, row, s_cnt);
    if (s >= a.num_seqs) {  // offsets that do not cover the row: nothing to do
      if (kDebugChecks && tid == 0) debug_flag(DBG_RAGGED);
      return;  // uniform over the workgroup
    }
  } else if (a.items) {
    // Work list: workgroup x serves kv head x mod Hkv of item x / Hkv, so the kv heads of one
    // item (which read neighbouring parts of the same blocks) are dispatched together.
    const uint32_t item = blockIdx.x / (uint32_t)a.hkv;
    kvh = (int)(blockIdx.x - item * (uint32_t)a.hkv);
    const uint32_t it = a.items[item];
    s = (int)(it & 0xffffu);
    part = (int)(it >> 16);
    if (s >= a.num_seqs) {  // an item naming no sequence: nothing to do
      if (kDebugChecks && tid == 0) debug_flag(DBG_RAGGED);
      return;  // uniform over the workgroup
    }
  } else {
    kvh = blockIdx.x;
    s = blockIdx.y;
    // Last partitions are dispatched first: they exist only for long contexts and are always
    // full, while partition 0 of every sequence (often partial) fills the tail of the launch.
    part = (int)gridDim.z - 1 - (int)blockIdx.z;
  }

  int ctx_s = a.ctx_lens[s];
  if (a.causal_rows) {
    ctx_s -= a.cu[s + 1] - 1 - row;  // keys 0..this row's position
  } else if (a.cu) {
    // In a ragged batch only single-row (decode) sequences are handled here.
    row = a.cu[s];
    if (a.cu[s + 1] - row != 1) return;
    if (kDebugChecks && (row < 0 || row >= a.num_rows)) {
      if (tid == 0) debug_flag(DBG_RAGGED);
      return;  // uniform over the workgroup
    }
  } else {
    row = s;
  }
  const int wi = a.causal_rows ? row : s;  // workspace index of this item's partials
  // A length beyond the table or the launch's partitions breaks the caller's contract; clamping
  // keeps every access inside the table and the workspace.
  const int ctx = max(0, min(ctx_s, min(a.max_blocks * a.bs, a.max_parts * a.partition)));
  const int nparts = ctx > 0 ? (ctx + a.partition - 1) / a.partition : 1;
  if (part >= nparts) return;  // uniform over the workgroup
  // Balanced split: the sequence's partitions get equal sizes (a multiple of 64 tokens, so each
  // starts on a block boundary) instead of leaving a short last partition.
  const int psz = min(a.partition, (((ctx + nparts - 1) / nparts) + 63) & ~63);
  const int t0 = part * psz;
  const int n = max(0, min(psz, ctx - t0));  // tokens of this partition (0 iff ctx == 0)
  const int nunits = (n + 7) >> 3;
  const int nw = nunits > wave ? (nunits - wave + kDecWaves - 1) / kDecWaves : 0;  // this wave's units

  // The sequence's new token (fused cache write). The workgroup of its last partition, which alone
  // reads the token's position, takes that row's K and V from k_new / v_new instead of the pool
  // (in the one unit holding it) and stores them into the pool at the end, so nothing waits for the
  // stores. tn: the token's index in this partition, -1 when nothing is stored here.
  int32_t new_slot = -1;
  if (a.new_slots && part == nparts - 1) {
    new_slot = a.new_slots[s];
    if (kDebugChecks && new_slot >= (int64_t)a.num_blocks * a.bs) {
      if (tid == 0) debug_flag(DBG_SLOT);
      new_slot = -1;
    }
  }
  const int tn = new_slot >= 0 && n > 0 ? n - 1 : -1;  // the newest token closes the last partition
  const T* const knew = a.new_slots ? static_cast<const T*>(a.k_new) + ((size_t)s * a.hkv + kvh) * D : nullptr;
  const T* const vnew = a.new_slots ? static_cast<const T*>(a.v_new) + ((size_t)s * a.hkv + kvh) * D : nullptr;

  // Block-table entries of this partition.
  const int nblk = (n + a.bs - 1) >> a.log2_bs;
  const int32_t* trow = a.tables + (size_t)s * a.max_blocks + (t0 >> a.log2_bs);
  for (int i = tid; i < nblk; i += kDecThreads) {
    int b = trow[i];
    if (kDebugChecks && (b < 0 || b >= a.num_blocks)) {
      debug_flag(DBG_BLOCK);
      b = 0;
    }
    s_tab[i] = b;
  }

  // Query slices of the G heads in the score mapping (three-phase kernel), or the query as the B
  // operand of S = K·Qᵀ (one-pass kernel): lane (head column hc, group gg) holds dims
  // 32·ks + 8·gg .. +7 of head hc for k-step ks, zero for the columns past G.
  constexpr int KS = D / 32;
  const int c = lane & 7;   // 16-byte chunk column
  const int r = lane >> 3;  // token row within a unit
  const int hc = lane & 15;  // MFMA mapping: token row (K operand) / head column (Q operand)
  const int gg = lane >> 4;  // MFMA mapping: 8-dim group of a k-step
  u32x4 qr[kFlash ? 1 : G][kFlash ? 1 : NCH];
  u32x4 qm[kFlash ? KS : 1];
  if constexpr (kFlash) {
    const T* qp = static_cast<const T*>(a.q) + ((size_t)row * a.hq + (size_t)kvh * G + min(hc, G - 1)) * D + 8 * gg;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(qp + 32 * ks);
      qm[ks] = hc < G ? w : u32x4{0, 0, 0, 0};
    }
  } else {
    const T* qb = static_cast<const T*>(a.q) + ((size_t)row * a.hq + (size_t)kvh * G) * D + c * VEC;
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) qr[g][ch] = *reinterpret_cast<const u32x4*>(qb + g * D + ch * 8 * VEC);
  }
  __syncthreads();

  // Base of the (physical block, kv head) tile holding unit u; units never straddle blocks. Rows of
  // a tile are D elements apart (head-major pool). PKV_TOKEN_MAJOR builds a tuning variant for the
  // token-major layout [N][B][H][D] (rows H·D apart), used only to measure the layout choice.
#ifdef PKV_TOKEN_MAJOR
  const size_t tile_rows = (size_t)a.bs * a.hkv;
  const size_t head_rows = (size_t)kvh;
  const size_t row_stride = (size_t)a.hkv * D;
#else
  const size_t tile_rows = (size_t)a.hkv * a.bs;
  const size_t head_rows = (size_t)kvh * a.bs;
  const size_t row_stride = D;
#endif
  auto tile = [&](const T* base, int u) -> const T* {
    const int phys = s_tab[(u * 8) >> a.log2_bs];
    return base + ((size_t)phys * tile_rows + head_rows) * D;
  };
  const T* kbase = static_cast<const T*>(a.kc);
  const T* vbase = static_cast<const T*>(a.vc);
  const int krow = r;                      // row offset of this lane within a unit
  const int cv = lane & 15;                // value mapping: column slice
  const int rv = lane >> 4;                // value mapping: token row within a pass of 4

  auto load_k = [&](int u, u32x4 (&dst)[NCH]) {
    const T* p = tile(kbase, u) + (size_t)((u * 8 + krow) & (a.bs - 1)) * row_stride + c * VEC;
    if (u == (tn >> 3) && tn >= 0) {  // uniform: the unit holding the new token
      if (u * 8 + krow == tn) p = knew + c * VEC;
    }
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) dst[ch] = load_tile(reinterpret_cast<const u32x4*>(p + ch * 8 * VEC));
  };
  auto load_v = [&](int u, Words<NWORDS> (&dst)[2]) {
    const T* p = tile(vbase, u) + cv * EPL;
#pragma unroll
    for (int ps = 0; ps < 2; ++ps) {
      const T* q = p + (size_t)((u * 8 + ps * 4 + rv) & (a.bs - 1)) * row_stride;
      if (u == (tn >> 3) && tn >= 0) {  // uniform: the unit holding the new token
        if (u * 8 + ps * 4 + rv == tn) q = vnew + cv * EPL;
      }
      dst[ps] = load_words<NWORDS>(q);
    }
  };

  // One-pass kernel: 16-token units, unit v to wave v mod 4. A token past the partition reads the
  // last one (a written row); its score is dropped and its probability is 0.
  const int nu16 = (n + 15) >> 4;
  const int nw16 = nu16 > wave ? (nu16 - wave + kDecWaves - 1) / kDecWaves : 0;
  const int last16 = wave + kDecWaves * (nw16 > 0 ? nw16 - 1 : 0);
  auto unit16 = [&](int i) { return min(wave + kDecWaves * i, last16); };
  // V of a unit: lane (chunk cw, row rw) loads 16 bytes of rows p·RP + rw.
  constexpr int CPR = D * ES / 16;  // 16-byte chunks per row
  constexpr int RP = 64 / CPR;      // rows per pass
  constexpr int NPV = 16 / RP;      // passes per 16-token unit
  const int cw = lane % CPR;
  const int rw = lane / CPR;
  auto load_v16 = [&](int v, u32x4 (&dst)[NPV]) {
#pragma unroll
    for (int ps = 0; ps < NPV; ++ps) {
      const int tk = min(16 * v + ps * RP + rw, n - 1);
      const int phys = s_tab[tk >> a.log2_bs];
      const T* q = vbase + ((size_t)phys * tile_rows + head_rows) * D + (size_t)(tk & (a.bs - 1)) * row_stride + cw * VEC;
      if (v == (tn >> 4) && tn >= 0) {  // uniform: the unit holding the new token
        if (tk == tn) q = vnew + cw * VEC;
      }
      dst[ps] = load_tile(reinterpret_cast<const u32x4*>(q));
    }
  };

  // K of a unit as the A operand of S = K·Qᵀ: lane (token hc, group gg) loads dims 32·ks + 8·gg ..
  // +7 of its token's row for k-step ks.
  auto load_k16 = [&](int v, u32x4 (&dst)[KS]) {
    const int tk = min(16 * v + hc, n - 1);
    const int phys = s_tab[tk >> a.log2_bs];
    const T* p = kbase + ((size_t)phys * tile_rows + head_rows) * D + (size_t)(tk & (a.bs - 1)) * row_stride + 8 * gg;
    if (v == (tn >> 4) && tn >= 0) {  // uniform: the unit holding the new token
      if (tk == tn) p = knew + 8 * gg;
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) dst[ks] = load_tile(reinterpret_cast<const u32x4*>(p + 32 * ks));
  };

  if constexpr (kFlash) {
    // ---- one pass: each wave streams its units' K and V together, with a running softmax -------
    // Scores S = K·Qᵀ of a unit leave lane (head hc, group gg) with tokens 4·gg .. +3 of head hc,
    // which is the B-operand layout of Oᵀ = Vᵀ·Pᵀ when K = 32 pairs the four tokens' rounded P
    // (k 8·gg .. +3) with their rounded remainders (k 8·gg + 4 .. +7), and the A operand repeats
    // the same four staged V rows in both halves: no probability leaves its lane and no score
    // goes through LDS. Each wave keeps its own running max, sum and Oᵀ; the maximum is raised
    // lazily (only when a unit's exceeds it by more than 2^8, so P ≤ 256 between rescales), and
    // the four waves are combined with log-sum-exp weights at the end.
    constexpr int NT = D / 16;
    constexpr int PFF = PKV_DECODE_FLASH_PF;
    constexpr float kLazy = 8.f;
    dec_f32x4 oacc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) oacc[t] = dec_f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;
    unsigned char* const stg = s_stage + wave * 16 * kSRow;
    // Transposing read of tile t: lane (i, group gg) gives staged row 4·gg + i / 4, columns
    // 16·t + 4·(i % 4) .. +3, and receives rows 4·gg .. +3 of column 16·t + i.
    const unsigned char* const trp = stg + (4 * gg + (hc >> 2)) * kSRow + 4 * (hc & 3) * ES;
    if (nw16 > 0) {
      u32x4 kf[PFF][KS];
      u32x4 vf[PFF][NPV];
#pragma unroll
      for (int j = 0; j < PFF; ++j) {
        load_k16(unit16(j), kf[j]);
        load_v16(unit16(j), vf[j]);
      }
      const int nwf_pad = (nw16 + PFF - 1) / PFF * PFF;
      for (int i0 = 0; i0 < nwf_pad; i0 += PFF) {
#pragma unroll
        for (int j = 0; j < PFF; ++j) {
          const int i = i0 + j;
          const int v = unit16(i);
          const bool live = i < nw16;  // uniform over the wave
          dec_f32x4 sacc = dec_f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) sacc = mfma16x32<DT>(kf[j][ks], qm[ks], sacc);
          if (live) {
#pragma unroll
            for (int ps = 0; ps < NPV; ++ps)
              *reinterpret_cast<u32x4*>(stg + (ps * RP + rw) * kSRow + cw * 16) = vf[j][ps];
          }
          load_k16(unit16(i + PFF), kf[j]);
          load_v16(unit16(i + PFF), vf[j]);
          if (live) {
            float sv[4];
            float mx = -INFINITY;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              sv[e] = 16 * v + 4 * gg + e < n ? sacc[e] * a.scale_log2 : -INFINITY;
              mx = fmaxf(mx, sv[e]);
            }
            mx = max_rows4(mx);  // over the unit's 16 tokens
            const float mc = fmaxf(m_run, mx);
            const bool need = mc > m_run + kLazy;  // always on the first unit (m_run = -inf)
            if (__ballot(need) != 0) {
              const float mn = need ? mc : m_run;
              const float al = fast_exp2(m_run - mn);
#pragma unroll
              for (int t = 0; t < NT; ++t) oacc[t] *= al;
              l_run *= al;
              m_run = mn;
            }
            dec_f32x4 pv;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              pv[e] = fast_exp2(sv[e] - m_run);
              l_run += pv[e];
            }
            const u32x4 pb = p_operand<DT>(pv);
#pragma unroll
            for (int t = 0; t < NT; ++t) {
              const u32x2 x = lds_read_tr16<DT>(trp + 32 * t);
              oacc[t] = mfma16x32<DT>(u32x4{x[0], x[1], x[0], x[1]}, pb, oacc[t]);
            }
          }
        }
      }
    }
    // ---- the four waves: log-sum-exp weights against the largest running max ------------------
    l_run = sum_rows4(l_run);  // the head's four lane groups
    if (gg == 0 && hc < G) {
      s_wm[wave * G + hc] = m_run;
      s_wl[wave * G + hc] = l_run;
    }
    __syncthreads();  // staging tiles are dead; the waves' maxima and sums are visible
    float mall = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) mall = fmaxf(mall, s_wm[w * G + (hc & (G - 1))]);
    const float wt = m_run == -INFINITY ? 0.f : fast_exp2(m_run - mall);  // a wave without units
    if (hc < G) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
        *reinterpret_cast<dec_f32x4*>(&s_red[(wave * G + hc) * D + 16 * t + 4 * gg]) = oacc[t] * wt;
    }
    if (tid < G) {
      float l = 0.f;
#pragma unroll
      for (int w = 0; w < kDecWaves; ++w) {
        const float mw = s_wm[w * G + tid];
        l += mw == -INFINITY ? 0.f : fast_exp2(mw - mall) * s_wl[w * G + tid];
      }
      s_m[tid] = mall;
      s_l[tid] = l;
    }
    __syncthreads();
  } else {
    // ---- phase 1: scores, PF units in flight per wave -------------------------------------------
    // Loads are unconditional (indices past the wave's last unit are clamped to it) so the wait
    // counts inside the unrolled ring are static; results of padding iterations are discarded.
    const int last = wave + kDecWaves * (nw > 0 ? nw - 1 : 0);
    auto unit_of = [&](int i) { return min(wave + kDecWaves * i, last); };
    const int nw_pad = (nw + PF - 1) / PF * PF;
    Words<NWORDS> vb[PF][2];
    if (nw > 0) {
      u32x4 kb[PF][NCH];
#pragma unroll
      for (int j = 0; j < PF; ++j) load_k(unit_of(j), kb[j]);
      for (int i0 = 0; i0 < nw_pad; i0 += PF) {
#pragma unroll
        for (int j = 0; j < PF; ++j) {
          const int i = i0 + j;
          const int u = unit_of(i);
          float sc[G];
#pragma unroll
          for (int g = 0; g < G; ++g) {
            float acc = 0.f;
#pragma unroll
            for (int ch = 0; ch < NCH; ++ch) acc = dot16B<DT>(qr[g][ch], kb[j][ch], acc);
            sc[g] = sum8(acc);
          }
          load_k(unit_of(i + PF), kb[j]);
          const int tl = u * 8 + r;
          float mine = sc[0];
#pragma unroll
          for (int g = 1; g < G; ++g) mine = (c == g) ? sc[g] : mine;
          // Branch-free store: lanes with nothing to keep write into the discard tail.
          const int dst = (c < G && i < nw) ? tl * G + c : kPart * G + lane;
          s_p[dst] = tl < n ? mine * a.scale_log2 : -INFINITY;
        }
      }
    }
    // Value loads of the first units go out before the softmax so they overlap it.
    if (nw > 0) {
#pragma unroll
      for (int j = 0; j < PF; ++j) load_v(unit_of(j), vb[j]);
    }
    __syncthreads();

    // ---- softmax over the partition, one wave per head ---------------------------------------
    for (int g = wave; g < G; g += kDecWaves) {
      float m = -INFINITY;
      for (int i = lane; i < n; i += kWave) m = fmaxf(m, s_p[i * G + g]);
      m = wave_max(m);
      float l = 0.f;
      for (int i = lane; i < nunits * 8; i += kWave) {
        const float p = i < n ? fast_exp2(s_p[i * G + g] - m) : 0.f;
        s_p[i * G + g] = p;
        l += p;
      }
      l = wave_sum(l);
      if (lane == 0) {
        s_m[g] = m;
        s_l[g] = l;
      }
    }
    __syncthreads();

    // ---- phase 2: probability-weighted values, PF units in flight per wave --------------------
    float acc[G][EPL];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;
    if (nw > 0) {
      for (int i0 = 0; i0 < nw_pad; i0 += PF) {
#pragma unroll
        for (int j = 0; j < PF; ++j) {
          const int i = i0 + j;
          const int u = unit_of(i);
          float vf[2][EPL];
          words_to_f32<DT, NWORDS, EPL>(vb[j][0], vf[0]);
          words_to_f32<DT, NWORDS, EPL>(vb[j][1], vf[1]);
          load_v(unit_of(i + PF), vb[j]);
#pragma unroll
          for (int ps = 0; ps < 2; ++ps) {
            const int tl = u * 8 + ps * 4 + rv;
            const bool valid = i < nw && tl < n;
            float pg[G];
#pragma unroll
            for (int g = 0; g < G; ++g) pg[g] = s_p[tl * G + g];  // 0 past the context
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
              const float x = valid ? vf[ps][e] : 0.f;  // unwritten slots may hold anything
#pragma unroll
              for (int g = 0; g < G; ++g) acc[g][e] = __builtin_fmaf(pg[g], x, acc[g][e]);
            }
          }
        }
      }
    }

    // ---- merge the four token rows of each wave, then the four waves --------------------------
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        acc[g][e] = sum_rows4(acc[g][e]);
      }
    __syncthreads();  // every wave is done reading probabilities before s_red overwrites them
    if (rv == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < EPL; ++e) s_red[(wave * G + g) * D + cv * EPL + e] = acc[g][e];
    }
    __syncthreads();
  }  // three-phase kernel

  // The new token's rows into the pool (the fused cache write): nothing in this launch reads them.
  if (new_slot >= 0) {
    constexpr int kRowChunks = D * ES / 16;  // 16-byte chunks of one row
    if (tid < 2 * kRowChunks) {
      const bool is_v = tid >= kRowChunks;
      const int ch = is_v ? tid - kRowChunks : tid;
      const int64_t blk = new_slot >> a.log2_bs, off = new_slot & (a.bs - 1);
#ifdef PKV_TOKEN_MAJOR
      const int64_t dst_row = (blk * a.bs + off) * a.hkv + kvh;
#else
      const int64_t dst_row = (blk * a.hkv + kvh) * a.bs + off;
#endif
      const u32x4 x = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(is_v ? vnew : knew) + ch * 16);
      *reinterpret_cast<u32x4*>(static_cast<char*>(const_cast<void*>(is_v ? a.vc : a.kc)) + dst_row * D * ES +
                                ch * 16) = x;
    }
  }

  const size_t out_row = (size_t)row * a.hq + (size_t)kvh * G;  // first of the G query heads
  const size_t item = ((size_t)wi * a.hkv + kvh) * a.max_parts + part;
  for (int o = tid; o < G * D; o += kDecThreads) {
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) v += s_red[w * G * D + o];
    const int g = o / D;
    if (nparts == 1) {
      const float l = s_l[g];
      store_out(a.out, out_row * D + o, l > 0.f ? v / l : 0.f, a.out_dt);
    } else {
      a.ws_acc[item * G * D + o] = v;
      if (o % D == 0) a.ws_ml[item * G + g] = make_float2(s_m[g], s_l[g]);
    }
  }
}

// Log-sum-exp merge of the partitions' partial results. A thread merges four consecutive output
// elements of one head (16-byte partial loads and output stores), and a workgroup covers
// 4 * 256 / NG elements of one sequence with NG threads each: thread group k merges partitions
// k, k + NG, ... with a running maximum, and the NG (max, sum, values) results of an element are
// then combined through LDS. NG grows with the partition count (up to 8), so that up to 64
// partitions take one round of loads per thread: a long context's merge is not a chain of
// dependent loads.
template <int NG>
__global__ __launch_bounds__(256) void paged_decode_merge_kernel(DecodeArgs a, int head_dim, int group) {
  constexpr int kOuts = 256 / NG;  // threads per thread group; each merges 4 elements
  typedef float f4 __attribute__((ext_vector_type(4)));
  __shared__ float s_ml[NG > 1 ? 6 * NG * kOuts : 1];
  __shared__ int s_cnt[4];
  const int oi = threadIdx.x % kOuts;
  const int grp = threadIdx.x / kOuts;
  const int o = 4 * (blockIdx.x * kOuts + oi);  // first of this thread's 4 elements (one head)
  const bool active = o < a.hq * head_dim;
  int s, row, ctx_s;
  if (a.causal_rows) {  // workgroup row y: one query row of a ragged batch
    row = blockIdx.y;
    s = seq_of_row(a.cu, a.num_seqs, row, s_cnt);
    if (s >= a.num_seqs) return;  // uniform; flagged by the partition kernel
    ctx_s = a.ctx_lens[s] - (a.cu[s + 1] - 1 - row);
  } else {
    s = blockIdx.y;
    row = s;
    if (a.cu) {
      row = a.cu[s];
      if (a.cu[s + 1] - row != 1) return;                              // uniform over the workgroup
      if (kDebugChecks && (row < 0 || row >= a.num_rows)) return;  // flagged by the partition kernel
    }
    ctx_s = a.ctx_lens[s];
  }
  const int ctx = max(0, min(ctx_s, min(a.max_blocks * a.bs, a.max_parts * a.partition)));
  const int nparts = ctx > 0 ? (ctx + a.partition - 1) / a.partition : 1;
  if (nparts <= 1) return;  // uniform
  const int h = active ? o / head_dim : 0;
  const int kvh = h / group;
  const int g = h - kvh * group;
  const int d = active ? o - h * head_dim : 0;
  const size_t item = ((size_t)(a.causal_rows ? row : s) * a.hkv + kvh) * a.max_parts;
  // This thread's partitions grp, grp + NG, ... are read in chunks of 8 whose loads are all issued
  // before any is used, and merged with a running log-sum-exp.
  constexpr int kChunk = 8;
  const int mine = nparts > grp ? (nparts - grp + NG - 1) / NG : 0;
  float mx = -INFINITY, l = 0.f;
  f4 v = f4{0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; active && j0 < mine; j0 += kChunk) {
    float2 ml[kChunk];
    f4 av[kChunk];
#pragma unroll
    for (int j = 0; j < kChunk; ++j) {
      const int p = grp + NG * min(j0 + j, mine - 1);  // padding re-reads the last one; dropped below
      ml[j] = a.ws_ml[(item + p) * group + g];
      av[j] = *reinterpret_cast<const f4*>(&a.ws_acc[((item + p) * group + g) * head_dim + d]);
    }
    float cm = mx;
#pragma unroll
    for (int j = 0; j < kChunk; ++j)
      if (j0 + j < mine) cm = fmaxf(cm, ml[j].x);
    const float r = fast_exp2(mx - cm);  // rescale what was merged so far (0 on the first chunk)
    l *= r;
    v *= r;
#pragma unroll
    for (int j = 0; j < kChunk; ++j) {
      if (j0 + j < mine) {
        const float w = fast_exp2(ml[j].x - cm);
        l = __builtin_fmaf(w, ml[j].y, l);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = __builtin_fmaf(w, av[j][e], v[e]);
      }
    }
    mx = cm;
  }
  if constexpr (NG > 1) {
    float* s_m = s_ml;
    float* s_l = s_ml + NG * kOuts;
    f4* s_v = reinterpret_cast<f4*>(s_ml + 2 * NG * kOuts);
    s_m[grp * kOuts + oi] = mx;
    s_l[grp * kOuts + oi] = l;
    s_v[grp * kOuts + oi] = v;
    __syncthreads();
    if (grp != 0) return;
    float m_all = mx;
#pragma unroll
    for (int k = 1; k < NG; ++k) m_all = fmaxf(m_all, s_m[k * kOuts + oi]);
    l = 0.f;
    v = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < NG; ++k) {
      const float mk = s_m[k * kOuts + oi];
      const float w = mk == -INFINITY ? 0.f : fast_exp2(mk - m_all);  // a group with no partition
      l = __builtin_fmaf(w, s_l[k * kOuts + oi], l);
      const f4 vk = s_v[k * kOuts + oi];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = __builtin_fmaf(w, vk[e], v[e]);
    }
  }
  const f4 res = l > 0.f ? f4{v[0] / l, v[1] / l, v[2] / l, v[3] / l} : f4{0.f, 0.f, 0.f, 0.f};
  if (active) store_out4(a.out, (size_t)row * a.hq * head_dim + o, res, a.out_dt);
}

static DecodeArgs make_args(const DecodeLaunch& L) {
  DecodeArgs a;
  a.out = L.out;
  a.q = L.q;
  a.kc = L.kc;
  a.vc = L.vc;
  a.tables = L.tables;
  a.ctx_lens = L.ctx_lens;
  a.cu = L.cu;
  a.ws_acc = L.ws_acc;
  a.ws_ml = reinterpret_cast<float2*>(L.ws_ml);
  a.out_dt = L.out_dt;
  a.max_blocks = L.max_blocks;
  a.hq = L.num_q_heads;
  a.hkv = L.num_kv_heads;
  a.bs = L.block_size;
  a.log2_bs = ilog2(L.block_size);
  a.scale_log2 = L.scale * 1.4426950408889634f;
  a.partition = L.partition;
  a.max_parts = L.max_parts;
  a.num_blocks = L.num_blocks;
  a.num_rows = L.num_rows;
  a.items = reinterpret_cast<const uint32_t*>(L.items);
  a.num_seqs = L.num_seqs;
  a.causal_rows = L.causal_rows;
  a.k_new = L.k_new;
  a.v_new = L.v_new;
  a.new_slots = L.new_slots;
  return a;
}

constexpr int kPrefetch = PKV_DECODE_PREFETCH;

template <int DT, int D, int G>
static hipError_t launch_decode_t(const DecodeLaunch& L, hipStream_t stream) {
  const DecodeArgs a = make_args(L);
  if (L.stage != 2) {
    const dim3 grid = L.causal_rows ? dim3((unsigned)L.num_rows * (unsigned)L.num_kv_heads, 1, L.max_parts)
                      : L.items     ? dim3((unsigned)L.num_items * (unsigned)L.num_kv_heads)
                                    : dim3(L.num_kv_heads, L.num_seqs, L.max_parts);
    if (!L.items || L.num_items > 0) {
      const hipError_t e = launch_kernel(paged_decode_kernel<DT, D, G, kPrefetch>, grid, dim3(kDecThreads), stream, a);
      if (e != hipSuccess) return e;
    }
  }
  if (L.stage != 1 && L.max_parts > 1) {
    const int outs = L.num_q_heads * D;
    // threads per output: enough that each merges at most one chunk of 8 partitions
    const int ng = L.max_parts <= 8 ? 1 : L.max_parts <= 16 ? 2 : L.max_parts <= 32 ? 4 : 8;
    const dim3 grid((unsigned)((outs / 4 * ng + 255) / 256), (unsigned)(L.causal_rows ? L.num_rows : L.num_seqs));
    switch (ng) {
      case 1: return launch_kernel(paged_decode_merge_kernel<1>, grid, dim3(256), stream, a, D, G);
      case 2: return launch_kernel(paged_decode_merge_kernel<2>, grid, dim3(256), stream, a, D, G);
      case 4: return launch_kernel(paged_decode_merge_kernel<4>, grid, dim3(256), stream, a, D, G);
      default: return launch_kernel(paged_decode_merge_kernel<8>, grid, dim3(256), stream, a, D, G);
    }
  }
  return hipSuccess;
}

template <int DT, int D>
static hipError_t launch_decode_d(const DecodeLaunch& L, hipStream_t stream) {
  switch (L.num_q_heads / L.num_kv_heads) {
    case 1: return launch_decode_t<DT, D, 1>(L, stream);
    case 2: return launch_decode_t<DT, D, 2>(L, stream);
    case 4: return launch_decode_t<DT, D, 4>(L, stream);
    case 8: return launch_decode_t<DT, D, 8>(L, stream);
  }
  return hipErrorInvalidConfiguration;
}

template <int DT>
static hipError_t launch_decode_dt(const DecodeLaunch& L, hipStream_t stream) {
  if (L.head_dim == 64) return launch_decode_d<DT, 64>(L, stream);
  if (L.head_dim == 128) return launch_decode_d<DT, 128>(L, stream);
  return hipErrorInvalidConfiguration;
}

hipError_t launch_decode(const DecodeLaunch& L, hipStream_t stream) {
  const int g = L.num_kv_heads > 0 ? L.num_q_heads / L.num_kv_heads : 0;
  if (g < 1 || L.partition > max_partition(g, L.dt, L.head_dim) || L.partition % 64 != 0) return hipErrorInvalidConfiguration;
  switch (L.dt) {
    case DT_F32: return launch_decode_dt<DT_F32>(L, stream);
    case DT_F16: return launch_decode_dt<DT_F16>(L, stream);
    case DT_BF16: return launch_decode_dt<DT_BF16>(L, stream);
  }
  return hipErrorInvalidConfiguration;
}

}  // namespace pkv
