// Prefill part of the ragged mixed step: causal attention of multi-row sequences over the paged
// cache, on MFMA (v_mfma_f32_16x16x32_{bf16,f16}).
//
// Selective batching flattens every request's new tokens into one batch and splits it per
// request only inside attention, where each request's phase decides whether it reads cached
// keys (「Paged Attention&Orca Paper笔记与解读」 §Orca的Solution). Here a workgroup takes a tile of
// 128 query rows of one prefill sequence for one query head; its four waves own 32 rows each.
// Keys and values are read through the block table in tiles of 64 (a tile spans 2-8 blocks) and
// staged in LDS: K row-major, V transposed (d-major) so both feed MFMA A-operands with plain
// 16- or 8-byte reads. Per key tile and wave:
//   Sᵀ = K·Qᵀ            (M = 64 keys, N = 32 rows, K = head_dim)   -> lane holds 4 keys x 1 row
//   online softmax        (row max across the 4 lane groups; fp32; exp2 on log2-scaled scores)
//   Oᵀ += Vᵀ·Pᵀ          (M = head_dim, N = 32 rows, K = 64 keys)    -> lane holds 4 dims x 1 row
// The P operand comes straight from the Sᵀ accumulators: MFMA sums over k, so any fixed order of
// the 32 keys of a k-step works as long as the Vᵀ operand uses the same order. P goes to MFMA as
// f16 rounded to nearest (11 bits, at most 2^-12 relative; one bf16 P, 8 bits, would cost up to
// ~1e-2 relative on short rows), so Vᵀ is staged as f16 too: a bf16 pool's values are converted,
// which is exact inside the f16 range. A tile whose V leaves that range is recomputed with bf16
// Vᵀ and P split into a bf16 high part and remainder (two MFMAs per step, about 16 bits).
// A query row at position p sees keys 0..p (the block-wise equation's ⌈i/B⌉ limit,
// 「PagedAttention原理」 §实现一个虚拟内存).
#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

namespace pkv {

PKV_DEBUG_UNIT(ragged)

constexpr int kPfThreads = 256;
constexpr int kPfRows = 128;  // query rows per workgroup (4 waves x 32)
constexpr int kPfKeys = 64;   // keys per tile

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int DT> struct Mfma;
template <> struct Mfma<DT_BF16> {
  using V8 = bf16x8;
  using S = __bf16;
  static __device__ __forceinline__ f32x4 mma(const V8& a, const V8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mfma<DT_F16> {
  using V8 = f16x8;
  using S = _Float16;
  static __device__ __forceinline__ f32x4 mma(const V8& a, const V8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

typedef float f32x2 __attribute__((ext_vector_type(2)));

// Split two probabilities x = hi + lo into bf16 high parts and bf16 remainders, each pair packed
// into one 32-bit operand word (element 0 in the low half). hi is truncated, the remainder
// carries the rest, so hi + lo keeps about 16 significant bits.
__device__ __forceinline__ void split_pair_bf16(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  const uint32_t u0 = __float_as_uint(x0), u1 = __float_as_uint(x1);
  hi = __builtin_amdgcn_perm(u1, u0, 0x07060302u);  // upper halves: bf16 truncation of both
  const f32x2 r = {x0 - __uint_as_float(u0 & 0xffff0000u), x1 - __uint_as_float(u1 & 0xffff0000u)};
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2));
}
// Two probabilities as f16 rounded to nearest, packed into one 32-bit operand word.
__device__ __forceinline__ uint32_t pack_f16(float x0, float x1) {
  const f32x2 x = {x0, x1};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, f16x2));
}

struct PrefillArgs {
  void* out;
  const uint16_t* q;
  const uint16_t* kc;
  const uint16_t* vc;
  const int32_t* tables;
  const int32_t* cu;
  const int32_t* ctx_lens;
  int out_dt;
  int max_blocks;
  int num_seqs;
  int hq;
  int hkv;
  int bs;
  int log2_bs;
  float scale_log2;
  int num_tokens;  // rows of q / out (debug builds check cu_seqlens against it)
  int num_blocks;  // pool blocks (debug builds check table entries)
  int min_rows;    // a sequence with at least this many query rows (1 or 2) gets row tiles
};

constexpr int kPfTab = 1024;  // block-table entries cached in LDS at a time

#ifndef PF_LOOKAHEAD
#define PF_LOOKAHEAD 2
#endif
#ifndef PF_SCHED
#define PF_SCHED 1
#endif
// Wave priority during the MFMA phases (Sᵀ and Oᵀ), back to 0 for softmax and staging: when the
// two waves sharing a SIMD want to issue at once, the one feeding the matrix core goes first and
// the other fills its gaps (+2.5 % on the 13B-shaped and on long prompts).
#ifndef PF_SETPRIO
#define PF_SETPRIO 1
#endif
#ifndef PF_LDS_EPILOGUE
#define PF_LDS_EPILOGUE 1
#endif
// Order of the MFMA steps: 1 runs the k-steps outermost (Sᵀ: every key tile's first k-step, then
// every second one; Oᵀ: every head-dim tile against keys 0..31, then against 32..63), so an MFMA's
// accumulator was last written 8 or 16 MFMAs earlier instead of 2: 1-2 % faster than 0.
#ifndef PF_ACC_ORDER
#define PF_ACC_ORDER 1
#endif
#ifndef PF_XCD
#define PF_XCD 1
#endif
constexpr int kPfLookahead = PF_LOOKAHEAD;  // MFMA operand reads issued this many steps ahead


template <int DT, int D>
// Two workgroups per CU: the register budget is capped at 256 per lane so that one wave's MFMA
// work overlaps the other's softmax and staging.
__global__ __launch_bounds__(kPfThreads, 2) void ragged_prefill_kernel(PrefillArgs a) {
  using M = Mfma<DT>;
  using V8 = typename M::V8;
  constexpr int KS = D / 32;         // k-steps of Sᵀ = K·Qᵀ
  constexpr int DT16 = D / 16;       // 16-row tiles of the head dim (M-tiles of Oᵀ)
  constexpr int KLD = D + 8;         // LDS row stride of the K tile (elements)
  // LDS row stride of the transposed V tile: 34 dwords, so the 16 rows one operand read touches
  // land on distinct bank pairs.
  constexpr int VLD = kPfKeys + 4;
  constexpr int CPR = D / 8;         // 16-byte chunks per K/V row
  constexpr int KIT = kPfKeys * CPR / kPfThreads;        // K chunks staged per thread
  constexpr int VIT = (kPfKeys / 2) * CPR / kPfThreads;  // V key-pair chunks staged per thread

  constexpr int KBUF = kPfKeys * KLD;  // elements of one K buffer
  constexpr int VBUF = D * VLD;        // elements of one transposed-V buffer
  __shared__ __attribute__((aligned(16))) uint16_t sK[2 * KBUF];
  __shared__ __attribute__((aligned(16))) uint16_t sVt[2 * VBUF];
  __shared__ int s_tab[kPfTab];
  __shared__ int s_wtot[kPfThreads / kWave];
  __shared__ int s_seq, s_tile, s_q0, s_ql, s_ctx;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches on it
  // Workgroups go to the eight XCDs (each with its own L2) in turn, so with a multiple of 8 heads
  // blockIdx.x mod 8 picks the XCD. With PF_XCD and several query heads per kv head (kv heads a
  // multiple of 8), blockIdx.x = 8t + r serves a query head of kv head r + 8 (t / g): all query
  // heads of a kv head, which read the same keys and values, share one XCD's L2.
  const int gq = a.hq / a.hkv;
  int hx = blockIdx.x;
  if (PF_XCD && gq > 1 && a.hkv % 8 == 0) {
    const int r = hx & 7, t = hx >> 3;
    hx = (r + 8 * (t / gq)) * gq + t % gq;
  }
  const int h = __builtin_amdgcn_readfirstlane(hx);
  // uniform (the integer division would otherwise leave it, and what depends on it, in VGPRs)
  const int kvh = __builtin_amdgcn_readfirstlane(h / gq);
  // ---- which (sequence, row tile) this workgroup owns ----------------------------------------
  // Slot y is the y-th row tile counted back from the last tile of the last sequence: the last
  // row tiles of the last sequences (the longest causal rows, hence the most key tiles) are
  // dispatched first and short ones fill the tail. One pass over the sequences, last first, one
  // sequence per thread: a wave prefix sum of the row-tile counts and the four wave totals give
  // each sequence's running count, and the thread whose sequence holds the slot publishes it with
  // its row offset, row count and context length (read in the same pass). Decode rows (one query
  // row) have no row tiles unless min_rows is 1 (the call runs no decode launch). Debug builds reject row offsets that are negative, decreasing or past
  // the batch, and treat such a sequence as empty.
  if (tid == 0) s_seq = -1;
  {
    const int slot = (int)(blockIdx.y + blockIdx.z * gridDim.y);
    int base = 0;  // row tiles of the sequences after this chunk
    for (int c0 = 0; c0 < a.num_seqs; c0 += kPfThreads) {
      const int sq = a.num_seqs - 1 - (c0 + tid);
      int nt = 0, cq0 = 0, cql = 0, cctx = 0;
      if (sq >= 0) {
        cq0 = a.cu[sq];
        const int c1 = a.cu[sq + 1];
        cctx = a.ctx_lens[sq];
        if (kDebugChecks && (cq0 < 0 || c1 < cq0 || c1 > a.num_tokens)) {
          debug_flag(DBG_RAGGED);
        } else {
          cql = c1 - cq0;
          nt = cql >= a.min_rows ? (cql + kPfRows - 1) / kPfRows : 0;
        }
      }
      int incl = nt;
#pragma unroll
      for (int d = 1; d < kWave; d <<= 1) {
        const int v = __shfl_up(incl, d);
        if (lane >= d) incl += v;
      }
      if (lane == kWave - 1) s_wtot[wave] = incl;
      __syncthreads();
      int total = 0;
#pragma unroll
      for (int w = 0; w < kPfThreads / kWave; ++w) {
        const int t = s_wtot[w];
        if (w < wave) incl += t;
        total += t;
      }
      const int target = slot - base;
      if (target < total) {  // uniform
        if (nt > 0 && incl > target && incl - nt <= target) {
          s_seq = sq;
          s_tile = nt - 1 - (target - (incl - nt));
          s_q0 = cq0;
          s_ql = cql;
          s_ctx = cctx;
        }
        break;
      }
      base += total;
      __syncthreads();  // s_wtot is rewritten by the next chunk
    }
  }
  __syncthreads();
  const int s = s_seq;
  if (s < 0) return;  // uniform: this slot of the launch has no tile
  const int q0 = s_q0;
  const int ql = s_ql;
  const int ctx = min(s_ctx, a.max_blocks * a.bs);  // contract: ctx fits the table
  const int row0 = s_tile * kPfRows;
  const int nrows = min(kPfRows, ql - row0);
  const int pos0 = ctx - ql + row0;      // position of the tile's first query row
  const int kend = pos0 + nrows;         // keys 0..kend-1 are visible to some row of the tile
  const int nkt = (kend + kPfKeys - 1) / kPfKeys;

  const int g = lane >> 4;   // lane group: k-slice of an operand / 4-row slice of a result
  const int lr = lane & 15;  // row (operand) or column (result) within a 16-tile

  // Q as the B operand of Sᵀ = K·Qᵀ: rows wave*32 + 16*nt + lr, dims 32*ks + 8*g .. +7.
  V8 qb[2][KS];
  int qpos[2];
  bool qvalid[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int r = wave * 32 + nt * 16 + lr;  // row within the tile
    qvalid[nt] = r < nrows;
    // A padding row (past the tile's last row) is masked like the last row, so it never sees a key
    // past the context: those keys' slots may hold anything, and its output is not stored, but
    // a non-finite value in it would still send the tile down the bf16 fallback path.
    qpos[nt] = pos0 + min(r, nrows - 1);
    const uint16_t* qp = a.q + ((size_t)(q0 + row0 + (qvalid[nt] ? r : 0)) * a.hq + h) * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 w = *reinterpret_cast<const u32x4*>(qp + 32 * ks);
      if (!qvalid[nt]) w = u32x4{0, 0, 0, 0};
      qb[nt][ks] = __builtin_bit_cast(V8, w);
    }
  }

  f32x4 oacc[DT16][2];
  float m_run[2];                              // reference max of each row (raw score units)
  const float lazy_thr = 8.f / a.scale_log2;  // 2^8 in probability terms, in raw score units
  // Row sums of the probabilities as MFMA'd (f16, or the bf16 parts): ones·Pᵀ accumulated beside
  // Oᵀ, so every element of a lane's accumulator holds its row's sum and the normaliser is taken
  // from the same rounded probabilities as the products.
  f32x4 lacc[2];

  const int32_t* trow = a.tables + (size_t)s * a.max_blocks;
  const uint32_t blk_elems = (uint32_t)(a.hkv * a.bs * D);  // elements of one pool block
  const uint32_t head_off = (uint32_t)(kvh * a.bs * D);      // this kv head's rows in a block
  const int nblk = (kend + a.bs - 1) >> a.log2_bs;

  // Position of this wave's last valid row; -1 (before every key) when the wave has none.
  const int wave_last_pos = wave * 32 < nrows ? pos0 + min(wave * 32 + 31, nrows - 1) : -1;

  // The key loop, in one of two modes for Oᵀ = Vᵀ·Pᵀ:
  //   kSplitP == false: Vᵀ as f16 in LDS (an f16 pool's values, or a bf16 pool's converted: exact
  //     for |v| in [2^-14, 65504], within 2^-25 below) and one f16 P rounded to nearest: one MFMA
  //     per step.
  //   kSplitP == true (bf16 pools only): Vᵀ as bf16 and P as a bf16 high part plus remainder: two
  //     MFMAs per step, exact for every bf16 value.
  // A bf16 pool runs the first mode; a value beyond the f16 range becomes infinite there and
  // reaches every output row of the tile as inf or NaN, and then the workgroup runs the key
  // loop again in the second mode.
  auto run_keys = [&](auto split_mode) {
    constexpr bool kSplitP = decltype(split_mode)::value;
    using PV = Mfma<kSplitP ? DT_BF16 : DT_F16>;
    using PV8 = typename PV::V8;
#pragma unroll
    for (int dt = 0; dt < DT16; ++dt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) oacc[dt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[0] = m_run[1] = -INFINITY;
    lacc[0] = lacc[1] = f32x4{0.f, 0.f, 0.f, 0.f};
    int tab_base = -kPfTab;  // first table entry held in s_tab

    // Global -> register staging of one key tile. Keys past kend are clamped to key kend-1 (a
    // written row, so finite): such keys are masked for every row that is stored, and their V
    // rows meet a zero probability. All loads are unconditional, so their table lookups and
    // addresses are computed together and the loads issue back to back.
    u32x4 kreg[KIT];
    u32x4 vreg[VIT][2];
    auto fetch = [&](int kt) {
      const int k0 = kt * kPfKeys;
      // K: in iteration it, wave w reads the 64 chunks it..., i.e. keys key0 .. key0 + 64/CPR - 1 of
      // the tile: 1 KiB that lies in one block (key0 is a multiple of 4 or 8, B of 8). Its base is
      // wave-uniform (table entry read at a uniform LDS address, scalar arithmetic); each lane adds
      // its own 16 bytes. A group past the context reads the last block's rows: those keys are
      // masked for every row of the tile (their scores may be NaN; masking selects).
      uint64_t kbase[KIT];
#pragma unroll
      for (int it = 0; it < KIT; ++it) {
        const int kk0 = k0 + (it * kPfThreads + kWave * wave) / CPR;  // uniform
        const int j = min(kk0 >> a.log2_bs, nblk - 1);
        const uint32_t phys = (uint32_t)__builtin_amdgcn_readfirstlane(s_tab[j - tab_base]);
        kbase[it] = (uint64_t)phys * blk_elems + head_off + (uint32_t)(kk0 & (a.bs - 1)) * D;
      }
      // Every V chunk of this thread covers the same key pair (kp = tid mod 32); the pair shares
      // a block because B is even.
      const int kv0 = min(k0 + 2 * (tid & (kPfKeys / 2 - 1)), kend - 1);
      const int kv1 = min(k0 + 2 * (tid & (kPfKeys / 2 - 1)) + 1, kend - 1);
      const uint32_t vphys = (uint32_t)s_tab[(kv0 >> a.log2_bs) - tab_base];
      const uint64_t vbase = (uint64_t)vphys * blk_elems + head_off;
      const uint32_t v0 = (uint32_t)(kv0 & (a.bs - 1)) * D, v1 = (uint32_t)(kv1 & (a.bs - 1)) * D;
#pragma unroll
      for (int it = 0; it < KIT; ++it) kreg[it] = *reinterpret_cast<const u32x4*>(a.kc + kbase[it] + 8 * lane);
#pragma unroll
      for (int it = 0; it < VIT; ++it) {
        const uint32_t ch8 = ((it * kPfThreads + tid) / (kPfKeys / 2)) * 8;
        vreg[it][0] = *reinterpret_cast<const u32x4*>(a.vc + (vbase + v0 + ch8));
        vreg[it][1] = *reinterpret_cast<const u32x4*>(a.vc + (vbase + v1 + ch8));
      }
    };
    // Registers -> LDS buffer b: K row-major, V transposed (word = two adjacent keys).
    auto stage = [&](int b) {
      uint16_t* k_dst = sK + b * KBUF;
      uint16_t* v_dst = sVt + b * VBUF;
#pragma unroll
      for (int it = 0; it < KIT; ++it) {
        const int idx = it * kPfThreads + tid;
        const int key = idx / CPR;
        const int ch = idx - key * CPR;
        *reinterpret_cast<u32x4*>(&k_dst[key * KLD + ch * 8]) = kreg[it];
      }
#pragma unroll
      for (int it = 0; it < VIT; ++it) {
        const int idx = it * kPfThreads + tid;
        const int kp = idx & (kPfKeys / 2 - 1);
        const int ch = idx / (kPfKeys / 2);
        const u32x4 w0 = vreg[it][0], w1 = vreg[it][1];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          uint32_t lo, hi;  // dims ch*8 + 2e and ch*8 + 2e + 1 of keys kv0 (low half), kv1
          if constexpr (DT == DT_BF16 && !kSplitP) {
            // bf16 -> f32 is a shift into the upper half; f32 -> f16 rounds to nearest
            lo = pack_f16(__uint_as_float(w0[e] << 16), __uint_as_float(w1[e] << 16));
            hi = pack_f16(__uint_as_float(w0[e] & 0xffff0000u), __uint_as_float(w1[e] & 0xffff0000u));
          } else {
            lo = __builtin_amdgcn_perm(w1[e], w0[e], 0x05040100u);  // low halves
            hi = __builtin_amdgcn_perm(w1[e], w0[e], 0x07060302u);  // high halves
          }
          *reinterpret_cast<uint32_t*>(&v_dst[(ch * 8 + 2 * e) * VLD + 2 * kp]) = lo;
          *reinterpret_cast<uint32_t*>(&v_dst[(ch * 8 + 2 * e + 1) * VLD + 2 * kp]) = hi;
        }
      }
    };
    // Makes s_tab hold the entries of key tiles kt (and kt+1 when it is in range). Uniform.
    auto ensure_table = [&](int kt) {
      const int jlo = (kt * kPfKeys) >> a.log2_bs;
      const int jhi = min(nblk, (min(kt + 2, nkt) * kPfKeys + a.bs - 1) >> a.log2_bs);
      if (jlo >= tab_base && jhi <= tab_base + kPfTab) return;
      __syncthreads();  // nobody still reads the old entries
      tab_base = jlo;
      for (int i = tid; i < kPfTab && jlo + i < nblk; i += kPfThreads) {
        int b = trow[jlo + i];
        if (kDebugChecks && (b < 0 || b >= a.num_blocks)) {
          debug_flag(DBG_BLOCK);
          b = 0;
        }
        s_tab[i] = b;
      }
      __syncthreads();
    };

    // Two LDS buffers: tile kt is computed from buffer kt&1 while tile kt+1 (loaded into registers
    // during the previous tile) is staged into the other one and tile kt+2's loads go out. One
    // barrier per tile separates a buffer's last reads from its next writes.
    if (nkt > 0) {  // nkt <= 0 only when a context is shorter than its query rows: nothing to read
      ensure_table(0);
      fetch(0);
      stage(0);
    }
    __syncthreads();
    if (nkt > 1) fetch(1);
    // Key tiles this wave computes: the rest (at most the last two of a causal row tile, or all
    // of them for a wave without valid rows) have every key masked for its rows.
    const int nkt_w = wave_last_pos < 0 ? 0 : min(nkt, wave_last_pos / kPfKeys + 1);
    for (int kt = 0; kt < nkt_w; ++kt) {
      const int k0 = kt * kPfKeys;
      const uint16_t* cK = sK + (kt & 1) * KBUF;
      const uint16_t* cV = sVt + (kt & 1) * VBUF;

#if PF_SETPRIO
      __builtin_amdgcn_s_setprio(PF_SETPRIO);  // MFMA phase: issue first, the other wave fills the gaps
#endif
      // ---- Sᵀ = K·Qᵀ: 4 key tiles x 2 row tiles -------------------------------------------------
      // Step st = (mt, ks) reads one K operand and feeds two MFMAs; operand reads run kPfLookahead
      // steps ahead of their MFMAs so that LDS latency overlaps matrix work. The steps go ks-major
      // (PF_ACC_ORDER).
      constexpr int NQK = 4 * KS;
      auto kread = [&](int st) {
        const int mt = PF_ACC_ORDER ? st % 4 : st / KS, ks = PF_ACC_ORDER ? st / 4 : st % KS;
        return __builtin_bit_cast(
            V8, *reinterpret_cast<const u32x4*>(&cK[(16 * mt + lr) * KLD + 32 * ks + 8 * g]));
      };
      f32x4 sacc[4][2];
      {
        V8 kop[kPfLookahead + 1];
#pragma unroll
        for (int i = 0; i < kPfLookahead; ++i) kop[i] = kread(i);
#pragma unroll
        for (int st = 0; st < NQK; ++st) {
          if (st + kPfLookahead < NQK) kop[(st + kPfLookahead) % (kPfLookahead + 1)] = kread(st + kPfLookahead);
          const int mt = PF_ACC_ORDER ? st % 4 : st / KS, ks = PF_ACC_ORDER ? st / 4 : st % KS;
          const V8 ka = kop[st % (kPfLookahead + 1)];
#pragma unroll
          for (int nt = 0; nt < 2; ++nt)
            sacc[mt][nt] = M::mma(ka, qb[nt][ks], ks == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : sacc[mt][nt]);
        }
#if PF_SCHED
        __builtin_amdgcn_sched_group_barrier(0x100, kPfLookahead, 1);
#pragma unroll
        for (int st = 0; st < NQK; ++st) {
          if (st + kPfLookahead < NQK) __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);
        }
#endif
      }

      // ---- causal mask and online softmax (per query row = per lane column) ----------------------
      // Scores stay unscaled here; exp2((s - m)·scale·log2 e) is one FMA per score. Only tiles that
      // reach past a wave's first row need the causal mask (a wave-uniform test).
#if PF_SETPRIO
      __builtin_amdgcn_s_setprio(0);
#endif
      const bool need_mask = k0 + kPfKeys - 1 > pos0 + wave * 32;
      // P operands [row tile][k-step of 32 keys]: the only part (f16) or the high part and the
      // remainder (bf16)
      PV8 phi[2][2], plo[2][2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        if (need_mask) {
          // key k0 + 16·mt + 4g + i is masked when 16·mt + i exceeds the row's threshold
          const int thr = qpos[nt] - k0 - 4 * g;
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (16 * mt + i > thr) sacc[mt][nt][i] = -INFINITY;
        }
        float mx = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          mx = fmaxf(fmaxf(mx, fmaxf(sacc[mt][nt][0], sacc[mt][nt][1])), fmaxf(sacc[mt][nt][2], sacc[mt][nt][3]));
        mx = max_rows4(mx);
        // Lazy rescaling: the reference max m_run only moves when some row's tile max exceeds it by
        // more than 2^8 in probability terms; until then probabilities may reach 2^8, which fp32
        // sums and the 16-bit split represent as well as values below 1.
        // The wave's first tile sets the reference max directly (the accumulators are still zero;
        // every row sees key 0, so the max is finite).
        const bool grow = mx > m_run[nt] + lazy_thr;
        if (kt == 0) {
          m_run[nt] = mx;
        } else if (__builtin_amdgcn_read_exec() & __ballot(grow)) {  // wave-uniform
          const float m_new = fmaxf(m_run[nt], mx);
          const float alpha = fast_exp2((m_run[nt] - m_new) * a.scale_log2);
          m_run[nt] = m_new;
          lacc[nt] *= alpha;
#pragma unroll
          for (int dt = 0; dt < DT16; ++dt) oacc[dt][nt] *= alpha;
        }
        // From the wave's first computed tile on, m_run is finite (every row, padding rows included,
        // sees key 0), so the offset and the rescale factor need no -inf case.
        const float off = -m_run[nt] * a.scale_log2;
        float p[4][4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) p[mt][i] = fast_exp2(__builtin_fmaf(sacc[mt][nt][i], a.scale_log2, off));
        // B operand of k-step j: keys 32j + 4g + (0..3) then 32j + 16 + 4g + (0..3); element e of
        // the operand is the low (e even) or high half of word e/2.
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          u32x4 hw, lw;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const int e = 2 * w;
            const float x0 = p[2 * j + (e >> 2)][e & 3], x1 = p[2 * j + (e >> 2)][(e & 3) + 1];
            if constexpr (kSplitP) {
              uint32_t h, l;
              split_pair_bf16(x0, x1, h, l);
              hw[w] = h;
              lw[w] = l;
            } else {
              hw[w] = pack_f16(x0, x1);
            }
          }
          phi[nt][j] = __builtin_bit_cast(PV8, hw);
          if constexpr (kSplitP) plo[nt][j] = __builtin_bit_cast(PV8, lw);
        }
      }

      // ---- the next tile goes to the other buffer; the one after it starts loading ---------------
      if (kt + 1 < nkt) {
        stage((kt + 1) & 1);
        if (kt + 2 < nkt) {
          ensure_table(kt + 2);
          fetch(kt + 2);
        }
      }

#if PF_SETPRIO
      __builtin_amdgcn_s_setprio(PF_SETPRIO);
#endif
      // ---- Oᵀ += Vᵀ·Pᵀ with the same key order in both operands ---------------------------------
      // Step st = (dt, j) reads one V operand and feeds two MFMAs per row tile with a split P (one
      // otherwise); reads run ahead as above. The steps go j-major (PF_ACC_ORDER).
      {
        constexpr int NPV = DT16 * 2;
        auto vread = [&](int st) {
          const int dt = PF_ACC_ORDER ? st % DT16 : st / 2, j = PF_ACC_ORDER ? st / DT16 : st % 2;
          const uint16_t* vrow = &cV[(16 * dt + lr) * VLD + 32 * j + 4 * g];
          const u32x2 x0 = *reinterpret_cast<const u32x2*>(vrow);
          const u32x2 x1 = *reinterpret_cast<const u32x2*>(vrow + 16);
          return __builtin_bit_cast(PV8, u32x4{x0[0], x0[1], x1[0], x1[1]});
        };
        PV8 vop[kPfLookahead + 1];
#pragma unroll
        for (int i = 0; i < kPfLookahead; ++i) vop[i] = vread(i);
#pragma unroll
        for (int st = 0; st < NPV; ++st) {
          if (st + kPfLookahead < NPV) vop[(st + kPfLookahead) % (kPfLookahead + 1)] = vread(st + kPfLookahead);
          const int dt = PF_ACC_ORDER ? st % DT16 : st / 2, j = PF_ACC_ORDER ? st / DT16 : st % 2;
          const PV8 va = vop[st % (kPfLookahead + 1)];
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) {
            oacc[dt][nt] = PV::mma(va, phi[nt][j], oacc[dt][nt]);
            if constexpr (kSplitP) oacc[dt][nt] = PV::mma(va, plo[nt][j], oacc[dt][nt]);
          }
        }
        // row sums: a ones operand against the same P operands (1.0 is 0x3c00 in f16, 0x3f80 in bf16)
        const uint32_t one2 = kSplitP ? 0x3f803f80u : 0x3c003c00u;
        const PV8 ones = __builtin_bit_cast(PV8, u32x4{one2, one2, one2, one2});
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) {
            lacc[nt] = PV::mma(ones, phi[nt][j], lacc[nt]);
            if constexpr (kSplitP) lacc[nt] = PV::mma(ones, plo[nt][j], lacc[nt]);
          }
#if PF_SCHED
        __builtin_amdgcn_sched_group_barrier(0x100, kPfLookahead, 2);
#pragma unroll
        for (int st = 0; st < NPV; ++st) {
          if (st + kPfLookahead < NPV) __builtin_amdgcn_sched_group_barrier(0x100, 1, 2);
          __builtin_amdgcn_sched_group_barrier(0x008, kSplitP ? 4 : 2, 2);
        }
#endif
      }
#if PF_SETPRIO
      __builtin_amdgcn_s_setprio(0);
#endif
      __syncthreads();  // buffer kt&1 is free for tile kt+2; buffer (kt+1)&1 is complete
    }
    // The masked tiles: no products or softmax, only this wave's share of the staging and the
    // same barriers as the other waves.
    for (int kt = nkt_w; kt < nkt; ++kt) {
      if (kt + 1 < nkt) {
        stage((kt + 1) & 1);
        if (kt + 2 < nkt) {
          ensure_table(kt + 2);
          fetch(kt + 2);
        }
      }
      __syncthreads();
    }
  };  // run_keys

  run_keys(std::false_type{});
  if constexpr (DT == DT_BF16) {
    // A value of V beyond the f16 range left inf or NaN in every row's output of this tile. The
    // test reads the exponent bits as an integer: this file is compiled assuming no NaN, so a
    // floating-point NaN test could be folded away.
    uint32_t bad = 0;
#pragma unroll
    for (int dt = 0; dt < DT16; ++dt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) bad |= (~__float_as_uint(oacc[dt][nt][i]) & 0x7f800000u) == 0u;
    if (__syncthreads_or((int)bad)) run_keys(std::true_type{});  // uniform over the workgroup
  }

  // ---- normalise and store ----------------------------------------------------------------------
#if PF_LDS_EPILOGUE
  if (a.out_dt != DT_F32) {
    // 16-bit output: the wave's 32 rows go through its share of the (now idle) K buffers as whole
    // rows, and leave as 16-byte stores, a row's 256 or 128 bytes contiguous.
    __syncthreads();  // every wave is done reading the K/V buffers
    constexpr int ORS = D + 8;  // LDS row stride (elements): rows start 16 bytes apart in the banks
    uint16_t* ot = sK + wave * 32 * ORS;
    static_assert(kPfRows * ORS <= 2 * KBUF, "output tile fits the K buffers");
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const float l = lacc[nt][0];
      const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
      for (int dt = 0; dt < DT16; ++dt) {
        const f32x4 v = oacc[dt][nt] * inv;
        uint32_t w0, w1;
        if (a.out_dt == DT_F16) {
          w0 = pack_f16(v[0], v[1]);
          w1 = pack_f16(v[2], v[3]);
        } else {
          w0 = f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16);
          w1 = f32_to_bf16_bits(v[2]) | ((uint32_t)f32_to_bf16_bits(v[3]) << 16);
        }
        *reinterpret_cast<u32x2*>(&ot[(nt * 16 + lr) * ORS + 16 * dt + 4 * g]) = u32x2{w0, w1};
      }
    }
    // Lane (chunk c, row r): 16-byte chunk c of row r; CPR chunks per row, 64 / CPR rows per pass.
    constexpr int RPP = kWave / CPR;
#pragma unroll
    for (int pass = 0; pass < 32 / RPP; ++pass) {
      const int r = pass * RPP + lane / CPR;
      const int c = lane % CPR;
      const int row = wave * 32 + r;
      if (row < nrows) {
        const u32x4 x = *reinterpret_cast<const u32x4*>(&ot[r * ORS + 8 * c]);
        *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.out) + ((size_t)(q0 + row0 + row) * a.hq + h) * D + 8 * c) = x;
      }
    }
    return;
  }
#endif
  // lane writes dims 16*dt + 4*g .. +3 of its row
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const float l = lacc[nt][0];
    if (!qvalid[nt]) continue;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const size_t orow = ((size_t)(q0 + wave * 32 + nt * 16 + lr + row0) * a.hq + h) * D;
#pragma unroll
    for (int dt = 0; dt < DT16; ++dt) store_out4(a.out, orow + 16 * dt + 4 * g, oacc[dt][nt] * inv, a.out_dt);
  }
}

template <int DT>
static hipError_t launch_prefill_dt(const PrefillLaunch& L, hipStream_t stream) {
  PrefillArgs a;
  a.out = L.out;
  a.q = static_cast<const uint16_t*>(L.q);
  a.kc = static_cast<const uint16_t*>(L.kc);
  a.vc = static_cast<const uint16_t*>(L.vc);
  a.tables = L.tables;
  a.cu = L.cu;
  a.ctx_lens = L.ctx_lens;
  a.out_dt = L.out_dt;
  a.max_blocks = L.max_blocks;
  a.num_seqs = L.num_seqs;
  a.hq = L.num_q_heads;
  a.hkv = L.num_kv_heads;
  a.bs = L.block_size;
  a.log2_bs = ilog2(L.block_size);
  a.scale_log2 = L.scale * 1.4426950408889634f;
  a.num_tokens = L.num_tokens;
  a.num_blocks = L.num_blocks;
  a.min_rows = L.min_rows;
  // Row tiles: sum over sequences of ceil(q_len / 128) <= T / 128 + (number of sequences with
  // at least min_rows rows, at most T / min_rows); slots past the real count exit at once.
  const int with_tiles = L.num_tokens / L.min_rows;
  const long long slots = (L.num_tokens + kPfRows - 1) / kPfRows + (L.num_seqs < with_tiles ? L.num_seqs : with_tiles);
  if (slots <= 0) return hipSuccess;
  // Heads are the fast grid dimension so the heaviest row tiles of every head go out first. Slots
  // run over y, then z (slot = y + z * gridDim.y keeps the dispatch order), so there is no limit
  // below the 2^31 row offsets: slots < T/128 + T + 1 < 65535^2.
  const unsigned gy = slots > 65535 ? 65535u : (unsigned)slots;
  const unsigned gz = (unsigned)((slots + gy - 1) / gy);
  const dim3 grid(L.num_q_heads, gy, gz);
  if (L.head_dim == 128) return launch_kernel(ragged_prefill_kernel<DT, 128>, grid, dim3(kPfThreads), stream, a);
  return launch_kernel(ragged_prefill_kernel<DT, 64>, grid, dim3(kPfThreads), stream, a);
}

hipError_t launch_ragged_prefill(const PrefillLaunch& L, hipStream_t stream) {
  if (L.min_rows != 1 && L.min_rows != 2) return hipErrorInvalidValue;
  if (L.dt == DT_BF16) return launch_prefill_dt<DT_BF16>(L, stream);
  if (L.dt == DT_F16) return launch_prefill_dt<DT_F16>(L, stream);
  return hipErrorInvalidConfiguration;
}

}  // namespace pkv
