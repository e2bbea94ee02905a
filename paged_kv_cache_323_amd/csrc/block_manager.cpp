// Host block manager: block tables, reference counts and copy-on-write decisions.
//
// Plain C++ with no HIP dependency (it also builds with g++ for host-only testing). The rules
// follow the pages:
//   - 「PagedAttention原理」 §从虚拟内存的启发: a sequence takes one block of B slots at a time,
//     only when its last block is full, so waste stays inside one block;
//   - 「PagedAttention原理」 §实现一个虚拟内存: per sequence, the physical block of each logical
//     block plus the number of filled slots;
//   - 「PagedAttention原理」 §解决COW: writing into a block whose reference count is 1 goes in
//     place; otherwise allocate a new block, record (old, new) for the device copy, remap the
//     logical block, drop the old block's count and write into the new block;
//   - 「Paged Attention&Orca Paper笔记与解读」 §PagedAttention的方法: fork shares every block of
//     the parent (count + 1); free drops counts and releases blocks that reach zero;
//   - 「PagedAttention原理」 §all-or-nothing 调度: an append either succeeds for every sequence of
//     the batch or changes nothing.
// Tie-breaks (any choice is valid; this one is the documented, reproducible contract): free
// blocks come from the head of the creation-time order, released blocks join its tail in
// logical-block order, sequences are served in the order given.
#include <stdint.h>

#include <deque>
#include <new>
#include <unordered_map>
#include <vector>

#include "../../include/pagedkv.h"

namespace {

struct Seq {
  std::vector<int32_t> table;
  int32_t len = 0;
};

}  // namespace

struct pkv_bm {
  int32_t num_blocks = 0;
  int32_t B = 0;
  std::deque<int32_t> free_list;
  std::vector<int32_t> rc;
  std::unordered_map<int64_t, Seq> seqs;

  int32_t take() {
    const int32_t b = free_list.front();
    free_list.pop_front();
    rc[b] = 1;
    return b;
  }

  // New blocks an append would take, simulating the batch in order (a sequence may appear
  // more than once). cow_out counts copy-on-write pairs. Returns <0 on an unknown sequence.
  int64_t preflight(const int64_t* ids, const int32_t* n, int32_t count, int64_t* cow_out) const {
    std::unordered_map<int64_t, int32_t> sim_len;     // length after earlier entries
    std::unordered_map<int64_t, bool> sim_private;    // last block already private this batch
    std::unordered_map<int32_t, int32_t> rc_delta;
    int64_t need = 0, cow = 0;
    for (int32_t i = 0; i < count; ++i) {
      auto it = seqs.find(ids[i]);
      if (it == seqs.end()) return PKV_ENOSEQ;
      if (n[i] < 0) return PKV_EINVAL;
      if (n[i] == 0) continue;
      const Seq& sq = it->second;
      auto ls = sim_len.find(ids[i]);
      const int64_t len = ls == sim_len.end() ? sq.len : ls->second;
      bool priv = sim_private.count(ids[i]) ? sim_private[ids[i]] : false;
      if (len % B != 0 && !priv) {
        const int32_t b = sq.table[len / B];
        const int32_t eff = rc[b] + rc_delta[b];
        if (eff > 1) {
          ++need;
          ++cow;
          --rc_delta[b];
        }
        priv = true;  // from here on the last block is this sequence's own
      }
      const int64_t before = (len + B - 1) / B;
      const int64_t after = (len + n[i] + B - 1) / B;
      if (after > before) priv = true;
      need += after - before;
      if (len + n[i] > INT32_MAX) return PKV_EINVAL;
      sim_len[ids[i]] = (int32_t)(len + n[i]);
      sim_private[ids[i]] = priv;
    }
    if (cow_out) *cow_out = cow;
    return need;
  }
};

extern "C" {

pkv_bm* pkv_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order) {
  if (num_blocks <= 0 || block_size <= 0) return nullptr;
  if ((int64_t)num_blocks * block_size > INT32_MAX) return nullptr;
  pkv_bm* bm = new (std::nothrow) pkv_bm();
  if (!bm) return nullptr;
  bm->num_blocks = num_blocks;
  bm->B = block_size;
  bm->rc.assign(num_blocks, 0);
  std::vector<char> seen(num_blocks, 0);
  for (int32_t i = 0; i < num_blocks; ++i) {
    const int32_t b = free_order ? free_order[i] : i;
    if (b < 0 || b >= num_blocks || seen[b]) {
      delete bm;
      return nullptr;
    }
    seen[b] = 1;
    bm->free_list.push_back(b);
  }
  return bm;
}

void pkv_bm_destroy(pkv_bm* bm) { delete bm; }

int32_t pkv_bm_add_seq(pkv_bm* bm, int64_t id) {
  if (!bm) return PKV_EINVAL;
  if (bm->seqs.count(id)) return PKV_EEXIST;
  bm->seqs.emplace(id, Seq());
  return PKV_OK;
}

int32_t pkv_bm_fork(pkv_bm* bm, int64_t parent, int64_t child) {
  if (!bm) return PKV_EINVAL;
  auto it = bm->seqs.find(parent);
  if (it == bm->seqs.end()) return PKV_ENOSEQ;
  if (bm->seqs.count(child)) return PKV_EEXIST;
  Seq c = it->second;  // copy before emplace may rehash
  for (int32_t b : c.table) bm->rc[b] += 1;
  bm->seqs.emplace(child, std::move(c));
  return PKV_OK;
}

int32_t pkv_bm_free_seq(pkv_bm* bm, int64_t id) {
  if (!bm) return PKV_EINVAL;
  auto it = bm->seqs.find(id);
  if (it == bm->seqs.end()) return PKV_ENOSEQ;
  for (int32_t b : it->second.table) {
    if (--bm->rc[b] == 0) bm->free_list.push_back(b);
  }
  bm->seqs.erase(it);
  return PKV_OK;
}

int64_t pkv_bm_blocks_needed(const pkv_bm* bm, const int64_t* ids, const int32_t* n, int32_t count) {
  if (!bm || count < 0 || (count > 0 && (!ids || !n))) return PKV_EINVAL;
  return bm->preflight(ids, n, count, nullptr);
}

int32_t pkv_bm_append(pkv_bm* bm, const int64_t* ids, const int32_t* n, int32_t count, int32_t* slots_out,
                      int32_t* cow_pairs_out, int32_t max_pairs, int32_t* num_pairs_out) {
  if (!bm || count < 0 || (count > 0 && (!ids || !n))) return PKV_EINVAL;
  int64_t cow = 0;
  const int64_t need = bm->preflight(ids, n, count, &cow);
  if (need < 0) return (int32_t)need;
  int64_t total = 0;
  for (int32_t i = 0; i < count; ++i) total += n[i];
  if (total > 0 && !slots_out) return PKV_EINVAL;
  if (cow > 0 && (!cow_pairs_out || cow > max_pairs)) return PKV_EINVAL;
  if (need > (int64_t)bm->free_list.size()) return PKV_ENOBLOCKS;

  const int32_t B = bm->B;
  int64_t w = 0;
  int32_t np = 0;
  for (int32_t i = 0; i < count; ++i) {
    Seq& sq = bm->seqs.find(ids[i])->second;
    for (int32_t k = 0; k < n[i]; ++k) {
      const int32_t p = sq.len;
      const int32_t j = p / B;
      const int32_t off = p % B;
      if (j == (int32_t)sq.table.size()) {
        sq.table.push_back(bm->take());  // previous block full (or none yet): fresh block
      } else if (bm->rc[sq.table[j]] > 1) {
        const int32_t old = sq.table[j];  // shared partial block: copy-on-write
        const int32_t nb = bm->take();
        cow_pairs_out[2 * np] = old;
        cow_pairs_out[2 * np + 1] = nb;
        ++np;
        sq.table[j] = nb;
        bm->rc[old] -= 1;
      }
      slots_out[w++] = sq.table[j] * B + off;
      sq.len = p + 1;
    }
  }
  if (num_pairs_out) *num_pairs_out = np;
  return PKV_OK;
}

int32_t pkv_bm_block_tables(const pkv_bm* bm, const int64_t* ids, int32_t count, int32_t max_blocks,
                            int32_t* tables_out, int32_t* ctx_out) {
  if (!bm || count < 0 || max_blocks < 0 || (count > 0 && (!ids || !tables_out))) return PKV_EINVAL;
  for (int32_t i = 0; i < count; ++i) {
    auto it = bm->seqs.find(ids[i]);
    if (it == bm->seqs.end()) return PKV_ENOSEQ;
    if ((int32_t)it->second.table.size() > max_blocks) return PKV_ESHAPE;
  }
  for (int32_t i = 0; i < count; ++i) {
    const Seq& sq = bm->seqs.find(ids[i])->second;
    int32_t* row = tables_out + (int64_t)i * max_blocks;
    const int32_t nt = (int32_t)sq.table.size();
    for (int32_t j = 0; j < max_blocks; ++j) row[j] = j < nt ? sq.table[j] : -1;
    if (ctx_out) ctx_out[i] = sq.len;
  }
  return PKV_OK;
}

int32_t pkv_bm_seq_table(const pkv_bm* bm, int64_t id, int32_t* out, int32_t cap) {
  if (!bm) return PKV_EINVAL;
  auto it = bm->seqs.find(id);
  if (it == bm->seqs.end()) return PKV_ENOSEQ;
  const int32_t nt = (int32_t)it->second.table.size();
  for (int32_t j = 0; j < nt && j < cap; ++j) out[j] = it->second.table[j];
  return nt;
}

int32_t pkv_bm_context_len(const pkv_bm* bm, int64_t id) {
  if (!bm) return PKV_EINVAL;
  auto it = bm->seqs.find(id);
  return it == bm->seqs.end() ? PKV_ENOSEQ : it->second.len;
}

int32_t pkv_bm_refcount(const pkv_bm* bm, int32_t block) {
  if (!bm || block < 0 || block >= bm->num_blocks) return PKV_EINVAL;
  return bm->rc[block];
}

int32_t pkv_bm_num_free(const pkv_bm* bm) { return bm ? (int32_t)bm->free_list.size() : PKV_EINVAL; }

int32_t pkv_bm_free_list(const pkv_bm* bm, int32_t* out, int32_t cap) {
  if (!bm) return PKV_EINVAL;
  int32_t i = 0;
  for (int32_t b : bm->free_list) {
    if (i < cap) out[i] = b;
    ++i;
  }
  return i;
}

}  // extern "C"
