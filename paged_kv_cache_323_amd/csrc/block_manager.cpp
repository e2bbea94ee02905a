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
//     the batch or changes nothing;
//   - 「PagedAttention原理」 §抢占与恢复 / §swap, 「Paged Attention&Orca Paper笔记与解读」
//     §PagedAttention的方法 (eviction to CPU memory): a set of sequences is swapped between the GPU
//     pool and a host swap pool as a whole or not at all; a swapped-out sequence cannot run, grow
//     or be forked. A block also referenced by a sequence outside the set is copied (its count
//     drops by the set's references) instead of moved.
// Tie-breaks (any choice is valid; this one is the documented, reproducible contract): free
// blocks come from the head of the creation-time order, released blocks join its tail in
// logical-block order, sequences are served in the order given.
#include <stdint.h>

#include <deque>
#include <new>
#include <algorithm>
#include <unordered_map>
#include <vector>

#include "../../include/pagedkv.h"

namespace {

struct Seq {
  std::vector<int32_t> table;  // GPU block ids, or host block ids while swapped out
  int32_t len = 0;
  bool on_host = false;
  // Scratch of the batch simulation in preflight(), valid while sim_epoch equals the manager's
  // current epoch (so no per-call maps are needed).
  mutable uint64_t sim_epoch = 0;
  mutable int32_t sim_len = 0;
  mutable bool sim_private = false;
};

}  // namespace

struct pkv_bm {
  int32_t num_blocks = 0;
  int32_t B = 0;
  std::deque<int32_t> free_list;
  std::vector<int32_t> rc;
  std::unordered_map<int64_t, Seq> seqs;
  int32_t num_host_blocks = 0;
  std::deque<int32_t> host_free;
  std::vector<int32_t> host_rc;
  // preflight() scratch: a batch number, and per block the batch that last changed its simulated
  // reference count and that change.
  mutable uint64_t epoch = 0;
  mutable std::vector<uint64_t> rc_epoch;
  mutable std::vector<int32_t> rc_delta;

  // Moves the blocks of a set of sequences to the other pool (see the file comment). On
  // success writes (src, dst) pairs in first-reference order.
  int32_t move(const int64_t* ids, int32_t count, bool to_host, int32_t* pairs_out, int32_t max_pairs,
               int32_t* num_pairs_out) {
    if (count < 0 || (count > 0 && !ids)) return PKV_EINVAL;
    std::vector<Seq*> set;
    set.reserve(count);
    for (int32_t i = 0; i < count; ++i) {
      auto it = seqs.find(ids[i]);
      if (it == seqs.end()) return PKV_ENOSEQ;
      if (it->second.on_host == to_host) return PKV_ENOTRESIDENT;
      for (int32_t k = 0; k < i; ++k)
        if (ids[k] == ids[i]) return PKV_EINVAL;
      set.push_back(&it->second);
    }
    std::vector<int32_t>& src_rc = to_host ? rc : host_rc;
    std::deque<int32_t>& src_free = to_host ? free_list : host_free;
    std::vector<int32_t>& dst_rc = to_host ? host_rc : rc;
    std::deque<int32_t>& dst_free = to_host ? host_free : free_list;
    std::vector<int32_t> order;
    std::unordered_map<int32_t, int32_t> refs;
    for (Seq* sq : set)
      for (int32_t b : sq->table) {
        auto r = refs.find(b);
        if (r == refs.end()) {
          refs.emplace(b, 1);
          order.push_back(b);
        } else {
          ++r->second;
        }
      }
    if ((int64_t)order.size() > (int64_t)dst_free.size()) return PKV_ENOBLOCKS;
    if (!order.empty() && (!pairs_out || (int64_t)order.size() > max_pairs)) return PKV_EINVAL;
    std::unordered_map<int32_t, int32_t> mapping;
    for (size_t i = 0; i < order.size(); ++i) {
      const int32_t nb = dst_free.front();
      dst_free.pop_front();
      dst_rc[nb] = refs[order[i]];
      mapping[order[i]] = nb;
      pairs_out[2 * i] = order[i];
      pairs_out[2 * i + 1] = nb;
    }
    for (Seq* sq : set) {
      for (int32_t& b : sq->table) b = mapping[b];
      sq->on_host = to_host;
    }
    for (int32_t b : order) {
      src_rc[b] -= refs[b];
      if (src_rc[b] == 0) src_free.push_back(b);
    }
    if (num_pairs_out) *num_pairs_out = (int32_t)order.size();
    return PKV_OK;
  }

  int32_t take() {
    const int32_t b = free_list.front();
    free_list.pop_front();
    rc[b] = 1;
    return b;
  }

  // New blocks an append would take, simulating the batch in order (a sequence may appear
  // more than once). cow_out counts copy-on-write pairs. Returns <0 on an unknown sequence.
  int64_t preflight(const int64_t* ids, const int32_t* n, int32_t count, int64_t* cow_out) const {
    const uint64_t ep = ++epoch;  // a sequence's or block's sim_* fields count only if stamped ep
    if (rc_epoch.size() != rc.size()) {
      rc_epoch.assign(rc.size(), 0);
      rc_delta.assign(rc.size(), 0);
    }
    int64_t need = 0, cow = 0;
    for (int32_t i = 0; i < count; ++i) {
      auto it = seqs.find(ids[i]);
      if (it == seqs.end()) return PKV_ENOSEQ;
      if (n[i] < 0) return PKV_EINVAL;
      if (it->second.on_host) return PKV_ENOTRESIDENT;
      if (n[i] == 0) continue;
      const Seq& sq = it->second;
      if (sq.sim_epoch != ep) {  // first entry of this sequence in the batch
        sq.sim_epoch = ep;
        sq.sim_len = sq.len;      // length after earlier entries
        sq.sim_private = false;   // last block already private this batch
      }
      const int64_t len = sq.sim_len;
      bool priv = sq.sim_private;
      if (len % B != 0 && !priv) {
        const int32_t b = sq.table[len / B];
        const int32_t delta = rc_epoch[b] == ep ? rc_delta[b] : 0;
        if (rc[b] + delta > 1) {
          ++need;
          ++cow;
          rc_epoch[b] = ep;
          rc_delta[b] = delta - 1;
        }
        priv = true;  // from here on the last block is this sequence's own
      }
      const int64_t before = (len + B - 1) / B;
      const int64_t after = (len + n[i] + B - 1) / B;
      if (after > before) priv = true;
      need += after - before;
      if (len + n[i] > INT32_MAX) return PKV_EINVAL;
      sq.sim_len = (int32_t)(len + n[i]);
      sq.sim_private = priv;
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

pkv_bm* pkv_bm_clone(const pkv_bm* bm) {
  if (!bm) return nullptr;
  try {
    return new pkv_bm(*bm);  // every member is a value: the copy shares nothing with the original
  } catch (const std::bad_alloc&) {
    return nullptr;
  }
}

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
  if (it->second.on_host) return PKV_ENOTRESIDENT;
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
  std::vector<int32_t>& rc = it->second.on_host ? bm->host_rc : bm->rc;
  std::deque<int32_t>& fl = it->second.on_host ? bm->host_free : bm->free_list;
  for (int32_t b : it->second.table) {
    if (--rc[b] == 0) fl.push_back(b);
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
  return pkv_bm_block_tables_ex(bm, ids, count, max_blocks, tables_out, ctx_out, 1);
}

int32_t pkv_bm_block_tables_ex(const pkv_bm* bm, const int64_t* ids, int32_t count, int32_t max_blocks,
                               int32_t* tables_out, int32_t* ctx_out, int32_t pad) {
  if (!bm || count < 0 || max_blocks < 0 || (count > 0 && (!ids || !tables_out))) return PKV_EINVAL;
  for (int32_t i = 0; i < count; ++i) {
    auto it = bm->seqs.find(ids[i]);
    if (it == bm->seqs.end()) return PKV_ENOSEQ;
    if (it->second.on_host) return PKV_ENOTRESIDENT;
    if ((int32_t)it->second.table.size() > max_blocks) return PKV_ESHAPE;
  }
  for (int32_t i = 0; i < count; ++i) {
    const Seq& sq = bm->seqs.find(ids[i])->second;
    int32_t* row = tables_out + (int64_t)i * max_blocks;
    const int32_t nt = (int32_t)sq.table.size();
    std::copy(sq.table.begin(), sq.table.end(), row);
    if (pad) std::fill(row + nt, row + max_blocks, -1);
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

int32_t pkv_bm_attach_host_pool(pkv_bm* bm, int32_t num_host_blocks, const int32_t* free_order) {
  if (!bm || num_host_blocks <= 0 || bm->num_host_blocks) return PKV_EINVAL;
  std::vector<char> seen(num_host_blocks, 0);
  std::deque<int32_t> fl;
  for (int32_t i = 0; i < num_host_blocks; ++i) {
    const int32_t b = free_order ? free_order[i] : i;
    if (b < 0 || b >= num_host_blocks || seen[b]) return PKV_EINVAL;
    seen[b] = 1;
    fl.push_back(b);
  }
  bm->num_host_blocks = num_host_blocks;
  bm->host_free.swap(fl);
  bm->host_rc.assign(num_host_blocks, 0);
  return PKV_OK;
}

int32_t pkv_bm_swap_out(pkv_bm* bm, const int64_t* seq_ids, int32_t n, int32_t* pairs_out, int32_t max_pairs,
                        int32_t* num_pairs_out) {
  if (!bm || !bm->num_host_blocks) return PKV_EINVAL;
  return bm->move(seq_ids, n, true, pairs_out, max_pairs, num_pairs_out);
}

int32_t pkv_bm_swap_in(pkv_bm* bm, const int64_t* seq_ids, int32_t n, int32_t* pairs_out, int32_t max_pairs,
                       int32_t* num_pairs_out) {
  if (!bm || !bm->num_host_blocks) return PKV_EINVAL;
  return bm->move(seq_ids, n, false, pairs_out, max_pairs, num_pairs_out);
}

int32_t pkv_bm_is_resident(const pkv_bm* bm, int64_t id) {
  if (!bm) return PKV_EINVAL;
  auto it = bm->seqs.find(id);
  return it == bm->seqs.end() ? PKV_ENOSEQ : (it->second.on_host ? 0 : 1);
}

int32_t pkv_bm_host_refcount(const pkv_bm* bm, int32_t block) {
  if (!bm || block < 0 || block >= bm->num_host_blocks) return PKV_EINVAL;
  return bm->host_rc[block];
}

int32_t pkv_bm_host_free_list(const pkv_bm* bm, int32_t* out, int32_t cap) {
  if (!bm) return PKV_EINVAL;
  int32_t i = 0;
  for (int32_t b : bm->host_free) {
    if (i < cap) out[i] = b;
    ++i;
  }
  return i;
}

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
