// Stress program for the host block manager, built with AddressSanitizer and UBSan by
// tests/test_bm_sanitize.py (host code only; no HIP).
//
// A seeded random script of add / fork / append (batches with repeated sequences) / free /
// swap-out / swap-in / table export drives the C API. After every operation it checks the
// bookkeeping invariants against its own recount:
//   - a block's reference count equals the number of tables (of sequences in its pool) that
//     name it;
//   - the free list holds exactly the blocks with count 0, each once, and num_free agrees;
//   - a sequence's table has ceil(len / B) entries and every appended slot lies in the table
//     entry of its position;
//   - a call that fails leaves the manager unchanged.
// Exit status 0 means every check passed; a failed check prints what differed.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <vector>

#include "pagedkv.h"

namespace {

uint64_t g_state;
uint64_t next_u64() {  // splitmix64
  uint64_t z = (g_state += 0x9e3779b97f4a7c15ull);
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}
int rnd(int n) { return (int)(next_u64() % (uint64_t)n); }

int g_failures = 0;
#define CHECK(cond, ...)                          \
  do {                                            \
    if (!(cond)) {                                \
      std::fprintf(stderr, "check failed: " __VA_ARGS__); \
      std::fprintf(stderr, "\n");                 \
      if (++g_failures > 20) std::exit(2);        \
    }                                             \
  } while (0)

constexpr int N = 64, HN = 48, B = 8;

std::vector<int32_t> table_of(pkv_bm* bm, int64_t s) {
  std::vector<int32_t> t(4096);
  const int32_t n = pkv_bm_seq_table(bm, s, t.data(), (int32_t)t.size());
  t.resize(n > 0 ? n : 0);
  return t;
}

// Recounts references per pool from the tables and compares with the manager's view.
void check_invariants(pkv_bm* bm, const std::map<int64_t, bool>& live) {
  std::vector<int> refs(N, 0), hrefs(HN, 0);
  for (const auto& kv : live) {
    const int64_t s = kv.first;
    const int32_t res = pkv_bm_is_resident(bm, s);
    CHECK(res == 0 || res == 1, "is_resident(%lld) = %d", (long long)s, res);
    const std::vector<int32_t> t = table_of(bm, s);
    const int32_t len = pkv_bm_context_len(bm, s);
    CHECK((int32_t)t.size() == (len + B - 1) / B, "seq %lld: %zu blocks for length %d", (long long)s, t.size(), len);
    for (int32_t b : t) {
      if (res == 1) {
        CHECK(b >= 0 && b < N, "seq %lld: GPU block %d out of range", (long long)s, b);
        if (b >= 0 && b < N) refs[b]++;
      } else {
        CHECK(b >= 0 && b < HN, "seq %lld: host block %d out of range", (long long)s, b);
        if (b >= 0 && b < HN) hrefs[b]++;
      }
    }
  }
  std::vector<int32_t> fl(N + 1), hfl(HN + 1);
  const int32_t nf = pkv_bm_free_list(bm, fl.data(), (int32_t)fl.size());
  const int32_t nhf = pkv_bm_host_free_list(bm, hfl.data(), (int32_t)hfl.size());
  CHECK(nf == pkv_bm_num_free(bm), "free list %d vs num_free %d", nf, pkv_bm_num_free(bm));
  std::vector<int> in_free(N, 0), in_hfree(HN, 0);
  for (int i = 0; i < nf; ++i) {
    CHECK(fl[i] >= 0 && fl[i] < N, "free list entry %d", fl[i]);
    if (fl[i] >= 0 && fl[i] < N) in_free[fl[i]]++;
  }
  for (int i = 0; i < nhf; ++i) {
    CHECK(hfl[i] >= 0 && hfl[i] < HN, "host free list entry %d", hfl[i]);
    if (hfl[i] >= 0 && hfl[i] < HN) in_hfree[hfl[i]]++;
  }
  for (int b = 0; b < N; ++b) {
    CHECK(pkv_bm_refcount(bm, b) == refs[b], "block %d: count %d, tables name it %d times", b,
          pkv_bm_refcount(bm, b), refs[b]);
    CHECK(in_free[b] == (refs[b] == 0 ? 1 : 0), "block %d: on the free list %d times with %d refs", b,
          in_free[b], refs[b]);
  }
  for (int b = 0; b < HN; ++b) {
    CHECK(pkv_bm_host_refcount(bm, b) == hrefs[b], "host block %d: count %d vs %d", b,
          pkv_bm_host_refcount(bm, b), hrefs[b]);
    CHECK(in_hfree[b] == (hrefs[b] == 0 ? 1 : 0), "host block %d: free %d times with %d refs", b, in_hfree[b],
          hrefs[b]);
  }
}

// The parts of the manager's state a failed call must leave untouched.
std::vector<int32_t> snapshot(pkv_bm* bm, const std::map<int64_t, bool>& live) {
  std::vector<int32_t> out(N + 1);
  out.resize(pkv_bm_free_list(bm, out.data(), (int32_t)out.size()));
  for (const auto& kv : live) {
    out.push_back(pkv_bm_context_len(bm, kv.first));
    out.push_back(pkv_bm_is_resident(bm, kv.first));
    for (int32_t b : table_of(bm, kv.first)) out.push_back(b);
  }
  for (int b = 0; b < N; ++b) out.push_back(pkv_bm_refcount(bm, b));
  return out;
}

std::vector<int64_t> pick(const std::map<int64_t, bool>& live, int want_resident, int max_n, bool distinct,
                          pkv_bm* bm) {
  std::vector<int64_t> cand;
  for (const auto& kv : live)
    if (want_resident < 0 || pkv_bm_is_resident(bm, kv.first) == want_resident) cand.push_back(kv.first);
  std::vector<int64_t> out;
  if (cand.empty()) return out;
  const int n = 1 + rnd(max_n);
  for (int i = 0; i < n; ++i) {
    const int64_t s = cand[rnd((int)cand.size())];
    bool dup = false;
    for (int64_t x : out) dup |= x == s;
    if (distinct && dup) continue;
    out.push_back(s);
  }
  return out;
}

}  // namespace

int main(int argc, char** argv) {
  g_state = argc > 1 ? std::strtoull(argv[1], nullptr, 10) : 1;
  const int steps = argc > 2 ? std::atoi(argv[2]) : 20000;
  std::vector<int32_t> order(N), horder(HN);
  for (int i = 0; i < N; ++i) order[i] = i;
  for (int i = N - 1; i > 0; --i) std::swap(order[i], order[rnd(i + 1)]);
  for (int i = 0; i < HN; ++i) horder[i] = i;
  pkv_bm* bm = pkv_bm_create(N, B, order.data());
  CHECK(bm != nullptr, "create");
  CHECK(pkv_bm_attach_host_pool(bm, HN, horder.data()) == PKV_OK, "attach");
  std::map<int64_t, bool> live;
  int64_t next_id = 0;
  std::vector<int32_t> slots(4096), pairs(4096), tables(64 * 512), ctx(64);
  int ok_ops = 0;
  for (int step = 0; step < steps; ++step) {
    const int op = rnd(100);
    if (op < 12 || live.empty()) {  // add
      CHECK(pkv_bm_add_seq(bm, next_id) == PKV_OK, "add %lld", (long long)next_id);
      CHECK(pkv_bm_add_seq(bm, next_id) == PKV_EEXIST, "duplicate add");
      live[next_id++] = true;
    } else if (op < 20) {  // fork
      const std::vector<int64_t> p = pick(live, 1, 1, true, bm);
      if (!p.empty()) {
        const int32_t st = pkv_bm_fork(bm, p[0], next_id);
        CHECK(st == PKV_OK, "fork %lld: %d", (long long)p[0], st);
        if (st == PKV_OK) live[next_id++] = true;
      }
    } else if (op < 60) {  // append, possibly with repeated sequences and zero counts
      const std::vector<int64_t> ids = pick(live, 1, 6, false, bm);
      if (ids.empty()) continue;
      std::vector<int32_t> n(ids.size());
      int64_t total = 0;
      for (auto& x : n) {
        x = rnd(3) == 0 ? rnd(24) : rnd(3);
        total += x;
      }
      std::vector<int32_t> len_before;
      for (int64_t s : ids) len_before.push_back(pkv_bm_context_len(bm, s));
      const int64_t need = pkv_bm_blocks_needed(bm, ids.data(), n.data(), (int32_t)ids.size());
      const std::vector<int32_t> before = snapshot(bm, live);
      int32_t np = 0;
      const int32_t st = pkv_bm_append(bm, ids.data(), n.data(), (int32_t)ids.size(), slots.data(), pairs.data(),
                                       (int32_t)ids.size(), &np);
      if (st == PKV_OK) {
        CHECK(need <= pkv_bm_num_free(bm) + need, "need");
        // every slot lies in its position's table entry
        std::map<int64_t, int32_t> pos;
        int64_t w = 0;
        for (size_t i = 0; i < ids.size(); ++i) {
          const int64_t s = ids[i];
          if (!pos.count(s)) pos[s] = len_before[i];
          const std::vector<int32_t> t = table_of(bm, s);
          for (int k = 0; k < n[i]; ++k, ++w) {
            const int32_t p = pos[s]++;
            CHECK(p / B < (int32_t)t.size() && slots[w] == t[p / B] * B + p % B, "slot of seq %lld pos %d",
                  (long long)s, p);
          }
        }
        CHECK(w == total, "slot count");
        ++ok_ops;
      } else {
        CHECK(st == PKV_ENOBLOCKS, "append status %d", st);
        CHECK(snapshot(bm, live) == before, "failed append changed the manager");
      }
    } else if (op < 72) {  // free
      const std::vector<int64_t> p = pick(live, -1, 1, true, bm);
      if (!p.empty()) {
        CHECK(pkv_bm_free_seq(bm, p[0]) == PKV_OK, "free");
        live.erase(p[0]);
        CHECK(pkv_bm_free_seq(bm, p[0]) == PKV_ENOSEQ, "double free");
      }
    } else if (op < 84) {  // swap out a set
      const std::vector<int64_t> ids = pick(live, 1, 3, true, bm);
      if (ids.empty()) continue;
      const std::vector<int32_t> before = snapshot(bm, live);
      int32_t np = 0;
      const int32_t st = pkv_bm_swap_out(bm, ids.data(), (int32_t)ids.size(), pairs.data(), 2048, &np);
      if (st != PKV_OK) {
        CHECK(st == PKV_ENOBLOCKS, "swap_out status %d", st);
        CHECK(snapshot(bm, live) == before, "failed swap_out changed the manager");
      }
    } else if (op < 94) {  // swap in a set
      const std::vector<int64_t> ids = pick(live, 0, 3, true, bm);
      if (ids.empty()) continue;
      const std::vector<int32_t> before = snapshot(bm, live);
      int32_t np = 0;
      const int32_t st = pkv_bm_swap_in(bm, ids.data(), (int32_t)ids.size(), pairs.data(), 2048, &np);
      if (st != PKV_OK) {
        CHECK(st == PKV_ENOBLOCKS, "swap_in status %d", st);
        CHECK(snapshot(bm, live) == before, "failed swap_in changed the manager");
      }
    } else {  // table export of resident sequences, and error paths that must change nothing
      const std::vector<int64_t> ids = pick(live, 1, 8, false, bm);
      if (!ids.empty()) {
        const int32_t st = pkv_bm_block_tables(bm, ids.data(), (int32_t)ids.size(), 512, tables.data(), ctx.data());
        CHECK(st == PKV_OK || st == PKV_ESHAPE, "tables status %d", st);
        if (st == PKV_OK)
          for (size_t i = 0; i < ids.size(); ++i) {
            const std::vector<int32_t> t = table_of(bm, ids[i]);
            for (int j = 0; j < 512; ++j)
              CHECK(tables[i * 512 + j] == (j < (int)t.size() ? t[j] : -1), "table export entry");
            CHECK(ctx[i] == pkv_bm_context_len(bm, ids[i]), "ctx export");
          }
      }
      const std::vector<int32_t> before = snapshot(bm, live);
      const int64_t ghost = next_id + 1000;
      const int32_t bad_n = -1;
      int32_t np = 0;
      CHECK(pkv_bm_append(bm, &ghost, &bad_n, 1, slots.data(), pairs.data(), 1, &np) != PKV_OK, "bad append");
      CHECK(pkv_bm_fork(bm, ghost, next_id) == PKV_ENOSEQ, "fork of unknown");
      CHECK(snapshot(bm, live) == before, "an error path changed the manager");
    }
    check_invariants(bm, live);
  }
  pkv_bm_destroy(bm);
  std::printf("ok: %d steps, %d successful appends, %d failures\n", steps, ok_ops, g_failures);
  return g_failures ? 1 : 0;
}
