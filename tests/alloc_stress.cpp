// Randomized stress of the host block manager through its C ABI, built with AddressSanitizer
// and UndefinedBehaviorSanitizer by tests/test_alloc_sanitized.py.  After every operation:
// the sum of reference counts equals the number of table entries, free + used = pool size,
// and every table holds ceil(len / block_size) valid ids; an append batch takes exactly the
// blocks pkv_alloc_append_need predicted, and fails for lack of blocks exactly when it said so.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <random>
#include <vector>

#include "pkv.h"

static int fail(const char* what, int step) {
  std::printf("FAIL %s at step %d\n", what, step);
  return 1;
}

int main(int argc, char** argv) {
  const int steps = argc > 1 ? std::atoi(argv[1]) : 20000;
  std::mt19937_64 rng(12345);
  const int32_t NB = 257, BS = 16;
  std::vector<int32_t> order(NB);
  for (int32_t i = 0; i < NB; ++i) order[i] = (i * 97) % NB;
  pkv_alloc_t* a = pkv_alloc_create(NB, BS, order.data());
  if (!a) return fail("create", -1);
  pkv_alloc_t* b = pkv_alloc_create(NB, BS, nullptr);
  if (!b) return fail("create default", -1);
  pkv_alloc_destroy(b);
  std::vector<int32_t> dup(NB, 0);  // not a permutation: refused
  if (pkv_alloc_create(NB, BS, dup.data()) != nullptr) return fail("create dup", -1);
  std::vector<int64_t> live;
  int64_t next = 0;
  std::vector<int32_t> table(4096);
  for (int step = 0; step < steps; ++step) {
    const int op = static_cast<int>(rng() % 12);
    if (op >= 10) {  // prompt from a small vocabulary so prefixes repeat and hit the cache
      std::vector<int32_t> toks(static_cast<size_t>(1 + rng() % (3 * BS)));
      for (auto& t : toks) t = static_cast<int32_t>(rng() % 3);
      int32_t cached = -1;
      pkv_status_t st =
          pkv_alloc_add_seq_cached(a, next, toks.data(), static_cast<int32_t>(toks.size()), &cached);
      if (st == PKV_OK) {
        live.push_back(next);
        if (cached < 0 || cached % BS || cached > static_cast<int32_t>(toks.size()))
          return fail("cached tokens", step);
      } else if (st != PKV_ENOMEM) {
        return fail("add_seq_cached status", step);
      }
      ++next;
    } else if ((op < 2 || live.empty()) && rng() % 2) {
      int32_t len = static_cast<int32_t>(rng() % (4 * BS));
      pkv_status_t st = pkv_alloc_add_seq(a, next, len);
      if (st == PKV_OK) live.push_back(next);
      else if (st != PKV_ENOMEM) return fail("add_seq status", step);
      ++next;
    } else if (op < 2 || live.empty()) {  // batched: up to 3 new sequences in one call
      const int32_t n = static_cast<int32_t>(1 + rng() % 3);
      std::vector<int64_t> ids(n);
      std::vector<int32_t> lens(n);
      for (int32_t i = 0; i < n; ++i) {
        ids[i] = next++;
        lens[i] = static_cast<int32_t>(rng() % (4 * BS));
      }
      int32_t done = -1;
      pkv_status_t st = pkv_alloc_add_seqs(a, ids.data(), lens.data(), n, &done);
      if ((st != PKV_OK && st != PKV_ENOMEM) || done < 0 || done > n ||
          (st == PKV_OK && done != n))
        return fail("add_seqs status", step);
      for (int32_t i = 0; i < done; ++i) live.push_back(ids[i]);
    } else if (op < 4 && rng() % 2) {
      int64_t p = live[rng() % live.size()];
      if (pkv_alloc_fork(a, p, next) != PKV_OK) return fail("fork", step);
      live.push_back(next++);
    } else if (op < 4) {  // batched: up to 4 children of random parents in one call
      const int32_t n = static_cast<int32_t>(1 + rng() % 4);
      std::vector<int64_t> parents(n), children(n);
      for (int32_t i = 0; i < n; ++i) {
        parents[i] = live[rng() % live.size()];
        children[i] = next++;
      }
      int32_t done = -1;
      if (pkv_alloc_fork_many(a, parents.data(), children.data(), n, &done) != PKV_OK ||
          done != n)
        return fail("fork_many", step);
      for (int64_t c : children) live.push_back(c);
    } else if (op < 5 && (rng() % 2 || live.size() < 2)) {
      size_t i = rng() % live.size();
      if (pkv_alloc_free_seq(a, live[i]) != PKV_OK) return fail("free", step);
      live.erase(live.begin() + static_cast<long>(i));
    } else if (op < 5) {  // batched: the last two live sequences in one call
      std::vector<int64_t> ids(live.end() - 2, live.end());
      int32_t done = -1;
      if (pkv_alloc_free_seqs(a, ids.data(), 2, &done) != PKV_OK || done != 2)
        return fail("free_seqs", step);
      live.resize(live.size() - 2);
    } else {
      const int32_t n = static_cast<int32_t>(std::min<size_t>(live.size(), 1 + rng() % 6));
      std::vector<int64_t> seqs(live.begin(), live.begin() + n);
      if (rng() % 3 == 0) seqs.push_back(seqs[0]);  // a sequence listed twice
      const int32_t m = static_cast<int32_t>(seqs.size());
      std::vector<int32_t> slots(m), pairs(2 * m);
      int32_t need = -1, ncow = -1, ndone = -1;
      if (pkv_alloc_append_need(a, seqs.data(), m, &need) != PKV_OK || need < 0 || need > m)
        return fail("append_need", step);
      const int32_t free_before = pkv_alloc_num_free(a);
      pkv_status_t st =
          pkv_alloc_append_slots(a, seqs.data(), m, slots.data(), pairs.data(), &ncow, &ndone);
      if (st != PKV_OK && st != PKV_ENOMEM) return fail("append status", step);
      if ((st == PKV_OK) != (need <= free_before)) return fail("append_need vs ENOMEM", step);
      if (st == PKV_OK && free_before - pkv_alloc_num_free(a) != need)
        return fail("append_need vs blocks taken", step);
      for (int32_t i = 0; i < ndone; ++i)
        if (slots[i] < 0 || slots[i] >= NB * BS) return fail("slot range", step);
      for (int32_t i = 0; i < ncow; ++i)
        if (pairs[2 * i] == pairs[2 * i + 1]) return fail("pair", step);
    }
    // invariants
    std::map<int32_t, int32_t> refs;
    int64_t entries = 0;
    for (int64_t s : live) {
      int32_t n = 0;
      if (pkv_alloc_block_table(a, s, table.data(), static_cast<int32_t>(table.size()), &n) != PKV_OK)
        return fail("block_table", step);
      const int32_t len = pkv_alloc_seq_len(a, s);
      if (n != (len + BS - 1) / BS) return fail("table length", step);
      for (int32_t j = 0; j < n; ++j) {
        if (table[j] < 0 || table[j] >= NB) return fail("block id", step);
        ++refs[table[j]];
        ++entries;
      }
    }
    int64_t sum = 0, used = 0;
    for (int32_t b = 0; b < NB; ++b) {
      const int32_t r = pkv_alloc_refcount(a, b);
      auto it = refs.find(b);
      if (r != (it == refs.end() ? 0 : it->second)) return fail("refcount", step);
      sum += r;
      used += r > 0;
    }
    if (sum != entries) return fail("ref sum", step);
    if (used + pkv_alloc_num_free(a) != NB) return fail("free + used", step);
    if (pkv_alloc_num_cached(a) < 0 || pkv_alloc_num_cached(a) > NB) return fail("cached", step);
    if (pkv_alloc_wasted_slots(a) < 0) return fail("waste", step);
  }
  // error paths
  int32_t slot, src, dst;
  if (pkv_alloc_append_slot(a, -42, &slot, &src, &dst) != PKV_EINVAL) return fail("unknown", -1);
  if (pkv_alloc_free_seq(a, -42) != PKV_EINVAL) return fail("unknown free", -1);
  if (pkv_alloc_add_seq(nullptr, 1, 1) != PKV_EINVAL) return fail("null", -1);
  int32_t done = -1;
  const int64_t bad[2] = {-42, -43};
  if (pkv_alloc_free_seqs(a, bad, 2, &done) != PKV_EINVAL || done != 0)
    return fail("unknown free_seqs", -1);
  if (pkv_alloc_fork_many(a, bad, bad, 1, nullptr) != PKV_EINVAL) return fail("null done", -1);
  pkv_alloc_destroy(a);
  std::printf("ok %d steps, %lld sequences\n", steps, static_cast<long long>(next));
  return 0;
}
