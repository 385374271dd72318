// Host block manager for the paged KV cache: plain C++, no device calls.
//
// On-demand allocation from a free list, per-block reference counts and the copy-on-write
// decision ("PagedAttention: Efficient LLM Serving with vLLM", "The PagedAttention
// Algorithm" steps 1-4, "Memory Efficiency", and "Advanced Features" -> "KV-Cache Sharing
// (Copy-on-Write)").  The policy is stated in include/pkv.h.
//
// Per decode step the scheduler calls pkv_alloc_append_slots once for the whole batch; the
// slots go to pkv_reshape_and_cache and the (src, dst) pairs to pkv_copy_blocks, which must
// run first on the same stream.
//
// Prefix cache ("PagedAttention: Efficient LLM Serving with vLLM", "Advanced Features" ->
// "Prefix Caching": the KV blocks of a common prefix are kept and reused by later requests).
// A full prompt block is keyed by (key id of the previous block, its block_size token ids);
// key ids are never reused, so an entry whose chain was evicted can never match again.  An
// unreferenced cached block is not freed but parked in least-recently-freed order; blocks are
// handed out from the plain free list first and only then by evicting the oldest parked one.
#include "pkv.h"

#include <algorithm>
#include <cstring>
#include <list>
#include <map>
#include <new>
#include <unordered_map>
#include <vector>

struct pkv_alloc {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> free_stack;  // back() is handed out next
  std::vector<int32_t> ref;
  struct Seq {
    std::vector<int32_t> table;
    int32_t len = 0;
  };
  std::unordered_map<int64_t, Seq> seqs;

  // prefix cache
  using Key = std::pair<int64_t, std::vector<int32_t>>;  // (parent key id, tokens)
  std::map<Key, int32_t> index;                           // key -> block
  std::vector<int64_t> key_id;                            // per block; 0 = not cached
  std::vector<std::map<Key, int32_t>::iterator> key_of;   // per cached block
  std::list<int32_t> parked;                              // unreferenced cached, oldest first
  std::vector<std::list<int32_t>::iterator> park_pos;
  std::vector<char> is_parked;
  int64_t next_key = 1;

  int32_t available() const {
    return static_cast<int32_t>(free_stack.size() + parked.size());
  }
  void uncache(int32_t b) {
    index.erase(key_of[b]);
    key_id[b] = 0;
  }
  int32_t take() {
    int32_t b;
    if (!free_stack.empty()) {
      b = free_stack.back();
      free_stack.pop_back();
    } else {  // evict the least recently parked cached block
      b = parked.front();
      parked.pop_front();
      is_parked[b] = 0;
      uncache(b);
    }
    ref[b] = 1;
    return b;
  }
  void drop(int32_t b) {
    if (--ref[b] == 0) {
      if (key_id[b] != 0) {
        park_pos[b] = parked.insert(parked.end(), b);
        is_parked[b] = 1;
      } else {
        free_stack.push_back(b);
      }
    }
  }
  void reuse(int32_t b) {  // a cache hit: one more reference
    if (is_parked[b]) {
      parked.erase(park_pos[b]);
      is_parked[b] = 0;
    }
    ++ref[b];
  }
};

extern "C" {

pkv_alloc_t* pkv_alloc_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order) {
  if (num_blocks <= 0 || block_size <= 0) return nullptr;
  pkv_alloc_t* a = new (std::nothrow) pkv_alloc_t();
  if (!a) return nullptr;
  a->num_blocks = num_blocks;
  a->block_size = block_size;
  a->ref.assign(num_blocks, 0);
  a->key_id.assign(num_blocks, 0);
  a->key_of.resize(num_blocks);
  a->park_pos.resize(num_blocks);
  a->is_parked.assign(num_blocks, 0);
  a->free_stack.resize(num_blocks);
  if (free_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      int32_t b = free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete a;
        return nullptr;
      }
      seen[b] = 1;
      a->free_stack[num_blocks - 1 - i] = b;
    }
  } else {
    for (int32_t i = 0; i < num_blocks; ++i) a->free_stack[num_blocks - 1 - i] = i;
  }
  return a;
}

void pkv_alloc_destroy(pkv_alloc_t* a) { delete a; }

pkv_status_t pkv_alloc_add_seq(pkv_alloc_t* a, int64_t seq, int32_t len) {
  if (!a || len < 0 || a->seqs.count(seq)) return PKV_EINVAL;
  int64_t n = (static_cast<int64_t>(len) + a->block_size - 1) / a->block_size;
  if (n > a->available()) return PKV_ENOMEM;
  pkv_alloc::Seq s;
  s.len = len;
  s.table.reserve(static_cast<size_t>(n));
  for (int64_t i = 0; i < n; ++i) s.table.push_back(a->take());
  a->seqs.emplace(seq, std::move(s));
  return PKV_OK;
}

pkv_status_t pkv_alloc_fork(pkv_alloc_t* a, int64_t parent, int64_t child) {
  if (!a) return PKV_EINVAL;
  auto it = a->seqs.find(parent);
  if (it == a->seqs.end() || a->seqs.count(child)) return PKV_EINVAL;
  pkv_alloc::Seq c = it->second;
  for (int32_t b : c.table) ++a->ref[b];
  a->seqs.emplace(child, std::move(c));
  return PKV_OK;
}

pkv_status_t pkv_alloc_append_slot(pkv_alloc_t* a, int64_t seq, int32_t* slot, int32_t* cow_src,
                                   int32_t* cow_dst) {
  if (!a || !slot || !cow_src || !cow_dst) return PKV_EINVAL;
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return PKV_EINVAL;
  pkv_alloc::Seq& s = it->second;
  if (s.len == INT32_MAX) return PKV_EINVAL;
  const int32_t j = s.len / a->block_size;
  const int32_t off = s.len % a->block_size;
  int32_t src = -1, dst = -1;
  if (j == static_cast<int32_t>(s.table.size())) {
    if (a->available() == 0) return PKV_ENOMEM;
    s.table.push_back(a->take());
  } else if (a->ref[s.table[j]] > 1) {
    if (a->available() == 0) return PKV_ENOMEM;
    src = s.table[j];
    dst = a->take();
    --a->ref[src];
    s.table[j] = dst;
  }
  const int64_t sl = static_cast<int64_t>(s.table[j]) * a->block_size + off;
  *slot = static_cast<int32_t>(sl);
  *cow_src = src;
  *cow_dst = dst;
  ++s.len;
  return PKV_OK;
}

pkv_status_t pkv_alloc_append_slots(pkv_alloc_t* a, const int64_t* seqs, int32_t n,
                                    int32_t* slots, int32_t* cow_pairs, int32_t* num_cow,
                                    int32_t* num_done) {
  if (!a || n < 0 || (n > 0 && (!seqs || !slots || !cow_pairs)) || !num_cow || !num_done)
    return PKV_EINVAL;
  *num_cow = 0;
  *num_done = 0;
  for (int32_t i = 0; i < n; ++i) {
    int32_t src, dst;
    pkv_status_t st = pkv_alloc_append_slot(a, seqs[i], &slots[i], &src, &dst);
    if (st != PKV_OK) return st;
    if (src >= 0) {
      cow_pairs[2 * *num_cow] = src;
      cow_pairs[2 * *num_cow + 1] = dst;
      ++*num_cow;
    }
    ++*num_done;
  }
  return PKV_OK;
}

// The blocks pkv_alloc_append_slots(seqs) would take, without changing anything.
//
// Sequences listed once (the usual case): one new block per sequence whose length is a
// multiple of the block size; and for a block with r references that k listed sequences are
// about to write into, min(k, r - 1) copies (each writer but the last copies while the count
// is above one).  Sequences listed more than once: the same decisions, replayed on per-call
// copies of each listed sequence's length and table size and of the reference counts that
// copy-on-write lowers.
pkv_status_t pkv_alloc_append_need(const pkv_alloc_t* a, const int64_t* seqs, int32_t n,
                                   int32_t* blocks) {
  if (!a || n < 0 || (n > 0 && !seqs) || !blocks) return PKV_EINVAL;
  thread_local std::vector<int64_t> ids;
  thread_local std::vector<int32_t> shared;  // target blocks with more than one reference
  ids.assign(seqs, seqs + n);
  std::sort(ids.begin(), ids.end());
  const bool distinct = std::adjacent_find(ids.begin(), ids.end()) == ids.end();
  int64_t need = 0;
  if (distinct) {
    shared.clear();
    for (int32_t i = 0; i < n; ++i) {
      auto it = a->seqs.find(seqs[i]);
      if (it == a->seqs.end()) return PKV_EINVAL;
      const pkv_alloc::Seq& s = it->second;
      if (s.len == INT32_MAX) return PKV_EINVAL;
      const int32_t j = s.len / a->block_size;
      if (j == static_cast<int32_t>(s.table.size())) {
        ++need;
      } else if (a->ref[s.table[j]] > 1) {
        shared.push_back(s.table[j]);
      }
    }
    std::sort(shared.begin(), shared.end());
    for (size_t i = 0; i < shared.size();) {
      size_t k = i;
      while (k < shared.size() && shared[k] == shared[i]) ++k;
      need += std::min<int64_t>(static_cast<int64_t>(k - i), a->ref[shared[i]] - 1);
      i = k;
    }
  } else {
    struct Sim {
      const pkv_alloc::Seq* seq;
      int32_t len;
      int32_t table_size;
      bool last_private;  // an earlier append of this call left its last block unshared
    };
    std::unordered_map<int64_t, Sim> sims;
    std::unordered_map<int32_t, int32_t> lowered;  // block -> references dropped by copies
    for (int32_t i = 0; i < n; ++i) {
      auto it = sims.find(seqs[i]);
      if (it == sims.end()) {
        auto s = a->seqs.find(seqs[i]);
        if (s == a->seqs.end()) return PKV_EINVAL;
        it = sims.emplace(seqs[i], Sim{&s->second, s->second.len,
                                       static_cast<int32_t>(s->second.table.size()), false})
                 .first;
      }
      Sim& m = it->second;
      if (m.len == INT32_MAX) return PKV_EINVAL;
      const int32_t j = m.len / a->block_size;
      if (j == m.table_size) {
        ++need;  // a new block, held by this sequence alone
        ++m.table_size;
        m.last_private = true;
      } else if (!m.last_private) {
        const int32_t b = m.seq->table[j];
        if (a->ref[b] - lowered[b] > 1) {
          ++need;  // a fresh block for the copy; the shared one loses a reference
          ++lowered[b];
        }
        m.last_private = true;
      }
      ++m.len;
    }
  }
  *blocks = static_cast<int32_t>(std::min<int64_t>(need, INT32_MAX));
  return PKV_OK;
}

pkv_status_t pkv_alloc_free_seq(pkv_alloc_t* a, int64_t seq) {
  if (!a) return PKV_EINVAL;
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return PKV_EINVAL;
  const std::vector<int32_t>& t = it->second.table;
  for (auto b = t.rbegin(); b != t.rend(); ++b) a->drop(*b);
  a->seqs.erase(it);
  return PKV_OK;
}

// Batched forms: the same calls in order, stopping at the first error (returned), with
// *num_done the number of calls that succeeded.
pkv_status_t pkv_alloc_add_seqs(pkv_alloc_t* a, const int64_t* seqs, const int32_t* lens,
                                int32_t n, int32_t* num_done) {
  if (!a || n < 0 || (n > 0 && (!seqs || !lens)) || !num_done) return PKV_EINVAL;
  *num_done = 0;
  for (int32_t i = 0; i < n; ++i) {
    const pkv_status_t st = pkv_alloc_add_seq(a, seqs[i], lens[i]);
    if (st != PKV_OK) return st;
    ++*num_done;
  }
  return PKV_OK;
}

pkv_status_t pkv_alloc_fork_many(pkv_alloc_t* a, const int64_t* parents, const int64_t* children,
                                 int32_t n, int32_t* num_done) {
  if (!a || n < 0 || (n > 0 && (!parents || !children)) || !num_done) return PKV_EINVAL;
  *num_done = 0;
  for (int32_t i = 0; i < n; ++i) {
    const pkv_status_t st = pkv_alloc_fork(a, parents[i], children[i]);
    if (st != PKV_OK) return st;
    ++*num_done;
  }
  return PKV_OK;
}

pkv_status_t pkv_alloc_free_seqs(pkv_alloc_t* a, const int64_t* seqs, int32_t n,
                                 int32_t* num_done) {
  if (!a || n < 0 || (n > 0 && !seqs) || !num_done) return PKV_EINVAL;
  *num_done = 0;
  for (int32_t i = 0; i < n; ++i) {
    const pkv_status_t st = pkv_alloc_free_seq(a, seqs[i]);
    if (st != PKV_OK) return st;
    ++*num_done;
  }
  return PKV_OK;
}

pkv_status_t pkv_alloc_block_table(const pkv_alloc_t* a, int64_t seq, int32_t* out, int32_t cap,
                                   int32_t* n) {
  if (!a || !n || cap < 0 || (cap > 0 && !out)) return PKV_EINVAL;
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return PKV_EINVAL;
  const std::vector<int32_t>& t = it->second.table;
  *n = static_cast<int32_t>(t.size());
  const size_t m = std::min(t.size(), static_cast<size_t>(cap));
  if (m) std::memcpy(out, t.data(), m * sizeof(int32_t));
  return PKV_OK;
}

pkv_status_t pkv_alloc_export(const pkv_alloc_t* a, const int64_t* seqs, int32_t n,
                              int32_t max_blocks, int32_t* tables, int32_t* lens) {
  if (!a || n < 0 || max_blocks < 0 || (n > 0 && (!seqs || !tables || !lens))) return PKV_EINVAL;
  for (int32_t i = 0; i < n; ++i) {
    auto it = a->seqs.find(seqs[i]);
    if (it == a->seqs.end()) return PKV_EINVAL;
    const std::vector<int32_t>& t = it->second.table;
    if (static_cast<int64_t>(t.size()) > max_blocks) return PKV_EINVAL;
    int32_t* row = tables + static_cast<int64_t>(i) * max_blocks;
    std::copy(t.begin(), t.end(), row);
    std::fill(row + t.size(), row + max_blocks, -1);
    lens[i] = it->second.len;
  }
  return PKV_OK;
}

int32_t pkv_alloc_seq_len(const pkv_alloc_t* a, int64_t seq) {
  if (!a) return -1;
  auto it = a->seqs.find(seq);
  return it == a->seqs.end() ? -1 : it->second.len;
}

int32_t pkv_alloc_num_free(const pkv_alloc_t* a) { return a ? a->available() : -1; }

pkv_status_t pkv_alloc_move_seqs(pkv_alloc_t* from, pkv_alloc_t* to, const int64_t* seqs,
                                 int32_t n, int32_t* pairs, int32_t capacity,
                                 int32_t* num_pairs) {
  if (!from || !to || from == to || n < 0 || (n > 0 && !seqs) || !num_pairs || capacity < 0 ||
      from->block_size != to->block_size)
    return PKV_EINVAL;
  *num_pairs = 0;
  // every listed sequence exists in `from`, none in `to`, no duplicates
  std::unordered_map<int64_t, int> listed;
  for (int32_t i = 0; i < n; ++i) {
    if (!from->seqs.count(seqs[i]) || to->seqs.count(seqs[i]) || listed.count(seqs[i]))
      return PKV_EINVAL;
    listed[seqs[i]] = i;
  }
  // distinct blocks in first-use order, and their references from the listed sequences
  std::vector<int32_t> order;
  std::unordered_map<int32_t, int32_t> refs_listed;
  for (int32_t i = 0; i < n; ++i)
    for (int32_t b : from->seqs[seqs[i]].table)
      if (refs_listed[b]++ == 0) order.push_back(b);
  for (const auto& kv : refs_listed)
    if (kv.second != from->ref[kv.first]) return PKV_EINVAL;  // shared with an unlisted seq
  const int32_t m = static_cast<int32_t>(order.size());
  if (m > capacity || (m > 0 && !pairs)) return PKV_EINVAL;
  if (m > to->available()) return PKV_ENOMEM;
  std::unordered_map<int32_t, int32_t> map;
  for (int32_t k = 0; k < m; ++k) {
    const int32_t d = to->take();
    to->ref[d] = 0;  // set below from the moved tables
    map[order[k]] = d;
    pairs[2 * k] = order[k];
    pairs[2 * k + 1] = d;
  }
  for (int32_t i = 0; i < n; ++i) {
    auto it = from->seqs.find(seqs[i]);
    pkv_alloc::Seq moved;
    moved.len = it->second.len;
    for (int32_t b : it->second.table) {
      moved.table.push_back(map[b]);
      ++to->ref[map[b]];
    }
    const std::vector<int32_t>& t = it->second.table;
    for (auto b = t.rbegin(); b != t.rend(); ++b) from->drop(*b);
    from->seqs.erase(it);
    to->seqs.emplace(seqs[i], std::move(moved));
  }
  *num_pairs = m;
  return PKV_OK;
}

int32_t pkv_alloc_num_cached(const pkv_alloc_t* a) {
  return a ? static_cast<int32_t>(a->index.size()) : -1;
}

pkv_status_t pkv_alloc_add_seq_cached(pkv_alloc_t* a, int64_t seq, const int32_t* tokens,
                                      int32_t len, int32_t* cached_tokens) {
  if (!a || len < 0 || (len > 0 && !tokens) || !cached_tokens || a->seqs.count(seq))
    return PKV_EINVAL;
  const int32_t BS = a->block_size;
  const int32_t full = len / BS;
  const int32_t n = (len + BS - 1) / BS;
  // 1. the longest chain of cached full blocks
  std::vector<int32_t> hits;
  int64_t parent = 0;
  for (int32_t j = 0; j < full; ++j) {
    pkv_alloc::Key key(parent, std::vector<int32_t>(tokens + static_cast<size_t>(j) * BS,
                                                    tokens + static_cast<size_t>(j + 1) * BS));
    auto it = a->index.find(key);
    if (it == a->index.end()) break;
    hits.push_back(it->second);
    parent = a->key_id[it->second];
  }
  // 2. room for the rest (a hit on a parked block takes it off the parked list)
  int32_t parked_hits = 0;
  for (int32_t b : hits) parked_hits += a->is_parked[b] ? 1 : 0;
  if (n - static_cast<int32_t>(hits.size()) > a->available() - parked_hits) return PKV_ENOMEM;
  pkv_alloc::Seq s;
  s.len = len;
  s.table.reserve(static_cast<size_t>(n));
  for (int32_t b : hits) {
    a->reuse(b);
    s.table.push_back(b);
  }
  // 3. fresh blocks; full ones are registered (the caller fills them before any later lookup)
  for (int32_t j = static_cast<int32_t>(hits.size()); j < n; ++j) {
    const int32_t b = a->take();
    s.table.push_back(b);
    if (j < full) {
      pkv_alloc::Key key(parent, std::vector<int32_t>(tokens + static_cast<size_t>(j) * BS,
                                                      tokens + static_cast<size_t>(j + 1) * BS));
      auto ins = a->index.emplace(std::move(key), b);
      a->key_of[b] = ins.first;
      a->key_id[b] = a->next_key++;
      parent = a->key_id[b];
    }
  }
  *cached_tokens = static_cast<int32_t>(hits.size()) * BS;
  a->seqs.emplace(seq, std::move(s));
  return PKV_OK;
}

int32_t pkv_alloc_refcount(const pkv_alloc_t* a, int32_t block) {
  if (!a || block < 0 || block >= a->num_blocks) return -1;
  return a->ref[block];
}

int64_t pkv_alloc_wasted_slots(const pkv_alloc_t* a) {
  if (!a) return -1;
  std::vector<int32_t> fill(a->num_blocks, 0);
  for (const auto& kv : a->seqs) {
    const auto& s = kv.second;
    for (size_t j = 0; j < s.table.size(); ++j) {
      int64_t in_block = static_cast<int64_t>(s.len) - static_cast<int64_t>(j) * a->block_size;
      int32_t f = static_cast<int32_t>(std::min<int64_t>(a->block_size, in_block));
      fill[s.table[j]] = std::max(fill[s.table[j]], f);
    }
  }
  int64_t w = 0;
  for (int32_t b = 0; b < a->num_blocks; ++b)
    if (a->ref[b] > 0) w += a->block_size - fill[b];
  return w;
}

}  // extern "C"
