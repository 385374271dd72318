// Host-side checks of the decode step's arguments and of the index data it uploads: plain C++,
// no device calls, so every error path can be exercised without a GPU.
//
// Preconditions the device calls cannot check themselves ("PagedAttention: Efficient LLM
// Serving with vLLM", "The PagedAttention Algorithm", step 2: each new token fills its own
// slot; "Advanced Features" -> "KV-Cache Sharing (Copy-on-Write)": a shared block is copied to
// a fresh one before the write):
//   - the slots of one cache append are distinct (two tokens in one slot leave either value);
//   - the destinations of one block copy are distinct and none is also a source (a copy would
//     otherwise read a block another copy of the same launch writes).
// pkv_stepper_step runs these on the index data it is about to upload, and
// pkv_stepper_check before it changes anything.
#include "pkv.h"
#include "pkv_internal.h"

#include <algorithm>
#include <cmath>
#include <vector>

namespace pkv {

bool slots_distinct(const int32_t* slots, int32_t n, int64_t num_slots,
                    std::vector<int32_t>& scratch) {
  scratch.clear();
  for (int32_t i = 0; i < n; ++i)
    if (slots[i] >= 0 && slots[i] < num_slots) scratch.push_back(slots[i]);  // others: skipped
  std::sort(scratch.begin(), scratch.end());
  return std::adjacent_find(scratch.begin(), scratch.end()) == scratch.end();
}

bool copy_pairs_valid(const int32_t* pairs, int32_t n, int32_t num_blocks,
                      std::vector<int64_t>& scratch) {
  // (block, role) keys, role 0 = source, 1 = destination, of the pairs a copy performs
  scratch.clear();
  for (int32_t p = 0; p < n; ++p) {
    const int32_t src = pairs[2 * p], dst = pairs[2 * p + 1];
    if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) continue;  // skipped
    scratch.push_back(2 * static_cast<int64_t>(src));
    scratch.push_back(2 * static_cast<int64_t>(dst) + 1);
  }
  std::sort(scratch.begin(), scratch.end());
  // a block named as a destination must appear exactly once among all keys
  for (size_t i = 0; i < scratch.size(); ++i) {
    if ((scratch[i] & 1) == 0) continue;
    const int64_t blk = scratch[i] >> 1;
    const bool dup_before = i > 0 && (scratch[i - 1] >> 1) == blk;
    const bool dup_after = i + 1 < scratch.size() && (scratch[i + 1] >> 1) == blk;
    if (dup_before || dup_after) return false;
  }
  return true;
}

}  // namespace pkv

extern "C" {

pkv_status_t pkv_check_slot_mapping(const pkv_cache_desc_t* desc, const int32_t* slots,
                                    int32_t num_tokens) {
  if (!desc || desc->num_blocks <= 0 || desc->block_size <= 0 || num_tokens < 0 ||
      (num_tokens > 0 && !slots))
    return PKV_EINVAL;
  std::vector<int32_t> scratch;
  const int64_t num_slots = static_cast<int64_t>(desc->num_blocks) * desc->block_size;
  return pkv::slots_distinct(slots, num_tokens, num_slots, scratch) ? PKV_OK : PKV_EINVAL;
}

pkv_status_t pkv_check_copy_pairs(const pkv_cache_desc_t* desc, const int32_t* pairs,
                                  int32_t num_pairs) {
  if (!desc || desc->num_blocks <= 0 || num_pairs < 0 || (num_pairs > 0 && !pairs))
    return PKV_EINVAL;
  std::vector<int64_t> scratch;
  return pkv::copy_pairs_valid(pairs, num_pairs, desc->num_blocks, scratch) ? PKV_OK
                                                                             : PKV_EINVAL;
}

pkv_status_t pkv_stepper_check(const pkv_alloc_t* alloc, const pkv_cache_desc_t* desc,
                               int32_t max_seqs, int32_t max_blocks_per_seq, const int64_t* seqs,
                               int32_t n, const pkv_layer_io_t* io, const void* workspace,
                               size_t workspace_bytes, int32_t* max_len) {
  if (!alloc || !io || !max_len) return PKV_EINVAL;
  *max_len = 0;
  pkv_status_t st = pkv::check_desc(desc);
  if (st != PKV_OK) return st;
  if (max_seqs <= 0 || max_blocks_per_seq <= 0 || n < 0 || n > max_seqs || (n > 0 && !seqs) ||
      io->num_layers < 0)
    return PKV_EINVAL;
  if (n == 0) return PKV_OK;
  const int32_t L = io->num_layers;
  if (L > 0 && (!io->k_pools || !io->v_pools || !io->q || !io->k_new || !io->v_new || !io->out))
    return PKV_EINVAL;
  if (L > 0 && !std::isfinite(io->scale)) return PKV_EINVAL;
  auto misaligned = [](const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 != 0; };
  for (int32_t l = 0; l < L; ++l)
    if (!io->k_pools[l] || !io->v_pools[l] || !io->k_new[l] || !io->v_new[l] || !io->q[l] ||
        !io->out[l] || misaligned(io->k_new[l]) || misaligned(io->v_new[l]) ||
        misaligned(io->k_pools[l]) || misaligned(io->v_pools[l]))
      return PKV_EINVAL;

  // every sequence known and listed once; its length after the append fits the table width
  thread_local std::vector<int64_t> sorted;
  sorted.assign(seqs, seqs + n);
  std::sort(sorted.begin(), sorted.end());
  if (std::adjacent_find(sorted.begin(), sorted.end()) != sorted.end()) return PKV_EINVAL;
  int64_t longest = 0;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t len = pkv_alloc_seq_len(alloc, seqs[i]);
    if (len < 0 || len == INT32_MAX) return PKV_EINVAL;
    const int64_t after = static_cast<int64_t>(len) + 1;
    if ((after + desc->block_size - 1) / desc->block_size > max_blocks_per_seq) return PKV_EINVAL;
    longest = std::max(longest, after);
  }
  *max_len = static_cast<int32_t>(longest);

  // the pool holds every block the append takes
  int32_t need = 0;
  st = pkv_alloc_append_need(alloc, seqs, n, &need);
  if (st != PKV_OK) return st;
  if (need > pkv_alloc_num_free(alloc)) return PKV_ENOMEM;

  // the attention launches: grid size and split-context workspace
  if (L > 0) {
    if (n > (1 << 20)) return PKV_EUNSUPPORTED;
    const int32_t part = pkv_decode_partition_tokens(desc, n, *max_len);
    const int64_t parts = part > 0 ? (*max_len + part - 1) / part : 1;
    if (static_cast<int64_t>(n) * parts * desc->num_heads > INT32_MAX) return PKV_EUNSUPPORTED;
    const size_t ws = pkv_decode_workspace_bytes(desc, n, *max_len);
    if (ws > 0) {
      if (!workspace || workspace_bytes < ws) return PKV_ENOMEM;
      if (misaligned(workspace)) return PKV_EINVAL;
    }
  }
  return PKV_OK;
}

}  // extern "C"
