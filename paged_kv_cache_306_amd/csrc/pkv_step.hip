// Decode-step driver: one decode iteration of a batch over every layer in one host call
// ("PagedAttention: Efficient LLM Serving with vLLM", "The PagedAttention Algorithm",
// steps 1-5).  Host code only: the block manager decides slots and copy-on-write pairs, the
// packed index data goes to the device in one asynchronous copy, then the cache-write and
// attention kernels are launched per layer on the caller's stream.
#include "pkv.h"
#include "pkv_internal.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <new>
#include <vector>

// Two stages are used alternately.  Stage k owns a pinned host area and a device area of
// d_index.  The upload of step i runs on the stepper's own copy stream after the kernels of
// step i-2 (the last reader of the same device area) and before the kernels of step i, so it
// overlaps the kernels of step i-1 whenever the host runs ahead of the device.
struct pkv_stepper {
  pkv_alloc_t* alloc = nullptr;
  pkv_cache_desc_t desc{};
  int32_t max_seqs = 0;
  int32_t max_blocks = 0;
  int32_t max_items = 0;  // decode work items per step, at most
  hipStream_t copy_stream = nullptr;
  std::vector<int32_t> keys, sorted_keys;  // per-step scratch for the sharing test
  struct Stage {
    int32_t* host = nullptr;      // pinned: tables | lens | slots | pairs (packed for n)
    char* dev = nullptr;          // device area of the same size inside d_index
    hipEvent_t copied = nullptr;  // recorded on the copy stream after the upload
    hipEvent_t consumed = nullptr;  // recorded on the caller's stream after the kernels
    bool copy_pending = false;
    bool used = false;
  } stage[2];
  int cur = 0;
};

namespace {

// Most decode work items n sequences with tables of max_blocks entries can produce.
int32_t max_work_items(const pkv_cache_desc_t* d, int32_t n, int32_t max_blocks) {
  const int64_t cap = static_cast<int64_t>(max_blocks) * d->block_size;
  const int32_t max_ctx = static_cast<int32_t>(std::min<int64_t>(cap, INT32_MAX));
  const int32_t part = pkv_decode_partition_tokens(d, n, max_ctx);
  const int64_t parts = part > 0 ? (max_ctx + part - 1) / part : 1;
  return static_cast<int32_t>(std::min<int64_t>(static_cast<int64_t>(n) * parts, INT32_MAX / 8));
}

size_t index_ints(int32_t n, int32_t max_blocks, int32_t max_items) {
  // tables [n][max_blocks], lens [n], slots [n], pairs [n][2], work items [max_items]
  return static_cast<size_t>(n) * max_blocks + 4 * static_cast<size_t>(n) + max_items;
}

}  // namespace

extern "C" {

static size_t stage_bytes(int32_t max_seqs, int32_t max_blocks_per_seq, int32_t max_items) {
  return static_cast<size_t>(pkv::align_up(
      static_cast<int64_t>(index_ints(max_seqs, max_blocks_per_seq, max_items) * 4), 256));
}

size_t pkv_stepper_index_bytes(const pkv_cache_desc_t* desc, int32_t max_seqs,
                               int32_t max_blocks_per_seq) {
  if (pkv::check_desc(desc) != PKV_OK || max_seqs <= 0 || max_blocks_per_seq <= 0) return 0;
  return 2 * stage_bytes(max_seqs, max_blocks_per_seq,
                         max_work_items(desc, max_seqs, max_blocks_per_seq));
}

pkv_stepper_t* pkv_stepper_create(pkv_alloc_t* alloc, const pkv_cache_desc_t* desc,
                                  int32_t max_seqs, int32_t max_blocks_per_seq, void* d_index) {
  if (!alloc || pkv::check_desc(desc) != PKV_OK || max_seqs <= 0 || max_blocks_per_seq <= 0 ||
      !d_index || reinterpret_cast<uintptr_t>(d_index) % 16)
    return nullptr;
  pkv_stepper_t* st = new (std::nothrow) pkv_stepper_t();
  if (!st) return nullptr;
  st->alloc = alloc;
  st->desc = *desc;
  st->max_seqs = max_seqs;
  st->max_blocks = max_blocks_per_seq;
  st->max_items = max_work_items(desc, max_seqs, max_blocks_per_seq);
  const size_t bytes = stage_bytes(max_seqs, max_blocks_per_seq, st->max_items);
  if (hipStreamCreateWithFlags(&st->copy_stream, hipStreamNonBlocking) != hipSuccess) {
    st->copy_stream = nullptr;
    pkv_stepper_destroy(st);
    return nullptr;
  }
  for (int k = 0; k < 2; ++k) {
    auto& sg = st->stage[k];
    sg.dev = static_cast<char*>(d_index) + k * bytes;
    if (hipHostMalloc(reinterpret_cast<void**>(&sg.host), bytes, hipHostMallocDefault) !=
            hipSuccess ||
        hipEventCreateWithFlags(&sg.copied, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&sg.consumed, hipEventDisableTiming) != hipSuccess) {
      pkv_stepper_destroy(st);
      return nullptr;
    }
  }
  return st;
}

void pkv_stepper_destroy(pkv_stepper_t* st) {
  if (!st) return;
  if (st->copy_stream) (void)hipStreamSynchronize(st->copy_stream);
  for (auto& sg : st->stage) {
    if (sg.consumed) {
      if (sg.used) (void)hipEventSynchronize(sg.consumed);
      (void)hipEventDestroy(sg.consumed);
    }
    if (sg.copied) (void)hipEventDestroy(sg.copied);
    if (sg.host) (void)hipHostFree(sg.host);
  }
  if (st->copy_stream) (void)hipStreamDestroy(st->copy_stream);
  delete st;
}

pkv_status_t pkv_stepper_step(pkv_stepper_t* st, const int64_t* seqs, int32_t n,
                              const pkv_layer_io_t* io, void* workspace, size_t workspace_bytes,
                              void* const* attn_events, int32_t* max_len, int32_t* num_cow,
                              int32_t* num_done, pkv_stream_t stream) {
  if (!st || !io || !max_len || !num_cow || !num_done || n < 0 || n > st->max_seqs ||
      (n > 0 && !seqs) || io->num_layers < 0)
    return PKV_EINVAL;
  *max_len = 0;
  *num_cow = 0;
  *num_done = 0;
  if (n == 0) return PKV_OK;
  const int32_t L = io->num_layers;
  if (L > 0 && (!io->k_pools || !io->v_pools || !io->q || !io->k_new || !io->v_new || !io->out))
    return PKV_EINVAL;

  st->cur ^= 1;
  auto& sg = st->stage[st->cur];
  if (sg.copy_pending) {
    // the upload issued from this host area two steps ago must have read it
    if (hipEventSynchronize(sg.copied) != hipSuccess) return PKV_EHIP;
    sg.copy_pending = false;
  }
  const int32_t MB = st->max_blocks;
  int32_t* tables = sg.host;
  int32_t* lens = tables + static_cast<size_t>(n) * MB;
  int32_t* slots = lens + n;
  int32_t* pairs = slots + n;

  pkv_status_t s = pkv_alloc_append_slots(st->alloc, seqs, n, slots, pairs, num_cow, num_done);
  if (s != PKV_OK) return s;
  s = pkv_alloc_export(st->alloc, seqs, n, MB, tables, lens);
  if (s != PKV_OK) return s;
  *max_len = *std::max_element(lens, lens + n);
  // Sequences whose first physical block is the same share a prefix: schedule them side by
  // side and read K/V with cache-allocating loads; otherwise longest first, nontemporal.
  st->keys.resize(static_cast<size_t>(n));
  for (int32_t i = 0; i < n; ++i) st->keys[i] = lens[i] > 0 ? tables[static_cast<size_t>(i) * MB] : -1 - i;
  st->sorted_keys.assign(st->keys.begin(), st->keys.end());
  std::sort(st->sorted_keys.begin(), st->sorted_keys.end());
  const bool shared =
      std::adjacent_find(st->sorted_keys.begin(), st->sorted_keys.end()) != st->sorted_keys.end();
  int32_t* items = pairs + 2 * static_cast<size_t>(*num_cow);
  const int32_t num_items =
      shared ? pkv_decode_schedule_grouped(&st->desc, lens, st->keys.data(), n, *max_len, items,
                                           st->max_items)
             : pkv_decode_schedule(&st->desc, lens, n, *max_len, items, st->max_items);
  if (num_items < 0) return PKV_EINVAL;
  const uint32_t decode_flags = shared ? PKV_DECODE_SHARED_KV : 0u;

  const size_t used = (static_cast<size_t>(n) * MB + 2 * static_cast<size_t>(n) +
                       2 * static_cast<size_t>(*num_cow) + num_items) * sizeof(int32_t);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  // upload after the last reader of this device area, then make the kernels wait for it
  if ((sg.used && hipStreamWaitEvent(st->copy_stream, sg.consumed, 0) != hipSuccess) ||
      hipMemcpyAsync(sg.dev, sg.host, used, hipMemcpyHostToDevice, st->copy_stream) !=
          hipSuccess ||
      hipEventRecord(sg.copied, st->copy_stream) != hipSuccess ||
      hipStreamWaitEvent(hs, sg.copied, 0) != hipSuccess)
    return PKV_EHIP;
  sg.copy_pending = true;

  const int32_t* d_tables = reinterpret_cast<const int32_t*>(sg.dev);
  const int32_t* d_lens = d_tables + static_cast<size_t>(n) * MB;
  const int32_t* d_slots = d_lens + n;
  const int32_t* d_pairs = d_slots + n;
  const int32_t* d_items = d_pairs + 2 * static_cast<size_t>(*num_cow);

  // launches; whatever happens, mark the end of this step's reads of the device area
  auto launch_all = [&]() -> pkv_status_t {
    if (*num_cow > 0 && L > 0) {
      pkv_status_t r =
          pkv_copy_blocks(&st->desc, io->k_pools, io->v_pools, L, d_pairs, *num_cow, stream);
      if (r != PKV_OK) return r;
    }
    for (int32_t l = 0; l < L; ++l) {
      pkv_status_t r = pkv_reshape_and_cache(&st->desc, io->k_new[l], io->v_new[l],
                                             io->k_pools[l], io->v_pools[l], d_slots, n, stream);
      if (r != PKV_OK) return r;
      if (attn_events &&
          hipEventRecord(static_cast<hipEvent_t>(attn_events[2 * l]), hs) != hipSuccess)
        return PKV_EHIP;
      r = pkv_paged_attention_decode_scheduled(
          &st->desc, io->out[l], io->q[l], io->k_pools[l], io->v_pools[l], d_tables, MB, d_lens,
          n, *max_len, io->scale, d_items, num_items, decode_flags, workspace, workspace_bytes,
          stream);
      if (r != PKV_OK) return r;
      if (attn_events &&
          hipEventRecord(static_cast<hipEvent_t>(attn_events[2 * l + 1]), hs) != hipSuccess)
        return PKV_EHIP;
    }
    return PKV_OK;
  };
  s = launch_all();
  if (hipEventRecord(sg.consumed, hs) != hipSuccess) return PKV_EHIP;
  sg.used = true;
  return s;
}

const void* pkv_stepper_last_index(const pkv_stepper_t* st) {
  return st ? st->stage[st->cur].dev : nullptr;
}

}  // extern "C"
