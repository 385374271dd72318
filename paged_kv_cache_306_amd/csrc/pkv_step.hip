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

struct pkv_stepper {
  pkv_alloc_t* alloc = nullptr;
  pkv_cache_desc_t desc{};
  int32_t max_seqs = 0;
  int32_t max_blocks = 0;
  char* d_index = nullptr;
  struct Stage {
    int32_t* host = nullptr;  // pinned: tables | lens | slots | pairs (packed for n)
    hipEvent_t copied = nullptr;
    bool pending = false;
  } stage[2];
  int cur = 0;
};

namespace {

size_t index_ints(int32_t n, int32_t max_blocks) {
  // tables [n][max_blocks], lens [n], slots [n], pairs [n][2]
  return static_cast<size_t>(n) * max_blocks + 4 * static_cast<size_t>(n);
}

}  // namespace

extern "C" {

size_t pkv_stepper_index_bytes(int32_t max_seqs, int32_t max_blocks_per_seq) {
  if (max_seqs <= 0 || max_blocks_per_seq <= 0) return 0;
  return index_ints(max_seqs, max_blocks_per_seq) * sizeof(int32_t);
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
  st->d_index = static_cast<char*>(d_index);
  const size_t bytes = pkv_stepper_index_bytes(max_seqs, max_blocks_per_seq);
  for (auto& sg : st->stage) {
    if (hipHostMalloc(reinterpret_cast<void**>(&sg.host), bytes, hipHostMallocDefault) !=
            hipSuccess ||
        hipEventCreateWithFlags(&sg.copied, hipEventDisableTiming) != hipSuccess) {
      pkv_stepper_destroy(st);
      return nullptr;
    }
  }
  return st;
}

void pkv_stepper_destroy(pkv_stepper_t* st) {
  if (!st) return;
  for (auto& sg : st->stage) {
    if (sg.copied) {
      if (sg.pending) (void)hipEventSynchronize(sg.copied);
      (void)hipEventDestroy(sg.copied);
    }
    if (sg.host) (void)hipHostFree(sg.host);
  }
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
  if (sg.pending) {
    // the copy issued from this staging area two steps ago must have read it
    if (hipEventSynchronize(sg.copied) != hipSuccess) return PKV_EHIP;
    sg.pending = false;
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

  const size_t used = (index_ints(n, MB) - 2 * static_cast<size_t>(n - *num_cow)) * sizeof(int32_t);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (hipMemcpyAsync(st->d_index, sg.host, used, hipMemcpyHostToDevice, hs) != hipSuccess ||
      hipEventRecord(sg.copied, hs) != hipSuccess)
    return PKV_EHIP;
  sg.pending = true;

  const int32_t* d_tables = reinterpret_cast<const int32_t*>(st->d_index);
  const int32_t* d_lens = d_tables + static_cast<size_t>(n) * MB;
  const int32_t* d_slots = d_lens + n;
  const int32_t* d_pairs = d_slots + n;

  if (*num_cow > 0 && L > 0) {
    s = pkv_copy_blocks(&st->desc, io->k_pools, io->v_pools, L, d_pairs, *num_cow, stream);
    if (s != PKV_OK) return s;
  }
  for (int32_t l = 0; l < L; ++l) {
    s = pkv_reshape_and_cache(&st->desc, io->k_new[l], io->v_new[l], io->k_pools[l],
                              io->v_pools[l], d_slots, n, stream);
    if (s != PKV_OK) return s;
    if (attn_events && hipEventRecord(static_cast<hipEvent_t>(attn_events[2 * l]), hs) != hipSuccess)
      return PKV_EHIP;
    s = pkv_paged_attention_decode(&st->desc, io->out[l], io->q[l], io->k_pools[l],
                                   io->v_pools[l], d_tables, MB, d_lens, n, *max_len, io->scale,
                                   workspace, workspace_bytes, stream);
    if (s != PKV_OK) return s;
    if (attn_events &&
        hipEventRecord(static_cast<hipEvent_t>(attn_events[2 * l + 1]), hs) != hipSuccess)
      return PKV_EHIP;
  }
  return PKV_OK;
}

}  // extern "C"
