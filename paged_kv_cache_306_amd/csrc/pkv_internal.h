// Host-side helpers shared by the libpkv entry points.
#pragma once

#include <stdint.h>

#include <vector>

#include "pkv.h"

namespace pkv {

inline int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

inline int dtype_bytes(int32_t dtype) {
  switch (dtype) {
    case PKV_F32: return 4;
    case PKV_F16: return 2;
    case PKV_BF16: return 2;
  }
  return 0;
}

// Shape checks common to every device call: positive sizes, and a shape the library has
// kernels for (head_dim 64 or 128, block_size 8, 16 or 32, dtype f32 / f16 / bf16).
// Slot numbers (block * block_size + offset) must fit in int32.
inline pkv_status_t check_desc(const pkv_cache_desc_t* d) {
  if (!d) return PKV_EINVAL;
  if (d->num_blocks <= 0 || d->num_heads <= 0 || d->block_size <= 0 || d->head_dim <= 0)
    return PKV_EINVAL;
  if (static_cast<int64_t>(d->num_blocks) * d->block_size > INT32_MAX) return PKV_EINVAL;
  if (d->head_dim != 64 && d->head_dim != 128) return PKV_EUNSUPPORTED;
  if (d->block_size != 8 && d->block_size != 16 && d->block_size != 32) return PKV_EUNSUPPORTED;
  if (dtype_bytes(d->dtype) == 0) return PKV_EUNSUPPORTED;
  return PKV_OK;
}

// pkv_paged_attention_decode_scheduled with optional timing: ev_start / ev_stop (hipEvent_t,
// created with timing, or null) take the start and end time of the attention launch itself.
// xcd_split (0, or 1..1023 of 1024): the share of the units dealt to the even XCDs (0: unit b
// to workgroup b).  stamps (with xcd_split 0 only, else null): device-visible memory of
// 4 uint32 per unit that each workgroup that attends tokens fills with its duration in 100 MHz
// ticks, its XCD | 0x100, its tokens and the low 32 bits of its start tick.
pkv_status_t decode_scheduled_timed(const pkv_cache_desc_t* desc, void* out, const void* q,
                                    const void* k_pool, const void* v_pool,
                                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                                    const int32_t* context_lens, int32_t num_seqs,
                                    int32_t max_context_len, float scale,
                                    const int32_t* work_items, int32_t num_items, uint32_t flags,
                                    void* workspace, size_t workspace_bytes, pkv_stream_t stream,
                                    void* ev_start, void* ev_stop, int32_t xcd_split = 0,
                                    uint32_t* stamps = nullptr);

// pkv_paged_attention_multi_query_packed with optional timing (ev_start / ev_stop as above).
pkv_status_t multi_query_packed_timed(const pkv_cache_desc_t* desc, void* out, const void* q,
                                      const void* k_pool, const void* v_pool,
                                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                                      const int32_t* context_lens, const int32_t* query_start,
                                      int32_t num_seqs, int32_t num_tokens, int32_t max_query_len,
                                      int32_t max_context_len, float scale, const int32_t* tiles,
                                      int32_t num_tiles, pkv_stream_t stream, void* ev_start,
                                      void* ev_stop);

// The XCD split the stand-alone decode calls on the current device use from now on (a step
// driver's measurement); out-of-range values are ignored.
void set_device_xcd_split(int32_t split);

// Host checks of a cache append's slots (distinct within [0, num_slots); others are skipped)
// and of a block copy's pairs (among in-range pairs, destinations distinct and never a
// source).  `scratch` is reused between calls to avoid allocating.
bool slots_distinct(const int32_t* slots, int32_t n, int64_t num_slots,
                    std::vector<int32_t>& scratch);
bool copy_pairs_valid(const int32_t* pairs, int32_t n, int32_t num_blocks,
                      std::vector<int64_t>& scratch);

}  // namespace pkv
