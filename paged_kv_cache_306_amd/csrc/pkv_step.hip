// Decode-step driver: one decode iteration of a batch over every layer in one host call
// ("PagedAttention: Efficient LLM Serving with vLLM", "The PagedAttention Algorithm",
// steps 1-5).  The block manager decides slots and copy-on-write pairs on the host; the
// packed index data (tables | lens | slots | pairs | work items) is written into pinned
// host memory and pulled to the device by the step's first kernel, which also appends the
// first layer's new K/V -- no copy engine, no second stream, no cross-queue wait.
#include "pkv.h"
#include "pkv_device.h"
#include "pkv_internal.h"
#include "pkv_xcd.h"

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <new>
#include <vector>

namespace {

constexpr int kPrologueThreads = 256;
constexpr int kCopyVecsPerThread = 4;

// Workgroups [0, copy_wgs) copy idx_vecs 16-byte vectors of index data from pinned host
// memory (device-mapped) to the device index area.  The remaining workgroups, when
// row_vecs > 0, write token i's K/V rows of the first layer at slot slots_host[i] -- the
// same copy as reshape_and_cache_kernel, reading the slot straight from host memory.
__global__ __launch_bounds__(kPrologueThreads) void step_prologue_kernel(
    const pkv::u32x4* __restrict__ idx_src, pkv::u32x4* __restrict__ idx_dst, int idx_vecs,
    int copy_wgs, const int32_t* __restrict__ slots_host, const pkv::u32x4* __restrict__ k,
    const pkv::u32x4* __restrict__ v, pkv::u32x4* __restrict__ k_pool,
    pkv::u32x4* __restrict__ v_pool, int64_t total_vecs, int row_vecs, int num_heads,
    int block_size, int64_t num_slots) {
  if (static_cast<int>(blockIdx.x) < copy_wgs) {
    const int base = blockIdx.x * kPrologueThreads * kCopyVecsPerThread + threadIdx.x;
    pkv::u32x4 r[kCopyVecsPerThread];
#pragma unroll
    for (int u = 0; u < kCopyVecsPerThread; ++u) {
      const int i = base + u * kPrologueThreads;
      if (i < idx_vecs) r[u] = idx_src[i];
    }
#pragma unroll
    for (int u = 0; u < kCopyVecsPerThread; ++u) {
      const int i = base + u * kPrologueThreads;
      if (i < idx_vecs) idx_dst[i] = r[u];
    }
    return;
  }
  const int64_t gid =
      static_cast<int64_t>(blockIdx.x - copy_wgs) * kPrologueThreads + threadIdx.x;
  if (gid >= total_vecs) return;
  const int64_t row = gid / row_vecs;  // token * num_heads + head
  const int c = static_cast<int>(gid - row * row_vecs);
  const int64_t tok = row / num_heads;
  const int h = static_cast<int>(row - tok * num_heads);
  const int32_t slot = slots_host[tok];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t blk = slot / block_size;
  const int off = slot - static_cast<int32_t>(blk) * block_size;
  const int64_t dst = ((blk * num_heads + h) * block_size + off) * row_vecs + c;
  k_pool[dst] = k[gid];
  v_pool[dst] = v[gid];
}

// Most decode work items n sequences with tables of max_blocks entries can produce.
int32_t max_work_items(const pkv_cache_desc_t* d, int32_t n, int32_t max_blocks) {
  const int64_t cap = static_cast<int64_t>(max_blocks) * d->block_size;
  const int32_t max_ctx = static_cast<int32_t>(std::min<int64_t>(cap, INT32_MAX));
  const int32_t part = pkv_decode_partition_tokens(d, n, max_ctx);
  const int64_t parts = part > 0 ? (max_ctx + part - 1) / part : 1;
  return static_cast<int32_t>(std::min<int64_t>(static_cast<int64_t>(n) * parts, INT32_MAX / 8));
}

size_t index_ints(int32_t n, int32_t max_blocks, int32_t max_items) {
  // tables [n][max_blocks], lens [n], slots [n], pairs [n][2], then either the decode work
  // items [max_items] or, for the multi-query path, query_start [n + 1], padding to 16 bytes
  // and packed tiles [n][4]
  return static_cast<size_t>(n) * max_blocks + 4 * static_cast<size_t>(n) +
         std::max<size_t>(max_items, 5 * static_cast<size_t>(n) + 4);
}

// Decode of sequences that share their first blocks goes through the multi-query kernel over
// packed tiles when its launch has at least this many workgroups, when at least two
// sequences share each tile on average, and when no context is longer than this (longer ones
// need the decode's split into partitions to spread over the chip).
constexpr int64_t kMqMinWorkgroups = 448;  // measured: 480 faster than the decode, 320 slower
constexpr int32_t kMqMaxContext = 4096;

size_t stage_bytes(int32_t max_seqs, int32_t max_blocks_per_seq, int32_t max_items) {
  return static_cast<size_t>(pkv::align_up(
      static_cast<int64_t>(index_ints(max_seqs, max_blocks_per_seq, max_items) * 4), 256));
}

}  // namespace

// kStages stages are used in turn.  Stage k owns a pinned host area and a device area of
// d_index.  The prologue of launch i reads the host area of its stage; the host refills that
// area at launch i + kStages only after a completion marker at or after launch i has fired.
// Every kMarkEvery-th prologue launch carries such a marker (its own completion event): a
// launch that carries one leaves the GPU idle for a few microseconds before the next kernel,
// so markers are spread over several steps, and with kMarkEvery < kStages the kStages
// launches before any launch always include a marked one.  The device area is rewritten at
// launch i + kStages by a kernel on the same stream, so launch i's readers are done.
constexpr int kStages = 8;
constexpr int kMarkEvery = 7;
static_assert(kMarkEvery < kStages, "a marked launch among any kStages consecutive ones");

struct pkv_stepper {
  pkv_alloc_t* alloc = nullptr;
  pkv_cache_desc_t desc{};
  int32_t max_seqs = 0;
  int32_t max_blocks = 0;
  int32_t max_items = 0;                   // decode work items per step, at most
  std::vector<int32_t> keys, sorted_keys;  // per-step scratch for the sharing test
  std::vector<int32_t> slot_scratch;       // per-step scratch for the index-data checks
  std::vector<int64_t> pair_scratch;
  // The stream of the last step that launched work, and an event that hands the shared areas
  // (staging, device index area, workspace) over when a step comes on another stream.
  hipStream_t last_stream = nullptr;
  bool launched = false;
  hipEvent_t handoff = nullptr;
  struct Stage {
    int32_t* host = nullptr;        // pinned: tables | lens | slots | pairs | items
    const char* host_dev = nullptr; // the same memory as the device sees it
    char* dev = nullptr;            // device area of the same size inside d_index
  } stage[kStages];
  // Completion markers of marked prologue launches (launch -1: free), the number of prologue
  // launches so far, and the last launch known on the host to have finished.
  struct Mark {
    hipEvent_t ev = nullptr;
    int64_t launch = -1;
  } mark[kStages];
  int64_t launches = 0;
  int64_t done_upto = -1;
  bool mq_ok = false;       // the multi-query kernel supports this cache's shape and type
  int32_t last_kernel = -1; // PKV_STEP_ATTN_* of the last step's attention launches
  // XCD balance: the split the attention launches deal their units with (0: none), and its
  // measurement from the stamps one attention launch leaves in pinned host memory.
  enum Cal { kCalPending, kCalInFlight, kCalDone };
  Cal cal = kCalPending;
  int cal_attempts = 0;
  int32_t xcd_split = 0;
  int32_t cal_outcome = 0;          // PKV_XCD_* of the last measurement
  double cal_rate[2] = {0.0, 0.0};  // tokens per tick of workgroup time, even and odd half
  uint32_t* cal_host = nullptr;     // pinned, 4 words per unit
  uint32_t* cal_dev = nullptr;      // the same memory as the device sees it
  int64_t cal_capacity = 0;         // units
  int64_t cal_units = 0;            // units of the stamped launch
  hipEvent_t cal_done = nullptr;    // end of the stamped launch
};

namespace {

// Measurement of the XCD halves: a launch that fills the chip (twice the 768 workgroups the
// fp16 decode keeps resident; below that the halves do not compete for bandwidth and look
// alike), enough measured workgroups per half, a bound on the split, and the difference below
// which the units stay evenly dealt.
constexpr int64_t kCalMinUnits = 1536;
constexpr int64_t kCalMinPerHalf = 256;
constexpr int kCalMaxAttempts = 4;
constexpr int32_t kSplitMin = 384, kSplitMax = 640, kSplitDeadband = 5;  // of 1024

// The split from the stamps of a launch that dealt unit b to workgroup b: each half's tokens
// per tick of workgroup time (both halves ran every item's units alike), left in rate[], over
// the workgroups that ended before the first XCD ran out of work -- after that the XCDs still
// busy share the chip's bandwidth among fewer workgroups and would look faster than they are.
// Returns -1 when the stamps are too few to tell, and 0 when the hardware did not place
// workgroup b on XCD b % 8 (*outcome PKV_XCD_UNMAPPED) or the halves are within the deadband.
int32_t split_from_stamps(const uint32_t* w, int64_t units, double rate[2], int32_t* outcome) {
  // start and end ticks relative to the first stamped workgroup's start (32-bit wrap-safe)
  bool have_ref = false;
  uint32_t ref = 0;
  int64_t last_end[pkv::kXcds];
  for (int x = 0; x < pkv::kXcds; ++x) last_end[x] = -1;
  for (int64_t b = 0; b < units; ++b) {
    const uint32_t* s = w + 4 * b;
    if (!(s[1] & 0x100u)) continue;  // a workgroup with nothing to attend
    const uint32_t xcc = s[1] & 15u;
    if (xcc != static_cast<uint32_t>(b % pkv::kXcds)) {
      *outcome = PKV_XCD_UNMAPPED;
      return 0;
    }
    if (!have_ref) {
      ref = s[3];
      have_ref = true;
    }
    const int64_t end = static_cast<int64_t>(static_cast<int32_t>(s[3] - ref)) + s[0];
    last_end[xcc] = std::max(last_end[xcc], end);
  }
  int64_t cutoff = -1;  // the first XCD's last end
  for (int x = 0; x < pkv::kXcds; ++x)
    if (last_end[x] >= 0) cutoff = cutoff < 0 ? last_end[x] : std::min(cutoff, last_end[x]);
  double tokens[2] = {0.0, 0.0}, ticks[2] = {0.0, 0.0};
  int64_t count[2] = {0, 0};
  for (int64_t b = 0; b < units; ++b) {
    const uint32_t* s = w + 4 * b;
    if (!(s[1] & 0x100u) || s[0] == 0 || s[2] == 0) continue;
    const int64_t end = static_cast<int64_t>(static_cast<int32_t>(s[3] - ref)) + s[0];
    if (end > cutoff) continue;
    const int half = static_cast<int>(s[1] & 1u);
    tokens[half] += s[2];
    ticks[half] += s[0];
    ++count[half];
  }
  if (count[0] < kCalMinPerHalf || count[1] < kCalMinPerHalf) {
    *outcome = PKV_XCD_TOO_FEW;
    return -1;
  }
  rate[0] = tokens[0] / ticks[0];
  rate[1] = tokens[1] / ticks[1];
  int32_t p = static_cast<int32_t>(std::lround(pkv::kXcdSplitOne * rate[0] / (rate[0] + rate[1])));
  p = std::min(std::max(p, kSplitMin), kSplitMax);
  *outcome = PKV_XCD_MEASURED;
  return std::abs(p - static_cast<int32_t>(pkv::kXcdSplitOne / 2)) < kSplitDeadband ? 0 : p;
}

// Reads the stamps once their launch is done; never waits for it.
void poll_calibration(pkv_stepper* st) {
  const hipError_t e = hipEventQuery(st->cal_done);
  if (e == hipErrorNotReady) return;
  if (e != hipSuccess) {
    (void)hipGetLastError();
    st->cal = pkv_stepper::kCalDone;
    st->cal_outcome = PKV_XCD_FAILED;
    return;
  }
  const int32_t p = split_from_stamps(st->cal_host, st->cal_units, st->cal_rate, &st->cal_outcome);
  if (p >= 0) {
    st->xcd_split = p;
    st->cal = pkv_stepper::kCalDone;
    // the device's stand-alone decode calls deal their units the same way from now on
    if (st->cal_outcome == PKV_XCD_MEASURED) pkv::set_device_xcd_split(p);
  } else {
    st->cal = ++st->cal_attempts < kCalMaxAttempts ? pkv_stepper::kCalPending
                                                    : pkv_stepper::kCalDone;
  }
}

}  // namespace

extern "C" {

size_t pkv_stepper_index_bytes(const pkv_cache_desc_t* desc, int32_t max_seqs,
                               int32_t max_blocks_per_seq) {
  if (pkv::check_desc(desc) != PKV_OK || max_seqs <= 0 || max_blocks_per_seq <= 0) return 0;
  return kStages * stage_bytes(max_seqs, max_blocks_per_seq,
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
  st->mq_ok = (desc->dtype == PKV_F16 || desc->dtype == PKV_BF16) && max_seqs <= (1 << 20) &&
              static_cast<int64_t>(max_seqs) * max_blocks_per_seq <= UINT32_MAX;
  const size_t bytes = stage_bytes(max_seqs, max_blocks_per_seq, st->max_items);
  for (int k = 0; k < kStages; ++k) {
    auto& sg = st->stage[k];
    sg.dev = static_cast<char*>(d_index) + k * bytes;
    // The staging area is fine-grained (coherent) host memory, so the prologue's reads of it
    // always fetch what the host last wrote and never leave a copy in the GPU's caches.  The
    // host only needs to know that the prologue has finished reading it before refilling it,
    // which the launch's completion signal tells without a system-scope release: the marker
    // is created without that fence (a cache writeback and invalidate between kernels).
    void* dptr = nullptr;
    if (hipHostMalloc(reinterpret_cast<void**>(&sg.host), bytes,
                      hipHostMallocMapped | hipHostMallocCoherent) != hipSuccess ||
        hipHostGetDevicePointer(&dptr, sg.host, 0) != hipSuccess ||
        hipEventCreateWithFlags(&st->mark[k].ev,
                                hipEventDisableTiming | hipEventDisableSystemFence) !=
            hipSuccess) {
      (void)hipGetLastError();
      pkv_stepper_destroy(st);
      return nullptr;
    }
    sg.host_dev = static_cast<const char*>(dptr);
  }
  if (hipEventCreateWithFlags(&st->handoff, hipEventDisableTiming) != hipSuccess) {
    (void)hipGetLastError();
    pkv_stepper_destroy(st);
    return nullptr;
  }
  // Calibration stamps: written by the device straight into coherent host memory, read by
  // the host after the launch's completion event.
  st->cal_capacity = static_cast<int64_t>(st->max_items) * desc->num_heads;
  void* cal_dptr = nullptr;
  if (hipHostMalloc(reinterpret_cast<void**>(&st->cal_host),
                    static_cast<size_t>(st->cal_capacity) * 16,
                    hipHostMallocMapped | hipHostMallocCoherent) != hipSuccess ||
      hipHostGetDevicePointer(&cal_dptr, st->cal_host, 0) != hipSuccess ||
      hipEventCreateWithFlags(&st->cal_done, hipEventDisableTiming) != hipSuccess) {
    (void)hipGetLastError();
    pkv_stepper_destroy(st);
    return nullptr;
  }
  st->cal_dev = static_cast<uint32_t*>(cal_dptr);
  return st;
}

void pkv_stepper_destroy(pkv_stepper_t* st) {
  if (!st) return;
  // prologues still reading the staging areas (the last ones carry no marker)
  for (auto& mk : st->mark)
    if (mk.ev && mk.launch >= 0) (void)hipEventSynchronize(mk.ev);
  if (st->launched && st->handoff &&
      hipEventRecord(st->handoff, st->last_stream) == hipSuccess)
    (void)hipEventSynchronize(st->handoff);
  (void)hipGetLastError();
  for (auto& mk : st->mark)
    if (mk.ev) (void)hipEventDestroy(mk.ev);
  for (auto& sg : st->stage)
    if (sg.host) (void)hipHostFree(sg.host);
  if (st->handoff) (void)hipEventDestroy(st->handoff);
  if (st->cal_done) {
    // a stamped launch still running writes into cal_host
    if (st->cal == pkv_stepper::kCalInFlight) (void)hipEventSynchronize(st->cal_done);
    (void)hipEventDestroy(st->cal_done);
  }
  if (st->cal_host) (void)hipHostFree(st->cal_host);
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
  st->last_kernel = -1;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (n == 0) {
    // nothing to attend: timing events, if any, are recorded back to back (zero duration)
    if (attn_events)
      for (int64_t e = 0; e < 2 * static_cast<int64_t>(io->num_layers); ++e)
        if (attn_events[e] && hipEventRecord(static_cast<hipEvent_t>(attn_events[e]), hs) !=
                                  hipSuccess)
          return PKV_EHIP;
    return PKV_OK;
  }
  // Every check that can fail comes before anything changes: arguments, sequences, table
  // width, pool capacity, workspace.
  int32_t expect_len = 0;
  pkv_status_t s = pkv_stepper_check(st->alloc, &st->desc, st->max_seqs, st->max_blocks, seqs,
                                     n, io, workspace, workspace_bytes, &expect_len);
  if (s != PKV_OK) return s;
  const int32_t L = io->num_layers;

  if (st->cal == pkv_stepper::kCalInFlight) poll_calibration(st);
  const int64_t launch = st->launches;  // this step's prologue launch
  auto& sg = st->stage[launch % kStages];
  const int64_t prev = launch - kStages;  // the launch that last read this host area
  if (prev > st->done_upto) {
    // wait for the oldest marker at or after it (one of the kStages launches before this one
    // carries a marker), which frees every area read up to that launch
    int pick = -1;
    for (int k = 0; k < kStages; ++k)
      if (st->mark[k].launch >= prev &&
          (pick < 0 || st->mark[k].launch < st->mark[pick].launch))
        pick = k;
    if (pick < 0 || hipEventSynchronize(st->mark[pick].ev) != hipSuccess) return PKV_EHIP;
    st->done_upto = st->mark[pick].launch;
    for (auto& mk : st->mark)
      if (mk.launch <= st->done_upto) mk.launch = -1;
  }
  // this launch's marker, if it carries one: a free marker (at most two are outstanding)
  int mark_slot = -1;
  if (launch % kMarkEvery == 0) {
    for (int k = 0; k < kStages && mark_slot < 0; ++k)
      if (st->mark[k].launch < 0) mark_slot = k;
    if (mark_slot < 0) return PKV_EHIP;
  }
  // A step on another stream than the last one first waits for all the last stream queued:
  // the two share the staging areas, the device index area and the workspace.
  (void)hipGetLastError();
  if (st->launched && hs != st->last_stream &&
      (hipEventRecord(st->handoff, st->last_stream) != hipSuccess ||
       hipStreamWaitEvent(hs, st->handoff, 0) != hipSuccess))
    return PKV_EHIP;

  const int32_t MB = st->max_blocks;
  int32_t* tables = sg.host;
  int32_t* lens = tables + static_cast<size_t>(n) * MB;
  int32_t* slots = lens + n;
  int32_t* pairs = slots + n;

  // cannot fail after the checks above (sequences known, room in the pool and the table)
  s = pkv_alloc_append_slots(st->alloc, seqs, n, slots, pairs, num_cow, num_done);
  if (s != PKV_OK) return s;
  s = pkv_alloc_export(st->alloc, seqs, n, MB, tables, lens);
  if (s != PKV_OK) return s;
  *max_len = *std::max_element(lens, lens + n);
  // the block manager's own guarantees, checked on what is about to be uploaded
  if (*max_len != expect_len ||
      !pkv::slots_distinct(slots, n, static_cast<int64_t>(st->desc.num_blocks) * st->desc.block_size,
                           st->slot_scratch) ||
      !pkv::copy_pairs_valid(pairs, *num_cow, st->desc.num_blocks, st->pair_scratch))
    return PKV_EINVAL;
  // Sequences whose first physical block is the same share a prefix: schedule them side by
  // side and read K/V with cache-allocating loads; otherwise longest first, nontemporal.
  st->keys.resize(static_cast<size_t>(n));
  for (int32_t i = 0; i < n; ++i)
    st->keys[i] = lens[i] > 0 ? tables[static_cast<size_t>(i) * MB] : -1 - i;
  st->sorted_keys.assign(st->keys.begin(), st->keys.end());
  std::sort(st->sorted_keys.begin(), st->sorted_keys.end());
  const bool shared =
      std::adjacent_find(st->sorted_keys.begin(), st->sorted_keys.end()) != st->sorted_keys.end();
  int32_t* items = pairs + 2 * static_cast<size_t>(*num_cow);
  // Groups that share their first blocks (parallel sampling, beam search, a cached prompt):
  // the multi-query kernel over packed tiles, one new token per sequence, stages each group's
  // shared blocks once for all its members, where the decode reads them once per member
  // (from L2).  It needs enough tiles to fill the chip and contexts short enough to need no
  // split.  The staging area then holds query_start (0 .. n) and the tiles after the pairs.
  const size_t qs_off = static_cast<size_t>(items - tables);
  const size_t tiles_off = (qs_off + n + 1 + 3) / 4 * 4;  // 16-byte aligned on the device
  int32_t num_tiles = 0;
  bool mq = false;
  bool mq_aligned = true;  // the multi-query kernel reads q and writes out 16 bytes at a time
  for (int32_t l = 0; l < L; ++l)
    mq_aligned = mq_aligned && reinterpret_cast<uintptr_t>(io->q[l]) % 16 == 0 &&
                 reinterpret_cast<uintptr_t>(io->out[l]) % 16 == 0;
  // (the multi-query kernel also takes only a positive scale; the decode takes any finite one)
  if (shared && st->mq_ok && mq_aligned && io->scale > 0.0f && *max_len <= kMqMaxContext) {
    for (int32_t i = 0; i <= n; ++i) tables[qs_off + i] = i;
    num_tiles = pkv_multi_query_schedule_packed(tables + qs_off, lens, tables, MB,
                                                st->desc.block_size, n, *max_len,
                                                tables + tiles_off, n);
    mq = num_tiles > 0 && 2 * static_cast<int64_t>(num_tiles) <= n &&
         static_cast<int64_t>(num_tiles) * st->desc.num_heads >= kMqMinWorkgroups;
  }
  int32_t num_items = 0;
  if (!mq) {
    num_items = shared ? pkv_decode_schedule_grouped(&st->desc, lens, st->keys.data(), n,
                                                     *max_len, items, st->max_items)
                       : pkv_decode_schedule(&st->desc, lens, n, *max_len, items, st->max_items);
    if (num_items < 0) return PKV_EINVAL;
  }
  const uint32_t decode_flags = shared ? PKV_DECODE_SHARED_KV : 0u;

  const size_t used_ints = mq ? tiles_off + 4 * static_cast<size_t>(num_tiles)
                              : qs_off + static_cast<size_t>(num_items);
  const int idx_vecs = static_cast<int>((used_ints * 4 + 15) / 16);
  const int copy_wgs = (idx_vecs + kPrologueThreads * kCopyVecsPerThread - 1) /
                       (kPrologueThreads * kCopyVecsPerThread);
  // The first layer's append rides in the prologue unless copy-on-write copies must land
  // first (a copy would overwrite the new token in its destination block).
  const bool fuse_append = L > 0 && *num_cow == 0;
  const int row_vecs = st->desc.head_dim * pkv::dtype_bytes(st->desc.dtype) / 16;
  const int64_t total_vecs =
      fuse_append ? static_cast<int64_t>(n) * st->desc.num_heads * row_vecs : 0;
  const int64_t append_wgs = (total_vecs + kPrologueThreads - 1) / kPrologueThreads;
  if (copy_wgs + append_wgs > INT32_MAX) return PKV_EUNSUPPORTED;

  const int32_t* slots_host_dev =
      reinterpret_cast<const int32_t*>(sg.host_dev) + static_cast<size_t>(n) * MB + n;
  // A marker that frees this staging area is a prologue launch's own completion (the launch
  // records it when the kernel ends): the prologue is the only reader of the area, and an
  // event recorded on the stream between two kernels would leave the GPU idle for a few
  // microseconds.  The host waits on one only kStages - kMarkEvery launches later, at least.
  hipExtLaunchKernelGGL(
      step_prologue_kernel, dim3(static_cast<unsigned>(copy_wgs + append_wgs)),
      dim3(kPrologueThreads), 0, hs, nullptr,
      mark_slot >= 0 ? st->mark[mark_slot].ev : nullptr, 0u,
      reinterpret_cast<const pkv::u32x4*>(sg.host_dev),
      reinterpret_cast<pkv::u32x4*>(sg.dev), idx_vecs, copy_wgs, slots_host_dev,
      fuse_append ? static_cast<const pkv::u32x4*>(io->k_new[0]) : nullptr,
      fuse_append ? static_cast<const pkv::u32x4*>(io->v_new[0]) : nullptr,
      fuse_append ? static_cast<pkv::u32x4*>(io->k_pools[0]) : nullptr,
      fuse_append ? static_cast<pkv::u32x4*>(io->v_pools[0]) : nullptr, total_vecs, row_vecs,
      st->desc.num_heads, st->desc.block_size,
      static_cast<int64_t>(st->desc.num_blocks) * st->desc.block_size);
  if (hipGetLastError() != hipSuccess) return PKV_EHIP;
  if (mark_slot >= 0) st->mark[mark_slot].launch = launch;
  st->launches = launch + 1;
  st->launched = true;
  st->last_stream = hs;

  const int32_t* d_tables = reinterpret_cast<const int32_t*>(sg.dev);
  const int32_t* d_lens = d_tables + static_cast<size_t>(n) * MB;
  const int32_t* d_slots = d_lens + n;
  const int32_t* d_pairs = d_slots + n;
  const int32_t* d_items = d_pairs + 2 * static_cast<size_t>(*num_cow);
  const int32_t* d_qs = d_tables + qs_off;
  const int32_t* d_tiles = d_tables + tiles_off;

  if (*num_cow > 0 && L > 0) {
    s = pkv_copy_blocks(&st->desc, io->k_pools, io->v_pools, L, d_pairs, *num_cow, stream);
    if (s != PKV_OK) return s;
  }
  // The first step with enough units measures the XCD halves on its layer-0 attention.
  const int64_t units = static_cast<int64_t>(num_items) * st->desc.num_heads;
  const bool stamp = !mq && st->cal == pkv_stepper::kCalPending && L > 0 &&
                     units >= kCalMinUnits && units <= st->cal_capacity;
  if (stamp) std::memset(st->cal_host, 0, static_cast<size_t>(units) * 16);
  for (int32_t l = 0; l < L; ++l) {
    if (!(l == 0 && fuse_append)) {
      s = pkv_reshape_and_cache(&st->desc, io->k_new[l], io->v_new[l], io->k_pools[l],
                                io->v_pools[l], d_slots, n, stream);
      if (s != PKV_OK) return s;
    }
    // timing, when asked for, comes from the attention launch itself
    const bool stamp_here = stamp && l == 0;
    if (mq) {
      s = pkv::multi_query_packed_timed(&st->desc, io->out[l], io->q[l], io->k_pools[l],
                                        io->v_pools[l], d_tables, MB, d_lens, d_qs, n, n, 1,
                                        *max_len, io->scale, d_tiles, num_tiles, stream,
                                        attn_events ? attn_events[2 * l] : nullptr,
                                        attn_events ? attn_events[2 * l + 1] : nullptr);
      if (s != PKV_OK) return s;
      continue;
    }
    s = pkv::decode_scheduled_timed(&st->desc, io->out[l], io->q[l], io->k_pools[l],
                                    io->v_pools[l], d_tables, MB, d_lens, n, *max_len, io->scale,
                                    d_items, num_items, decode_flags, workspace, workspace_bytes,
                                    stream, attn_events ? attn_events[2 * l] : nullptr,
                                    attn_events ? attn_events[2 * l + 1] : nullptr,
                                    stamp_here ? 0 : st->xcd_split,
                                    stamp_here ? st->cal_dev : nullptr);
    if (s != PKV_OK) return s;
    if (stamp_here) {
      if (hipEventRecord(st->cal_done, hs) != hipSuccess) return PKV_EHIP;
      st->cal = pkv_stepper::kCalInFlight;
      st->cal_units = units;
    }
  }
  st->last_kernel = mq ? PKV_STEP_ATTN_MULTI_QUERY : PKV_STEP_ATTN_DECODE;
  return PKV_OK;
}

int32_t pkv_stepper_last_attention(const pkv_stepper_t* st) { return st ? st->last_kernel : -1; }

const void* pkv_stepper_last_index(const pkv_stepper_t* st) {
  return st ? st->stage[st->launches > 0 ? (st->launches - 1) % kStages : 0].dev : nullptr;
}

int32_t pkv_stepper_xcd_split(const pkv_stepper_t* st) { return st ? st->xcd_split : -1; }

int32_t pkv_xcd_split_from_stamps(const uint32_t* stamps, int64_t units, double* even,
                                  double* odd, int32_t* outcome) {
  if (!stamps || units <= 0 || !even || !odd || !outcome) return -2;
  double rate[2] = {0.0, 0.0};
  *outcome = PKV_XCD_NONE;
  const int32_t p = split_from_stamps(stamps, units, rate, outcome);
  *even = rate[0];
  *odd = rate[1];
  return p;
}

pkv_status_t pkv_stepper_xcd_rates(const pkv_stepper_t* st, double* even, double* odd,
                                   int32_t* outcome) {
  if (!st || !even || !odd || !outcome) return PKV_EINVAL;
  *even = st->cal_rate[0];
  *odd = st->cal_rate[1];
  *outcome = st->cal == pkv_stepper::kCalInFlight ? PKV_XCD_IN_FLIGHT : st->cal_outcome;
  return PKV_OK;
}

pkv_status_t pkv_stepper_set_xcd_split(pkv_stepper_t* st, int32_t split) {
  if (!st || split < -1 || split >= pkv::kXcdSplitOne) return PKV_EINVAL;
  if (st->cal == pkv_stepper::kCalInFlight) {
    // the stamped launch may still write into cal_host, which a new measurement reuses
    if (hipEventSynchronize(st->cal_done) != hipSuccess) {
      (void)hipGetLastError();
      return PKV_EHIP;
    }
  }
  if (split < 0) {
    st->cal = pkv_stepper::kCalPending;
    st->cal_attempts = 0;
  } else {
    st->xcd_split = split;
    st->cal = pkv_stepper::kCalDone;
  }
  return PKV_OK;
}

}  // extern "C"
