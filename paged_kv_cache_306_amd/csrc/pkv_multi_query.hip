// Multi-query paged attention for gfx950 (CDNA4, wave64): several new tokens of each
// sequence attend at once, each to the sequence's tokens up to its own position, with every
// key read through the block table.  These are the remaining prompt tokens after a
// prefix-cache hit ("PagedAttention: Efficient LLM Serving with vLLM", "Advanced Features" ->
// "Prefix Caching"), a chunk of a long prompt, or the draft tokens a target model checks
// (same page, "Speculative Decoding Integration"); gathering K/V through the page table is
// step 5 of "The PagedAttention Algorithm" on that page.
//
// With many queries per sequence this is a dense contraction, so both products run on the
// matrix cores (v_mfma_f32_16x16x32_{f16,bf16}, fp32 accumulate):
//   * one workgroup = 128 consecutive new tokens of one (sequence, head), 16 per wave (one
//     MFMA query tile; the shape is a compile-time choice, see below); or, in packed mode,
//     128 consecutive rows of q spanning several sequences that hold the same first blocks
//     (requests sharing a cached prompt, "Prefix Caching" and "KV-Cache Sharing" on the same
//     page): their shared keys are staged once for all the rows, then each sequence's own
//     keys for its rows, so the tiles of short new-token runs are full;
//   * keys go 64 at a time through a double-buffered LDS stage, K and V rows loaded straight
//     from HBM into LDS (global_load_lds_dwordx4), stage c + 1 landing while stage c is
//     computed as two 32-key steps, one barrier per stage; the stage rows are XOR-swizzled
//     so that every read pattern below hits distinct banks;
//   * scores S^T = K Q^T: K rows are the A operand (16-byte LDS reads), the wave's q rows
//     (in registers for the whole run) the B operand; lane (r, g) = (lane % 16, lane / 16)
//     receives the scores of query r against keys 4g .. 4g+3 of each 16-key half;
//   * softmax runs per query in log2 units against a reference shared by the four lanes of a
//     query and moved only when a score exceeds it by a margin (the cross-lane max is taken
//     only then); each lane's probabilities are directly the
//     B operand of O^T = V^T P^T when slot 8g + j of the contraction is key 4g + j (j < 4)
//     or key 16 + 4g + j - 4 (j >= 4);
//   * the V^T operand comes from the row-major V stage through gfx950's transposing LDS read
//     (ds_read_b64_tr_b16): within each 16-lane group, component m of lane i is element
//     i % 4 of the 4 x 16-bit piece addressed by lane 4m + i / 4, so lane (r, g) addresses
//     key row 4g + r / 4 (then 16 + 4g + r / 4) at head-dim column 16 t + 4 (r % 4);
//   * O^T accumulates in 16 x 16 tiles: lane (r, g) holds output elements d = 16 t + 4 g + i
//     of query r.  The softmax denominator sums the same rounded probabilities: with v_dot2
//     per lane at fp16, through one more tile whose V^T rows are all ones at bf16.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <type_traits>
#include <vector>

#include "pkv.h"
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

// Workgroup shape: 8 waves x one 16-query tile each (128 new tokens per workgroup) with a
// 64-key stage (64 KiB of LDS) runs at 118 VGPRs: two workgroups and four waves per SIMD
// share each CU.  Against 4 waves with a 32-key stage (64 tokens, 32 KiB) it halves the K/V
// reads per query and the barriers per key; on the prefix-hit workload, side by side, 4%
// faster at fp16 and 1.5% at bf16 (each change alone was not faster).  Two tiles per wave
// (each K/V fragment feeding two products) halves the LDS bytes per flop but needs 184 VGPRs
// and two waves per SIMD; it tied or lost.  All shapes give bit-identical outputs.
constexpr int kMqWaves = 8;                                 // waves per workgroup
constexpr int kMqQt = 1;                                    // 16-query MFMA tiles per wave
constexpr int kMqThreads = 64 * kMqWaves;
constexpr int kMqWaveQueries = 16 * kMqQt;
constexpr int kMqTileQueries = kMqWaves * kMqWaveQueries;   // new tokens per workgroup
constexpr int kMqChunk = 32;                                // keys per compute step
constexpr int kMqSub = 2;                                   // compute steps per LDS stage
constexpr int kMqStage = kMqChunk * kMqSub;                 // keys staged per barrier
constexpr float kMqSlack = 8.0f;  // log2 units a score may exceed the softmax reference by
constexpr int kMqXcds = 8;        // XCDs of the chip, each with its own L2
constexpr int kMqXcdChunk = 64;   // items an XCD runs per head (its resident workgroups)
constexpr int kMqItemSeqBits = 20;                          // work item = sequence | tile << 20
constexpr int kMqItemSeqMask = (1 << kMqItemSeqBits) - 1;
constexpr int kMqMaxTiles = 1 << (31 - kMqItemSeqBits);

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// One 16x16x32 product on fragments held as four 32-bit words each, and how a probability
// enters the second product.  fp16 carries 11 significant bits: one rounded copy (relative
// error <= 2^-11).  bfloat16 carries only 8, which could move an output by ~2^-9 |v| when a
// query sees few keys, so p goes in as two parts, hi = bf16(p) and lo = bf16(p - hi) (p - hi
// is exact in fp32), through two products: relative error <= 2^-16.
template <class Ty>
struct Mma;

template <>
struct Mma<F16> {
  static constexpr bool kSplit = false;
  static constexpr uint32_t kOnes = 0x3C003C00u;  // two fp16 1.0
  static __device__ __forceinline__ f32x4 run(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                   __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ void pack(float x, float y, uint32_t& hi, uint32_t& lo) {
    const f16x2 v = {static_cast<_Float16>(x), static_cast<_Float16>(y)};
    hi = __builtin_bit_cast(uint32_t, v);
    lo = 0;
  }
  // l + both halves of a packed pair, each exactly as rounded (times 1.0), in fp32
  static __device__ __forceinline__ float sum2(uint32_t w, float l) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w), f16x2{1.0f16, 1.0f16}, l, false);
  }
};

template <>
struct Mma<BF16> {
  static constexpr bool kSplit = true;
  static constexpr uint32_t kOnes = 0x3F803F80u;  // two bf16 1.0
  static __device__ __forceinline__ f32x4 run(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ void pack(float x, float y, uint32_t& hi, uint32_t& lo) {
    // round to nearest even (v_cvt_pk_bf16_f32); x - hi(x) is exact in fp32
    const bf16x2 h = {static_cast<__bf16>(x), static_cast<__bf16>(y)};
    hi = __builtin_bit_cast(uint32_t, h);
    const bf16x2 l = {static_cast<__bf16>(x - __uint_as_float(hi << 16)),
                      static_cast<__bf16>(y - __uint_as_float(hi & 0xFFFF0000u))};
    lo = __builtin_bit_cast(uint32_t, l);
  }
};

// Stage layout: K and V rows of D halves, unpadded; the 16-byte piece p of row t sits at piece
// p ^ swz(t), which keeps a row's pieces in the row and spreads the reads over the banks:
// K reads take rows r = 0..15 at one logical piece (a distinct piece per row), the V reads
// take 4 rows x 4 columns per 16-lane group (8 distinct pieces x 2 halves).
template <int D>
__device__ __forceinline__ int k_swz(int t) {
  return D == 128 ? (t & 15) : ((t ^ (t >> 3)) & 7);
}
template <int D>
__device__ __forceinline__ int v_swz(int t) {
  return D == 128 ? ((2 * (t & 3)) | (((t >> 2) & 1) << 3)) : (2 * (t & 3));
}

// Zeros that stand in for the K/V rows of the last chunk that the workgroup does not see.
// One wave's load covers 1 KiB.
__device__ const u32x4 kMqZeros[64] = {};

// 16 bytes per lane from global memory straight into LDS: lane l's bytes land at lds + 16 l
// (gfx950 global_load_lds_dwordx4; lds must be the same in every lane).
__device__ __forceinline__ void load16_to_lds(gptr_t src, uint16_t* lds) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src),
                                   (__attribute__((address_space(3))) void*)(lds), 16, 0, 0);
}

// Wait until this wave's loads (the direct-to-LDS ones included) have landed:
// s_waitcnt vmcnt(0), leaving the other counters free.
__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Transposing LDS read of four 16-bit elements (see the lane mapping above).
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t* p) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  return __builtin_bit_cast(uint2, v);
}

// Four waves per SIMD (two workgroups per CU) is what the kernel's latency hiding rests on:
// the register budget is held to that (128 VGPRs); the segment bookkeeping of packed tiles
// would otherwise take it to 136-138.  PACKED: the work list holds packed tiles (several
// sequences per tile); otherwise every tile is one sequence's, and the segment bookkeeping
// folds away at compile time.
template <class Ty, int D, int BS, bool PACKED>
__global__ __launch_bounds__(kMqThreads) __attribute__((amdgpu_waves_per_eu(4))) void
multi_query_kernel(
    typename Ty::store_t* __restrict__ out, const typename Ty::store_t* __restrict__ q,
    const char* __restrict__ k_pool, const char* __restrict__ v_pool,
    const int32_t* __restrict__ block_tables, int max_blocks,
    const int32_t* __restrict__ context_lens, const int32_t* __restrict__ query_start,
    const int32_t* __restrict__ work, const int32_t* __restrict__ packed, int num_seqs,
    int num_tokens, int tiles_per_seq,
    int num_heads, int num_blocks, int max_len, float scale_log2) {
  using T = typename Ty::store_t;
  constexpr int KSTEPS = D / 32;    // k-steps of the score product
  constexpr int DTILES = D / 16;    // 16-row tiles of O^T
  constexpr int COLS = D / 8;       // 16-byte pieces per K/V row
  constexpr int GROUP_ROWS = 64 / COLS;                      // key rows of one wave's pieces
  constexpr int CHUNK_GROUPS = kMqStage / GROUP_ROWS;         // piece groups per stage
  constexpr int GROUPS = (CHUNK_GROUPS + kMqWaves - 1) / kMqWaves;  // ... per wave (at most)
  constexpr bool ALL_GROUPS = CHUNK_GROUPS % kMqWaves == 0;   // every wave loads GROUPS
  constexpr int ROW_BYTES = D * sizeof(T);
  static_assert(sizeof(T) == 2, "16-bit storage only");
  static_assert(BS % GROUP_ROWS == 0, "a wave's piece group lies in one block");

  // The two stage buffers are separate LDS arrays, and the stage loop below is unrolled by
  // two so that each stage's buffers are known at compile time.  Then the compiler can tell
  // that the reads of stage c never touch the buffer that stage c + 1's direct-to-LDS loads
  // fill, and it issues them without waiting for those loads; with one array indexed by
  // c & 1 it waits for every outstanding load first, which serialises loading and computing.
  __shared__ __attribute__((aligned(16))) uint16_t ks0[kMqStage * D];
  __shared__ __attribute__((aligned(16))) uint16_t ks1[kMqStage * D];
  __shared__ __attribute__((aligned(16))) uint16_t vs0[kMqStage * D];
  __shared__ __attribute__((aligned(16))) uint16_t vs1[kMqStage * D];

  // Which (item, head) this workgroup computes.  Workgroups are dealt to the XCDs in turn
  // (workgroup b to XCD b % 8), and each XCD has an L2 of its own.  With a head count that is
  // a multiple of 8, XCD x takes heads x, x + 8, ... and runs kMqXcdChunk consecutive items
  // of one of them before the next, so its L2 holds one head's K/V at a time and the blocks
  // that the items share (a prefix-cache hit's prompt) come from HBM about once per head
  // rather than once per head per pass over the L2.  Otherwise heads go fastest.
  int h, j;
  if (num_heads % kMqXcds == 0) {
    const int hx = num_heads / kMqXcds;                  // heads per XCD
    const int x = static_cast<int>(blockIdx.x % kMqXcds);
    const int k = static_cast<int>(blockIdx.x / kMqXcds);  // this XCD's k-th workgroup
    const int items = static_cast<int>(gridDim.x) / num_heads;
    const int chunk = k / (kMqXcdChunk * hx), within = k % (kMqXcdChunk * hx);
    const int in_chunk = min(kMqXcdChunk, items - chunk * kMqXcdChunk);  // last chunk: fewer
    h = x + kMqXcds * (within / in_chunk);
    j = chunk * kMqXcdChunk + within % in_chunk;
  } else {
    h = static_cast<int>(blockIdx.x % num_heads);
    j = static_cast<int>(blockIdx.x / num_heads);
  }
  // The tile: up to kMqTileQueries consecutive rows of q, from row `first` of sequence sa's
  // new tokens through sequence sb (the rows of consecutive sequences are consecutive in q).
  // Its keys come in segments: the first `pre` keys, which every sequence of the tile holds
  // in the same blocks and every row of it sees, with no mask; then each sequence's keys from
  // `pre` on, seen by that sequence's rows only (pre = 0: one segment per sequence).
  int sa, sb, first, pre;
  if constexpr (PACKED) {
    const int32_t* it = packed + 4 * static_cast<size_t>(j);
    sa = it[0];
    sb = it[1];
    first = it[2];
    pre = it[3];
    if (sa < 0 || sb < sa || sb >= num_seqs || first < 0 || pre < 0 || pre % kMqStage != 0)
      return;  // not a tile of this call
  } else {
    int s, tile;
    if (work) {
      const int item = work[j];
      s = item & kMqItemSeqMask;
      tile = item >> kMqItemSeqBits;
      if (s >= num_seqs || tile >= tiles_per_seq) return;  // not an item of this call
    } else {
      s = j / tiles_per_seq;
      tile = j % tiles_per_seq;
    }
    sa = sb = s;
    first = tile * kMqTileQueries;
    pre = 0;
  }
  // One round of loads serves the common tile of one sequence.
  const int qa = query_start[sa], qa1 = query_start[sa + 1];
  const int La = min(context_lens[sa], max_len);
  if (first >= qa1 - qa) return;  // tile past sa's new tokens (uniform)
  if (qa < 0 || qa1 < qa || qa1 > num_tokens) return;  // rows outside q / out: touch nothing
  for (int m = sa + 1; m <= sb; ++m) {
    const int a = query_start[m], b = query_start[m + 1];
    if (a < 0 || b < a || b > num_tokens) return;
  }
  const int R0 = qa + first;                                     // the tile's first row of q
  const int nq = min(kMqTileQueries, (sb == sa ? qa1 : query_start[sb + 1]) - R0);  // its rows
  const size_t row_stride = static_cast<size_t>(num_heads) * D;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int r = lane & 15, g = lane >> 4;

  // Sequence m's rows of the tile are [lo, hi) (tile-relative), and tile row i sits at
  // position base + i of it; ok: its new tokens are the last tokens of its context (its rows
  // are NaN otherwise).
  struct Member {
    int lo, hi, base;
    bool ok;
  };
  auto member = [&](int m) {
    const int a = m == sa ? qa : query_start[m], b = m == sa ? qa1 : query_start[m + 1];
    const int L = m == sa ? La : min(context_lens[m], max_len);
    Member x;
    x.lo = max(a, R0) - R0;
    x.hi = min(b, R0 + nq) - R0;
    x.base = L - (b - a) - a + R0;
    x.ok = b - a <= L;
    return x;
  };
  // The shared keys: at most what every sequence's first row sees, a whole number of stages,
  // and only if the tables agree on their blocks (otherwise every sequence reads its own).  A
  // tile of one sequence reads its keys in one segment: the same stages.
  if (sb == sa) pre = 0;
  for (int m = sa; m <= sb && pre > 0; ++m) {
    const Member x = member(m);
    if (x.hi > x.lo) pre = x.ok ? min(pre, x.base + x.lo) : 0;
  }
  pre = max(pre, 0) / kMqStage * kMqStage;
  if (pre > 0) {
    const int32_t* ta = block_tables + static_cast<size_t>(sa) * max_blocks;
    bool differ = false;
    for (int m = sa + 1; m <= sb; ++m) {
      const int32_t* tm = block_tables + static_cast<size_t>(m) * max_blocks;
      for (int e = lane; e < pre / BS; e += 64) differ |= tm[e] != ta[e];
    }
    if (__builtin_amdgcn_ballot_w64(differ)) pre = 0;
  }

  // A cursor over the stages: segment m (sa - 1: the shared keys, read through sa's table),
  // its keys from kb (a stage), its end and the offset of its table row.  The table is
  // indexed from the kernel argument at each read: a pointer carried through the loop would
  // hide that it is read-only, and the block ids would then come through vector loads whose
  // wait also waits for the stage loads.
  struct Cur {
    int m, kb, end;
    uint32_t row;
  };
  auto seg_begin = [&](Cur& cu, int m) {
    for (; m <= sb; ++m) {
      if (m < sa) {
        if (pre == 0) continue;
        cu.kb = 0;
        cu.end = pre;
        cu.row = static_cast<uint32_t>(sa) * max_blocks;
      } else {
        const Member x = member(m);
        if (x.hi <= x.lo || !x.ok) continue;
        cu.kb = pre;
        cu.end = x.base + x.hi;
        cu.row = static_cast<uint32_t>(m) * max_blocks;
      }
      break;
    }
    cu.m = m;
  };
  auto advance = [&](Cur& cu) {
    cu.kb += kMqStage;
    if (PACKED && cu.kb >= cu.end) seg_begin(cu, cu.m + 1);  // one segment otherwise
  };
  Cur c0;
  int nstages = 0;
  if (sb == sa) {  // one segment, from key 0
    const Member x = member(sa);
    c0 = {x.ok ? sa : sa + 1, 0, x.base + x.hi, static_cast<uint32_t>(sa) * max_blocks};
    nstages = x.ok ? (c0.end + kMqStage - 1) / kMqStage : 0;
  } else {
    seg_begin(c0, sa - 1);
    for (Cur cu = c0; cu.m <= sb; seg_begin(cu, cu.m + 1))
      nstages += (cu.end - cu.kb + kMqStage - 1) / kMqStage;
  }
  if (nstages == 0) {  // no sequence of the tile has a valid context: NaN rows
    for (int e = tid; e < nq * D; e += kMqThreads)
      out[static_cast<size_t>(R0 + e / D) * row_stride + static_cast<size_t>(h) * D + e % D] =
          Ty::store(NAN);
    return;
  }

  // This wave's rows are [w0, w1) of the tile; a lane's row i past the tile's end computes a
  // copy of its last row.
  const int w0 = wave * kMqWaveQueries;
  const int w1 = min(w0 + kMqWaveQueries, nq);
  const bool wave_on = w0 < nq;
  bool qt_on[kMqQt];
  int qi[kMqQt];
#pragma unroll
  for (int qt = 0; qt < kMqQt; ++qt) {
    qt_on[qt] = w0 + 16 * qt < nq;
    qi[qt] = min(w0 + 16 * qt + r, nq - 1);
  }

  // q rows as B fragments: lane (r, g) holds q[r][32k + 8g .. 32k + 8g + 7] of each tile.
  u32x4 qf[kMqQt][KSTEPS];
#pragma unroll
  for (int qt = 0; qt < kMqQt; ++qt) {
    const T* qrow = q + static_cast<size_t>(R0 + qi[qt]) * row_stride + static_cast<size_t>(h) * D;
#pragma unroll
    for (int k = 0; k < KSTEPS; ++k) qf[qt][k] = load16(qrow + 32 * k + 8 * g);
  }

  // Staging.  Piece group i of this wave covers key rows row0 .. row0 + GROUP_ROWS - 1 of a
  // chunk, 1 KiB that one direct-to-LDS load of the wave fills: lane l lands at stage row
  // l / COLS, stage piece l % COLS, which under the stage swizzle holds logical piece
  // (l % COLS) ^ swz(row), so that is the piece lane l loads.  The rows lie in one block: its
  // id is a scalar and a lane's byte offset inside the group never changes.  In the last
  // chunk, rows the workgroup does not see read zeros; a block id outside the pool is
  // clamped into it for the read and turns the outputs into NaN.
  // Loop-invariant parts of a group's address: stages start at whole multiples of the stage
  // (segments too), which is a whole number of blocks, so the group's row inside its block
  // never changes.
  static_assert(kMqStage % BS == 0 || BS % kMqStage == 0, "stages align with blocks");
  const uint64_t block_stride = static_cast<uint64_t>(num_heads) * BS * ROW_BYTES;
  const gptr_t zeros = uniform_ptr(reinterpret_cast<const char*>(kMqZeros)) + 16 * lane;
  gptr_t kgrp[GROUPS], vgrp[GROUPS];
  uint32_t grp_row[GROUPS], koff[GROUPS], voff[GROUPS];
#pragma unroll
  for (int i = 0; i < GROUPS; ++i) {
    grp_row[i] = (i * kMqWaves + wave) * GROUP_ROWS;
    const uint64_t off = (static_cast<uint64_t>(h) * BS + grp_row[i] % BS) * ROW_BYTES;
    kgrp[i] = uniform_ptr(k_pool) + off;
    vgrp[i] = uniform_ptr(v_pool) + off;
    const int t = static_cast<int>(grp_row[i] + lane / COLS) % kMqChunk;
    const int lc = static_cast<int>(lane % COLS);
    koff[i] = (lane / COLS) * ROW_BYTES + 16 * (lc ^ k_swz<D>(t));
    voff[i] = (lane / COLS) * ROW_BYTES + 16 * (lc ^ v_swz<D>(t));
  }
  uint32_t bid[GROUPS] = {};  // block ids of the groups of the next chunk to fetch, loaded early
  // Largest block id fetched.  An id outside the pool is clamped into it (the read stays in
  // bounds) and turns the outputs into NaN at the end.  Groups of a segment's last stage that
  // reach past its keys read the block of its last key (clamped table index).
  uint32_t max_bid = 0;
  const uint32_t last_block = static_cast<uint32_t>(num_blocks - 1);
  auto load_ids = [&](const Cur& cu) {
    const uint32_t last = static_cast<uint32_t>(cu.end - 1);
#pragma unroll
    for (int i = 0; i < GROUPS; ++i)
      if (ALL_GROUPS || grp_row[i] < kMqStage)
        bid[i] = block_tables[static_cast<size_t>(cu.row) +
                              min(static_cast<uint32_t>(cu.kb) + grp_row[i], last) / BS];
  };
  // the stage at cursor cu -> stage buffers (kst, vst), asynchronously (complete after
  // wait_loads)
  auto fetch = [&](const Cur& cu, uint16_t* kst, uint16_t* vst) {
    const bool tail = cu.kb + kMqStage > cu.end;  // uniform
#pragma unroll
    for (int i = 0; i < GROUPS; ++i) {
      if (!ALL_GROUPS && grp_row[i] >= kMqStage) continue;  // more waves than groups
      max_bid = max(max_bid, bid[i]);
      const uint64_t off = static_cast<uint64_t>(min(bid[i], last_block)) * block_stride;
      gptr_t kp = kgrp[i] + off + koff[i];
      gptr_t vp = vgrp[i] + off + voff[i];
      if (tail && cu.kb + static_cast<int>(grp_row[i] + lane / COLS) >= cu.end) {
        kp = zeros;
        vp = zeros;
      }
      load16_to_lds(kp, &kst[grp_row[i] * D]);
      load16_to_lds(vp, &vst[grp_row[i] * D]);
    }
  };

  f32x4 acc[kMqQt][DTILES];
#pragma unroll
  for (int qt = 0; qt < kMqQt; ++qt)
#pragma unroll
    for (int t = 0; t < DTILES; ++t) acc[qt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Softmax reference m (log2 units, equal in a query's four lanes) and the denominator, the
  // sum of exactly the probabilities that enter the output products.  fp16 adds its rounded
  // probability pairs with v_dot2 into a per-lane partial (a query's four lanes are added at
  // the end); bf16, whose probabilities enter in two parts, accumulates them through one more
  // 16 x 16 output tile whose V^T rows are all ones, in every lane of the query (two products
  // per step cost it less than eight v_dot2).
  using den_t = std::conditional_t<Mma<Ty>::kSplit, f32x4, float>;
  // The move test runs on raw scores against mraw = (m + kMqSlack) / scale, so a lane need
  // not scale its largest score first; rounding here only shifts the point at which the exact
  // test below is made.  m starts finite: a step in which a query sees no key (in a packed
  // tile, another sequence's keys) then adds exp2(-inf) = 0 for it, not NaN; its first key
  // seen moves m (mraw starts at -inf) and scales the empty accumulators by exp2(-1e30 - m).
  const float inv_scale = 1.0f / scale_log2;
  float m[kMqQt], mraw[kMqQt];
  den_t den[kMqQt];
#pragma unroll
  for (int qt = 0; qt < kMqQt; ++qt) {
    m[qt] = -1e30f;
    mraw[qt] = -INFINITY;
    den[qt] = den_t{};
  }
  // The last key each lane's query sees in the current segment (-1: the segment belongs to
  // another sequence), and the wave's bounds there: keys past wave_keys are seen by none of
  // its queries, keys below wave_unmasked by all of them.
  int qpos[kMqQt];
  int seg_m = sa - 2, wave_keys = 0, wave_unmasked = 0;
  bool seg_on = false;
  auto enter_segment = [&](int mm) {
    seg_m = mm;
    if (mm < sa) {  // the shared keys: every query sees all of them
      seg_on = wave_on;
      wave_keys = wave_unmasked = pre;
#pragma unroll
      for (int qt = 0; qt < kMqQt; ++qt) qpos[qt] = pre;
      return;
    }
    const Member x = member(mm);
    const int a = max(w0, x.lo), b = min(w1, x.hi);
    seg_on = a < b;
    wave_keys = x.base + b;
    wave_unmasked = (a == w0 && b == w1) ? x.base + a + 1 : 0;
#pragma unroll
    for (int qt = 0; qt < kMqQt; ++qt)
      qpos[qt] = (qi[qt] >= x.lo && qi[qt] < x.hi) ? x.base + qi[qt] : -1;
  };

  // One chunk of keys, from position kpos on, for the query tiles of the wave.  mask: the
  // chunk holds keys that some query of the wave does not see (its own later positions, keys
  // past the segment's, another sequence's); wave-uniform.
  auto chunk_step = [&](const uint16_t* kst, const uint16_t* vst, int kpos, bool mask) {
    // all K fragments of the chunk first, then the products k-step by k-step over the
    // independent accumulators (query tiles x two 16-key halves)
    u32x4 kf[2][KSTEPS];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int k = 0; k < KSTEPS; ++k)
        kf[hh][k] = *reinterpret_cast<const u32x4*>(
            &kst[(16 * hh + r) * D + 8 * ((4 * k + g) ^ k_swz<D>(16 * hh + r))]);
    f32x4 sc[kMqQt][2];
#pragma unroll
    for (int qt = 0; qt < kMqQt; ++qt) sc[qt][0] = sc[qt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < KSTEPS; ++k)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int qt = 0; qt < kMqQt; ++qt) sc[qt][hh] = Mma<Ty>::run(kf[hh][k], qf[qt][k], sc[qt][hh]);
    float z[kMqQt][8];
#pragma unroll
    for (int qt = 0; qt < kMqQt; ++qt)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int i = 0; i < 4; ++i) z[qt][4 * hh + i] = sc[qt][hh][i];
    if (mask) {
      // score e of lane (r, g) is key kpos + 4g + 16 (e / 4) + e % 4: compared against the
      // query's last key taken relative to kpos + 4g, each test is against a constant
#pragma unroll
      for (int qt = 0; qt < kMqQt; ++qt) {
        const int rel = qpos[qt] - kpos - 4 * g;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (16 * (e >> 2) + (e & 3) > rel) z[qt][e] = -INFINITY;
      }
    }
    // Online softmax with a lazily moved reference: m moves only when a scaled score exceeds
    // it by more than kMqSlack, so probabilities stay below 2^kMqSlack and the accumulators
    // are rescaled only on those rare moves.  scale > 0, so the largest raw score gives the
    // largest scaled one, and exp2(scale * s - m) is one FMA and one exp.  A lane first
    // checks its own scores; only when some lane of the wave would move is the maximum over
    // each query's four lanes taken (so the four lanes of a query always agree on m).
    float rmax[kMqQt];
#pragma unroll
    for (int qt = 0; qt < kMqQt; ++qt) {
      // IEEE-754 maximum (a NaN propagates; a NaN score spoils its query either way): gfx950
      // has it as a three-input instruction that takes the products' results as they are
      auto mx = [](float a, float b) { return __builtin_elementwise_maximum(a, b); };
      const float a = mx(mx(z[qt][0], z[qt][1]), z[qt][2]);
      const float b = mx(mx(z[qt][3], z[qt][4]), z[qt][5]);
      rmax[qt] = mx(b, mx(mx(z[qt][6], z[qt][7]), a));
    }
    float alpha[kMqQt];
    bool move = false;
#pragma unroll
    for (int qt = 0; qt < kMqQt; ++qt) {
      alpha[qt] = 1.0f;
      move |= rmax[qt] > mraw[qt];  // raw-score form of: rmax * scale > m + kMqSlack
    }
    if (__builtin_amdgcn_ballot_w64(move)) {
#pragma unroll
      for (int qt = 0; qt < kMqQt; ++qt) {
        const float lmax = rmax[qt] * scale_log2;
        float cm = fmaxf(lmax, __shfl_xor(lmax, 16, 64));
        cm = fmaxf(cm, __shfl_xor(cm, 32, 64));
        if (cm > m[qt] + kMqSlack) {
          alpha[qt] = __builtin_amdgcn_exp2f(m[qt] - cm);
          m[qt] = cm;
          mraw[qt] = (cm + kMqSlack) * inv_scale;
        }
      }
      // the accumulators follow the moved reference (alpha = 1 where it did not move)
#pragma unroll
      for (int qt = 0; qt < kMqQt; ++qt) {
#pragma unroll
        for (int t = 0; t < DTILES; ++t) acc[qt][t] *= alpha[qt];
        den[qt] *= alpha[qt];
      }
    }
    u32x4 pf[kMqQt], pfl[kMqQt];
#pragma unroll
    for (int qt = 0; qt < kMqQt; ++qt) {
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) p[e] = __builtin_amdgcn_exp2f(fmaf(z[qt][e], scale_log2, -m[qt]));
      uint32_t ph[4], pl[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        Mma<Ty>::pack(p[2 * w], p[2 * w + 1], ph[w], pl[w]);
        if constexpr (!Mma<Ty>::kSplit) den[qt] = Mma<Ty>::sum2(ph[w], den[qt]);
      }
      pf[qt] = u32x4{ph[0], ph[1], ph[2], ph[3]};
      pfl[qt] = u32x4{pl[0], pl[1], pl[2], pl[3]};
    }
    // outputs: V^T fragments through the transposing read
    // lane (r, g) reads 4 elements of key row 4g + r / 4 (and 16 more) at head-dim column
    // 16 t + 4 (r % 4): 16-byte piece 2t + (r / 2) % 2, half r % 2 of it
    const int vr = 4 * g + (r >> 2);
    const int vpc = ((r >> 1) & 1) ^ v_swz<D>(vr);       // v_swz(vr + 16) == v_swz(vr)
    const uint16_t* vrow = &vst[vr * D + 4 * (r & 1)];
#pragma unroll
    for (int t = 0; t < DTILES; ++t) {
      const int off = 8 * ((2 * t) ^ vpc);
      const uint2 lo = lds_read_tr16(vrow + off);
      const uint2 hi = lds_read_tr16(vrow + 16 * D + off);
      const u32x4 a = {lo.x, lo.y, hi.x, hi.y};
#pragma unroll
      for (int qt = 0; qt < kMqQt; ++qt) {
        acc[qt][t] = Mma<Ty>::run(a, pf[qt], acc[qt][t]);
        if constexpr (Mma<Ty>::kSplit) acc[qt][t] = Mma<Ty>::run(a, pfl[qt], acc[qt][t]);
      }
    }
    if constexpr (Mma<Ty>::kSplit) {
      const u32x4 ones = {Mma<Ty>::kOnes, Mma<Ty>::kOnes, Mma<Ty>::kOnes, Mma<Ty>::kOnes};
#pragma unroll
      for (int qt = 0; qt < kMqQt; ++qt) {
        den[qt] = Mma<Ty>::run(ones, pf[qt], den[qt]);
        den[qt] = Mma<Ty>::run(ones, pfl[qt], den[qt]);
      }
    }
  };

  if (!PACKED) enter_segment(sa);
  // cursors at stage c (computed), c + 1 (being fetched) and c + 2 (its block ids read)
  Cur cc = c0, cf = c0;
  load_ids(c0);
  fetch(c0, ks0, vs0);
  advance(cf);
  if (nstages > 1) load_ids(cf);
  Cur ci = cf;
  advance(ci);
  wait_loads();
  __syncthreads();
  // One stage: load stage c + 1 into (knext, vnext) while stage c is read from (kcur, vcur).
  auto step = [&](int c, const uint16_t* kcur, const uint16_t* vcur, uint16_t* knext,
                  uint16_t* vnext) {
    if (c + 1 < nstages) {
      fetch(cf, knext, vnext);  // the other buffer was last read during stage c - 1
      if (c + 2 < nstages) load_ids(ci);
    }
    if (PACKED && cc.m != seg_m) enter_segment(cc.m);
    // a tile past the wave's queries, or one whose queries all come before this step, gets
    // only masked scores and adds nothing
#pragma unroll
    for (int u = 0; u < kMqSub; ++u) {
      const int kpos = cc.kb + u * kMqChunk;  // 32-key compute step
      if (seg_on && kpos < wave_keys)
        chunk_step(kcur + u * kMqChunk * D, vcur + u * kMqChunk * D, kpos,
                   kpos + kMqChunk > wave_unmasked);
    }
    wait_loads();  // stage c + 1 has landed in this wave's part of the other buffer
    __syncthreads();
    cc = cf;
    cf = ci;
    advance(ci);
  };
  for (int c = 0; c < nstages; c += 2) {
    step(c, ks0, vs0, ks1, vs1);
    if (c + 1 < nstages) step(c + 1, ks1, vs1, ks0, vs0);
  }

  // Every wave reads what the others staged: a bad id seen by any wave spoils them all.  The
  // K stage is idle after the loop's last barrier; it carries one flag per wave.
  if (lane == 0) ks0[wave] = max_bid > last_block ? 1 : 0;
  __syncthreads();
  bool any_bad = false;
#pragma unroll
  for (int w = 0; w < kMqWaves; ++w) any_bad |= ks0[w] != 0;
#pragma unroll
  for (int qt = 0; qt < kMqQt; ++qt) {
    float l;
    if constexpr (Mma<Ty>::kSplit) {
      l = den[qt][0];
    } else {
      l = den[qt] + __shfl_xor(den[qt], 16, 64);  // the query's four lanes
      l += __shfl_xor(l, 32, 64);
    }
    const int i = w0 + 16 * qt + r;  // the lane's row of the tile
    if (!qt_on[qt] || i >= nq) continue;
    bool row_ok = !any_bad;           // and the rows of a sequence with n_s > L_s are NaN
    for (int mm = sa; mm <= sb; ++mm) {
      const Member x = member(mm);
      if (!x.ok && i >= x.lo && i < x.hi) row_ok = false;
    }
    const float inv = row_ok ? 1.0f / l : NAN;
    T* orow = out + static_cast<size_t>(R0 + i) * row_stride + static_cast<size_t>(h) * D;
#pragma unroll
    for (int t = 0; t < DTILES; ++t) {
      T o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = Ty::store(acc[qt][t][i] * inv);
      uint2 w;
      __builtin_memcpy(&w, o, sizeof(w));
      *reinterpret_cast<uint2*>(orow + 16 * t + 4 * g) = w;
    }
  }
}

// ------------------------------------------------------------------ host side
struct MqArgs {
  void* out;
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_tables;
  int max_blocks;
  const int32_t* context_lens;
  const int32_t* query_start;
  const int32_t* work;
  const int32_t* packed;
  int64_t wgs;
  int num_seqs;
  int num_tokens;
  int tiles_per_seq;
  int num_heads;
  int num_blocks;
  int max_len;
  float scale_log2;
  hipStream_t stream;
  hipEvent_t start, stop;  // taken by the launch itself, or null
};

template <class Ty, int D, int BS>
static void launch_mq(const MqArgs& a) {
  using T = typename Ty::store_t;
  if (a.wgs <= 0) return;
  hipExtLaunchKernelGGL((a.packed ? multi_query_kernel<Ty, D, BS, true>
                                  : multi_query_kernel<Ty, D, BS, false>),
                     dim3(static_cast<unsigned>(a.wgs)),
                     dim3(kMqThreads), 0, a.stream, a.start, a.stop, 0u, static_cast<T*>(a.out),
                     static_cast<const T*>(a.q), static_cast<const char*>(a.k_pool),
                     static_cast<const char*>(a.v_pool), a.block_tables, a.max_blocks,
                     a.context_lens, a.query_start, a.work, a.packed, a.num_seqs, a.num_tokens,
                     a.tiles_per_seq, a.num_heads, a.num_blocks, a.max_len, a.scale_log2);
}

template <class Ty, int D>
static pkv_status_t mq_dispatch_bs(int bs, const MqArgs& a) {
  switch (bs) {
    case 8: launch_mq<Ty, D, 8>(a); return PKV_OK;
    case 16: launch_mq<Ty, D, 16>(a); return PKV_OK;
    case 32: launch_mq<Ty, D, 32>(a); return PKV_OK;
  }
  return PKV_EUNSUPPORTED;
}

template <class Ty>
static pkv_status_t mq_dispatch_d(int dim, int bs, const MqArgs& a) {
  switch (dim) {
    case 64: return mq_dispatch_bs<Ty, 64>(bs, a);
    case 128: return mq_dispatch_bs<Ty, 128>(bs, a);
  }
  return PKV_EUNSUPPORTED;
}

static bool aligned16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" {

int32_t pkv_multi_query_tile(void) { return kMqTileQueries; }

int32_t pkv_multi_query_schedule_grouped(const int32_t* query_start,
                                         const int32_t* context_lens, const int32_t* group_keys,
                                         int32_t num_seqs, int32_t max_context_len,
                                         int32_t* items, int32_t capacity) {
  if (num_seqs < 0 || max_context_len < 0 || capacity < 0 || num_seqs > kMqItemSeqMask + 1 ||
      (num_seqs > 0 && (!query_start || !context_lens || !items)))
    return -1;
  struct Item {
    int64_t group_keys;  // keys read by the largest tile of the sequence's group
    int32_t leader;      // first sequence of the group
    int64_t seq_keys;    // keys read by the sequence's largest tile
    int64_t keys;        // keys read by this tile
    int32_t s, tile;
  };
  // group leader = first sequence with the same key (sequences sharing prefix blocks); with
  // no keys every sequence is a group of its own
  std::vector<int32_t> leader(static_cast<size_t>(num_seqs));
  if (group_keys) {
    std::vector<std::pair<int32_t, int32_t>> kv;
    kv.reserve(static_cast<size_t>(num_seqs));
    for (int32_t s = 0; s < num_seqs; ++s) kv.push_back({group_keys[s], s});
    std::sort(kv.begin(), kv.end());
    for (size_t i = 0; i < kv.size(); ++i)
      leader[kv[i].second] = (i > 0 && kv[i].first == kv[i - 1].first)
                                 ? leader[kv[i - 1].second] : kv[i].second;
  } else {
    for (int32_t s = 0; s < num_seqs; ++s) leader[s] = s;
  }
  std::vector<Item> list;
  std::vector<int64_t> best(static_cast<size_t>(num_seqs), 0);
  for (int s = 0; s < num_seqs; ++s) {
    const int64_t n = static_cast<int64_t>(query_start[s + 1]) - query_start[s];
    if (n < 0) return -1;
    if (n == 0) continue;
    const int64_t tiles = (n + kMqTileQueries - 1) / kMqTileQueries;
    if (tiles > kMqMaxTiles) return -1;
    const int64_t L = std::min<int64_t>(context_lens[s], max_context_len);
    const int64_t base = std::max<int64_t>(L - n, 0);
    best[leader[s]] = std::max(best[leader[s]], base + n);
    for (int64_t t = 0; t < tiles; ++t) {
      const int64_t keys = base + std::min<int64_t>(n, (t + 1) * kMqTileQueries);
      list.push_back({0, leader[s], base + n, keys, s, static_cast<int32_t>(t)});
    }
  }
  if (static_cast<int64_t>(list.size()) > capacity) return -1;
  for (Item& it : list) it.group_keys = best[it.leader];
  // Groups that read the most keys first, a group's sequences adjacent (so the prefix blocks
  // they share stay in L2 while they run), inside a group the longest sequences first, and a
  // sequence's tiles adjacent (largest first) so that they share its own K/V in L2 too.
  std::stable_sort(list.begin(), list.end(), [](const Item& x, const Item& y) {
    if (x.group_keys != y.group_keys) return x.group_keys > y.group_keys;
    if (x.leader != y.leader) return x.leader < y.leader;
    if (x.seq_keys != y.seq_keys) return x.seq_keys > y.seq_keys;
    if (x.s != y.s) return x.s < y.s;
    return x.keys > y.keys;
  });
  for (size_t i = 0; i < list.size(); ++i)
    items[i] = list[i].s | (list[i].tile << kMqItemSeqBits);
  return static_cast<int32_t>(list.size());
}

int32_t pkv_multi_query_schedule(const int32_t* query_start, const int32_t* context_lens,
                                 int32_t num_seqs, int32_t max_context_len, int32_t* items,
                                 int32_t capacity) {
  return pkv_multi_query_schedule_grouped(query_start, context_lens, nullptr, num_seqs,
                                          max_context_len, items, capacity);
}

int32_t pkv_multi_query_schedule_packed(const int32_t* query_start,
                                        const int32_t* context_lens,
                                        const int32_t* block_tables, int32_t max_blocks,
                                        int32_t block_size, int32_t num_seqs,
                                        int32_t max_context_len, int32_t* tiles,
                                        int32_t capacity) {
  if (num_seqs < 0 || max_context_len < 0 || capacity < 0 || max_blocks <= 0 ||
      block_size <= 0 ||
      (num_seqs > 0 && (!query_start || !context_lens || !block_tables || !tiles)))
    return -1;
  if (num_seqs == 0) return 0;
  for (int32_t s = 0; s < num_seqs; ++s)
    if (query_start[s + 1] < query_start[s]) return -1;
  const int64_t width = std::min<int64_t>(max_context_len,
                                          static_cast<int64_t>(max_blocks) * block_size);
  auto cached = [&](int32_t s) {  // tokens before the first new one, at most the table's
    const int64_t n = static_cast<int64_t>(query_start[s + 1]) - query_start[s];
    return std::min<int64_t>(context_lens[s], width) - n;
  };
  // keys that sequences s and t hold in the same blocks, in whole stages
  auto shared = [&](int32_t s, int32_t t, int64_t cap) -> int64_t {
    if (kMqStage % block_size != 0) return 0;
    const int32_t* ts = block_tables + static_cast<size_t>(s) * max_blocks;
    const int32_t* tt = block_tables + static_cast<size_t>(t) * max_blocks;
    int64_t keys = std::max<int64_t>(std::min({cap, cached(s), cached(t)}), 0);
    keys = keys / kMqStage * kMqStage;
    for (int64_t e = 0; e < keys / block_size; ++e)
      if (ts[e] != tt[e]) return e * block_size / kMqStage * kMqStage;
    return keys;
  };
  struct Tile {
    int64_t run_keys;  // keys read by the run's largest tile
    int32_t run;       // first sequence of the run
    int64_t keys;      // keys read by this tile
    int32_t sa, sb, first, pre;
  };
  std::vector<Tile> list;
  int32_t s = 0;
  while (s < num_seqs) {
    if (query_start[s + 1] == query_start[s]) {
      ++s;
      continue;
    }
    // A run: consecutive sequences with new tokens that all hold the same first `pre` keys
    // (at least one stage) in the same blocks; the second member fixes pre, and a sequence
    // that shares fewer of them starts a run of its own.
    int32_t t = s + 1;
    int64_t pre = 0;
    for (; t < num_seqs && query_start[t + 1] > query_start[t]; ++t) {
      const int64_t p = shared(s, t, t == s + 1 ? INT64_MAX : pre);
      if (t == s + 1 ? p < kMqStage : p != pre) break;
      pre = p;
    }
    if (t == s + 1) pre = 0;
    const int64_t rows = static_cast<int64_t>(query_start[t]) - query_start[s];
    const size_t begin = list.size();
    int32_t m = s;
    for (int64_t r0 = 0; r0 < rows; r0 += kMqTileQueries) {
      const int64_t R0 = query_start[s] + r0;
      const int64_t R1 = std::min<int64_t>(R0 + kMqTileQueries, query_start[t]);
      while (query_start[m + 1] <= R0) ++m;
      Tile tl{0, s, 0, m, m, static_cast<int32_t>(R0 - query_start[m]),
              static_cast<int32_t>(pre)};
      int64_t keys = pre;
      for (int32_t mm = m; mm < t && query_start[mm] < R1; ++mm) {
        tl.sb = mm;
        // keys of mm's last row in the tile, past the shared ones
        const int64_t last = std::min<int64_t>(R1, query_start[mm + 1]) - 1;
        keys += std::max<int64_t>(cached(mm) + (last - query_start[mm]) + 1 - pre, 0);
      }
      tl.keys = keys;
      list.push_back(tl);
    }
    int64_t most = 0;
    for (size_t i = begin; i < list.size(); ++i) most = std::max(most, list[i].keys);
    for (size_t i = begin; i < list.size(); ++i) list[i].run_keys = most;
    s = t;
  }
  if (static_cast<int64_t>(list.size()) > capacity) return -1;
  // Runs that read the most keys first, a run's tiles adjacent (so the blocks they share stay
  // in L2 while they run), inside a run the tiles reading the most keys first.
  std::stable_sort(list.begin(), list.end(), [](const Tile& x, const Tile& y) {
    if (x.run_keys != y.run_keys) return x.run_keys > y.run_keys;
    if (x.run != y.run) return x.run < y.run;
    return x.keys > y.keys;
  });
  for (size_t i = 0; i < list.size(); ++i) {
    tiles[4 * i + 0] = list[i].sa;
    tiles[4 * i + 1] = list[i].sb;
    tiles[4 * i + 2] = list[i].first;
    tiles[4 * i + 3] = list[i].pre;
  }
  return static_cast<int32_t>(list.size());
}

// What both launch entry points check, and the launch.
static pkv_status_t mq_launch(const pkv_cache_desc_t* desc, void* out, const void* q,
                              const void* k_pool, const void* v_pool,
                              const int32_t* block_tables, int32_t max_blocks_per_seq,
                              const int32_t* context_lens, const int32_t* query_start,
                              int32_t num_seqs, int32_t num_tokens, int32_t max_query_len,
                              int32_t max_context_len, float scale, const int32_t* work_items,
                              const int32_t* packed, bool use_packed, int32_t num_items,
                              pkv_stream_t stream, void* ev_start = nullptr,
                              void* ev_stop = nullptr) {
  pkv_status_t st = check_desc(desc);
  if (st != PKV_OK) return st;
  if (desc->dtype != PKV_F16 && desc->dtype != PKV_BF16) return PKV_EUNSUPPORTED;
  if (num_seqs < 0 || num_tokens < 0 || max_query_len < 0 || max_context_len < 0 ||
      max_blocks_per_seq <= 0 || !std::isfinite(scale) || !(scale > 0.0f) || num_items < 0)
    return PKV_EINVAL;
  if (num_seqs == 0 || num_tokens == 0 || max_query_len == 0) return PKV_OK;
  if (use_packed && num_items == 0) return PKV_OK;
  if (use_packed && (!packed || reinterpret_cast<uintptr_t>(packed) % 16 != 0))
    return PKV_EINVAL;
  if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens || !query_start)
    return PKV_EINVAL;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool))
    return PKV_EINVAL;
  if (num_seqs > kMqItemSeqMask + 1) return PKV_EUNSUPPORTED;
  // table rows are addressed with 32-bit offsets
  if (static_cast<int64_t>(num_seqs) * max_blocks_per_seq > UINT32_MAX) return PKV_EUNSUPPORTED;
  const int64_t tiles = (static_cast<int64_t>(max_query_len) + kMqTileQueries - 1) / kMqTileQueries;
  if (tiles > kMqMaxTiles) return PKV_EUNSUPPORTED;

  MqArgs a{};
  if (use_packed || work_items) {
    if (num_items > static_cast<int64_t>(num_seqs) * tiles) return PKV_EINVAL;
    a.wgs = static_cast<int64_t>(num_items) * desc->num_heads;
  } else {
    a.wgs = static_cast<int64_t>(num_seqs) * tiles * desc->num_heads;
  }
  if (a.wgs > INT32_MAX) return PKV_EUNSUPPORTED;
  a.out = out;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_tables = block_tables;
  a.max_blocks = max_blocks_per_seq;
  a.context_lens = context_lens;
  a.query_start = query_start;
  a.work = use_packed ? nullptr : work_items;
  a.packed = use_packed ? packed : nullptr;
  a.num_seqs = num_seqs;
  a.num_tokens = num_tokens;
  a.tiles_per_seq = static_cast<int>(tiles);
  a.num_heads = desc->num_heads;
  a.num_blocks = desc->num_blocks;
  a.max_len = static_cast<int>(std::min<int64_t>(
      max_context_len, static_cast<int64_t>(max_blocks_per_seq) * desc->block_size));
  a.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  a.stream = static_cast<hipStream_t>(stream);
  a.start = static_cast<hipEvent_t>(ev_start);
  a.stop = static_cast<hipEvent_t>(ev_stop);

  (void)hipGetLastError();  // clear a stale error so it is not blamed on this launch
  st = desc->dtype == PKV_F16 ? mq_dispatch_d<F16>(desc->head_dim, desc->block_size, a)
                              : mq_dispatch_d<BF16>(desc->head_dim, desc->block_size, a);
  if (st != PKV_OK) return st;
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_EHIP;
}

}  // extern "C"

pkv_status_t pkv::multi_query_packed_timed(
    const pkv_cache_desc_t* desc, void* out, const void* q, const void* k_pool,
    const void* v_pool, const int32_t* block_tables, int32_t max_blocks_per_seq,
    const int32_t* context_lens, const int32_t* query_start, int32_t num_seqs,
    int32_t num_tokens, int32_t max_query_len, int32_t max_context_len, float scale,
    const int32_t* tiles, int32_t num_tiles, pkv_stream_t stream, void* ev_start,
    void* ev_stop) {
  return mq_launch(desc, out, q, k_pool, v_pool, block_tables, max_blocks_per_seq,
                   context_lens, query_start, num_seqs, num_tokens, max_query_len,
                   max_context_len, scale, nullptr, tiles, true, num_tiles, stream, ev_start,
                   ev_stop);
}

extern "C" {

pkv_status_t pkv_paged_attention_multi_query(
    const pkv_cache_desc_t* desc, void* out, const void* q, const void* k_pool,
    const void* v_pool, const int32_t* block_tables, int32_t max_blocks_per_seq,
    const int32_t* context_lens, const int32_t* query_start, int32_t num_seqs,
    int32_t num_tokens, int32_t max_query_len, int32_t max_context_len, float scale,
    const int32_t* work_items, int32_t num_items, pkv_stream_t stream) {
  return mq_launch(desc, out, q, k_pool, v_pool, block_tables, max_blocks_per_seq,
                   context_lens, query_start, num_seqs, num_tokens, max_query_len,
                   max_context_len, scale, work_items, nullptr, false,
                   work_items ? num_items : 0, stream);
}

pkv_status_t pkv_paged_attention_multi_query_packed(
    const pkv_cache_desc_t* desc, void* out, const void* q, const void* k_pool,
    const void* v_pool, const int32_t* block_tables, int32_t max_blocks_per_seq,
    const int32_t* context_lens, const int32_t* query_start, int32_t num_seqs,
    int32_t num_tokens, int32_t max_query_len, int32_t max_context_len, float scale,
    const int32_t* tiles, int32_t num_tiles, pkv_stream_t stream) {
  return mq_launch(desc, out, q, k_pool, v_pool, block_tables, max_blocks_per_seq,
                   context_lens, query_start, num_seqs, num_tokens, max_query_len,
                   max_context_len, scale, nullptr, tiles, true, num_tiles, stream);
}

}  // extern "C"
