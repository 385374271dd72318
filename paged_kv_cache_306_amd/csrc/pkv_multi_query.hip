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
//   * one workgroup = four waves = 64 consecutive new tokens of one (sequence, head); each
//     wave owns 16 of them;
//   * keys go 32 at a time through LDS: K rows as stored, V transposed (row = head dim);
//   * scores S^T = K Q^T: K rows are the A operand, the wave's q rows (kept in registers for
//     the whole run) the B operand; lane (r, g) = (lane % 16, lane / 16) receives the scores
//     of query r against keys 4g .. 4g+3 of each 16-key half of the chunk;
//   * softmax runs per query in log2 units with the running max shared by the four lanes of
//     a query (two cross-row shuffles per chunk); each lane's probabilities, in the storage
//     type, are directly the B operand of O^T = V^T P^T once the V^T columns are
//     stored in the matching key order (slot 8g + j holds key 4g + j for j < 4 and key
//     16 + 4g + j - 4 for j >= 4);
//   * O^T accumulates in 16 x 16 tiles: lane (r, g) holds output elements d = 16 t + 4 g + i
//     of query r.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <vector>

#include "pkv.h"
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kMqThreads = 256;     // four waves
constexpr int kMqTileQueries = 64;  // new tokens per workgroup, 16 per wave
constexpr int kMqChunk = 32;        // keys staged in LDS per step
constexpr int kMqItemSeqBits = 20;  // work item = sequence | tile << 20
constexpr int kMqItemSeqMask = (1 << kMqItemSeqBits) - 1;
constexpr int kMqMaxTiles = 1 << (31 - kMqItemSeqBits);

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

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
  static __device__ __forceinline__ f32x4 run(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                   __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ void pack(float x, float y, uint32_t& hi, uint32_t& lo) {
    const f16x2 v = {static_cast<_Float16>(x), static_cast<_Float16>(y)};
    hi = __builtin_bit_cast(uint32_t, v);
    lo = 0;
  }
};

template <>
struct Mma<BF16> {
  static constexpr bool kSplit = true;
  static __device__ __forceinline__ f32x4 run(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ void split(float x, uint32_t& hi, uint32_t& lo) {
    hi = BF16::store(x);  // probabilities are finite, in [0, 1]
    lo = BF16::store(x - __uint_as_float(hi << 16));
  }
  static __device__ __forceinline__ void pack(float x, float y, uint32_t& hi, uint32_t& lo) {
    uint32_t hx, lx, hy, ly;
    split(x, hx, lx);
    split(y, hy, ly);
    hi = hx | (hy << 16);
    lo = lx | (ly << 16);
  }
};

// Position of V^T's 16-byte slot group `grp` in LDS row d: the groups of a row are permuted
// by bits 3..4 of d so that the transposing writes of one instruction (rows 8 apart) spread
// over more banks.  Reads stay one whole 1 KiB tile per instruction, conflict free.
__device__ __forceinline__ int vt_group(int d, int grp) { return grp ^ ((d >> 3) & 3); }

template <class Ty, int D, int BS>
__global__ __launch_bounds__(kMqThreads) void multi_query_kernel(
    typename Ty::store_t* __restrict__ out, const typename Ty::store_t* __restrict__ q,
    const char* __restrict__ k_pool, const char* __restrict__ v_pool,
    const int32_t* __restrict__ block_tables, int max_blocks,
    const int32_t* __restrict__ context_lens, const int32_t* __restrict__ query_start,
    const int32_t* __restrict__ work, int tiles_per_seq, int num_heads, int num_blocks,
    int max_len, float scale_log2) {
  using T = typename Ty::store_t;
  constexpr int KSTEPS = D / 32;             // k-steps of the score product
  constexpr int DTILES = D / 16;             // 16-row tiles of O^T
  constexpr int KROW = D + 8;                // halves per K row in LDS (16 bytes of padding)
  constexpr int COLS = D / 8;                // 16-byte column groups of a K/V row
  constexpr int LOADERS = (kMqChunk / 2) * COLS;
  constexpr size_t ROW_BYTES = D * sizeof(T);
  static_assert(sizeof(T) == 2, "16-bit storage only");
  static_assert(LOADERS <= kMqThreads, "one key pair per loader thread");
  static_assert(BS % 2 == 0, "a key pair never straddles two blocks");

  __shared__ __attribute__((aligned(16))) uint16_t ks[kMqChunk * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t vt[D * kMqChunk];

  // Head-fastest order: neighbouring workgroups read the same blocks' other heads.
  const int h = blockIdx.x % num_heads;
  const int j = blockIdx.x / num_heads;
  int s, tile;
  if (work) {
    const int item = work[j];
    s = item & kMqItemSeqMask;
    tile = item >> kMqItemSeqBits;
  } else {
    s = j / tiles_per_seq;
    tile = j % tiles_per_seq;
  }
  const int q0 = query_start[s];
  const int n = query_start[s + 1] - q0;
  const int first = tile * kMqTileQueries;
  if (first >= n) return;  // tile past this sequence's new tokens (uniform)
  const int nq = min(kMqTileQueries, n - first);
  const int L = min(context_lens[s], max_len);
  const size_t row_stride = static_cast<size_t>(num_heads) * D;
  const int tid = threadIdx.x;

  if (n > L) {  // the new tokens must be the last tokens of the context: NaN rows
    for (int e = tid; e < nq * D; e += kMqThreads)
      out[static_cast<size_t>(q0 + first + e / D) * row_stride + static_cast<size_t>(h) * D +
          e % D] = Ty::store(NAN);
    return;
  }

  const int wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, g = lane >> 4;
  const int qi = first + wave * 16 + r;          // this lane's query (may be past n)
  const int qc = min(qi, n - 1);                 // clamped: rows past n compute a copy
  const int qpos = L - n + qc;                   // last key the query sees
  const int wave_first = first + wave * 16;
  const bool wave_on = wave_first < n;
  const int wave_keys = L - n + min(wave_first + 16, n);  // keys any query of the wave sees
  const int tile_keys = L - n + first + nq;               // keys any query of the tile sees
  const int nchunks = (tile_keys + kMqChunk - 1) / kMqChunk;

  // The wave's q rows as B fragments: lane (r, g) holds q[r][32k + 8g .. 32k + 8g + 7].
  u32x4 qf[KSTEPS];
  {
    const T* qrow = q + static_cast<size_t>(q0 + qc) * row_stride + static_cast<size_t>(h) * D;
#pragma unroll
    for (int k = 0; k < KSTEPS; ++k) qf[k] = load16(qrow + 32 * k + 8 * g);
  }

  // Staging: loader thread (column group lc, pair lp) moves 16 bytes at column 8 lc of keys
  // 2 lp and 2 lp + 1 of each chunk; keys the tile does not see are staged as zeros, so NaN
  // in slots past the context never reaches a product.
  const bool loader = tid < LOADERS;
  const int lc = tid % COLS, lp = tid / COLS;
  const int32_t* table = block_tables + static_cast<size_t>(s) * max_blocks;
  const gptr_t kbase = uniform_ptr(k_pool);
  const gptr_t vbase = uniform_ptr(v_pool);
  u32x4 k0, k1, v0, v1;
  int bad = 0;
  auto fetch = [&](int c) {
    const u32x4 zero = {0u, 0u, 0u, 0u};
    k0 = k1 = v0 = v1 = zero;
    const int t = c * kMqChunk + 2 * lp;
    if (!loader || t >= tile_keys) return;
    const int blk = table[t / BS];
    if (blk < 0 || blk >= num_blocks) {  // never dereferenced; the outputs become NaN
      bad = 1;
      return;
    }
    const size_t off =
        ((static_cast<size_t>(blk) * num_heads + h) * BS + t % BS) * ROW_BYTES + lc * 16;
    k0 = load16<false>(kbase + off);
    v0 = load16<false>(vbase + off);
    if (t + 1 < tile_keys) {
      k1 = load16<false>(kbase + off + ROW_BYTES);
      v1 = load16<false>(vbase + off + ROW_BYTES);
    }
  };
  auto stage = [&]() {
    if (!loader) return;
    const int t = 2 * lp;
    *reinterpret_cast<u32x4*>(&ks[t * KROW + 8 * lc]) = k0;
    *reinterpret_cast<u32x4*>(&ks[(t + 1) * KROW + 8 * lc]) = k1;
    // key t -> V^T slot 8 grp + 4 half + i (t = 16 half + 4 grp + i); keys t, t+1 share a word
    const int half = t >> 4, grp = (t >> 2) & 3, i = t & 3;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = 8 * lc + e;
      const uint32_t w0 = v0[e >> 1], w1 = v1[e >> 1];
      const uint32_t pair = (e & 1) ? ((w0 >> 16) | (w1 & 0xFFFF0000u))
                                    : ((w0 & 0xFFFFu) | (w1 << 16));
      *reinterpret_cast<uint32_t*>(&vt[d * kMqChunk + 8 * vt_group(d, grp) + 4 * half + i]) =
          pair;
    }
  };

  f32x4 acc[DTILES];
#pragma unroll
  for (int t = 0; t < DTILES; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY;  // running max (log2 units) of query r, equal in its four lanes
  float lsum = 0.0f;    // this lane's share of the softmax denominator

  fetch(0);
  for (int c = 0; c < nchunks; ++c) {
    __syncthreads();  // every wave is done with the previous chunk
    stage();
    __syncthreads();
    if (c + 1 < nchunks) fetch(c + 1);  // in flight while this chunk is computed
    if (!wave_on || c * kMqChunk >= wave_keys) continue;

    f32x4 sc[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      sc[hh] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < KSTEPS; ++k) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(&ks[(16 * hh + r) * KROW + 32 * k + 8 * g]);
        sc[hh] = Mma<Ty>::run(a, qf[k], sc[hh]);
      }
    }
    float z[8];
    float cmax = -INFINITY;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = c * kMqChunk + 16 * hh + 4 * g + i;
        const float v = key <= qpos ? sc[hh][i] * scale_log2 : -INFINITY;
        z[4 * hh + i] = v;
        cmax = fmaxf(cmax, v);
      }
    cmax = fmaxf(cmax, __shfl_xor(cmax, 16, 64));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32, 64));
    const float mn = fmaxf(m, cmax);  // finite: chunk 0 holds key 0, which every query sees
    const float alpha = __builtin_amdgcn_exp2f(m - mn);
    float p[8], ps = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[e] = __builtin_amdgcn_exp2f(z[e] - mn);
      ps += p[e];
    }
    lsum = fmaf(lsum, alpha, ps);
    m = mn;
    uint32_t ph[4], pl[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) Mma<Ty>::pack(p[2 * w], p[2 * w + 1], ph[w], pl[w]);
    const u32x4 pf = {ph[0], ph[1], ph[2], ph[3]};
    const u32x4 pfl = {pl[0], pl[1], pl[2], pl[3]};
#pragma unroll
    for (int t = 0; t < DTILES; ++t) {
      const int d = 16 * t + r;
      const u32x4 a =
          *reinterpret_cast<const u32x4*>(&vt[d * kMqChunk + 8 * vt_group(d, g)]);
      acc[t] = Mma<Ty>::run(a, pf, acc[t] * alpha);
      if constexpr (Mma<Ty>::kSplit) acc[t] = Mma<Ty>::run(a, pfl, acc[t]);
    }
  }

  const int any_bad = __syncthreads_or(bad);
  if (!wave_on) return;
  float lt = lsum + __shfl_xor(lsum, 16, 64);
  lt += __shfl_xor(lt, 32, 64);
  if (qi >= n) return;
  const float inv = any_bad ? NAN : 1.0f / lt;
  T* orow = out + static_cast<size_t>(q0 + qi) * row_stride + static_cast<size_t>(h) * D;
#pragma unroll
  for (int t = 0; t < DTILES; ++t) {
    T o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = Ty::store(acc[t][i] * inv);
    uint2 w;
    __builtin_memcpy(&w, o, sizeof(w));
    *reinterpret_cast<uint2*>(orow + 16 * t + 4 * g) = w;
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
  int64_t wgs;
  int tiles_per_seq;
  int num_heads;
  int num_blocks;
  int max_len;
  float scale_log2;
  hipStream_t stream;
};

template <class Ty, int D, int BS>
static void launch_mq(const MqArgs& a) {
  using T = typename Ty::store_t;
  if (a.wgs <= 0) return;
  hipLaunchKernelGGL((multi_query_kernel<Ty, D, BS>), dim3(static_cast<unsigned>(a.wgs)),
                     dim3(kMqThreads), 0, a.stream, static_cast<T*>(a.out),
                     static_cast<const T*>(a.q), static_cast<const char*>(a.k_pool),
                     static_cast<const char*>(a.v_pool), a.block_tables, a.max_blocks,
                     a.context_lens, a.query_start, a.work, a.tiles_per_seq, a.num_heads,
                     a.num_blocks, a.max_len, a.scale_log2);
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

int32_t pkv_multi_query_schedule(const int32_t* query_start, const int32_t* context_lens,
                                 int32_t num_seqs, int32_t max_context_len, int32_t* items,
                                 int32_t capacity) {
  if (num_seqs < 0 || max_context_len < 0 || capacity < 0 || num_seqs > kMqItemSeqMask + 1 ||
      (num_seqs > 0 && (!query_start || !context_lens || !items)))
    return -1;
  struct Item {
    int64_t seq_keys;   // keys read by the sequence's largest tile
    int64_t keys;       // keys read by this tile
    int32_t s, tile;
  };
  std::vector<Item> list;
  for (int s = 0; s < num_seqs; ++s) {
    const int64_t n = static_cast<int64_t>(query_start[s + 1]) - query_start[s];
    if (n < 0) return -1;
    if (n == 0) continue;
    const int64_t tiles = (n + kMqTileQueries - 1) / kMqTileQueries;
    if (tiles > kMqMaxTiles) return -1;
    const int64_t L = std::min<int64_t>(context_lens[s], max_context_len);
    const int64_t base = std::max<int64_t>(L - n, 0);
    for (int64_t t = 0; t < tiles; ++t) {
      const int64_t keys = base + std::min<int64_t>(n, (t + 1) * kMqTileQueries);
      list.push_back({base + n, keys, s, static_cast<int32_t>(t)});
    }
  }
  if (static_cast<int64_t>(list.size()) > capacity) return -1;
  // Longest sequences first; a sequence's tiles stay adjacent (largest first) so that its
  // K/V, read by every tile, is shared in L2 while they run.
  std::stable_sort(list.begin(), list.end(), [](const Item& x, const Item& y) {
    if (x.seq_keys != y.seq_keys) return x.seq_keys > y.seq_keys;
    if (x.s != y.s) return x.s < y.s;
    return x.keys > y.keys;
  });
  for (size_t i = 0; i < list.size(); ++i)
    items[i] = list[i].s | (list[i].tile << kMqItemSeqBits);
  return static_cast<int32_t>(list.size());
}

pkv_status_t pkv_paged_attention_multi_query(
    const pkv_cache_desc_t* desc, void* out, const void* q, const void* k_pool,
    const void* v_pool, const int32_t* block_tables, int32_t max_blocks_per_seq,
    const int32_t* context_lens, const int32_t* query_start, int32_t num_seqs,
    int32_t max_query_len, int32_t max_context_len, float scale, const int32_t* work_items,
    int32_t num_items, pkv_stream_t stream) {
  pkv_status_t st = check_desc(desc);
  if (st != PKV_OK) return st;
  if (desc->dtype != PKV_F16 && desc->dtype != PKV_BF16) return PKV_EUNSUPPORTED;
  if (num_seqs < 0 || max_query_len < 0 || max_context_len < 0 || max_blocks_per_seq <= 0 ||
      !std::isfinite(scale))
    return PKV_EINVAL;
  if (num_seqs == 0 || max_query_len == 0) return PKV_OK;
  if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens || !query_start)
    return PKV_EINVAL;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool))
    return PKV_EINVAL;
  if (num_seqs > kMqItemSeqMask + 1) return PKV_EUNSUPPORTED;
  const int64_t tiles = (static_cast<int64_t>(max_query_len) + kMqTileQueries - 1) / kMqTileQueries;
  if (tiles > kMqMaxTiles) return PKV_EUNSUPPORTED;

  MqArgs a{};
  if (work_items) {
    if (num_items < 0 || num_items > static_cast<int64_t>(num_seqs) * tiles) return PKV_EINVAL;
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
  a.work = work_items;
  a.tiles_per_seq = static_cast<int>(tiles);
  a.num_heads = desc->num_heads;
  a.num_blocks = desc->num_blocks;
  a.max_len = static_cast<int>(std::min<int64_t>(
      max_context_len, static_cast<int64_t>(max_blocks_per_seq) * desc->block_size));
  a.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  a.stream = static_cast<hipStream_t>(stream);

  (void)hipGetLastError();  // clear a stale error so it is not blamed on this launch
  st = desc->dtype == PKV_F16 ? mq_dispatch_d<F16>(desc->head_dim, desc->block_size, a)
                              : mq_dispatch_d<BF16>(desc->head_dim, desc->block_size, a);
  if (st != PKV_OK) return st;
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_EHIP;
}

}  // extern "C"
