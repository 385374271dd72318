// Paged decode attention for gfx950: one query per (sequence, head) attends over that
// sequence's K/V, which sit in fixed-size blocks scattered through a physical pool and are
// reached through the sequence's block table ("PagedAttention: Efficient LLM Serving with
// vLLM", "The PagedAttention Algorithm", steps 4-5).
//
// Work split.  A workgroup of 4 waves takes one (sequence, head, partition); a partition is
// a run of `part_tokens` consecutive tokens (the whole sequence in single-pass mode).  The
// partition is cut into chunks of CHUNK tokens (8 KiB of K and 8 KiB of V per chunk at
// fp16/bf16, head_dim 128) dealt round-robin to the 4 waves.
//
// Lane mapping.  A token's K row (head_dim elements) is read by LPT consecutive lanes, 16
// bytes each, so one wave-wide 16-byte load covers TPL = 64 / LPT whole token rows and a
// (block, head) tile of block_size rows -- contiguous in the pool -- is read by fully
// coalesced loads.  At fp16/bf16 head_dim 128: LPT = 16 lanes (one DPP row), TPL = 4.
// The q.K dot product is a per-lane 16-byte partial (v_dot2 for f16/bf16) summed over the
// LPT lanes with DPP.  Each 16-lane row then owns every TPL-th token of the chunk and keeps
// its own online-softmax state (running max m, running sum l, fp32 output slice), so the
// hot loop has no cross-row traffic; the 4 x TPL states are merged once per workgroup
// through LDS.  Scores are kept in log2 units (scale * log2 e folded into one multiply) so
// the exponentials are single v_exp_f32 instructions.
//
// Split-context mode.  Each partition writes (m, l, o = acc / l) to the workspace and a
// second kernel merges them: M = max m_p, out = sum_p 2^(m_p - M) l_p o_p / sum_p 2^(m_p - M) l_p.
// Sequences that fit in one partition are written out directly by the first kernel.
//
// Masking.  Only the last chunk of a partition can hold tokens at or past the end; their
// scores become -inf and their V rows are replaced by zero before the multiply (the slots
// may hold stale data or NaN, and NaN * 0 is NaN).  Blocks past the last valid one are never
// dereferenced: the block index is clamped to the last valid block.
#include "pkv.h"
#include "pkv_device.h"
#include "pkv_internal.h"
#include "pkv_xcd.h"

#include <hip/hip_ext.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <mutex>
#include <vector>

namespace pkv {

// Tuning constants, the values that measured best on MI355X: waves per workgroup (4: three
// workgroups per CU at 167 VGPRs), tokens per partition of a long sequence, the longest
// sequence attended in one pass, and K bytes per wave per chunk.
constexpr int kDecodeWaves = 4;
constexpr int kDecodeThreads = 64 * kDecodeWaves;
constexpr int kPartTokens = 2048;
constexpr int kSingleMax = 4096;
constexpr int kChunkBytesPerWave = 8192;
// s_getreg operand for HW_REG_XCC_ID (register 20), bits 3:0: the XCD a wave runs on.
constexpr int kHwRegXccId = 20 | (3 << 11);
// Longest run of tokens one workgroup attends: bounds the LDS copy of its block ids.
constexpr int kMaxPartTokens = 4096;
static_assert(kPartTokens <= kMaxPartTokens && kSingleMax <= kMaxPartTokens, "part");

template <class Ty, int D, int BS>
struct DecodeCfg {
  static constexpr int kEPL = 16 / Ty::kBytes;         // elements per lane per 16-byte load
  static constexpr int kLPT = D / kEPL;                // lanes per token row
  static constexpr int kTPL = 64 / kLPT;               // token rows per wave-wide load
  static constexpr int kChunkBytes = kChunkBytesPerWave;  // K bytes per wave per iteration
  static constexpr int kChunkByBytes = kChunkBytes / (D * Ty::kBytes);
  static constexpr int kChunk = kChunkByBytes > BS ? kChunkByBytes : BS;  // tokens
  static constexpr int kBlocksPerChunk = kChunk / BS;
  static constexpr int kLoads = kChunk / kTPL;         // 16-byte K loads per lane per chunk
  static constexpr int kStates = kDecodeWaves * kTPL;  // softmax states per workgroup
  static constexpr int kMaxBlocks = kMaxPartTokens / BS;
  static_assert(kLPT == 8 || kLPT == 16 || kLPT == 32, "row width");
  static_assert(BS % kTPL == 0, "a wave load must not straddle two blocks");
  static_assert(kChunk % BS == 0, "chunks hold whole blocks");
};

// A sequence of at most kSingleMax tokens is attended by one workgroup per head; a longer
// one is cut into partitions of part_tokens tokens whose partial results are merged.
__host__ __device__ __forceinline__ int partition_len(int L, int part_tokens) {
  return L <= kSingleMax ? (L > 0 ? L : 1) : part_tokens;
}
// Host-built work items: sequence index in the low 20 bits, partition index above.
constexpr int kItemPartShift = 20;
constexpr int kItemSeqMask = (1 << kItemPartShift) - 1;

// Clamp a device-provided length to what the launch was sized for.
__device__ __forceinline__ int effective_len(int L, int max_len) {
  return L < 0 ? 0 : (L > max_len ? max_len : L);
}

// One wave's online-softmax state: running max m (log2 units), running sum l, and the
// fp32 output slice of this lane (kEPL elements of the head).
template <class Ty, class C>
struct RowState {
  float m = -INFINITY, l = 0.0f;
  float acc[C::kEPL];
  __device__ RowState() {
#pragma unroll
    for (int e = 0; e < C::kEPL; ++e) acc[e] = 0.0f;
  }
  // Fold one chunk: kr/vr hold this lane's 16-byte slices of the chunk's K and V rows.
  template <bool MASKED>
  __device__ __forceinline__ void fold(const u32x4 qv, u32x4* kr, u32x4* vr, float scale_log2,
                                       int c0, int t1, int row) {
    float sc[C::kLoads];
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i)
      sc[i] = group_sum<C::kLPT>(Ty::dot(qv, kr[i])) * scale_log2;
    if constexpr (MASKED) {
#pragma unroll
      for (int i = 0; i < C::kLoads; ++i) {
        const bool valid = c0 + i * C::kTPL + row < t1;
        sc[i] = valid ? sc[i] : -INFINITY;
        vr[i] = valid ? vr[i] : u32x4{0u, 0u, 0u, 0u};
      }
    }
    float mx = m;
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i) mx = fmaxf(mx, sc[i]);
    const float ms = (mx == -INFINITY) ? 0.0f : mx;
    const float alpha = __builtin_amdgcn_exp2f(m - ms);
    l *= alpha;
#pragma unroll
    for (int e = 0; e < C::kEPL; ++e) acc[e] *= alpha;
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i) {
      const float pr = __builtin_amdgcn_exp2f(sc[i] - ms);
      l += pr;
      Ty::axpy(acc, pr, vr[i]);
    }
    m = mx;
  }
};

template <class Ty, int D, int BS, bool NT>
__global__ __launch_bounds__(kDecodeThreads) void decode_partition_kernel(
    typename Ty::store_t* __restrict__ out, const typename Ty::store_t* __restrict__ q,
    const typename Ty::store_t* __restrict__ k_pool, const typename Ty::store_t* __restrict__ v_pool,
    const int32_t* __restrict__ block_tables, int max_blocks, const int32_t* __restrict__ context_lens,
    int num_seqs, int num_heads, int num_blocks, int max_len, float scale_log2, int part_tokens,
    int max_parts, const int32_t* __restrict__ work, float* __restrict__ ws_ml,
    float* __restrict__ ws_o, int64_t units, int xcd_split, uint32_t* __restrict__ stamps) {
  using C = DecodeCfg<Ty, D, BS>;
  using T = typename Ty::store_t;
  __shared__ int sm_blk[C::kMaxBlocks];
  __shared__ float sm_m[C::kStates];
  __shared__ float sm_l[C::kStates];
  __shared__ __attribute__((aligned(16))) float sm_acc[C::kStates][D];

  // Unit b = (work item, head), head fastest: the workgroups of one (sequence, partition) run
  // side by side and read adjacent head tiles of the same blocks.  Workgroup slot blockIdx.x
  // runs unit blockIdx.x, or with xcd_split > 0 the unit that the XCD-weighted deal gives it
  // (see xcd_slot_unit).  Work item j is either listed by the host (sequence | partition <<
  // 20, longest first) or enumerated as (j / max_parts, j % max_parts).
  int64_t unit = blockIdx.x;
  if (xcd_split > 0) {
    unit = xcd_slot_unit(blockIdx.x, units, xcd_split);
    if (unit < 0) return;  // a slot past its half's share
  }
  const uint64_t stamp0 = stamps ? __builtin_amdgcn_s_memrealtime() : 0;
  const int h = static_cast<int>(unit % num_heads);
  const int j = static_cast<int>(unit / num_heads);
  int s, p;
  if (work) {
    const int item = work[j];
    s = item & kItemSeqMask;
    p = item >> kItemPartShift;
    if (s >= num_seqs || p >= max_parts) return;  // not an item of this call: touch nothing
  } else {
    s = j / max_parts;
    p = j % max_parts;
  }

  const int L = effective_len(context_lens[s], max_len);
  const int plen = partition_len(L, part_tokens);
  const int t0 = p * plen;
  if (p > 0 && t0 >= L) return;  // uniform across the workgroup
  const int t1 = min(L, t0 + plen);
  const int nparts = (L + plen - 1) / plen;

  // This workgroup's physical block ids, read once into LDS; an id outside the pool is
  // replaced by block 0 (in bounds) and poisons the output.
  const int lb0 = t0 / BS;
  const int nblk = (t1 - t0 + BS - 1) / BS;
  const int32_t* table = block_tables + static_cast<size_t>(s) * max_blocks + lb0;
  int bad = 0;
  for (int i = threadIdx.x; i < nblk; i += kDecodeThreads) {
    int pb = table[i];
    if (static_cast<unsigned>(pb) >= static_cast<unsigned>(num_blocks)) {
      bad = 1;
      pb = 0;
    }
    sm_blk[i] = pb;
  }

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = lane / C::kLPT;
  const int col = lane % C::kLPT;

  const size_t head_off = (static_cast<size_t>(s) * num_heads + h) * D;
  const u32x4 qv = load16(q + head_off + col * C::kEPL);

  const size_t blk_stride = static_cast<size_t>(num_heads) * BS * D;  // elements per block
  // Uniform (SGPR) base of head h in block 0, plus this lane's 32-bit byte offset inside a
  // (block, head) tile: loads then take the scalar-base + vector-offset form.
  const char* k_head = reinterpret_cast<const char*>(k_pool + static_cast<size_t>(h) * BS * D);
  const char* v_head = reinterpret_cast<const char*>(v_pool + static_cast<size_t>(h) * BS * D);
  const uint32_t lane_off = static_cast<uint32_t>((row * D + col * C::kEPL) * sizeof(T));

  const int any_bad_ids = __syncthreads_or(bad);

  // issue the 16-byte K and V loads of the chunk starting at token c0
  auto issue = [&](int c0, u32x4* kr, u32x4* vr) {
#pragma unroll
    for (int b = 0; b < C::kBlocksPerChunk; ++b) {
      const int j = min((c0 - t0) / BS + b, nblk - 1);
      const size_t boff =
          static_cast<size_t>(__builtin_amdgcn_readfirstlane(sm_blk[j])) * blk_stride * sizeof(T);
      const gptr_t kb = uniform_ptr(k_head + boff);
      const gptr_t vb = uniform_ptr(v_head + boff);
      constexpr int kPerBlock = BS / C::kTPL;  // wave loads per (block, head) tile
#pragma unroll
      for (int u = 0; u < kPerBlock; ++u) {
        const uint32_t off = lane_off + static_cast<uint32_t>(u * C::kTPL * D * sizeof(T));
        kr[b * kPerBlock + u] = load16<NT>(kb + off);
        vr[b * kPerBlock + u] = load16<NT>(vb + off);
      }
    }
    // keep every load of the chunk ahead of the arithmetic that consumes it
    __builtin_amdgcn_sched_barrier(0);
  };
  RowState<Ty, C> st;
  auto consume = [&](int c0, u32x4* kr, u32x4* vr) {
    if (c0 + C::kChunk > t1)
      st.template fold<true>(qv, kr, vr, scale_log2, c0, t1, row);
    else
      st.template fold<false>(qv, kr, vr, scale_log2, c0, t1, row);
  };
  constexpr int kStride = kDecodeWaves * C::kChunk;
  if (t1 > t0) {
    // Software pipeline over this wave's chunks c(k) = first + k * kStride, k < n: the loads
    // of chunk k+1 are in flight while chunk k is folded.  The loop body issues
    // unconditionally so the compiler waits only for the older chunk's loads.
    u32x4 ka[C::kLoads], va[C::kLoads], kb[C::kLoads], vb[C::kLoads];
    const int first = t0 + wave * C::kChunk;
    const int n = first < t1 ? (t1 - first + kStride - 1) / kStride : 0;
    if (n > 0) {
      issue(first, ka, va);
      int k = 0;
      for (; k + 2 < n; k += 2) {
        const int c = first + k * kStride;
        issue(c + kStride, kb, vb);
        consume(c, ka, va);
        issue(c + 2 * kStride, ka, va);
        consume(c + kStride, kb, vb);
      }
      const int c = first + k * kStride;
      if (k + 1 < n) {
        issue(c + kStride, kb, vb);
        consume(c, ka, va);
        consume(c + kStride, kb, vb);
      } else {
        consume(c, ka, va);
      }
    }
  }

  // ---- merge the kStates (wave, row) states of this workgroup
  const int stx = wave * C::kTPL + row;
  if (col == 0) {
    sm_m[stx] = st.m;
    sm_l[stx] = st.l;
  }
#pragma unroll
  for (int e = 0; e < C::kEPL; ++e) sm_acc[stx][col * C::kEPL + e] = st.acc[e];
  __syncthreads();

  const int d = threadIdx.x;
  if (d < D) {
    float M = -INFINITY;
#pragma unroll
    for (int j = 0; j < C::kStates; ++j) M = fmaxf(M, sm_m[j]);
    const float Ms = (M == -INFINITY) ? 0.0f : M;
    float num = 0.0f, den = 0.0f;
#pragma unroll
    for (int j = 0; j < C::kStates; ++j) {
      const float w = __builtin_amdgcn_exp2f(sm_m[j] - Ms);
      den = fmaf(w, sm_l[j], den);
      num = fmaf(w, sm_acc[j][d], num);
    }
    float o = den > 0.0f ? num / den : 0.0f;
    if (any_bad_ids) o = __builtin_nanf("");
    if (nparts <= 1) {
      out[head_off + d] = Ty::store(o);
    } else {
      const size_t slot = (static_cast<size_t>(s) * num_heads + h) * max_parts + p;
      ws_o[slot * D + d] = o;
      if (d == 0) {
        ws_ml[2 * slot] = M;
        ws_ml[2 * slot + 1] = den;
      }
    }
  }
  // Calibration stamps: the workgroup's time in 100 MHz ticks, the XCD it ran on (valid bit
  // 0x100), the tokens it attended and the low 32 bits of its start tick.
  if (stamps && threadIdx.x == 0) {
    const uint64_t stamp1 = __builtin_amdgcn_s_memrealtime();
    const uint32_t xcc = static_cast<uint32_t>(__builtin_amdgcn_s_getreg(kHwRegXccId)) & 15u;
    *reinterpret_cast<u32x4*>(stamps + 4 * static_cast<size_t>(blockIdx.x)) =
        u32x4{static_cast<uint32_t>(stamp1 - stamp0), xcc | 0x100u,
              static_cast<uint32_t>(t1 - t0), static_cast<uint32_t>(stamp0)};
  }
}

// Merge the partitions of every (sequence, head) that was split.  One workgroup of D
// threads per (sequence, head); thread d owns output element d.
template <class Ty, int D>
__global__ __launch_bounds__(D) void decode_reduce_kernel(
    typename Ty::store_t* __restrict__ out, const int32_t* __restrict__ context_lens, int num_heads,
    int max_len, int part_tokens, int max_parts, const float* __restrict__ ws_ml,
    const float* __restrict__ ws_o) {
  const int h = blockIdx.x % num_heads;
  const int s = blockIdx.x / num_heads;
  const int L = effective_len(context_lens[s], max_len);
  const int plen = partition_len(L, part_tokens);
  const int nparts = (L + plen - 1) / plen;
  if (nparts <= 1) return;  // written by the partition kernel
  const size_t base = (static_cast<size_t>(s) * num_heads + h) * max_parts;
  const int d = threadIdx.x;
  float M = -INFINITY;
  for (int p = 0; p < nparts; ++p) M = fmaxf(M, ws_ml[2 * (base + p)]);
  float num = 0.0f, den = 0.0f;
  for (int p = 0; p < nparts; ++p) {
    const float w = __builtin_amdgcn_exp2f(ws_ml[2 * (base + p)] - M) * ws_ml[2 * (base + p) + 1];
    den += w;
    num = fmaf(w, ws_o[(base + p) * D + d], num);
  }
  out[(static_cast<size_t>(s) * num_heads + h) * D + d] = Ty::store(num / den);
}

// ------------------------------------------------------------------ host side

static int effective_max_len(int32_t max_context_len, int32_t max_blocks, int32_t block_size) {
  const int64_t cap = static_cast<int64_t>(max_blocks) * block_size;
  return static_cast<int>(std::min<int64_t>(max_context_len, cap));
}

// 0 when every sequence fits one workgroup (max_len <= kSingleMax); otherwise the length of
// the partitions longer sequences are cut into.
static int partition_tokens(const pkv_cache_desc_t* d, int32_t num_seqs, int32_t max_len) {
  (void)d;
  (void)num_seqs;
  return max_len > kSingleMax ? kPartTokens : 0;
}

static int max_partitions(int max_len, int part) {
  return part > 0 ? (max_len + part - 1) / part : 1;
}

struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_tables;
  int max_blocks;
  const int32_t* context_lens;
  int num_seqs;
  int num_heads;
  int num_blocks;
  int max_len;
  float scale_log2;
  int part_tokens;
  int max_parts;
  const int32_t* work;  // device work items or null
  int num_items;
  bool shared_kv;       // ordinary (cache-allocating) loads instead of nontemporal ones
  float* ws_ml;
  float* ws_o;
  hipStream_t stream;
  hipEvent_t ev_start;  // optional: takes the start of the launch (hipExtLaunchKernel)
  hipEvent_t ev_stop;   // optional: takes its end (the reduce kernel's, in split mode)
  int xcd_split;        // 0: workgroup b runs unit b; else the XCD-weighted deal (1..1023)
  uint32_t* stamps;     // optional, with xcd_split 0: 4 words per workgroup (see the kernel)
};

template <class Ty, int D, int BS>
static void launch_decode(const DecodeArgs& a) {
  using T = typename Ty::store_t;
  const int64_t items =
      a.work ? a.num_items : static_cast<int64_t>(a.num_seqs) * a.max_parts;
  const int64_t units = items * a.num_heads;
  const int64_t wgs = a.xcd_split > 0 ? xcd_grid(units, a.xcd_split) : units;
  auto kernel = a.shared_kv ? decode_partition_kernel<Ty, D, BS, false>
                            : decode_partition_kernel<Ty, D, BS, true>;
  const bool reduce = a.part_tokens > 0;
  // Timing events ride on the launches themselves (the dispatch records its own start and end
  // time), so no event packet sits between kernels; with nothing launched they are recorded
  // on the stream instead.
  hipEvent_t start = a.ev_start, stop = a.ev_stop;
  if (wgs > 0) {
    hipEvent_t stop_here = reduce ? nullptr : stop;
    if (start || stop_here)
      hipExtLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(wgs)), dim3(kDecodeThreads), 0,
                            a.stream, start, stop_here, 0u, static_cast<T*>(a.out),
                            static_cast<const T*>(a.q), static_cast<const T*>(a.k_pool),
                            static_cast<const T*>(a.v_pool), a.block_tables, a.max_blocks,
                            a.context_lens, a.num_seqs, a.num_heads, a.num_blocks, a.max_len,
                            a.scale_log2, a.part_tokens, a.max_parts, a.work, a.ws_ml, a.ws_o,
                            units, a.xcd_split, a.stamps);
    else
      hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(wgs)), dim3(kDecodeThreads), 0,
                         a.stream, static_cast<T*>(a.out), static_cast<const T*>(a.q),
                         static_cast<const T*>(a.k_pool), static_cast<const T*>(a.v_pool),
                         a.block_tables, a.max_blocks, a.context_lens, a.num_seqs, a.num_heads,
                         a.num_blocks, a.max_len, a.scale_log2, a.part_tokens, a.max_parts,
                         a.work, a.ws_ml, a.ws_o, units, a.xcd_split, a.stamps);
    start = nullptr;
    if (!reduce) stop = nullptr;
  } else if (start) {
    (void)hipEventRecord(start, a.stream);
    start = nullptr;
  }
  if (reduce) {
    const int64_t units = static_cast<int64_t>(a.num_seqs) * a.num_heads;
    if (stop)
      hipExtLaunchKernelGGL((decode_reduce_kernel<Ty, D>), dim3(static_cast<unsigned>(units)),
                            dim3(D), 0, a.stream, nullptr, stop, 0u, static_cast<T*>(a.out),
                            a.context_lens, a.num_heads, a.max_len, a.part_tokens, a.max_parts,
                            a.ws_ml, a.ws_o);
    else
      hipLaunchKernelGGL((decode_reduce_kernel<Ty, D>), dim3(static_cast<unsigned>(units)),
                         dim3(D), 0, a.stream, static_cast<T*>(a.out), a.context_lens,
                         a.num_heads, a.max_len, a.part_tokens, a.max_parts, a.ws_ml, a.ws_o);
    stop = nullptr;
  }
  if (stop) (void)hipEventRecord(stop, a.stream);
}

template <class Ty, int D>
static pkv_status_t dispatch_bs(int bs, const DecodeArgs& a) {
  switch (bs) {
    case 8: launch_decode<Ty, D, 8>(a); return PKV_OK;
    case 16: launch_decode<Ty, D, 16>(a); return PKV_OK;
    case 32: launch_decode<Ty, D, 32>(a); return PKV_OK;
  }
  return PKV_EUNSUPPORTED;
}

template <class Ty>
static pkv_status_t dispatch_d(int dim, int bs, const DecodeArgs& a) {
  switch (dim) {
    case 64: return dispatch_bs<Ty, 64>(bs, a);
    case 128: return dispatch_bs<Ty, 128>(bs, a);
  }
  return PKV_EUNSUPPORTED;
}

static pkv_status_t decode_impl(const pkv_cache_desc_t* desc, void* out, const void* q,
                                const void* k_pool, const void* v_pool,
                                const int32_t* block_tables, int32_t max_blocks_per_seq,
                                const int32_t* context_lens, int32_t num_seqs,
                                int32_t max_context_len, float scale, const int32_t* work,
                                int32_t num_items, uint32_t flags, void* workspace,
                                size_t workspace_bytes, pkv_stream_t stream,
                                void* ev_start = nullptr, void* ev_stop = nullptr,
                                int32_t xcd_split = 0, uint32_t* stamps = nullptr) {
  pkv_status_t st = check_desc(desc);
  if (st != PKV_OK) return st;
  if (num_seqs < 0 || max_context_len < 0 || max_blocks_per_seq <= 0 || !std::isfinite(scale) ||
      (flags & ~static_cast<uint32_t>(PKV_DECODE_SHARED_KV)))
    return PKV_EINVAL;
  if (num_seqs == 0) return PKV_OK;
  if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens) return PKV_EINVAL;
  if (num_seqs > kItemSeqMask + 1) return PKV_EUNSUPPORTED;

  const int max_len = effective_max_len(max_context_len, max_blocks_per_seq, desc->block_size);
  const int part = partition_tokens(desc, num_seqs, max_len);
  const int max_parts = max_partitions(max_len, part);
  if (work) {
    if (num_items < 0 || static_cast<int64_t>(num_items) > static_cast<int64_t>(num_seqs) * max_parts)
      return PKV_EINVAL;
    if (static_cast<int64_t>(num_items) * desc->num_heads > INT32_MAX) return PKV_EUNSUPPORTED;
  } else if (static_cast<int64_t>(num_seqs) * desc->num_heads * max_parts > INT32_MAX) {
    return PKV_EUNSUPPORTED;
  }

  DecodeArgs a{};
  if (part > 0) {
    const size_t need = pkv_decode_workspace_bytes(desc, num_seqs, max_len);
    if (!workspace || workspace_bytes < need) return PKV_ENOMEM;
    if (reinterpret_cast<uintptr_t>(workspace) % 16) return PKV_EINVAL;
    const int64_t slots = static_cast<int64_t>(num_seqs) * desc->num_heads * max_parts;
    a.ws_ml = static_cast<float*>(workspace);
    a.ws_o = reinterpret_cast<float*>(static_cast<char*>(workspace) + align_up(slots * 8, 256));
  }
  a.out = out;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_tables = block_tables;
  a.max_blocks = max_blocks_per_seq;
  a.context_lens = context_lens;
  a.num_seqs = num_seqs;
  a.num_heads = desc->num_heads;
  a.num_blocks = desc->num_blocks;
  a.max_len = max_len;
  a.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  a.part_tokens = part;
  a.max_parts = max_parts;
  a.work = work;
  a.num_items = num_items;
  a.shared_kv = (flags & PKV_DECODE_SHARED_KV) != 0;
  a.stream = static_cast<hipStream_t>(stream);
  a.ev_start = static_cast<hipEvent_t>(ev_start);
  a.ev_stop = static_cast<hipEvent_t>(ev_stop);
  // the weighted deal needs a few more workgroup slots than units; past the grid limit the
  // units keep their own slots
  const int64_t units = static_cast<int64_t>(work ? num_items : static_cast<int64_t>(num_seqs) * max_parts) *
                        desc->num_heads;
  a.xcd_split = xcd_split > 0 && xcd_grid(units, xcd_split) <= INT32_MAX ? xcd_split : 0;
  a.stamps = stamps;

  (void)hipGetLastError();  // clear a stale error so it is not blamed on this launch
  switch (desc->dtype) {
    case PKV_F32: st = dispatch_d<F32>(desc->head_dim, desc->block_size, a); break;
    case PKV_F16: st = dispatch_d<F16>(desc->head_dim, desc->block_size, a); break;
    case PKV_BF16: st = dispatch_d<BF16>(desc->head_dim, desc->block_size, a); break;
    default: return PKV_EUNSUPPORTED;
  }
  if (st != PKV_OK) return st;
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_EHIP;
}

// Split-context scratch for callers that cannot allocate (pkv_paged_attention_decode_noalloc):
// one array per GPU, held until the process ends.  In host code `scratch` names a host-side
// stand-in, so its device address is looked up once per device (hipGetSymbolAddress, with
// that device current) and only that address is ever passed to a kernel.
static __device__ __align__(256) unsigned char scratch[PKV_DECODE_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices] = {};

// The XCD split the stand-alone decode calls deal their units with, per device (0: evenly):
// what a step driver on that device measured last, or what pkv_decode_set_xcd_split set.
static std::atomic<int32_t> g_device_split[kMaxDevices];

static int32_t current_device_split() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return dev >= 0 && dev < kMaxDevices ? g_device_split[dev].load(std::memory_order_relaxed) : 0;
}

void set_device_xcd_split(int32_t split) {
  int dev = -1;
  if (split < 0 || split >= kXcdSplitOne || hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return;
  }
  if (dev >= 0 && dev < kMaxDevices) g_device_split[dev].store(split, std::memory_order_relaxed);
}

static pkv_status_t scratch_for_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return PKV_EHIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return PKV_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return PKV_EHIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PKV_OK;
}

pkv_status_t decode_scheduled_timed(const pkv_cache_desc_t* desc, void* out, const void* q,
                                    const void* k_pool, const void* v_pool,
                                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                                    const int32_t* context_lens, int32_t num_seqs,
                                    int32_t max_context_len, float scale,
                                    const int32_t* work_items, int32_t num_items, uint32_t flags,
                                    void* workspace, size_t workspace_bytes, pkv_stream_t stream,
                                    void* ev_start, void* ev_stop, int32_t xcd_split,
                                    uint32_t* stamps) {
  if (!work_items || xcd_split < 0 || xcd_split >= kXcdSplitOne || (stamps && xcd_split != 0))
    return PKV_EINVAL;
  return decode_impl(desc, out, q, k_pool, v_pool, block_tables, max_blocks_per_seq, context_lens,
                     num_seqs, max_context_len, scale, work_items, num_items, flags, workspace,
                     workspace_bytes, stream, ev_start, ev_stop, xcd_split, stamps);
}

}  // namespace pkv

using namespace pkv;

extern "C" {

int32_t pkv_decode_partition_tokens(const pkv_cache_desc_t* desc, int32_t num_seqs,
                                    int32_t max_context_len) {
  if (!desc || num_seqs < 0 || max_context_len < 0) return 0;
  return partition_tokens(desc, num_seqs, max_context_len);
}

int32_t pkv_decode_single_pass_max(void) { return kSingleMax; }

pkv_status_t pkv_decode_set_xcd_split(int32_t split) {
  if (split < 0 || split >= kXcdSplitOne) return PKV_EINVAL;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return PKV_EHIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return PKV_EUNSUPPORTED;
  g_device_split[dev].store(split, std::memory_order_relaxed);
  return PKV_OK;
}

int32_t pkv_decode_xcd_split(void) { return current_device_split(); }

int64_t pkv_decode_xcd_grid(int64_t units, int32_t split) {
  if (units < 0 || split < 0 || split >= kXcdSplitOne) return -1;
  return split == 0 ? units : xcd_grid(units, split);
}

int64_t pkv_decode_xcd_slot_unit(int64_t slot, int64_t units, int32_t split) {
  if (units < 0 || split < 0 || split >= kXcdSplitOne || slot < 0 ||
      slot >= pkv_decode_xcd_grid(units, split))
    return -2;
  return split == 0 ? slot : xcd_slot_unit(slot, units, split);
}

size_t pkv_decode_workspace_bytes(const pkv_cache_desc_t* desc, int32_t num_seqs,
                                  int32_t max_context_len) {
  if (!desc || num_seqs <= 0 || max_context_len <= 0 || desc->head_dim <= 0 ||
      desc->num_heads <= 0)
    return 0;
  const int part = partition_tokens(desc, num_seqs, max_context_len);
  if (part == 0) return 0;
  const int64_t parts = max_partitions(max_context_len, part);
  const int64_t slots = static_cast<int64_t>(num_seqs) * desc->num_heads * parts;
  const int64_t ml = align_up(slots * 2 * 4, 256);
  return static_cast<size_t>(ml + slots * desc->head_dim * 4);
}

int32_t pkv_decode_schedule_grouped(const pkv_cache_desc_t* desc, const int32_t* lens,
                                    const int32_t* group_keys, int32_t num_seqs,
                                    int32_t max_context_len, int32_t* items, int32_t capacity) {
  if (!desc || num_seqs < 0 || max_context_len < 0 || capacity < 0 ||
      (num_seqs > 0 && (!lens || !items)) || num_seqs > kItemSeqMask + 1)
    return -1;
  const int part = partition_tokens(desc, num_seqs, max_context_len);
  struct Item {
    int32_t tokens;  // tokens this item attends
    int32_t rank;    // group's largest item (keys given) or the item's own tokens
    int32_t key;     // first sequence of its group
    int32_t p;       // partition
    int32_t code;    // s | p << kItemPartShift
  };
  // group leader = first sequence with the same key (sequences sharing prefix blocks)
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
  list.reserve(static_cast<size_t>(num_seqs));
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int L = lens[s] < 0 ? 0 : std::min(lens[s], max_context_len);
    const int plen = partition_len(L, part);
    const int n = (L + plen - 1) / plen;
    if (n == 0) {
      list.push_back({0, 0, leader[s], 0, s});  // length 0: one workgroup writes zeros
      continue;
    }
    if (n - 1 > (INT32_MAX >> kItemPartShift)) return -1;
    for (int p = 0; p < n; ++p)
      list.push_back({std::min(plen, L - p * plen), 0, leader[s], p, s | (p << kItemPartShift)});
  }
  if (static_cast<int64_t>(list.size()) > capacity) return -1;
  if (group_keys) {
    std::vector<int32_t> best(static_cast<size_t>(num_seqs), 0);
    for (const Item& it : list) best[it.key] = std::max(best[it.key], it.tokens);
    for (Item& it : list) it.rank = best[it.key];
  } else {
    for (Item& it : list) it.rank = it.tokens;
  }
  // longest groups (or items) first; inside a group, partition by partition so the members
  // read their shared blocks together
  std::stable_sort(list.begin(), list.end(), [](const Item& x, const Item& y) {
    if (x.rank != y.rank) return x.rank > y.rank;
    if (x.key != y.key) return x.key < y.key;
    return x.p < y.p;
  });
  for (size_t i = 0; i < list.size(); ++i) items[i] = list[i].code;
  return static_cast<int32_t>(list.size());
}

int32_t pkv_decode_schedule(const pkv_cache_desc_t* desc, const int32_t* lens, int32_t num_seqs,
                            int32_t max_context_len, int32_t* items, int32_t capacity) {
  return pkv_decode_schedule_grouped(desc, lens, nullptr, num_seqs, max_context_len, items,
                                     capacity);
}

pkv_status_t pkv_paged_attention_decode(const pkv_cache_desc_t* desc, void* out, const void* q,
                                        const void* k_pool, const void* v_pool,
                                        const int32_t* block_tables, int32_t max_blocks_per_seq,
                                        const int32_t* context_lens, int32_t num_seqs,
                                        int32_t max_context_len, float scale, void* workspace,
                                        size_t workspace_bytes, pkv_stream_t stream) {
  return decode_impl(desc, out, q, k_pool, v_pool, block_tables, max_blocks_per_seq, context_lens,
                     num_seqs, max_context_len, scale, nullptr, 0, 0u, workspace, workspace_bytes,
                     stream, nullptr, nullptr, current_device_split());
}

pkv_status_t pkv_paged_attention_decode_scheduled(
    const pkv_cache_desc_t* desc, void* out, const void* q, const void* k_pool,
    const void* v_pool, const int32_t* block_tables, int32_t max_blocks_per_seq,
    const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len, float scale,
    const int32_t* work_items, int32_t num_items, uint32_t flags, void* workspace,
    size_t workspace_bytes, pkv_stream_t stream) {
  if (!work_items) return PKV_EINVAL;
  return decode_impl(desc, out, q, k_pool, v_pool, block_tables, max_blocks_per_seq, context_lens,
                     num_seqs, max_context_len, scale, work_items, num_items, flags, workspace,
                     workspace_bytes, stream, nullptr, nullptr, current_device_split());
}

pkv_status_t pkv_paged_attention_decode_noalloc(const pkv_cache_desc_t* desc, void* out,
                                                const void* q, const void* k_pool,
                                                const void* v_pool, const int32_t* block_tables,
                                                int32_t max_blocks_per_seq,
                                                const int32_t* context_lens, int32_t num_seqs,
                                                int32_t max_context_len, float scale,
                                                pkv_stream_t stream) {
  pkv_status_t st = check_desc(desc);
  if (st != PKV_OK) return st;
  if (num_seqs < 0 || max_context_len < 0 || max_blocks_per_seq <= 0) return PKV_EINVAL;
  // the partials this call needs, from the same bound the launch is sized with; rejected
  // before any device call when they exceed the array
  const int max_len = effective_max_len(max_context_len, max_blocks_per_seq, desc->block_size);
  const size_t need = num_seqs > 0 ? pkv_decode_workspace_bytes(desc, num_seqs, max_len) : 0;
  if (need > static_cast<size_t>(PKV_DECODE_NOALLOC_SCRATCH_BYTES)) return PKV_ENOMEM;
  void* ws = nullptr;
  if (need > 0) {
    st = scratch_for_current_device(&ws);
    if (st != PKV_OK) return st;
  }
  return decode_impl(desc, out, q, k_pool, v_pool, block_tables, max_blocks_per_seq, context_lens,
                     num_seqs, max_context_len, scale, nullptr, 0, 0u, ws,
                     ws ? static_cast<size_t>(PKV_DECODE_NOALLOC_SCRATCH_BYTES) : 0, stream,
                     nullptr, nullptr, current_device_split());
}

}  // extern "C"
