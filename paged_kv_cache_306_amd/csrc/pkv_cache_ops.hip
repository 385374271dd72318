// Cache writes and block copies for the paged KV cache (gfx950).
//
// reshape_and_cache: a generated token's K and V rows go into the slot the block manager
// gave it ("PagedAttention: Efficient LLM Serving with vLLM", "The PagedAttention
// Algorithm", step 2).  copy_blocks: copy-on-write of a shared block in every layer (same
// page, "Advanced Features" -> "KV-Cache Sharing (Copy-on-Write)").  Both are pure 16-byte
// vector copies, so results are bit-exact; both are HBM-bound with no reuse.
#include "pkv.h"
#include "pkv_device.h"
#include "pkv_internal.h"

#include <algorithm>
#include <vector>

namespace pkv {

constexpr int kCopyThreads = 256;

// One thread per 16-byte piece of a (token, head) row; `row_vecs` pieces per row.
__global__ __launch_bounds__(kCopyThreads) void reshape_and_cache_kernel(
    const u32x4* __restrict__ k, const u32x4* __restrict__ v, u32x4* __restrict__ k_pool,
    u32x4* __restrict__ v_pool, const int32_t* __restrict__ slot_mapping, int64_t total_vecs,
    int row_vecs, int num_heads, int block_size, int64_t num_slots) {
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * kCopyThreads + threadIdx.x;
  if (gid >= total_vecs) return;
  const int64_t row = gid / row_vecs;           // token * num_heads + head
  const int c = static_cast<int>(gid - row * row_vecs);
  const int64_t tok = row / num_heads;
  const int h = static_cast<int>(row - tok * num_heads);
  const int32_t slot = slot_mapping[tok];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t blk = slot / block_size;
  const int off = slot - static_cast<int32_t>(blk) * block_size;
  const int64_t dst = ((blk * num_heads + h) * block_size + off) * row_vecs + c;
  k_pool[dst] = k[gid];
  v_pool[dst] = v[gid];
}

constexpr int kMaxLayersPerLaunch = 64;
constexpr int kVecsPerThread = 4;
constexpr int kVecsPerWG = kCopyThreads * kVecsPerThread;  // 16 KiB per workgroup

// Source and destination pools of up to kMaxLayersPerLaunch layers (the same pools for a
// copy-on-write copy, different ones for a swap between HBM and pinned host memory).
struct LayerPools {
  const u32x4* ks[kMaxLayersPerLaunch];
  const u32x4* vs[kMaxLayersPerLaunch];
  u32x4* kd[kMaxLayersPerLaunch];
  u32x4* vd[kMaxLayersPerLaunch];
};

// grid.x = pair * pieces_per_block + piece, grid.y = layer within this launch.
__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(
    LayerPools pools, const int32_t* __restrict__ pairs, int pieces_per_block, int64_t block_vecs,
    int src_blocks, int dst_blocks) {
  const int pair = blockIdx.x / pieces_per_block;
  const int piece = blockIdx.x - pair * pieces_per_block;
  const int src = pairs[2 * pair];
  const int dst = pairs[2 * pair + 1];
  if (static_cast<unsigned>(src) >= static_cast<unsigned>(src_blocks) ||
      static_cast<unsigned>(dst) >= static_cast<unsigned>(dst_blocks))
    return;
  const u32x4* ks = pools.ks[blockIdx.y] + src * block_vecs;
  const u32x4* vs = pools.vs[blockIdx.y] + src * block_vecs;
  u32x4* kd = pools.kd[blockIdx.y] + dst * block_vecs;
  u32x4* vd = pools.vd[blockIdx.y] + dst * block_vecs;
  const int64_t base = static_cast<int64_t>(piece) * kVecsPerWG + threadIdx.x;
  u32x4 kr[kVecsPerThread], vr[kVecsPerThread];
#pragma unroll
  for (int r = 0; r < kVecsPerThread; ++r) {
    const int64_t i = base + r * kCopyThreads;
    if (i < block_vecs) {
      kr[r] = ks[i];
      vr[r] = vs[i];
    }
  }
#pragma unroll
  for (int r = 0; r < kVecsPerThread; ++r) {
    const int64_t i = base + r * kCopyThreads;
    if (i < block_vecs) {
      kd[i] = kr[r];
      vd[i] = vr[r];
    }
  }
}

}  // namespace pkv

using namespace pkv;

extern "C" {

int32_t pkv_abi_version(void) { return PKV_ABI_VERSION; }

const char* pkv_status_string(pkv_status_t s) {
  switch (s) {
    case PKV_OK: return "ok";
    case PKV_EINVAL: return "invalid argument";
    case PKV_EUNSUPPORTED: return "unsupported shape or dtype";
    case PKV_ENOMEM: return "out of blocks or workspace too small";
    case PKV_EHIP: return "HIP runtime error";
  }
  return "unknown status";
}

pkv_status_t pkv_reshape_and_cache(const pkv_cache_desc_t* desc, const void* k, const void* v,
                                   void* k_pool, void* v_pool, const int32_t* slot_mapping,
                                   int32_t num_tokens, pkv_stream_t stream) {
  pkv_status_t st = check_desc(desc);
  if (st != PKV_OK) return st;
  if (num_tokens < 0) return PKV_EINVAL;
  if (num_tokens == 0) return PKV_OK;
  if (!k || !v || !k_pool || !v_pool || !slot_mapping) return PKV_EINVAL;
  for (const void* p : {k, v, static_cast<const void*>(k_pool), static_cast<const void*>(v_pool)})
    if (reinterpret_cast<uintptr_t>(p) % 16) return PKV_EINVAL;
  const int row_vecs = desc->head_dim * dtype_bytes(desc->dtype) / 16;
  const int64_t total = static_cast<int64_t>(num_tokens) * desc->num_heads * row_vecs;
  const int64_t wgs = (total + kCopyThreads - 1) / kCopyThreads;
  if (wgs > INT32_MAX) return PKV_EUNSUPPORTED;
  const int64_t num_slots = static_cast<int64_t>(desc->num_blocks) * desc->block_size;
  (void)hipGetLastError();
  hipLaunchKernelGGL(reshape_and_cache_kernel, dim3(static_cast<unsigned>(wgs)), dim3(kCopyThreads),
                     0, static_cast<hipStream_t>(stream), static_cast<const u32x4*>(k),
                     static_cast<const u32x4*>(v), static_cast<u32x4*>(k_pool),
                     static_cast<u32x4*>(v_pool), slot_mapping, total, row_vecs, desc->num_heads,
                     desc->block_size, num_slots);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_EHIP;
}

namespace {

// Launch copy_blocks_kernel over all layers, kMaxLayersPerLaunch at a time.
pkv_status_t launch_block_copies(const pkv_cache_desc_t* desc, const void* const* src_k,
                                 const void* const* src_v, void* const* dst_k, void* const* dst_v,
                                 int32_t num_layers, const int32_t* pairs, int32_t num_pairs,
                                 int32_t src_blocks, int32_t dst_blocks, hipStream_t stream) {
  const int64_t block_vecs = static_cast<int64_t>(desc->num_heads) * desc->block_size *
                             desc->head_dim * dtype_bytes(desc->dtype) / 16;
  const int64_t pieces = (block_vecs + kVecsPerWG - 1) / kVecsPerWG;
  if (pieces * num_pairs > INT32_MAX) return PKV_EUNSUPPORTED;
  (void)hipGetLastError();
  for (int32_t l0 = 0; l0 < num_layers; l0 += kMaxLayersPerLaunch) {
    const int n = std::min<int32_t>(kMaxLayersPerLaunch, num_layers - l0);
    LayerPools lp{};
    for (int i = 0; i < n; ++i) {
      lp.ks[i] = static_cast<const u32x4*>(src_k[l0 + i]);
      lp.vs[i] = static_cast<const u32x4*>(src_v[l0 + i]);
      lp.kd[i] = static_cast<u32x4*>(dst_k[l0 + i]);
      lp.vd[i] = static_cast<u32x4*>(dst_v[l0 + i]);
    }
    hipLaunchKernelGGL(copy_blocks_kernel, dim3(static_cast<unsigned>(pieces * num_pairs), n),
                       dim3(kCopyThreads), 0, stream, lp, pairs, static_cast<int>(pieces),
                       block_vecs, src_blocks, dst_blocks);
    if (hipGetLastError() != hipSuccess) return PKV_EHIP;
  }
  return PKV_OK;
}

bool aligned16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

// Address a kernel can use for `p`: device memory as is, pinned host memory through its device
// mapping; anything else (pageable host memory, unknown pointers) is refused.
bool device_address(const void* p, const void** out) {
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  if (attr.type == hipMemoryTypeDevice) {
    *out = p;
    return true;
  }
  if (attr.type == hipMemoryTypeHost && attr.devicePointer) {
    const char* base_h = static_cast<const char*>(attr.hostPointer);
    const char* base_d = static_cast<const char*>(attr.devicePointer);
    *out = base_h ? base_d + (static_cast<const char*>(p) - base_h) : base_d;
    return true;
  }
  return false;
}

}  // namespace

pkv_status_t pkv_copy_blocks(const pkv_cache_desc_t* desc, void* const* k_pools,
                             void* const* v_pools, int32_t num_layers, const int32_t* pairs,
                             int32_t num_pairs, pkv_stream_t stream) {
  pkv_status_t st = check_desc(desc);
  if (st != PKV_OK) return st;
  if (num_layers < 0 || num_pairs < 0) return PKV_EINVAL;
  if (num_layers == 0 || num_pairs == 0) return PKV_OK;
  if (!k_pools || !v_pools || !pairs) return PKV_EINVAL;
  for (int32_t l = 0; l < num_layers; ++l) {
    if (!k_pools[l] || !v_pools[l]) return PKV_EINVAL;
    if (!aligned16(k_pools[l]) || !aligned16(v_pools[l])) return PKV_EINVAL;
  }
  return launch_block_copies(desc, k_pools, v_pools, k_pools, v_pools, num_layers, pairs,
                             num_pairs, desc->num_blocks, desc->num_blocks,
                             static_cast<hipStream_t>(stream));
}

pkv_status_t pkv_swap_blocks(const pkv_cache_desc_t* src_desc, const pkv_cache_desc_t* dst_desc,
                             const void* const* src_k, const void* const* src_v,
                             void* const* dst_k, void* const* dst_v, int32_t num_layers,
                             const int32_t* pairs, int32_t num_pairs, pkv_stream_t stream) {
  pkv_status_t st = check_desc(src_desc);
  if (st != PKV_OK) return st;
  if ((st = check_desc(dst_desc)) != PKV_OK) return st;
  if (src_desc->num_heads != dst_desc->num_heads || src_desc->block_size != dst_desc->block_size ||
      src_desc->head_dim != dst_desc->head_dim || src_desc->dtype != dst_desc->dtype)
    return PKV_EINVAL;
  if (num_layers < 0 || num_pairs < 0) return PKV_EINVAL;
  if (num_layers == 0 || num_pairs == 0) return PKV_OK;
  if (!src_k || !src_v || !dst_k || !dst_v || !pairs) return PKV_EINVAL;
  std::vector<const void*> sk(num_layers), sv(num_layers);
  std::vector<void*> dk(num_layers), dv(num_layers);
  const void* pr = nullptr;
  if (!device_address(pairs, &pr)) return PKV_EINVAL;
  for (int32_t l = 0; l < num_layers; ++l) {
    const void* a[4];
    const void* in[4] = {src_k[l], src_v[l], dst_k[l], dst_v[l]};
    for (int i = 0; i < 4; ++i)
      if (!in[i] || !aligned16(in[i]) || !device_address(in[i], &a[i])) return PKV_EINVAL;
    sk[l] = a[0];
    sv[l] = a[1];
    dk[l] = const_cast<void*>(a[2]);
    dv[l] = const_cast<void*>(a[3]);
  }
  return launch_block_copies(src_desc, sk.data(), sv.data(), dk.data(), dv.data(), num_layers,
                             static_cast<const int32_t*>(pr), num_pairs, src_desc->num_blocks,
                             dst_desc->num_blocks, static_cast<hipStream_t>(stream));
}

}  // extern "C"
