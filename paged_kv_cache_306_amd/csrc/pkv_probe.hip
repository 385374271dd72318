// Measurement probes for gfx950 (declared in pkv_probe.h): read bandwidth for a contiguous
// stream and for a visit of whole fixed-size tiles in a given order (the access pattern of a
// paged K/V gather); and the sustained rate of back-to-back 16x16x32 fp16 matrix products,
// alone, each fed by one 16-byte LDS read per lane, or interleaved with independent vector
// instructions.
// Measurement aids only; nothing on the paged-attention path calls them.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "pkv_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int kStreamUnroll = 8;        // 16-byte loads in flight per lane, contiguous read
constexpr int kTileLoadsInFlight = 16;  // 16-byte loads in flight per lane, tile visit
constexpr uint32_t kNever = 0x9E3779B9u;

template <bool NT>
__device__ __forceinline__ u32x4 load16(const u32x4* p) {
  if constexpr (NT)
    return __builtin_nontemporal_load(p);
  else
    return *p;
}

__device__ __forceinline__ uint32_t fold(u32x4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

// Contiguous read: workgroup b streams its own span of the buffer (the spans tile it in
// order), 256 threads x kStreamUnroll consecutive 16-byte vectors (32 KiB) per iteration.
template <bool NT>
__global__ __launch_bounds__(kThreads) void read_stream_kernel(const u32x4* __restrict__ p,
                                                               int64_t n16,
                                                               uint32_t* __restrict__ sink) {
  constexpr int64_t kStep = static_cast<int64_t>(kThreads) * kStreamUnroll;
  const int64_t steps = (n16 + kStep - 1) / kStep;
  const int64_t per_wg = (steps + gridDim.x - 1) / gridDim.x;
  const int64_t begin = static_cast<int64_t>(blockIdx.x) * per_wg * kStep;
  const int64_t end = begin + per_wg * kStep < n16 ? begin + per_wg * kStep : n16;
  uint32_t acc = 0;
  for (int64_t i = begin + threadIdx.x; i < end; i += kStep) {
    u32x4 v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) {
      const int64_t j = i + static_cast<int64_t>(u) * kThreads;
      v[u] = j < end ? load16<NT>(p + j) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) acc ^= fold(v[u]);
  }
  if (acc == kNever) sink[0] = acc;
}

// Whole tiles of VPL x 1 KiB (one wave-wide 16-byte load covers 1 KiB): wave w of the grid
// visits order[w], order[w + waves], ...; TILES of them are in flight at once, so every lane
// keeps kTileLoadsInFlight loads outstanding whatever the tile size.  split > 0 (of 1024):
// the waves of the even XCDs (workgroup b runs on XCD b % 8) visit the first
// num_tiles * split / 1024 entries of the order and those of the odd XCDs the rest, each half
// with its own waves -- the decode launches' weighting of the two halves.
template <bool NT, int VPL>
__global__ __launch_bounds__(kThreads) void read_tiles_kernel(const u32x4* __restrict__ p,
                                                              const int32_t* __restrict__ order,
                                                              int64_t num_tiles, int split,
                                                              uint32_t* __restrict__ sink) {
  constexpr int TILES = kTileLoadsInFlight / VPL;
  constexpr int kWavesPerGroup = kThreads / 64;
  const int lane = threadIdx.x & 63;
  int64_t wave = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) >> 6;
  int64_t waves = (static_cast<int64_t>(gridDim.x) * kThreads) >> 6;
  int64_t first = 0, last = num_tiles;
  if (split > 0) {
    const int x = static_cast<int>(blockIdx.x % 8);
    const int64_t even_tiles = num_tiles * split / 1024;
    first = (x & 1) ? even_tiles : 0;
    last = (x & 1) ? num_tiles : even_tiles;
    wave = ((static_cast<int64_t>(blockIdx.x / 8) * 4 + (x >> 1)) * kWavesPerGroup) +
           (threadIdx.x >> 6);
    waves = static_cast<int64_t>(gridDim.x / 2) * kWavesPerGroup;
  }
  uint32_t acc = 0;
  for (int64_t t0 = first + wave; t0 < last; t0 += TILES * waves) {
    u32x4 v[TILES][VPL];
#pragma unroll
    for (int k = 0; k < TILES; ++k) {
      const int64_t t = t0 + k * waves;
      const bool on = t < last;
      const int64_t base = static_cast<int64_t>(on ? order[t] : 0) * (64 * VPL) + lane;
#pragma unroll
      for (int u = 0; u < VPL; ++u)
        v[k][u] = on ? load16<NT>(p + base + 64 * u) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int k = 0; k < TILES; ++k)
#pragma unroll
      for (int u = 0; u < VPL; ++u) acc ^= fold(v[k][u]);
  }
  if (acc == kNever) sink[0] = acc;
}

template <bool NT>
hipError_t launch_tiles(const u32x4* p, const int32_t* order, int64_t num_tiles, int tile_bytes,
                        int split, uint32_t* sink, int wgs, hipStream_t s) {
  switch (tile_bytes) {
    case 2048:
      hipLaunchKernelGGL((read_tiles_kernel<NT, 2>), dim3(wgs), dim3(kThreads), 0, s, p, order,
                         num_tiles, split, sink);
      break;
    case 4096:
      hipLaunchKernelGGL((read_tiles_kernel<NT, 4>), dim3(wgs), dim3(kThreads), 0, s, p, order,
                         num_tiles, split, sink);
      break;
    default:
      hipLaunchKernelGGL((read_tiles_kernel<NT, 8>), dim3(wgs), dim3(kThreads), 0, s, p, order,
                         num_tiles, split, sink);
      break;
  }
  return hipGetLastError();
}

// Back-to-back v_mfma_f32_16x16x32_f16 on eight independent accumulators per wave.  LDS:
// each product's A operand is a 16-byte-per-lane LDS read (1 KiB per wave and product, the
// ratio of the multi-query kernel's K and V fragment reads); otherwise it stays in
// registers.  NV > 0: every product is followed by NV vector instructions (v_fma_f32, or a
// v_mul_f32 and a v_exp_f32 when EXP) on registers the products never read, which shows how
// much independent vector work the SIMD overlaps with its matrix products.
constexpr int kMfmaChains = 8;
constexpr int kMfmaLdsVectors = 2048;  // 32 KiB

template <bool LDS, int NV, bool EXP>
__global__ __launch_bounds__(kThreads) void mfma_rate_kernel(int iters, float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) u32x4 lds[LDS ? kMfmaLdsVectors : 1];
  const f16x8 a0 = {(_Float16)0.001f, (_Float16)0.002f, (_Float16)0.003f, (_Float16)0.001f,
                    (_Float16)0.002f, (_Float16)0.001f, (_Float16)0.003f, (_Float16)0.002f};
  if constexpr (LDS) {
    for (int i = threadIdx.x; i < kMfmaLdsVectors; i += kThreads) lds[i] = __builtin_bit_cast(u32x4, a0);
    __syncthreads();
  }
  const f16x8 b = a0 * static_cast<_Float16>(threadIdx.x & 3);
  f32x4 c[kMfmaChains];
  float v[kMfmaChains];
#pragma unroll
  for (int j = 0; j < kMfmaChains; ++j) {
    c[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    v[j] = 1.0f + 0.001f * static_cast<float>(threadIdx.x + j);
  }
  const uint32_t lane = threadIdx.x & 63;
  for (int it = 0; it < iters; ++it) {
    // eight consecutive 1 KiB rows (one per product), a different 8 KiB quarter each round
    const u32x4* row = &lds[LDS ? lane + 512 * (it & 3) : 0];
#pragma unroll
    for (int j = 0; j < kMfmaChains; ++j) {
      f16x8 a = a0;
      if constexpr (LDS) a = __builtin_bit_cast(f16x8, row[64 * j]);
      c[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c[j], 0, 0, 0);
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        float& x = v[(j + u) % kMfmaChains];
        if constexpr (EXP)
          x = __builtin_amdgcn_exp2f(x * -0.5f);
        else
          x = fmaf(x, 0.999f, 0.0001f);
      }
    }
  }
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < kMfmaChains; ++j) sum += c[j][0] + c[j][1] + c[j][2] + c[j][3] + v[j];
  out[static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x] = sum;
}

}  // namespace

extern "C" int32_t pkv_probe_read(const void* buf, int64_t bytes, int32_t tile_bytes,
                                  const int32_t* order, int64_t num_tiles, int32_t nontemporal,
                                  int32_t split, uint32_t* sink, int32_t workgroups,
                                  void* stream) {
  if (!buf || !sink || bytes <= 0 || bytes % 16 ||
      reinterpret_cast<uintptr_t>(buf) % 16 || workgroups < 1 || workgroups > 65536)
    return 1;
  if (split < 0 || split >= 1024 || (split > 0 && (tile_bytes == 0 || workgroups % 8)))
    return 1;
  if (tile_bytes != 0 && tile_bytes != 2048 && tile_bytes != 4096 && tile_bytes != 8192)
    return 1;
  if (tile_bytes != 0 && (!order || num_tiles <= 0 || num_tiles > bytes / tile_bytes))
    return 1;
  const u32x4* p = static_cast<const u32x4*>(buf);
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  hipError_t e;
  if (tile_bytes == 0) {
    if (nontemporal)
      hipLaunchKernelGGL(read_stream_kernel<true>, dim3(workgroups), dim3(kThreads), 0, s, p,
                         bytes / 16, sink);
    else
      hipLaunchKernelGGL(read_stream_kernel<false>, dim3(workgroups), dim3(kThreads), 0, s, p,
                         bytes / 16, sink);
    e = hipGetLastError();
  } else {
    e = nontemporal
            ? launch_tiles<true>(p, order, num_tiles, tile_bytes, split, sink, workgroups, s)
            : launch_tiles<false>(p, order, num_tiles, tile_bytes, split, sink, workgroups, s);
  }
  return e == hipSuccess ? 0 : 2;
}

extern "C" int32_t pkv_probe_mfma(int32_t mode, int32_t iters, int32_t workgroups, float* out,
                                  void* stream) {
  if (!out || iters < 1 || workgroups < 1 || workgroups > 65536 || mode < 0 || mode > 6) return 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 g(workgroups), blk(kThreads);
  (void)hipGetLastError();
  switch (mode) {
    case 0: hipLaunchKernelGGL((mfma_rate_kernel<false, 0, false>), g, blk, 0, s, iters, out); break;
    case 1: hipLaunchKernelGGL((mfma_rate_kernel<true, 0, false>), g, blk, 0, s, iters, out); break;
    case 2: hipLaunchKernelGGL((mfma_rate_kernel<false, 2, false>), g, blk, 0, s, iters, out); break;
    case 3: hipLaunchKernelGGL((mfma_rate_kernel<false, 4, false>), g, blk, 0, s, iters, out); break;
    case 4: hipLaunchKernelGGL((mfma_rate_kernel<false, 8, false>), g, blk, 0, s, iters, out); break;
    case 5: hipLaunchKernelGGL((mfma_rate_kernel<false, 1, true>), g, blk, 0, s, iters, out); break;
    default: hipLaunchKernelGGL((mfma_rate_kernel<false, 2, true>), g, blk, 0, s, iters, out); break;
  }
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
