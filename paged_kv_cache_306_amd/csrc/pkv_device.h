// Device helpers shared by the libpkv kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

// Reinterpret one 32-bit word as a pair of 16-bit floats.  The word is taken by value on
// purpose: clang's __builtin_bit_cast applied directly to an ext_vector element (v.y) reads
// the vector's first element instead, so every element goes through a plain copy first.
__device__ __forceinline__ f16x2 as_f16x2(uint32_t w) { return __builtin_bit_cast(f16x2, w); }
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t w) { return __builtin_bit_cast(bf16x2, w); }

// ------------------------------------------------------------------ element types
// Each storage type says how a lane's 16-byte slice of a q row and a K row make a partial
// dot product (fp32 accumulate), how a 16-byte slice of a V row is accumulated into fp32,
// and how an fp32 result is stored.
struct F32 {
  using store_t = float;
  static constexpr int kBytes = 4;
  static __device__ __forceinline__ float dot(u32x4 q, u32x4 k) {
    float a = __uint_as_float(q.x) * __uint_as_float(k.x);
    a = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), a);
    a = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), a);
    a = fmaf(__uint_as_float(q.w), __uint_as_float(k.w), a);
    return a;
  }
  static __device__ __forceinline__ void axpy(float* acc, float p, u32x4 v) {
    acc[0] = fmaf(p, __uint_as_float(v.x), acc[0]);
    acc[1] = fmaf(p, __uint_as_float(v.y), acc[1]);
    acc[2] = fmaf(p, __uint_as_float(v.z), acc[2]);
    acc[3] = fmaf(p, __uint_as_float(v.w), acc[3]);
  }
  static __device__ __forceinline__ float store(float x) { return x; }
};

struct F16 {
  using store_t = _Float16;
  static constexpr int kBytes = 2;
  static __device__ __forceinline__ float dot(u32x4 q, u32x4 k) {
    float a = __builtin_amdgcn_fdot2(as_f16x2(q.x), as_f16x2(k.x), 0.0f, false);
    a = __builtin_amdgcn_fdot2(as_f16x2(q.y), as_f16x2(k.y), a, false);
    a = __builtin_amdgcn_fdot2(as_f16x2(q.z), as_f16x2(k.z), a, false);
    a = __builtin_amdgcn_fdot2(as_f16x2(q.w), as_f16x2(k.w), a, false);
    return a;
  }
  static __device__ __forceinline__ void axpy2(float* acc, float p, uint32_t w) {
    f16x2 h = as_f16x2(w);
    acc[0] = fmaf(p, static_cast<float>(h.x), acc[0]);
    acc[1] = fmaf(p, static_cast<float>(h.y), acc[1]);
  }
  static __device__ __forceinline__ void axpy(float* acc, float p, u32x4 v) {
    axpy2(acc + 0, p, v.x);
    axpy2(acc + 2, p, v.y);
    axpy2(acc + 4, p, v.z);
    axpy2(acc + 6, p, v.w);
  }
  static __device__ __forceinline__ _Float16 store(float x) { return static_cast<_Float16>(x); }
};

struct BF16 {
  using store_t = uint16_t;
  static constexpr int kBytes = 2;
  static __device__ __forceinline__ float dot(u32x4 q, u32x4 k) {
    float a = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q.x), as_bf16x2(k.x), 0.0f, false);
    a = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q.y), as_bf16x2(k.y), a, false);
    a = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q.z), as_bf16x2(k.z), a, false);
    a = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q.w), as_bf16x2(k.w), a, false);
    return a;
  }
  static __device__ __forceinline__ void axpy2(float* acc, float p, uint32_t w) {
    // a bfloat16 is the upper half of a binary32
    acc[0] = fmaf(p, __uint_as_float(w << 16), acc[0]);
    acc[1] = fmaf(p, __uint_as_float(w & 0xFFFF0000u), acc[1]);
  }
  static __device__ __forceinline__ void axpy(float* acc, float p, u32x4 v) {
    axpy2(acc + 0, p, v.x);
    axpy2(acc + 2, p, v.y);
    axpy2(acc + 4, p, v.z);
    axpy2(acc + 6, p, v.w);
  }
  // binary32 -> bfloat16, round to nearest even; NaN stays a quiet NaN of the same sign.
  static __device__ __forceinline__ uint16_t store(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return static_cast<uint16_t>((u >> 16) | 0x0040u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
  }
};

// ------------------------------------------------------------------ lane reductions
// DPP controls (GCN/CDNA encoding).
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppRowMirror = 0x140;   // lane i of a 16-lane row reads lane 15-i
constexpr int kDppRowHalfMirror = 0x141;  // lane i of an 8-lane half-row reads lane 7-i

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over each aligned group of N lanes (N = 8, 16 or 32); every lane of the group receives
// the same bits (each step adds two commuted operands).
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 8 || N == 16 || N == 32, "group size");
  x += dpp<kDppQuadXor1>(x);
  x += dpp<kDppQuadXor2>(x);
  x += dpp<kDppRowHalfMirror>(x);
  if constexpr (N >= 16) x += dpp<kDppRowMirror>(x);
  if constexpr (N >= 32) x += __shfl_xor(x, 16, 64);
  return x;
}

typedef const __attribute__((address_space(1))) char* gptr_t;  // global memory

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// K/V tile loads.  NT: nontemporal (streaming) loads, for K/V that each sequence reads alone
// once per step; otherwise ordinary loads, so sequences that share blocks hit in L2.
template <bool NT>
__device__ __forceinline__ u32x4 load16(gptr_t p) {
  const __attribute__((address_space(1))) u32x4* v =
      reinterpret_cast<const __attribute__((address_space(1))) u32x4*>(p);
  if constexpr (NT)
    return __builtin_nontemporal_load(v);
  else
    return *v;
}

// A wave-uniform pointer passed through readfirstlane: the optimizer can no longer fold
// lane-varying offsets into it, so loads from `uniform_ptr(base) + lane_offset` keep the
// scalar-base + 32-bit vector-offset addressing form.
__device__ __forceinline__ gptr_t uniform_ptr(const char* p) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
  return reinterpret_cast<gptr_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

}  // namespace pkv
