// Device-side helpers shared by the gfx950 kernels: element types, vector types, 16-byte loads and
// stores, wave-level reductions, and the MFMA fragment helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16_t;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

#define MOE_WAVE 64

namespace moe {

// ------------------------------------------------------------------------------------------------
// element conversion
// ------------------------------------------------------------------------------------------------
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16_t v) { return (float)v; }

template <typename T>
__device__ __forceinline__ T from_f32(float v);
template <>
__device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) { return (bf16_t)v; }  // RNE (v_cvt_pk_bf16_f32)

// ------------------------------------------------------------------------------------------------
// 16-byte vectors: 8 bf16 or 4 fp32 per vector
// ------------------------------------------------------------------------------------------------
template <typename T>
struct Vec;
template <>
struct Vec<float> {
  static constexpr int N = 4;
};
template <>
struct Vec<bf16_t> {
  static constexpr int N = 8;
};

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ void st16_nt(void* p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ u32x4 ld16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// unpack a 16-byte vector into fp32 values
__device__ __forceinline__ void unpack(u32x4 v, float (&o)[4]) {
  o[0] = __uint_as_float(v.x);
  o[1] = __uint_as_float(v.y);
  o[2] = __uint_as_float(v.z);
  o[3] = __uint_as_float(v.w);
}
__device__ __forceinline__ void unpack(u32x4 v, float (&o)[8]) {
  // bf16 -> fp32 is a 16-bit left shift of the bit pattern
  o[0] = __uint_as_float(v.x << 16);
  o[1] = __uint_as_float(v.x & 0xffff0000u);
  o[2] = __uint_as_float(v.y << 16);
  o[3] = __uint_as_float(v.y & 0xffff0000u);
  o[4] = __uint_as_float(v.z << 16);
  o[5] = __uint_as_float(v.z & 0xffff0000u);
  o[6] = __uint_as_float(v.w << 16);
  o[7] = __uint_as_float(v.w & 0xffff0000u);
}

__device__ __forceinline__ u32x4 pack(const float (&o)[4]) {
  u32x4 v;
  v.x = __float_as_uint(o[0]);
  v.y = __float_as_uint(o[1]);
  v.z = __float_as_uint(o[2]);
  v.w = __float_as_uint(o[3]);
  return v;
}
__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
  bf16_t lo = (bf16_t)a, hi = (bf16_t)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
}
__device__ __forceinline__ u32x4 pack(const float (&o)[8]) {
  u32x4 v;
  v.x = pack2_bf16(o[0], o[1]);
  v.y = pack2_bf16(o[2], o[3]);
  v.z = pack2_bf16(o[4], o[5]);
  v.w = pack2_bf16(o[6], o[7]);
  return v;
}

// ------------------------------------------------------------------------------------------------
// wave helpers
// ------------------------------------------------------------------------------------------------
__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (MOE_WAVE - 1)); }
__device__ __forceinline__ uint64_t lanemask_lt() {
  const int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Workgroup barrier for LDS hand-offs only: waits for this wave's LDS operations, then s_barrier.
// __syncthreads() also fences global memory, which makes every wave wait for all of its global loads
// in flight (s_waitcnt vmcnt(0)) and so drains a software prefetch pipeline at each barrier. The
// "memory" clobber keeps the compiler from moving LDS accesses across the barrier.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

}  // namespace moe
