// MFMA instruction traits shared by the GEMM kernels (gfx950).
#pragma once

#include "common.h"

namespace moe {

// MFMA instruction choices. Each op multiplies S x KS by KS x S fragments into an S x S fp32 tile.
// Lane l supplies 8 consecutive K of fragment row (l % S), starting at K = (l / S) * 8; A and B use
// the same K assignment, so any K order inside a step gives the same sum.
//   Op16: v_mfma_f32_16x16x32_bf16  (S = 16, KS = 32; output rows 4*(l/16) + q, q < 4)
//   Op32: v_mfma_f32_32x32x16_bf16  (S = 32, KS = 16; output rows 8*(q/4) + 4*(l/32) + q%4, q < 16)
//   OpF32: eight v_mfma_f32_16x16x4_f32 (S = 16, KS = 32); step q takes K = (l/16)*8 + q
// On MI355X the 32x32x16 bf16 form runs at twice the rate of the 16x16x32 form (measured 2.27 vs
// 1.2 PFLOP/s with independent chains), so compute-bound tiles use Op32.
struct Op16 {
  static constexpr int S = 16, KS = 32, VPF = 1, NR = 4;
  using Acc = f32x4;
  static __device__ __forceinline__ void step(Acc& acc, const u32x4 (&a)[1], const u32x4 (&b)[1]) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[0]), __builtin_bit_cast(bf16x8, b[0]),
                                                  acc, 0, 0, 0);
  }
  static __device__ __forceinline__ int out_row(int lane, int q) { return (lane >> 4) * 4 + q; }
};

struct Op32 {
  static constexpr int S = 32, KS = 16, VPF = 1, NR = 16;
  using Acc = f32x16;
  static __device__ __forceinline__ void step(Acc& acc, const u32x4 (&a)[1], const u32x4 (&b)[1]) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[0]), __builtin_bit_cast(bf16x8, b[0]),
                                                  acc, 0, 0, 0);
  }
  static __device__ __forceinline__ int out_row(int lane, int q) { return (q >> 2) * 8 + (lane >> 5) * 4 + (q & 3); }
};

struct OpF32 {
  static constexpr int S = 16, KS = 32, VPF = 2, NR = 4;
  using Acc = f32x4;
  static __device__ __forceinline__ void step(Acc& acc, const u32x4 (&a)[2], const u32x4 (&b)[2]) {
    float fa[8], fb[8];
    unpack(a[0], *reinterpret_cast<float(*)[4]>(&fa[0]));
    unpack(a[1], *reinterpret_cast<float(*)[4]>(&fa[4]));
    unpack(b[0], *reinterpret_cast<float(*)[4]>(&fb[0]));
    unpack(b[1], *reinterpret_cast<float(*)[4]>(&fb[4]));
#pragma unroll
    for (int q = 0; q < 8; ++q) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[q], fb[q], acc, 0, 0, 0);
  }
  static __device__ __forceinline__ int out_row(int lane, int q) { return (lane >> 4) * 4 + q; }
};

}  // namespace moe
