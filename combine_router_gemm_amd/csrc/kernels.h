// Host-side declarations of the kernel launchers (one translation unit per stage) used by the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

inline int ceil_div_host(int a, int b) { return (a + b - 1) / b; }
inline int64_t ceil_div_host64(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// ---- route ----
struct RouteTiles {
  int BM, BN;
  bool planes;  // the plane GEMM (router weight split once into three bf16 planes in the workspace)
};
RouteTiles route_tiles(int T, int H, int E, int xdt_bf16);
bool route_fused(int T, int E);  // one fused kernel, no workspace
// the launch plan: K splits, and the workspace: planes (planes_bytes, 256-aligned) then the fp32 partial
// sums (partial_bytes, only with several splits)
struct RoutePlan {
  RouteTiles tiles;
  int splits, k_split, nsplit;
  size_t planes_bytes, partial_bytes;
};
RoutePlan route_plan(int T, int H, int E, int xdt_bf16, int num_cus);
hipError_t launch_route(const void* x, int xdt_bf16, const float* w_router, const float* bias,
                        int64_t bias_stride, int T, int H, int E, int k, float* logits, int* ids, float* wts,
                        void* workspace, const RoutePlan& plan, hipStream_t stream);

// ---- dispatch ----
constexpr int DISPATCH_TB = 256;  // tokens per counting block
int dispatch_num_blocks(int T);
hipError_t launch_dispatch(const void* x, int xdt_bf16, const int* ids, const moe_layout_t& L, void* send_buf,
                           int* blk_count, int* pair_local, hipStream_t stream);
hipError_t launch_dispatch_fp8(const void* x, const int* ids, const moe_layout_t& L, uint8_t* send_q,
                               float* send_scale, int* blk_count, int* pair_local, hipStream_t stream);

// ---- expert MLP ----
struct MlpTiles {
  int BM;       // rows per tile (shared by both GEMMs; the plan is built for it)
  int variant;  // kernel family, see mlp.hip
};
MlpTiles mlp_pick_tiles(int64_t rows_max, int El, int H, int F, int xdt_bf16);
size_t mlp_plan_ints(int El);
// a_scale != nullptr: send_buf holds E4M3 codes with these block scales; they are expanded to bf16 in
// out_buf first and the bf16 GEMMs read them from there
// y != nullptr: the combine is fused into the down GEMM (y [T, H], counter [T, ceil(H / mlp_down_cols)])
hipError_t launch_expert_mlp(const void* send_buf, int xdt_bf16, const moe_layout_t& L, const void* w_gate_up,
                             const void* w_down, int F, void* out_buf, int* plan, int* perm, void* hbuf,
                             const MlpTiles& tiles, int num_cus, hipStream_t stream, const float* a_scale,
                             const float* topk_w = nullptr, void* y = nullptr, int* counter = nullptr);
// columns per down-GEMM tile (the band of the fused combine's counters)
int mlp_down_cols(const MlpTiles& tiles);
// whether the variant's GEMM kernels read the plan kernel's output (then it is always launched)
bool mlp_reads_plan(const MlpTiles& tiles);

// ---- combine ----
hipError_t launch_combine(const void* out_buf, int xdt_bf16, const moe_layout_t& L, const float* topk_w, void* y,
                          hipStream_t stream);
// sender-side partial accumulation: partial [R, T, H] rank-major
hipError_t launch_combine_send(const void* out_buf, int xdt_bf16, const moe_layout_t& L, const float* topk_w,
                               void* partial, hipStream_t stream);
hipError_t launch_combine_recv(const void* partial, int xdt_bf16, const moe_layout_t& L, void* y, hipStream_t stream);

}  // namespace moe
