// C ABI of the MoE-layer hot path: argument validation on the host, workspace carving, launches.
// Every entry point validates before its first HIP call, allocates nothing and only enqueues work on
// the caller's stream.
#include <string.h>

#include <mutex>

#include "common.h"
#include "kernels.h"

namespace {

// Scratch of moe_dispatch_noalloc: one static device array per GPU (each device that loads the library
// holds its own copy). In host code `scratch` names a host-side stand-in, not device memory: kernels and
// copies are only ever given the device address that hipGetSymbolAddress returns for the current device.
__device__ __align__(256) unsigned char scratch[MOE_DISPATCH_NOALLOC_MAX_WORKSPACE];
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices] = {};

// The device address of `scratch` on the current device, looked up on the first call there.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MOE_ERR_HIP;
  if (dev >= kScratchDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

// Compute units of the current device (cached per device id; a benign race fills the same value).
int device_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64 && cache[dev] > 0) return cache[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  if (dev < 64) cache[dev] = n;
  return n;
}

// the split-K plan of the router is fixed for the target chip (256 CUs), so the workspace size is a
// function of the shape alone
constexpr int ROUTE_PLAN_CUS = 256;

bool valid_dtype(moe_dtype_t d) { return d == MOE_F32 || d == MOE_BF16; }

// the kernels move activations, weights and rows in 16-byte vectors and int / fp32 arrays in 4-byte words
// (a null pointer passes: the null checks come first)
bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool al4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int check_layout(const moe_layout_t* L) {
  if (!L) return MOE_ERR_INVALID;
  if (L->T < 0 || L->C < 0 || L->E < 1 || L->R < 1 || L->k < 1 || L->H < 1) return MOE_ERR_INVALID;
  if (L->E > MOE_MAX_EXPERTS || L->k > MOE_MAX_TOPK || L->k > L->E) return MOE_ERR_INVALID;
  if (L->E % L->R != 0) return MOE_ERR_INVALID;
  if (L->H % 8 != 0) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)L->T * L->k > (int64_t)INT32_MAX) return MOE_ERR_UNSUPPORTED;
  if (!L->expert_count || !L->expert_kept || !L->expert_overflow || !L->expert_offset) return MOE_ERR_INVALID;
  const int64_t rows = moe_rows_max(L->T, L->k, L->E, L->C);
  if (rows > 0 && (!L->row_token || !L->row_slot)) return MOE_ERR_INVALID;
  if (L->T > 0 && !L->pair_row) return MOE_ERR_INVALID;
  if (!al4(L->expert_count) || !al4(L->expert_kept) || !al4(L->expert_overflow) || !al4(L->expert_offset) ||
      !al4(L->row_token) || !al4(L->row_slot) || !al4(L->pair_row))
    return MOE_ERR_INVALID;
  return MOE_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case MOE_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

int64_t moe_rows_max(int T, int k, int E, int C) {
  if (T <= 0 || k <= 0 || E <= 0 || C <= 0) return 0;
  const int64_t a = (int64_t)T * k, b = (int64_t)E * C;
  return a < b ? a : b;
}

size_t moe_route_workspace_bytes(int T, int H, int E, moe_dtype_t xdt) {
  if (T <= 0 || H <= 0 || E <= 0 || !valid_dtype(xdt)) return 0;
  const moe::RoutePlan plan = moe::route_plan(T, H, E, xdt == MOE_BF16, ROUTE_PLAN_CUS);
  return plan.planes_bytes + plan.partial_bytes;
}

int moe_route(const void* x, moe_dtype_t xdt, const float* w_router, const float* logit_bias,
              int64_t bias_row_stride, int T, int H, int E, int k, float* logits, int32_t* topk_ids,
              float* topk_w, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!valid_dtype(xdt)) return MOE_ERR_UNSUPPORTED;
  if (T < 0 || H < 1 || E < 1 || E > MOE_MAX_EXPERTS || k < 1 || k > MOE_MAX_TOPK || k > E)
    return MOE_ERR_INVALID;
  if (H % 8 != 0) return MOE_ERR_UNSUPPORTED;
  if (logit_bias && bias_row_stride < 0) return MOE_ERR_INVALID;
  if ((int64_t)T * E > (int64_t)INT32_MAX) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !w_router || !logits || !topk_ids || !topk_w) return MOE_ERR_INVALID;
  if (!al16(x) || !al16(w_router) || !al16(workspace) || !al4(logit_bias) || !al4(logits) || !al4(topk_ids) ||
      !al4(topk_w))
    return MOE_ERR_INVALID;
  const size_t need = moe_route_workspace_bytes(T, H, E, xdt);
  if (need > 0 && (!workspace || workspace_bytes < need)) return MOE_ERR_INVALID;
  const moe::RoutePlan plan = moe::route_plan(T, H, E, xdt == MOE_BF16, ROUTE_PLAN_CUS);
  return hip_status(moe::launch_route(x, xdt == MOE_BF16, w_router, logit_bias, logit_bias ? bias_row_stride : 0,
                                      T, H, E, k, logits, topk_ids, topk_w, workspace, plan, stream));
}

size_t moe_dispatch_workspace_bytes(int T, int k, int E) {
  if (T < 0 || k < 0 || E < 0) return 0;
  const size_t nblk = (size_t)moe::dispatch_num_blocks(T);
  return moe::align256(nblk * (size_t)E * sizeof(int)) + moe::align256((size_t)T * k * sizeof(int));
}

int moe_dispatch(const void* x, moe_dtype_t xdt, const int32_t* topk_ids, const moe_layout_t* layout,
                 void* send_buf, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!valid_dtype(xdt)) return MOE_ERR_UNSUPPORTED;
  const int st = check_layout(layout);
  if (st != MOE_OK) return st;
  const moe_layout_t& L = *layout;
  const int64_t rows = moe_rows_max(L.T, L.k, L.E, L.C);
  if (L.T > 0 && (!x || !topk_ids)) return MOE_ERR_INVALID;
  if (rows > 0 && !send_buf) return MOE_ERR_INVALID;
  if (!al16(x) || !al16(send_buf) || !al16(workspace) || !al4(topk_ids)) return MOE_ERR_INVALID;
  const size_t need = moe_dispatch_workspace_bytes(L.T, L.k, L.E);
  if (need > 0 && (!workspace || workspace_bytes < need)) return MOE_ERR_INVALID;
  char* ws = static_cast<char*>(workspace);
  int* blk_count = reinterpret_cast<int*>(ws);
  int* pair_local =
      reinterpret_cast<int*>(ws + moe::align256((size_t)moe::dispatch_num_blocks(L.T) * L.E * sizeof(int)));
  return hip_status(moe::launch_dispatch(x, xdt == MOE_BF16, topk_ids, L, send_buf, blk_count, pair_local, stream));
}

int moe_dispatch_noalloc(const void* x, moe_dtype_t xdt, const int32_t* topk_ids, const moe_layout_t* layout,
                         void* send_buf, hipStream_t stream) {
  if (!valid_dtype(xdt)) return MOE_ERR_UNSUPPORTED;
  const int st = check_layout(layout);
  if (st != MOE_OK) return st;
  const moe_layout_t& L = *layout;
  const int64_t rows = moe_rows_max(L.T, L.k, L.E, L.C);
  if (L.T > 0 && (!x || !topk_ids)) return MOE_ERR_INVALID;
  if (rows > 0 && !send_buf) return MOE_ERR_INVALID;
  if (!al16(x) || !al16(send_buf) || !al4(topk_ids)) return MOE_ERR_INVALID;
  if (moe_dispatch_workspace_bytes(L.T, L.k, L.E) > MOE_DISPATCH_NOALLOC_MAX_WORKSPACE) return MOE_ERR_UNSUPPORTED;
  void* ws = nullptr;
  const int sst = scratch_address(&ws);
  if (sst != MOE_OK) return sst;
  // the same carving as moe_dispatch's workspace; the kernels write every entry they later read, so
  // the array's contents from an earlier call need no clearing
  char* base = static_cast<char*>(ws);
  int* blk_count = reinterpret_cast<int*>(base);
  int* pair_local =
      reinterpret_cast<int*>(base + moe::align256((size_t)moe::dispatch_num_blocks(L.T) * L.E * sizeof(int)));
  return hip_status(moe::launch_dispatch(x, xdt == MOE_BF16, topk_ids, L, send_buf, blk_count, pair_local, stream));
}

size_t moe_expert_mlp_workspace_bytes(int T, int k, int E, int R, int C, int F, moe_dtype_t xdt) {
  if (E <= 0 || R <= 0 || E % R != 0 || F <= 0) return 0;
  const int El = E / R;
  const int64_t rows = moe_rows_max(T, k, E, C);
  const size_t esz = xdt == MOE_BF16 ? 2 : 4;
  return moe::align256(moe::mlp_plan_ints(El) * sizeof(int)) + moe::align256((size_t)rows * sizeof(int)) +
         moe::align256((size_t)rows * (size_t)F * esz);
}

namespace {
// counters of the fused combine: one per (token, down-GEMM column band)
size_t combine_counter_bytes(int T, int k, int E, int R, int C, int H, int F, moe_dtype_t xdt) {
  const int64_t rows = moe_rows_max(T, k, E, C);
  const moe::MlpTiles tiles = moe::mlp_pick_tiles(rows, E / R, H, F, xdt == MOE_BF16);
  const int64_t bands = (H + moe::mlp_down_cols(tiles) - 1) / moe::mlp_down_cols(tiles);
  return moe::align256((size_t)((int64_t)T * bands) * sizeof(int));
}
}  // namespace

size_t moe_expert_mlp_combine_workspace_bytes(int T, int k, int E, int R, int C, int H, int F, moe_dtype_t xdt) {
  if (E <= 0 || R <= 0 || E % R != 0 || F <= 0 || H <= 0 || T < 0) return 0;
  return moe_expert_mlp_workspace_bytes(T, k, E, R, C, F, xdt) + combine_counter_bytes(T, k, E, R, C, H, F, xdt);
}

namespace {
// Shared by moe_expert_mlp, moe_expert_mlp_fp8 and moe_expert_mlp_combine: validation, workspace carving,
// launch. a_scale != nullptr means send_buf holds E4M3 codes with these block scales; y != nullptr fuses
// the combine into the down GEMM.
int expert_mlp(const void* send_buf, const float* a_scale, moe_dtype_t xdt, const moe_layout_t* layout,
               const void* w_gate_up, const void* w_down, int F, void* out_buf, void* workspace,
               size_t workspace_bytes, hipStream_t stream, const float* topk_w = nullptr, void* y = nullptr) {
  if (!valid_dtype(xdt)) return MOE_ERR_UNSUPPORTED;
  const int st = check_layout(layout);
  if (st != MOE_OK) return st;
  const moe_layout_t& L = *layout;
  if (F < 1) return MOE_ERR_INVALID;
  if (F % 8 != 0) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)2 * F > (int64_t)INT32_MAX / 2) return MOE_ERR_UNSUPPORTED;
  const int64_t rows = moe_rows_max(L.T, L.k, L.E, L.C);
  if (!w_gate_up || !w_down) return MOE_ERR_INVALID;
  if (rows > 0 && (!send_buf || !out_buf)) return MOE_ERR_INVALID;
  if (!al16(send_buf) || !al16(w_gate_up) || !al16(w_down) || !al16(out_buf) || !al16(workspace) || !al16(y) ||
      !al4(topk_w) || !al4(a_scale))
    return MOE_ERR_INVALID;
  const size_t need = y ? moe_expert_mlp_combine_workspace_bytes(L.T, L.k, L.E, L.R, L.C, L.H, F, xdt)
                        : moe_expert_mlp_workspace_bytes(L.T, L.k, L.E, L.R, L.C, F, xdt);
  if (!workspace || workspace_bytes < need) return MOE_ERR_INVALID;
  const int El = L.E / L.R;
  char* ws = static_cast<char*>(workspace);
  int* plan = reinterpret_cast<int*>(ws);
  ws += moe::align256(moe::mlp_plan_ints(El) * sizeof(int));
  int* perm = reinterpret_cast<int*>(ws);
  ws += moe::align256((size_t)rows * sizeof(int));
  void* hbuf = ws;
  ws += moe::align256((size_t)rows * (size_t)F * (xdt == MOE_BF16 ? 2 : 4));
  int* counter = y ? reinterpret_cast<int*>(ws) : nullptr;
  const moe::MlpTiles tiles = moe::mlp_pick_tiles(rows, El, L.H, F, xdt == MOE_BF16);
  return hip_status(moe::launch_expert_mlp(send_buf, xdt == MOE_BF16, L, w_gate_up, w_down, F, out_buf, plan, perm,
                                           hbuf, tiles, device_cus(), stream, a_scale, topk_w, y, counter));
}

}  // namespace

int moe_expert_mlp(const void* send_buf, moe_dtype_t xdt, const moe_layout_t* layout, const void* w_gate_up,
                   const void* w_down, int F, void* out_buf, void* workspace, size_t workspace_bytes,
                   hipStream_t stream) {
  return expert_mlp(send_buf, nullptr, xdt, layout, w_gate_up, w_down, F, out_buf, workspace, workspace_bytes,
                    stream);
}

int moe_expert_mlp_combine(const void* send_buf, moe_dtype_t xdt, const moe_layout_t* layout, const void* w_gate_up,
                           const void* w_down, int F, const float* topk_w, void* out_buf, void* y, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  const int st = check_layout(layout);
  if (st != MOE_OK) return st;
  if (layout->T > 0 && (!topk_w || !y)) return MOE_ERR_INVALID;
  if (layout->T == 0) {  // nothing to combine: the plain expert MLP (its plan kernel only)
    return expert_mlp(send_buf, nullptr, xdt, layout, w_gate_up, w_down, F, out_buf, workspace, workspace_bytes,
                      stream);
  }
  return expert_mlp(send_buf, nullptr, xdt, layout, w_gate_up, w_down, F, out_buf, workspace, workspace_bytes,
                    stream, topk_w, y);
}

int moe_dispatch_fp8(const void* x, moe_dtype_t xdt, const int32_t* topk_ids, const moe_layout_t* layout,
                     uint8_t* send_q, float* send_scale, void* workspace, size_t workspace_bytes,
                     hipStream_t stream) {
  if (xdt != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  const int st = check_layout(layout);
  if (st != MOE_OK) return st;
  const moe_layout_t& L = *layout;
  if (L.H % MOE_FP8_BLOCK != 0) return MOE_ERR_UNSUPPORTED;
  const int64_t rows = moe_rows_max(L.T, L.k, L.E, L.C);
  if (L.T > 0 && (!x || !topk_ids)) return MOE_ERR_INVALID;
  if (rows > 0 && (!send_q || !send_scale)) return MOE_ERR_INVALID;
  if (!al16(x) || !al16(send_q) || !al16(workspace) || !al4(send_scale) || !al4(topk_ids)) return MOE_ERR_INVALID;
  const size_t need = moe_dispatch_workspace_bytes(L.T, L.k, L.E);
  if (need > 0 && (!workspace || workspace_bytes < need)) return MOE_ERR_INVALID;
  char* ws = static_cast<char*>(workspace);
  int* blk_count = reinterpret_cast<int*>(ws);
  int* pair_local =
      reinterpret_cast<int*>(ws + moe::align256((size_t)moe::dispatch_num_blocks(L.T) * L.E * sizeof(int)));
  return hip_status(moe::launch_dispatch_fp8(x, topk_ids, L, send_q, send_scale, blk_count, pair_local, stream));
}

int moe_expert_mlp_fp8(const uint8_t* send_q, const float* send_scale, const moe_layout_t* layout,
                       const void* w_gate_up, const void* w_down, int F, void* out_buf, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  const int st = check_layout(layout);
  if (st != MOE_OK) return st;
  const moe_layout_t& L = *layout;
  if (L.H % MOE_FP8_BLOCK != 0) return MOE_ERR_UNSUPPORTED;
  const int64_t rows = moe_rows_max(L.T, L.k, L.E, L.C);
  if (rows > 0 && !send_scale) return MOE_ERR_INVALID;
  // with no rows there is nothing to decode: the bf16 path launches only the (empty) plan
  return expert_mlp(send_q, rows > 0 ? send_scale : nullptr, MOE_BF16, layout, w_gate_up, w_down, F, out_buf,
                    workspace, workspace_bytes, stream);
}

int moe_combine(const void* out_buf, moe_dtype_t xdt, const moe_layout_t* layout, const float* topk_w, void* y,
                hipStream_t stream) {
  if (!valid_dtype(xdt)) return MOE_ERR_UNSUPPORTED;
  const int st = check_layout(layout);
  if (st != MOE_OK) return st;
  const moe_layout_t& L = *layout;
  if (L.T == 0) return MOE_OK;
  const int64_t rows = moe_rows_max(L.T, L.k, L.E, L.C);
  if (!topk_w || !y) return MOE_ERR_INVALID;
  if (rows > 0 && !out_buf) return MOE_ERR_INVALID;
  if (!al16(out_buf) || !al16(y) || !al4(topk_w)) return MOE_ERR_INVALID;
  return hip_status(moe::launch_combine(out_buf, xdt == MOE_BF16, L, topk_w, y, stream));
}

int moe_combine_send(const void* out_buf, moe_dtype_t xdt, const moe_layout_t* layout, const float* topk_w,
                     void* partial, hipStream_t stream) {
  if (!valid_dtype(xdt)) return MOE_ERR_UNSUPPORTED;
  const int st = check_layout(layout);
  if (st != MOE_OK) return st;
  const moe_layout_t& L = *layout;
  if (L.T == 0) return MOE_OK;
  const int64_t rows = moe_rows_max(L.T, L.k, L.E, L.C);
  if (!topk_w || !partial) return MOE_ERR_INVALID;
  if (rows > 0 && !out_buf) return MOE_ERR_INVALID;
  if (!al16(out_buf) || !al16(partial) || !al4(topk_w)) return MOE_ERR_INVALID;
  return hip_status(moe::launch_combine_send(out_buf, xdt == MOE_BF16, L, topk_w, partial, stream));
}

int moe_combine_recv(const void* partial, moe_dtype_t xdt, const moe_layout_t* layout, void* y, hipStream_t stream) {
  if (!valid_dtype(xdt)) return MOE_ERR_UNSUPPORTED;
  const int st = check_layout(layout);
  if (st != MOE_OK) return st;
  const moe_layout_t& L = *layout;
  if (L.T == 0) return MOE_OK;
  if (!partial || !y) return MOE_ERR_INVALID;
  if (!al16(partial) || !al16(y)) return MOE_ERR_INVALID;
  return hip_status(moe::launch_combine_recv(partial, xdt == MOE_BF16, L, y, stream));
}

}  // extern "C"
