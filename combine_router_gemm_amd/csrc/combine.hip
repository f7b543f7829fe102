// Combine: y[t] = sum over kept slots j (ascending) of w[t, j] * out_buf[pair_row[t, j]].
//
// The combine reads each token's expert outputs from the per-expert buffers, takes the buffer and the
// weight of every expert from the routing table, and writes the weighted sum into caller-owned tensors
// ("Efficient and portable mixture-of-experts communication", section "Combine"). One wave per token:
// the k row indices and weights are read by k lanes and broadcast, then every lane accumulates its
// 16-byte column slices over the k rows in slot order in fp32 and rounds once to the output type.
// A token with every pair dropped writes zeros.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(const T* __restrict__ out_buf, const int* __restrict__ pair_row,
                                                     const float* __restrict__ topk_w, int T_, int H, int k,
                                                     T* __restrict__ y) {
  constexpr int VN = Vec<T>::N;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  if (t >= T_) return;
  int r = -1;
  float w = 0.f;
  if (lane < k) {
    r = pair_row[(int64_t)t * k + lane];
    w = topk_w[(int64_t)t * k + lane];
  }
  int rows[MOE_MAX_TOPK];
  float ws[MOE_MAX_TOPK];
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK; ++j) {
    rows[j] = __shfl(r, j, 64);
    ws[j] = __shfl(w, j, 64);
  }
  const int nvec = H / VN;
  T* dst = y + (int64_t)t * H;
  for (int v = lane; v < nvec; v += 64) {
    float acc[VN];
#pragma unroll
    for (int i = 0; i < VN; ++i) acc[i] = 0.f;
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) {
      if (j < k && rows[j] >= 0) {
        float val[VN];
        unpack(ld16(out_buf + (int64_t)rows[j] * H + (int64_t)v * VN), val);
#pragma unroll
        for (int i = 0; i < VN; ++i) acc[i] = fmaf(ws[j], val[i], acc[i]);
      }
    }
    st16(dst + (int64_t)v * VN, pack(acc));
  }
}

}  // namespace

hipError_t launch_combine(const void* out_buf, int xdt_bf16, const moe_layout_t& L, const float* topk_w, void* y,
                          hipStream_t stream) {
  const int blocks = ceil_div_host(L.T, 4);
  if (xdt_bf16)
    combine_kernel<bf16_t><<<blocks, 256, 0, stream>>>(static_cast<const bf16_t*>(out_buf), L.pair_row, topk_w, L.T,
                                                       L.H, L.k, static_cast<bf16_t*>(y));
  else
    combine_kernel<float><<<blocks, 256, 0, stream>>>(static_cast<const float*>(out_buf), L.pair_row, topk_w, L.T,
                                                      L.H, L.k, static_cast<float*>(y));
  return hipGetLastError();
}

}  // namespace moe
