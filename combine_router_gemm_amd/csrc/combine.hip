// Combine: y[t] = sum over kept slots j (ascending) of w[t, j] * out_buf[pair_row[t, j]].
//
// The combine reads each token's expert outputs from the per-expert buffers, takes the buffer and the
// weight of every expert from the routing table, and writes the weighted sum into caller-owned tensors
// ("Efficient and portable mixture-of-experts communication", section "Combine"). Each thread owns a few
// 16-byte column slices of one token: it loads those slices of all k rows at once (independent loads,
// one memory round trip), accumulates them in slot order in fp32 and rounds once to the output type.
// A token with every pair dropped writes zeros.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

// grid: T * chunks workgroups of 256 threads; workgroup (t, c) owns the 16-byte column slices
// c*256*VPT + i*256 + tid (i < VPT) of token t, so all k*VPT loads of a thread are in flight at once.
template <typename T, int VPT>
__global__ __launch_bounds__(256) void combine_kernel(const T* __restrict__ out_buf, const int* __restrict__ pair_row,
                                                     const float* __restrict__ topk_w, int H, int k, int chunks,
                                                     T* __restrict__ y) {
  constexpr int VN = Vec<T>::N;
  __shared__ int s_row[MOE_MAX_TOPK];
  __shared__ float s_w[MOE_MAX_TOPK];
  const int t = blockIdx.x / chunks;
  const int v0 = (blockIdx.x % chunks) * 256 * VPT + threadIdx.x;
  if (threadIdx.x < k) {
    s_row[threadIdx.x] = pair_row[(int64_t)t * k + threadIdx.x];
    s_w[threadIdx.x] = topk_w[(int64_t)t * k + threadIdx.x];
  }
  __syncthreads();
  const int nvec = H / VN;
  u32x4 raw[VPT][MOE_MAX_TOPK];
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int v = v0 + i * 256;
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) {
      raw[i][j] = u32x4{0u, 0u, 0u, 0u};
      if (v < nvec && j < k && s_row[j] >= 0) {
        const T* src = out_buf + (int64_t)s_row[j] * H + (int64_t)v * VN;
        raw[i][j] = ld16_nt(src);  // each expert-output row is read once: streaming loads measured faster
      }
    }
  }
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int v = v0 + i * 256;
    if (v >= nvec) break;
    float acc[VN];
#pragma unroll
    for (int q = 0; q < VN; ++q) acc[q] = 0.f;
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) {
      if (j < k && s_row[j] >= 0) {  // slot order: ascending j
        float val[VN];
        unpack(raw[i][j], val);
#pragma unroll
        for (int q = 0; q < VN; ++q) acc[q] = fmaf(s_w[j], val[q], acc[q]);
      }
    }
    st16(y + (int64_t)t * H + (int64_t)v * VN, pack(acc));
  }
}

template <typename T, int VPT>
void launch_combine_t(const void* out_buf, const moe_layout_t& L, const float* topk_w, void* y, hipStream_t stream) {
  const int nvec = L.H / Vec<T>::N;
  const int chunks = ceil_div_host(nvec, 256 * VPT);
  const unsigned blocks = (unsigned)((int64_t)L.T * chunks);
  combine_kernel<T, VPT><<<blocks, 256, 0, stream>>>(static_cast<const T*>(out_buf), L.pair_row, topk_w, L.H, L.k,
                                                      chunks, static_cast<T*>(y));
}

// 16-byte slices per thread: enough loads in flight per thread without idling most of a long row
inline int slices_per_thread(int nvec) { return nvec >= 768 ? 4 : (nvec >= 384 ? 2 : 1); }

}  // namespace

hipError_t launch_combine(const void* out_buf, int xdt_bf16, const moe_layout_t& L, const float* topk_w, void* y,
                          hipStream_t stream) {
  const int vpt = slices_per_thread(L.H / (xdt_bf16 ? 8 : 4));
  if (xdt_bf16) {
    if (vpt == 4) launch_combine_t<bf16_t, 4>(out_buf, L, topk_w, y, stream);
    else if (vpt == 2) launch_combine_t<bf16_t, 2>(out_buf, L, topk_w, y, stream);
    else launch_combine_t<bf16_t, 1>(out_buf, L, topk_w, y, stream);
  } else {
    if (vpt == 4) launch_combine_t<float, 4>(out_buf, L, topk_w, y, stream);
    else if (vpt == 2) launch_combine_t<float, 2>(out_buf, L, topk_w, y, stream);
    else launch_combine_t<float, 1>(out_buf, L, topk_w, y, stream);
  }
  return hipGetLastError();
}

}  // namespace moe
