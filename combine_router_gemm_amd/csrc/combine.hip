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
  if ((int)threadIdx.x < k) {
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
    // y is not read again in the layer: non-temporal stores (16384 tokens x 7168 from 67528 rows:
    // 238 -> 234 us; 4096 x 7168 from 32768 rows: 89.5 -> 86.1 us)
    st16_nt(y + (int64_t)t * H + (int64_t)v * VN, pack(acc));
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

// ---- combine with sender-side partial accumulation ----
// The expert side sums, per token and per destination rank, the weighted rows it holds, so one row per
// (rank, token) crosses the link instead of one per kept pair; the token's side then sums the partial
// rows ("Enabling trillion-parameter models on AWS EFA", section "Оценка": DeepEP accumulates at the
// sender to move fewer bytes, at a cost in precision). Partial rows are rank-major, [R, T, H].

// Rank of row p: the r with offset[r * El] <= p < offset[(r + 1) * El] (last such r when ranks are empty).
__device__ __forceinline__ int row_rank(int p, const int* __restrict__ offset, int El, int R) {
  int lo = 0, hi = R;  // invariant: offset[lo * El] <= p < offset[hi * El]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offset[mid * El] <= p) lo = mid;
    else hi = mid;
  }
  return lo;
}

// grid as combine_kernel. For every rank r holding kept slots of token t: partial[r, t] = sum over those
// slots (ascending) of w * row, fp32, rounded once. Slot j "leads" rank r when it is r's first kept slot;
// s_members[j] is the bit set of r's kept slots.
template <typename T, int VPT>
__global__ __launch_bounds__(256) void combine_send_kernel(const T* __restrict__ out_buf, const int* __restrict__ pair_row,
                                                          const float* __restrict__ topk_w,
                                                          const int* __restrict__ offset, int T_, int H, int k, int El,
                                                          int R, int chunks, T* __restrict__ partial) {
  constexpr int VN = Vec<T>::N;
  __shared__ int s_row[MOE_MAX_TOPK];
  __shared__ int s_rank[MOE_MAX_TOPK];
  __shared__ float s_w[MOE_MAX_TOPK];
  __shared__ unsigned s_members[MOE_MAX_TOPK];
  const int t = blockIdx.x / chunks;
  const int v0 = (blockIdx.x % chunks) * 256 * VPT + threadIdx.x;
  if ((int)threadIdx.x < k) {
    const int row = pair_row[(int64_t)t * k + threadIdx.x];
    s_row[threadIdx.x] = row;
    s_w[threadIdx.x] = topk_w[(int64_t)t * k + threadIdx.x];
    s_rank[threadIdx.x] = row >= 0 ? row_rank(row, offset, El, R) : -1;
  }
  __syncthreads();
  if ((int)threadIdx.x < k) {
    const int j = threadIdx.x, r = s_rank[j];
    unsigned m = 0;
    bool lead = r >= 0;
    for (int i = 0; i < k; ++i) {
      if (s_rank[i] == r) {
        if (i < j) lead = false;
        m |= 1u << i;
      }
    }
    s_members[j] = lead ? m : 0u;
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
      if (v < nvec && j < k && s_row[j] >= 0) raw[i][j] = ld16_nt(out_buf + (int64_t)s_row[j] * H + (int64_t)v * VN);
    }
  }
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK; ++j) {
    const unsigned m = j < k ? s_members[j] : 0u;
    if (m == 0) continue;
    T* dst = partial + ((int64_t)s_rank[j] * T_ + t) * H;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int v = v0 + i * 256;
      if (v >= nvec) break;
      float acc[VN];
#pragma unroll
      for (int q = 0; q < VN; ++q) acc[q] = 0.f;
#pragma unroll
      for (int s = 0; s < MOE_MAX_TOPK; ++s) {
        if ((m >> s) & 1u) {  // ascending slots of this rank
          float val[VN];
          unpack(raw[i][s], val);
#pragma unroll
          for (int q = 0; q < VN; ++q) acc[q] = fmaf(s_w[s], val[q], acc[q]);
        }
      }
      st16(dst + (int64_t)v * VN, pack(acc));
    }
  }
}

// grid as combine_kernel. y[t] = sum over the ranks holding kept slots of t (ascending) of partial[r, t],
// fp32, rounded once; a token with no kept slot gets 0.
template <typename T, int VPT>
__global__ __launch_bounds__(256) void combine_recv_kernel(const T* __restrict__ partial, const int* __restrict__ pair_row,
                                                          const int* __restrict__ offset, int T_, int H, int k, int El,
                                                          int R, int chunks, T* __restrict__ y) {
  constexpr int VN = Vec<T>::N;
  __shared__ int s_rank[MOE_MAX_TOPK];
  __shared__ int s_nr;
  const int t = blockIdx.x / chunks;
  const int v0 = (blockIdx.x % chunks) * 256 * VPT + threadIdx.x;
  if ((int)threadIdx.x < k) {
    const int row = pair_row[(int64_t)t * k + threadIdx.x];
    s_rank[threadIdx.x] = row >= 0 ? row_rank(row, offset, El, R) : -1;
  }
  __syncthreads();
  if (threadIdx.x == 0) {  // the distinct ranks, ascending (k <= MOE_MAX_TOPK: insertion sort)
    int d[MOE_MAX_TOPK];
    int n = 0;
    for (int j = 0; j < k; ++j) {
      const int r = s_rank[j];
      bool dup = r < 0;
      for (int i = 0; i < n; ++i) dup = dup || d[i] == r;
      if (dup) continue;
      int p = n++;
      while (p > 0 && d[p - 1] > r) {
        d[p] = d[p - 1];
        --p;
      }
      d[p] = r;
    }
    for (int i = 0; i < n; ++i) s_rank[i] = d[i];
    s_nr = n;
  }
  __syncthreads();
  const int nr = s_nr;
  const int nvec = H / VN;
  u32x4 raw[VPT][MOE_MAX_TOPK];
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int v = v0 + i * 256;
#pragma unroll
    for (int m = 0; m < MOE_MAX_TOPK; ++m) {
      raw[i][m] = u32x4{0u, 0u, 0u, 0u};
      if (v < nvec && m < nr) raw[i][m] = ld16_nt(partial + ((int64_t)s_rank[m] * T_ + t) * H + (int64_t)v * VN);
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
    for (int m = 0; m < MOE_MAX_TOPK; ++m) {
      if (m < nr) {
        float val[VN];
        unpack(raw[i][m], val);
#pragma unroll
        for (int q = 0; q < VN; ++q) acc[q] += val[q];
      }
    }
    st16(y + (int64_t)t * H + (int64_t)v * VN, pack(acc));
  }
}

template <typename T, int VPT>
void launch_combine_sr_t(bool send, const void* src, const moe_layout_t& L, const float* topk_w, void* dst,
                         hipStream_t stream) {
  const int nvec = L.H / Vec<T>::N;
  const int chunks = ceil_div_host(nvec, 256 * VPT);
  const unsigned blocks = (unsigned)((int64_t)L.T * chunks);
  const int El = L.E / L.R;
  if (send)
    combine_send_kernel<T, VPT><<<blocks, 256, 0, stream>>>(static_cast<const T*>(src), L.pair_row, topk_w,
                                                             L.expert_offset, L.T, L.H, L.k, El, L.R, chunks,
                                                             static_cast<T*>(dst));
  else
    combine_recv_kernel<T, VPT><<<blocks, 256, 0, stream>>>(static_cast<const T*>(src), L.pair_row, L.expert_offset,
                                                             L.T, L.H, L.k, El, L.R, chunks, static_cast<T*>(dst));
}

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

static hipError_t launch_combine_sr(bool send, const void* src, int xdt_bf16, const moe_layout_t& L,
                                    const float* topk_w, void* dst, hipStream_t stream) {
  const int vpt = slices_per_thread(L.H / (xdt_bf16 ? 8 : 4));
  if (xdt_bf16) {
    if (vpt == 4) launch_combine_sr_t<bf16_t, 4>(send, src, L, topk_w, dst, stream);
    else if (vpt == 2) launch_combine_sr_t<bf16_t, 2>(send, src, L, topk_w, dst, stream);
    else launch_combine_sr_t<bf16_t, 1>(send, src, L, topk_w, dst, stream);
  } else {
    if (vpt == 4) launch_combine_sr_t<float, 4>(send, src, L, topk_w, dst, stream);
    else if (vpt == 2) launch_combine_sr_t<float, 2>(send, src, L, topk_w, dst, stream);
    else launch_combine_sr_t<float, 1>(send, src, L, topk_w, dst, stream);
  }
  return hipGetLastError();
}

hipError_t launch_combine_send(const void* out_buf, int xdt_bf16, const moe_layout_t& L, const float* topk_w,
                               void* partial, hipStream_t stream) {
  return launch_combine_sr(true, out_buf, xdt_bf16, L, topk_w, partial, stream);
}

hipError_t launch_combine_recv(const void* partial, int xdt_bf16, const moe_layout_t& L, void* y, hipStream_t stream) {
  return launch_combine_sr(false, partial, xdt_bf16, L, nullptr, y, stream);
}

}  // namespace moe
