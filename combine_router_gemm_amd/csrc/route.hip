// Router: logits = x W_r^T (+ bias) in fp32, then per-token top-k and softmax over the k selected.
// Few experts and tokens (E <= 16, T <= 4096) take one fused kernel (route_small); otherwise:
//
// The router is a small linear layer scoring every expert; the k best experts are chosen and their
// weights come from the router's distribution ("Efficient and portable mixture-of-experts
// communication", section "Introductie").
//
// Kernel 1 (route_gemm): split-K GEMM. Grid (token tiles, expert tiles, K splits); each workgroup
//   writes an fp32 partial [T, E] for its K range. fp32 activations run on fp32 MFMA. bf16
//   activations run on bf16 MFMA with the router weight split exactly into three bf16 parts, so
//   every product is the exact fp32 product of the inputs and the sum is accumulated in fp32. With
//   many tokens the weight is split once per call into three planes in the workspace
//   (route_planes), which a direct-to-LDS GEMM then reads (route_gemm_planes); with few, each
//   workgroup splits its weight tile on the way into LDS.
// Kernel 2 (route_topk): sums the K-split partials in a fixed order (deterministic), adds the bias,
//   (with a single split the partial buffer is the logits buffer itself, read then overwritten in place),
//   writes the logits and selects the top-k per token with a lane-group arg-max: G lanes per token,
//   each holding E/G logits, k rounds of a butterfly max over (value desc, expert id asc). When E is a
//   multiple of 64 (route_topk_rows), a wave per token: each lane sorts its E/64 logits once and the k
//   rounds take the wave maximum of the lanes' current heads (same selection).
#include <algorithm>
#include <climits>
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "mfma.h"

namespace moe {

namespace {

constexpr int kRouteMaxSplits = 16;
constexpr int kRouteFusedMaxT = 4096;
constexpr int kRouteTopkWideMaxT = 1024;

constexpr int RG_BM = 64;   // tokens per tile
constexpr int RG_BN = 64;   // experts per tile
constexpr int RG_BK = 32;   // K per LDS stage
constexpr int RG_LDS = RG_BK + 4;  // padded LDS row (floats): 144-byte rows keep b128 reads conflict-free

// Load 8 consecutive elements of row `r`, K offset `kc`, widened to fp32 (zero outside the matrix).
template <typename T>
__device__ __forceinline__ void load8_f32(const T* base, int64_t ld, int r, int nrows, int kc, int kend,
                                          float (&o)[8]);

template <>
__device__ __forceinline__ void load8_f32<float>(const float* base, int64_t ld, int r, int nrows, int kc,
                                                 int kend, float (&o)[8]) {
  if (r < nrows && kc < kend) {
    const float* p = base + (int64_t)r * ld + kc;
    float a[4], b[4];
    unpack(ld16(p), a);
    unpack(ld16(p + 4), b);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[i] = a[i];
      o[4 + i] = b[i];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = 0.f;
  }
}

// grid: (ceil(T/64), ceil(E/64), splits); block 256 = 4 waves in 2x2, each wave a 32x32 output tile.
template <typename TX>
__global__ __launch_bounds__(256) void route_gemm_kernel(const TX* __restrict__ x, const float* __restrict__ w,
                                                         int T, int H, int E, int k_split,
                                                         float* __restrict__ partial) {
  __shared__ float As[RG_BM][RG_LDS];
  __shared__ float Bs[RG_BN][RG_LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int t0 = blockIdx.x * RG_BM;
  const int e0 = blockIdx.y * RG_BN;
  const int kbeg = blockIdx.z * k_split;
  const int kend = min(H, kbeg + k_split);

  // loader: 64 rows x 32 K = 256 groups of 8 -> one group per thread for each matrix
  const int lr = tid >> 2;        // row in tile
  const int lk = (tid & 3) * 8;   // K offset in stage

  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  float ra[8], rb[8];
  const TX* xa = x + (int64_t)t0 * H;
  const float* wb = w + (int64_t)e0 * H;
  load8_f32<TX>(xa, H, lr, T - t0, kbeg + lk, kend, ra);
  load8_f32<float>(wb, H, lr, E - e0, kbeg + lk, kend, rb);

  for (int k0 = kbeg; k0 < kend; k0 += RG_BK) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      As[lr][lk + i] = ra[i];
      Bs[lr][lk + i] = rb[i];
    }
    __syncthreads();
    if (k0 + RG_BK < kend) {
      load8_f32<TX>(xa, H, lr, T - t0, k0 + RG_BK + lk, kend, ra);
      load8_f32<float>(wb, H, lr, E - e0, k0 + RG_BK + lk, kend, rb);
    }
    // lane l supplies row (l % 16) and K = (l / 16) * 8 + i for MFMA step i; A and B use the same
    // K assignment, so the 8 steps together cover the 32-wide stage exactly once.
    const int fr = lane & 15;
    const int fk = (lane >> 4) * 8;
    float af[2][8], bfr[2][8];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const float* pa = &As[wm * 32 + i * 16 + fr][fk];
      const float* pb = &Bs[wn * 32 + i * 16 + fr][fk];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        af[i][q] = pa[q];
        bfr[i][q] = pb[q];
      }
    }
#pragma unroll
    for (int q = 0; q < 8; ++q)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[i][q], bfr[j][q], acc[i][j], 0, 0, 0);
  }

  // C fragment: lane l holds column (l % 16), rows 4 * (l / 16) + r
  float* out = partial + (int64_t)blockIdx.z * T * E;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = e0 + wn * 32 + j * 16 + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = t0 + wm * 32 + i * 16 + (lane >> 4) * 4 + r;
        if (row < T && col < E) out[(int64_t)row * E + col] = acc[i][j][r];
      }
    }
}

// Exact three-way split of an fp32 weight into bf16 parts, w = hi + mid + lo: hi keeps the top 8
// significant bits (truncation), mid the next 8 of the exact remainder, lo the last 8 (exact in bf16).
// With a bf16 activation every product x*hi, x*mid, x*lo is exact in fp32, so three bf16 MFMAs
// accumulating in fp32 give the fp32 dot product up to accumulation order.
__device__ __forceinline__ void split3_bf16(float w, uint16_t& h, uint16_t& m, uint16_t& l) {
  const uint32_t u = __float_as_uint(w);
  const float fh = __uint_as_float(u & 0xffff0000u);
  const float r1 = w - fh;  // exact: the bits of w below hi
  const uint32_t u1 = __float_as_uint(r1);
  const float fm = __uint_as_float(u1 & 0xffff0000u);
  const float r2 = r1 - fm;  // exact, at most 8 significant bits
  h = (uint16_t)(u >> 16);
  m = (uint16_t)(u1 >> 16);
  l = __builtin_bit_cast(uint16_t, (bf16_t)r2);
}

// bf16 activations: BM x BN tiles, 32-deep stages, WM x WN waves of Op MFMAs (32x32x16 bf16 by
// default); the router weight stage is split into its three bf16 planes on the way into LDS.
template <typename Op, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM* WN * 64) void route_gemm_bf16x3_kernel(const bf16_t* __restrict__ x,
                                                                       const float* __restrict__ w, int T, int H,
                                                                       int E, int k_split, float* __restrict__ partial) {
  constexpr int BK = 32;
  constexpr int LDR = BK + 8;  // 80-byte LDS rows: b128 fragment reads stay conflict-free
  constexpr int NTH = WM * WN * 64;
  constexpr int A_VEC = BM * (BK / 8) / NTH;  // 16-byte bf16 vectors per thread
  constexpr int B_VEC = BN * (BK / 4) / NTH;  // 16-byte fp32 vectors per thread
  constexpr int S = Op::S;
  constexpr int TM = BM / WM / S, TN = BN / WN / S;
  static_assert(TM * S * WM == BM && TN * S * WN == BN, "wave tile must tile by the MFMA size");
  static_assert(A_VEC >= 1 && B_VEC >= 1 && BM * (BK / 8) % NTH == 0 && BN * (BK / 4) % NTH == 0, "loader");
  __shared__ __attribute__((aligned(16))) uint16_t As[BM * LDR];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[3][BN * LDR];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int t0 = blockIdx.x * BM, e0 = blockIdx.y * BN;
  const int kbeg = blockIdx.z * k_split;
  const int kend = min(H, kbeg + k_split);

  typename Op::Acc acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < Op::NR; ++q) acc[i][j][q] = 0.f;

  // loads are unconditional from clamped, valid addresses and masked when written to LDS, so the
  // compiler can keep the next stage's loads in flight across the barriers
  u32x4 ra[A_VEC], rb[B_VEC];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < A_VEC; ++i) {
      const int idx = tid + i * NTH, r = idx / (BK / 8), c = (idx % (BK / 8)) * 8;
      ra[i] = ld16(x + (int64_t)min(t0 + r, T - 1) * H + min(k0 + c, kend - 8));
    }
#pragma unroll
    for (int i = 0; i < B_VEC; ++i) {
      const int idx = tid + i * NTH, r = idx / (BK / 4), c = (idx % (BK / 4)) * 4;
      rb[i] = ld16(w + (int64_t)min(e0 + r, E - 1) * H + min(k0 + c, kend - 4));
    }
  };
  const u32x4 zero = {0u, 0u, 0u, 0u};
  load(kbeg);
  for (int k0 = kbeg; k0 < kend; k0 += BK) {
    lds_barrier();
#pragma unroll
    for (int i = 0; i < A_VEC; ++i) {
      const int idx = tid + i * NTH, r = idx / (BK / 8), c = (idx % (BK / 8)) * 8;
      st16(&As[r * LDR + c], (t0 + r < T && k0 + c < kend) ? ra[i] : zero);
    }
#pragma unroll
    for (int i = 0; i < B_VEC; ++i) {
      const int idx = tid + i * NTH, r = idx / (BK / 4), c = (idx % (BK / 4)) * 4;
      uint16_t hv[4], mv[4], lv[4];
      float f[4];
      unpack((e0 + r < E && k0 + c < kend) ? rb[i] : zero, f);
#pragma unroll
      for (int q = 0; q < 4; ++q) split3_bf16(f[q], hv[q], mv[q], lv[q]);
      typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
      *reinterpret_cast<u32x2*>(&Bs[0][r * LDR + c]) = u32x2{hv[0] | ((uint32_t)hv[1] << 16), hv[2] | ((uint32_t)hv[3] << 16)};
      *reinterpret_cast<u32x2*>(&Bs[1][r * LDR + c]) = u32x2{mv[0] | ((uint32_t)mv[1] << 16), mv[2] | ((uint32_t)mv[3] << 16)};
      *reinterpret_cast<u32x2*>(&Bs[2][r * LDR + c]) = u32x2{lv[0] | ((uint32_t)lv[1] << 16), lv[2] | ((uint32_t)lv[3] << 16)};
    }
    lds_barrier();
    load(k0 + BK);  // past the end the addresses clamp to valid data that is never stored
    const int fr = lane % S, fk = (lane / S) * 8;
#pragma unroll
    for (int kk = 0; kk < BK; kk += Op::KS) {
      u32x4 af[TM][1];
#pragma unroll
      for (int i = 0; i < TM; ++i) af[i][0] = ld16(&As[(wm * (BM / WM) + i * S + fr) * LDR + kk + fk]);
#pragma unroll
      for (int pl = 0; pl < 3; ++pl) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          u32x4 bfr[1];
          bfr[0] = ld16(&Bs[pl][(wn * (BN / WN) + j * S + fr) * LDR + kk + fk]);
#pragma unroll
          for (int i = 0; i < TM; ++i) Op::step(acc[i][j], af[i], bfr);
        }
      }
    }
  }
  float* out = partial + (int64_t)blockIdx.z * T * E;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = e0 + wn * (BN / WN) + j * S + (lane % S);
#pragma unroll
      for (int q = 0; q < Op::NR; ++q) {
        const int row = t0 + wm * (BM / WM) + i * S + Op::out_row(lane, q);
        if (row < T && col < E) out[(int64_t)row * E + col] = acc[i][j][q];
      }
    }
}

// (value, id) ordering of the selection: larger value first, then lower id. NaN never wins a
// comparison, so it is treated as -inf.
__device__ __forceinline__ bool better(float v, int e, float bv, int be) {
  return (v > bv) || (v == bv && e < be);
}

// k rounds of a butterfly arg-max over G lanes (lane g holds the values of experts i * G + g; taken
// marks values out of the running), then the softmax over the k winners; lanes g < k write slot g.
template <int G, int VMAX>
__device__ __forceinline__ void select_topk(const float (&val)[VMAX], bool (&taken)[VMAX], int g, int t, bool live,
                                            int k, int* __restrict__ topk_ids, float* __restrict__ topk_w) {
  float sel_v[MOE_MAX_TOPK];
  int sel_e[MOE_MAX_TOPK];
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK; ++j) {
    if (j < k) {
      float bv = -INFINITY;
      int be = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < VMAX; ++i) {
        const int e = i * G + g;
        if (!taken[i] && better(val[i], e, bv, be)) {
          bv = val[i];
          be = e;
        }
      }
#pragma unroll
      for (int off = G / 2; off > 0; off >>= 1) {
        const float ov = __shfl_xor(bv, off, G);
        const int oe = __shfl_xor(be, off, G);
        if (better(ov, oe, bv, be)) {
          bv = ov;
          be = oe;
        }
      }
      sel_v[j] = bv;
      sel_e[j] = be;
      if ((be & (G - 1)) == g) {
        const int ii = be / G;
#pragma unroll
        for (int i = 0; i < VMAX; ++i)
          if (i == ii) taken[i] = true;
      }
    }
  }

  if (live && g < k) {
    // softmax over the k selected logits (slot 0 holds the largest)
    const float m = sel_v[0];
    float sum = 0.f, mine = 0.f;
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) {
      if (j < k) {
        const float z = expf(sel_v[j] - m);
        sum += z;
        if (j == g) mine = z;
      }
    }
    int myid = 0;
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j)
      if (j == g) myid = sel_e[j];
    topk_ids[(int64_t)t * k + g] = myid;
    topk_w[(int64_t)t * k + g] = mine / sum;
  }
}

// Maximum of x over the 64 lanes of the wave, in every lane: DPP swaps within quads, 8- and 16-lane
// mirrors (VALU operations, no LDS), then the four row maxima read into scalar registers.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_f32<0xB1>(x));   // quad_perm [1, 0, 3, 2]
  x = fmaxf(x, dpp_f32<0x4E>(x));   // quad_perm [2, 3, 0, 1]
  x = fmaxf(x, dpp_f32<0x141>(x));  // row_half_mirror
  x = fmaxf(x, dpp_f32<0x140>(x));  // row_mirror
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}
// Sum of x over the 64 lanes of the wave, in every lane, in a fixed order: pairs, quads, 8- and 16-lane
// groups by DPP (each partner adds the same two values, so every lane of a row holds the same bits),
// then (row 0 + row 1) + (row 2 + row 3).
__device__ __forceinline__ float wave_sum(float x) {
  x += dpp_f32<0xB1>(x);
  x += dpp_f32<0x4E>(x);
  x += dpp_f32<0x141>(x);
  x += dpp_f32<0x140>(x);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
  return (r0 + r1) + (r2 + r3);
}

// The selection of select_topk for one token per wave with lane g holding experts g * V + i (i < V): each
// round takes every lane's best untaken value (the lowest i on ties), the wave maximum of those, and as
// winner the lowest lane holding that maximum -- lanes hold ascending expert ranges, so that is the
// lowest expert id among the equal values, the same (value desc, id asc) order. No LDS traffic: a DPP
// maximum, a ballot and lane reads into scalar registers per round.
template <int VMAX>
__device__ __forceinline__ void select_topk_wave(const float (&val)[VMAX], bool (&taken)[VMAX], int g, int t,
                                                 bool live, int k, int V, int* __restrict__ topk_ids,
                                                 float* __restrict__ topk_w) {
  float sel_v[MOE_MAX_TOPK];
  int sel_e[MOE_MAX_TOPK];
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK; ++j) {
    if (j < k) {
      float bv = -INFINITY;
      int bi = -1;
#pragma unroll
      for (int i = 0; i < VMAX; ++i) {
        if (!taken[i] && (bi < 0 || val[i] > bv)) {
          bv = val[i];
          bi = i;
        }
      }
      const float m = wave_max(bv);
      const uint64_t cand = __ballot(bi >= 0 && bv == m);
      const int wl = __builtin_ctzll(cand);  // k <= E: some lane still holds a value
      const int we = __builtin_amdgcn_readlane(g * V + bi, wl);
      sel_v[j] = m;
      sel_e[j] = we;
      if (g == wl) {
#pragma unroll
        for (int i = 0; i < VMAX; ++i)
          if (i == bi) taken[i] = true;
      }
    }
  }
  if (live && g < k) {
    // softmax over the k selected logits (slot 0 holds the largest)
    const float m = sel_v[0];
    float sum = 0.f, mine = 0.f;
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) {
      if (j < k) {
        const float z = expf(sel_v[j] - m);
        sum += z;
        if (j == g) mine = z;
      }
    }
    int myid = 0;
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j)
      if (j == g) myid = sel_e[j];
    topk_ids[(int64_t)t * k + g] = myid;
    topk_w[(int64_t)t * k + g] = mine / sum;
  }
}

// G lanes per token (power of two, 8..64), V = ceil(E / G) logits per lane, expert of lane g's
// i-th value is i * G + g.
template <int G>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* partial, int splits,
                                                         const float* __restrict__ bias, int64_t bias_stride,
                                                         int T, int E, int k, float* logits,
                                                         int* __restrict__ topk_ids, float* __restrict__ topk_w) {
  // G < 64 is only chosen when E <= G (one logit per lane); G == 64 covers E <= 512 (8 per lane)
  constexpr int VMAX = G < 64 ? 1 : MOE_MAX_EXPERTS / 64;
  const int g = threadIdx.x & (G - 1);
  const int t = (blockIdx.x * blockDim.x + threadIdx.x) / G;
  const bool live = t < T;
  const int V = (E + G - 1) / G;

  float val[VMAX];
  bool taken[VMAX];
  float sum[VMAX];
#pragma unroll
  for (int i = 0; i < VMAX; ++i) {
    const int e = i * G + g;
    taken[i] = !(i < V && e < E && live);
    sum[i] = taken[i] ? 0.f : partial[(int64_t)t * E + e];
  }
  // the remaining K-split partials, SPF splits of loads in flight at a time, added in split order
  constexpr int SPF = 4;
  const int64_t TE = (int64_t)T * E;
  for (int sp0 = 1; sp0 < splits; sp0 += SPF) {
    float tmp[SPF][VMAX];
#pragma unroll
    for (int u = 0; u < SPF; ++u)
#pragma unroll
      for (int i = 0; i < VMAX; ++i)
        tmp[u][i] = (!taken[i] && sp0 + u < splits) ? partial[(sp0 + u) * TE + (int64_t)t * E + i * G + g] : 0.f;
#pragma unroll
    for (int u = 0; u < SPF; ++u)
#pragma unroll
      for (int i = 0; i < VMAX; ++i)
        if (sp0 + u < splits) sum[i] += tmp[u][i];
  }
#pragma unroll
  for (int i = 0; i < VMAX; ++i) {
    val[i] = -INFINITY;
    if (!taken[i]) {
      const int e = i * G + g;
      float s = sum[i];
      if (bias) s += bias[(int64_t)t * bias_stride + e];
      logits[(int64_t)t * E + e] = s;
      s = s + 0.0f;                       // -0 -> +0: equal values compare equal either way
      val[i] = (s == s) ? s : -INFINITY;  // NaN ranks as -inf
    }
  }

  select_topk<G, VMAX>(val, taken, g, t, live, k, topk_ids, topk_w);
}

// Integer max over the 64 lanes of the wave, in every lane (same DPP pattern as wave_max; v_max_i32 needs
// no NaN handling).
template <int CTRL>
__device__ __forceinline__ int dpp_i32(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ int wave_max_i32(int x) {
  x = max(x, dpp_i32<0xB1>(x));   // quad_perm [1, 0, 3, 2]
  x = max(x, dpp_i32<0x4E>(x));   // quad_perm [2, 3, 0, 1]
  x = max(x, dpp_i32<0x141>(x));  // row_half_mirror
  x = max(x, dpp_i32<0x140>(x));  // row_mirror
  const int r0 = __builtin_amdgcn_readlane(x, 0), r1 = __builtin_amdgcn_readlane(x, 16);
  const int r2 = __builtin_amdgcn_readlane(x, 32), r3 = __builtin_amdgcn_readlane(x, 48);
  return max(max(r0, r1), max(r2, r3));
}
// Order-preserving integer key of a float that is not NaN and not -0: a larger float has a larger key,
// equal floats have equal keys, and key_float inverts it.
__device__ __forceinline__ int float_key(float v) {
  const int b = __float_as_int(v);
  return b >= 0 ? b : b ^ 0x7fffffff;
}
__device__ __forceinline__ float key_float(int key) { return __int_as_float(key >= 0 ? key : key ^ 0x7fffffff); }

// The same selection as select_topk_wave (the k largest values of the wave, ties to the lowest expert, expert
// of lane g's i-th value g * V + i, then the softmax over the k selected values), for VT values per lane
// known at compile time. val[i] for i >= V must be absent (passed as any value; they are never selected).
// Each lane first sorts its values by key, descending and stable (equal values keep ascending i); every
// round then takes the wave maximum of the lanes' current heads, and the lowest lane holding it (so the
// lowest expert among equal values) moves its head on. No branches and no dynamic indexing.
template <int VT>
__device__ __forceinline__ void select_topk_sorted(const float (&val)[VT], int g, int t, int k, int V,
                                                   int* __restrict__ topk_ids, float* __restrict__ topk_w) {
  int key[VT], idx[VT];
#pragma unroll
  for (int i = 0; i < VT; ++i) {
    key[i] = i < V ? float_key(val[i]) : INT_MIN;  // INT_MIN is below every value's key (-inf included)
    idx[i] = i;
  }
#pragma unroll
  for (int a = 1; a < VT; ++a)
#pragma unroll
    for (int b = a; b > 0; --b) {
      const bool sw = key[b] > key[b - 1];  // strictly greater: equal keys keep their order
      const int k0 = key[b - 1], k1 = key[b], i0 = idx[b - 1], i1 = idx[b];
      key[b - 1] = sw ? k1 : k0;
      key[b] = sw ? k0 : k1;
      idx[b - 1] = sw ? i1 : i0;
      idx[b] = sw ? i0 : i1;
    }
  int ptr = 0;  // this lane's next unselected position
  float sel_v[MOE_MAX_TOPK];
  int sel_e[MOE_MAX_TOPK];
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK; ++j) {
    if (j < k) {
      int head = INT_MIN, hidx = 0;
#pragma unroll
      for (int p = 0; p < VT; ++p) {
        head = ptr == p ? key[p] : head;
        hidx = ptr == p ? idx[p] : hidx;
      }
      const int m = wave_max_i32(head);
      const uint64_t cand = __ballot(head == m);  // k <= E: m is a present value's key
      const int wl = __builtin_ctzll(cand);
      sel_e[j] = __builtin_amdgcn_readlane(g * V + hidx, wl);
      sel_v[j] = key_float(m);
      ptr += g == wl ? 1 : 0;
    }
  }
  if (g < k) {
    // softmax over the k selected logits (slot 0 holds the largest)
    const float m = sel_v[0];
    float sum = 0.f, mine = 0.f;
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) {
      if (j < k) {
        const float z = expf(sel_v[j] - m);
        sum += z;
        if (j == g) mine = z;
      }
    }
    int myid = 0;
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j)
      if (j == g) myid = sel_e[j];
    topk_ids[(int64_t)t * k + g] = myid;
    topk_w[(int64_t)t * k + g] = mine / sum;
  }
}

// E = 64 V (V <= 8): one wave per token, lane g holding the V consecutive experts g V .. g V + V - 1, so
// the lane reads its part of each split's row with V / VW loads of VW floats (VW = 4, 2 or 1, dividing V,
// with partial and logits aligned to it) instead of V single-float loads; the bias of the token is read
// with its first split, and SPF further splits are in flight at a time. Same sums, in the same order, as
// route_topk_kernel. VT is V rounded up to 1, 2, 4 or 8; the selection is select_topk_sorted.
template <int VW, int SPF, int VT>
__global__ __launch_bounds__(256) void route_topk_rows_kernel(const float* partial, int splits,
                                                              const float* __restrict__ bias, int64_t bias_stride,
                                                              int T, int E, int k, float* logits,
                                                              int* __restrict__ topk_ids, float* __restrict__ topk_w) {
  constexpr int VMAX = VT;  // V = E / 64 logits per lane, rounded up to 1, 2, 4 or 8
  const int g = threadIdx.x & 63;
  const int t = (int)(((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6);
  const bool live = t < T;  // the same for the whole wave
  const int V = E >> 6;
  const int64_t row = (int64_t)(live ? t : 0) * E + (int64_t)g * V;  // this lane's first value
  auto load_row = [&](const float* p, float (&v)[VMAX]) {
#pragma unroll
    for (int i = 0; i < VMAX; i += VW) {
      if (i < V) {
        if (VW == 4) {
          unpack(ld16(p + i), *reinterpret_cast<float(*)[4]>(&v[i]));
        } else if (VW == 2) {
          const f32x2 q = *reinterpret_cast<const f32x2*>(p + i);
          v[i] = q.x;
          v[i + 1] = q.y;
        } else {
          v[i] = p[i];
        }
      }
    }
  };
  float sum[VMAX], b[VMAX];
  bool taken[VMAX];
#pragma unroll
  for (int i = 0; i < VMAX; ++i) {
    taken[i] = !(i < V && live);
    sum[i] = 0.f;
    b[i] = 0.f;
  }
  if (live) {
    load_row(partial + row, sum);
    if (bias) {
      const float* pb = bias + (int64_t)t * bias_stride + (int64_t)g * V;
#pragma unroll
      for (int i = 0; i < VMAX; ++i)
        if (i < V) b[i] = pb[i];
    }
    // the remaining K-split partials, added in split order
    const int64_t TE = (int64_t)T * E;
    for (int sp0 = 1; sp0 < splits; sp0 += SPF) {
      float tmp[SPF][VMAX];
#pragma unroll
      for (int u = 0; u < SPF; ++u)
        if (sp0 + u < splits) load_row(partial + (sp0 + u) * TE + row, tmp[u]);
#pragma unroll
      for (int u = 0; u < SPF; ++u)
#pragma unroll
        for (int i = 0; i < VMAX; ++i)
          if (sp0 + u < splits && i < V) sum[i] += tmp[u][i];
    }
  }
  float val[VMAX];
#pragma unroll
  for (int i = 0; i < VMAX; ++i) {
    val[i] = -INFINITY;
    if (!taken[i]) {
      float s = sum[i];
      if (bias) s += b[i];
      sum[i] = s;
      s = s + 0.0f;                       // -0 -> +0: equal values compare equal either way
      val[i] = (s == s) ? s : -INFINITY;  // NaN ranks as -inf
    }
  }
  if (live) {
    float* pl = logits + row;
#pragma unroll
    for (int i = 0; i < VMAX; i += VW) {
      if (i < V) {
        if (VW == 4) {
          st16(pl + i, pack(*reinterpret_cast<const float(*)[4]>(&sum[i])));
        } else if (VW == 2) {
          *reinterpret_cast<f32x2*>(pl + i) = f32x2{sum[i], sum[i + 1]};
        } else {
          pl[i] = sum[i];
        }
      }
    }
  }
  // live is uniform across the wave (one token per wave)
  if (live) select_topk_sorted<VMAX>(val, g, t, k, V, topk_ids, topk_w);
}

// Few experts: one workgroup of 256 threads per token computes the logits directly. Thread i
// accumulates in fp32 the products of the 16-byte x chunks i, i + 256, ... with the matching fp32
// router-weight slices of every expert (all loads of a chunk in flight at once; the router weight is
// an L2 hit after the first token), a DPP reduction sums each expert over the wave, and wave 0 adds the
// four wave sums in wave order (deterministic). Lane e (< E) of wave 0 then holds logit e for the
// same selection as route_topk.
template <typename TX, int EMAX>
__global__ __launch_bounds__(256) void route_small_kernel(const TX* __restrict__ x, const float* __restrict__ w,
                                                          const float* __restrict__ bias, int64_t bias_stride,
                                                          int T, int H, int E, int k, float* __restrict__ logits,
                                                          int* __restrict__ topk_ids, float* __restrict__ topk_w) {
  constexpr int VN = Vec<TX>::N;  // x elements per 16-byte chunk
  __shared__ float s_part[4][EMAX];
  const int lane = lane_id(), wave = (int)(threadIdx.x >> 6);
  const int t = blockIdx.x;
  float acc[EMAX];
#pragma unroll
  for (int e = 0; e < EMAX; ++e) acc[e] = 0.f;
  const TX* xr = x + (int64_t)t * H;
#pragma unroll 2
  for (int c = threadIdx.x; c * VN < H; c += 256) {
    float xv[VN];
    unpack(ld16(xr + c * VN), xv);
    u32x4 wraw[EMAX][VN / 4];
#pragma unroll
    for (int e = 0; e < EMAX; ++e)
#pragma unroll
      for (int q = 0; q < VN / 4; ++q)
        if (e < E) wraw[e][q] = ld16(w + (int64_t)e * H + c * VN + q * 4);
#pragma unroll
    for (int e = 0; e < EMAX; ++e) {
      if (e < E) {
#pragma unroll
        for (int q = 0; q < VN / 4; ++q) {
          float wv[4];
          unpack(wraw[e][q], wv);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[e] = fmaf(xv[q * 4 + r], wv[r], acc[e]);
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < EMAX; ++e) {
    if (e < E) {
      const float v = wave_sum(acc[e]);
      if (lane == 0) s_part[wave][e] = v;
    }
  }
  __syncthreads();
  if (wave != 0) return;
  float val[1];
  bool taken[1];
  taken[0] = lane >= E;
  val[0] = -INFINITY;
  if (!taken[0]) {
    float s = ((s_part[0][lane] + s_part[1][lane]) + s_part[2][lane]) + s_part[3][lane];
    if (bias) s += bias[(int64_t)t * bias_stride + lane];
    logits[(int64_t)t * E + lane] = s;
    s = s + 0.0f;                          // -0 -> +0
    val[0] = (s == s) ? s : -INFINITY;     // NaN ranks as -inf
  }
  select_topk_wave<1>(val, taken, lane, t, true, k, 1, topk_ids, topk_w);
}

// ------------------------------------------------------------------------------------------------
// Many tokens (bf16, T >= 2048, H % 64 == 0): the router weight split once per call into its three
// exact bf16 planes, then a direct-to-LDS GEMM over the planes
// ------------------------------------------------------------------------------------------------
// planes [3][E][H] bf16: plane p of expert e at planes + (p * E + e) * H (split3_bf16 per element)
__global__ __launch_bounds__(256) void route_planes_kernel(const float* __restrict__ w, int E, int H,
                                                           uint16_t* __restrict__ planes) {
  const int64_t n4 = (int64_t)E * H / 4;
  const int64_t stride = (int64_t)gridDim.x * 256;
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
    float f[4];
    unpack(ld16(w + i * 4), f);
    uint16_t hv[4], mv[4], lv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) split3_bf16(f[q], hv[q], mv[q], lv[q]);
    const int64_t plane = (int64_t)E * H;
    *reinterpret_cast<u32x2*>(planes + i * 4) = u32x2{hv[0] | ((uint32_t)hv[1] << 16), hv[2] | ((uint32_t)hv[3] << 16)};
    *reinterpret_cast<u32x2*>(planes + plane + i * 4) =
        u32x2{mv[0] | ((uint32_t)mv[1] << 16), mv[2] | ((uint32_t)mv[3] << 16)};
    *reinterpret_cast<u32x2*>(planes + 2 * plane + i * 4) =
        u32x2{lv[0] | ((uint32_t)lv[1] << 16), lv[2] | ((uint32_t)lv[3] << 16)};
  }
}

template <int N>
__device__ __forceinline__ void route_wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// 256 tokens x 128 experts x 64-deep stages, 8 waves (4 x 2) of 64 x 64, two stage slots of 80 KB:
// A = 256 x rows, B = the 3 planes x 128 experts (row p * 128 + e). Operands go global -> LDS with
// buffer_load_dwordx4 ... lds (one wave instruction = 8 rows of 128 bytes), chunk c of LDS row r at
// c ^ ((r >> 1) & 7), rows past T or E fetched at an out-of-range offset (zeros). Schedule: the barrier
// that publishes stage s + 1 sits before the MFMAs of stage s's last K step; right after it the x loads
// of stage s + 2 (the HBM stream) go into stage s's slot, one between MFMAs, and the plane loads of stage
// s + 1 (L2-resident) go out between the MFMAs of stage s's first K step. Per K step a wave multiplies
// its 2 x blocks by 2 expert blocks of each plane into the same accumulators. The grid is one
// workgroup per (K split, token tile, expert tile), cut into eight contiguous ranges, one per XCD, so
// the expert tiles of one token tile share an L2. Writes an fp32 partial [T, E] per K split.
constexpr int RP_BM = 256, RP_BN = 128, RP_BK = 64, RP_WM = 4, RP_WN = 2, RP_NW = RP_WM * RP_WN;
__global__ __launch_bounds__(RP_NW * 64) void route_gemm_planes_kernel(const bf16_t* __restrict__ x,
                                                                      const uint16_t* __restrict__ planes, int T,
                                                                      int H, int E, int k_split, int n_ttiles,
                                                                      int n_etiles, int n_items,
                                                                      float* __restrict__ partial) {
  using Op = Op32;
  constexpr int S = 32, ROWB = RP_BK * 2, CPR = 8, RPI = 8;
  constexpr int A_ROWS = RP_BM, B_ROWS = 3 * RP_BN;
  constexpr int A_INS = A_ROWS / RPI, B_INS = B_ROWS / RPI;
  static_assert(A_INS % RP_NW == 0 && B_INS % RP_NW == 0, "even loads per wave");
  constexpr int AW = A_INS / RP_NW, BW = B_INS / RP_NW, LPW = AW + BW;
  constexpr int A_BYTES = A_ROWS * ROWB, STAGE = (A_ROWS + B_ROWS) * ROWB;
  constexpr int TM = RP_BM / RP_WM / S, TN = RP_BN / RP_WN / S;
  constexpr int KSTEPS = RP_BK / Op::KS;
  static_assert(2 * STAGE <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * STAGE];

  // work item of this workgroup: (split, token tile, expert tile), expert tile fastest
  int item = blockIdx.x;
  if ((n_items & 7) == 0 && (int)gridDim.x == n_items) item = (blockIdx.x & 7) * (n_items >> 3) + (blockIdx.x >> 3);
  const int et = item % n_etiles, tt = (item / n_etiles) % n_ttiles, split = item / (n_etiles * n_ttiles);
  const int t0 = tt * RP_BM, e0 = et * RP_BN;
  const int kbeg = split * k_split, kend = min(H, kbeg + k_split);
  const int nk = (kend - kbeg) / RP_BK;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / RP_WN, wn = wave % RP_WN;
  const int OOB = 0x7ffffff0;
  const __amdgpu_buffer_rsrc_t x_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)x, (short)0, (int)((int64_t)T * H * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t p_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)planes, (short)0, (int)((int64_t)3 * E * H * 2), 0x00020000);
  auto swz = [](int r) { return (r >> 1) & 7; };

  // this wave's loads: q < AW are x rows (instructions wave * AW + q), the rest plane rows
  int voff[LPW];
#pragma unroll
  for (int q = 0; q < LPW; ++q) {
    const int r_in = lane / CPR, pos = lane % CPR;
    if (q < AW) {
      const int r = (wave * AW + q) * RPI + r_in;
      voff[q] = t0 + r < T ? ((t0 + r) * H + kbeg) * 2 + ((pos ^ swz(r)) << 4) : OOB;
    } else {
      const int r = (wave * BW + q - AW) * RPI + r_in;  // B row: plane r / BN, expert e0 + r % BN
      const int p = r / RP_BN, e = e0 + r % RP_BN;
      voff[q] = e < E ? ((p * E + e) * H + kbeg) * 2 + ((pos ^ swz(r)) << 4) : OOB;
    }
  }
  auto loff = [&](int q) { return q < AW ? (wave * AW + q) * 1024 : A_BYTES + (wave * BW + q - AW) * 1024; };
  auto issue_one = [&](int st, int slot, int q) {
    const int vo = voff[q] == OOB ? OOB : voff[q] + st * RP_BK * 2;
    auto* dst = (__attribute__((address_space(3))) void*)(smem + slot * STAGE + loff(q));
    if (q < AW) __builtin_amdgcn_raw_ptr_buffer_load_lds(x_rsrc, dst, 16, vo, 0, 0, 0);
    else __builtin_amdgcn_raw_ptr_buffer_load_lds(p_rsrc, dst, 16, vo, 0, 0, 0);
  };

  typename Op::Acc acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < Op::NR; ++q) acc[i][j][q] = 0.f;

  const int fr = lane & 31, fq = lane >> 5;
  auto load_frags = [&](const unsigned char* base, int kk, u32x4 (&af)[TM][1], u32x4 (&bfg)[3][TN][1]) {
    const int c = kk / 8 + fq;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int r = wm * (RP_BM / RP_WM) + i * S + fr;
      af[i][0] = ld16(base + r * ROWB + ((c ^ swz(r)) << 4));
    }
#pragma unroll
    for (int p = 0; p < 3; ++p)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int r = p * RP_BN + wn * (RP_BN / RP_WN) + j * S + fr;
        bfg[p][j][0] = ld16(base + A_BYTES + r * ROWB + ((c ^ swz(r)) << 4));
      }
  };

  if (nk > 0) {
    // prologue: stage 0 into slot 0, the x loads of stage 1 into slot 1
#pragma unroll
    for (int q = 0; q < AW; ++q) issue_one(0, 0, q);
#pragma unroll
    for (int q = AW; q < LPW; ++q) issue_one(0, 0, q);
    if (nk > 1) {
#pragma unroll
      for (int q = 0; q < AW; ++q) issue_one(1, 1, q);
      route_wait_vmcnt<AW>();
    } else {
      route_wait_vmcnt<0>();
    }
    lds_barrier();
    u32x4 af[2][TM][1], bfg[2][3][TN][1];
    load_frags(smem, 0, af[0], bfg[0]);
    auto stage = [&](int s, auto HAVE1, auto HAVE2) {
      constexpr bool have1 = decltype(HAVE1)::value, have2 = decltype(HAVE2)::value;
      const int slot = s & 1;
      const unsigned char* base = smem + slot * STAGE;
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        if (ks + 1 < KSTEPS) {
          load_frags(base, (ks + 1) * Op::KS, af[(ks + 1) & 1], bfg[(ks + 1) & 1]);
        } else if (have1) {
          route_wait_vmcnt<0>();  // this wave's loads of stage s + 1
          lds_barrier();          // stage s + 1 visible; no wave reads slot s & 1 any more
          load_frags(smem + (slot ^ 1) * STAGE, 0, af[0], bfg[0]);
        }
        // the next K step's fragment reads stay ahead of this step's MFMAs (the scheduler would
        // otherwise sink each read to just before its use and wait on it there)
        __builtin_amdgcn_sched_barrier(0);
        int m = 0;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) {
#pragma unroll
            for (int p = 0; p < 3; ++p) Op::step(acc[i][j], af[ks & 1][i], bfg[ks & 1][p][j]);
            // one load between each group of three MFMAs: plane loads of stage s + 1 in the first K step,
            // x loads of stage s + 2 in the last
            if (ks == 0 && have1 && m < BW) issue_one(s + 1, slot ^ 1, AW + m);
            if (ks == KSTEPS - 1 && have2 && m < AW) issue_one(s + 2, slot, m);
            ++m;
          }
        if (ks == 0 && have1) {
#pragma unroll
          for (int q = TM * TN; q < BW; ++q) issue_one(s + 1, slot ^ 1, AW + q);
        }
        if (ks == KSTEPS - 1 && have2) {
#pragma unroll
          for (int q = TM * TN; q < AW; ++q) issue_one(s + 2, slot, q);
        }
      }
    };
    using Yes = std::integral_constant<bool, true>;
    using No = std::integral_constant<bool, false>;
    int s = 0;
    for (; s + 2 < nk; ++s) stage(s, Yes{}, Yes{});
    if (s + 1 < nk) stage(s++, Yes{}, No{});
    stage(s, No{}, No{});
  }

  float* out = partial + (int64_t)split * T * E;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = e0 + wn * (RP_BN / RP_WN) + j * S + fr;
#pragma unroll
      for (int q = 0; q < Op::NR; ++q) {
        const int row = t0 + wm * (RP_BM / RP_WM) + i * S + Op::out_row(lane, q);
        if (row < T && col < E) out[(int64_t)row * E + col] = acc[i][j][q];
      }
    }
}

}  // namespace

// Host-side planning. Tile shape: fp32 activations use 64x64 fp32-MFMA tiles; bf16 activations use the
// plane GEMM (256 x 128 tiles, the weight split once into three bf16 planes) for many tokens when the
// row length is a multiple of 64 and the operands fit 31-bit buffer offsets, 64x64 bf16x3 tiles for few.
// The split-K factor gives enough workgroups to cover the chip (twice for the register-staged tiles,
// once for the plane GEMM, whose 160 KB of LDS take a whole CU), each split at least 256 K-elements long
// and a multiple of the stage depth.
RouteTiles route_tiles(int T, int H, int E, int xdt_bf16) {
  if (xdt_bf16 && T >= 2048 && H % RP_BK == 0 && (int64_t)T * H * 2 < 0x7ffffff0ll - 256 &&
      (int64_t)3 * E * H * 2 < 0x7ffffff0ll - 256)
    return RouteTiles{RP_BM, RP_BN, true};
  return RouteTiles{64, 64, false};
}

bool route_fused(int T, int E) { return E <= 16 && T <= kRouteFusedMaxT; }

RoutePlan route_plan(int T, int H, int E, int xdt_bf16, int num_cus) {
  RoutePlan p{};
  p.tiles = route_tiles(T, H, E, xdt_bf16);
  if (route_fused(T, E) || T <= 0) {
    p.splits = p.nsplit = 1;
    p.k_split = H;
    return p;
  }
  const int tiles = ceil_div_host(T, p.tiles.BM) * ceil_div_host(E, p.tiles.BN);
  int s = ceil_div_host((p.tiles.planes ? 1 : 2) * num_cus, tiles > 0 ? tiles : 1);
  // at least 256 K per split, and few enough splits that the partial sums stay a small share of the
  // traffic (the top-k kernel reads them all back)
  int smax = H / 256 > 0 ? H / 256 : 1;
  if (smax > kRouteMaxSplits) smax = kRouteMaxSplits;
  if (s > smax) s = smax;
  if (s < 1) s = 1;
  const int align = p.tiles.planes ? RP_BK : RG_BK;
  p.splits = s;
  p.k_split = ceil_div_host(ceil_div_host(H, s), align) * align;
  p.nsplit = ceil_div_host(H, p.k_split);
  p.planes_bytes = p.tiles.planes ? align256((size_t)3 * E * H * 2) : 0;
  p.partial_bytes = p.nsplit > 1 ? (size_t)p.nsplit * T * E * sizeof(float) : 0;
  return p;
}

hipError_t launch_route(const void* x, int xdt_bf16, const float* w_router, const float* bias,
                        int64_t bias_stride, int T, int H, int E, int k, float* logits, int* ids, float* wts,
                        void* workspace, const RoutePlan& plan, hipStream_t stream) {
  if (route_fused(T, E)) {
    const unsigned blocks = (unsigned)T;
    const bool e8 = E <= 8;
#define MOE_ROUTE_SMALL(TX, EM)                                                                         \
  route_small_kernel<TX, EM><<<blocks, 256, 0, stream>>>(static_cast<const TX*>(x), w_router, bias,         \
                                                         bias_stride, T, H, E, k, logits, ids, wts)
    if (xdt_bf16) {
      if (e8) MOE_ROUTE_SMALL(bf16_t, 8);
      else MOE_ROUTE_SMALL(bf16_t, 16);
    } else {
      if (e8) MOE_ROUTE_SMALL(float, 8);
      else MOE_ROUTE_SMALL(float, 16);
    }
#undef MOE_ROUTE_SMALL
    return hipGetLastError();
  }
  const int k_split = plan.k_split;
  const int nsplit = plan.nsplit;
  const RouteTiles rt = plan.tiles;
  // the partial sums: in the workspace past the planes with several K splits, else the logits themselves
  float* partial = nsplit > 1 ? reinterpret_cast<float*>(static_cast<char*>(workspace) + plan.planes_bytes) : logits;
  dim3 grid(ceil_div_host(T, rt.BM), ceil_div_host(E, rt.BN), nsplit);
  if (rt.planes) {
    uint16_t* planes = static_cast<uint16_t*>(workspace);
    const int64_t n4 = (int64_t)E * H / 4;
    const unsigned pb = (unsigned)std::min<int64_t>(ceil_div_host64(n4, 256), 2048);
    route_planes_kernel<<<pb, 256, 0, stream>>>(w_router, E, H, planes);
    const int n_tt = ceil_div_host(T, RP_BM), n_et = ceil_div_host(E, RP_BN), n_items = n_tt * n_et * nsplit;
    route_gemm_planes_kernel<<<n_items, RP_NW * 64, 0, stream>>>(static_cast<const bf16_t*>(x), planes, T, H, E, k_split,
                                                                n_tt, n_et, n_items, partial);
  } else if (xdt_bf16)
    route_gemm_bf16x3_kernel<Op32, 64, 64, 2, 2><<<grid, 256, 0, stream>>>(static_cast<const bf16_t*>(x), w_router, T, H, E,
                                                                     k_split, partial);
  else
    route_gemm_kernel<float><<<grid, 256, 0, stream>>>(static_cast<const float*>(x), w_router, T, H, E, k_split,
                                                       partial);
  if (E % 64 == 0) {
    const int V = E / 64;
    const uintptr_t al = reinterpret_cast<uintptr_t>(partial) | reinterpret_cast<uintptr_t>(logits);
    const int blocks = ceil_div_host(T, 4);  // four tokens (waves) per workgroup
    // with few tokens every split is loaded at once (latency); with many, four at a time (occupancy)
    const bool wide = T <= kRouteTopkWideMaxT;
    // VT: logits per lane rounded up to 1, 2, 4 or 8 (E <= 512); VW: the vector width of the row loads
    auto rows = [&](auto VW_C, auto VT_C) {
      constexpr int VW = decltype(VW_C)::value, VT = decltype(VT_C)::value;
      if (wide)
        route_topk_rows_kernel<VW, kRouteMaxSplits, VT><<<blocks, 256, 0, stream>>>(partial, nsplit, bias, bias_stride,
                                                                                    T, E, k, logits, ids, wts);
      else
        route_topk_rows_kernel<VW, 4, VT><<<blocks, 256, 0, stream>>>(partial, nsplit, bias, bias_stride, T, E, k,
                                                                      logits, ids, wts);
    };
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I4 = std::integral_constant<int, 4>;
    using I8 = std::integral_constant<int, 8>;
    const int vw = V % 4 == 0 && al % 16 == 0 ? 4 : (V % 2 == 0 && al % 8 == 0 ? 2 : 1);
    if (V == 1) rows(I1{}, I1{});
    else if (V == 2) (vw >= 2 ? rows(I2{}, I2{}) : rows(I1{}, I2{}));
    else if (V <= 4) (vw == 4 ? rows(I4{}, I4{}) : vw == 2 ? rows(I2{}, I4{}) : rows(I1{}, I4{}));
    else (vw == 4 ? rows(I4{}, I8{}) : vw == 2 ? rows(I2{}, I8{}) : rows(I1{}, I8{}));
    return hipGetLastError();
  }
  // lane-group size: smallest power of two >= E, between 8 and 64
  int G = 8;
  while (G < E && G < 64) G *= 2;
  const int threads = 256;
  const int blocks = ceil_div_host(T * G, threads);
  switch (G) {
    case 8:
      route_topk_kernel<8><<<blocks, threads, 0, stream>>>(partial, nsplit, bias, bias_stride, T, E, k, logits,
                                                          ids, wts);
      break;
    case 16:
      route_topk_kernel<16><<<blocks, threads, 0, stream>>>(partial, nsplit, bias, bias_stride, T, E, k, logits,
                                                           ids, wts);
      break;
    case 32:
      route_topk_kernel<32><<<blocks, threads, 0, stream>>>(partial, nsplit, bias, bias_stride, T, E, k, logits,
                                                           ids, wts);
      break;
    default:
      route_topk_kernel<64><<<blocks, threads, 0, stream>>>(partial, nsplit, bias, bias_stride, T, E, k, logits,
                                                           ids, wts);
      break;
  }
  return hipGetLastError();
}

}  // namespace moe
