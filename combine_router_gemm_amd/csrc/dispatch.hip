// Dispatch: partition (token, slot) pairs by expert into contiguous, rank-aligned per-expert rows.
//
// The pages' send side counts tokens per expert with on-chip atomics, turns the counts into offsets with
// a cumulative sum and packs every token into its expert's contiguous region ("Enabling
// trillion-parameter models on AWS EFA", section "Диспетчеризация и комбинирование"); the per-expert
// capacity drops pairs beyond C, overflow = max(assigned - C, 0) ("80. MoE Expert Parallel
// Benchmark", Step 2). The pages' receive side orders tokens through an atomic counter, so its order
// is not deterministic ("Efficient and portable mixture-of-experts communication", section
// "Dispatch"); here every row position is the stable one: pair (t, j) of expert e lands at
// position #(earlier pairs in row-major order with expert e).
//
// Three kernels:
//   dispatch_rank    one workgroup per DISPATCH_TB tokens. Each wave walks a contiguous slice of the
//                    block's pairs 64 at a time; lanes with the same expert find each other with one
//                    ballot per id bit (a wave-wide match), which gives the stable rank inside the 64;
//                    one lane per distinct expert does an LDS atomic add of the group size on a
//                    wave-private counter (per-wave counters keep the order stable). The four waves'
//                    counts are then scanned in LDS, giving the block histogram (to blk_count) and each
//                    pair's rank inside its block (to pair_local).
//   dispatch_scan    one workgroup: per expert, an exclusive scan of blk_count over blocks (in place),
//                    count / kept / overflow, then an exclusive scan of kept over experts -> offsets.
//   dispatch_scatter one wave per token: position = block base + rank in block; kept pairs write the
//                    layout entries, and each 16-byte slice of the token row is read once and stored to
//                    every kept row (non-temporal stores).
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int DR_THREADS = 256;
constexpr int DR_WAVES = DR_THREADS / MOE_WAVE;
static_assert(2 * DR_THREADS >= MOE_MAX_EXPERTS, "the one-block scan gives each thread two experts");

// Exclusive scan of v over the DR_THREADS threads of the workgroup (thread order); *total gets the sum.
__device__ __forceinline__ int block_exclusive_scan(int v, int* s_wsum, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int u = __shfl_up(incl, off, 64);
    if (lane >= off) incl += u;
  }
  if (lane == 63) s_wsum[wave] = incl;
  __syncthreads();
  int wbase = 0, sum = 0;
#pragma unroll
  for (int w = 0; w < DR_WAVES; ++w) {
    if (w < wave) wbase += s_wsum[w];
    sum += s_wsum[w];
  }
  *total = sum;
  return wbase + incl - v;
}

// Stable ranks of the pairs [p_begin, p_end) of one workgroup of DR_THREADS threads. Wave w takes the
// 64 k pairs from p_begin + 64 k w in k chunks of 64; lanes with the same expert find each other with one
// ballot per id bit (a wave-wide match), which gives the stable rank inside the 64, and one lane per
// distinct expert does an LDS atomic add of the group size on a wave-private counter (per-wave counters
// keep the order stable). On return (after a barrier) cnt[w][e] holds wave w's base for expert e inside
// the workgroup and tot[e] the workgroup's count of expert e; lane chunk c's pair (p = w_begin + 64 c +
// lane) has expert mye[c] (-1: no pair, or an id out of range) and rank myrank[c] in its wave.
__device__ __forceinline__ void rank_pairs(const int* __restrict__ ids, int64_t p_begin, int64_t p_end, int k, int E,
                                           int (*cnt)[MOE_MAX_EXPERTS], int* tot, int (&myrank)[MOE_MAX_TOPK],
                                           int (&mye)[MOE_MAX_TOPK], int64_t& w_begin) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  for (int i = tid; i < DR_WAVES * E; i += DR_THREADS) cnt[i / E][i % E] = 0;
  __syncthreads();
  // each wave takes DISPATCH_TB * k / DR_WAVES = 64 * k consecutive pairs: k chunks of 64
  w_begin = p_begin + (int64_t)wave * 64 * k;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  // the ids of all k chunks in flight together, before the first ballot waits on one
  int ide[MOE_MAX_TOPK];
#pragma unroll
  for (int c = 0; c < MOE_MAX_TOPK; ++c) {
    const int64_t p = w_begin + (int64_t)c * 64 + lane;
    ide[c] = (c < k && p < p_end) ? ids[p] : -1;
  }
#pragma unroll
  for (int c = 0; c < MOE_MAX_TOPK; ++c) {
    myrank[c] = 0;
    mye[c] = -1;
    if (c < k) {
      int e = ide[c];
      if (e < 0 || e >= E) e = -1;  // out-of-range ids are ignored
      const bool valid = e >= 0;
      uint64_t same = __ballot(valid);
      for (int b = 0; b < nbits; ++b) {
        const bool bit = valid && ((e >> b) & 1);
        const uint64_t m = __ballot(bit);
        same &= bit ? m : ~m;
      }
      // one LDS atomic per distinct expert in the 64 pairs: the highest lane of each group of equal
      // ids adds the group size to the wave's counter and hands the old value to its group
      const int leader = valid ? 63 - __clzll(same) : lane;
      int old = 0;
      if (valid && lane == leader) old = atomicAdd(&cnt[wave][e], __popcll(same));
      const int base = __shfl(old, leader, 64);
      if (valid) {
        myrank[c] = base + __popcll(same & lanemask_lt());
        mye[c] = e;
      }
    }
  }
  __syncthreads();
  // exclusive scan over the waves (pair order), per expert; the workgroup total is the histogram row
  for (int e = tid; e < E; e += DR_THREADS) {
    int acc = 0;
#pragma unroll
    for (int w = 0; w < DR_WAVES; ++w) {
      const int c = cnt[w][e];
      cnt[w][e] = acc;
      acc += c;
    }
    tot[e] = acc;
  }
  __syncthreads();
}

// Counts of the whole batch (one workgroup, T <= DISPATCH_TB): count / kept / overflow, and the offsets
// (an exclusive scan of kept over experts; thread i owns experts 2i and 2i + 1, E <= 2 * DR_THREADS),
// also into s_off when non-null. write: store them to the layout.
__device__ __forceinline__ void batch_offsets(const int* tot, int E, int C, int* s_wsum, int* s_off, bool write,
                                              int* __restrict__ count, int* __restrict__ kept,
                                              int* __restrict__ overflow, int* __restrict__ offset) {
  const int e0 = 2 * threadIdx.x, e1 = e0 + 1;
  const int k0 = e0 < E ? min(tot[e0], C) : 0;
  const int k1 = e1 < E ? min(tot[e1], C) : 0;
  int total = 0;
  const int excl = block_exclusive_scan(k0 + k1, s_wsum, &total);
  if (s_off) {
    if (e0 < E) s_off[e0] = excl;
    if (e1 < E) s_off[e1] = excl + k0;
  }
  if (!write) return;
  if (e0 < E) {
    count[e0] = tot[e0];
    kept[e0] = k0;
    overflow[e0] = tot[e0] - k0;
    offset[e0] = excl;
  }
  if (e1 < E) {
    count[e1] = tot[e1];
    kept[e1] = k1;
    overflow[e1] = tot[e1] - k1;
    offset[e1] = excl + k0;
  }
  if (threadIdx.x == 0) offset[E] = total;
}

// One workgroup per DISPATCH_TB tokens: the ranks of its pairs (to pair_local) and its histogram row (to
// blk_count). SCAN (one block, T <= DISPATCH_TB): the block is the whole batch, so its per-expert bases
// are 0 and the block also writes count / kept / overflow and the expert offsets, in place of
// dispatch_scan.
template <bool SCAN>
__global__ __launch_bounds__(DR_THREADS) void dispatch_rank_kernel(const int* __restrict__ ids, int T, int k,
                                                                  int E, int* __restrict__ blk_count,
                                                                  int* __restrict__ pair_local, int C,
                                                                  int* __restrict__ count, int* __restrict__ kept,
                                                                  int* __restrict__ overflow,
                                                                  int* __restrict__ offset) {
  __shared__ int cnt[DR_WAVES][MOE_MAX_EXPERTS];
  __shared__ int s_tot[MOE_MAX_EXPERTS];
  __shared__ int s_wsum[DR_WAVES];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t p_begin = (int64_t)blockIdx.x * DISPATCH_TB * k;
  const int64_t p_end = min((int64_t)(blockIdx.x + 1) * DISPATCH_TB, (int64_t)T) * k;
  int myrank[MOE_MAX_TOPK], mye[MOE_MAX_TOPK];
  int64_t w_begin;
  rank_pairs(ids, p_begin, p_end, k, E, cnt, s_tot, myrank, mye, w_begin);
  for (int e = threadIdx.x; e < E; e += DR_THREADS) blk_count[(int64_t)(SCAN ? 0 : blockIdx.x) * E + e] = SCAN ? 0 : s_tot[e];
  if (SCAN) batch_offsets(s_tot, E, C, s_wsum, nullptr, true, count, kept, overflow, offset);
#pragma unroll
  for (int c = 0; c < MOE_MAX_TOPK; ++c) {
    if (c < k) {
      const int64_t p = w_begin + (int64_t)c * 64 + lane;
      if (p < p_end) pair_local[p] = mye[c] >= 0 ? cnt[wave][mye[c]] + myrank[c] : -1;
    }
  }
}

constexpr int DS_THREADS = 512;  // >= MOE_MAX_EXPERTS: one thread per expert

__global__ __launch_bounds__(DS_THREADS) void dispatch_scan_kernel(int* __restrict__ blk_count, int nblk, int E,
                                                                  int C, int* __restrict__ count,
                                                                  int* __restrict__ kept,
                                                                  int* __restrict__ overflow,
                                                                  int* __restrict__ offset) {
  __shared__ int wsum[DS_THREADS / MOE_WAVE];
  const int e = threadIdx.x;
  const int lane = e & 63;
  const int wave = e >> 6;
  int total = 0;
  if (e < E) {
    // 16 blocks at a time: the loads are independent, so they are all in flight together
    for (int b0 = 0; b0 < nblk; b0 += 16) {
      int c[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) c[i] = b0 + i < nblk ? blk_count[(int64_t)(b0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (b0 + i < nblk) blk_count[(int64_t)(b0 + i) * E + e] = total;  // the block's base for expert e
        total += c[i];
      }
    }
  }
  const int kp = e < E ? min(total, C) : 0;
  if (e < E) {
    count[e] = total;
    kept[e] = kp;
    overflow[e] = total - kp;
  }
  // exclusive scan of kept over experts: wave-level inclusive scan, then wave totals
  int incl = kp;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off, 64);
    if (lane >= off) incl += v;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int wbase = 0;
  for (int w = 0; w < wave; ++w) wbase += wsum[w];
  if (e < E) offset[e] = wbase + incl - kp;
  if (e == E - 1) offset[E] = wbase + incl;
}

// One wave per token, SCATTER_WAVES tokens per workgroup. Lanes j < k resolve the rows of pairs
// (t, j) and write their layout entries; the kept rows are shared through a ballot and lane reads (no
// workgroup barrier). Each lane then has VPL 16-byte column slices of x[t] in flight at once
// (lane + 64 i, one pass per 64 * VPL slices) and stores each to every kept row with non-temporal
// stores. A token whose pairs were all dropped is not read.
constexpr int SCATTER_WAVES = 4;
constexpr int FP8_SPLIT_TOKENS = 1024;

// Row of pair (t, lane) for lanes < k (-1 if dropped or not a pair), with the layout entries written
// when `write` is set.
__device__ __forceinline__ int resolve_pair_row(int t, int lane, const int* __restrict__ ids, int k, int E, int C,
                                                const int* __restrict__ blk_base, const int* __restrict__ pair_local,
                                                const int* __restrict__ offset, int* __restrict__ row_token,
                                                int* __restrict__ row_slot, int* __restrict__ pair_row,
                                                bool write = true) {
  int row = -1;
  if (lane < k) {
    const int64_t p = (int64_t)t * k + lane;
    const int e = ids[p];
    const int local = pair_local[p];
    if (e >= 0 && e < E && local >= 0) {
      const int pos = blk_base[(int64_t)(t / DISPATCH_TB) * E + e] + local;
      if (pos < C) row = offset[e] + pos;
    }
    if (write) {
      pair_row[p] = row;
      if (row >= 0) {
        row_token[row] = t;
        row_slot[row] = lane;
      }
    }
  }
  return row;
}

// One wave copies token row t of x to the kept rows (lane j < k holds the row of pair (t, j), -1 if
// dropped): VPL 16-byte slices per lane in flight, each read once and stored to every kept row. The
// stores use the default cache policy: a wave writes whole rows, and non-temporal stores of this
// pattern were slower (16384 tokens x 7168, 67528 kept rows: 213 -> 193 us; 4096 x 7168 to 32768
// rows: 97 -> 78 us).
template <typename T, int VPL>
__device__ __forceinline__ void copy_token_row(const T* __restrict__ x, int t, int H, int row,
                                               T* __restrict__ send_buf) {
  const int lane = lane_id();
  uint64_t kept = __ballot(row >= 0);  // only lanes < k can hold a row
  if (kept == 0) return;               // every pair of this token was dropped: nothing to copy
  constexpr int VN = Vec<T>::N;
  const int nvec = H / VN;
  const T* src = x + (int64_t)t * H;
  for (int base = 0; base < nvec; base += 64 * VPL) {
    u32x4 val[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int v = base + lane + i * 64;
      if (v < nvec) val[i] = ld16(src + (int64_t)v * VN);
    }
    for (uint64_t m = kept; m; m &= m - 1) {
      const int j = __builtin_ctzll(m);
      T* dst = send_buf + (int64_t)__shfl(row, j, 64) * H;
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const int v = base + lane + i * 64;
        if (v < nvec) st16(dst + (int64_t)v * VN, val[i]);
      }
    }
  }
}

template <typename T, int VPL>
__global__ __launch_bounds__(SCATTER_WAVES * 64) void dispatch_scatter_kernel(
    const T* __restrict__ x, const int* __restrict__ ids, int T_, int H, int k, int E, int C,
    const int* __restrict__ blk_base, const int* __restrict__ pair_local, const int* __restrict__ offset,
    int* __restrict__ row_token, int* __restrict__ row_slot, int* __restrict__ pair_row, T* __restrict__ send_buf) {
  const int t = blockIdx.x * SCATTER_WAVES + (int)(threadIdx.x >> 6);
  if (t >= T_) return;
  const int row =
      resolve_pair_row(t, lane_id(), ids, k, E, C, blk_base, pair_local, offset, row_token, row_slot, pair_row);
  copy_token_row<T, VPL>(x, t, H, row, send_buf);
}

// The whole dispatch in one launch for a batch of at most DISPATCH_TB tokens: every workgroup ranks all
// pairs and scans the counts itself (the work of the one-block dispatch_rank, repeated per workgroup, in
// LDS), workgroup 0 writes count / kept / overflow / offsets, and then each wave scatters one token as
// dispatch_scatter does. This saves a launch and its dependent global round trips on decode batches.
template <typename T, int VPL>
__global__ __launch_bounds__(DR_THREADS) void dispatch_small_kernel(
    const T* __restrict__ x, const int* __restrict__ ids, int T_, int H, int k, int E, int C, int* __restrict__ count,
    int* __restrict__ kept, int* __restrict__ overflow, int* __restrict__ offset, int* __restrict__ row_token,
    int* __restrict__ row_slot, int* __restrict__ pair_row, T* __restrict__ send_buf) {
  static_assert(DR_THREADS == SCATTER_WAVES * 64, "one wave per token");
  __shared__ int cnt[DR_WAVES][MOE_MAX_EXPERTS];
  __shared__ int s_tot[MOE_MAX_EXPERTS];
  __shared__ int s_off[MOE_MAX_EXPERTS];
  __shared__ int s_wsum[DR_WAVES];
  __shared__ int s_pos[DISPATCH_TB * MOE_MAX_TOPK];  // pair -> position in its expert, -1: no expert
  __shared__ int s_exp[DISPATCH_TB * MOE_MAX_TOPK];  // pair -> expert, -1: out of range
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t n_pairs = (int64_t)T_ * k;
  int myrank[MOE_MAX_TOPK], mye[MOE_MAX_TOPK];
  int64_t w_begin;
  rank_pairs(ids, 0, n_pairs, k, E, cnt, s_tot, myrank, mye, w_begin);
  batch_offsets(s_tot, E, C, s_wsum, s_off, blockIdx.x == 0, count, kept, overflow, offset);
#pragma unroll
  for (int c = 0; c < MOE_MAX_TOPK; ++c) {
    if (c < k) {
      const int64_t p = w_begin + (int64_t)c * 64 + lane;
      if (p < n_pairs) {
        s_pos[p] = mye[c] >= 0 ? cnt[wave][mye[c]] + myrank[c] : -1;
        s_exp[p] = mye[c];
      }
    }
  }
  __syncthreads();
  const int t = blockIdx.x * SCATTER_WAVES + wave;
  if (t >= T_) return;
  int row = -1;
  if (lane < k) {
    const int p = t * k + lane;
    const int e = s_exp[p], pos = s_pos[p];
    if (e >= 0 && pos < C) row = s_off[e] + pos;
    pair_row[p] = row;
    if (row >= 0) {
      row_token[row] = t;
      row_slot[row] = lane;
    }
  }
  copy_token_row<T, VPL>(x, t, H, row, send_buf);
}

template <typename T, int VPL>
void launch_scatter_t(const void* x, const int* ids, const moe_layout_t& L, void* send_buf, const int* blk_base,
                      const int* pair_local, hipStream_t stream) {
  const unsigned blocks = (unsigned)ceil_div_host(L.T, SCATTER_WAVES);
  dispatch_scatter_kernel<T, VPL><<<blocks, SCATTER_WAVES * 64, 0, stream>>>(
      static_cast<const T*>(x), ids, L.T, L.H, L.k, L.E, L.C, blk_base, pair_local, L.expert_offset, L.row_token,
      L.row_slot, L.pair_row, static_cast<T*>(send_buf));
}

// ---- fp8 block-scaled rows ----
// OCP E4M3 codes of four values |y| <= 448, packed little-endian: v_cvt_pk_fp8_f32 rounds to the nearest
// E4M3 value, ties to the even mantissa, and keeps the sign of a value that rounds to zero (gfx950
// writes OCP E4M3).
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// Exponent E of the block scale: the smallest integer with amax / 2^E <= 448. With amax = f * 2^fe,
// f in [0.5, 1), amax / 448 = (f / 0.875) * 2^(fe - 9), and f / 0.875 is in (0.5, 1] iff f <= 0.875.
__device__ __forceinline__ int e4m3_block_exp(float amax) {
  if (amax == 0.0f) return 0;
  int fe;
  const float f = frexpf(amax, &fe);
  return fe - 9 + (f > 0.875f ? 1 : 0);
}

// One wave per (token, row segment): blockIdx.y picks the segment, gridDim.y segments split the row
// (one segment when there are tokens enough to fill the GPU; with few tokens the encoding work of a row
// is spread over more waves), and only segment 0 writes the layout entries. A pass covers 64 * VPL
// 16-byte chunks of 8 bf16 values; a 128-element block is 16 chunks held by 16 consecutive lanes, which
// find the block maximum with shuffles. Each lane stores its 8 codes (8 bytes) to every kept row; the
// block's first lane stores the scale.
template <int VPL>
__global__ __launch_bounds__(SCATTER_WAVES * 64) void dispatch_scatter_fp8_kernel(
    const bf16_t* __restrict__ x, const int* __restrict__ ids, int T_, int H, int k, int E, int C,
    const int* __restrict__ blk_base, const int* __restrict__ pair_local, const int* __restrict__ offset,
    int* __restrict__ row_token, int* __restrict__ row_slot, int* __restrict__ pair_row, uint8_t* __restrict__ send_q,
    float* __restrict__ send_scale) {
  const int lane = lane_id();
  const int t = blockIdx.x * SCATTER_WAVES + (int)(threadIdx.x >> 6);
  if (t >= T_) return;
  const int row = resolve_pair_row(t, lane, ids, k, E, C, blk_base, pair_local, offset, row_token, row_slot, pair_row,
                                   blockIdx.y == 0);
  const uint64_t kept = __ballot(row >= 0);
  if (kept == 0) return;
  const int nvec = H / 8;  // H % 128 == 0, so every pass holds whole blocks
  const int nblk = H / 128;
  const bf16_t* src = x + (int64_t)t * H;
  for (int base = blockIdx.y * 64 * VPL; base < nvec; base += gridDim.y * 64 * VPL) {
    u32x4 val[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int v = base + lane + i * 64;
      if (v < nvec) val[i] = ld16(src + (int64_t)v * 8);
    }
    u32x2 q[VPL];
    float sc[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int v = base + lane + i * 64;
      float f[8];
      unpack(v < nvec ? val[i] : u32x4{0u, 0u, 0u, 0u}, f);
      float am = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) am = fmaxf(am, fabsf(f[j]));
      // block maximum over the 16 lanes of this block (lane groups of 16 are aligned: base % 64 == 0)
#pragma unroll
      for (int off = 8; off > 0; off >>= 1) am = fmaxf(am, __shfl_xor(am, off, 64));
      const int E8 = e4m3_block_exp(am);
      sc[i] = ldexpf(1.0f, E8);
      float y[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) y[j] = ldexpf(f[j], -E8);  // exact scaling by 2^-E, |y| <= 448
      q[i].x = e4m3x4(y[0], y[1], y[2], y[3]);
      q[i].y = e4m3x4(y[4], y[5], y[6], y[7]);
    }
    for (uint64_t m = kept; m; m &= m - 1) {
      const int j = __builtin_ctzll(m);
      const int r = __shfl(row, j, 64);
      uint8_t* dq = send_q + (int64_t)r * H;
      float* ds = send_scale + (int64_t)r * nblk;
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const int v = base + lane + i * 64;
        if (v < nvec) {
          *reinterpret_cast<u32x2*>(dq + (int64_t)v * 8) = q[i];  // default policy, as in copy_token_row
          if ((lane & 15) == 0) ds[v >> 4] = sc[i];
        }
      }
    }
  }
}

}  // namespace

int dispatch_num_blocks(int T) { return ceil_div_host(T, DISPATCH_TB); }

// histogram + scan: the per-block ranks, counts, kept / overflow and offsets
static hipError_t launch_counts(const int* ids, const moe_layout_t& L, int* blk_count, int* pair_local,
                                hipStream_t stream) {
  const int nblk = dispatch_num_blocks(L.T);
  if (nblk == 1) {  // one block: it scans too
    dispatch_rank_kernel<true><<<1, DR_THREADS, 0, stream>>>(ids, L.T, L.k, L.E, blk_count, pair_local, L.C,
                                                             L.expert_count, L.expert_kept, L.expert_overflow,
                                                             L.expert_offset);
  } else {
    if (nblk > 0)
      dispatch_rank_kernel<false><<<nblk, DR_THREADS, 0, stream>>>(ids, L.T, L.k, L.E, blk_count, pair_local, L.C,
                                                                   nullptr, nullptr, nullptr, nullptr);
    // with no tokens the scan still writes zero counts and offsets
    dispatch_scan_kernel<<<1, DS_THREADS, 0, stream>>>(blk_count, nblk, L.E, L.C, L.expert_count, L.expert_kept,
                                                       L.expert_overflow, L.expert_offset);
  }
  return hipGetLastError();
}

hipError_t launch_dispatch(const void* x, int xdt_bf16, const int* ids, const moe_layout_t& L, void* send_buf,
                           int* blk_count, int* pair_local, hipStream_t stream) {
  // slices per lane in flight: enough for the whole row in one pass up to 1024 slices (bf16 H <= 8192)
  const int nvec = L.H / (xdt_bf16 ? 8 : 4);
  const int vpl = nvec > 256 ? 16 : (nvec > 64 ? 4 : 1);
  if (L.T > 0 && dispatch_num_blocks(L.T) == 1) {  // one launch: every workgroup ranks the whole batch
    const unsigned blocks = (unsigned)ceil_div_host(L.T, SCATTER_WAVES);
#define MOE_DISPATCH_SMALL(TY, VPL)                                                                         \
  dispatch_small_kernel<TY, VPL><<<blocks, DR_THREADS, 0, stream>>>(                                         \
      static_cast<const TY*>(x), ids, L.T, L.H, L.k, L.E, L.C, L.expert_count, L.expert_kept, L.expert_overflow, \
      L.expert_offset, L.row_token, L.row_slot, L.pair_row, static_cast<TY*>(send_buf))
    if (xdt_bf16) {
      if (vpl == 16) MOE_DISPATCH_SMALL(bf16_t, 16);
      else if (vpl == 4) MOE_DISPATCH_SMALL(bf16_t, 4);
      else MOE_DISPATCH_SMALL(bf16_t, 1);
    } else {
      if (vpl == 16) MOE_DISPATCH_SMALL(float, 16);
      else if (vpl == 4) MOE_DISPATCH_SMALL(float, 4);
      else MOE_DISPATCH_SMALL(float, 1);
    }
#undef MOE_DISPATCH_SMALL
    return hipGetLastError();
  }
  const hipError_t st = launch_counts(ids, L, blk_count, pair_local, stream);
  if (st != hipSuccess || L.T == 0) return st;
  if (xdt_bf16) {
    if (vpl == 16) launch_scatter_t<bf16_t, 16>(x, ids, L, send_buf, blk_count, pair_local, stream);
    else if (vpl == 4) launch_scatter_t<bf16_t, 4>(x, ids, L, send_buf, blk_count, pair_local, stream);
    else launch_scatter_t<bf16_t, 1>(x, ids, L, send_buf, blk_count, pair_local, stream);
  } else {
    if (vpl == 16) launch_scatter_t<float, 16>(x, ids, L, send_buf, blk_count, pair_local, stream);
    else if (vpl == 4) launch_scatter_t<float, 4>(x, ids, L, send_buf, blk_count, pair_local, stream);
    else launch_scatter_t<float, 1>(x, ids, L, send_buf, blk_count, pair_local, stream);
  }
  return hipGetLastError();
}

hipError_t launch_dispatch_fp8(const void* x, const int* ids, const moe_layout_t& L, uint8_t* send_q,
                               float* send_scale, int* blk_count, int* pair_local, hipStream_t stream) {
  const hipError_t st = launch_counts(ids, L, blk_count, pair_local, stream);
  if (st != hipSuccess || L.T == 0) return st;
  const int nvec = L.H / 8;
  const unsigned blocks = (unsigned)ceil_div_host(L.T, SCATTER_WAVES);
  // with fewer tokens than FP8_SPLIT_TOKENS, segments of 64 chunks (one per lane) split each row
  const bool split = L.T < FP8_SPLIT_TOKENS;
  const dim3 grid(blocks, split ? (unsigned)std::min(ceil_div_host(nvec, 64), 65535) : 1u);  // y stride covers the rest
#define MOE_SCATTER_FP8(VPL)                                                                                 \
  dispatch_scatter_fp8_kernel<VPL><<<grid, SCATTER_WAVES * 64, 0, stream>>>(                                \
      static_cast<const bf16_t*>(x), ids, L.T, L.H, L.k, L.E, L.C, blk_count, pair_local, L.expert_offset,       \
      L.row_token, L.row_slot, L.pair_row, send_q, send_scale)
  if (split || nvec <= 64) MOE_SCATTER_FP8(1);
  else if (nvec > 256) MOE_SCATTER_FP8(16);
  else MOE_SCATTER_FP8(4);
#undef MOE_SCATTER_FP8
  return hipGetLastError();
}

}  // namespace moe
