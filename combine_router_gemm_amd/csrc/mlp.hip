// Expert SwiGLU MLP as a persistent grouped GEMM over every local expert.
//
// The dispatched rows are multiplied by the expert weights with grouped GEMM kernels ("Enabling
// trillion-parameter models on AWS EFA", section "MoE all-to-all через EFA"); one persistent GEMM
// processes every expert of the rank without relaunching ("Mixture-of-experts acceleration through
// overlap"). A row of global expert e uses local expert l = e mod El: the R rank segments of the send
// buffer each hold rows for every local expert, and one GPU's share runs them all against its El weight
// sets.
//
// Kernels:
//   mlp_plan      M_l = sum_r kept[r*El + l]; prefix sums give each local expert's first row in "plan
//                 order" (local expert major, then rank segment, then token) and its first M-tile;
//                 perm[p] = send-buffer row of plan row p. Every workgroup recomputes the small scans
//                 and fills perm for its own slice of rows. Everything the GEMMs need is derived on the
//                 device from the dispatch counts: no host synchronisation.
//   mlp_gemm      persistent MFMA GEMM, C[p, n] = sum_k A[p, k] * B[n, k] ("NT": both operands are
//                 K-contiguous, the nn.Linear [out, in] layout). Tiles are visited local expert major,
//                 then N tile, then M tile, so workgroups running side by side share a weight slice;
//                 the tile list is cut into 8 equal contiguous ranges, one per XCD (workgroups are dealt
//                 to the 8 XCDs round robin, and each XCD has its own L2).
//                 Gate/up pass: A rows gathered through perm from the send buffer, B = the gate and the
//                 up rows of the same output columns, epilogue h = silu(g) * u (fp32) stored as xdt.
//                 Down pass: A = h in plan order, epilogue stores to out_buf[perm[p]] as xdt.
//   Two kernel families share that structure:
//     mlp_gemm_kernel     operands staged global -> registers -> LDS (buffer loads, several register
//                         stages in flight). Few rows per expert (weight streaming, 32- or 64-row tiles
//                         on v_mfma_f32_16x16x32_bf16), fp32 (v_mfma_f32_16x16x4_f32), and the bf16
//                         fallback for shapes the other family does not take.
//     mlp_gemm_dl_kernel  many rows per expert: operands go global -> LDS directly (buffer loads with
//                         the LDS bit), NS LDS stages in flight, 128-row tiles on
//                         v_mfma_f32_32x32x16_bf16, epilogue staged through LDS.
//     mlp_gemm_xs_kernel  the same loads for 320-row tiles that hold a whole expert: two stage slots,
//                         loads interleaved with the MFMAs, the next tile's first stage prefetched.
//     mlp_gemm_pp_kernel  256-row tiles for experts of 1024+ rows: two wave groups alternate between
//                         loading and multiplying (ping-pong).
//   All accumulate in fp32.
//   fp8_rows_to_bf16  fp8 block-scaled send rows (E4M3 codes + power-of-two scales) expanded to bf16 in
//                     out_buf before the GEMMs, which then read them like bf16 rows.
//   COMBINE           the down pass of either family with the combine fused in: each tile counts its
//                     rows per (token, column band) and the tile completing a band combines it
//                     (tile_arrive_combine; combine_prep clears the counters first).
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "mfma.h"

namespace moe {

namespace {

// ------------------------------------------------------------------------------------------------
// plan
// ------------------------------------------------------------------------------------------------
// plan layout (int32): [0] total M-tiles, [1] total rows, [2 .. 2+El] row start per local expert
// (El+1 entries), [3+El .. 3+2El] M-tile start per local expert (El+1 entries), then kSplitSlots counters
// of the K-split tail tiles of the whole-expert gate/up GEMM, zeroed by the plan kernel before every GEMM.
constexpr int PLAN_THREADS = 1024;  // >= MOE_MAX_EXPERTS: one thread per (local or global) expert
constexpr int kSplitSlots = 512;
constexpr int PLAN_ROWS_PER_WG = 4096;

__global__ __launch_bounds__(PLAN_THREADS) void mlp_plan_kernel(const int* __restrict__ kept,
                                                               const int* __restrict__ offset, int E, int El,
                                                               int BM, int* __restrict__ plan,
                                                               int* __restrict__ perm) {
  __shared__ int s_rows[MOE_MAX_EXPERTS + 1];   // per local expert: first plan row (exclusive scan)
  __shared__ int s_tiles[MOE_MAX_EXPERTS + 1];  // per local expert: first M-tile
  __shared__ int s_kept[MOE_MAX_EXPERTS];
  __shared__ int s_off[MOE_MAX_EXPERTS + 1];
  __shared__ int s_dst[MOE_MAX_EXPERTS];        // per global expert: first plan row
  __shared__ int s_wsum[2][PLAN_THREADS / MOE_WAVE];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int R = E / El;
  if (tid < E) {
    s_kept[tid] = kept[tid];
    s_off[tid] = offset[tid];
  }
  __syncthreads();
  int m = 0, tl = 0;
  if (tid < El) {
    for (int r = 0; r < R; ++r) m += s_kept[r * El + tid];
    tl = (m + BM - 1) / BM;
  }
  // exclusive scan of (rows, tiles) over local experts: wave scans, then wave totals
  int im = m, it = tl;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int vm = __shfl_up(im, off, 64), vt = __shfl_up(it, off, 64);
    if (lane >= off) {
      im += vm;
      it += vt;
    }
  }
  if (lane == 63) {
    s_wsum[0][wave] = im;
    s_wsum[1][wave] = it;
  }
  __syncthreads();
  int bm = 0, bt = 0;
  for (int w = 0; w < wave; ++w) {
    bm += s_wsum[0][w];
    bt += s_wsum[1][w];
  }
  if (tid < El) {
    s_rows[tid] = bm + im - m;
    s_tiles[tid] = bt + it - tl;
  }
  if (tid == El - 1) {
    s_rows[El] = bm + im;
    s_tiles[El] = bt + it;
    if (blockIdx.x == 0) {
      plan[0] = bt + it;
      plan[1] = bm + im;
    }
  }
  __syncthreads();
  int* row_start = plan + 2;
  int* tile_start = plan + 3 + El;
  if (blockIdx.x == 0 && tid <= El) {
    row_start[tid] = s_rows[tid];
    tile_start[tid] = s_tiles[tid];
  }
  if (blockIdx.x == 0)
    for (int i = tid; i < kSplitSlots; i += PLAN_THREADS) plan[4 + 2 * El + i] = 0;
  // global expert e = r*El + l lands after the rows of experts l, El + l, ..., (r-1)*El + l
  if (tid < E) {
    const int l = tid % El, r = tid / El;
    int dst = s_rows[l];
    for (int rr = 0; rr < r; ++rr) dst += s_kept[rr * El + l];
    s_dst[tid] = dst;
  }
  if (tid == 0) s_off[E] = offset[E];
  __syncthreads();
  // perm[p] = send-buffer row of plan row p. Workgroup b handles send-buffer rows
  // [b * PLAN_ROWS_PER_WG, (b + 1) * PLAN_ROWS_PER_WG): the expert of row q is found by a binary search
  // over the offsets, and q goes to its expert's plan range.
  const int total = s_off[E];
  const int q_end = min(total, (int)((blockIdx.x + 1) * PLAN_ROWS_PER_WG));
  for (int q = blockIdx.x * PLAN_ROWS_PER_WG + tid; q < q_end; q += PLAN_THREADS) {
    int lo = 0, hi = E;  // invariant: s_off[lo] <= q < s_off[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_off[mid] <= q) lo = mid;
      else hi = mid;
    }
    perm[s_dst[lo] + (q - s_off[lo])] = q;
  }
}

// ------------------------------------------------------------------------------------------------
// GEMM
// ------------------------------------------------------------------------------------------------
__device__ __forceinline__ float silu_f32(float g) { return g / (1.0f + expf(-g)); }

constexpr bool kKRotate = true;


struct GemmArgs {
  const void* A;        // activations: send_buf (gate/up) or h (down)
  int lda;              // row length of A (= K)
  const int* a_perm;    // gather map for A rows (gate/up) or nullptr (A in plan order)
  const void* W;        // [El, ...] expert weights
  int64_t w_stride;     // elements per expert
  int K;
  int N;                // output columns per expert (F for gate/up, H for down)
  int up_offset;        // gate/up: row offset of the up half inside an expert's weights (= F)
  void* Out;
  int ldo;
  const int* out_perm;  // scatter map for output rows (down) or nullptr (plan order)
  const int* plan;       // the plan kernel's output, or nullptr: build the plan from `offset` (R = 1)
  const int* offset;     // [E + 1] the layout's expert offsets (used when plan is nullptr)
  int El;
  int a_bytes;          // bytes of A (rows_max x lda elements) when it fits 31-bit buffer offsets, else 0
  int w_bytes;          // bytes of one expert's weights (w_stride elements), same rule
  int k_rotate;         // start each tile's K loop at a tile-dependent stage (see k_rotation)
  // down GEMM with the combine fused in (see tile_arrive_combine); unused otherwise
  const int* row_token;  // [rows] token of each send row
  const int* pair_row;   // [T, k] send row of each (token, slot), -1 if dropped
  const float* topk_w;   // [T, k] routing weights
  int* counter;          // [T, column bands] rows of the token finished per band (zeroed before the GEMM)
  void* y;               // [T, N] combine output
  int k;
  int out_bytes;         // bytes of Out when 31-bit buffer offsets cover it, else 0
  int* split_ctr;        // gate/up: kSplitSlots zeroed counters for the K-split tail tiles, or nullptr
};

// Eight OCP E4M3 codes (q.x, q.y, little-endian bytes) times their block scale sc (a power of two) as
// eight bf16 values. v_cvt_pk_f32_fp8 decodes two codes exactly (gfx950 reads them as OCP E4M3); code *
// scale has at most 4 significant bits, so the product and its bf16 rounding are exact.
__device__ __forceinline__ u32x4 e4m3x8_to_bf16(uint32_t qx, uint32_t qy, float sc) {
  float f[8];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t w = h ? qy : qx;
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
    f[4 * h + 0] = lo.x * sc;
    f[4 * h + 1] = lo.y * sc;
    f[4 * h + 2] = hi.x * sc;
    f[4 * h + 3] = hi.y * sc;
  }
  return pack(f);
}

// fp8 rows (E4M3 codes with one power-of-two scale per 128 elements) expanded to bf16 rows, for GEMM
// tiles that load their A operand straight into LDS. A chunk is 16 codes at flat index 16 c of the first
// *total_rows rows; with H % 128 == 0 the flat index / 128 is also the flat index of the block's scale
// in [rows, H / 128]. Each thread expands FP8_EXPAND_CHUNKS chunks, all loads issued before any store.
constexpr int FP8_EXPAND_CHUNKS = 4;
__global__ __launch_bounds__(256) void fp8_rows_to_bf16_kernel(const uint8_t* __restrict__ q,
                                                               const float* __restrict__ scale,
                                                               const int* __restrict__ total_rows, int H,
                                                               bf16_t* __restrict__ out) {
  const int64_t n = (int64_t)(*total_rows) * (H / 16);
  const int64_t c0 = (int64_t)blockIdx.x * (256 * FP8_EXPAND_CHUNKS) + threadIdx.x;
  if (c0 >= n) return;
  u32x4 c[FP8_EXPAND_CHUNKS];
  float sc[FP8_EXPAND_CHUNKS];
#pragma unroll
  for (int u = 0; u < FP8_EXPAND_CHUNKS; ++u) {
    const int64_t ci = c0 + u * 256;
    if (ci < n) {
      c[u] = ld16_nt(q + ci * 16);
      sc[u] = scale[ci >> 3];
    }
  }
#pragma unroll
  for (int u = 0; u < FP8_EXPAND_CHUNKS; ++u) {
    const int64_t ci = c0 + u * 256;
    if (ci < n) {
      st16(out + ci * 16, e4m3x8_to_bf16(c[u].x, c[u].y, sc[u]));
      st16(out + ci * 16 + 8, e4m3x8_to_bf16(c[u].z, c[u].w, sc[u]));
    }
  }
}

// Weight rows whose pitch is a multiple of 4 KB put the same K slice of every row of a tile on the same
// few HBM channels while all tiles walk K in step: a read probe of the weight-streaming tile pattern
// measured 5.4 TB/s at an 8192-byte pitch against 6.0 TB/s at 8448 bytes, and rotating each tile's
// starting stage recovers it (the 28 KB rows of Mixtral's down weights: 3-4 % faster). Tiles that share
// weights (the M tiles of one expert and N tile) get the same rotation, so they keep sharing them
// through L2.
constexpr int kKRotStride = 7;
__device__ __forceinline__ int k_rotation(int on, int l, int n_tiles, int nt, int nk) {
  return on ? (int)(((int64_t)l * n_tiles + nt) * kKRotStride % nk) : 0;
}
inline int k_rotate_for(int K, int elem_bytes) { return kKRotate && ((int64_t)K * elem_bytes) % 4096 == 0; }

// The plan's per-expert row and M-tile starts in LDS (row_start[0..El], tile_start[0..El]), by every
// workgroup of NTH threads; returns the number of M tiles. With a plan they are copied from it. Without
// one (one rank: the send rows are already grouped by expert, so plan order is send order and the row
// map is the identity) they are built from the layout's expert offsets: row_start = offset and
// tile_start = the exclusive scan of ceil(rows / BM), each thread taking a run of consecutive experts.
template <int NTH>
__device__ __forceinline__ int load_plan(const GemmArgs& args, int BM, int* row_start, int* tile_start) {
  static_assert(NTH % 64 == 0 && NTH <= 1024, "whole waves");
  const int El = args.El, tid = threadIdx.x;
  if (args.plan) {
    for (int i = tid; i <= El; i += NTH) {
      row_start[i] = args.plan[2 + i];
      tile_start[i] = args.plan[3 + El + i];
    }
    __syncthreads();
    return args.plan[0];
  }
  __shared__ int s_wsum[NTH / 64];
  const int lane = tid & 63, wave = tid >> 6;
  const int per = (El + NTH - 1) / NTH, e0 = tid * per;
  int sum = 0;
  for (int i = 0; i < per; ++i) {
    const int e = e0 + i;
    if (e < El) {
      const int a = args.offset[e];
      row_start[e] = a;
      sum += (args.offset[e + 1] - a + BM - 1) / BM;
    }
  }
  int incl = sum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int u = __shfl_up(incl, off, 64);
    if (lane >= off) incl += u;
  }
  if (lane == 63) s_wsum[wave] = incl;
  __syncthreads();
  int run = incl - sum, total = 0;
#pragma unroll
  for (int w = 0; w < NTH / 64; ++w) {
    if (w < wave) run += s_wsum[w];
    total += s_wsum[w];
  }
  for (int i = 0; i < per; ++i) {
    const int e = e0 + i;
    if (e < El) {
      tile_start[e] = run;
      run += (args.offset[e + 1] - row_start[e] + BM - 1) / BM;
    }
  }
  if (tid == 0) {
    row_start[El] = args.offset[El];
    tile_start[El] = total;
  }
  __syncthreads();
  return total;
}

// ---- the combine fused into the down GEMM ----
// Expert-output rows that another tile combines travel through agent-scope (sc1) loads and stores: they
// are coherent across the XCDs' L2 caches by themselves, so no cache-wide writeback or invalidate is
// needed, and the L2 keeps the operands the other workgroups are reusing.
__device__ __forceinline__ u32x4 ld16_agent(const void* p) {
  const uint64_t* q = static_cast<const uint64_t*>(p);
  const uint64_t a = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t b = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return u32x4{(uint32_t)a, (uint32_t)(a >> 32), (uint32_t)b, (uint32_t)(b >> 32)};
}
// 16-byte agent-scope (sc1) buffer accesses, where the buffer fits 31-bit offsets
__device__ __forceinline__ u32x4 ld16_agent(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 16));
}
__device__ __forceinline__ void st16_agent(__amdgpu_buffer_rsrc_t r, int off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 16);
}
__device__ __forceinline__ void st_agent(bf16_t* p, float v) {
  const bf16_t h = (bf16_t)v;
  __hip_atomic_store(reinterpret_cast<uint16_t*>(p), __builtin_bit_cast(uint16_t, h), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(float* p, float v) {
  __hip_atomic_store(reinterpret_cast<uint32_t*>(p), __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Tile-level overlap of the grouped GEMM with the combine: once a down-GEMM tile has stored its rows
// (columns [n0, n0 + OUT_COLS) of some tokens' expert outputs), it counts them per (token, column band).
// The tile that brings a token's count to its number of kept slots holds the last missing piece of that
// band, and combines it at once: y[t, band] = sum over kept slots j, ascending, of w[t, j] * out[row_j],
// fp32, rounded once (the combine's own arithmetic, so the result equals moe_combine's bit for bit).
// The combine of early bands thus runs while later tiles are still being computed. Nothing ever waits:
// a workgroup either finishes a band or leaves it to the tile that will.
// Ordering between the tile that stores rows and the tile that combines them. Every access to the shared
// rows is an agent-scope atomic access (sc1: stores write through to, and loads read from, the level that
// is coherent across the XCDs' L2 caches), and the counters are agent-scope atomic adds. In the gfx942 /
// gfx950 code sequences of the LLVM AMDGPU memory model, an agent-scope release is "buffer_wbl2 sc1;
// s_waitcnt vmcnt(0)" before the releasing operation and an acquire is "s_waitcnt vmcnt(0); buffer_inv sc1"
// after the acquiring one. The cache writeback and invalidate exist for non-atomic accesses, which may sit
// in a non-coherent L2; accesses made with sc1 never do, so for these rows the release reduces to its wait
// and the acquire to issuing the later loads after the acquiring operation has returned. Both are here:
// every thread waits (vmcnt(0)) until its row stores are complete before the workgroup barrier that
// precedes the counter adds, and the combining tile issues its sc1 row loads only after the add that
// returned the last count (its result decides, through LDS and a barrier, which tokens are combined).
// The L2 writeback and invalidate of a full release / acquire per tile cost more than twice the down
// GEMM's time when they were tried (they discard the operands the other workgroups are reusing).
// LDS: s_list holds at least BM + 1 ints and is free on entry.
template <typename T, int NTH, int OUT_COLS>
__device__ __forceinline__ void tile_arrive_combine(const GemmArgs& a, int p0, int m_rows, int n0, int nt,
                                                    int n_bands, int* s_list) {
  constexpr int VN = Vec<T>::N;
  const int tid = threadIdx.x;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this thread's rows have reached the coherent level
  if (tid == 0) s_list[0] = 0;
  __syncthreads();
  for (int r = tid; r < m_rows; r += NTH) {
    const int p = p0 + r;
    const int orow = a.out_perm ? a.out_perm[p] : p;
    const int t = a.row_token[orow];
    int kept = 0;
    for (int j = 0; j < a.k; ++j) kept += a.pair_row[(int64_t)t * a.k + j] >= 0 ? 1 : 0;
    const int old = atomicAdd(&a.counter[(int64_t)t * n_bands + nt], 1);
    if (old == kept - 1) s_list[1 + atomicAdd(&s_list[0], 1)] = t;
  }
  __syncthreads();
  const int n = s_list[0];
  if (n > 0) {
    const T* out = static_cast<const T*>(a.Out);
    const __amdgpu_buffer_rsrc_t out_rsrc = __builtin_amdgcn_make_buffer_rsrc(a.Out, (short)0, a.out_bytes, 0x00020000);
    T* y = static_cast<T*>(a.y);
    const int cpb = (min(OUT_COLS, a.N - n0) + VN - 1) / VN;  // 16-byte chunks of the band (N % VN == 0)
    for (int idx = tid; idx < n * cpb; idx += NTH) {
      const int t = s_list[1 + idx / cpb];
      const int col = n0 + (idx % cpb) * VN;
      // all k rows in flight at once, then the sum in slot order
      int rows[MOE_MAX_TOPK];
      u32x4 raw[MOE_MAX_TOPK];
#pragma unroll
      for (int j = 0; j < MOE_MAX_TOPK; ++j) rows[j] = j < a.k ? a.pair_row[(int64_t)t * a.k + j] : -1;
#pragma unroll
      for (int j = 0; j < MOE_MAX_TOPK; ++j)
        raw[j] = rows[j] < 0 ? u32x4{0u, 0u, 0u, 0u}
                 : a.out_bytes > 0 ? ld16_agent(out_rsrc, (rows[j] * a.ldo + col) * (int)sizeof(T))
                                   : ld16_agent(out + (int64_t)rows[j] * a.ldo + col);
      float acc[VN];
#pragma unroll
      for (int q = 0; q < VN; ++q) acc[q] = 0.f;
#pragma unroll
      for (int j = 0; j < MOE_MAX_TOPK; ++j) {
        if (rows[j] >= 0) {
          const float w = a.topk_w[(int64_t)t * a.k + j];
          float val[VN];
          unpack(raw[j], val);
#pragma unroll
          for (int q = 0; q < VN; ++q) acc[q] = fmaf(w, val[q], acc[q]);
        }
      }
      st16(y + (int64_t)t * a.N + col, pack(acc));
    }
  }
  __syncthreads();  // s_list is free again before the next tile reuses the buffers
}

// Before a GEMM with the fused combine: zero the per-(token, band) counters, and write y = 0 for the
// tokens with no kept slot (no tile ever completes them). One thread per counter / per 16-byte chunk.
template <typename T>
__global__ __launch_bounds__(256) void combine_prep_kernel(const int* __restrict__ pair_row, int T_, int k, int H,
                                                           int n_bands, int* __restrict__ counter,
                                                           T* __restrict__ y) {
  constexpr int VN = Vec<T>::N;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t ncnt = (int64_t)T_ * n_bands;
  if (i < ncnt) counter[i] = 0;
  const int cpr = H / VN;
  if (i < (int64_t)T_ * cpr) {
    const int t = (int)(i / cpr);
    bool any = false;
    for (int j = 0; j < k; ++j) any = any || pair_row[(int64_t)t * k + j] >= 0;
    if (!any) st16(y + (int64_t)t * H + (i % cpr) * VN, u32x4{0u, 0u, 0u, 0u});
  }
}

// BM x BN tile, BK-deep LDS stages, WM x WN waves, MFMA op Op. GATED: the B tile holds BN/2 gate rows
// then the BN/2 up rows of the same output columns, and each wave owns matching gate and up
// accumulators.
template <typename T, typename Op, int BM, int BN, int BK, int WM, int WN, bool GATED, int RS, int LDB, bool BNT,
          bool BUF, bool COMBINE>
struct RegTile {
  static constexpr int NTH = WM * WN * 64;
  static constexpr int VN = Vec<T>::N;           // elements per 16-byte vector
  static constexpr int PAD = 16 / sizeof(T);     // one vector of padding per LDS row
  static constexpr int LDR = BK + PAD;           // LDS row length (elements)
  static constexpr int VPR = BK / VN;            // vectors per tile row per stage
  static constexpr int A_VEC = BM * VPR / NTH;   // A vectors loaded per thread per stage
  static constexpr int B_VEC = BN * VPR / NTH;
  static constexpr int WTM = BM / WM, WTN = BN / WN;  // wave tile
  static constexpr int S = Op::S;
  static constexpr int TM = WTM / S;
  static constexpr int TN = GATED ? (BN / 2 / WN) / S : WTN / S;  // per half when gated
  static constexpr int NACC = GATED ? 2 * TN : TN;
  static constexpr int OUT_COLS = GATED ? BN / 2 : BN;  // output columns per tile
  static_assert(BM * VPR % NTH == 0 && BN * VPR % NTH == 0, "loader must tile evenly");
  static_assert(TM >= 1 && TN >= 1, "wave tile too small");
  static_assert(BK % Op::KS == 0 && BK % 32 == 0, "BK must be a multiple of the MFMA K step");
  static_assert(TM * S == WTM && (GATED ? TN * S * WN * 2 == BN : TN * S == WTN), "wave tile must tile by S");

  static_assert(LDB == 1 || LDB == 2, "one or two LDS stages");

  // One tile: `tile` indexes the (local expert, N tile, M tile) list of the plan (row_start and
  // tile_start hold its per-expert starts); As / Bs are the LDB LDS stages of A and B.
  __device__ __forceinline__ static void run(const GemmArgs& args, int tile, const int* row_start,
                                             const int* tile_start, T (*As)[BM * LDR], T (*Bs)[BN * LDR]) {
    const T* __restrict__ A = static_cast<const T*>(args.A);
    const T* __restrict__ W = static_cast<const T*>(args.W);
    T* __restrict__ Out = static_cast<T*>(args.Out);
    constexpr int A_OOB = 0x7ffffff0;
    const __amdgpu_buffer_rsrc_t a_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)A, (short)0, BUF ? args.a_bytes : 0, 0x00020000);
    const int El = args.El;
    const int n_tiles = (args.N + OUT_COLS - 1) / OUT_COLS;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
  // tile -> (local expert l, n tile, m tile): l is the last expert with tile_start[l]*n_tiles <= tile
  int lo = 0, hi = El;  // invariant: tile_start[lo]*n_tiles <= tile < tile_start[hi]*n_tiles
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (tile_start[mid] * n_tiles <= tile) lo = mid;
    else hi = mid;
  }
  const int l = lo;
  const int mt_l = tile_start[l + 1] - tile_start[l];
  const int local = tile - tile_start[l] * n_tiles;
  const int nt = local / mt_l, mt = local % mt_l;
  const int p0 = row_start[l] + mt * BM;
  const int m_rows = min(BM, row_start[l + 1] - p0);
  const int n0 = nt * OUT_COLS;
  const T* Wl = W + (int64_t)l * args.w_stride;

  // per-thread source rows (fixed for the whole K loop). Every load is issued unconditionally from a
  // valid address (rows past the tile end read the tile's first row, columns past K read the last
  // vector of the row) and masked to zero when it is written to LDS: a load under a branch would
  // make the compiler wait for every load in flight before the registers are reused.
  // BUF: A and W are read with buffer loads (32-bit offsets instead of 64-bit pointers), and rows
  // past the tile or past N use an offset past the buffer, which the hardware answers with zeros and
  // no memory request (a tile of an expert with few rows then moves only its real rows)
  const T* a_src[A_VEC];
  int a_off[A_VEC];
  int a_lds[A_VEC];
  bool a_ok[A_VEC];
#pragma unroll
  for (int i = 0; i < A_VEC; ++i) {
    const int idx = tid + i * NTH;
    const int r = idx / VPR, c = (idx % VPR) * VN;
    a_lds[i] = r * LDR + c;
    a_ok[i] = r < m_rows;
    const int p = p0 + (a_ok[i] ? r : 0);
    const int src_row = args.a_perm ? args.a_perm[p] : p;
    a_src[i] = A + (int64_t)src_row * args.lda;
    a_off[i] = (BUF && a_ok[i]) ? src_row * args.lda * (int)sizeof(T) : A_OOB;  // < a_bytes when BUF
  }
  const T* b_src[B_VEC];
  int b_off[B_VEC];
  int b_lds[B_VEC];
  bool b_ok[B_VEC];
  const __amdgpu_buffer_rsrc_t b_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)Wl, (short)0, BUF ? args.w_bytes : 0, 0x00020000);
#pragma unroll
  for (int i = 0; i < B_VEC; ++i) {
    const int idx = tid + i * NTH;
    const int r = idx / VPR, c = (idx % VPR) * VN;
    b_lds[i] = r * LDR + c;
    int wrow, ncol;
    if (GATED) {
      const int half = r / (BN / 2), rr = r % (BN / 2);
      ncol = n0 + rr;
      wrow = ncol + half * args.up_offset;
    } else {
      ncol = n0 + r;
      wrow = ncol;
    }
    b_ok[i] = ncol < args.N;
    b_src[i] = Wl + (int64_t)(b_ok[i] ? wrow : 0) * args.K;
    b_off[i] = (BUF && b_ok[i]) ? wrow * args.K * (int)sizeof(T) : A_OOB;  // < w_bytes when BUF
  }

  typename Op::Acc acc[TM][NACC];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < NACC; ++j)
#pragma unroll
      for (int q = 0; q < Op::NR; ++q) acc[i][j][q] = 0.f;

  // RS register stages of global loads in flight: stage s + RS is requested before the MFMAs of
  // stage s run, and stage s + 1 moves from registers to LDS after them (one barrier per stage).
  const int nk = (args.K + BK - 1) / BK;
  const int rot = k_rotation(args.k_rotate, l, n_tiles, nt, nk);
  // stage st of the loop reads K slice (st + rot) mod nk
  auto kslice = [&](int st) { return (st + rot < nk ? st + rot : st + rot - nk) * BK; };
  u32x4 ra[RS][A_VEC], rb[RS][B_VEC];
  const u32x4 zero = {0u, 0u, 0u, 0u};
  auto load_stage = [&](int st, u32x4 (&xa)[A_VEC], u32x4 (&xb)[B_VEC]) {
    const int k0 = kslice(st);
#pragma unroll
    for (int i = 0; i < A_VEC; ++i) {
      const int col = min(k0 + a_lds[i] % LDR, args.K - VN);
      if (BUF) {
        const int vo = a_off[i] == A_OOB ? A_OOB : a_off[i] + col * (int)sizeof(T);
        xa[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(a_rsrc, vo, 0, 0));
      } else {
        xa[i] = ld16(a_src[i] + col);
      }
    }
#pragma unroll
    for (int i = 0; i < B_VEC; ++i) {
      // weights are read once per tile: streaming (non-temporal) loads keep the reused activation
      // rows resident in L2 when many tiles share them
      const int col = min(k0 + b_lds[i] % LDR, args.K - VN);
      if (BUF) {
        const int vo = b_off[i] == A_OOB ? A_OOB : b_off[i] + col * (int)sizeof(T);
        xb[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(b_rsrc, vo, 0, BNT ? 2 : 0));
      } else {
        const T* pb = b_src[i] + col;
        xb[i] = BNT ? ld16_nt(pb) : ld16(pb);
      }
    }
  };
  auto store_stage = [&](int st, int buf, const u32x4 (&xa)[A_VEC], const u32x4 (&xb)[B_VEC]) {
    const int k0 = kslice(st);
#pragma unroll
    for (int i = 0; i < A_VEC; ++i) {
      st16(&As[buf][a_lds[i]], (a_ok[i] && k0 + a_lds[i] % LDR < args.K) ? xa[i] : zero);
    }
#pragma unroll
    for (int i = 0; i < B_VEC; ++i) st16(&Bs[buf][b_lds[i]], (b_ok[i] && k0 + b_lds[i] % LDR < args.K) ? xb[i] : zero);
  };
  const int fr = lane % S;
  const int fk = (lane / S) * 8;  // 8 consecutive K per lane inside each K step
  auto compute = [&](int buf) {
#pragma unroll
    for (int kk = 0; kk < BK; kk += Op::KS) {
      u32x4 af[TM][Op::VPF];
      u32x4 bfg[NACC][Op::VPF];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const T* pa = &As[buf][(wm * WTM + i * S + fr) * LDR + kk + fk];
#pragma unroll
        for (int q = 0; q < Op::VPF; ++q) af[i][q] = ld16(pa + q * VN);
      }
#pragma unroll
      for (int j = 0; j < NACC; ++j) {
        int brow;
        if (GATED) {
          const int half = j / TN, jj = j % TN;
          brow = half * (BN / 2) + wn * (BN / 2 / WN) + jj * S + fr;
        } else {
          brow = wn * WTN + j * S + fr;
        }
        const T* pb = &Bs[buf][brow * LDR + kk + fk];
#pragma unroll
        for (int q = 0; q < Op::VPF; ++q) bfg[j][q] = ld16(pb + q * VN);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < NACC; ++j) Op::step(acc[i][j], af[i], bfg[j]);
    }
  };

  // stages past the last one re-read the last stage (an L2 hit) so that no load sits under a branch
#pragma unroll
  for (int u = 0; u < RS; ++u) load_stage(min(u, nk - 1), ra[u], rb[u]);
  if (LDB == 2) {
    store_stage(0, 0, ra[0], rb[0]);
    lds_barrier();
  }
  for (int s0 = 0; s0 < nk; s0 += RS) {
#pragma unroll
    for (int u = 0; u < RS; ++u) {
      const int st = s0 + u;  // register slot u holds stage st
      if (st < nk) {
        if (LDB == 2) {  // stage st is already in LDS
          load_stage(min(st + RS, nk - 1), ra[u], rb[u]);
          compute(st & 1);
          if (st + 1 < nk) store_stage(st + 1, (st + 1) & 1, ra[(u + 1) % RS], rb[(u + 1) % RS]);
          lds_barrier();
        } else {
          lds_barrier();  // every wave is done reading the previous stage
          store_stage(st, 0, ra[u], rb[u]);
          lds_barrier();
          load_stage(min(st + RS, nk - 1), ra[u], rb[u]);
          compute(0);
        }
      }
    }
  }
  if (LDB == 1) lds_barrier();  // the next tile overwrites the LDS stage

  // epilogue: lane l holds column l % S of each S x S accumulator; Op::out_row gives the rows. The
  // destination rows are loaded first, unconditionally (rows past the tile read its last row), so the
  // loads are in flight together instead of one per store under the store's branch.
  int orows[TM][Op::NR];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int q = 0; q < Op::NR; ++q) {
      const int p = p0 + min(wm * WTM + i * S + Op::out_row(lane, q), m_rows - 1);
      orows[i][q] = args.out_perm ? args.out_perm[p] : p;
    }
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int cl = GATED ? wn * (BN / 2 / WN) + j * S + (lane % S) : wn * WTN + j * S + (lane % S);
      const int col = n0 + cl;
#pragma unroll
      for (int q = 0; q < Op::NR; ++q) {
        const int row = wm * WTM + i * S + Op::out_row(lane, q);
        if (row < m_rows && col < args.N) {
          float v;
          if (GATED) v = silu_f32(acc[i][j][q]) * acc[i][j + TN][q];
          else v = acc[i][j][q];
          const int orow = orows[i][q];
          if (COMBINE) st_agent(Out + (int64_t)orow * args.ldo + col, v);
          else Out[(int64_t)orow * args.ldo + col] = from_f32<T>(v);
        }
      }
    }
  }
  if (COMBINE) {
    static_assert(BM * LDR * sizeof(T) >= (BM + 1) * sizeof(int), "token list must fit the A stage");
    if (LDB == 2) lds_barrier();  // the last stage's fragments are read before As is reused
    tile_arrive_combine<T, NTH, OUT_COLS>(args, p0, m_rows, n0, nt, n_tiles, reinterpret_cast<int*>(&As[0][0]));
  }
  }
};

template <typename T, typename Op, int BM, int BN, int BK, int WM, int WN, bool GATED, int RS, int LDB, bool BNT,
          bool BUF, bool COMBINE = false>
__global__ __launch_bounds__(WM* WN * 64) __attribute__((amdgpu_waves_per_eu(1)))
void mlp_gemm_kernel(GemmArgs args) {
  static_assert(!COMBINE || !GATED, "the combine follows the down GEMM");
  using Tile = RegTile<T, Op, BM, BN, BK, WM, WN, GATED, RS, LDB, BNT, BUF, COMBINE>;
  constexpr int NTH = Tile::NTH, LDR = Tile::LDR;
  // LDB = 2: two LDS stages, the MFMAs read one while the next stage is written into the other (one
  // barrier per stage). LDB = 1: one LDS stage and two barriers per stage, half the LDS, so more
  // workgroups fit on a CU; the RS register stages keep the global loads in flight either way.
  __shared__ __attribute__((aligned(16))) T As[LDB][BM * LDR];
  __shared__ __attribute__((aligned(16))) T Bs[LDB][BN * LDR];

  const int n_tiles = (args.N + Tile::OUT_COLS - 1) / Tile::OUT_COLS;
  // the plan's row and tile starts in LDS: every tile start then resolves its expert with LDS reads
  // instead of a chain of dependent global loads
  __shared__ int s_plan[2 * (MOE_MAX_EXPERTS + 1)];
  int* row_start = s_plan;
  int* tile_start = s_plan + MOE_MAX_EXPERTS + 1;
  const int total = load_plan<NTH>(args, BM, row_start, tile_start) * n_tiles;

  // XCD-aware order: workgroup b runs on XCD b % 8. The tile list is cut into 8 near-equal contiguous
  // ranges, one per XCD (neighbouring tiles share operands in that XCD's L2), and the XCD's
  // workgroups stride through its range, so every XCD gets the same share of the work.
  const int G = gridDim.x;
  int t_begin = blockIdx.x, t_end = total, t_step = G;
  if ((G & 7) == 0 && G >= 8) {
    const int x = blockIdx.x & 7, per = (total + 7) >> 3;
    t_begin = x * per + (blockIdx.x >> 3);
    t_end = min(total, (x + 1) * per);
    t_step = G >> 3;
  }
  for (int tile = t_begin; tile < t_end; tile += t_step) Tile::run(args, tile, row_start, tile_start, As, Bs);
}

// ------------------------------------------------------------------------------------------------
// Compute-bound bf16 GEMM with direct global -> LDS loads (buffer_load_dwordx4 ... lds)
// ------------------------------------------------------------------------------------------------
// The operands never pass through registers on their way to LDS, so NS stages of loads can be in
// flight at once without register cost, leaving the register file to the accumulators. One wave load
// instruction writes 1 KB of LDS: 8 rows of a 64-deep (128-byte) stage. Rows are stored unpadded and
// the 16-byte chunks of row r are XOR-swizzled (chunk c at position c ^ swz(r)) by choosing which
// global chunk each lane fetches, so the 32-row MFMA fragment reads hit distinct LDS banks. Rows past
// the tile are fetched at an offset beyond the buffer's record count, which the hardware returns as
// zeros. Requires K % 64 == 0 and operand buffers below 2 GiB (the host falls back otherwise).

// chunk swizzle of row r for CPR 16-byte chunks per row (CPR = 8 for 128-byte rows, 4 for 64-byte rows);
// SWZ 1 spreads 16 consecutive rows over distinct (row parity, chunk) bank slots
template <int SWZ, int CPR>
__device__ __forceinline__ int dl_swz(int r) {
  if (CPR == 8) return SWZ == 0 ? (r & 7) : ((r >> 1) & 7);
  return SWZ == 0 ? (r & 3) : ((r >> 2) & 3);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int BM, int BN, int BK, int WM, int WN, bool GATED, int NS, int SWZ, bool SPREAD, bool COMBINE = false>
__global__ __launch_bounds__(WM* WN * 64) void mlp_gemm_dl_kernel(GemmArgs args, int a_bytes) {
  static_assert(!COMBINE || !GATED, "the combine follows the down GEMM");
  using Op = Op32;
  static_assert(BK == 32 || BK == 64, "32- or 64-deep stages");
  constexpr int S = 32, ROWB = BK * 2;
  constexpr int CPR = BK / 8;            // 16-byte chunks per LDS row
  constexpr int RPI = 64 / CPR;          // rows per 1 KB wave load
  constexpr int NW = WM * WN;
  constexpr int A_INS = BM / RPI, B_INS = BN / RPI;  // 1 KB wave loads per stage
  static_assert((A_INS + B_INS) % NW == 0, "wave loads must split evenly");
  constexpr int LPW = (A_INS + B_INS) / NW;
  constexpr int A_BYTES = BM * ROWB, STAGE = (BM + BN) * ROWB;
  constexpr int WTM = BM / WM, TM = WTM / S;
  constexpr int TN = GATED ? (BN / 2 / WN) / S : (BN / WN) / S;
  constexpr int NACC = GATED ? 2 * TN : TN;
  constexpr int OUT_COLS = GATED ? BN / 2 : BN;
  static_assert(NS >= 2 && NS <= 6, "2..6 LDS stages");
  static_assert(TM >= 1 && TN >= 1, "wave tile too small");
  // the NS stages, then the tile's destination rows (BM ints) for the epilogue. This must stay the
  // kernel's only LDS object: with a second one the compiler adds waits for every load in flight
  // before LDS reads (4 more vmcnt(0) per kernel body), which cost 13 % to 2x
  __shared__ __attribute__((aligned(1024))) unsigned char smem[NS * STAGE + BM * 4];

  const bf16_t* A = static_cast<const bf16_t*>(args.A);
  const bf16_t* W = static_cast<const bf16_t*>(args.W);
  bf16_t* __restrict__ Out = static_cast<bf16_t*>(args.Out);
  const int El = args.El;
  // the plan kernel's output (scalar loads: the plan is the same for the whole workgroup); this kernel
  // always runs with a plan
  const int* row_start = args.plan + 2;
  const int* tile_start = args.plan + 3 + El;
  const int n_tiles = (args.N + OUT_COLS - 1) / OUT_COLS;
  const int total = args.plan[0] * n_tiles;
  const int tid = threadIdx.x, lane = tid & 63;
  // the wave index is uniform across the wave: keeping it scalar keeps the buffer descriptor and the
  // LDS destination of every load in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int nk = args.K / BK;
  const int OOB = 0x7ffffff0;
  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)A, (short)0, a_bytes, 0x00020000);
  const int w_bytes = (int)(args.w_stride * 2);

  const int G = gridDim.x;
  int t_begin = blockIdx.x, t_end = total, t_step = G;
  if ((G & 7) == 0 && G >= 8) {
    const int x = blockIdx.x & 7, per = (total + 7) >> 3;
    t_begin = x * per + (blockIdx.x >> 3);
    t_end = min(total, (x + 1) * per);
    t_step = G >> 3;
  }

  for (int tile = t_begin; tile < t_end; tile += t_step) {
    int lo = 0, hi = El;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (tile_start[mid] * n_tiles <= tile) lo = mid;
      else hi = mid;
    }
    const int l = lo;
    const int mt_l = tile_start[l + 1] - tile_start[l];
    const int local = tile - tile_start[l] * n_tiles;
    const int nt = local / mt_l, mt = local % mt_l;
    const int p0 = row_start[l] + mt * BM;
    const int m_rows = min(BM, row_start[l + 1] - p0);
    const int n0 = nt * OUT_COLS;
    const __amdgpu_buffer_rsrc_t b_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)(W + (int64_t)l * args.w_stride), (short)0, w_bytes, 0x00020000);

    // this wave's LPW load instructions per stage: byte offset (without k) and LDS offset of each.
    // The source rows of the A instructions are looked up first, unconditionally (rows past the tile
    // read its last row), so the lookups are in flight together rather than one wait each.
    int srcs[LPW];
#pragma unroll
    for (int q = 0; q < LPW; ++q) {
      const int p = p0 + min((wave * LPW + q) * RPI + lane / CPR, m_rows - 1);
      srcs[q] = (args.a_perm && wave * LPW + q < A_INS) ? args.a_perm[p] : p;
    }
    int voff[LPW], loff[LPW];
    bool isa[LPW];
#pragma unroll
    for (int q = 0; q < LPW; ++q) {
      const int ins = wave * LPW + q;
      const int r_in = lane / CPR, pos = lane % CPR;
      if (ins < A_INS) {
        const int r = ins * RPI + r_in;
        const int chunk = pos ^ dl_swz<SWZ, CPR>(r);
        isa[q] = true;
        loff[q] = ins * 1024;
        voff[q] = r < m_rows ? srcs[q] * args.lda * 2 + chunk * 16 : OOB;
      } else {
        const int r = (ins - A_INS) * RPI + r_in;
        const int chunk = pos ^ dl_swz<SWZ, CPR>(r);
        isa[q] = false;
        loff[q] = A_BYTES + (ins - A_INS) * 1024;
        int wrow, ncol;
        if (GATED) {
          const int half = r / (BN / 2), rr = r % (BN / 2);
          ncol = n0 + rr;
          wrow = ncol + half * args.up_offset;
        } else {
          ncol = n0 + r;
          wrow = ncol;
        }
        voff[q] = ncol < args.N ? wrow * args.K * 2 + chunk * 16 : OOB;
      }
    }
    // issue this wave's loads q with q % parts == part of stage st into LDS slot `slot`
    auto issue_part = [&](int st, int slot, int part, int parts) {
      const int kb = st * BK * 2;
#pragma unroll
      for (int q = 0; q < LPW; ++q) {
        if (q % parts != part) continue;
        const int vo = voff[q] == OOB ? OOB : voff[q] + kb;
        auto* dst = (__attribute__((address_space(3))) void*)(smem + slot * STAGE + loff[q]);
        if (isa[q]) __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, dst, 16, vo, 0, 0, 0);
        else __builtin_amdgcn_raw_ptr_buffer_load_lds(b_rsrc, dst, 16, vo, 0, 0, 0);
      }
    };
    auto issue = [&](int st, int slot) { issue_part(st, slot, 0, 1); };

    typename Op::Acc acc[TM][NACC];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < NACC; ++j)
#pragma unroll
        for (int q = 0; q < Op::NR; ++q) acc[i][j][q] = 0.f;

    const int fr = lane & 31, fq = lane >> 5;
    // 32-row blocks of this wave's rows that hold tile rows: the blocks past the tile's last row are
    // neither read from LDS nor multiplied (wave-uniform), so a ragged tile of an expert's last rows
    // costs matrix time only for its real blocks
    const int mb = min(TM, max(0, (m_rows - wm * WTM + S - 1) / S));
    // fragments of K step kk + 1 are requested before the MFMAs of step kk are issued (two fragment
    // buffers), so LDS latency overlaps the matrix work of the same wave
    auto load_frags = [&](const unsigned char* base, int kk, u32x4 (&af)[TM][1], u32x4 (&bfg)[NACC][1]) {
      const int c = kk / 8 + fq;  // logical 16-byte chunk of this lane's 8 K values
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = wm * WTM + i * S + fr;
        if (i < mb) af[i][0] = ld16(base + r * ROWB + ((c ^ dl_swz<SWZ, CPR>(r)) << 4));
      }
#pragma unroll
      for (int j = 0; j < NACC; ++j) {
        int r;
        if (GATED) {
          const int half = j / TN, jj = j % TN;
          r = half * (BN / 2) + wn * (BN / 2 / WN) + jj * S + fr;
        } else {
          r = wn * (BN / WN) + j * S + fr;
        }
        bfg[j][0] = ld16(base + A_BYTES + r * ROWB + ((c ^ dl_swz<SWZ, CPR>(r)) << 4));
      }
    };
    // the loads of stage `next` (into slot next_slot, if next >= 0) are spread over the K steps, so
    // the address units and LDS writes of every wave do not all burst right after the barrier
    auto compute = [&](int slot, int next, int next_slot) {
      const unsigned char* base = smem + slot * STAGE;
      constexpr int KSTEPS = BK / Op::KS;
      u32x4 af[2][TM][1], bfg[2][NACC][1];
      load_frags(base, 0, af[0], bfg[0]);
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        if (SPREAD && next >= 0) issue_part(next, next_slot, ks, KSTEPS);
        if (!SPREAD && next >= 0 && ks == 0) issue(next, next_slot);
        if (ks + 1 < KSTEPS) load_frags(base, (ks + 1) * Op::KS, af[(ks + 1) & 1], bfg[(ks + 1) & 1]);
#pragma unroll
        for (int i = 0; i < TM; ++i)
          if (i < mb) {
#pragma unroll
            for (int j = 0; j < NACC; ++j) Op::step(acc[i][j], af[ks & 1][i], bfg[ks & 1][j]);
          }
      }
    };

    // earlier stores of this wave are done and every wave is done with the LDS of the previous tile
    wait_vmcnt<0>();
    lds_barrier();
#pragma unroll
    for (int st = 0; st < NS - 1; ++st)
      if (st < nk) issue(st, st);
    for (int s = 0; s < nk; ++s) {
      // stage s has landed once at most min(NS - 2, nk - 1 - s) younger stages are still in flight
      const int younger = min(NS - 2, nk - 1 - s);
      if (NS > 5 && younger >= 4) wait_vmcnt<4 * LPW>();
      else if (NS > 4 && younger == 3) wait_vmcnt<3 * LPW>();
      else if (NS > 3 && younger == 2) wait_vmcnt<2 * LPW>();
      else if (younger == 1) wait_vmcnt<LPW>();
      else wait_vmcnt<0>();
      lds_barrier();  // stage s visible to every wave; every wave is done with stage s - 1
      const int next = s + NS - 1 < nk ? s + NS - 1 : -1;
      compute(s % NS, next, next >= 0 ? next % NS : 0);
    }

    // epilogue through LDS, free once every wave is past the last stage: the waves write their bf16
    // results (lane l holds column l % 32, rows 8*(q/4) + 4*(l/32) + q%4 of each 32x32 block), then
    // every lane stores whole 16-byte row chunks. Chunk c of tile row r sits at c ^ (4 * ((r >> 2) & 1)),
    // which puts rows r and r + 4 (written by one instruction) on different LDS banks. An output tile
    // larger than the stage buffers goes out in OCH column parts, each written by the waves owning it.
    constexpr int OCH = (BM * OUT_COLS * 2 <= NS * STAGE) ? 1 : 2;
    constexpr int OCW = OUT_COLS / OCH;  // columns per part
    constexpr int CPO = OCW / 8;         // 16-byte chunks per output row of a part
    static_assert(WN % OCH == 0 && BM * OCW * 2 <= NS * STAGE && CPO >= 8, "output parts must fit the stage buffers");
    auto out_off = [&](int r, int cl) { return r * OCW * 2 + (((cl >> 3) ^ (((r >> 2) & 1) << 2)) << 4) + (cl & 7) * 2; };
    // the destination row of each tile row: one load per row, all in flight together while the
    // accumulators go to LDS, then kept in LDS. A row-map load inside the store loop would wait for
    // every store before it (one counter covers loads and stores) and serialise the tile's stores.
    static_assert(BM <= NW * 64, "one row per thread");
    int* s_orow = reinterpret_cast<int*>(smem + NS * STAGE);
    int my_orow = 0;
    if (tid < BM) {
      const int p = p0 + min(tid, m_rows - 1);
      my_orow = args.out_perm ? args.out_perm[p] : p;
    }
    // with the fused combine, Out (below 2 GiB here, like every operand of this kernel) is stored at agent scope
    const __amdgpu_buffer_rsrc_t out_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)Out, (short)0, COMBINE ? args.out_bytes : 0, 0x00020000);
#pragma unroll
    for (int oc = 0; oc < OCH; ++oc) {
      lds_barrier();  // the stages (or the previous part) are no longer read
      if (wn / (WN / OCH) == oc) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const int cl = (GATED ? wn * (BN / 2 / WN) + j * S + fr : wn * (BN / WN) + j * S + fr) - oc * OCW;
#pragma unroll
            for (int q = 0; q < Op::NR; ++q) {
              const int row = wm * WTM + i * S + Op::out_row(lane, q);
              float v;
              if (GATED) v = silu_f32(acc[i][j][q]) * acc[i][j + TN][q];
              else v = acc[i][j][q];
              *reinterpret_cast<bf16_t*>(smem + out_off(row, cl)) = (bf16_t)v;
            }
          }
        }
      }
      if (oc == 0 && tid < BM) s_orow[tid] = my_orow;
      lds_barrier();
      for (int idx = tid; idx < BM * CPO; idx += NW * 64) {
        const int row = idx / CPO, ch = idx % CPO;
        const int col = n0 + oc * OCW + ch * 8;
        if (row < m_rows && col < args.N) {
          const int orow = s_orow[row];
          if (COMBINE) st16_agent(out_rsrc, (orow * args.ldo + col) * 2, ld16(smem + out_off(row, ch * 8)));
          else st16(Out + (int64_t)orow * args.ldo + col, ld16(smem + out_off(row, ch * 8)));
        }
      }
    }
    if (COMBINE) {
      lds_barrier();  // every wave has read its output chunks before the token list overwrites them
      tile_arrive_combine<bf16_t, NW * 64, OUT_COLS>(args, p0, m_rows, n0, nt, n_tiles, reinterpret_cast<int*>(smem));
    }
  }
}


// ------------------------------------------------------------------------------------------------
// Whole-expert tiles: direct global -> LDS loads, cross-stage schedule, cross-tile prefetch
// ------------------------------------------------------------------------------------------------
// The loads and fragment layout of mlp_gemm_dl_kernel (64-deep stages, 1 KB wave loads of 8 rows,
// XOR-swizzled 16-byte chunks), with two stage slots (stage s in slot s & 1) and this schedule:
//  - The barrier that publishes stage s + 1 sits before the MFMAs of stage s's last K step, whose
//    fragments are already in registers; those MFMAs cover the barrier's skew and the fragment reads
//    of stage s + 1's first K step.
//  - Right after that barrier stage s's slot is free: it takes the B (weight) loads of stage s + 2, one
//    between each pair of MFMAs of the last K step, a full stage ahead of their use. The A loads of
//    stage s + 1 (activation rows, L2-resident, shorter latency) go out between the MFMAs of stage s's
//    first K step. Every wave issues AW A loads and BW B loads per stage, so whether a load reads A or
//    B is known at compile time, and no wave waits behind a burst of a whole stage's loads.
//  - Cross-tile prefetch (even stage counts): the next tile's stage 0 is the continuation of the
//    pipeline - its B loads go out in stage nk - 2's last K step and its A loads in stage nk - 1's
//    first, into slot 0, while the output tile is staged through slot 1 and the space past it. The
//    next tile's expert, rows and A-row lookups are found during stage nk - 2, from a copy of the
//    plan's per-expert starts in LDS.
// Requires K % 64 == 0 and operand buffers below 2 GiB (the host falls back otherwise).
template <int BM, int BN, int WM, int WN, bool GATED, bool COMBINE = false>
__global__ __launch_bounds__(WM* WN * 64) void mlp_gemm_xs_kernel(GemmArgs args, int a_bytes) {
  static_assert(!COMBINE || !GATED, "the combine follows the down GEMM");
  using Op = Op32;
  constexpr int BK = 64, S = 32, ROWB = BK * 2, CPR = BK / 8, RPI = 64 / CPR;
  constexpr int NW = WM * WN;
  constexpr int A_INS = BM / RPI, B_INS = BN / RPI;  // 1 KB wave loads per stage
  static_assert(A_INS % NW == 0 && B_INS % NW == 0, "every wave issues the same number of A and B loads");
  constexpr int AW = A_INS / NW, BW = B_INS / NW, LPW = AW + BW;
  constexpr int A_BYTES = BM * ROWB, STAGE = (BM + BN) * ROWB;
  constexpr int WTM = BM / WM, TM = WTM / S;
  constexpr int TN = GATED ? (BN / 2 / WN) / S : (BN / WN) / S;
  constexpr int NACC = GATED ? 2 * TN : TN;
  constexpr int OUT_COLS = GATED ? BN / 2 : BN;
  constexpr int KSTEPS = BK / Op::KS;
  static_assert(TM >= 1 && TN >= 1, "wave tile too small");
  // LDS: slot 0 at 0, slot 1 at STAGE. After the last stage the output tile goes out in OCH column
  // parts staged from slot 1 on (slot 0 may hold the next tile's stage 0), then the destination rows,
  // then the plan copy (row starts, M-tile starts).
  constexpr int OCW = 128, OCH = OUT_COLS / OCW, CPO = OCW / 8;
  static_assert(OUT_COLS % OCW == 0 && WN % OCH == 0, "output parts");
  constexpr int STG_OFF = STAGE, OROW_OFF = STG_OFF + BM * OCW * 2, PLAN_OFF = OROW_OFF + BM * 4;
  constexpr int PLAN_INTS = MOE_MAX_EXPERTS + 1;
  constexpr int SMEM_END = PLAN_OFF + 2 * PLAN_INTS * 4;
  constexpr int SMEM = SMEM_END > 2 * STAGE ? SMEM_END : 2 * STAGE;
  static_assert(PLAN_OFF >= 2 * STAGE || OROW_OFF >= 2 * STAGE, "the plan copy lies past the stage slots");
  static_assert(SMEM <= 160 * 1024, "LDS");
  static_assert(BM <= NW * 64 && (BM + 1) * 4 <= BM * OCW * 2, "one row per thread; token list fits");
  // the kernel's only LDS object (see mlp_gemm_dl_kernel)
  __shared__ __attribute__((aligned(1024))) unsigned char smem[SMEM];
  int* s_rs = reinterpret_cast<int*>(smem + PLAN_OFF);  // row start per local expert [0..El]
  int* s_ts = s_rs + PLAN_INTS;                          // M-tile start per local expert [0..El]
  int* s_orow = reinterpret_cast<int*>(smem + OROW_OFF);

  const bf16_t* A = static_cast<const bf16_t*>(args.A);
  const bf16_t* W = static_cast<const bf16_t*>(args.W);
  bf16_t* __restrict__ Out = static_cast<bf16_t*>(args.Out);
  const int El = args.El;
  int tid = threadIdx.x, lane = tid & 63;  // made opaque at each tile start (below)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int nk = args.K / BK;
  const int OOB = 0x7ffffff0;
  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)A, (short)0, a_bytes, 0x00020000);
  const int w_bytes = (int)(args.w_stride * 2);
  const int n_tiles = (args.N + OUT_COLS - 1) / OUT_COLS;
  const int total = args.plan[0] * n_tiles;
  for (int i = tid; i <= El; i += NW * 64) {
    s_rs[i] = args.plan[2 + i];
    s_ts[i] = args.plan[3 + El + i];
  }
  lds_barrier();

  // Work units. The tile list is cut into eight equal contiguous ranges, one per XCD (when the grid is a
  // multiple of 8: workgroup b runs on XCD b % 8); the gx workgroups of XCD x take its n_x tiles in rounds,
  // workgroup j the tiles j, j + gx, ... When the last round is at most half full (0 < tail <= gx / 2; gate/up
  // GEMM, stage count a multiple of 4, room for the partials), each tail tile is cut into two K halves and
  // workgroup j of the last round takes half j & 1 of tail tile j >> 1, so no workgroup idles through it.
  // Both halves store their fp32 accumulators and count their arrival; the second to arrive adds the other
  // half's and finishes the tile (the sum of the two halves is the same whichever arrives first).
  const int G = gridDim.x;
  int xcd = 0, wj = blockIdx.x, gx = G, base = 0, n_x = total;
  if ((G & 7) == 0 && G >= 8) {
    const int per = (total + 7) >> 3;
    xcd = blockIdx.x & 7;
    wj = blockIdx.x >> 3;
    gx = G >> 3;
    base = xcd * per;
    n_x = max(0, min(total, base + per) - base);
  }
  const int rounds = n_x / gx, tail = n_x - rounds * gx;
  constexpr int PART_BYTES = NW * 64 * TM * NACC * Op::NR * 4;  // one half's fp32 accumulators
  int part_off = 0;
  bool split = false;
  if (GATED && args.split_ctr != nullptr && (nk & 3) == 0 && tail > 0 && 2 * tail <= gx && (G >> 1) <= kSplitSlots &&
      args.out_bytes > 0) {
    // the partials live in Out's rows past the GEMM's rows (h rows that no later step reads)
    const int64_t off = ((int64_t)args.plan[1] * args.ldo * 2 + 255) & ~(int64_t)255;
    split = off + (int64_t)(G >> 1) * 2 * PART_BYTES <= (int64_t)args.out_bytes;
    part_off = (int)off;
  }
  const int n_full = rounds + (!split && wj < tail ? 1 : 0);
  const int n_units = n_full + (split && wj < 2 * tail ? 1 : 0);
  if (n_units == 0) return;

  // a unit's expert, N tile, rows and K range. Tiles list (local expert, N tile, M tile) in expert order and
  // a workgroup's tiles increase, so the expert is found by scanning on from the previous tile's.
  struct TileP {
    int l, nt, p0, m_rows, n0;
    int k0, nks, half, slot;  // first stage, stages, K half (-1: the whole K) and its counter
  };
  auto tile_params = [&](int u, int l) {
    const bool hu = GATED && u >= n_full;  // only the gate/up GEMM splits
    const int tile = hu ? base + rounds * gx + (wj >> 1) : base + wj + u * gx;
    while (__builtin_amdgcn_readfirstlane(s_ts[l + 1]) * n_tiles <= tile) ++l;
    const int ts = __builtin_amdgcn_readfirstlane(s_ts[l]), mt_l = __builtin_amdgcn_readfirstlane(s_ts[l + 1]) - ts;
    const int local = tile - ts * n_tiles;
    const int nt = local / mt_l, mt = local % mt_l;
    TileP t;
    t.l = l;
    t.nt = nt;
    t.p0 = __builtin_amdgcn_readfirstlane(s_rs[l]) + mt * BM;
    t.m_rows = min(BM, __builtin_amdgcn_readfirstlane(s_rs[l + 1]) - t.p0);
    t.n0 = nt * OUT_COLS;
    t.half = hu ? (wj & 1) : -1;
    t.nks = hu ? nk >> 1 : nk;
    t.k0 = hu ? t.half * t.nks : 0;
    t.slot = xcd * (gx >> 1) + (wj >> 1);
    return t;
  };
  // this wave's loads: q < AW are A instructions wave * AW + q, q >= AW are B instructions wave * BW + q - AW;
  // voff: byte offset without k (OOB past the tile), loff: LDS offset within a slot
  int voff[LPW];
  auto a_src_row = [&](const TileP& t, int q) { return t.p0 + min((wave * AW + q) * RPI + lane / CPR, t.m_rows - 1); };
  auto setup_a = [&](const TileP& t, const int (&src)[AW]) {
#pragma unroll
    for (int q = 0; q < AW; ++q) {
      const int r = (wave * AW + q) * RPI + lane / CPR;
      const int chunk = (lane % CPR) ^ dl_swz<1, CPR>(r);
      voff[q] = r < t.m_rows ? src[q] * args.lda * 2 + chunk * 16 + t.k0 * BK * 2 : OOB;
    }
  };
  auto lookup_a = [&](const TileP& t, int (&src)[AW]) {
#pragma unroll
    for (int q = 0; q < AW; ++q) src[q] = args.a_perm ? args.a_perm[a_src_row(t, q)] : a_src_row(t, q);
  };
  auto setup_b = [&](const TileP& t) {
#pragma unroll
    for (int q = AW; q < LPW; ++q) {
      const int r = (wave * BW + q - AW) * RPI + lane / CPR;
      const int chunk = (lane % CPR) ^ dl_swz<1, CPR>(r);
      int wrow, ncol;
      if (GATED) {
        const int half = r / (BN / 2), rr = r % (BN / 2);
        ncol = t.n0 + rr;
        wrow = ncol + half * args.up_offset;
      } else {
        ncol = t.n0 + r;
        wrow = ncol;
      }
      voff[q] = ncol < args.N ? wrow * args.K * 2 + chunk * 16 + t.k0 * BK * 2 : OOB;
    }
  };
  auto b_rsrc_of = [&](const TileP& t) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)(W + (int64_t)t.l * args.w_stride), (short)0, w_bytes, 0x00020000);
  };
  auto loff = [&](int q) { return q < AW ? (wave * AW + q) * 1024 : A_BYTES + (wave * BW + q - AW) * 1024; };
  __amdgpu_buffer_rsrc_t b_rsrc;
  // this wave's load q (a compile-time index) of stage st into slot. A whole expert's rows share each
  // weight tile, so every weight byte is read once: the weight loads are non-temporal (cache policy bit
  // 1), which leaves the L2 to the activation rows that the expert's N tiles share. On 256 experts of
  // 192-512 rows at H 7168, F 2048: down 2530 -> 2347 us, gate/up 4362 -> 4324 us (same output bits)
  auto issue_one = [&](int st, int slot, int q) {
    const int vo = voff[q] == OOB ? OOB : voff[q] + st * BK * 2;
    auto* dst = (__attribute__((address_space(3))) void*)(smem + slot * STAGE + loff(q));
    if (q < AW) __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, dst, 16, vo, 0, 0, 0);
    else __builtin_amdgcn_raw_ptr_buffer_load_lds(b_rsrc, dst, 16, vo, 0, 0, 2);
  };

  int fr = lane & 31, fq = lane >> 5;
  // fragments of K step kk of the stage at base: every A block (rows past the tile hold zeros), and B
  auto load_frags = [&](const unsigned char* base, int kk, u32x4 (&af)[TM][1], u32x4 (&bfg)[NACC][1]) {
    const int c = kk / 8 + fq;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int r = wm * WTM + i * S + fr;
      af[i][0] = ld16(base + r * ROWB + ((c ^ dl_swz<1, CPR>(r)) << 4));
    }
#pragma unroll
    for (int j = 0; j < NACC; ++j) {
      int r;
      if (GATED) {
        const int half = j / TN, jj = j % TN;
        r = half * (BN / 2) + wn * (BN / 2 / WN) + jj * S + fr;
      } else {
        r = wn * (BN / WN) + j * S + fr;
      }
      bfg[j][0] = ld16(base + A_BYTES + r * ROWB + ((c ^ dl_swz<1, CPR>(r)) << 4));
    }
  };

  // PF: the stage count is even, so every tile's stage 0 is issued by the tile before it (the first
  // one's before the loop). Every tile then takes the same path, and the loads each wave has in
  // flight are the same at every point of it (their count must be known where the fragment reads
  // wait on LDS, or those waits fall back to waiting for everything).
  auto run = [&](auto PF_C) {
  constexpr bool PF = decltype(PF_C)::value;
  TileP cur = tile_params(0, 0);
  {
    int src[AW];
    lookup_a(cur, src);
    setup_a(cur, src);
    setup_b(cur);
    b_rsrc = b_rsrc_of(cur);
  }
  if (PF) {
    wait_vmcnt<0>();  // the A row lookups
#pragma unroll
    for (int q = AW; q < LPW; ++q) issue_one(0, 0, q);
#pragma unroll
    for (int q = 0; q < AW; ++q) issue_one(0, 0, q);
  }
  for (int u = 0; u < n_units; ++u) {
    const int next = u + 1;
    const bool has_next = next < n_units;
    const int nk = GATED ? cur.nks : args.K / BK;  // this unit's stages
    const bool pf = PF && has_next;
    typename Op::Acc acc[TM][NACC];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < NACC; ++j)
#pragma unroll
        for (int q = 0; q < Op::NR; ++q) acc[i][j][q] = 0.f;
    // The lane indices pass through an empty asm statement at each tile start, so the per-lane values
    // derived from them (fragment and load offsets, staging addresses) are computed in each tile and are
    // dead in its epilogue. Computed once before the tile loop, they do not fit the registers next to
    // the accumulators: the compiler keeps about 40 of them in scratch memory and reloads them after the
    // output stores, and each reload waits for those stores (one in-order counter covers loads and
    // stores). 164 -> 8 bytes of scratch per lane; on 256 experts of 192-512 rows at H 7168, F 2048:
    // gate/up 4330 -> 4247 us, down 2354 -> 2246 us (same output bits)
    asm volatile("" : "+v"(tid), "+v"(lane), "+v"(fr), "+v"(fq));
    // 32-row blocks of this wave's rows that hold tile rows (wave-uniform): the others are not multiplied
    const int mb = min(TM, max(0, (cur.m_rows - wm * WTM + S - 1) / S));

    // earlier stores and loads of this wave are done, and every wave is past the previous tile's LDS use
    wait_vmcnt<0>();
    lds_barrier();
    if (!PF) {
#pragma unroll
      for (int q = AW; q < LPW; ++q) issue_one(0, 0, q);
#pragma unroll
      for (int q = 0; q < AW; ++q) issue_one(0, 0, q);
    }
    if (nk > 1) {
#pragma unroll
      for (int q = AW; q < LPW; ++q) issue_one(1, 1, q);
      wait_vmcnt<BW>();  // everything but stage 1's B loads has landed
    } else {
      wait_vmcnt<0>();
    }
    lds_barrier();
    u32x4 af[2][TM][1], bfg[2][NACC][1];
    load_frags(smem, 0, af[0], bfg[0]);
    TileP nxt = cur;
    int nsrc[AW];

    // one stage. HAVE1 / HAVE2: stages s + 1 / s + 2 of this tile exist; PRE: 1 for stage nk - 2 and 2
    // for stage nk - 1, where the next tile's stage 0 goes out when pf
    auto stage = [&](int s, auto HAVE1, auto HAVE2, auto PRE) {
      constexpr bool have1 = decltype(HAVE1)::value, have2 = decltype(HAVE2)::value;
      constexpr int pre = decltype(PRE)::value;
      const int slot = s & 1;
      const unsigned char* base = smem + slot * STAGE;
      if (pre == 2 && pf) setup_a(nxt, nsrc);
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        if (ks + 1 < KSTEPS) {
          load_frags(base, (ks + 1) * Op::KS, af[(ks + 1) & 1], bfg[(ks + 1) & 1]);
        } else if (have1) {
          wait_vmcnt<0>();  // this wave's loads of stage s + 1
          lds_barrier();    // stage s + 1 visible to every wave; no wave reads slot s & 1 any more
          load_frags(smem + (slot ^ 1) * STAGE, 0, af[0], bfg[0]);
        }
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          if (i < mb) {
#pragma unroll
            for (int j = 0; j < NACC; ++j) Op::step(acc[i][j], af[ks & 1][i], bfg[ks & 1][j]);
          }
          if (ks == 0 && i < AW && have1) issue_one(s + 1, slot ^ 1, i);
          if (ks == KSTEPS - 1 && i < BW && have2) issue_one(s + 2, slot, AW + i);
          // the next tile's stage 0 into slot 0 (slot here is 0 at pre 1 and 1 at pre 2: nk is even)
          if (pre == 1 && ks == KSTEPS - 1 && i < BW && pf) issue_one(0, 0, AW + i);
          if (pre == 2 && ks == 0 && i < AW && pf) issue_one(0, 0, i);
        }
        if (ks == 0 && have1) {
#pragma unroll
          for (int q = TM; q < AW; ++q) issue_one(s + 1, slot ^ 1, q);
        }
        if (ks == KSTEPS - 1 && have2) {
#pragma unroll
          for (int q = TM; q < BW; ++q) issue_one(s + 2, slot, AW + q);
        }
        if (pre == 1 && ks == KSTEPS - 1 && pf) {
#pragma unroll
          for (int q = TM; q < BW; ++q) issue_one(0, 0, AW + q);
        }
        if (pre == 2 && ks == 0 && pf) {
#pragma unroll
          for (int q = TM; q < AW; ++q) issue_one(0, 0, q);
        }
        // after stage nk - 2's first K step this tile has issued all its loads: switch the B operand to
        // the next tile and start the lookups of its A rows (used at stage nk - 1)
        if (pre == 1 && ks == 0 && pf) {
          nxt = tile_params(next, cur.l);
          setup_b(nxt);
          b_rsrc = b_rsrc_of(nxt);
          lookup_a(nxt, nsrc);
        }
      }
    };
    using Yes = std::integral_constant<bool, true>;
    using No = std::integral_constant<bool, false>;
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    using P2 = std::integral_constant<int, 2>;
    int s = 0;
    for (; s + 2 < nk; ++s) stage(s, Yes{}, Yes{}, P0{});
    if (s + 1 < nk) stage(s++, Yes{}, No{}, P1{});
    stage(s, No{}, No{}, P2{});

    // a K half: store this half's fp32 accumulators (agent scope, written through to the level coherent
    // across the XCDs), wait for them, then count the arrival. The first half to arrive is done; the second
    // adds the first's accumulators (loaded only after its count returned) and finishes the tile. The
    // ordering argument is the fused combine's (tile_arrive_combine).
    if (GATED && cur.half >= 0) {
      const __amdgpu_buffer_rsrc_t p_rsrc =
          __builtin_amdgcn_make_buffer_rsrc((void*)Out, (short)0, args.out_bytes, 0x00020000);
      const int own = part_off + (cur.slot * 2 + cur.half) * PART_BYTES + tid * 16;
      const int oth = part_off + (cur.slot * 2 + (cur.half ^ 1)) * PART_BYTES + tid * 16;
      constexpr int SEGS = Op::NR / 4;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int jj = 0; jj < NACC; ++jj)
#pragma unroll
          for (int q4 = 0; q4 < SEGS; ++q4) {
            const int seg = (i * NACC + jj) * SEGS + q4;
            const u32x4 v = {__float_as_uint(acc[i][jj][4 * q4]), __float_as_uint(acc[i][jj][4 * q4 + 1]),
                             __float_as_uint(acc[i][jj][4 * q4 + 2]), __float_as_uint(acc[i][jj][4 * q4 + 3])};
            st16_agent(p_rsrc, own + seg * (NW * 64 * 16), v);
          }
      wait_vmcnt<0>();
      lds_barrier();
      if (tid == 0) s_orow[0] = atomicAdd(&args.split_ctr[cur.slot], 1);
      lds_barrier();
      if (__builtin_amdgcn_readfirstlane(s_orow[0]) == 0) break;  // a half unit is a workgroup's last unit
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int jj = 0; jj < NACC; ++jj)
#pragma unroll
          for (int q4 = 0; q4 < SEGS; ++q4) {
            const int seg = (i * NACC + jj) * SEGS + q4;
            const u32x4 v = ld16_agent(p_rsrc, oth + seg * (NW * 64 * 16));
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][jj][4 * q4 + e] += __uint_as_float(v[e]);
          }
    }

    // epilogue: the waves write their bf16 results to the staging area (lane l holds column l % 32,
    // rows 8*(q/4) + 4*(l/32) + q%4 of each 32x32 block), then every lane stores whole 16-byte row chunks.
    // Chunk c of staged row r sits at c ^ (4 * ((r >> 2) & 1)): rows r and r + 4 (one instruction) use
    // different LDS banks.
    // (stg is STG_OFF through an opaque move: otherwise the compiler hoists all of this lane's staging
    // addresses out of the tile loop, where they do not fit the registers and go to scratch memory)
    int stg;
    asm volatile("s_mov_b32 %0, %1" : "=s"(stg) : "n"(STG_OFF));
    auto out_off = [&](int r, int cl) {
      return stg + r * OCW * 2 + (((cl >> 3) ^ (((r >> 2) & 1) << 2)) << 4) + (cl & 7) * 2;
    };
    // the destination row of each tile row, looked up once per tile (all in flight together)
    int my_orow = 0;
    if (tid < BM) {
      const int p = cur.p0 + min(tid, cur.m_rows - 1);
      my_orow = args.out_perm ? args.out_perm[p] : p;
    }
    // with the fused combine, Out (below 2 GiB here, like every operand of this kernel) is stored at agent scope
    const __amdgpu_buffer_rsrc_t out_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)Out, (short)0, COMBINE ? args.out_bytes : 0, 0x00020000);
#pragma unroll
    for (int oc = 0; oc < OCH; ++oc) {
      lds_barrier();  // slot 1 (or the previous part) is no longer read
      if (wn / (WN / OCH) == oc) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const int cl = (GATED ? wn * (BN / 2 / WN) + j * S + fr : wn * (BN / WN) + j * S + fr) - oc * OCW;
#pragma unroll
            for (int q = 0; q < Op::NR; ++q) {
              const int row = wm * WTM + i * S + Op::out_row(lane, q);
              float v;
              if (GATED) v = silu_f32(acc[i][j][q]) * acc[i][j + TN][q];
              else v = acc[i][j][q];
              *reinterpret_cast<bf16_t*>(smem + out_off(row, cl)) = (bf16_t)v;
            }
          }
        }
      }
      if (oc == 0 && tid < BM) s_orow[tid] = my_orow;
      lds_barrier();
      for (int idx = tid; idx < BM * CPO; idx += NW * 64) {
        const int row = idx / CPO, ch = idx % CPO;
        const int col = cur.n0 + oc * OCW + ch * 8;
        if (row < cur.m_rows && col < args.N) {
          const int orow = s_orow[row];
          if (COMBINE) st16_agent(out_rsrc, (orow * args.ldo + col) * 2, ld16(smem + out_off(row, ch * 8)));
          else st16(Out + (int64_t)orow * args.ldo + col, ld16(smem + out_off(row, ch * 8)));
        }
      }
    }
    if (COMBINE) {
      lds_barrier();  // every wave has read its output chunks before the token list overwrites them
      tile_arrive_combine<bf16_t, NW * 64, OUT_COLS>(args, cur.p0, cur.m_rows, cur.n0, cur.nt, n_tiles,
                                                     reinterpret_cast<int*>(smem + STG_OFF));
    }
    if (pf) {
      cur = nxt;
    } else if (has_next) {
      cur = tile_params(next, cur.l);
      int src[AW];
      lookup_a(cur, src);
      setup_a(cur, src);
      setup_b(cur);
      b_rsrc = b_rsrc_of(cur);
    }
  }
  };
  if (nk >= 2 && (nk & 1) == 0) run(std::integral_constant<bool, true>{});
  else run(std::integral_constant<bool, false>{});
}

// ------------------------------------------------------------------------------------------------
// Compute-bound bf16 GEMM, direct global -> LDS loads, ping-pong wave schedule
// ------------------------------------------------------------------------------------------------
// Eight waves, two per SIMD (wave w runs on SIMD w % 4), each owning a 64 x 128 block of the tile (2 x 4
// MFMA 32x32x16 accumulators). The waves form two groups, 0..3 and 4..7, one wave of each on every SIMD.
// The K loop is cut into phases separated by workgroup barriers; in every phase one group reads a whole
// 64-deep stage of fragments from LDS into registers (its memory phase) while the other group issues the
// 32 MFMAs of the stage it read in the phase before (its compute phase), so each SIMD's matrix unit
// always has a wave feeding it and the barrier and LDS latency fall in the memory phases:
//   phase 2s:     group 0 reads stage s      group 1 computes stage s - 1
//   phase 2s + 1: group 0 computes stage s   group 1 reads stage s
// Two LDS stage buffers. Stage s + 1 is loaded into the buffer stage s - 1 left, by every wave, in phase
// 2s (group 1 interleaves its loads with its MFMAs), and waited for at the end of phase 2s + 1. Stages 0
// and 1 are loaded before phase 0. Every wave passes the same 2 nk + 1 barriers per tile.
// Chunks are XOR-swizzled in LDS as in the other direct-to-LDS kernel (chunk c of row r at c ^ ((r >> 1)
// & 7)), so the 32-row fragment reads hit distinct banks. Requires K % 64 == 0 and operand buffers below
// 2 GiB.
constexpr int kPpKph = 2;
// calls f(std::integral_constant<int, i>) for i = 0 .. N - 1 (compile-time loop index)
template <int N, int I = 0, typename Fn>
__device__ __forceinline__ void static_for(Fn&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}
template <int BM, int BN, int WM, int WN, bool GATED, bool COMBINE = false>
__global__ __launch_bounds__(512) void mlp_gemm_pp_kernel(GemmArgs args, int a_bytes) {
  static_assert(!COMBINE || !GATED, "the combine follows the down GEMM");
  using Op = Op32;
  constexpr int NW = 8, BK = 64, S = 32, ROWB = BK * 2, CPR = 8, RPI = 8;
  static_assert(WM * WN == NW, "eight waves");
  constexpr int A_INS = BM / RPI, B_INS = BN / RPI;  // 1 KB wave loads per stage
  static_assert((A_INS + B_INS) % NW == 0, "wave loads must split evenly");
  constexpr int LPW = (A_INS + B_INS) / NW;
  constexpr int A_BYTES = BM * ROWB, STAGE = (BM + BN) * ROWB;
  constexpr int WTM = BM / WM, TM = WTM / S;
  constexpr int TN = GATED ? (BN / 2 / WN) / S : (BN / WN) / S;
  constexpr int NACC = GATED ? 2 * TN : TN;
  constexpr int OUT_COLS = GATED ? BN / 2 : BN;
  constexpr int KSTEPS = BK / Op::KS;
  constexpr int KPH = kPpKph, UPS = KSTEPS / KPH;  // K steps per phase, phases per stage and group
  static_assert(KSTEPS % KPH == 0, "phases split a stage evenly");
  constexpr int OUT_BYTES = BM * OUT_COLS * 2;
  constexpr int PLAN_OFF = (2 * STAGE > OUT_BYTES + BM * 4 ? 2 * STAGE : OUT_BYTES + BM * 4);
  constexpr int PLAN_INTS = MOE_MAX_EXPERTS + 1;
  constexpr int SMEM = PLAN_OFF + 2 * PLAN_INTS * 4;
  static_assert(TM >= 1 && TN >= 1, "wave tile too small");
  static_assert(SMEM <= 160 * 1024, "LDS");
  // the two stage buffers (after the last stage the output tile and its destination rows reuse them),
  // then a copy of the plan's per-expert starts
  __shared__ __attribute__((aligned(1024))) unsigned char smem[SMEM];
  int* s_rs = reinterpret_cast<int*>(smem + PLAN_OFF);  // row start per local expert [0..El]
  int* s_ts = s_rs + PLAN_INTS;                          // M-tile start per local expert [0..El]

  const bf16_t* A = static_cast<const bf16_t*>(args.A);
  const bf16_t* W = static_cast<const bf16_t*>(args.W);
  bf16_t* __restrict__ Out = static_cast<bf16_t*>(args.Out);
  const int El = args.El;
  const int n_tiles = (args.N + OUT_COLS - 1) / OUT_COLS;
  const int total = args.plan[0] * n_tiles;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int wm = wave / WN, wn = wave % WN;
  const int nk = args.K / BK;
  const int OOB = 0x7ffffff0;
  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)A, (short)0, a_bytes, 0x00020000);
  const int w_bytes = (int)(args.w_stride * 2);

  const int G = gridDim.x;
  int t_begin = blockIdx.x, t_end = total, t_step = G;
  if ((G & 7) == 0 && G >= 8) {
    const int x = blockIdx.x & 7, per = (total + 7) >> 3;
    t_begin = x * per + (blockIdx.x >> 3);
    t_end = min(total, (x + 1) * per);
    t_step = G >> 3;
  }

  for (int i = tid; i <= El; i += NW * 64) {
    s_rs[i] = args.plan[2 + i];
    s_ts[i] = args.plan[3 + El + i];
  }
  lds_barrier();

  const int fr = lane & 31, fq = lane >> 5;
  int l = 0;
  for (int tile = t_begin; tile < t_end; tile += t_step) {
    // tiles list (local expert, N tile, M tile) in expert order and a workgroup's tiles increase: the
    // expert is found by scanning on from the previous tile's (8 dependent scalar loads of a binary
    // search over the plan in memory had cost about 2 us per tile)
    while (__builtin_amdgcn_readfirstlane(s_ts[l + 1]) * n_tiles <= tile) ++l;
    const int ts = __builtin_amdgcn_readfirstlane(s_ts[l]);
    const int mt_l = __builtin_amdgcn_readfirstlane(s_ts[l + 1]) - ts;
    const int local = tile - ts * n_tiles;
    const int nt = local / mt_l, mt = local % mt_l;
    const int p0 = __builtin_amdgcn_readfirstlane(s_rs[l]) + mt * BM;
    const int m_rows = min(BM, __builtin_amdgcn_readfirstlane(s_rs[l + 1]) - p0);
    const int n0 = nt * OUT_COLS;
    const __amdgpu_buffer_rsrc_t b_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)(W + (int64_t)l * args.w_stride), (short)0, w_bytes, 0x00020000);

    // this wave's LPW load instructions per stage (instruction wave * LPW + q of the stage's A_INS + B_INS):
    // byte offset without k, and whether it loads A. The A rows are looked up together first.
    int srcs[LPW];
#pragma unroll
    for (int q = 0; q < LPW; ++q) {
      const int p = p0 + min((wave * LPW + q) * RPI + lane / CPR, m_rows - 1);
      srcs[q] = (args.a_perm && wave * LPW + q < A_INS) ? args.a_perm[p] : p;
    }
    int voff[LPW];
#pragma unroll
    for (int q = 0; q < LPW; ++q) {
      const int ins = wave * LPW + q;
      const int r_in = lane / CPR, pos = lane % CPR;
      if (ins < A_INS) {
        const int r = ins * RPI + r_in;
        const int chunk = pos ^ dl_swz<1, CPR>(r);
        voff[q] = r < m_rows ? srcs[q] * args.lda * 2 + chunk * 16 : OOB;
      } else {
        const int r = (ins - A_INS) * RPI + r_in;
        const int chunk = pos ^ dl_swz<1, CPR>(r);
        int wrow, ncol;
        if (GATED) {
          const int half = r / (BN / 2), rr = r % (BN / 2);
          ncol = n0 + rr;
          wrow = ncol + half * args.up_offset;
        } else {
          ncol = n0 + r;
          wrow = ncol;
        }
        voff[q] = ncol < args.N ? wrow * args.K * 2 + chunk * 16 : OOB;
      }
    }
    auto issue = [&](int st) {
      const int kb = st * BK * 2;
      unsigned char* base = smem + (st & 1) * STAGE;
#pragma unroll
      for (int q = 0; q < LPW; ++q) {
        const int ins = wave * LPW + q;  // wave-uniform: A or B, and the LDS offset, are scalar
        const int vo = voff[q] == OOB ? OOB : voff[q] + kb;
        if (ins < A_INS) {
          auto* dst = (__attribute__((address_space(3))) void*)(base + ins * 1024);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, dst, 16, vo, 0, 0, 0);
        } else {
          auto* dst = (__attribute__((address_space(3))) void*)(base + A_BYTES + (ins - A_INS) * 1024);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(b_rsrc, dst, 16, vo, 0, 0, 0);
        }
      }
    };

    typename Op::Acc acc[TM][NACC];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < NACC; ++j)
#pragma unroll
        for (int q = 0; q < Op::NR; ++q) acc[i][j][q] = 0.f;

    // one phase's fragments (KPH K steps of a stage): [K step][A blocks, then B blocks]
    u32x4 frag[KPH][TM + NACC];
    // K steps ks0 .. ks0 + KPH - 1 of the stage in buffer `slot`. Every fragment row r = (32-aligned block
    // base) + fr, so its chunk swizzle (r >> 1) & 7 is (fr >> 1) & 7 for every block.
    auto read_unit = [&](int slot, auto ks0_c) {
      constexpr int ks0 = decltype(ks0_c)::value;
      const unsigned char* base = smem + slot * STAGE + fr * ROWB;
      const int sw = (fr >> 1) & 7;
#pragma unroll
      for (int ks = 0; ks < KPH; ++ks) {
        const int xo = ((((ks0 + ks) * 2 + fq) ^ sw) << 4);  // this lane's 16-byte chunk of the K step
#pragma unroll
        for (int i = 0; i < TM; ++i) frag[ks][i] = ld16(base + (wm * WTM + i * S) * ROWB + xo);
#pragma unroll
        for (int j = 0; j < NACC; ++j) {
          int r0;
          if (GATED) {
            const int half = j / TN, jj = j % TN;
            r0 = half * (BN / 2) + wn * (BN / 2 / WN) + jj * S;
          } else {
            r0 = wn * (BN / WN) + j * S;
          }
          frag[ks][TM + j] = ld16(base + A_BYTES + r0 * ROWB + xo);
        }
      }
    };
    auto compute_unit = [&]() {
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int ks = 0; ks < KPH; ++ks)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < NACC; ++j) {
            const u32x4 a1[1] = {frag[ks][i]};
            const u32x4 b1[1] = {frag[ks][TM + j]};
            Op::step(acc[i][j], a1, b1);
          }
      __builtin_amdgcn_s_setprio(0);
    };
    auto phase_end = [&](bool wait_loads) {
      if (wait_loads) wait_vmcnt<0>();
      __builtin_amdgcn_sched_barrier(0);
      lds_barrier();
      __builtin_amdgcn_sched_barrier(0);
    };

    // the previous tile's output stores are done and every wave is past its LDS reads
    wait_vmcnt<0>();
    lds_barrier();
    issue(0);
    if (nk > 1) issue(1);
    if (nk > 1) wait_vmcnt<LPW>();
    else wait_vmcnt<0>();
    lds_barrier();
    // Every wave runs the same sequence: read unit u, barrier, compute unit u, barrier. Group 1 passes one
    // barrier first, so it runs one phase behind group 0, and group 0 passes one at the end.
    if (grp == 1) phase_end(false);
    for (int st = 0; st < nk; ++st) {
      const int slot = st & 1;
      static_for<UPS>([&](auto j_c) {
        constexpr int j = decltype(j_c)::value;
        // stage st + 1 goes into the buffer stage st - 1 left: group 0 is at global phase 2 UPS st, group 1 at
        // the phase after, and both groups finished reading stage st - 1 at global phase 2 UPS st - 1
        if (j == 0 && st >= 1 && st + 1 < nk) issue(st + 1);
        read_unit(slot, std::integral_constant<int, j * KPH>{});
        // stage st + 1 must have landed by the end of global phase 2 UPS (st + 1) - 1: that is the end of
        // this read phase for group 1 and of the compute phase below for group 0
        phase_end(j == UPS - 1 && grp == 1);
        compute_unit();
        phase_end(j == UPS - 1 && grp == 0);
      });
    }
    if (grp == 0) phase_end(false);

    // epilogue through LDS (both stage buffers are free): the waves write their bf16 results, then every
    // lane stores whole 16-byte row chunks. Chunk c of tile row r sits at c ^ (4 * ((r >> 2) & 1)).
    constexpr int CPO = OUT_COLS / 8;
    static_assert(CPO >= 8, "output rows of at least 64 columns");
    auto out_off = [&](int r, int cl) { return r * OUT_COLS * 2 + (((cl >> 3) ^ (((r >> 2) & 1) << 2)) << 4) + (cl & 7) * 2; };
    int* s_orow = reinterpret_cast<int*>(smem + OUT_BYTES);
    int my_orow = 0;
    if (tid < BM) {
      const int pp = p0 + min(tid, m_rows - 1);
      my_orow = args.out_perm ? args.out_perm[pp] : pp;
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int cl = GATED ? wn * (BN / 2 / WN) + j * S + fr : wn * (BN / WN) + j * S + fr;
#pragma unroll
        for (int qq = 0; qq < Op::NR; ++qq) {
          const int row = wm * WTM + i * S + Op::out_row(lane, qq);
          float v;
          if (GATED) v = silu_f32(acc[i][j][qq]) * acc[i][j + TN][qq];
          else v = acc[i][j][qq];
          *reinterpret_cast<bf16_t*>(smem + out_off(row, cl)) = (bf16_t)v;
        }
      }
    }
    if (tid < BM) s_orow[tid] = my_orow;
    lds_barrier();
    const __amdgpu_buffer_rsrc_t out_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)Out, (short)0, COMBINE ? args.out_bytes : 0, 0x00020000);
    for (int idx = tid; idx < BM * CPO; idx += NW * 64) {
      const int row = idx / CPO, ch = idx % CPO;
      const int col = n0 + ch * 8;
      if (row < m_rows && col < args.N) {
        const int orow = s_orow[row];
        if (COMBINE) st16_agent(out_rsrc, (orow * args.ldo + col) * 2, ld16(smem + out_off(row, ch * 8)));
        else st16(Out + (int64_t)orow * args.ldo + col, ld16(smem + out_off(row, ch * 8)));
      }
    }
    if (COMBINE) {
      lds_barrier();  // every wave has read its output chunks before the token list overwrites them
      tile_arrive_combine<bf16_t, NW * 64, OUT_COLS>(args, p0, m_rows, n0, nt, n_tiles, reinterpret_cast<int*>(smem));
    }
  }
}

template <typename T, typename Op, int BM, int BN, int BK, int WM, int WN, bool GATED, int RS, int LDB, bool BNT,
          bool COMBINE = false>
void launch_gemm(const GemmArgs& a, int grid, hipStream_t stream) {
  if (a.a_bytes > 0 && a.w_bytes > 0)
    mlp_gemm_kernel<T, Op, BM, BN, BK, WM, WN, GATED, RS, LDB, BNT, true, COMBINE><<<grid, WM * WN * 64, 0, stream>>>(a);
  else
    mlp_gemm_kernel<T, Op, BM, BN, BK, WM, WN, GATED, RS, LDB, BNT, false, COMBINE><<<grid, WM * WN * 64, 0, stream>>>(a);
}

// Persistent grid sizes in workgroups per CU, and the register-staged compute-bound tile (the fallback for
// shapes the direct-to-LDS kernels do not take).
constexpr int kDecWpc = 3;
constexpr int kPreWpc = 1;
// many-rows-per-expert (compute-bound) tiles: BM x BN x BK with WM x WN waves
constexpr int kPreBm = 128;
constexpr int kPreBn = 256;
constexpr int kPreBk = 64;
constexpr int kPreWm = 2;
constexpr int kPreWn = 4;


// register stages of global prefetch in flight
constexpr int kPreRs = 2;
constexpr int kDecRs = 2;
constexpr int kDecDnRs = kDecRs;
constexpr int kPreLdb = 2;
// Many rows per expert (operands loaded straight into LDS), by the capacity per local expert:
//   >= kDlTallMinRows  256 x 256 tiles, ping-pong wave schedule (twice the MFMA work per byte staged of a
//                      128-row tile; an expert's ragged last tile wastes little)
//   256 .. 1023        320 x 256 tiles: one M tile holds a whole expert of up to 320 rows, so its weights are
//                      read once (waves skip the 32-row blocks past the tile's rows)
//   128 .. 255         128 x 256 tiles
// BK-deep stages, WM x WN waves, NS LDS stages; one workgroup per CU (kDlWpc), LDS row swizzle kDlSwz.
constexpr bool kPreDl = true;
constexpr int kDlSwz = 1;
constexpr int kDlWpc = 1;
constexpr int kDlBk = 64;
constexpr int kDlTallMinRows = 1024;
// 128-row tile
constexpr int kDlBn = 256;
constexpr int kDlWm = 2;
constexpr int kDlWn = 4;
constexpr int kDlNs = 3;
constexpr bool kDlSpread = true;
// 256-row tiles (ping-pong schedule): 256 weight rows per tile
constexpr int kPpBn = 256;
constexpr int kDecLdb = 1;
// few-rows-per-expert (weight streaming) tiles: 32 or 64 rows, BN weight rows, BK deep. 64-row tiles
// are used when the capacity per local expert is at least kDecTallMinRows rows: an expert then
// often holds more than 32 rows, and one 64-row tile streams its weights once where two 32-row tiles
// would stream them twice.
constexpr int kDecTallMinRows = 32;
constexpr int kDecGuBn = 128;
constexpr int kDecGuBk = 64;
constexpr int kDecDnBn = 64;
constexpr int kDecDnBk = 128;
constexpr int DEC_GU_WN = kDecGuBn / 32 < 4 ? kDecGuBn / 32 : 4;
constexpr int DEC_DN_WN = kDecDnBn / 16 < 4 ? kDecDnBn / 16 : 4;
using PreOp = Op32;


// wpc = 0: one workgroup per tile of the worst-case tile count (workgroups past the real tile count
// exit at once) and the hardware dispatcher balances the load
// a buffer's byte size when 31-bit buffer offsets (with room for the out-of-range marker) cover it, else 0
int buffer_bytes(int64_t bytes) { return bytes > 0 && bytes < 0x7ffffff0ll - 256 ? (int)bytes : 0; }

int persistent_grid(int64_t max_tiles, int num_cus, int wpc) {
  int64_t g = wpc > 0 ? (int64_t)num_cus * wpc : max_tiles;
  if (max_tiles < g) g = max_tiles;
  if (g >= 8) g &= ~7ll;  // a multiple of the XCD count keeps the XCD-aware order exact
  return (int)(g > 0 ? g : 1);
}

}  // namespace

size_t mlp_plan_ints(int El) { return 2 + 2 * (size_t)(El + 1) + kSplitSlots; }

namespace {
// the direct-to-LDS kernel addresses its operands with 31-bit buffer offsets and stages 64-deep K slices
bool dl_fits(int64_t rows_max, int H, int F) {
  const int64_t lim = 0x7ffffff0ll - 256;
  const int64_t send_bytes = rows_max * (int64_t)H * 2, h_bytes = rows_max * (int64_t)F * 2;
  const int64_t wgu_bytes = (int64_t)2 * F * H * 2, wdn_bytes = (int64_t)H * F * 2;
  return kPreDl && H % kDlBk == 0 && F % kDlBk == 0 && send_bytes < lim && h_bytes < lim &&
         wgu_bytes < lim && wdn_bytes < lim;
}


template <int BM, int BN, int WM, int WN, bool COMBINE>
void launch_pp(const GemmArgs& gu, const GemmArgs& dn, int64_t max_mtiles, int H, int F, int64_t send_bytes,
               int64_t h_bytes, int num_cus, hipStream_t stream) {
  const int g1 = persistent_grid(max_mtiles * ceil_div_host(F, BN / 2), num_cus, 1);
  mlp_gemm_pp_kernel<BM, BN, WM, WN, true><<<g1, 512, 0, stream>>>(gu, (int)send_bytes);
  const int g2 = persistent_grid(max_mtiles * ceil_div_host(H, BN), num_cus, 1);
  mlp_gemm_pp_kernel<BM, BN, WM, WN, false, COMBINE><<<g2, 512, 0, stream>>>(dn, (int)h_bytes);
}

template <int BM, int BN, int WM, int WN, int NS, bool SPREAD, bool COMBINE>
void launch_dl(const GemmArgs& gu, const GemmArgs& dn, int64_t max_mtiles, int H, int F, int64_t send_bytes,
               int64_t h_bytes, int num_cus, hipStream_t stream) {
  const int g1 = persistent_grid(max_mtiles * ceil_div_host(F, BN / 2), num_cus, kDlWpc);
  mlp_gemm_dl_kernel<BM, BN, kDlBk, WM, WN, true, NS, kDlSwz, SPREAD><<<g1, WM * WN * 64, 0, stream>>>(
      gu, (int)send_bytes);
  const int g2 = persistent_grid(max_mtiles * ceil_div_host(H, BN), num_cus, kDlWpc);
  mlp_gemm_dl_kernel<BM, BN, kDlBk, WM, WN, false, NS, kDlSwz, SPREAD, COMBINE><<<g2, WM * WN * 64, 0, stream>>>(
      dn, (int)h_bytes);
}

template <int BM, int BN, int WM, int WN, bool COMBINE>
void launch_xs(const GemmArgs& gu, const GemmArgs& dn, int64_t max_mtiles, int H, int F, int64_t send_bytes,
               int64_t h_bytes, int num_cus, hipStream_t stream) {
  const int g1 = persistent_grid(max_mtiles * ceil_div_host(F, BN / 2), num_cus, 1);
  mlp_gemm_xs_kernel<BM, BN, WM, WN, true><<<g1, WM * WN * 64, 0, stream>>>(gu, (int)send_bytes);
  const int g2 = persistent_grid(max_mtiles * ceil_div_host(H, BN), num_cus, 1);
  mlp_gemm_xs_kernel<BM, BN, WM, WN, false, COMBINE><<<g2, WM * WN * 64, 0, stream>>>(dn, (int)h_bytes);
}

template <int BM, bool COMBINE>
void launch_decode(const GemmArgs& gu, const GemmArgs& dn, int64_t max_mtiles, int H, int F, int num_cus,
                   hipStream_t stream) {
  // every weight byte is read by one tile only, so both GEMMs stream the weights with non-temporal
  // loads: Mixtral-shaped gate/up 350 -> 324 us and down 174 -> 165 us, the Kimi-share down GEMM
  // 235 -> 224 us (interleaved pairs on one GPU)
  const int g1 = persistent_grid(max_mtiles * ceil_div_host(F, kDecGuBn / 2), num_cus, kDecWpc);
  launch_gemm<bf16_t, Op16, BM, kDecGuBn, kDecGuBk, 1, DEC_GU_WN, true, kDecRs, kDecLdb, true>(
      gu, g1, stream);
  const int g2 = persistent_grid(max_mtiles * ceil_div_host(H, kDecDnBn), num_cus, kDecWpc);
  launch_gemm<bf16_t, Op16, BM, kDecDnBn, kDecDnBk, 1, DEC_DN_WN, false, kDecDnRs, kDecLdb, true,
              COMBINE>(dn, g2, stream);
}
}  // namespace

// variants: 0 bf16 many rows per expert, register-staged; 1 and 5 bf16 few rows per expert (weight
// streaming) with 32- and 64-row tiles; 2 fp32; 3 and 4 bf16 many rows per expert, direct-to-LDS with
// 128- and 256-row tiles
MlpTiles mlp_pick_tiles(int64_t rows_max, int El, int H, int F, int xdt_bf16) {
  if (!xdt_bf16) return MlpTiles{32, 2};
  const int64_t per_expert = El > 0 ? rows_max / El : rows_max;
  if (per_expert < 128) return per_expert >= kDecTallMinRows ? MlpTiles{64, 5} : MlpTiles{32, 1};
  if (!dl_fits(rows_max, H, F)) return MlpTiles{kPreBm, 0};
  if (per_expert >= kDlTallMinRows) return MlpTiles{256, 4};
  if (per_expert >= 256) return MlpTiles{320, 6};
  return MlpTiles{128, 3};
}

// the direct-to-LDS kernels (variants 3, 4 and 6) always read the plan kernel's output; the
// register-staged ones build it themselves when there is one rank
bool mlp_reads_plan(const MlpTiles& tiles) { return tiles.variant == 3 || tiles.variant == 4 || tiles.variant == 6; }

int mlp_down_cols(const MlpTiles& tiles) {
  switch (tiles.variant) {
    case 3: return kDlBn;
    case 4: return kPpBn;
    case 6: return 256;
    case 0: return kPreBn;
    case 1:
    case 5: return kDecDnBn;
    default: return 64;  // fp32
  }
}

namespace {
template <bool COMBINE>
void launch_gemms(const GemmArgs& gu, const GemmArgs& dn, const MlpTiles& tiles, int64_t max_mtiles, int64_t rows_max,
                  int H, int F, int num_cus, hipStream_t stream) {
  switch (tiles.variant) {
    case 3:  // 128 x 256 direct-to-LDS tiles
      launch_dl<128, kDlBn, kDlWm, kDlWn, kDlNs, kDlSpread, COMBINE>(
          gu, dn, max_mtiles, H, F, rows_max * (int64_t)H * 2, rows_max * (int64_t)F * 2, num_cus, stream);
      break;
    case 4:  // 256 x 256 tiles with the ping-pong wave schedule
      launch_pp<256, kPpBn, 4, 2, COMBINE>(gu, dn, max_mtiles, H, F, rows_max * (int64_t)H * 2,
                                           rows_max * (int64_t)F * 2, num_cus, stream);
      break;
    case 6:  // one 320-row tile holds a whole expert of up to 320 rows: its weights are read once. On 256
             // experts of 192-512 rows at H 7168, F 2048 (same output bits; two kernel traces each):
             // the cross-stage schedule took gate/up 4707 -> 4382 us and down 2620 -> 2555 us, the
             // cross-tile prefetch then 4411 -> 4360 and 2562 -> 2528
      launch_xs<320, 256, 2, 4, COMBINE>(gu, dn, max_mtiles, H, F, rows_max * (int64_t)H * 2, rows_max * (int64_t)F * 2,
                                         num_cus, stream);
      break;
    case 0: {  // bf16, many rows per expert, operands staged through registers
      const int g1 = persistent_grid(max_mtiles * ceil_div_host(F, kPreBn / 2), num_cus, kPreWpc);
      launch_gemm<bf16_t, PreOp, kPreBm, kPreBn, kPreBk, kPreWm, kPreWn, true, kPreRs,
                  kPreLdb, false>(gu, g1, stream);
      const int g2 = persistent_grid(max_mtiles * ceil_div_host(H, kPreBn), num_cus, kPreWpc);
      launch_gemm<bf16_t, PreOp, kPreBm, kPreBn, kPreBk, kPreWm, kPreWn, false, kPreRs,
                  kPreLdb, false, COMBINE>(dn, g2, stream);
      break;
    }
    case 1:  // bf16, few rows per expert: stream the weights through 32- or 64-row tiles
      launch_decode<32, COMBINE>(gu, dn, max_mtiles, H, F, num_cus, stream);
      break;
    case 5:
      launch_decode<64, COMBINE>(gu, dn, max_mtiles, H, F, num_cus, stream);
      break;
    default: {  // fp32
      const int g1 = persistent_grid(max_mtiles * ceil_div_host(F, 32), num_cus, 2);
      launch_gemm<float, OpF32, 32, 64, 32, 1, 2, true, 2, 2, false>(gu, g1, stream);
      const int g2 = persistent_grid(max_mtiles * ceil_div_host(H, 64), num_cus, 2);
      launch_gemm<float, OpF32, 32, 64, 32, 1, 2, false, 2, 2, false, COMBINE>(dn, g2, stream);
      break;
    }
  }
}
}  // namespace

hipError_t launch_expert_mlp(const void* send_buf, int xdt_bf16, const moe_layout_t& L, const void* w_gate_up,
                             const void* w_down, int F, void* out_buf, int* plan, int* perm, void* hbuf,
                             const MlpTiles& tiles, int num_cus, hipStream_t stream, const float* a_scale,
                             const float* topk_w, void* y, int* counter) {
  if (a_scale != nullptr && moe_rows_max(L.T, L.k, L.E, L.C) > 0) {
    // fp8 rows: expand them to bf16 in out_buf (rows_max x H bf16, unused until the down GEMM writes it in
    // a later launch) and run the bf16 GEMMs on them. Decoding inside the gate/up GEMM instead (codes
    // through registers) measured slower on every workload: it rules out the direct-to-LDS tiles.
    // one thread per FP8_EXPAND_CHUNKS chunks of the rows_max rows; those past the kept rows exit at once
    const int64_t chunks = moe_rows_max(L.T, L.k, L.E, L.C) * (int64_t)(L.H / 16);
    const int g = (int)ceil_div_host64(chunks, 256 * FP8_EXPAND_CHUNKS);
    fp8_rows_to_bf16_kernel<<<g, 256, 0, stream>>>(static_cast<const uint8_t*>(send_buf), a_scale,
                                                   L.expert_offset + L.E, L.H, static_cast<bf16_t*>(out_buf));
    send_buf = out_buf;
  }
  const int El = L.E / L.R;
  const int H = L.H;
  const int64_t rows_max = moe_rows_max(L.T, L.k, L.E, L.C);
  // with one rank the send rows are already grouped by local expert: the register-staged GEMMs build the
  // plan's starts from the expert offsets themselves and read rows in send order, with no plan launch
  // (the direct-to-LDS kernels always read the plan kernel's output)
  const bool own_plan = L.R > 1 || mlp_reads_plan(tiles);
  if (own_plan) {
    const int plan_blocks = (int)(rows_max > 0 ? ceil_div_host64(rows_max, PLAN_ROWS_PER_WG) : 1);
    mlp_plan_kernel<<<plan_blocks, PLAN_THREADS, 0, stream>>>(L.expert_kept, L.expert_offset, L.E, El, tiles.BM,
                                                              plan, perm);
  }

  const int64_t max_mtiles = ceil_div_host64(rows_max, tiles.BM) + El;

  GemmArgs gu{};
  gu.A = send_buf;
  gu.lda = H;
  gu.a_perm = own_plan ? perm : nullptr;
  gu.W = w_gate_up;
  gu.w_stride = (int64_t)2 * F * H;
  gu.K = H;
  gu.N = F;
  gu.up_offset = F;
  gu.Out = hbuf;
  gu.ldo = F;
  gu.out_perm = nullptr;
  gu.plan = own_plan ? plan : nullptr;
  gu.offset = L.expert_offset;
  gu.El = El;
  gu.a_bytes = buffer_bytes(rows_max * H * (xdt_bf16 ? 2 : 4));
  gu.w_bytes = buffer_bytes(gu.w_stride * (xdt_bf16 ? 2 : 4));
  gu.k_rotate = k_rotate_for(H, xdt_bf16 ? 2 : 4);
  // the whole-expert kernel keeps the fp32 partials of its K-split tail tiles in h's rows past the total
  gu.out_bytes = buffer_bytes(rows_max * F * (xdt_bf16 ? 2 : 4));
  gu.split_ctr = own_plan ? plan + 4 + 2 * El : nullptr;

  GemmArgs dn{};
  dn.A = hbuf;
  dn.lda = F;
  dn.a_perm = nullptr;
  dn.W = w_down;
  dn.w_stride = (int64_t)H * F;
  dn.K = F;
  dn.N = H;
  dn.up_offset = 0;
  dn.Out = out_buf;
  dn.ldo = H;
  dn.out_perm = own_plan ? perm : nullptr;
  dn.plan = own_plan ? plan : nullptr;
  dn.offset = L.expert_offset;
  dn.El = El;
  dn.a_bytes = buffer_bytes(rows_max * F * (xdt_bf16 ? 2 : 4));
  dn.w_bytes = buffer_bytes(dn.w_stride * (xdt_bf16 ? 2 : 4));
  dn.k_rotate = k_rotate_for(F, xdt_bf16 ? 2 : 4);

  // the direct-to-LDS kernels dereference the plan: never launch them without one
  if (mlp_reads_plan(tiles) && (gu.plan == nullptr || dn.plan == nullptr)) return hipErrorInvalidValue;
  if (y != nullptr) {
    // the combine fused into the down GEMM: counters zeroed and the y rows of tokens with no kept slot
    // cleared first
    const int n_bands = ceil_div_host(H, mlp_down_cols(tiles));
    dn.row_token = L.row_token;
    dn.pair_row = L.pair_row;
    dn.topk_w = topk_w;
    dn.counter = counter;
    dn.y = y;
    dn.k = L.k;
    dn.out_bytes = buffer_bytes(rows_max * H * (xdt_bf16 ? 2 : 4));
    const int64_t work = std::max<int64_t>((int64_t)L.T * n_bands, (int64_t)L.T * (H / (xdt_bf16 ? 8 : 4)));
    if (work > 0) {
      const unsigned g = (unsigned)ceil_div_host64(work, 256);
      if (xdt_bf16)
        combine_prep_kernel<bf16_t><<<g, 256, 0, stream>>>(L.pair_row, L.T, L.k, H, n_bands, counter,
                                                           static_cast<bf16_t*>(y));
      else
        combine_prep_kernel<float><<<g, 256, 0, stream>>>(L.pair_row, L.T, L.k, H, n_bands, counter,
                                                          static_cast<float*>(y));
    }
    launch_gemms<true>(gu, dn, tiles, max_mtiles, rows_max, H, F, num_cus, stream);
  } else {
    launch_gemms<false>(gu, dn, tiles, max_mtiles, rows_max, H, F, num_cus, stream);
  }
  return hipGetLastError();
}

}  // namespace moe
