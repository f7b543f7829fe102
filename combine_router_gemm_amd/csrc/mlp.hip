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
//                 the workgroup -> tile map groups consecutive tiles on one XCD (workgroups are dealt
//                 to the 8 XCDs round robin, and each XCD has its own L2).
//                 Gate/up pass: A rows gathered through perm from the send buffer, B = the gate and the
//                 up rows of the same output columns, epilogue h = silu(g) * u (fp32) stored as xdt.
//                 Down pass: A = h in plan order, epilogue stores to out_buf[perm[p]] as xdt.
//   Operands are staged global -> registers -> LDS with several stages of global loads in flight and
//   two LDS stages (one barrier per stage). Compute-bound bf16 tiles use v_mfma_f32_32x32x16_bf16,
//   weight-streaming bf16 tiles v_mfma_f32_16x16x32_bf16, fp32 v_mfma_f32_16x16x4_f32; all accumulate
//   in fp32.
#include "common.h"
#include "kernels.h"
#include "mfma.h"

namespace moe {

namespace {

// ------------------------------------------------------------------------------------------------
// plan
// ------------------------------------------------------------------------------------------------
// plan layout (int32): [0] total M-tiles, [1] total rows, [2 .. 2+El] row start per local expert
// (El+1 entries), [3+El .. 3+2El] M-tile start per local expert (El+1 entries).
constexpr int PLAN_THREADS = 1024;  // >= MOE_MAX_EXPERTS: one thread per (local or global) expert
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
  const int* plan;
  int El;
};

// BM x BN tile, BK-deep LDS stages, WM x WN waves, MFMA op Op. GATED: the B tile holds BN/2 gate rows
// then the BN/2 up rows of the same output columns, and each wave owns matching gate and up
// accumulators.
template <typename T, typename Op, int BM, int BN, int BK, int WM, int WN, bool GATED, int RS, int LDB, bool BNT>
__global__ __launch_bounds__(WM* WN * 64) void mlp_gemm_kernel(GemmArgs args) {
  constexpr int NTH = WM * WN * 64;
  constexpr int VN = Vec<T>::N;           // elements per 16-byte vector
  constexpr int PAD = 16 / sizeof(T);     // one vector of padding per LDS row
  constexpr int LDR = BK + PAD;           // LDS row length (elements)
  constexpr int VPR = BK / VN;            // vectors per tile row per stage
  constexpr int A_VEC = BM * VPR / NTH;   // A vectors loaded per thread per stage
  constexpr int B_VEC = BN * VPR / NTH;
  constexpr int WTM = BM / WM, WTN = BN / WN;  // wave tile
  constexpr int S = Op::S;
  constexpr int TM = WTM / S;
  constexpr int TN = GATED ? (BN / 2 / WN) / S : WTN / S;  // per half when gated
  constexpr int NACC = GATED ? 2 * TN : TN;
  constexpr int OUT_COLS = GATED ? BN / 2 : BN;  // output columns per tile
  static_assert(BM * VPR % NTH == 0 && BN * VPR % NTH == 0, "loader must tile evenly");
  static_assert(TM >= 1 && TN >= 1, "wave tile too small");
  static_assert(BK % Op::KS == 0 && BK % 32 == 0, "BK must be a multiple of the MFMA K step");
  static_assert(TM * S == WTM && (GATED ? TN * S * WN * 2 == BN : TN * S == WTN), "wave tile must tile by S");

  // LDB = 2: two LDS stages, the MFMAs read one while the next stage is written into the other (one
  // barrier per stage). LDB = 1: one LDS stage and two barriers per stage, half the LDS, so more
  // workgroups fit on a CU; the RS register stages keep the global loads in flight either way.
  static_assert(LDB == 1 || LDB == 2, "one or two LDS stages");
  __shared__ __attribute__((aligned(16))) T As[LDB][BM * LDR];
  __shared__ __attribute__((aligned(16))) T Bs[LDB][BN * LDR];

  const T* __restrict__ A = static_cast<const T*>(args.A);
  const T* __restrict__ W = static_cast<const T*>(args.W);
  T* __restrict__ Out = static_cast<T*>(args.Out);
  const int El = args.El;
  const int* row_start = args.plan + 2;
  const int* tile_start = args.plan + 3 + El;
  const int n_tiles = (args.N + OUT_COLS - 1) / OUT_COLS;
  const int total = args.plan[0] * n_tiles;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // XCD-aware order: workgroup b runs on XCD b % 8; give each XCD a contiguous run of tile ids
  const int G = gridDim.x;
  int vb = blockIdx.x;
  if ((G & 7) == 0) vb = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);

  for (int tile = vb; tile < total; tile += G) {
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
    const T* a_src[A_VEC];
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
    }
    const T* b_src[B_VEC];
    int b_lds[B_VEC];
    bool b_ok[B_VEC];
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
    u32x4 ra[RS][A_VEC], rb[RS][B_VEC];
    const u32x4 zero = {0u, 0u, 0u, 0u};
    auto load_stage = [&](int st, u32x4 (&xa)[A_VEC], u32x4 (&xb)[B_VEC]) {
      const int k0 = st * BK;
#pragma unroll
      for (int i = 0; i < A_VEC; ++i) xa[i] = ld16(a_src[i] + min(k0 + a_lds[i] % LDR, args.K - VN));
#pragma unroll
      for (int i = 0; i < B_VEC; ++i) {
        // weights are read once per tile: streaming (non-temporal) loads keep the reused activation
        // rows resident in L2 when many tiles share them
        const T* pb = b_src[i] + min(k0 + b_lds[i] % LDR, args.K - VN);
        xb[i] = BNT ? ld16_nt(pb) : ld16(pb);
      }
    };
    auto store_stage = [&](int st, int buf, const u32x4 (&xa)[A_VEC], const u32x4 (&xb)[B_VEC]) {
      const int k0 = st * BK;
#pragma unroll
      for (int i = 0; i < A_VEC; ++i) st16(&As[buf][a_lds[i]], (a_ok[i] && k0 + a_lds[i] % LDR < args.K) ? xa[i] : zero);
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

    // epilogue: lane l holds column l % S of each S x S accumulator; Op::out_row gives the rows
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
            const int p = p0 + row;
            const int orow = args.out_perm ? args.out_perm[p] : p;
            Out[(int64_t)orow * args.ldo + col] = from_f32<T>(v);
          }
        }
      }
    }
  }
}

template <typename T, typename Op, int BM, int BN, int BK, int WM, int WN, bool GATED, int RS, int LDB, bool BNT>
void launch_gemm(const GemmArgs& a, int grid, hipStream_t stream) {
  mlp_gemm_kernel<T, Op, BM, BN, BK, WM, WN, GATED, RS, LDB, BNT><<<grid, WM * WN * 64, 0, stream>>>(a);
}

// Persistent grid sizes in workgroups per CU and the compute-bound tile shapes; overridable at compile
// time for tuning sweeps.
#ifndef MOE_DEC_WPC
#define MOE_DEC_WPC 3
#endif
#ifndef MOE_PRE_WPC
#define MOE_PRE_WPC 1
#endif
// many-rows-per-expert (compute-bound) tiles: BM x BN x BK with WM x WN waves
#ifndef MOE_PRE_BM
#define MOE_PRE_BM 128
#endif
#ifndef MOE_PRE_BN
#define MOE_PRE_BN 256
#endif
#ifndef MOE_PRE_BK
#define MOE_PRE_BK 64
#endif
#ifndef MOE_PRE_WM
#define MOE_PRE_WM 2
#endif
#ifndef MOE_PRE_WN
#define MOE_PRE_WN 4
#endif

#ifndef MOE_PRE_OP
#define MOE_PRE_OP Op32
#endif
// register stages of global prefetch in flight
#ifndef MOE_PRE_RS
#define MOE_PRE_RS 2
#endif
#ifndef MOE_DEC_RS
#define MOE_DEC_RS 2
#endif
#ifndef MOE_PRE_LDB
#define MOE_PRE_LDB 2
#endif
#ifndef MOE_DEC_LDB
#define MOE_DEC_LDB 1
#endif
// few-rows-per-expert (weight streaming) tiles: 32 rows, BN weight rows, BK deep
#ifndef MOE_DEC_GU_BN
#define MOE_DEC_GU_BN 128
#endif
#ifndef MOE_DEC_GU_BK
#define MOE_DEC_GU_BK 64
#endif
#ifndef MOE_DEC_DN_BN
#define MOE_DEC_DN_BN 64
#endif
#ifndef MOE_DEC_DN_BK
#define MOE_DEC_DN_BK 128
#endif
constexpr int DEC_GU_WN = MOE_DEC_GU_BN / 32 < 4 ? MOE_DEC_GU_BN / 32 : 4;
constexpr int DEC_DN_WN = MOE_DEC_DN_BN / 16 < 4 ? MOE_DEC_DN_BN / 16 : 4;
using PreOp = MOE_PRE_OP;


int persistent_grid(int64_t max_tiles, int num_cus, int wpc) {
  int64_t g = (int64_t)num_cus * wpc;
  if (max_tiles < g) g = max_tiles;
  if (g >= 8) g &= ~7ll;  // a multiple of the XCD count keeps the XCD-aware order exact
  return (int)(g > 0 ? g : 1);
}

}  // namespace

size_t mlp_plan_ints(int El) { return 2 + 2 * (size_t)(El + 1); }

// variant 0: bf16 prefill tiles, 1: bf16 decode tiles (few rows per expert), 2: fp32
MlpTiles mlp_pick_tiles(int64_t rows_max, int El, int xdt_bf16) {
  if (!xdt_bf16) return MlpTiles{32, 2};
  const int64_t per_expert = El > 0 ? rows_max / El : rows_max;
  if (per_expert >= 128) return MlpTiles{MOE_PRE_BM, 0};
  return MlpTiles{32, 1};
}

hipError_t launch_expert_mlp(const void* send_buf, int xdt_bf16, const moe_layout_t& L, const void* w_gate_up,
                             const void* w_down, int F, void* out_buf, int* plan, int* perm, void* hbuf,
                             const MlpTiles& tiles, int num_cus, hipStream_t stream) {
  const int El = L.E / L.R;
  const int H = L.H;
  const int64_t rows_max = moe_rows_max(L.T, L.k, L.E, L.C);
  const int plan_blocks = (int)(rows_max > 0 ? ceil_div_host64(rows_max, PLAN_ROWS_PER_WG) : 1);
  mlp_plan_kernel<<<plan_blocks, PLAN_THREADS, 0, stream>>>(L.expert_kept, L.expert_offset, L.E, El, tiles.BM, plan,
                                                            perm);

  const int64_t max_mtiles = ceil_div_host64(rows_max, tiles.BM) + El;

  GemmArgs gu{};
  gu.A = send_buf;
  gu.lda = H;
  gu.a_perm = perm;
  gu.W = w_gate_up;
  gu.w_stride = (int64_t)2 * F * H;
  gu.K = H;
  gu.N = F;
  gu.up_offset = F;
  gu.Out = hbuf;
  gu.ldo = F;
  gu.out_perm = nullptr;
  gu.plan = plan;
  gu.El = El;

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
  dn.out_perm = perm;
  dn.plan = plan;
  dn.El = El;

  switch (tiles.variant) {
    case 0: {  // bf16, many rows per expert
      const int g1 = persistent_grid(max_mtiles * ceil_div_host(F, MOE_PRE_BN / 2), num_cus, MOE_PRE_WPC);
      launch_gemm<bf16_t, PreOp, MOE_PRE_BM, MOE_PRE_BN, MOE_PRE_BK, MOE_PRE_WM, MOE_PRE_WN, true, MOE_PRE_RS, MOE_PRE_LDB, false>(gu, g1, stream);
      const int g2 = persistent_grid(max_mtiles * ceil_div_host(H, MOE_PRE_BN), num_cus, MOE_PRE_WPC);
      launch_gemm<bf16_t, PreOp, MOE_PRE_BM, MOE_PRE_BN, MOE_PRE_BK, MOE_PRE_WM, MOE_PRE_WN, false, MOE_PRE_RS, MOE_PRE_LDB, false>(dn, g2, stream);
      break;
    }
    case 1: {  // bf16, few rows per expert: stream the weights through 32-row tiles
      // with many local experts of few rows each, streaming (non-temporal) weight loads in the gate/up
      // pass measured faster; with few experts the default cache policy did
      const int g1 = persistent_grid(max_mtiles * ceil_div_host(F, MOE_DEC_GU_BN / 2), num_cus, MOE_DEC_WPC);
      if (El >= 16)
        launch_gemm<bf16_t, Op16, 32, MOE_DEC_GU_BN, MOE_DEC_GU_BK, 1, DEC_GU_WN, true, MOE_DEC_RS, MOE_DEC_LDB, true>(
            gu, g1, stream);
      else
        launch_gemm<bf16_t, Op16, 32, MOE_DEC_GU_BN, MOE_DEC_GU_BK, 1, DEC_GU_WN, true, MOE_DEC_RS, MOE_DEC_LDB, false>(
            gu, g1, stream);
      const int g2 = persistent_grid(max_mtiles * ceil_div_host(H, MOE_DEC_DN_BN), num_cus, MOE_DEC_WPC);
      launch_gemm<bf16_t, Op16, 32, MOE_DEC_DN_BN, MOE_DEC_DN_BK, 1, DEC_DN_WN, false, MOE_DEC_RS, MOE_DEC_LDB, false>(
          dn, g2, stream);
      break;
    }
    default: {  // fp32
      const int g1 = persistent_grid(max_mtiles * ceil_div_host(F, 32), num_cus, 2);
      launch_gemm<float, OpF32, 32, 64, 32, 1, 2, true, 2, 2, false>(gu, g1, stream);
      const int g2 = persistent_grid(max_mtiles * ceil_div_host(H, 64), num_cus, 2);
      launch_gemm<float, OpF32, 32, 64, 32, 1, 2, false, 2, 2, false>(dn, g2, stream);
      break;
    }
  }
  return hipGetLastError();
}

}  // namespace moe
