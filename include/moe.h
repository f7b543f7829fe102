/*
 * moe.h -- C ABI of the MI355X (gfx950) MoE-layer hot path: one GPU's share of an expert-parallel
 * Mixture-of-Experts layer, run as four calls on one HIP stream:
 *
 *   moe_route      -> router logits, top-k experts and their weights per token
 *   moe_dispatch   -> per-expert histogram, prefix scan with a capacity limit, stable scatter of
 *                     token rows into contiguous, destination-rank-aligned per-expert rows
 *   moe_expert_mlp -> per-expert SwiGLU MLP over the dispatched rows (grouped bf16 MFMA GEMM)
 *   moe_combine    -> router-weighted sum of each token's expert outputs, back in token order
 *
 * plus an fp8 variant of the dispatch and of the expert MLP (moe_dispatch_fp8, moe_expert_mlp_fp8).
 *
 * Sources (cited by page title and section):
 *   [EPM] "Efficient and portable mixture-of-experts communication" (Perplexity, 2025)
 *   [EFA] "Enabling trillion-parameter models on AWS EFA" (Perplexity, 2025)
 *   [OVL] "Mixture-of-experts acceleration through overlap" (thecoregrid.dev)
 *   [EPB] "80. MoE Expert Parallel Benchmark" (datawhalechina llm-algo-leetcode)
 *   [DMoE] "DistributedMoE" (README)
 *
 * Conventions shared by every call:
 *   - All pointers except `moe_layout_t*` itself are DEVICE pointers, owned by the caller. The library
 *     allocates nothing, keeps no state between calls and never synchronises with the host; each
 *     call only enqueues kernels on `stream` (NULL = the default stream) and returns.
 *   - Row-major layouts, 32-bit indices. Activations and expert weights share one type `xdt`
 *     (MOE_F32 or MOE_BF16); the router weight, bias, logits and routing weights are fp32.
 *   - Alignment: activations, expert and router weights, send / output / partial rows (and fp8 codes)
 *     and workspaces must be 16-byte aligned; int32 and fp32 arrays (ids, weights, logits, bias, block
 *     scales, layout arrays) 4-byte aligned. Anything else is MOE_ERR_INVALID. hipMalloc and PyTorch
 *     allocations are 256-byte aligned.
 *   - Return value: MOE_OK, or a negative status. Arguments are validated on the host before any
 *     HIP call; on MOE_ERR_INVALID / MOE_ERR_UNSUPPORTED nothing was enqueued. MOE_ERR_HIP means a
 *     launch failed (hipGetLastError); earlier kernels of the same call may have run.
 *   - Same inputs give bitwise-identical outputs: no floating-point atomics anywhere.
 *   - Calls on different streams with disjoint buffers are independent.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype_t;

enum {
  MOE_OK = 0,
  MOE_ERR_INVALID = -1,     /* null or misaligned pointer, out-of-range size, inconsistent layout */
  MOE_ERR_UNSUPPORTED = -2, /* a shape or dtype the kernels do not handle (e.g. H % 8 != 0) */
  MOE_ERR_HIP = -3          /* a kernel launch failed */
};

/* Limits checked on the host. */
#define MOE_MAX_EXPERTS 512
#define MOE_MAX_TOPK 8

/* Text for a status code (static storage). */
const char* moe_status_string(int status);

/*
 * Layout descriptor of the per-rank send buffers ([EFA] "Диспетчеризация и комбинирование": counts
 * per expert, a cumulative sum gives the offsets, tokens are packed into contiguous per-peer send
 * buffers; [OVL]: each tile belongs to one destination rank, so a transfer is one contiguous write;
 * [EPM] "Dispatch": the receiver keeps (source rank, expert, token) for the combine).
 *
 * The caller fills the scalars and allocates the arrays (device memory, int32); moe_dispatch fills
 * the arrays. E experts are split over R destination ranks, El = E / R per rank, expert e on rank
 * e / El. Rows are ordered by expert id and, inside an expert, by token (stable). Rank r's segment is
 * rows [expert_offset[r*El], expert_offset[(r+1)*El]). Rows >= expert_offset[E] are unspecified.
 *
 *   expert_count[E]     tokens routed to each expert (the router histogram)
 *   expert_kept[E]      min(count, C)                      ([EPB] Step 2)
 *   expert_overflow[E]  max(count - C, 0)                  ([EPB] Step 2)
 *   expert_offset[E+1]  exclusive prefix sum of kept; [E] = total rows
 *   row_token[rows_max] source token of each row
 *   row_slot[rows_max]  k-slot of each row
 *   pair_row[T*k]       row of pair (t, j), or -1 if the pair was dropped by the capacity limit
 *
 * rows_max = moe_rows_max(T, k, E, C) = min(T*k, E*C) bounds the row count from host scalars alone.
 */
typedef struct moe_layout {
  int32_t T;  /* tokens */
  int32_t k;  /* experts per token, 1..MOE_MAX_TOPK */
  int32_t E;  /* experts, 1..MOE_MAX_EXPERTS */
  int32_t R;  /* destination ranks, E % R == 0 */
  int32_t C;  /* per-expert capacity, >= 0 (an integer: the caller rounds cf*T*k/E) */
  int32_t H;  /* hidden size, % 8 == 0 */
  int32_t* expert_count;
  int32_t* expert_kept;
  int32_t* expert_overflow;
  int32_t* expert_offset;
  int32_t* row_token;
  int32_t* row_slot;
  int32_t* pair_row;
} moe_layout_t;

/* min(T*k, E*C): the most rows dispatch can produce. Negative arguments give 0. */
int64_t moe_rows_max(int T, int k, int E, int C);

/*
 * moe_route -- router scores and top-k selection.
 * [EPM] "Introductie": the router is a small linear layer giving a probability distribution over the
 * experts; the top-K experts are chosen and the output is a weighted average with weights derived
 * from that distribution. [EFA] "Введение": a small routing linear layer picks the experts.
 *
 *   x            [T, H] activations (xdt)
 *   w_router     [E, H] fp32 router weight
 *   logit_bias   NULL, or fp32 bias added to the logits; row t reads logit_bias[t*bias_row_stride + e]
 *                (stride 0: one [E] row for all tokens; stride E: a [T, E] matrix)
 *   logits       [T, E] fp32 output: sum_h x[t,h] * w_router[e,h] + bias, accumulated in fp32. Every
 *                product is the exact fp32 product: with E <= 16 and T <= 4096 by fp32 FMAs, one
 *                workgroup per token; otherwise on MFMA (bf16 x: bf16 MFMA with w_router split exactly
 *                into three bf16 parts; fp32 x: fp32 MFMA)
 *   topk_ids     [T, k] int32 output: the k largest logits, descending, equal logits ordered by the
 *                lower expert id, -0 == +0 (slot 0 = best); a NaN logit ranks as -inf (ties among
 *                infinities and NaN also go to the lower id)
 *   topk_w       [T, k] fp32 output: softmax over the k selected logits (sums to 1); unspecified for a
 *                token whose selected logits are not all finite
 *   workspace    device scratch of at least moe_route_workspace_bytes(T, H, E, xdt) bytes
 * Requires 1 <= k <= min(E, MOE_MAX_TOPK), E <= MOE_MAX_EXPERTS, H % 8 == 0, T >= 0 (T == 0 is a
 * no-op).
 */
int moe_route(const void* x, moe_dtype_t xdt, const float* w_router, const float* logit_bias,
              int64_t bias_row_stride, int T, int H, int E, int k, float* logits, int32_t* topk_ids,
              float* topk_w, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of scratch `workspace` moe_route needs for (T, H, E, xdt): for bf16 activations with
 * T >= 2048 and H % 64 == 0, the router weight split into three exact bf16 planes (3 * E * H * 2
 * bytes); fp32 partial sums when the H reduction is split across workgroups. 0 when neither applies
 * (e.g. for E <= 16 and T <= 4096; workspace may then be NULL). */
size_t moe_route_workspace_bytes(int T, int H, int E, moe_dtype_t xdt);

/* Bytes of scratch `workspace` moe_dispatch needs for (T, k, E). */
size_t moe_dispatch_workspace_bytes(int T, int k, int E);

/*
 * moe_dispatch -- partition (token, slot) pairs by expert into contiguous per-expert rows.
 * [EFA] "Диспетчеризация и комбинирование": per-expert counts by atomic accumulation in on-chip
 * memory, a cumulative sum of the counts gives the offsets, tokens are packed into contiguous send
 * buffers. [EPB] Step 2: capacity is the per-expert limit of one step; overflow = max(assigned -
 * capacity, 0). [EPM] "Dispatch": tokens are regrouped into contiguous per-expert buffers that feed
 * the grouped GEMM, and (rank, expert, token) is kept per row for the combine.
 *
 * Pairs are admitted first come first served in row-major (t, j) order: pair (t, j) of expert e is
 * kept iff fewer than C earlier pairs chose e; kept rows are bit copies of x[t].
 *   x          [T, H] activations (xdt); T, H, k, E, R, C are read from `layout`
 *   topk_ids   [T, k] int32 expert ids (distinct within a token, in [0, E))
 *   layout     host struct with scalars set and device arrays allocated (see moe_layout_t)
 *   send_buf   [rows_max, H] (xdt) output rows
 *   workspace  device scratch of at least moe_dispatch_workspace_bytes(T, k, E) bytes
 * Ids outside [0, E) give unspecified output (they are not written anywhere out of bounds).
 */
int moe_dispatch(const void* x, moe_dtype_t xdt, const int32_t* topk_ids, const moe_layout_t* layout,
                 void* send_buf, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * moe_dispatch_noalloc -- moe_dispatch for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation): no workspace argument.
 * Its scratch (per-block expert counts and in-block ranks) is a static device array of
 * MOE_DISPATCH_NOALLOC_MAX_WORKSPACE bytes inside the library, one per GPU, held until the process
 * ends; its address is looked up once per device on the first call there. Arguments, outputs and
 * results are those of moe_dispatch, bit for bit.
 * Returns MOE_ERR_UNSUPPORTED (nothing enqueued) when moe_dispatch_workspace_bytes(T, k, E) exceeds
 * MOE_DISPATCH_NOALLOC_MAX_WORKSPACE (e.g. 65536 tokens x top-8 x 512 experts still fits), and
 * MOE_ERR_HIP if the array's address cannot be found. Every call on one GPU uses the same array:
 * calls that may overlap on one GPU (different streams without ordering between them) race and
 * must not be made. Calls on one stream are ordered and safe.
 */
#define MOE_DISPATCH_NOALLOC_MAX_WORKSPACE (4u << 20)
int moe_dispatch_noalloc(const void* x, moe_dtype_t xdt, const int32_t* topk_ids, const moe_layout_t* layout,
                         void* send_buf, hipStream_t stream);

/* Bytes of scratch `workspace` moe_expert_mlp needs for this layout and FFN width. */
size_t moe_expert_mlp_workspace_bytes(int T, int k, int E, int R, int C, int F, moe_dtype_t xdt);

/*
 * moe_expert_mlp -- per-expert SwiGLU MLP on the dispatched rows, as a grouped GEMM.
 * [EFA] "MoE all-to-all через EFA": grouped GEMM kernels multiply the regrouped tokens by the expert
 * weights. [OVL]: one persistent GEMM processes every expert of the rank without relaunching.
 * [DMoE] "Результаты": grouped GEMM helps most when many experts are active.
 *
 * A row of global expert e uses local expert l = e mod El (El = E / R):
 *   g = x Wg[l]^T, u = x Wu[l]^T (fp32 accumulate), h = silu(g) * u stored as xdt,
 *   out = h Wd[l]^T (fp32 accumulate) stored as xdt.
 *   send_buf   [rows_max, H] rows written by moe_dispatch (xdt)
 *   layout     the layout moe_dispatch filled (expert_kept / expert_offset are read on the device)
 *   w_gate_up  [El, 2F, H] (xdt): rows 0..F-1 are Wg, rows F..2F-1 are Wu (nn.Linear [out, in])
 *   w_down     [El, H, F] (xdt)
 *   out_buf    [rows_max, H] (xdt) output, row-aligned with send_buf; rows >= total unspecified
 *   workspace  device scratch of at least moe_expert_mlp_workspace_bytes(...) bytes: the tile plan and
 *              its counters, the gather map and h; no contents need clearing between calls, and calls
 *              that overlap must use separate workspaces
 * Requires H % 8 == 0 and F % 8 == 0. bf16 runs on bf16 MFMA, fp32 on fp32 MFMA.
 */
int moe_expert_mlp(const void* send_buf, moe_dtype_t xdt, const moe_layout_t* layout,
                   const void* w_gate_up, const void* w_down, int F, void* out_buf, void* workspace,
                   size_t workspace_bytes, hipStream_t stream);

/*
 * moe_combine -- router-weighted sum back in token order.
 * [EPM] "Combine": the payloads are read from the per-expert buffers, the routing table says which
 * buffer to read and which weight each expert gets, and the result is written to caller-allocated
 * tensors. [EFA] "Буферы отправки и получения": combine reads the receive buffer and computes the
 * weighted average of the tokens into the output tensors.
 *
 *   y[t] = sum over kept slots j, ascending, of topk_w[t,j] * out_buf[pair_row[t,j]],
 *   accumulated in fp32 and rounded once to xdt; a token with every pair dropped gets y[t] = 0.
 *   out_buf  [rows_max, H] (xdt) expert outputs, row-aligned with send_buf
 *   layout   the layout moe_dispatch filled (pair_row is read on the device)
 *   topk_w   [T, k] fp32 routing weights
 *   y        [T, H] (xdt) output
 */
int moe_combine(const void* out_buf, moe_dtype_t xdt, const moe_layout_t* layout,
                const float* topk_w, void* y, hipStream_t stream);

/*
 * moe_expert_mlp_combine -- moe_expert_mlp with moe_combine fused into its down GEMM: one call writes
 * out_buf and y.
 * [OVL] "tile-level signalling": the GEMM epilogue publishes per-tile readiness and the consumer starts
 * on a segment as soon as the tiles it needs are done, instead of after the whole GEMM. Here every
 * down-GEMM tile, once it has stored its rows, counts them per (token, column band); the tile that
 * completes a token's band computes that band of y at once, so the combine of early bands overlaps the
 * tiles still running. No workgroup ever waits for another.
 *   y[t] = sum over kept slots j, ascending, of topk_w[t,j] * out_buf[pair_row[t,j]], accumulated in
 *   fp32 and rounded once; equal bit for bit to moe_expert_mlp followed by moe_combine.
 *   send_buf, layout, w_gate_up, w_down, F, out_buf  as for moe_expert_mlp
 *   topk_w     [T, k] fp32 routing weights
 *   y          [T, H] (xdt) output
 *   workspace  device scratch of at least moe_expert_mlp_combine_workspace_bytes(T, k, E, R, C, H, F, xdt)
 *              bytes: the expert-MLP scratch plus one int per (token, column band), cleared by the call
 * Calls that overlap on one stream or device must use separate workspaces.
 */
size_t moe_expert_mlp_combine_workspace_bytes(int T, int k, int E, int R, int C, int H, int F, moe_dtype_t xdt);
int moe_expert_mlp_combine(const void* send_buf, moe_dtype_t xdt, const moe_layout_t* layout,
                           const void* w_gate_up, const void* w_down, int F, const float* topk_w,
                           void* out_buf, void* y, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/*
 * Combine with sender-side partial accumulation: moe_combine_send then moe_combine_recv.
 * [EFA] "Оценка": the pages' combine accumulates only at the receiver, so one row per kept pair crosses
 * the link; DeepEP accumulates at the sender to move fewer bytes, with a possible precision cost. Here
 * the expert side sends one partial row per (destination rank, token) instead, and the token's side sums
 * them. The rank of a row is the r with expert_offset[r*El] <= row < expert_offset[(r+1)*El].
 *
 * moe_combine_send -- for every token t and rank r holding at least one kept slot of t:
 *   partial[r, t] = sum over those slots j, ascending, of topk_w[t,j] * out_buf[pair_row[t,j]],
 *   accumulated in fp32 and rounded once to xdt (the extra rounding is the precision cost).
 *   out_buf  [rows_max, H] (xdt) expert outputs, as for moe_combine
 *   topk_w   [T, k] fp32 routing weights
 *   partial  [R, T, H] (xdt), rank-major: what rank r returns is one contiguous block. Slots (r, t)
 *            with no kept slot are not written.
 * moe_combine_recv -- y[t] = sum over the ranks r holding kept slots of t, ascending, of partial[r, t],
 *   accumulated in fp32 and rounded once; a token with every pair dropped gets y[t] = 0.
 *   partial  as written by moe_combine_send for the same layout
 *   y        [T, H] (xdt) output
 * With R == 1 the result equals moe_combine's bit for bit. Both return MOE_OK at once when T == 0.
 */
int moe_combine_send(const void* out_buf, moe_dtype_t xdt, const moe_layout_t* layout, const float* topk_w,
                     void* partial, hipStream_t stream);
int moe_combine_recv(const void* partial, moe_dtype_t xdt, const moe_layout_t* layout, void* y,
                     hipStream_t stream);

/*
 * fp8 block-scaled dispatch.
 * [EPM] "Dispatch": the send side packs the tokens together with their block scale factors.
 * [EFA] "Оценка": dispatch runs with fp8 block scaling, combine in bf16. The pages fix neither the fp8
 * format nor the block or the scale; the readings here:
 *   - codes: OCP FP8 E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; largest finite 448,
 *     no infinities);
 *   - one scale per MOE_FP8_BLOCK consecutive hidden elements of a row, a power of two 2^E with E the
 *     smallest integer such that max|x| / 2^E <= 448 (E = 0 for an all-zero block);
 *   - code = x / 2^E rounded to the nearest E4M3 value, ties to the even mantissa, magnitudes above 448
 *     clamped to 448, sign kept for values rounding to zero;
 *   - the value a code stands for, code * 2^E, is exactly a bfloat16 value.
 */
#define MOE_FP8_BLOCK 128

/*
 * moe_dispatch_fp8 -- moe_dispatch whose send rows are fp8 block-scaled instead of copies of x.
 * The layout (counts, capacity drops, offsets, row_token / row_slot / pair_row) is exactly the one
 * moe_dispatch writes; send row i holds x[row_token[i]] quantised as above.
 *   x          [T, H] bf16 activations (xdt must be MOE_BF16), finite (the codes of a block holding an
 *              infinity or NaN are unspecified); H % MOE_FP8_BLOCK == 0
 *   topk_ids   [T, k] int32 expert ids
 *   layout     as for moe_dispatch
 *   send_q     [rows_max, H] uint8 E4M3 codes (output)
 *   send_scale [rows_max, H / MOE_FP8_BLOCK] fp32 block scales (output), each a power of two
 *   workspace  device scratch of at least moe_dispatch_workspace_bytes(T, k, E) bytes
 */
int moe_dispatch_fp8(const void* x, moe_dtype_t xdt, const int32_t* topk_ids, const moe_layout_t* layout,
                     uint8_t* send_q, float* send_scale, void* workspace, size_t workspace_bytes,
                     hipStream_t stream);

/*
 * moe_expert_mlp_fp8 -- moe_expert_mlp on fp8 block-scaled rows: each activation enters the gate/up
 * GEMM as the bf16 value code * scale (exact); everything else is moe_expert_mlp in bf16. The rows are
 * first expanded to bf16 in out_buf, which the down GEMM then overwrites with the results.
 *   send_q, send_scale  rows written by moe_dispatch_fp8
 *   layout              the layout moe_dispatch_fp8 filled
 *   w_gate_up, w_down   bf16 expert weights, as for moe_expert_mlp
 *   out_buf             [rows_max, H] bf16 output, row-aligned with send_q (feeds moe_combine)
 *   workspace           device scratch of at least moe_expert_mlp_workspace_bytes(T, k, E, R, C, F, MOE_BF16)
 * Requires H % MOE_FP8_BLOCK == 0 and F % 8 == 0 (else MOE_ERR_UNSUPPORTED).
 */
int moe_expert_mlp_fp8(const uint8_t* send_q, const float* send_scale, const moe_layout_t* layout,
                       const void* w_gate_up, const void* w_down, int F, void* out_buf, void* workspace,
                       size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
