/*
 * moe_route.h -- C ABI of the MI355X (gfx950) MoE expert-parallel layer.
 *
 * One MoE layer on one GPU's share, in four calls that follow the layer's
 * data flow as drawn in "MoE 专家并行的 All-to-All 通信瓶颈" (wiblog.cn),
 * section "All-to-All 分发与回收的机制", flowchart: the router picks the
 * Top-K experts (moe_route_topk); tokens are grouped and packed by
 * destination card (moe_dispatch); each expert runs a grouped GEMM over its
 * variable number of tokens (moe_grouped_ffn); the outputs are merged back to
 * token order with the gate weights (moe_combine).  "MoE Inference
 * Communication", section "系统剖析", names the same stages Gate -> dispatch
 * -> Expert FFN -> combine -> Aggregation.  On one GPU the two all-to-all
 * exchanges become the local pack into W virtual-rank send slices and the
 * unpack back to token order.
 *
 * Conventions shared by every call
 *   - Arrays are caller-owned DEVICE pointers, row-major and contiguous, and
 *     16-byte aligned.  The library never allocates, never synchronises the
 *     host and keeps no pointer after a call returns.
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL is the
 *     default stream).  The caller keeps buffers alive until the stream has
 *     passed them.
 *   - Every argument check happens on the host before any launch: a non-OK
 *     status means nothing was enqueued, except MOE_ERR_HIP, which reports a
 *     failed launch (hipGetLastError) after enqueueing.
 *   - moe_last_error() gives a thread-local message for the last failure.
 *   - No global mutable state: calls are thread-safe.
 *   - dtype is a moe_dtype_t value: MOE_DTYPE_F32 or MOE_DTYPE_BF16.  It is
 *     the storage type of activations and weights; arithmetic accumulates in
 *     fp32 and rounds to the storage type (round-to-nearest-even) where a
 *     value is stored.
 */
#ifndef MOE_ROUTE_H
#define MOE_ROUTE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* a null pointer, a size out of range, ... */
  MOE_ERR_UNSUPPORTED = 2, /* legal but beyond this implementation's limits */
  MOE_ERR_WORKSPACE = 3,   /* workspace missing or too small */
  MOE_ERR_HIP = 4          /* a HIP launch failed */
} moe_status_t;

typedef enum { MOE_DTYPE_F32 = 0, MOE_DTYPE_BF16 = 1 } moe_dtype_t;

/* Gate function of the router scores (moe_route_topk_gated). */
typedef enum { MOE_GATE_SOFTMAX = 0, MOE_GATE_SIGMOID = 1 } moe_gate_t;

#define MOE_ABI_VERSION 1
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_TOPK 16
#define MOE_MAX_RANKS 64

/* Version of this ABI (MOE_ABI_VERSION). */
int moe_abi_version(void);

/* Static text naming a status code. */
const char* moe_status_string(int status);

/* Thread-local detail of this thread's last failed call ("" if none). */
const char* moe_last_error(void);

/*
 * Per-expert capacity ceil(C * N * K / E), host only.
 * "MoE 推理服务工程真相 2026", section 2.2 (Expert Capacity Factor): an expert
 * that receives more tokens than its capacity drops the excess.  The page's
 * formula lost its symbols; the budget here is the mean per-expert load
 * N*K/E scaled by C and rounded up, computed exactly on the rational value of
 * the double C.  Returns -2 if C is not finite and > 0, or N < 0, K < 1,
 * E < 1, or the result exceeds INT64_MAX.  Callers pass -1 to moe_dispatch
 * for a dropless layer.
 */
int64_t moe_capacity(double C, int64_t N, int32_t K, int32_t E);

/*
 * Top-K routing.  "MoE 专家并行的 All-to-All 通信瓶颈", section
 * "一个反直觉的扩容结果": the router picks the Top-K experts of each token;
 * "MoE 推理服务工程真相 2026", section 一: it yields the top-k expert weights.
 *
 *   logits     [N, E] fp32, finite (unchecked precondition).
 *   topk_idx   [N, K] int32 out: the K experts with the largest logits,
 *              best first; equal logits go to the lower expert index.
 *   topk_w     [N, K] fp32 out: softmax probability of the chosen expert over
 *              all E logits (max-subtracted); if renormalize != 0, divided by
 *              the sum of the K chosen probabilities.
 * Checks: pointers non-null; N >= 0; 1 <= K <= E (INVALID_ARG);
 *         E <= MOE_MAX_EXPERTS, K <= MOE_MAX_TOPK (UNSUPPORTED).
 * N == 0 enqueues nothing.
 */
int moe_route_topk(const float* logits, int32_t N, int32_t E, int32_t K,
                   int32_t renormalize, int32_t* topk_idx, float* topk_w,
                   void* stream);

/*
 * Top-K routing with a choice of gate.  "MoE 推理服务工程真相 2026", section
 * 2.3, names sigmoid routing as a remedy for router-level imbalance.
 *   gate == MOE_GATE_SOFTMAX: as moe_route_topk.
 *   gate == MOE_GATE_SIGMOID: topk_w[t, k] = 1 / (1 + exp(-logit)) of the
 *   chosen expert (each expert's score independent of the others); if
 *   renormalize != 0, divided by the sum of the K chosen scores.
 * The choice of experts (topk_idx) is the same for both gates.
 * Checks: as moe_route_topk; gate a moe_gate_t value (INVALID_ARG).
 */
int moe_route_topk_gated(const float* logits, int32_t N, int32_t E, int32_t K, int32_t gate,
                         int32_t renormalize, int32_t* topk_idx, float* topk_w, void* stream);

/* Bytes of device workspace moe_reroute_overflow needs for these sizes. */
size_t moe_reroute_workspace_bytes(int32_t N, int32_t E, int32_t K);

/*
 * One round of token re-routing of capacity overflow, between routing and
 * dispatch.  "MoE 推理服务工程真相 2026", section 2.3: the dispatch
 * pseudocode counts each expert's tokens against the capacity and re-maps
 * the expert ids of the overflow; section 4.3 ("Token drop"): an
 * over-capacity token goes to a next-best expert instead of losing that
 * expert's output.  The pages leave the rule open; this call takes:
 *   1. slot (t, k) overflows iff its expert was named by `capacity` slots
 *      earlier in (token, slot) order -- the slots moe_dispatch drops;
 *   2. token t's j-th overflowing slot (j = 0, 1, .. in slot order) is
 *      offered the expert at position K + j of the token's order (larger
 *      logit first, ties to the lower index): its best experts outside its
 *      own top K; none if K + j >= E;
 *   3. candidates are admitted in (token, slot) order while their expert
 *      has room left by step 1 (capacity minus its surviving slots);
 *   4. an admitted slot gets the new expert in topk_idx and its gate score
 *      in topk_w: moe_route_topk_gated's formula for that expert (with
 *      renormalize, divided by the sum of the token's original K scores),
 *      equal to a routing call's weight to within fp32 rounding.
 * Other slots are left unchanged; moe_dispatch with the same capacity then
 * keeps the step-1 survivors plus every admitted slot and drops the rest.
 *   logits       [N, E] fp32, the routing input (finite).
 *   topk_idx     [N, K] int32 in/out, as moe_route_topk(_gated) wrote it
 *                (distinct experts, best first: unchecked precondition).
 *   topk_w       [N, K] fp32 in/out.
 *   gate, renormalize  as given to the routing call.
 *   capacity     per-expert budget; -1 (dropless) makes the call a no-op.
 *   rerouted     [E] int32 out, admitted slots per expert; may be NULL.
 *   workspace    device scratch of moe_reroute_workspace_bytes(N, E, K).
 * Results are deterministic (no atomics decide anything).
 * Checks: as moe_route_topk_gated; N >= 1, capacity >= -1 (INVALID_ARG);
 *         workspace (WORKSPACE).
 */
int moe_reroute_overflow(const float* logits, int32_t N, int32_t E, int32_t K, int32_t gate,
                         int32_t renormalize, int64_t capacity, int32_t* topk_idx,
                         float* topk_w, int32_t* rerouted, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * Router projection: logits[t, e] = sum_i x[t, i] * w_router[e, i] for all
 * N tokens and E experts, accumulated in fp32 and stored as fp32 (the input
 * of moe_route_topk).  The router turns each token's hidden state into
 * expert scores before the Top-K choice ("MoE 推理服务工程真相 2026",
 * section 一; "MoE 专家并行的 All-to-All 通信瓶颈", flowchart step
 * "路由器选 Top-K 专家").  Summation order differs from any reference, so
 * logits agree with an exact sum to within the fp32 summation bound and
 * near-ties may order differently.
 *   x          [N, d] of dtype; w_router [E, d] of dtype; logits [N, E] fp32 out.
 * Results are deterministic (every logit's terms are added in a fixed
 * order for given N, d and E).
 * Checks: pointers non-null; N, d, E >= 1; d a multiple of 8
 *         (INVALID_ARG); dtype; E <= MOE_MAX_EXPERTS; N*E < 2^31 and
 *         256 * d * element size < 2^31 (UNSUPPORTED).
 */
int moe_router_logits(const void* x, int32_t dtype, int32_t N, int32_t d,
                      const void* w_router, int32_t E, float* logits, void* stream);

/* Bytes of device workspace moe_dispatch needs for these sizes. */
size_t moe_dispatch_workspace_bytes(int32_t N, int32_t E, int32_t K);

/*
 * Dispatch: histogram, capacity drop, prefix scan and permutation of the
 * tokens into per-expert contiguous rows laid out by destination rank.
 * Follows the dispatch pseudocode of "MoE 推理服务工程真相 2026", section 2.3
 * (bincount of the expert ids, overflow against the capacity, grouping for
 * the all-to-all), the expert drop of section 4.3 (a dropped pair's output is
 * zero), and the dense token-to-expert mapping table and cumsum of "MoE
 * Inference Communication", section "MoE 计算核优化".
 *
 *   x          [N, d] activations of type dtype.
 *   topk_idx   [N, K] int32 from moe_route_topk (distinct, in [0, E);
 *              unchecked precondition).
 *   W          virtual ranks; rank r owns experts [r*E/W, (r+1)*E/W).
 *   capacity   -1 dropless, else 0 <= capacity: the r-th token (r from 0,
 *              in token order) routed to an expert is kept iff r < capacity,
 *              so an overflowing expert drops its later tokens.
 *   x_perm     [N*K, d] out: row offsets[e] + r holds a bit copy of the
 *              token that is the r-th kept token of expert e.  Rows at and
 *              beyond offsets[E] are not written.  Rank r's send slice is rows
 *              [rank_offsets[r], rank_offsets[r+1]).
 *   perm_token [N*K] int32 out: row -> source token (rows < offsets[E]).
 *   dest       [N, K] int32 out: (t, k) -> row, or -1 if dropped.
 *   demand     [E] int32 out: tokens routed to each expert (before the drop).
 *   counts     [E] int32 out: tokens kept per expert = min(demand, capacity).
 *   offsets    [E+1] int32 out: exclusive prefix sum of counts.
 *   rank_offsets [W+1] int32 out: offsets[r*E/W].
 *   workspace  device scratch of moe_dispatch_workspace_bytes(N, E, K).
 * Checks: pointers non-null; N >= 1; d >= 1 and d*sizeof(dtype) a multiple
 *         of 16; 1 <= K <= E; W >= 1 and E % W == 0; capacity >= -1;
 *         N*K < 2^31 (INVALID_ARG); E, K limits and dtype (UNSUPPORTED);
 *         workspace (WORKSPACE).
 */
int moe_dispatch(const void* x, int32_t dtype, int32_t N, int32_t d,
                 const int32_t* topk_idx, int32_t E, int32_t K, int32_t W,
                 int64_t capacity, void* x_perm, int32_t* perm_token,
                 int32_t* dest, int32_t* demand, int32_t* counts,
                 int32_t* offsets, int32_t* rank_offsets, void* workspace,
                 size_t workspace_bytes, void* stream);

/* Bytes of the plan buffer moe_route_plan and moe_dispatch_planned use. */
size_t moe_route_plan_bytes(int32_t N, int32_t E, int32_t K);

/*
 * Routing that also counts for the dispatch.  "MoE Inference
 * Communication", section "MoE 计算核优化", fuses the gate's top-k with the
 * counting and cumsum that build the token-to-expert table, to save
 * launches.  This call routes as moe_route_topk_gated and, in the same
 * launch, ranks each block's tokens per expert and counts them, into
 * `plan`; where the table of counts is of middling size, the launch's last
 * block also scans it.  moe_dispatch_planned then needs no counting pass of
 * its own (and, after such a scan, no scan either).
 *
 *   logits, N, E, K, gate, renormalize, topk_idx, topk_w: as
 *              moe_route_topk_gated (the same results, bit for bit).
 *   W, capacity, demand, counts, offsets, rank_offsets: as moe_dispatch.
 *              The four outputs are complete once moe_dispatch_planned has
 *              run on this plan; this call may fill them first.  Pass the
 *              same buffers and values to both calls.
 *   plan       device memory of moe_route_plan_bytes(N, E, K) bytes that
 *              receives each (token, slot)'s rank among the tokens of its
 *              block with the same expert, each block's per-expert counts
 *              and their scan.  Its first 256 bytes hold an arrival counter
 *              that must be zero before the plan's first use (allocate it
 *              zeroed); every call leaves it zero.  A counter that was not
 *              zero gives wrong dispatch results (moe_dispatch_planned still
 *              writes only inside its output buffers).  Calls that may
 *              overlap (different streams) need plans of their own.
 * Checks: as moe_route_topk_gated; N >= 1, W >= 1, E % W == 0, capacity >=
 *         -1 (INVALID_ARG); N*E beyond the plan's 32-bit addressing
 *         (UNSUPPORTED); plan (WORKSPACE).
 */
int moe_route_plan(const float* logits, int32_t N, int32_t E, int32_t K, int32_t gate,
                   int32_t renormalize, int32_t W, int64_t capacity, int32_t* topk_idx,
                   float* topk_w, int32_t* demand, int32_t* counts, int32_t* offsets,
                   int32_t* rank_offsets, void* plan, size_t plan_bytes, void* stream);

/*
 * moe_dispatch from a plan: the same operation ("MoE 推理服务工程真相
 * 2026", section 2.3: counts per expert, the capacity drop, grouping for the
 * all-to-all; the dense token-to-expert table built from a cumsum of "MoE
 * Inference Communication", section "MoE 计算核优化") and the same results,
 * without moe_dispatch's counting pass over topk_idx.
 *
 *   plan       filled by moe_route_plan for this N, E, K, W, capacity and
 *              topk_idx (all unchanged since); this call may also write its
 *              scan of the block counts into it.
 *   x, dtype, N, d, topk_idx, E, K, W, capacity, perm_token, dest, demand,
 *   counts, offsets, rank_offsets: as moe_dispatch.
 *   x_scale    NULL: x_perm [N*K, d] receives bit copies of x's rows, as
 *              moe_dispatch.  Otherwise x is bf16, d a multiple of 128, and
 *              x_perm (uint8 codes) and x_scale receive the e4m3 payload of
 *              moe_dispatch_fp8.
 * Checks: as moe_dispatch, with the plan in place of the workspace
 *         (WORKSPACE); x_scale with a non-bf16 dtype or d % 128 != 0
 *         (INVALID_ARG).
 */
int moe_dispatch_planned(const void* x, int32_t dtype, int32_t N, int32_t d,
                         const int32_t* topk_idx, int32_t E, int32_t K, int32_t W,
                         int64_t capacity, void* plan, size_t plan_bytes, void* x_perm,
                         float* x_scale, int32_t* perm_token, int32_t* dest, int32_t* demand,
                         int32_t* counts, int32_t* offsets, int32_t* rank_offsets,
                         void* stream);

/*
 * moe_dispatch for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops and harnesses that forbid
 * hipMalloc.  Same operation, arguments, checks and results as moe_dispatch,
 * without the workspace arguments: its scratch is a fixed array of
 * MOE_DISPATCH_NOALLOC_SCRATCH_BYTES bytes in the library's device memory,
 * one per GPU, held from the first call on that GPU until the process ends.
 * The call allocates nothing (its first call on a GPU looks the array's
 * address up once).  Every call on one GPU shares that GPU's array and
 * leaves its contents behind; nothing in it needs to start at zero.  Calls
 * that may overlap on one GPU (different streams or host threads without
 * ordering) race on the array.
 * Checks: as moe_dispatch; sizes whose moe_dispatch_workspace_bytes(N, E, K)
 *         exceed MOE_DISPATCH_NOALLOC_SCRATCH_BYTES (UNSUPPORTED); a device
 *         ordinal of 64 or more (UNSUPPORTED).
 */
#define MOE_DISPATCH_NOALLOC_SCRATCH_BYTES (4u << 20)
int moe_dispatch_noalloc(const void* x, int32_t dtype, int32_t N, int32_t d,
                         const int32_t* topk_idx, int32_t E, int32_t K, int32_t W,
                         int64_t capacity, void* x_perm, int32_t* perm_token, int32_t* dest,
                         int32_t* demand, int32_t* counts, int32_t* offsets,
                         int32_t* rank_offsets, void* stream);

/* Bytes of device workspace moe_grouped_ffn needs for these sizes. */
size_t moe_grouped_ffn_workspace_bytes(int64_t max_rows, int32_t E,
                                       int32_t dtype);

/*
 * Ragged grouped-GEMM SwiGLU expert FFN over the packed rows: per expert e,
 * on rows R = x_perm[offsets[e] : offsets[e+1]],
 *   h = silu(R w_gate[e]^T) * (R w_up[e]^T)      (stored in dtype)
 *   y = h w_down[e]^T                            (stored in dtype)
 * with fp32 accumulation.  "MoE 专家并行的 All-to-All 通信瓶颈", flowchart
 * step "Grouped GEMM 专家计算" and section "容量因子、专家复制与 dropless 的
 * 取舍": one call handles every expert's variable token count, without drop
 * or padding.  The row count M = offsets[E] stays on the device.
 *
 *   x_perm     [max_rows, d] from moe_dispatch.
 *   offsets    [E+1] int32 device, from moe_dispatch; offsets[E] <= max_rows
 *              (rows beyond max_rows are ignored).
 *   max_rows   host-side upper bound on M (N*K for a dispatch output); sizes
 *              the launch grid.
 *   w_gate, w_up [E, ffn, d]; w_down [E, d, ffn] (rows contiguous along the
 *              reduction dimension).
 *   h          [max_rows, ffn] out (rows < offsets[E] written).
 *   y_perm     [max_rows, d] out (rows < offsets[E] written).
 *   workspace  device scratch of moe_grouped_ffn_workspace_bytes(...).
 * Checks: pointers non-null; d, ffn >= 1; E >= 1; max_rows >= 0
 *         (INVALID_ARG); bf16 needs d and ffn multiples of 64, fp32 needs
 *         multiples of 8; E limit; max_rows < 2^31 and d*ffn*sizeof(dtype) < 2^31
 *         (UNSUPPORTED); workspace
 *         (WORKSPACE).  max_rows == 0 enqueues nothing.
 */
int moe_grouped_ffn(const void* x_perm, int32_t dtype, int32_t d, int32_t ffn,
                    int32_t E, const int32_t* offsets, int64_t max_rows,
                    const void* w_gate, const void* w_up, const void* w_down,
                    void* h, void* y_perm, void* workspace,
                    size_t workspace_bytes, void* stream);

/* Which packed weight matrix moe_packed_ffn_weight_bytes sizes. */
typedef enum {
  MOE_FFN_GATE_UP = 0, /* w_gate and w_up together */
  MOE_FFN_DOWN = 1     /* w_down */
} moe_ffn_part_t;

/*
 * Bytes of one packed bf16 weight matrix for E experts (0 for invalid sizes).
 * MOE_FFN_GATE_UP: E * 2 * ffn * d * 2; MOE_FFN_DOWN: E * ceil(d / 128) *
 * 128 * ffn * 2.
 */
size_t moe_packed_ffn_weight_bytes(int32_t E, int32_t d, int32_t ffn, int32_t part);

/*
 * Pack bf16 expert weights for moe_grouped_ffn_packed: a one-time
 * rearrangement (at weight-load time) into the order in which the gfx950
 * matrix cores consume them; the values are bit copies.  Per expert, each
 * matrix becomes panels of 128 rows; a panel holds, for each 16-wide
 * reduction step s, four 1 KB fragments of 32 rows, fragment i holding for
 * lane l = 0..63 the 8 values W[row(i, l % 32)][16 s + 8 (l / 32) .. + 8].
 *   gate/up panel p: fragments gate rows 64p..64p+31, gate 64p+32..64p+63,
 *     up 64p..64p+31, up 64p+32..64p+63 (P = ffn / 64 panels per expert);
 *   down panel p: rows 128p .. 128p+127 of w_down, rows past d zero
 *     (P = ceil(d / 128)).
 *   byte offset of (expert e, panel p, step s, fragment i, lane l) =
 *     (((e * P + p) * S + s) * 4 + i) * 1024 + 16 l, S = reduction / 16.
 *   w_gate, w_up [E, ffn, d] bf16; w_down [E, d, ffn] bf16 (device).
 *   packed_up   out, moe_packed_ffn_weight_bytes(E, d, ffn, MOE_FFN_GATE_UP).
 *   packed_down out, moe_packed_ffn_weight_bytes(E, d, ffn, MOE_FFN_DOWN).
 * Checks: pointers non-null; E, d, ffn >= 1 (INVALID_ARG); d and ffn
 *         multiples of 64, E limit, packed matrices of one expert below 2 GiB
 *         (UNSUPPORTED).
 */
int moe_pack_ffn_weights(const void* w_gate, const void* w_up, const void* w_down,
                         int32_t E, int32_t d, int32_t ffn, void* packed_up,
                         void* packed_down, void* stream);

/*
 * moe_grouped_ffn for bf16 layers whose weights were packed by
 * moe_pack_ffn_weights: same operation, arguments and results (h and y_perm
 * equal moe_grouped_ffn's up to the grouping of split reductions), with the
 * weights streamed from the packed layout straight into the matrix cores'
 * registers.  workspace: moe_grouped_ffn_workspace_bytes(max_rows, E,
 * MOE_DTYPE_BF16) bytes.
 * Checks: as moe_pack_ffn_weights for the sizes; pointers non-null;
 *         max_rows >= 0 (INVALID_ARG); max_rows < 2^31 (UNSUPPORTED);
 *         workspace (WORKSPACE).  max_rows == 0 enqueues nothing.
 */
int moe_grouped_ffn_packed(const void* x_perm, int32_t d, int32_t ffn, int32_t E,
                           const int32_t* offsets, int64_t max_rows, const void* packed_up,
                           const void* packed_down, void* h, void* y_perm, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * Combine: inverse permutation with the gate-weighted sum.
 * "MoE 专家并行的 All-to-All 通信瓶颈", flowchart step "加权合并回原 token
 * 顺序"; a dropped pair adds zero ("MoE 推理服务工程真相 2026", section 4.3).
 *   out[t] = sum over k = 0..K-1 with dest[t,k] >= 0 of
 *            topk_w[t,k] * y_perm[dest[t,k]]
 * accumulated in fp32 in ascending k and rounded to dtype; a token with every
 * pair dropped gets a zero row.
 *   y_perm [rows, d]; dest [N, K] int32 (each >= 0 entry a valid row:
 *   unchecked precondition); topk_w [N, K] fp32; out [N, d] of dtype.
 * Checks: pointers non-null; N >= 1; d >= 1 and d*sizeof(dtype) a multiple
 *         of 16; 1 <= K (INVALID_ARG); K limit and dtype (UNSUPPORTED).
 */
int moe_combine(const void* y_perm, int32_t dtype, int32_t N, int32_t d,
                int32_t K, const int32_t* dest, const float* topk_w, void* out,
                void* stream);

/*
 * Combine of a Residual-MoE layer.  "MoE Inference Communication", section
 * "PR-MoE：从”所有层一样多专家”到”哪里需要哪里多”", Phenomenon-II: every token
 * also passes through one fixed dense MLP, whose output is added to the
 * routed expert's (with top-1 routing this matches top-2 in quality at
 * top-1's exchange volume).  The shared MLP is an ordinary SwiGLU FFN: run
 * moe_grouped_ffn or moe_grouped_ffn_packed on x with E = 1 and offsets =
 * {0, N} to get `shared`.
 *   out[t] = shared[t] + sum over k = 0..K-1 with dest[t,k] >= 0 of
 *            topk_w[t,k] * y_perm[dest[t,k]]
 * accumulated in fp32 starting from shared[t] (unweighted), then ascending
 * k, rounded once to dtype; a token with every pair dropped gets shared[t].
 *   shared [N, d] of dtype (row-major, caller-owned device memory); the
 *   other arguments as in moe_combine.
 * Checks: as moe_combine, plus shared non-null (INVALID_ARG).
 */
int moe_combine_residual(const void* y_perm, int32_t dtype, int32_t N, int32_t d, int32_t K,
                         const int32_t* dest, const float* topk_w, const void* shared,
                         void* out, void* stream);

/*
 * FP8 exchange payload.  "MoE 推理服务工程真相 2026", section 6.3: the
 * all-to-all token data goes as FP8 instead of BF16, halving its bytes.
 * Format: rows of d columns (d a multiple of 128) are cut into groups of
 * 128; a group is stored as OCP FP8 E4M3 codes (uint8: sign, 4-bit exponent
 * with bias 7, 3-bit mantissa, largest finite 448) of x * (448 / amax),
 * amax the group's largest |x| (zero codes when amax < 2^-100), and its
 * fp32 scale amax / 448 in a [rows, d / 128] array; it is read back as
 * code value * scale.  Each step is one fp32 operation with
 * round-to-nearest-even, so codes are an exact function of the inputs.
 * Activations are bf16.
 */

/*
 * moe_dispatch with an fp8 payload: identical routing outputs (perm_token,
 * dest, demand, counts, offsets, rank_offsets), and row p of the packed
 * buffer is the fp8 form of x[perm_token[p]]:
 *   x       [N, d] bf16;  x8 [N*K, d] uint8 out;  x_scale [N*K, d/128] fp32 out.
 * Checks: as moe_dispatch, plus d a positive multiple of 128 (INVALID_ARG).
 */
int moe_dispatch_fp8(const void* x, int32_t N, int32_t d, const int32_t* topk_idx, int32_t E,
                     int32_t K, int32_t W, int64_t capacity, uint8_t* x8, float* x_scale,
                     int32_t* perm_token, int32_t* dest, int32_t* demand, int32_t* counts,
                     int32_t* offsets, int32_t* rank_offsets, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * moe_combine reading fp8 expert outputs: out[t] = sum over kept k of
 * topk_w[t,k] * (code value * scale) of row dest[t,k], in fp32, ascending k,
 * rounded to bf16.
 *   y8 [rows, d] uint8; y_scale [rows, d/128] fp32; dest, topk_w as in
 *   moe_combine; out [N, d] bf16.
 * Checks: pointers non-null; N, K >= 1; d a positive multiple of 128
 *         (INVALID_ARG); K limit (UNSUPPORTED).
 */
int moe_combine_fp8(const uint8_t* y8, const float* y_scale, int32_t N, int32_t d, int32_t K,
                    const int32_t* dest, const float* topk_w, void* out, void* stream);

/*
 * Row passes at either end of an fp8 exchange, over rows [0, min(*n_rows,
 * max_rows)) where n_rows is a DEVICE int32 (e.g. offsets + E, so the row
 * count never visits the host); other rows are not touched.
 *   quantize:   src [max_rows, d] bf16 -> q [max_rows, d] uint8, scale
 *               [max_rows, d/128] fp32.
 *   dequantize: q, scale -> dst [max_rows, d] bf16 (code value * scale,
 *               rounded to nearest even).
 * Checks: pointers non-null; 0 <= max_rows < 2^31; d a positive multiple of
 *         128 (INVALID_ARG).  max_rows == 0 enqueues nothing.
 */
int moe_fp8_quantize_rows(const void* src, const int32_t* n_rows, int64_t max_rows, int32_t d,
                          uint8_t* q, float* scale, void* stream);
int moe_fp8_dequantize_rows(const uint8_t* q, const float* scale, const int32_t* n_rows,
                            int64_t max_rows, int32_t d, void* dst, void* stream);

/* Bytes of device workspace moe_exchange_plan needs for these sizes. */
size_t moe_exchange_workspace_bytes(int32_t E, int32_t W);

/*
 * Plan of the virtual multi-source exchange: the two local permutations on
 * either side of the expert-parallel all-to-all, for W source ranks on one
 * GPU.  "MoE 专家并行的 All-to-All 通信瓶颈", section "All-to-All 分发与回收的
 * 机制": each card packs its tokens by destination card, the all-to-all
 * moves them, and each card groups what it received by expert.  Source rank
 * s owns tokens [floor(s*N/W), floor((s+1)*N/W)); rank r owns experts
 * [r*E/W, (r+1)*E/W).  Layouts of the kept pairs:
 *   send       [source][expert][token] (hence grouped by destination);
 *   receive    [destination][source][expert][token] (after the all-to-all);
 *   regrouped  [destination][expert][source][token], which is the
 *              expert-contiguous order moe_dispatch produces.
 * "MoE Inference Communication", Aurora, Theorem 4.2: the traffic matrix
 * bounds the all-to-all time from below.
 *
 *   topk_idx, dest, perm_token, offsets  moe_dispatch's inputs/outputs for
 *              the whole batch (device).
 *   max_rows   row bound of the map arrays (N*K for a dispatch output).
 *   src_counts [W, E] int32 out: kept pairs per (source, expert).
 *   traffic    [W, W] int32 out: D[s][r], kept pairs source s sends to rank r.
 *   send_row   [N, K] int32 out: send-buffer row of each kept pair, -1 if
 *              dropped.
 *   send_token [max_rows] int32 out: send row -> token (gather map that
 *              packs the send buffer from x).
 *   a2a_src    [max_rows] int32 out: receive row -> send row (the
 *              all-to-all as a gather).
 *   regroup_src [max_rows] int32 out: regrouped row -> receive row.
 *   Rows at and beyond offsets[E] of the three maps are not written.
 * Checks: pointers non-null; N >= 1; 1 <= K <= E; W >= 1, E % W == 0;
 *         N*K, max_rows < 2^31 (INVALID_ARG); E, K, W <= MOE_MAX_RANKS
 *         limits (UNSUPPORTED); workspace (WORKSPACE).
 */
int moe_exchange_plan(const int32_t* topk_idx, const int32_t* dest,
                      const int32_t* perm_token, const int32_t* offsets, int32_t N,
                      int32_t E, int32_t K, int32_t W, int64_t max_rows,
                      int32_t* src_counts, int32_t* traffic, int32_t* send_row,
                      int32_t* send_token, int32_t* a2a_src, int32_t* regroup_src,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Move whole rows by a map: dst[i] = src[map[i]] (scatter == 0, a gather)
 * or dst[map[i]] = src[i] (scatter != 0), for i < min(*n_rows, max_rows),
 * where n_rows is a DEVICE pointer (e.g. offsets + E, so the row count
 * never reaches the host).  Used with the maps of moe_exchange_plan to pack
 * send buffers, emulate the all-to-all and regroup, and (as scatters) to run
 * the same permutations backwards for the combine direction.
 *   src, dst   row-major buffers of row_bytes per row; must not overlap.
 *   map        int32 row indices, each a valid row of the other buffer
 *              (unchecked precondition).
 * Checks: pointers non-null; max_rows >= 0 and < 2^31; row_bytes a positive
 *         multiple of 16; src != dst (INVALID_ARG).
 */
int moe_rows_permute(const void* src, void* dst, const int32_t* map, const int32_t* n_rows,
                     int64_t max_rows, int32_t row_bytes, int32_t scatter, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_ROUTE_H */
