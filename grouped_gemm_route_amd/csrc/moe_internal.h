// Internal declarations shared by the HIP translation units of libmoe_route.
// Not part of the public ABI (include/moe_route.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4;

constexpr int kWave = 64;

// Dispatch: tokens handled by one block of the rank kernel (one per thread).
constexpr int kRankBlockTokens = 256;

// Grouped FFN tile heights (rows of the packed buffer per tile).
constexpr int kBf16TileRows = 128;
constexpr int kF32TileRows = 32;

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Sigmoid gate score of logit l as a ratio to the score of a logit l0 >= l,
// s(l) / s(l0) with s(z) = 1 / (1 + exp(-z)), in a form where no exponential
// overflows and the ratio does not vanish with the scores themselves (all
// chosen logits far below zero round every plain fp32 score to 0):
//   l0 < 0:  exp(l - l0) (1 + exp(l0)) / (1 + exp(l))
//   l0 >= 0: (1 + exp(-l0)) / (1 + exp(-l))
// The ratio for l = l0 is exactly 1, so a sum of ratios that includes l0's is
// at least 1.  Used for renormalised sigmoid weights, which are these ratios
// divided by their sum over the K chosen experts.
__device__ __forceinline__ float sigmoid_ratio(float l, float l0) {
  return l0 < 0.0f ? expf(l - l0) * (1.0f + expf(l0)) / (1.0f + expf(l))
                   : (1.0f + expf(-l0)) / (1.0f + expf(-l));
}

// ---- launchers (each returns the hipError_t of its launches) -------------

hipError_t launch_route_topk(const float* logits, int N, int E, int K, bool sigmoid,
                             int renormalize, int32_t* topk_idx, float* topk_w,
                             hipStream_t stream);

// Routing fused with the dispatch's ranking (route_topk.hip): blocks of
// kRoutePlanThreads threads route route_plan_tokens(E) tokens each and write
// their ranks and per-block counts into the plan buffer: [arrival counter |
// pad to 256 B][block_counts [B, E] | pad][block_excl [B, E] | pad]
// [local_rank [N, K]], B = ceil(N / tokens).
constexpr int kRoutePlanThreads = 1024;
struct RoutePlan {
  unsigned* arrive;       // 0 between calls (each call that uses it leaves it 0)
  int32_t* block_counts;  // [B, E]
  int32_t* block_excl;    // [B, E]
  int32_t* local_rank;    // [N, K]
};
// Where the block counts of a plan are scanned: by every scatter block
// (tables of up to kPlanFusedMaxCounts counts and kPlanFusedMaxExperts
// experts), by the routing launch's last block (up to
// kPlanRouteScanMaxCounts), else by the dispatch's scan kernel.
enum class PlanScan { kInScatter, kInRoute, kKernel };
constexpr int64_t kPlanFusedMaxCounts = 1024;
constexpr int kPlanFusedMaxExperts = 256;
constexpr int64_t kPlanRouteScanMaxCounts = 32768;
PlanScan plan_scan_mode(int N, int E);
int route_plan_tokens(int E);
size_t route_plan_bytes(int N, int E, int K);
RoutePlan route_plan(void* base, int N, int E, int K);
hipError_t launch_route_plan(const float* logits, int N, int E, int K, bool sigmoid,
                             int renormalize, int W, int64_t capacity, int32_t* topk_idx,
                             float* topk_w, int32_t* demand, int32_t* counts, int32_t* offsets,
                             int32_t* rank_offsets, const RoutePlan& plan, hipStream_t stream);

// Workspace carve-up of moe_dispatch.
struct DispatchWorkspace {
  int32_t* block_counts;  // [B, E]
  int32_t* block_excl;    // [B, E]
  int32_t* local_rank;    // [N, K]
};
size_t dispatch_workspace_bytes(int N, int E, int K);
DispatchWorkspace dispatch_workspace(void* base, int N, int E, int K);

// x_scale == nullptr: x_perm rows are bit copies of x's rows; otherwise x is
// bf16 and x_perm / x_scale receive the fp8 payload (fp8_codec.h).
hipError_t launch_dispatch(const void* x, size_t row_bytes, int N,
                           const int32_t* topk_idx, int E, int K, int W,
                           int64_t capacity, void* x_perm, float* x_scale,
                           int32_t* perm_token, int32_t* dest,
                           int32_t* demand, int32_t* counts,
                           int32_t* offsets, int32_t* rank_offsets,
                           const DispatchWorkspace& ws, hipStream_t stream);

// The dispatch from a plan that launch_route_plan filled for the same
// topk_idx, W and capacity: the scan of the plan's block counts unless the
// routing launch did it (plan_scan_mode), and the scatter; no counting pass.
hipError_t launch_dispatch_planned(const void* x, size_t row_bytes, int N,
                                   const int32_t* topk_idx, int E, int K, int W,
                                   int64_t capacity, const RoutePlan& plan, void* x_perm,
                                   float* x_scale, int32_t* perm_token, int32_t* dest,
                                   int32_t* demand, int32_t* counts, int32_t* offsets,
                                   int32_t* rank_offsets, hipStream_t stream);

// Stable per-(token, slot) ranks of a [N, K] expert-id table (entries
// outside [0, E) are skipped) and their per-expert scan with one rank:
// block_counts / block_excl [B, E], local_rank [N, K], demand / counts [E],
// offsets [E + 1], rank_offsets [2], as in moe_dispatch.
hipError_t launch_rank_scan(const int32_t* idx, int N, int E, int K, int64_t capacity,
                            int32_t* block_counts, int32_t* block_excl,
                            int32_t* local_rank, int32_t* demand, int32_t* counts,
                            int32_t* offsets, int32_t* rank_offsets, hipStream_t stream);

size_t reroute_workspace_bytes(int N, int E, int K);

hipError_t launch_reroute(const float* logits, int N, int E, int K, bool sigmoid,
                          int renormalize, int64_t capacity, int32_t* topk_idx,
                          float* topk_w, int32_t* rerouted, void* workspace,
                          hipStream_t stream);

// Grouped FFN on packed bf16 weights (grouped_ffn_packed.hip).  Panels of
// the packed gate/up (gate_up) or down matrix, its bytes for E experts, the
// row-tile height the launch picks and the split partials it needs.
int packed_panels(int d, int ffn, bool gate_up);
size_t packed_ffn_weight_bytes(int E, int d, int ffn, bool gate_up);
int packed_ffn_tile_rows(int64_t max_rows, int E);
size_t packed_ffn_partial_bytes(int64_t max_rows, int E);
hipError_t launch_pack_ffn_weights(const void* w_gate, const void* w_up, const void* w_down,
                                   int E, int d, int ffn, void* packed_up, void* packed_down,
                                   hipStream_t stream);
hipError_t launch_grouped_ffn_packed(const void* x_perm, int d, int ffn, int E,
                                     const int32_t* offsets, int64_t max_rows,
                                     const void* packed_up, const void* packed_down, void* h,
                                     void* y_perm, void* workspace, hipStream_t stream);

// shared: the Residual-MoE shared MLP's output [N, d] added to each token's
// sum, or null for the plain combine.
hipError_t launch_combine(const void* y_perm, bool bf16_data, int N, int d,
                          int K, const int32_t* dest, const float* topk_w,
                          const void* shared, void* out, hipStream_t stream);

// fp8 payload (fp8_codec.h).  Row kernels act on rows [0, min(*n_rows,
// max_rows)) of d columns; d is a multiple of 128.
hipError_t launch_combine_fp8(const uint8_t* y8, const float* y_scale, int N, int d, int K,
                              const int32_t* dest, const float* topk_w, void* out,
                              hipStream_t stream);
hipError_t launch_fp8_quantize_rows(const void* src, const int32_t* n_rows, int max_rows,
                                    int d, uint8_t* q, float* scale, hipStream_t stream);
hipError_t launch_fp8_dequantize_rows(const uint8_t* q, const float* scale,
                                      const int32_t* n_rows, int max_rows, int d, void* dst,
                                      hipStream_t stream);

size_t grouped_ffn_workspace_bytes(int64_t max_rows, int E, bool bf16_data);

hipError_t launch_grouped_ffn(const void* x_perm, bool bf16_data, int d,
                              int ffn, int E, const int32_t* offsets,
                              int64_t max_rows, const void* w_gate,
                              const void* w_up, const void* w_down, void* h,
                              void* y_perm, void* workspace,
                              hipStream_t stream);

hipError_t launch_router_logits(const void* x, bool bf16_data, int N, int d,
                                const void* w_router, int E, float* logits,
                                hipStream_t stream);

size_t exchange_workspace_bytes(int E, int W);

hipError_t launch_exchange_plan(const int32_t* topk_idx, const int32_t* dest,
                                const int32_t* perm_token, const int32_t* offsets, int N,
                                int E, int K, int W, int max_rows, int32_t* src_counts,
                                int32_t* traffic, int32_t* send_row, int32_t* send_token,
                                int32_t* a2a_src, int32_t* regroup_src, void* workspace,
                                hipStream_t stream);

hipError_t launch_rows_permute(const void* src, void* dst, const int32_t* map,
                               const int32_t* n_rows, int max_rows, int row_bytes, bool scatter,
                               hipStream_t stream);

}  // namespace moe
