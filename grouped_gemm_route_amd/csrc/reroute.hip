// One round of token re-routing of capacity overflow.
//
// "MoE 推理服务工程真相 2026", section 2.3: the dispatch pseudocode counts
// each expert's tokens, compares them with the capacity and re-maps the
// expert ids of the overflow before the all-to-all; section 4.3 ("Token
// drop"): an over-capacity token is sent to a next-best expert instead of
// losing that expert's output.  The rule, where the pages leave it open:
//   1. slot (t, k) overflows iff its expert was already named by `capacity`
//      slots earlier in (token, slot) order (the slots moe_dispatch drops);
//   2. token t's j-th overflowing slot is offered the expert at position
//      K + j of the token's order (descending logit, ties to the lower
//      index), i.e. its best experts outside its own top K;
//   3. candidates are admitted in (token, slot) order while the expert has
//      room left by step 1 (capacity minus its surviving slots);
//   4. an admitted slot takes the new expert and its gate score (divided by
//      the sum of the token's original K scores if renormalised).
// moe_dispatch with the same capacity then keeps the step-1 survivors plus
// every admitted slot: an expert with room had no overflow, and one that
// overflowed has no room.
//
// Kernels, all integer decisions exact:
//   rank + scan (the dispatch's stable-rank kernels) on topk_idx: each
//     slot's position among its expert's slots, and per-expert survivors;
//   candidates (one wave per token): the token's overflowing slots from
//     those positions; then, slot by slot, the best expert strictly behind
//     the previous pick in the (logit desc, index asc) order, starting from
//     the token's K-th expert, so no exclusion list is needed;
//   rank + scan on the candidate table (-1 = none): each candidate's
//     position among its expert's candidates;
//   finalize (one thread per slot): admits a candidate iff its position is
//     below the expert's room, and writes each expert's admitted count
//     min(candidates, room) -- no atomics, so results are reproducible.
#include "moe_internal.h"

#include <limits.h>
#include <math.h>

namespace moe {
namespace {

constexpr int kTokWaves = 4;  // tokens (waves) per block of the candidate kernel

struct RerouteWorkspace {
  int32_t* block_counts;  // [B, E]
  int32_t* block_excl;    // [B, E]
  int32_t* local_rank;    // [N, K]
  int32_t* cand;          // [N, K] candidate expert or -1
  float* cand_w;          // [N, K] its weight
  int32_t* kept1;         // [E] survivors of the capacity check
  int32_t* demand1;       // [E]
  int32_t* cand_demand;   // [E] candidates per expert
  int32_t* scratch;       // [E] + [E + 1] + [2]: unused scan outputs
};

inline size_t rr_bytes(size_t n) { return align_up(n, 256); }

RerouteWorkspace reroute_workspace(void* base, int N, int E, int K) {
  const size_t B = (size_t)(N + kRankBlockTokens - 1) / kRankBlockTokens;
  const size_t NK = (size_t)N * K;
  char* p = static_cast<char*>(base);
  RerouteWorkspace ws;
  ws.block_counts = reinterpret_cast<int32_t*>(p); p += rr_bytes(B * E * 4);
  ws.block_excl = reinterpret_cast<int32_t*>(p); p += rr_bytes(B * E * 4);
  ws.local_rank = reinterpret_cast<int32_t*>(p); p += rr_bytes(NK * 4);
  ws.cand = reinterpret_cast<int32_t*>(p); p += rr_bytes(NK * 4);
  ws.cand_w = reinterpret_cast<float*>(p); p += rr_bytes(NK * 4);
  ws.kept1 = reinterpret_cast<int32_t*>(p); p += rr_bytes((size_t)E * 4);
  ws.demand1 = reinterpret_cast<int32_t*>(p); p += rr_bytes((size_t)E * 4);
  ws.cand_demand = reinterpret_cast<int32_t*>(p); p += rr_bytes((size_t)E * 4);
  ws.scratch = reinterpret_cast<int32_t*>(p);
  return ws;
}

// (a, ia) comes before (b, ib) in the token's order
__device__ __forceinline__ bool before(float a, int ia, float b, int ib) {
  return a > b || (a == b && ia < ib);
}

template <int VPL, bool kSigmoid>
__global__ __launch_bounds__(kTokWaves * kWave) void reroute_candidates_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ topk_idx, int N, int E,
    int K, int renormalize, int64_t capacity, const int32_t* __restrict__ block_excl,
    const int32_t* __restrict__ local_rank, int32_t* __restrict__ cand,
    float* __restrict__ cand_w) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * kTokWaves + (int)(threadIdx.x / kWave);
  if (t >= N) return;  // wave-uniform
  const float* row = logits + (size_t)t * E;
  const size_t slot0 = (size_t)t * K;

  // this token's overflowing slots (lanes k < K)
  int my_e = 0;
  bool over = false;
  float my_l = 0.0f;
  if (lane < K) {
    my_e = topk_idx[slot0 + lane];
    my_l = row[my_e];
    const int b = t / kRankBlockTokens;
    const int r = block_excl[(size_t)b * E + my_e] + local_rank[slot0 + lane];
    over = capacity >= 0 && (int64_t)r >= capacity;
  }
  const unsigned long long mask = __ballot(over);
  if (lane < K) cand[slot0 + lane] = -1;
  if (mask == 0ull) return;

  float v[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + i * kWave;
    v[i] = e < E ? row[e] : -INFINITY;
  }
  float m = 0.0f, s = 1.0f;
  if (!kSigmoid) {  // softmax maximum and denominator over all E logits
    m = v[0];
#pragma unroll
    for (int i = 1; i < VPL; ++i) m = fmaxf(m, v[i]);
#pragma unroll
    for (int off = kWave / 2; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    s = 0.0f;
#pragma unroll
    for (int i = 0; i < VPL; ++i) s += expf(v[i] - m);
#pragma unroll
    for (int off = kWave / 2; off >= 1; off >>= 1) s += __shfl_xor(s, off);
  }
  // Renormalised sigmoid scores are taken as ratios to the score of slot 0's
  // logit (sigmoid_ratio: finite and not all zero however negative the
  // logits), which the division by their sum cancels.  Weights follow the
  // routing kernel's formulas; its sums run in another order, so they agree
  // with its weights to within fp32 rounding.
  const float l0 = __shfl(my_l, 0);
  auto score = [&](float l) {
    if (kSigmoid && renormalize) return sigmoid_ratio(l, l0);
    return kSigmoid ? 1.0f / (1.0f + expf(-l)) : expf(l - m) / s;
  };
  float norm = 1.0f;
  if (renormalize) {  // sum of the original K scores, slot order
    const float mine = lane < K ? score(my_l) : 0.0f;
    float acc = 0.0f;
    for (int k = 0; k < K; ++k) acc += __shfl(mine, k);
    norm = acc;
  }

  // start behind the token's K-th expert
  float thr_l = __shfl(my_l, K - 1);
  int thr_e = __shfl(my_e, K - 1);
  for (int k = 0; k < K; ++k) {
    if (!((mask >> k) & 1ull)) continue;  // uniform
    float bv = -INFINITY;
    int bi = INT_MAX;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = lane + i * kWave;
      if (e < E && before(thr_l, thr_e, v[i], e) && before(v[i], e, bv, bi)) {
        bv = v[i];
        bi = e;
      }
    }
#pragma unroll
    for (int off = kWave / 2; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (before(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (bi == INT_MAX) break;  // no expert left behind the last pick
    if (lane == 0) {
      cand[slot0 + k] = bi;
      cand_w[slot0 + k] = score(bv) / norm;
    }
    thr_l = bv;
    thr_e = bi;
  }
}

__global__ __launch_bounds__(256) void reroute_finalize_kernel(
    const int32_t* __restrict__ cand, const float* __restrict__ cand_w, int N, int E, int K,
    int64_t capacity, const int32_t* __restrict__ block_excl,
    const int32_t* __restrict__ local_rank, const int32_t* __restrict__ kept1,
    const int32_t* __restrict__ cand_demand, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, int32_t* __restrict__ rerouted) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (rerouted != nullptr && i < E) {
    const int64_t room = capacity < 0 ? 0 : capacity - kept1[i];
    rerouted[i] = (int32_t)min((int64_t)cand_demand[i], room);
  }
  if (i >= (int64_t)N * K) return;
  const int c = cand[i];
  if (c < 0) return;
  const int t = (int)(i / K);
  const int r = block_excl[(size_t)(t / kRankBlockTokens) * E + c] + local_rank[i];
  if ((int64_t)r < capacity - kept1[c]) {
    topk_idx[i] = c;
    topk_w[i] = cand_w[i];
  }
}

template <int VPL>
hipError_t launch_candidates(const float* logits, const int32_t* topk_idx, int N, int E,
                             int K, bool sigmoid, int renormalize, int64_t capacity,
                             const RerouteWorkspace& ws, hipStream_t stream) {
  const int blocks = (N + kTokWaves - 1) / kTokWaves;
  if (sigmoid)
    reroute_candidates_kernel<VPL, true><<<blocks, kTokWaves * kWave, 0, stream>>>(
        logits, topk_idx, N, E, K, renormalize, capacity, ws.block_excl, ws.local_rank,
        ws.cand, ws.cand_w);
  else
    reroute_candidates_kernel<VPL, false><<<blocks, kTokWaves * kWave, 0, stream>>>(
        logits, topk_idx, N, E, K, renormalize, capacity, ws.block_excl, ws.local_rank,
        ws.cand, ws.cand_w);
  return hipGetLastError();
}

}  // namespace

size_t reroute_workspace_bytes(int N, int E, int K) {
  const size_t B = (size_t)(N + kRankBlockTokens - 1) / kRankBlockTokens;
  const size_t NK = (size_t)N * K;
  return 2 * rr_bytes(B * E * 4) + 3 * rr_bytes(NK * 4) + 3 * rr_bytes((size_t)E * 4) +
         rr_bytes((size_t)(2 * E + 3) * 4);
}

hipError_t launch_reroute(const float* logits, int N, int E, int K, bool sigmoid,
                          int renormalize, int64_t capacity, int32_t* topk_idx,
                          float* topk_w, int32_t* rerouted, void* workspace,
                          hipStream_t stream) {
  const RerouteWorkspace ws = reroute_workspace(workspace, N, E, K);
  int32_t* s_counts = ws.scratch;           // [E]
  int32_t* s_offsets = ws.scratch + E;      // [E + 1]
  int32_t* s_rank_off = ws.scratch + 2 * E + 1;  // [2]
  // 1. positions of the routed slots; survivors per expert
  hipError_t err = launch_rank_scan(topk_idx, N, E, K, capacity, ws.block_counts,
                                    ws.block_excl, ws.local_rank, ws.demand1, ws.kept1,
                                    s_offsets, s_rank_off, stream);
  if (err != hipSuccess) return err;
  // 2. candidates
  if (E <= 64) err = launch_candidates<1>(logits, topk_idx, N, E, K, sigmoid, renormalize, capacity, ws, stream);
  else if (E <= 128) err = launch_candidates<2>(logits, topk_idx, N, E, K, sigmoid, renormalize, capacity, ws, stream);
  else if (E <= 256) err = launch_candidates<4>(logits, topk_idx, N, E, K, sigmoid, renormalize, capacity, ws, stream);
  else if (E <= 512) err = launch_candidates<8>(logits, topk_idx, N, E, K, sigmoid, renormalize, capacity, ws, stream);
  else err = launch_candidates<16>(logits, topk_idx, N, E, K, sigmoid, renormalize, capacity, ws, stream);
  if (err != hipSuccess) return err;
  // 3. positions of the candidates (the first pass's positions are spent)
  err = launch_rank_scan(ws.cand, N, E, K, -1, ws.block_counts, ws.block_excl,
                         ws.local_rank, ws.cand_demand, s_counts, s_offsets, s_rank_off,
                         stream);
  if (err != hipSuccess) return err;
  // 4. admission
  const int64_t work = (int64_t)N * K > E ? (int64_t)N * K : E;
  const int blocks = (int)((work + 255) / 256);
  reroute_finalize_kernel<<<blocks, 256, 0, stream>>>(
      ws.cand, ws.cand_w, N, E, K, capacity, ws.block_excl, ws.local_rank, ws.kept1,
      ws.cand_demand, topk_idx, topk_w, rerouted);
  return hipGetLastError();
}

}  // namespace moe
