// Top-K routing: per token, softmax over the E router logits (or the sigmoid
// of each logit) and the K best experts, best first, ties to the lower
// expert index.
//
// "MoE 专家并行的 All-to-All 通信瓶颈", section "一个反直觉的扩容结果": the
// router chooses Top-K experts per token.  "MoE 推理服务工程真相 2026",
// section 2.3, names sigmoid routing as a remedy for router-level
// imbalance: with kSigmoid the weight is 1 / (1 + exp(-logit)) and the
// softmax reductions are skipped; the choice is the same.
//
// "MoE Inference Communication", section "MoE 计算核优化", fuses the gate's
// top-k with the cumsum and scatter that follow it, to save launches.
// route_plan_kernel takes the dispatch's counting into the gate: a block of
// 1024 threads routes 1024 / L consecutive tokens and ranks them per expert
// in token order (a bit per token in an LDS mask per expert; a pair's rank
// is the popcount of the bits below its token), and writes the block's
// per-expert totals.  Where the table of totals is of middling size
// (plan_scan_mode), the block also counts itself in on an arrival counter
// and the last block to arrive scans the table (rank_scan.h), so the
// dispatch is one scatter launch; a small table is scanned by every scatter
// block, a large one by the dispatch's scan kernel (one block scanning a
// large table in the routing launch's tail would hold up the routing call).
//
// Mapping: a group of L lanes (L = 8 or 16) owns one token and holds VPL =
// ceil(E / L) logits per lane, expert e = lane_in_group + i * L, so a
// group's loads are contiguous and a wave routes 64 / L tokens at once.  The
// group maximum and the sum of exponentials are reductions whose steps pair
// lanes inside 16-lane rows by DPP lane moves (quad swaps, half-row and row
// mirrors); each step combines two values commutatively, so every lane of
// the group ends with the same bits.  A round of the top-K takes the group
// maximum of the remaining logits; each lane then names the lowest of its
// experts holding that maximum, and a group minimum over those names gives
// the lowest expert index with the maximum logit.  That is the order (a > b)
// or (a == b and lower index), a total order on (logit, index) pairs.  Lane
// k of the group keeps round k's winner and logit; after the K rounds lanes
// 0 .. K - 1 compute their gate weights together and store the token's K
// results (K <= 16 <= L whenever E > 8).
#include "moe_internal.h"
#include "rank_scan.h"

#include <math.h>

#include <type_traits>

namespace moe {
namespace {

// One DPP lane move of a float (row and bank masks full).
template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float a) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, a), kCtrl, 0xf, 0xf, false));
}
constexpr int kDppXor1 = 0xb1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4e;        // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141; // lane i <- 7 - i within each 8 lanes
constexpr int kDppMirror = 0x140;     // lane i <- 15 - i within each 16 lanes

// Maximum (kMax) or sum of a over each aligned group of L = 8 or 16 lanes,
// the same bits in every lane of the group.  After the two quad steps every
// lane holds its quad's value; the half mirror pairs each lane with one of
// the other quad of its 8, the mirror with one of the other 8 of its 16.
template <int L, bool kMax>
__device__ __forceinline__ float group_reduce(float a) {
  static_assert(L == 8 || L == 16, "groups of 8 or 16 lanes");
  auto op = [](float x, float y) __attribute__((always_inline)) {
    return kMax ? fmaxf(x, y) : x + y;
  };
  a = op(a, dpp_f32<kDppXor1>(a));
  a = op(a, dpp_f32<kDppXor2>(a));
  a = op(a, dpp_f32<kDppHalfMirror>(a));
  if (L == 16) a = op(a, dpp_f32<kDppMirror>(a));
  return a;
}

// Minimum of an int over each aligned group of L = 8 or 16 lanes.
template <int L>
__device__ __forceinline__ int group_min(int a) {
  a = min(a, __builtin_amdgcn_mov_dpp(a, kDppXor1, 0xf, 0xf, false));
  a = min(a, __builtin_amdgcn_mov_dpp(a, kDppXor2, 0xf, 0xf, false));
  a = min(a, __builtin_amdgcn_mov_dpp(a, kDppHalfMirror, 0xf, 0xf, false));
  if (L == 16) a = min(a, __builtin_amdgcn_mov_dpp(a, kDppMirror, 0xf, 0xf, false));
  return a;
}

constexpr int kRouteBufferFlags = 0x00020000;  // raw 32-bit buffer accesses

// Routes the wave's 64 / L tokens tok0, tok0 + 1, ... (tok0 wave-uniform),
// one per group of L lanes; lane j < K of a group returns slot j's expert
// and gate weight (other lanes: unspecified).  Tokens at or past N read
// zeros and their results are meaningless.
template <int L, int VPL, bool kSigmoid>
__device__ __forceinline__ void route_wave(const float* __restrict__ logits, int N, int E,
                                           int K, int renormalize, int tok0, int* out_idx,
                                           float* out_w) {
  constexpr int kGroupsPerWave = kWave / L;
  const int lane = threadIdx.x & (kWave - 1);
  const int j = lane % L;

  // the wave's rows through one buffer descriptor (wave-uniform, so it sits
  // in scalar registers): the range ends at the wave's last token below N,
  // so a token past N reads zeros without a branch; an expert past E reads
  // whatever follows and becomes -inf
  float v[VPL];
  const int wave_bytes =
      __builtin_amdgcn_readfirstlane(max(0, min(kGroupsPerWave, N - tok0)) * E * 4);
  const __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(logits + (size_t)tok0 * E), 0, (uint32_t)wave_bytes, kRouteBufferFlags);
  const int row_off = (lane / L) * E * 4;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = j + i * L;
    const float raw = __builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(rr, row_off + e * 4, 0, 0));
    v[i] = e < E ? raw : -INFINITY;
  }

  float m = 0.0f, s = 1.0f;
  if (!kSigmoid) {
    m = v[0];
#pragma unroll
    for (int i = 1; i < VPL; ++i) m = fmaxf(m, v[i]);
    m = group_reduce<L, true>(m);
    s = 0.0f;
#pragma unroll
    // v_exp_f32 on (v - m) log2(e): within about 2^-22 of expf relative
    // to the largest term, far inside the weights' tolerance
    for (int i = 0; i < VPL; ++i) s += __expf(v[i] - m);  // padding: exp(-inf) = 0
    s = group_reduce<L, false>(s);
  }

  int my_idx = 0;
  float my_logit = -INFINITY;
  for (int k = 0; k < K; ++k) {
    float lb = v[0];
#pragma unroll
    for (int i = 1; i < VPL; ++i) lb = fmaxf(lb, v[i]);
    const float bv = group_reduce<L, true>(lb);
    // this lane's lowest expert holding bv (E if none), then the group's
    int le = E;
#pragma unroll
    for (int i = VPL - 1; i >= 0; --i)
      if (v[i] == bv) le = j + i * L;
    const int bi = group_min<L>(le);
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (j + i * L == bi) v[i] = -INFINITY;  // taken: never wins again
    if (j == k) {
      my_idx = bi;
      my_logit = bv;
    }
  }
  // the K gate weights at once, lane k holding slot k's (renormalised: over
  // the sum of the K weights, a group sum)
  float w = 0.0f;
  if (kSigmoid && renormalize) {
    // ratios to slot 0's score (sigmoid_ratio), whose sum is at least 1
    const float l0 = group_reduce<L, true>(my_logit);  // lanes >= K hold -inf
    if (j < K) w = sigmoid_ratio(my_logit, l0);
    w = w / group_reduce<L, false>(w);
  } else {
    if (j < K) w = kSigmoid ? 1.0f / (1.0f + expf(-my_logit)) : __expf(my_logit - m) / s;
    if (renormalize) w = w / group_reduce<L, false>(w);
  }
  *out_idx = my_idx;
  *out_w = w;
}

template <int L, int VPL, bool kSigmoid>
__global__ __launch_bounds__(256) void route_topk_kernel(
    const float* __restrict__ logits, int N, int E, int K, int renormalize,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
  constexpr int kGroupsPerWave = kWave / L;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int j = lane % L;
  const int tok0 = __builtin_amdgcn_readfirstlane(
      (blockIdx.x * (blockDim.x / kWave) + wave) * kGroupsPerWave);
  const int tok = tok0 + lane / L;
  int idx;
  float w;
  route_wave<L, VPL, kSigmoid>(logits, N, E, K, renormalize, tok0, &idx, &w);
  if (tok < N && j < K) {
    topk_idx[(size_t)tok * K + j] = idx;
    topk_w[(size_t)tok * K + j] = w;
  }
}

// Routing fused with the dispatch's ranking (see the top of the file).
// Block b routes tokens [b T, (b + 1) T), T = route_plan_tokens(E) =
// kRoutePlanThreads / L.  Outputs: topk_idx / topk_w as route_topk_kernel;
// plan.local_rank[t][k] = the number of tokens t' < t of the same block that
// chose the same expert; plan.block_counts[b][e] = the block's tokens that
// chose e.  Waves whose tokens all lie past N skip the routing arithmetic
// (a wave-uniform branch), so that a block holding few tokens costs the
// SIMDs no more than those tokens' waves.
//
// kScan: the last block to finish also scans the block counts
// (scan_rank_table: block_excl, demand, counts, offsets, rank_offsets).
// Ordering without a device-wide fence (the protocol of the grouped FFN's
// split partials): each block's totals are stored with the system-scope
// policy (written through L1 and L2 to memory, and counted in vmcnt until
// they are there), every thread waits for its stores (vmcnt(0)) before the
// block barrier, and only then does thread 0 take its turn on the arrival
// counter, a device-scope atomic.  The block whose atomicInc returns B - 1
// arrived after every other block's stores were in memory, and it reads the
// table with system-scope loads, which read memory.  atomicInc wraps the
// counter back to 0 at that last arrival, ready for the next call.
template <int L, int VPL, bool kSigmoid, bool kScan>
__global__ __launch_bounds__(kRoutePlanThreads) void route_plan_kernel(
    const float* __restrict__ logits, int N, int E, int K, int renormalize,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, int W, int64_t capacity,
    int32_t* __restrict__ demand, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ rank_offsets, RoutePlan plan) {
  constexpr int kGroupsPerWave = kWave / L;
  constexpr int kTB = kRoutePlanThreads / L;   // tokens per block
  constexpr int kWords = (kTB + 63) / 64;      // 64-bit mask words per expert
  extern __shared__ unsigned long long masks[];  // [E][kWords]
  __shared__ RankScanShared sh;
  __shared__ int last;
  const int tid = threadIdx.x;
  for (int i = tid; i < E * kWords; i += kRoutePlanThreads) masks[i] = 0ull;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int j = lane % L;
  const int tok0 = __builtin_amdgcn_readfirstlane(
      (blockIdx.x * (kRoutePlanThreads / kWave) + wave) * kGroupsPerWave);
  const int tok = tok0 + lane / L;
  int idx = -1;
  float w = 0.0f;
  if (tok0 < N) route_wave<L, VPL, kSigmoid>(logits, N, E, K, renormalize, tok0, &idx, &w);
  const bool mine = tok < N && j < K;
  const bool named = mine && (unsigned)idx < (unsigned)E;
  if (mine) {
    topk_idx[(size_t)tok * K + j] = idx;
    topk_w[(size_t)tok * K + j] = w;
  }
  const int tl = tok - blockIdx.x * kTB;  // token within the block
  __syncthreads();                        // masks cleared
  if (named) atomicOr(&masks[idx * kWords + tl / 64], 1ull << (tl % 64));
  __syncthreads();
  if (mine) {
    int r = 0;
    if (named) {
      const unsigned long long* m = masks + idx * kWords;
      r = __popcll(m[tl / 64] & ((1ull << (tl % 64)) - 1ull));
      for (int wd = 0; wd < tl / 64; ++wd) r += __popcll(m[wd]);
    }
    plan.local_rank[(size_t)tok * K + j] = r;
  }
  const __amdgpu_buffer_rsrc_t cr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(plan.block_counts + (size_t)blockIdx.x * E), 0, (uint32_t)(E * sizeof(int32_t)),
      kRankScanBufferFlags);
  for (int e = tid; e < E; e += kRoutePlanThreads) {
    int c = 0;
#pragma unroll
    for (int wd = 0; wd < kWords; ++wd) c += __popcll(masks[e * kWords + wd]);
    __builtin_amdgcn_raw_buffer_store_b32((unsigned)c, cr, e * (int)sizeof(int32_t), 0,
                                          kScan ? kRankScanCoherent : 0);
  }
  if constexpr (kScan) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) last = atomicInc(plan.arrive, gridDim.x - 1) == gridDim.x - 1;
    __syncthreads();
    if (!last) return;
    scan_rank_table<true>(plan.block_counts, gridDim.x, E, W, capacity, plan.block_excl, demand,
                          counts, offsets, rank_offsets, sh);
  }
}

template <int L, int VPL>
hipError_t launch(const float* logits, int N, int E, int K, bool sigmoid, int renormalize,
                  int32_t* topk_idx, float* topk_w, hipStream_t stream) {
  constexpr int kThreads = 256;
  constexpr int kTokensPerBlock = kThreads / L;
  const int blocks = (N + kTokensPerBlock - 1) / kTokensPerBlock;
  if (sigmoid)
    route_topk_kernel<L, VPL, true><<<blocks, kThreads, 0, stream>>>(
        logits, N, E, K, renormalize, topk_idx, topk_w);
  else
    route_topk_kernel<L, VPL, false><<<blocks, kThreads, 0, stream>>>(
        logits, N, E, K, renormalize, topk_idx, topk_w);
  return hipGetLastError();
}

// Calls f(L, VPL) (integral constants) for E: groups of 8 lanes up to 8
// experts, else 16 lanes with ceil(E / 16) logits per lane, rounded up to a
// power of two.
template <typename F>
hipError_t with_route_shape(int E, F&& f) {
  using std::integral_constant;
  if (E <= 8) return f(integral_constant<int, 8>{}, integral_constant<int, 1>{});
  if (E <= 16) return f(integral_constant<int, 16>{}, integral_constant<int, 1>{});
  if (E <= 32) return f(integral_constant<int, 16>{}, integral_constant<int, 2>{});
  if (E <= 64) return f(integral_constant<int, 16>{}, integral_constant<int, 4>{});
  if (E <= 128) return f(integral_constant<int, 16>{}, integral_constant<int, 8>{});
  if (E <= 256) return f(integral_constant<int, 16>{}, integral_constant<int, 16>{});
  if (E <= 512) return f(integral_constant<int, 16>{}, integral_constant<int, 32>{});
  return f(integral_constant<int, 16>{}, integral_constant<int, 64>{});
}

}  // namespace

hipError_t launch_route_topk(const float* logits, int N, int E, int K, bool sigmoid,
                             int renormalize, int32_t* topk_idx, float* topk_w,
                             hipStream_t stream) {
  if (N == 0) return hipSuccess;
  return with_route_shape(E, [&](auto l_c, auto vpl_c) {
    return launch<decltype(l_c)::value, decltype(vpl_c)::value>(
        logits, N, E, K, sigmoid, renormalize, topk_idx, topk_w, stream);
  });
}

int route_plan_tokens(int E) { return kRoutePlanThreads / (E <= 8 ? 8 : 16); }

PlanScan plan_scan_mode(int N, int E) {
  const int64_t B = ((int64_t)N + route_plan_tokens(E) - 1) / route_plan_tokens(E);
  if (B * E <= kPlanFusedMaxCounts && E <= kPlanFusedMaxExperts) return PlanScan::kInScatter;
  if (B * E <= kPlanRouteScanMaxCounts) return PlanScan::kInRoute;
  return PlanScan::kKernel;
}

size_t route_plan_bytes(int N, int E, int K) {
  const size_t B = (size_t)(N + route_plan_tokens(E) - 1) / route_plan_tokens(E);
  return 256 + 2 * align_up(B * E * sizeof(int32_t), 256) +
         align_up((size_t)N * K * sizeof(int32_t), 256);
}

RoutePlan route_plan(void* base, int N, int E, int K) {
  const size_t B = (size_t)(N + route_plan_tokens(E) - 1) / route_plan_tokens(E);
  char* p = static_cast<char*>(base);
  RoutePlan plan;
  plan.arrive = reinterpret_cast<unsigned*>(p);
  p += 256;
  plan.block_counts = reinterpret_cast<int32_t*>(p);
  p += align_up(B * E * sizeof(int32_t), 256);
  plan.block_excl = reinterpret_cast<int32_t*>(p);
  p += align_up(B * E * sizeof(int32_t), 256);
  plan.local_rank = reinterpret_cast<int32_t*>(p);
  return plan;
}

hipError_t launch_route_plan(const float* logits, int N, int E, int K, bool sigmoid,
                             int renormalize, int W, int64_t capacity, int32_t* topk_idx,
                             float* topk_w, int32_t* demand, int32_t* counts, int32_t* offsets,
                             int32_t* rank_offsets, const RoutePlan& plan, hipStream_t stream) {
  if (N == 0) return hipSuccess;
  const bool scan = plan_scan_mode(N, E) == PlanScan::kInRoute;
  return with_route_shape(E, [&](auto l_c, auto vpl_c) {
    constexpr int L = decltype(l_c)::value;
    constexpr int VPL = decltype(vpl_c)::value;
    constexpr int kTB = kRoutePlanThreads / L;
    constexpr int kWords = (kTB + 63) / 64;
    const int blocks = (N + kTB - 1) / kTB;
    const size_t lds = (size_t)E * kWords * sizeof(unsigned long long);
    auto go = [&](auto sig_c, auto scan_c) {
      route_plan_kernel<L, VPL, decltype(sig_c)::value, decltype(scan_c)::value>
          <<<blocks, kRoutePlanThreads, lds, stream>>>(logits, N, E, K, renormalize, topk_idx,
                                                       topk_w, W, capacity, demand, counts,
                                                       offsets, rank_offsets, plan);
    };
    using T = std::true_type;
    using F = std::false_type;
    if (sigmoid) {
      if (scan) go(T{}, T{});
      else go(T{}, F{});
    } else {
      if (scan) go(F{}, T{});
      else go(F{}, F{});
    }
    return hipGetLastError();
  });
}

}  // namespace moe
