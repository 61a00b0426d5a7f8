// Top-K routing: per token, softmax over the E router logits (or the sigmoid
// of each logit) and the K best experts, best first, ties to the lower
// expert index.
//
// "MoE 专家并行的 All-to-All 通信瓶颈", section "一个反直觉的扩容结果": the
// router chooses Top-K experts per token.  "MoE Inference Communication",
// section "MoE 计算核优化", fuses the gate's top-k with the following
// cumsum/scatter to save launches; here the gate is one launch and the
// histogram, scan and scatter are the dispatch call's.  "MoE 推理服务工程真相
// 2026", section 2.3, names sigmoid routing as a remedy for router-level
// imbalance: with kSigmoid the weight is 1 / (1 + exp(-logit)) and the
// softmax reductions are skipped; the choice is the same.
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

#include <math.h>

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

template <int L, int VPL, bool kSigmoid>
__global__ __launch_bounds__(256) void route_topk_kernel(
    const float* __restrict__ logits, int N, int E, int K, int renormalize,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
  constexpr int kGroupsPerWave = kWave / L;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int j = lane % L;
  const int tok = (blockIdx.x * (blockDim.x / kWave) + wave) * kGroupsPerWave +
                  lane / L;
  const bool valid = tok < N;

  // the wave's rows through one buffer descriptor (wave-uniform, so it sits
  // in scalar registers): the range ends at the wave's last token below N,
  // so a token past N reads zeros without a branch; an expert past E reads
  // whatever follows and becomes -inf
  float v[VPL];
  const int tok0 = __builtin_amdgcn_readfirstlane(
      (blockIdx.x * (blockDim.x / kWave) + wave) * kGroupsPerWave);
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
  if (valid && j < K) {
    topk_idx[(size_t)tok * K + j] = my_idx;
    topk_w[(size_t)tok * K + j] = w;
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

}  // namespace

hipError_t launch_route_topk(const float* logits, int N, int E, int K, bool sigmoid,
                             int renormalize, int32_t* topk_idx, float* topk_w,
                             hipStream_t stream) {
  if (N == 0) return hipSuccess;
  const bool g = sigmoid;
  if (E <= 8) return launch<8, 1>(logits, N, E, K, g, renormalize, topk_idx, topk_w, stream);
  if (E <= 16) return launch<16, 1>(logits, N, E, K, g, renormalize, topk_idx, topk_w, stream);
  if (E <= 32) return launch<16, 2>(logits, N, E, K, g, renormalize, topk_idx, topk_w, stream);
  if (E <= 64) return launch<16, 4>(logits, N, E, K, g, renormalize, topk_idx, topk_w, stream);
  if (E <= 128) return launch<16, 8>(logits, N, E, K, g, renormalize, topk_idx, topk_w, stream);
  if (E <= 256) return launch<16, 16>(logits, N, E, K, g, renormalize, topk_idx, topk_w, stream);
  if (E <= 512) return launch<16, 32>(logits, N, E, K, g, renormalize, topk_idx, topk_w, stream);
  return launch<16, 64>(logits, N, E, K, g, renormalize, topk_idx, topk_w, stream);
}

}  // namespace moe
