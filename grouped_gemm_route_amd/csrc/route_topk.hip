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
// Mapping: a group of L lanes (L = 8..64, a power of two) owns one token and
// holds VPL = ceil(E / L) logits per lane, expert e = lane_in_group + i * L,
// so a group's loads are contiguous.  The max, the sum of exponentials and K
// argmax rounds are butterfly reductions inside the group (xor shuffles never
// leave an aligned group).  The comparator is (a > b) or (a == b and lower
// index), a total order on (logit, index) pairs, so every lane of the group
// ends each round with the same winner.
#include "moe_internal.h"

#include <math.h>

namespace moe {
namespace {

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

  float v[VPL];
  const float* row = logits + (size_t)(valid ? tok : 0) * E;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = j + i * L;
    v[i] = e < E ? (valid ? row[e] : 0.0f) : -INFINITY;
  }

  float m = 0.0f, s = 1.0f;
  if (!kSigmoid) {
    m = v[0];
#pragma unroll
    for (int i = 1; i < VPL; ++i) m = fmaxf(m, v[i]);
#pragma unroll
    for (int off = L / 2; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    s = 0.0f;
#pragma unroll
    for (int i = 0; i < VPL; ++i) s += expf(v[i] - m);  // padding: exp(-inf) = 0
#pragma unroll
    for (int off = L / 2; off >= 1; off >>= 1) s += __shfl_xor(s, off);
  }

  float wsum = 0.0f;
  int32_t* idx_out = topk_idx + (size_t)tok * K;
  float* w_out = topk_w + (size_t)tok * K;
  for (int k = 0; k < K; ++k) {
    float bv = v[0];
    int bi = j;
#pragma unroll
    for (int i = 1; i < VPL; ++i) {
      if (v[i] > bv) {  // later i has a higher index: strict > keeps ties low
        bv = v[i];
        bi = j + i * L;
      }
    }
#pragma unroll
    for (int off = L / 2; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    const float p = kSigmoid ? 1.0f / (1.0f + expf(-bv)) : expf(bv - m) / s;
    wsum += p;
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (j + i * L == bi) v[i] = -INFINITY;  // taken: never wins again
    if (valid && j == 0) {
      idx_out[k] = bi;
      w_out[k] = p;
    }
  }
  if (renormalize && valid && j == 0) {
    for (int k = 0; k < K; ++k) w_out[k] = w_out[k] / wsum;
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
  if (E <= 32) return launch<32, 1>(logits, N, E, K, g, renormalize, topk_idx, topk_w, stream);
  if (E <= 64) return launch<64, 1>(logits, N, E, K, g, renormalize, topk_idx, topk_w, stream);
  if (E <= 128) return launch<64, 2>(logits, N, E, K, g, renormalize, topk_idx, topk_w, stream);
  if (E <= 256) return launch<64, 4>(logits, N, E, K, g, renormalize, topk_idx, topk_w, stream);
  if (E <= 512) return launch<64, 8>(logits, N, E, K, g, renormalize, topk_idx, topk_w, stream);
  return launch<64, 16>(logits, N, E, K, g, renormalize, topk_idx, topk_w, stream);
}

}  // namespace moe
