// Combine: inverse permutation with the gate-weighted sum.
//
// "MoE 专家并行的 All-to-All 通信瓶颈", flowchart step "加权合并回原 token
// 顺序": expert outputs return to token order and are merged with the gate
// weights.  A dropped pair (dest = -1) adds nothing ("MoE 推理服务工程真相
// 2026", section 4.3: the dropped expert's output is zero).
//
// One wave per token.  Lanes 0..K-1 fetch the token's K destination rows and
// weights; the wave then walks the output row in 16-byte chunks, gathers the
// same chunk of each kept row (each a contiguous HBM row, so the reads
// coalesce), accumulates w * y in fp32 in ascending k, rounds once, and
// writes the token's row.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kCombineWaves = 4;
constexpr int kUnroll = 2;

template <bool kBf16>
__global__ __launch_bounds__(kCombineWaves * kWave) void combine_kernel(
    const uint4* __restrict__ y_perm, int row_chunks, int N, int K,
    const int32_t* __restrict__ dest, const float* __restrict__ topk_w,
    uint4* __restrict__ out) {
  constexpr int kElems = kBf16 ? 8 : 4;  // elements per 16-byte chunk
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * kCombineWaves + threadIdx.x / kWave;
  if (t >= N) return;

  int row = -1;
  float w = 0.0f;
  if (lane < K) {
    row = dest[(size_t)t * K + lane];
    w = topk_w[(size_t)t * K + lane];
  }
  uint4* dst = out + (size_t)t * row_chunks;
  for (int c0 = 0; c0 < row_chunks; c0 += kWave * kUnroll) {
    float acc[kUnroll][kElems];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
      for (int i = 0; i < kElems; ++i) acc[u][i] = 0.0f;
    for (int k = 0; k < K; ++k) {
      const int rk = __shfl(row, k);
      const float wk = __shfl(w, k);
      if (rk < 0) continue;  // uniform across the wave
      const uint4* src = y_perm + (size_t)rk * row_chunks;
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int c = c0 + u * kWave + lane;
        if (c >= row_chunks) continue;
        const uint4 raw = src[c];
        if constexpr (kBf16) {
          const bf16x8 v = __builtin_bit_cast(bf16x8, raw);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[u][i] = fmaf(wk, (float)v[i], acc[u][i]);
        } else {
          const f32x4 v = __builtin_bit_cast(f32x4, raw);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[u][i] = fmaf(wk, v[i], acc[u][i]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int c = c0 + u * kWave + lane;
      if (c >= row_chunks) continue;
      if constexpr (kBf16) {
        bf16x8 o;
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = (bf16)acc[u][i];
        dst[c] = __builtin_bit_cast(uint4, o);
      } else {
        f32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = acc[u][i];
        dst[c] = __builtin_bit_cast(uint4, o);
      }
    }
  }
}

}  // namespace

hipError_t launch_combine(const void* y_perm, bool bf16_data, int N, int d,
                          int K, const int32_t* dest, const float* topk_w,
                          void* out, hipStream_t stream) {
  const int row_chunks = bf16_data ? d / 8 : d / 4;
  const int blocks = (N + kCombineWaves - 1) / kCombineWaves;
  if (bf16_data)
    combine_kernel<true><<<blocks, kCombineWaves * kWave, 0, stream>>>(
        static_cast<const uint4*>(y_perm), row_chunks, N, K, dest, topk_w,
        static_cast<uint4*>(out));
  else
    combine_kernel<false><<<blocks, kCombineWaves * kWave, 0, stream>>>(
        static_cast<const uint4*>(y_perm), row_chunks, N, K, dest, topk_w,
        static_cast<uint4*>(out));
  return hipGetLastError();
}

}  // namespace moe
