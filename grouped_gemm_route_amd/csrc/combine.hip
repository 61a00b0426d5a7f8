// Combine: inverse permutation with the gate-weighted sum.
//
// "MoE 专家并行的 All-to-All 通信瓶颈", flowchart step "加权合并回原 token
// 顺序": expert outputs return to token order and are merged with the gate
// weights.  A dropped pair (dest = -1) adds nothing ("MoE 推理服务工程真相
// 2026", section 4.3: the dropped expert's output is zero).
//
// One wave per (token, slice of the output row); a slice is 64 lanes x U
// 16-byte pieces.  Lanes 0..K-1 fetch the token's destination rows and
// weights.  The wave first issues the loads of its slice of every kept row
// (all K x U pieces in flight at once: K x U <= 16), then accumulates
// w * y in fp32 in ascending k, rounds once to the storage type and writes
// the slice.  Each kept row is a contiguous HBM row, so the loads coalesce;
// splitting rows into slices gives small batches (decode) enough waves.
//
// Residual-MoE ("MoE Inference Communication", section "PR-MoE：从”所有层一样
// 多专家”到”哪里需要哪里多”", Phenomenon-II: a dense MLP that every token
// passes through, its output added to the routed expert's): with kShared the
// token's row of the shared MLP's output is loaded with the kept rows and
// the fp32 sum starts from it, unweighted; the kept pairs follow in
// ascending k, and the sum is rounded once.
#include "moe_internal.h"

namespace moe {
namespace {

template <bool kBf16, int KMAX, int U, bool kShared>
__global__ __launch_bounds__(256) void combine_kernel(
    const uint4* __restrict__ y_perm, int row_chunks, int n_slices, int N, int K,
    const int32_t* __restrict__ dest, const float* __restrict__ topk_w,
    const uint4* __restrict__ shared, uint4* __restrict__ out) {
  constexpr int kElems = kBf16 ? 8 : 4;  // elements per 16-byte piece
  const int lane = threadIdx.x & (kWave - 1);
  const int item = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (item >= N * n_slices) return;  // whole wave leaves together
  const int t = item / n_slices;
  const int slice = item - t * n_slices;

  int row = -1;
  float w = 0.0f;
  if (lane < K) {
    row = dest[(size_t)t * K + lane];
    w = topk_w[(size_t)t * K + lane];
  }
  const int c0 = slice * kWave * U + lane;

  uint4 sv[U];
  if constexpr (kShared) {
    const uint4* src = shared + (size_t)t * row_chunks;
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (c0 + u * kWave < row_chunks) sv[u] = src[c0 + u * kWave];
  }
  uint4 v[KMAX][U];
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    const int rk = __shfl(row, k);  // -1 past K as well (lanes >= K hold -1)
    if (rk < 0) continue;           // uniform across the wave
    const uint4* src = y_perm + (size_t)rk * row_chunks;
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (c0 + u * kWave < row_chunks) v[k][u] = src[c0 + u * kWave];
  }

  float acc[U][kElems];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if constexpr (kShared && kBf16) {
      const bf16x8 x = __builtin_bit_cast(bf16x8, sv[u]);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[u][i] = (float)x[i];
    } else if constexpr (kShared) {
      const f32x4 x = __builtin_bit_cast(f32x4, sv[u]);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[u][i] = x[i];
    } else {
#pragma unroll
      for (int i = 0; i < kElems; ++i) acc[u][i] = 0.0f;
    }
  }
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    const int rk = __shfl(row, k);
    const float wk = __shfl(w, k);
    if (rk < 0) continue;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if constexpr (kBf16) {
        const bf16x8 x = __builtin_bit_cast(bf16x8, v[k][u]);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[u][i] = fmaf(wk, (float)x[i], acc[u][i]);
      } else {
        const f32x4 x = __builtin_bit_cast(f32x4, v[k][u]);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[u][i] = fmaf(wk, x[i], acc[u][i]);
      }
    }
  }

  uint4* dst = out + (size_t)t * row_chunks;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int c = c0 + u * kWave;
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

template <bool kBf16, int KMAX, int U>
hipError_t launch(const void* y_perm, int row_chunks, int N, int K, const int32_t* dest,
                  const float* topk_w, const void* shared, void* out, hipStream_t stream) {
  const int n_slices = (row_chunks + kWave * U - 1) / (kWave * U);
  const long long items = (long long)N * n_slices;
  const int blocks = (int)((items + 3) / 4);
  if (shared)
    combine_kernel<kBf16, KMAX, U, true><<<blocks, 256, 0, stream>>>(
        static_cast<const uint4*>(y_perm), row_chunks, n_slices, N, K, dest, topk_w,
        static_cast<const uint4*>(shared), static_cast<uint4*>(out));
  else
    combine_kernel<kBf16, KMAX, U, false><<<blocks, 256, 0, stream>>>(
        static_cast<const uint4*>(y_perm), row_chunks, n_slices, N, K, dest, topk_w, nullptr,
        static_cast<uint4*>(out));
  return hipGetLastError();
}

// KMAX >= K rows per token, U pieces per lane with KMAX * U = 16 loads in
// flight per lane (fewer pieces when a row is short).
template <bool kBf16, int KMAX>
hipError_t launch_k(const void* y_perm, int row_chunks, int N, int K, const int32_t* dest,
                    const float* topk_w, const void* shared, void* out, hipStream_t stream) {
  constexpr int kU = 16 / KMAX;
  const int per_lane = (row_chunks + kWave - 1) / kWave;
  if (kU >= 8 && per_lane >= 8)
    return launch<kBf16, KMAX, (kU >= 8 ? 8 : 1)>(y_perm, row_chunks, N, K, dest, topk_w,
                                                  shared, out, stream);
  if (kU >= 4 && per_lane >= 4)
    return launch<kBf16, KMAX, (kU >= 4 ? 4 : 1)>(y_perm, row_chunks, N, K, dest, topk_w,
                                                  shared, out, stream);
  if (kU >= 2 && per_lane >= 2)
    return launch<kBf16, KMAX, (kU >= 2 ? 2 : 1)>(y_perm, row_chunks, N, K, dest, topk_w,
                                                  shared, out, stream);
  return launch<kBf16, KMAX, 1>(y_perm, row_chunks, N, K, dest, topk_w, shared, out, stream);
}

template <bool kBf16>
hipError_t launch_dtype(const void* y_perm, int row_chunks, int N, int K, const int32_t* dest,
                        const float* topk_w, const void* shared, void* out,
                        hipStream_t stream) {
  if (K <= 2)
    return launch_k<kBf16, 2>(y_perm, row_chunks, N, K, dest, topk_w, shared, out, stream);
  if (K <= 4)
    return launch_k<kBf16, 4>(y_perm, row_chunks, N, K, dest, topk_w, shared, out, stream);
  if (K <= 8)
    return launch_k<kBf16, 8>(y_perm, row_chunks, N, K, dest, topk_w, shared, out, stream);
  return launch_k<kBf16, 16>(y_perm, row_chunks, N, K, dest, topk_w, shared, out, stream);
}

}  // namespace

hipError_t launch_combine(const void* y_perm, bool bf16_data, int N, int d,
                          int K, const int32_t* dest, const float* topk_w,
                          const void* shared, void* out, hipStream_t stream) {
  const int row_chunks = bf16_data ? d / 8 : d / 4;
  if (bf16_data)
    return launch_dtype<true>(y_perm, row_chunks, N, K, dest, topk_w, shared, out, stream);
  return launch_dtype<false>(y_perm, row_chunks, N, K, dest, topk_w, shared, out, stream);
}

}  // namespace moe
