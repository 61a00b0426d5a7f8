// FP8 exchange payload: combine from fp8 expert outputs, and the row
// quantize / dequantize passes at either end of an exchange.
//
// "MoE 推理服务工程真相 2026", section 6.3: the all-to-all token data goes as
// FP8 (here OCP e4m3 with one fp32 scale per 128 columns, fp8_codec.h)
// instead of BF16.  The dispatch side packs fp8 directly (moe_dispatch_fp8);
// the receiver turns its rows back into bf16 for the grouped GEMM
// (dequantize); the expert outputs go back as fp8 (quantize) and the
// combine reads them as fp8, so both exchanges carry one byte per value
// plus 4 bytes per 128 values.
#include "fp8_codec.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kPiece = 16;                    // fp8 values per 16-byte piece
constexpr int kPiecesPerGroup = kFp8Group / kPiece;

__device__ __forceinline__ void decode16(const uint4 raw, float scale, float* f) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x2 a = e4m3_decode2<false>(w[i]);
    const f32x2 b = e4m3_decode2<true>(w[i]);
    f[4 * i + 0] = a.x * scale;
    f[4 * i + 1] = a.y * scale;
    f[4 * i + 2] = b.x * scale;
    f[4 * i + 3] = b.y * scale;
  }
}

__device__ __forceinline__ void store_bf16x16(uint4* dst, const float* f) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (bf16)f[i];
    b[i] = (bf16)f[8 + i];
  }
  dst[0] = __builtin_bit_cast(uint4, a);
  dst[1] = __builtin_bit_cast(uint4, b);
}

// One wave per (token, slice of the row); a slice is 64 lanes x U pieces of
// 16 codes.  As in the bf16 combine, the loads of every kept row (and of
// their scales) are issued first, then w * value is summed in fp32 in
// ascending k and rounded once to bf16.
template <int KMAX, int U>
__global__ __launch_bounds__(256) void combine_fp8_kernel(
    const uint4* __restrict__ y8, const float* __restrict__ y_scale, int row_pieces,
    int groups, int n_slices, int N, int K, const int32_t* __restrict__ dest,
    const float* __restrict__ topk_w, uint4* __restrict__ out) {
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

  uint4 v[KMAX][U];
  float sc[KMAX][U];
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    const int rk = __shfl(row, k);
    if (rk < 0) continue;  // uniform across the wave
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * kWave;
      if (c < row_pieces) {
        v[k][u] = y8[(size_t)rk * row_pieces + c];
        sc[k][u] = y_scale[(size_t)rk * groups + c / kPiecesPerGroup];
      }
    }
  }
  float acc[U][kPiece];
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int i = 0; i < kPiece; ++i) acc[u][i] = 0.0f;
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    const int rk = __shfl(row, k);
    const float wk = __shfl(w, k);
    if (rk < 0) continue;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (c0 + u * kWave >= row_pieces) continue;
      float f[kPiece];
      decode16(v[k][u], sc[k][u], f);
#pragma unroll
      for (int i = 0; i < kPiece; ++i) acc[u][i] = fmaf(wk, f[i], acc[u][i]);
    }
  }
  uint4* dst = out + (size_t)t * row_pieces * 2;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int c = c0 + u * kWave;
    if (c < row_pieces) store_bf16x16(dst + 2 * c, acc[u]);
  }
}

template <int KMAX, int U>
hipError_t launch_combine(const uint8_t* y8, const float* y_scale, int row_pieces, int N,
                          int K, const int32_t* dest, const float* topk_w, void* out,
                          hipStream_t stream) {
  const int n_slices = (row_pieces + kWave * U - 1) / (kWave * U);
  const long long items = (long long)N * n_slices;
  const int blocks = (int)((items + 3) / 4);
  combine_fp8_kernel<KMAX, U><<<blocks, 256, 0, stream>>>(
      reinterpret_cast<const uint4*>(y8), y_scale, row_pieces, row_pieces / kPiecesPerGroup,
      n_slices, N, K, dest, topk_w, static_cast<uint4*>(out));
  return hipGetLastError();
}

// KMAX >= K rows per token; U pieces per lane with KMAX * U <= 8 loads in
// flight per lane (each piece is 16 values, twice a bf16 piece).
template <int KMAX>
hipError_t launch_combine_k(const uint8_t* y8, const float* y_scale, int row_pieces, int N,
                            int K, const int32_t* dest, const float* topk_w, void* out,
                            hipStream_t stream) {
  constexpr int kU = 8 / KMAX > 0 ? 8 / KMAX : 1;
  const int per_lane = (row_pieces + kWave - 1) / kWave;
  if (kU >= 4 && per_lane >= 4)
    return launch_combine<KMAX, (kU >= 4 ? 4 : 1)>(y8, y_scale, row_pieces, N, K, dest, topk_w,
                                                   out, stream);
  if (kU >= 2 && per_lane >= 2)
    return launch_combine<KMAX, (kU >= 2 ? 2 : 1)>(y8, y_scale, row_pieces, N, K, dest, topk_w,
                                                   out, stream);
  return launch_combine<KMAX, 1>(y8, y_scale, row_pieces, N, K, dest, topk_w, out, stream);
}

// One block per row; thread c takes 16-byte pieces c, c + 256, ...: 8 bf16
// values in, 8 codes out (16 lanes per 128-column group agree on the scale).
__global__ __launch_bounds__(256) void fp8_quantize_rows_kernel(
    const uint4* __restrict__ src, const int32_t* __restrict__ n_rows, int max_rows,
    int row_chunks, uint2* __restrict__ q, float* __restrict__ scale) {
  const int row = blockIdx.x;
  if (row >= min(*n_rows, max_rows)) return;
  const int groups = row_chunks / (kFp8Group / 8);
  for (int c = threadIdx.x; c < row_chunks; c += blockDim.x) {
    float s;
    const uint2 codes = quantize_piece(src[(size_t)row * row_chunks + c], &s);
    q[(size_t)row * row_chunks + c] = codes;
    if (c % (kFp8Group / 8) == 0) scale[(size_t)row * groups + c / (kFp8Group / 8)] = s;
  }
}

// One block per row; thread c takes fp8 pieces c, c + 256, ...: 16 codes in,
// 16 bf16 values (value * scale, rounded to nearest even) out.
__global__ __launch_bounds__(256) void fp8_dequantize_rows_kernel(
    const uint4* __restrict__ q, const float* __restrict__ scale,
    const int32_t* __restrict__ n_rows, int max_rows, int row_pieces,
    uint4* __restrict__ dst) {
  const int row = blockIdx.x;
  if (row >= min(*n_rows, max_rows)) return;
  const int groups = row_pieces / kPiecesPerGroup;
  for (int c = threadIdx.x; c < row_pieces; c += blockDim.x) {
    float f[kPiece];
    decode16(q[(size_t)row * row_pieces + c], scale[(size_t)row * groups + c / kPiecesPerGroup],
             f);
    store_bf16x16(dst + ((size_t)row * row_pieces + c) * 2, f);
  }
}

}  // namespace

hipError_t launch_combine_fp8(const uint8_t* y8, const float* y_scale, int N, int d, int K,
                              const int32_t* dest, const float* topk_w, void* out,
                              hipStream_t stream) {
  const int row_pieces = d / kPiece;
  if (K <= 2) return launch_combine_k<2>(y8, y_scale, row_pieces, N, K, dest, topk_w, out, stream);
  if (K <= 4) return launch_combine_k<4>(y8, y_scale, row_pieces, N, K, dest, topk_w, out, stream);
  if (K <= 8) return launch_combine_k<8>(y8, y_scale, row_pieces, N, K, dest, topk_w, out, stream);
  return launch_combine_k<16>(y8, y_scale, row_pieces, N, K, dest, topk_w, out, stream);
}

hipError_t launch_fp8_quantize_rows(const void* src, const int32_t* n_rows, int max_rows,
                                    int d, uint8_t* q, float* scale, hipStream_t stream) {
  if (max_rows == 0) return hipSuccess;
  fp8_quantize_rows_kernel<<<max_rows, 256, 0, stream>>>(
      static_cast<const uint4*>(src), n_rows, max_rows, d / 8, reinterpret_cast<uint2*>(q),
      scale);
  return hipGetLastError();
}

hipError_t launch_fp8_dequantize_rows(const uint8_t* q, const float* scale,
                                      const int32_t* n_rows, int max_rows, int d, void* dst,
                                      hipStream_t stream) {
  if (max_rows == 0) return hipSuccess;
  fp8_dequantize_rows_kernel<<<max_rows, 256, 0, stream>>>(
      reinterpret_cast<const uint4*>(q), scale, n_rows, max_rows, d / kPiece,
      static_cast<uint4*>(dst));
  return hipGetLastError();
}

}  // namespace moe
