// Router projection: logits[t, e] = sum_i x[t, i] * w_router[e, i], fp32.
//
// The router turns each token's hidden state into its expert scores before
// the Top-K choice ("MoE 推理服务工程真相 2026", section 一; "MoE 专家并行的
// All-to-All 通信瓶颈", flowchart step "路由器选 Top-K 专家").
//
// bf16, more than 64 experts and d a multiple of 64: an MFMA GEMM
// (v_mfma_f32_32x32x16_bf16, fp32 accumulate).
// Block tile 64 tokens x 256 experts x 64 reduction elements; wave w owns
// experts [64 w, 64 w + 64) of the tile for all 64 tokens (2 x 2 MFMA tiles),
// so a token row is read from HBM once per 256 experts.  Both operands are
// loaded straight into LDS (two stages, 40 KB each) with the chunk swizzle
// of the grouped GEMM (bank-conflict-free 128-byte rows); loads past the
// last token or expert return zeros.  Each lane's accumulator holds 4
// consecutive experts of one token, stored as 16 bytes.
// fp32 (small layers): one thread per logit, a plain dot product.
#include "moe_internal.h"

#include <mutex>

namespace moe {
namespace {

constexpr int kRThreads = 256;
constexpr int kRT = 64;        // tokens per block
constexpr int kRE = 256;       // experts per block
constexpr int kRK = 64;        // reduction elements per stage
constexpr int kRRow = kRK * 2; // 128-byte LDS rows
constexpr int kRStage = (kRT + kRE) * kRRow;
constexpr int kRBufferFlags = 0x00020000;

typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ int rswz(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

__global__ __launch_bounds__(kRThreads, 1) void router_logits_bf16_kernel(
    const bf16* __restrict__ x, int N, int d, const bf16* __restrict__ w, int E,
    float* __restrict__ logits) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int t0 = blockIdx.x * kRT;
  const int e0 = blockIdx.y * kRE;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int nt = min(kRT, N - t0);
  const int ne = min(kRE, E - e0);
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(x + (size_t)t0 * d), 0, (uint32_t)((size_t)nt * d * 2), kRBufferFlags);
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(w + (size_t)e0 * d), 0, (uint32_t)((size_t)ne * d * 2), kRBufferFlags);
  // wave-wide direct-to-LDS loads: 8 rows of 128 bytes each; x rows 0..63
  // (2 loads per wave), expert rows 0..255 (8 loads per wave)
  const int grow = lane >> 3;
  int x_src[2], w_src[8];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int lr = (i * 4 + wave) * 8 + grow;
    x_src[i] = (lr * d + rswz(lr, lane & 7) * 8) * 2;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int lr = (i * 4 + wave) * 8 + grow;
    w_src[i] = (lr * d + rswz(lr, lane & 7) * 8) * 2;
  }
  auto issue = [&](int stage, int k0) __attribute__((always_inline)) {
    char* base = lds + stage * kRStage;
    const int soff = k0 * 2;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int v = x_src[i];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          xr, (lds_void_t*)(base + (i * 4 + wave) * 8 * kRRow), 16, v, soff, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int v = w_src[i];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          wr, (lds_void_t*)(base + kRT * kRRow + (i * 4 + wave) * 8 * kRRow), 16, v, soff, 0,
          0);
    }
  };

  const int lrow = lane & 31;
  const int lhalf = lane >> 5;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nk = d / kRK;
  issue(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int stage = kt & 1;
    if (kt + 1 < nk) issue(stage ^ 1, (kt + 1) * kRK);
    const char* sb = lds + stage * kRStage;
#pragma unroll
    for (int ks = 0; ks < kRK / 16; ++ks) {
      const int chunk = ks * 2 + lhalf;
      bf16x8 wf[2], xf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = wave * 64 + i * 32 + lrow;
        wf[i] = *reinterpret_cast<const bf16x8*>(sb + kRT * kRRow + row * kRRow +
                                                 rswz(row, chunk) * 16);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int row = j * 32 + lrow;
        xf[j] = *reinterpret_cast<const bf16x8*>(sb + row * kRRow + rswz(row, chunk) * 16);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[i], xf[j], acc[i][j], 0, 0, 0);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }

  // accumulator register r of lane l: expert (r / 4) * 8 + (l / 32) * 4 + r % 4
  // of its 32-expert tile, token l % 32 of its 32-token tile
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int t = t0 + j * 32 + lrow;
    if (t >= N) continue;
    float* orow = logits + (size_t)t * E;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int e = e0 + wave * 64 + i * 32 + r4 * 8 + lhalf * 4;
        if (e + 3 < E && (E & 3) == 0) {
          f32x4 o;
#pragma unroll
          for (int q = 0; q < 4; ++q) o[q] = acc[i][j][r4 * 4 + q];
          *reinterpret_cast<f32x4*>(orow + e) = o;
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (e + q < E) orow[e + q] = acc[i][j][r4 * 4 + q];
        }
      }
    }
  }
}

// Skinny form, for up to 64 experts per block (all E <= 64, and any E when
// d is not a multiple of 64): the projection is bound by reading x once, so
// a block takes only 16 tokens (enough blocks to cover the CUs) and its 8
// waves split the reduction into 8 contiguous ranges of 32-element steps.
// v_mfma_f32_16x16x32_bf16 with the 16 tokens as A and up to 4 tiles of 16
// experts as B: lane l loads 8 consecutive elements (16 bytes) of token row
// l % 16, or of expert row l % 16, at the same step offset 8 (l / 16), and
// accumulator register i of lane l holds token 4 (l / 16) + i, expert
// l % 16 of the tile.  Rows past N or E read zero through the buffer
// descriptors; elements past d (d a multiple of 8, so a 16-byte piece is
// wholly inside or outside the row) are zeroed in the token operand.  The
// loads of up to 16 steps are issued before their MFMAs.  The 8 partial tiles meet in
// LDS and are added in wave order, so the result is deterministic.
constexpr int kSkWaves = 8;
constexpr int kSkTokens = 16;
constexpr int kSkMaxTiles = 4;  // 16-expert tiles per block (64 experts)

// steps whose loads are issued together: 16 (a wave's whole range for d up
// to 4096) while the loads fit in registers, else 8
template <int NET>
constexpr int skinny_steps_in_flight() { return NET <= 2 ? 16 : 8; }

template <int NET>
__global__ __launch_bounds__(kSkWaves * kWave) void router_logits_skinny_kernel(
    const bf16* __restrict__ x, int N, int d, const bf16* __restrict__ w, int E,
    float* __restrict__ logits) {
  constexpr int kRU = skinny_steps_in_flight<NET>();
  __shared__ f32x4 red[kSkWaves][NET][kWave];
  const int t0 = blockIdx.x * kSkTokens;
  const int e0 = blockIdx.y * (kSkMaxTiles * 16);
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int r = lane & 15;
  const int g = lane >> 4;
  const int nt = min(kSkTokens, N - t0);
  const int ne = min(NET * 16, E - e0);
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(x + (size_t)t0 * d), 0, (uint32_t)((size_t)nt * d * 2), kRBufferFlags);
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(w + (size_t)e0 * d), 0, (uint32_t)((size_t)ne * d * 2), kRBufferFlags);
  const int nk = (d + 31) / 32;
  const int s0 = wave * nk / kSkWaves;
  const int s1 = (wave + 1) * nk / kSkWaves;
  const int xoff = r * d * 2;
  int woff[NET];
#pragma unroll
  for (int j = 0; j < NET; ++j) woff[j] = (j * 16 + r) * d * 2;
  f32x4 acc[NET];
#pragma unroll
  for (int j = 0; j < NET; ++j) acc[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  for (int sb = s0; sb < s1; sb += kRU) {
    bf16x8 a[kRU], b[kRU][NET];
#pragma unroll
    for (int u = 0; u < kRU; ++u) {
      // the column offset rides in the per-lane offset, which the range
      // check covers (the scalar offset is not checked): a step past the
      // last row's end reads zero
      const int kb = ((sb + u) * 32 + g * 8) * 2;
      a[u] = __builtin_bit_cast(bf16x8,
                                __builtin_amdgcn_raw_buffer_load_b128(xr, xoff + kb, 0, 0));
#pragma unroll
      for (int j = 0; j < NET; ++j)
        b[u][j] = __builtin_bit_cast(
            bf16x8, __builtin_amdgcn_raw_buffer_load_b128(wr, woff[j] + kb, 0, 0));
    }
#pragma unroll
    for (int u = 0; u < kRU; ++u) {
      const int k = (sb + u) * 32 + g * 8;
      if (sb + u >= s1 || k >= d) a[u] = bf16x8{};  // past this wave's range or the row
#pragma unroll
      for (int j = 0; j < NET; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], b[u][j], acc[j], 0, 0, 0);
    }
  }
#pragma unroll
  for (int j = 0; j < NET; ++j) red[wave][j][lane] = acc[j];
  __syncthreads();
  // output (token m, expert n) of tile j sits in register m % 4 of lane
  // (m / 4) * 16 + n
  for (int o = threadIdx.x; o < NET * 256; o += kSkWaves * kWave) {
    const int j = o / 256, m = (o / 16) % 16, n = o % 16;
    const int src = (m / 4) * 16 + n;
    float v = 0.0f;
#pragma unroll
    for (int wv = 0; wv < kSkWaves; ++wv) v += red[wv][j][src][m % 4];
    const int t = t0 + m, e = e0 + j * 16 + n;
    if (t < N && e < E) logits[(size_t)t * E + e] = v;
  }
}

__global__ __launch_bounds__(256) void router_logits_f32_kernel(
    const float* __restrict__ x, int N, int d, const float* __restrict__ w, int E,
    float* __restrict__ logits) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long long)N * E) return;
  const int t = (int)(i / E), e = (int)(i % E);
  const float* xr = x + (size_t)t * d;
  const float* wr = w + (size_t)e * d;
  float acc = 0.0f;
  for (int k = 0; k < d; ++k) acc = fmaf(xr[k], wr[k], acc);
  logits[i] = acc;
}

}  // namespace

template <int NET>
hipError_t launch_skinny(const bf16* x, int N, int d, const bf16* w, int E, float* logits,
                         hipStream_t stream) {
  const dim3 grid((N + kSkTokens - 1) / kSkTokens, (E + kSkMaxTiles * 16 - 1) / (kSkMaxTiles * 16));
  router_logits_skinny_kernel<NET><<<grid, kSkWaves * kWave, 0, stream>>>(x, N, d, w, E, logits);
  return hipGetLastError();
}

hipError_t launch_router_logits(const void* x, bool bf16_data, int N, int d,
                                const void* w_router, int E, float* logits,
                                hipStream_t stream) {
  if (bf16_data && (E <= kSkMaxTiles * 16 || d % kRK != 0)) {
    const bf16* xb = static_cast<const bf16*>(x);
    const bf16* wb = static_cast<const bf16*>(w_router);
    if (E <= 16) return launch_skinny<1>(xb, N, d, wb, E, logits, stream);
    if (E <= 32) return launch_skinny<2>(xb, N, d, wb, E, logits, stream);
    return launch_skinny<4>(xb, N, d, wb, E, logits, stream);
  }
  if (bf16_data) {
    static std::once_flag once;
    static hipError_t attr = hipSuccess;
    std::call_once(once, [] {
      attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&router_logits_bf16_kernel),
                                 hipFuncAttributeMaxDynamicSharedMemorySize, 2 * kRStage);
    });
    if (attr != hipSuccess) return attr;
    const dim3 grid((N + kRT - 1) / kRT, (E + kRE - 1) / kRE);
    router_logits_bf16_kernel<<<grid, kRThreads, 2 * kRStage, stream>>>(
        static_cast<const bf16*>(x), N, d, static_cast<const bf16*>(w_router), E, logits);
    return hipGetLastError();
  }
  const long long n = (long long)N * E;
  router_logits_f32_kernel<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(
      static_cast<const float*>(x), N, d, static_cast<const float*>(w_router), E, logits);
  return hipGetLastError();
}

}  // namespace moe
