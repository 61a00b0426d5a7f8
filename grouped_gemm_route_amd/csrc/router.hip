// Router projection: logits[t, e] = sum_i x[t, i] * w_router[e, i], fp32.
//
// The router turns each token's hidden state into its expert scores before
// the Top-K choice ("MoE 推理服务工程真相 2026", section 一; "MoE 专家并行的
// All-to-All 通信瓶颈", flowchart step "路由器选 Top-K 专家").
//
// bf16, more than 64 experts (and d a multiple of 64), when N leaves enough
// token blocks: an MFMA GEMM (v_mfma_f32_32x32x16_bf16, fp32 accumulate)
// on block tiles of TT tokens x TE experts, 64 reduction elements per stage.
// A block moves (TT + TE) rows of d elements through its CU, so a CU moves
// ceil(blocks / CUs) (TT + TE) rows in all; the launcher takes whichever of
// 128 x 256 (16 waves), 64 x 64 (8 waves) and the skinny form below makes
// that count smallest.  Both operands go straight
// into LDS (buffer loads to LDS) in a ring of S stages, S - 1 of them in
// flight while one is multiplied, with one fence-free barrier per stage;
// the chunk swizzle of the grouped GEMM keeps the 128-byte rows
// bank-conflict-free, and loads past the last token or expert return zeros.
// The waves form WT x WE wave tiles of 64 x 64 (32 x 32 in the small tile)
// and two waves share each wave tile, one taking the even and one the odd
// 16-wide steps of every stage (two waves per SIMD hide each other's LDS
// reads); the second leaves its partial tile in LDS and the first adds it
// (a fixed order: deterministic).  Each lane's accumulator holds 4
// consecutive experts of one token, stored as 16 bytes.
// fp32 (small layers): one thread per logit, a plain dot product.
#include "moe_internal.h"

#include <mutex>

namespace moe {
namespace {

constexpr int kRK = 64;        // reduction elements per stage
constexpr int kRRow = kRK * 2; // 128-byte LDS rows
constexpr int kRBufferFlags = 0x00020000;
constexpr int kRLds = 160 * 1024;

typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ int rswz(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

template <int TT, int TE>
constexpr int router_stages() {
  return (TT + TE) * kRRow * 4 <= kRLds ? 4 : 3;
}

template <int TT, int TE, int WT, int WE, int NW>
__global__ __launch_bounds__(NW * kWave, 1) void router_logits_tiled_kernel(
    const bf16* __restrict__ x, int N, int d, const bf16* __restrict__ w, int E,
    float* __restrict__ logits) {
  constexpr int KS = NW / (WT * WE);           // waves sharing one wave tile
  constexpr int MT = TT / WT / 32;             // 32-token operands per wave
  constexpr int ME = TE / WE / 32;             // 32-expert operands per wave
  constexpr int kRows = TT + TE;
  constexpr int kStage = kRows * kRRow;
  constexpr int S = router_stages<TT, TE>();
  constexpr int L = kRows / (8 * NW);          // loads per wave and stage
  static_assert(WT * WE * KS == NW && TT % (8 * NW) == 0 && TE % (8 * NW) == 0 &&
                    TT % (32 * WT) == 0 && TE % (32 * WE) == 0,
                "tile shape");
  static_assert(S * kStage <= kRLds, "LDS ring");
  static_assert((KS - 1) * WT * WE * MT * ME * 16 * kWave * 4 <= S * kStage, "partial tiles");
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int t0 = blockIdx.x * TT;
  const int e0 = blockIdx.y * TE;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int ks = wave / (WT * WE);
  const int wt = (wave % (WT * WE)) / WE;
  const int we = wave % WE;
  const int nt = min(TT, N - t0);
  const int ne = min(TE, E - e0);
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(x + (size_t)t0 * d), 0, (uint32_t)((size_t)nt * d * 2), kRBufferFlags);
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(w + (size_t)e0 * d), 0, (uint32_t)((size_t)ne * d * 2), kRBufferFlags);
  // load i of a wave fills LDS rows (NW i + wave) * 8 .. + 8 of a stage: token
  // rows first, then expert rows; lane l carries 16 bytes of row l / 8 (the
  // global chunk that the swizzle puts at LDS chunk l % 8).  The column
  // offset rides in the per-lane offset, which the range check covers.
  const int grow = lane >> 3;
  int src[L];
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const int lr = (i * NW + wave) * 8 + grow;
    const int row = lr < TT ? lr : lr - TT;
    src[i] = (row * d + rswz(lr, lane & 7) * 8) * 2;
  }
  auto issue = [&](int slot, int k0) __attribute__((always_inline)) {
    char* base = lds + slot * kStage;
    const int koff = k0 * 2;
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int v = src[i] + koff;
      char* dst = base + (i * NW + wave) * 8 * kRRow;
      if (i * NW * 8 < TT)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_void_t*)dst, 16, v, 0, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_void_t*)dst, 16, v, 0, 0, 0);
    }
  };

  const int lrow = lane & 31;
  const int lhalf = lane >> 5;
  f32x16 acc[ME][MT];
#pragma unroll
  for (int j = 0; j < ME; ++j)
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.0f;

  const int nk = d / kRK;
#pragma unroll
  for (int s = 0; s < S - 1; ++s)
    if (s < nk) issue(s, s * kRK);
  for (int kt = 0; kt < nk; ++kt) {
    // this wave's loads of stage kt are done once at most the later issued
    // stages (up to S - 2 of them) remain in flight
    const int later = min(S - 2, nk - 1 - kt);
    if (later >= 2)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * L) : "memory");
    else if (later == 1)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(L) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    // every wave's loads of stage kt have landed, and every wave is done
    // with stage kt - 1, whose slot the next issue refills.  The barrier
    // carries no memory fence: a fence would also wait for the later
    // stages' loads still in flight.
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (kt + S - 1 < nk) issue((kt + S - 1) % S, (kt + S - 1) * kRK);
    const char* sb = lds + (kt % S) * kStage;
#pragma unroll
    for (int st = ks; st < kRK / 16; st += KS) {
      const int chunk = st * 2 + lhalf;
      bf16x8 wf[ME], xf[MT];
#pragma unroll
      for (int j = 0; j < ME; ++j) {
        const int row = TT + we * (TE / WE) + j * 32 + lrow;
        wf[j] = *reinterpret_cast<const bf16x8*>(sb + row * kRRow + rswz(row, chunk) * 16);
      }
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const int row = wt * (TT / WT) + i * 32 + lrow;
        xf[i] = *reinterpret_cast<const bf16x8*>(sb + row * kRRow + rswz(row, chunk) * 16);
      }
#pragma unroll
      for (int j = 0; j < ME; ++j)
#pragma unroll
        for (int i = 0; i < MT; ++i)
          acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[j], xf[i], acc[j][i], 0, 0, 0);
    }
  }

  // accumulator register r of lane l: expert (r / 4) * 8 + (l / 32) * 4 + r % 4
  // of its 32-expert operand, token l % 32 of its 32-token operand
  auto store = [&](int j, int i, const f32x16& v) __attribute__((always_inline)) {
    const int t = t0 + wt * (TT / WT) + i * 32 + lrow;
    if (t >= N) return;
    float* orow = logits + (size_t)t * E;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int e = e0 + we * (TE / WE) + j * 32 + r4 * 8 + lhalf * 4;
      if (e + 3 < E && (E & 3) == 0) {
        f32x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = v[r4 * 4 + q];
        *reinterpret_cast<f32x4*>(orow + e) = o;
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (e + q < E) orow[e + q] = v[r4 * 4 + q];
      }
    }
  };
  if constexpr (KS == 1) {
#pragma unroll
    for (int j = 0; j < ME; ++j)
#pragma unroll
      for (int i = 0; i < MT; ++i) store(j, i, acc[j][i]);
  } else {
    // reduction shares 1..KS-1 leave their tiles in LDS (the ring is free
    // once every wave has passed this barrier: the last stage was waited
    // for with vmcnt(0)); share 0 adds them in share order and stores
    __syncthreads();
    f32x4* part = reinterpret_cast<f32x4*>(lds);
    const int tile = wt * WE + we;
    auto slot = [&](int p, int j, int i, int q) __attribute__((always_inline)) {
      return (((((p - 1) * WT * WE + tile) * ME + j) * MT + i) * 4 + q) * kWave + lane;
    };
    if (ks > 0) {
#pragma unroll
      for (int j = 0; j < ME; ++j)
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            f32x4 v;
#pragma unroll
            for (int c = 0; c < 4; ++c) v[c] = acc[j][i][q * 4 + c];
            part[slot(ks, j, i, q)] = v;
          }
    }
    __syncthreads();
    if (ks > 0) return;
#pragma unroll
    for (int j = 0; j < ME; ++j)
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        f32x16 v = acc[j][i];
#pragma unroll
        for (int p = 1; p < KS; ++p)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x4 u = part[slot(p, j, i, q)];
#pragma unroll
            for (int c = 0; c < 4; ++c) v[q * 4 + c] += u[c];
          }
        store(j, i, v);
      }
  }
}

// Skinny form, for up to 64 experts per block (all E <= 64, any E when d is
// not a multiple of 64, and blocks of 16 experts when there are too few
// tokens for the tiled kernel to reach the CUs): the projection is bound by
// reading x once, so
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
    const bf16* __restrict__ x, int N, int d, const bf16* __restrict__ w, int E, int epb,
    float* __restrict__ logits) {
  constexpr int kRU = skinny_steps_in_flight<NET>();
  __shared__ f32x4 red[kSkWaves][NET][kWave];
  const int t0 = blockIdx.x * kSkTokens;
  const int e0 = blockIdx.y * epb;  // epb <= NET * 16 experts per block
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int r = lane & 15;
  const int g = lane >> 4;
  const int nt = min(kSkTokens, N - t0);
  const int ne = min(epb, E - e0);
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
    if (t < N && j * 16 + n < ne) logits[(size_t)t * E + e] = v;
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

template <int NET>
hipError_t launch_skinny(const bf16* x, int N, int d, const bf16* w, int E, float* logits,
                         hipStream_t stream, int epb = NET * 16) {
  const dim3 grid((N + kSkTokens - 1) / kSkTokens, (E + epb - 1) / epb);
  router_logits_skinny_kernel<NET>
      <<<grid, kSkWaves * kWave, 0, stream>>>(x, N, d, w, E, epb, logits);
  return hipGetLastError();
}

template <int TT, int TE, int WT, int WE, int NW>
hipError_t launch_tiled(const bf16* x, int N, int d, const bf16* w, int E, float* logits,
                        hipStream_t stream) {
  constexpr int lds_bytes = router_stages<TT, TE>() * (TT + TE) * kRRow;
  static std::once_flag once;
  static hipError_t attr = hipSuccess;
  std::call_once(once, [] {
    attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&router_logits_tiled_kernel<TT, TE, WT, WE, NW>),
        hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
  });
  if (attr != hipSuccess) return attr;
  const dim3 grid((N + TT - 1) / TT, (E + TE - 1) / TE);
  router_logits_tiled_kernel<TT, TE, WT, WE, NW><<<grid, NW * kWave, lds_bytes, stream>>>(
      x, N, d, w, E, logits);
  return hipGetLastError();
}

int router_cus() {
  constexpr int kMaxDevices = 64;
  static int cache[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < kMaxDevices && cache[dev] > 0) return cache[dev];
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  if (dev < kMaxDevices) cache[dev] = cus;
  return cus;
}

// Rows of d elements a CU moves for the projection, in units of one block's
// rounds: ceil(blocks / CUs) x (tokens + experts a block reads).
int64_t router_cost(int N, int E, int tt, int te, int cus) {
  const int64_t blocks = (int64_t)((N + tt - 1) / tt) * ((E + te - 1) / te);
  return (blocks + cus - 1) / cus * (int64_t)(min(tt, N) + min(te, E));
}

}  // namespace

hipError_t launch_router_logits(const void* x, bool bf16_data, int N, int d,
                                const void* w_router, int E, float* logits,
                                hipStream_t stream) {
  if (bf16_data) {
    const bf16* xb = static_cast<const bf16*>(x);
    const bf16* wb = static_cast<const bf16*>(w_router);
    // up to 64 experts, or d not a multiple of 64: the skinny form with
    // one block over all experts
    if (E <= kSkMaxTiles * 16 || d % kRK != 0) {
      if (E <= 16) return launch_skinny<1>(xb, N, d, wb, E, logits, stream);
      if (E <= 32) return launch_skinny<2>(xb, N, d, wb, E, logits, stream);
      return launch_skinny<4>(xb, N, d, wb, E, logits, stream);
    }
    // more experts: the cheapest of the large tile, the small tile and the
    // skinny form on blocks of 16, 8, 4 or 2 experts (few tokens: x, read
    // by every block of its token rows, comes from L2 and w_router is spread
    // over more CUs)
    const int cus = router_cus();
    const int64_t big = router_cost(N, E, 128, 256, cus);
    const int64_t small = router_cost(N, E, 64, 64, cus);
    int epb = 16;
    int64_t skinny = router_cost(N, E, kSkTokens, 16, cus);
    for (int c = 8; c >= 2; c /= 2) {
      const int64_t cost = router_cost(N, E, kSkTokens, c, cus);
      if (cost < skinny) skinny = cost, epb = c;
    }
    if (skinny < small && skinny < big)
      return launch_skinny<1>(xb, N, d, wb, E, logits, stream, epb);
    if (big <= small) return launch_tiled<128, 256, 2, 4, 16>(xb, N, d, wb, E, logits, stream);
    return launch_tiled<64, 64, 2, 2, 8>(xb, N, d, wb, E, logits, stream);
  }
  const long long n = (long long)N * E;
  router_logits_f32_kernel<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(
      static_cast<const float*>(x), N, d, static_cast<const float*>(w_router), E, logits);
  return hipGetLastError();
}

}  // namespace moe
