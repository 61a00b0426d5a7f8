// Ragged grouped-GEMM SwiGLU expert FFN.
//
// "MoE 专家并行的 All-to-All 通信瓶颈", flowchart step "Grouped GEMM 专家计算"
// and section "容量因子、专家复制与 dropless 的取舍": each expert multiplies
// its own, variable number of token rows, all experts in one call, with no
// padding of the token count.  Per expert e on rows R = x_perm[offsets[e] :
// offsets[e+1]]:  h = silu(R Wg[e]^T) * (R Wu[e]^T);  y = h Wd[e]^T.
//
// Scheduling.  A one-block kernel turns offsets[] (which stays on the device)
// into a list of row tiles (expert, first row, end row), each at most
// kTileRows rows of one expert.  The GEMM grid is sized on the host from the
// upper bound max_rows; block (n_tile, slot) with slot >= the real tile count
// exits at once.  Slots vary fastest, so the blocks that run together share
// one weight tile (the large operand) and it is fetched from HBM about once.
//
// bf16 GEMM (gfx950 MFMA v_mfma_f32_32x32x16_bf16, fp32 accumulate).  Both
// operands are contiguous along the reduction dimension (x_perm and h rows;
// weight rows), so every MFMA operand is one 16-byte LDS read.  The weight
// is the MFMA "A" operand (32 output features) and the activations the "B"
// operand (32 tokens): each lane's accumulator then holds runs of 4
// consecutive features of one token, which the epilogue stores as 8 bytes.
//   block tile: 128 tokens x 256 weight rows x 64 reduction elements;
//     the gate/up pass loads 128 gate rows and the same 128 up rows, so a
//     wave holds matching gate and up accumulators and applies SwiGLU in
//     registers; the down pass loads 256 rows of Wd.
//   4 waves in 2 x 2; each wave: 4 weight tiles x 2 token tiles of 32 x 32.
//   LDS: two stages of (256 + 128) rows x 128 bytes = 96 KB; 16-byte chunks
//     XOR-swizzled by (row & 7) so the 8 lanes of an LDS read phase hit 8
//     different bank groups.
//   pipeline: the next reduction tile is loaded to registers while the
//     current one feeds the MFMAs, then written to the other LDS stage; one
//     barrier per reduction tile.
// fp32 path: a plain LDS-tiled FMA kernel (64 x 64 tiles), used for fp32
// layers, which are small.
#include "moe_internal.h"
#include "block_scan.h"

#include <mutex>

namespace moe {
namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------------------
// tile schedule
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(1024) void ffn_schedule_kernel(
    const int32_t* __restrict__ offsets, int E, int tile_rows, int max_rows,
    int max_tiles, int4* __restrict__ tiles, int* __restrict__ num_tiles) {
  __shared__ int wave_sums[1024 / kWave];
  const int e = threadIdx.x;
  int a = 0, b = 0, nt = 0;
  if (e < E) {
    a = min(max(offsets[e], 0), max_rows);
    b = min(max(offsets[e + 1], a), max_rows);
    nt = (b - a + tile_rows - 1) / tile_rows;
  }
  int total = 0;
  const int base = block_exclusive_scan(nt, wave_sums, &total);
  for (int i = 0; i < nt; ++i) {
    const int slot = base + i;
    if (slot < max_tiles) {
      const int r0 = a + i * tile_rows;
      tiles[slot] = make_int4(e, r0, min(b, r0 + tile_rows), 0);
    }
  }
  if (e == 0) *num_tiles = min(total, max_tiles);
}

inline int max_tiles_for(int64_t max_rows, int E, int tile_rows) {
  return (int)((max_rows + tile_rows - 1) / tile_rows +
               (max_rows < E ? max_rows : E));
}

// ---------------------------------------------------------------------------
// bf16 MFMA GEMM
// ---------------------------------------------------------------------------

constexpr int kBM = kBf16TileRows;  // 128 token rows
constexpr int kBW = 256;            // weight rows per block tile
constexpr int kBK = 64;             // reduction elements per stage
constexpr int kWElems = kBW * kBK;
constexpr int kAElems = kBM * kBK;
constexpr int kStageElems = kWElems + kAElems;
constexpr size_t kBf16Lds = 2 * kStageElems * sizeof(bf16);  // 96 KB

// Element offset of 16-byte chunk `chunk` (0..7) of LDS row `row`.
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kBK + ((chunk ^ (row & 7)) << 3);
}

template <bool kDual>
__global__ __launch_bounds__(kThreads, 1) void ffn_gemm_bf16_kernel(
    const bf16* __restrict__ act, int Kdim, const bf16* __restrict__ w0,
    const bf16* __restrict__ w1, int Nout, bf16* __restrict__ out,
    const int4* __restrict__ tiles, const int* __restrict__ num_tiles,
    int m_slots) {
  extern __shared__ __attribute__((aligned(16))) bf16 lds[];
  const int slot = blockIdx.x % m_slots;
  const int n_tile = blockIdx.x / m_slots;
  if (slot >= *num_tiles) return;
  const int4 tile = tiles[slot];
  const int e = tile.x;
  const int row0 = tile.y;
  const int rows = tile.z - tile.y;
  constexpr int kNOut = kDual ? kBW / 2 : kBW;  // output columns per block
  const int n0 = n_tile * kNOut;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int ld_row = tid >> 3;   // 0..31
  const int ld_chunk = tid & 7;  // 16-byte chunk within a 128-byte row

  // Global sources of this thread's 8 weight rows and 4 token rows.
  const size_t wbase = (size_t)e * Nout * Kdim;
  const bf16* wsrc[8];
  int w_off[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int lr = i * 32 + ld_row;
    int n;
    const bf16* base;
    if (kDual) {
      n = n0 + (lr & (kBW / 2 - 1));
      base = lr < kBW / 2 ? w0 : w1;
    } else {
      n = n0 + lr;
      base = w0;
    }
    n = min(n, Nout - 1);  // rows past the edge are loaded but not stored
    wsrc[i] = base + wbase + (size_t)n * Kdim + ld_chunk * 8;
    w_off[i] = swz(lr, ld_chunk);
  }
  const bf16* asrc[4];
  int a_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int lr = i * 32 + ld_row;
    const int r = row0 + min(lr, rows - 1);
    asrc[i] = act + (size_t)r * Kdim + ld_chunk * 8;
    a_off[i] = kWElems + swz(lr, ld_chunk);
  }

  uint4 wreg[8], areg[4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) wreg[i] = *reinterpret_cast<const uint4*>(wsrc[i] + k0);
#pragma unroll
    for (int i = 0; i < 4; ++i) areg[i] = *reinterpret_cast<const uint4*>(asrc[i] + k0);
  };
  auto lstore = [&](int stage) {
    bf16* s = lds + stage * kStageElems;
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<uint4*>(s + w_off[i]) = wreg[i];
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(s + a_off[i]) = areg[i];
  };

  // Wave tiling: wm picks 64 of the 128 tokens, wn half of the weight rows.
  const int wm = wave & 1;
  const int wn = wave >> 1;
  int wrow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    wrow[i] = kDual ? (i >> 1) * (kBW / 2) + wn * 64 + (i & 1) * 32 : wn * 128 + i * 32;
  const int arow0 = wm * 64;
  const int lrow = lane & 31;
  const int lhalf = lane >> 5;

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nk = Kdim / kBK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * kBK);
    const bf16* s = lds + cur * kStageElems;
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      const int chunk = ks * 2 + lhalf;
      bf16x8 af[4], bfr[2];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(s + swz(wrow[i] + lrow, chunk));
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8*>(s + kWElems + swz(arow0 + j * 32 + lrow, chunk));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) lstore(cur ^ 1);
    __syncthreads();
  }

  // Epilogue.  Accumulator register r of lane l holds feature
  // (r / 4) * 8 + (l / 32) * 4 + r % 4 of its 32-row weight tile and token
  // l % 32 of its 32-row token tile.
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int m_local = arow0 + j * 32 + lrow;
    if (m_local >= rows) continue;
    bf16* orow = out + (size_t)(row0 + m_local) * Nout;
    if (kDual) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int f = n0 + wn * 64 + i * 32 + r4 * 8 + lhalf * 4;
          if (f >= Nout) continue;
          bf16x4 o;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float g = acc[i][j][r4 * 4 + q];
            const float u = acc[i + 2][j][r4 * 4 + q];
            o[q] = (bf16)(g / (1.0f + __expf(-g)) * u);
          }
          *reinterpret_cast<bf16x4*>(orow + f) = o;
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int f = n0 + wn * 128 + i * 32 + r4 * 8 + lhalf * 4;
          if (f >= Nout) continue;
          bf16x4 o;
#pragma unroll
          for (int q = 0; q < 4; ++q) o[q] = (bf16)acc[i][j][r4 * 4 + q];
          *reinterpret_cast<bf16x4*>(orow + f) = o;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 FMA GEMM (small layers)
// ---------------------------------------------------------------------------

constexpr int kFM = kF32TileRows;  // 64 tokens
constexpr int kFN = 64;            // output columns
constexpr int kFK = 16;

template <bool kDual>
__global__ __launch_bounds__(kThreads) void ffn_gemm_f32_kernel(
    const float* __restrict__ act, int Kdim, const float* __restrict__ w0,
    const float* __restrict__ w1, int Nout, float* __restrict__ out,
    const int4* __restrict__ tiles, const int* __restrict__ num_tiles,
    int m_slots) {
  __shared__ float a_s[kFK][kFM + 1];
  __shared__ float w0_s[kFK][kFN + 1];
  __shared__ float w1_s[kDual ? kFK : 1][kFN + 1];
  const int slot = blockIdx.x % m_slots;
  const int n_tile = blockIdx.x / m_slots;
  if (slot >= *num_tiles) return;
  const int4 tile = tiles[slot];
  const int e = tile.x;
  const int row0 = tile.y;
  const int rows = tile.z - tile.y;
  const int n0 = n_tile * kFN;
  const int tid = threadIdx.x;
  const int tx = tid % 16;  // columns tx*4 ..
  const int ty = tid / 16;  // rows ty*4 ..
  const size_t wbase = (size_t)e * Nout * Kdim;

  float acc0[4][4] = {}, acc1[4][4] = {};
  for (int k0 = 0; k0 < Kdim; k0 += kFK) {
#pragma unroll
    for (int i = 0; i < (kFM * kFK) / kThreads; ++i) {
      const int q = tid + i * kThreads;
      const int r = q / kFK, kk = q % kFK;
      const int k = k0 + kk;
      const int row = row0 + min(r, rows - 1);
      a_s[kk][r] = k < Kdim ? act[(size_t)row * Kdim + k] : 0.0f;
      const int n = min(n0 + r, Nout - 1);
      w0_s[kk][r] = k < Kdim ? w0[wbase + (size_t)n * Kdim + k] : 0.0f;
      if (kDual) w1_s[kk][r] = k < Kdim ? w1[wbase + (size_t)n * Kdim + k] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kFK; ++kk) {
      float a[4], b0[4], b1[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = a_s[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        b0[j] = w0_s[kk][tx * 4 + j];
        if (kDual) b1[j] = w1_s[kk][tx * 4 + j];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc0[i][j] = fmaf(a[i], b0[j], acc0[i][j]);
          if (kDual) acc1[i][j] = fmaf(a[i], b1[j], acc1[i][j]);
        }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = ty * 4 + i;
    if (m >= rows) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n >= Nout) continue;
      float v = acc0[i][j];
      if (kDual) v = v / (1.0f + __expf(-v)) * acc1[i][j];
      out[(size_t)(row0 + m) * Nout + n] = v;
    }
  }
}

std::once_flag g_lds_once;
hipError_t g_lds_status = hipSuccess;

hipError_t ensure_lds_attributes() {
  std::call_once(g_lds_once, [] {
    hipError_t e1 = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&ffn_gemm_bf16_kernel<true>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)kBf16Lds);
    hipError_t e2 = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&ffn_gemm_bf16_kernel<false>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)kBf16Lds);
    g_lds_status = e1 != hipSuccess ? e1 : e2;
  });
  return g_lds_status;
}

}  // namespace

size_t grouped_ffn_workspace_bytes(int64_t max_rows, int E, bool bf16_data) {
  const int tr = bf16_data ? kBf16TileRows : kF32TileRows;
  return 256 + (size_t)max_tiles_for(max_rows, E, tr) * sizeof(int4);
}

hipError_t launch_grouped_ffn(const void* x_perm, bool bf16_data, int d,
                              int ffn, int E, const int32_t* offsets,
                              int64_t max_rows, const void* w_gate,
                              const void* w_up, const void* w_down, void* h,
                              void* y_perm, void* workspace,
                              hipStream_t stream) {
  if (max_rows == 0) return hipSuccess;
  const int tr = bf16_data ? kBf16TileRows : kF32TileRows;
  const int m_slots = max_tiles_for(max_rows, E, tr);
  int* num_tiles = static_cast<int*>(workspace);
  int4* tiles = reinterpret_cast<int4*>(static_cast<char*>(workspace) + 256);
  ffn_schedule_kernel<<<1, 1024, 0, stream>>>(offsets, E, tr, (int)max_rows,
                                              m_slots, tiles, num_tiles);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  if (bf16_data) {
    err = ensure_lds_attributes();
    if (err != hipSuccess) return err;
    const int n_up = (ffn + kBW / 2 - 1) / (kBW / 2);
    ffn_gemm_bf16_kernel<true><<<n_up * m_slots, kThreads, kBf16Lds, stream>>>(
        static_cast<const bf16*>(x_perm), d, static_cast<const bf16*>(w_gate),
        static_cast<const bf16*>(w_up), ffn, static_cast<bf16*>(h), tiles,
        num_tiles, m_slots);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int n_dn = (d + kBW - 1) / kBW;
    ffn_gemm_bf16_kernel<false><<<n_dn * m_slots, kThreads, kBf16Lds, stream>>>(
        static_cast<const bf16*>(h), ffn, static_cast<const bf16*>(w_down),
        nullptr, d, static_cast<bf16*>(y_perm), tiles, num_tiles, m_slots);
    return hipGetLastError();
  }
  const int n_up = (ffn + kFN - 1) / kFN;
  ffn_gemm_f32_kernel<true><<<n_up * m_slots, kThreads, 0, stream>>>(
      static_cast<const float*>(x_perm), d, static_cast<const float*>(w_gate),
      static_cast<const float*>(w_up), ffn, static_cast<float*>(h), tiles,
      num_tiles, m_slots);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int n_dn = (d + kFN - 1) / kFN;
  ffn_gemm_f32_kernel<false><<<n_dn * m_slots, kThreads, 0, stream>>>(
      static_cast<const float*>(h), ffn, static_cast<const float*>(w_down),
      nullptr, d, static_cast<float*>(y_perm), tiles, num_tiles, m_slots);
  return hipGetLastError();
}

}  // namespace moe
