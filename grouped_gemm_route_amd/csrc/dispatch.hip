// Dispatch: histogram, capacity drop, prefix scan and the stable permutation
// of tokens into per-expert contiguous rows, rank-major.
//
// Follows the dispatch pseudocode of "MoE 推理服务工程真相 2026", section 2.3
// (bincount of expert ids -> overflow against the capacity -> grouping for
// the all-to-all), with the capacity of section 2.2 and the expert drop of
// section 4.3, and the dense token-to-expert mapping table built from a
// cumsum in "MoE Inference Communication", section "MoE 计算核优化".
//
// Row of a kept pair (t, k) with expert e: offsets[e] + r, where r is the
// number of tokens t' < t routed to e (each token names an expert at most
// once).  r is assembled from three integer parts, so every row position is
// exact and independent of scheduling:
//   rank kernel    (one thread per token, 256 tokens per block): within a
//                  wave, lane l routed to e sets bit l of mask[wave][e] with
//                  an LDS atomic OR (order-free); its rank inside the block
//                  is popcount(mask[wave][e] & lanes-below-l) plus the
//                  popcounts of the earlier waves' masks.  The block's
//                  per-expert totals go to block_counts[b][e].
//   scan kernel    (one block, rank_scan.h): per expert, an exclusive scan
//                  of the block totals over blocks (block_excl) and their
//                  sum (demand); counts = min(demand, capacity); offsets =
//                  exclusive scan of counts over experts; rank_offsets[r] =
//                  offsets[r*E/W].
//   scatter kernel (one block per token): loads the token's row once from
//                  HBM in 16-byte pieces; meanwhile r = block_excl + local
//                  rank, kept iff capacity < 0 or r < capacity, and dest and
//                  perm_token are written; then every piece is stored to
//                  each kept destination row.  When the per-block count
//                  table is small, every scatter block scans it itself and
//                  the scan kernel is not launched.
// Because experts are numbered rank by rank, the (expert, token) order is
// rank-major: rank r's send slice is rows [rank_offsets[r], rank_offsets[r+1]).
// The planned dispatch (launch_dispatch_planned) has no rank kernel: the
// routing kernel's fused variant (route_topk.hip) has already ranked the
// tokens and counted them per expert, in blocks of its own size.
#include "moe_route.h"
#include "moe_internal.h"
#include "block_scan.h"
#include "fp8_codec.h"
#include "rank_scan.h"

#include <type_traits>

namespace moe {
namespace {

constexpr int kRankWaves = kRankBlockTokens / kWave;  // 4

__global__ __launch_bounds__(kRankBlockTokens) void dispatch_rank_kernel(
    const int32_t* __restrict__ topk_idx, int N, int E, int K,
    int32_t* __restrict__ block_counts, int32_t* __restrict__ local_rank) {
  extern __shared__ unsigned long long masks[];  // [kRankWaves][E]
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  for (int i = tid; i < kRankWaves * E; i += blockDim.x) masks[i] = 0ull;
  __syncthreads();

  const int t = blockIdx.x * kRankBlockTokens + tid;
  const bool valid = t < N;
  if (valid) {
    for (int k = 0; k < K; ++k) {
      const int e = topk_idx[(size_t)t * K + k];
      if ((unsigned)e < (unsigned)E) atomicOr(&masks[wave * E + e], 1ull << lane);
    }
  }
  __syncthreads();

  if (valid) {
    const unsigned long long below = (1ull << lane) - 1ull;
    for (int k = 0; k < K; ++k) {
      const int e = topk_idx[(size_t)t * K + k];
      int r = 0;
      if ((unsigned)e < (unsigned)E) {
        r = __popcll(masks[wave * E + e] & below);
        for (int w = 0; w < wave; ++w) r += __popcll(masks[w * E + e]);
      }
      local_rank[(size_t)t * K + k] = r;
    }
  }
  for (int e = tid; e < E; e += blockDim.x) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < kRankWaves; ++w) c += __popcll(masks[w * E + e]);
    block_counts[(size_t)blockIdx.x * E + e] = c;
  }
}

// One block: the per-expert scan of the rank kernel's count table
// (rank_scan.h).
__global__ __launch_bounds__(kRankScanThreads) void dispatch_scan_kernel(
    const int32_t* __restrict__ block_counts, int B, int E, int W,
    int64_t capacity, int32_t* __restrict__ block_excl,
    int32_t* __restrict__ demand, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ rank_offsets) {
  __shared__ RankScanShared sh;
  scan_rank_table<false>(block_counts, B, E, W, capacity, block_excl, demand, counts, offsets,
                         rank_offsets, sh);
}

// Threads of a scatter block (one token): 64, 128 or the most, 256.
constexpr int kScatterMaxThreads = 256;
// Largest per-block count table (blocks x experts), and most experts, that
// every scatter block scans for itself instead of waiting for the one-block
// scan kernel.
constexpr int kFusedScanMaxCounts = 1024;
constexpr int kFusedScanMaxExperts = 256;
// At most this many 16-byte pieces of the token's row per thread are loaded
// before the index work (rows of up to 4 * threads pieces are held whole in
// registers); launches pick the fewest that hold the row.
constexpr int kMaxHeld = 4;
// Below this many tokens the scatter runs 256 threads per token whatever the
// row width.
constexpr int kScatterFewTokens = 1024;
// buffer resource word 3 for raw 32-bit accesses (data format 32)
constexpr int kRowBufferFlags = 0x00020000;

// One block per token.  Every thread first loads its pieces of the token's
// row into registers; meanwhile wave 0 finds the token's K destination rows,
// and after one barrier the block stores each piece to every kept row.
//   kFusedScan: the per-block count table is small, so wave 0 copies it into
//   LDS (one coalesced round trip) and computes the expert offsets and the
//   token's per-expert bases from it (block 0 also writes demand / counts /
//   offsets / rank_offsets); otherwise block_excl and offsets come from the
//   scan kernel.
//   kFp8: the payload is the fp8 form of the bf16 row (fp8_codec.h): a
//   piece's 16 lanes of one 128-column group agree on its scale, and each
//   lane stores its 8 codes (8 bytes) and, once per group, the scale to
//   every kept row.
//   kHeld: pieces per thread loaded ahead (1, 2 or kMaxHeld); pieces past
//   kHeld * kThreads are loaded and stored one at a time afterwards.
//   tpb: tokens per rank block (the rank kernel's or the fused routing
//   kernel's block), the rows of block_counts / block_excl.
//   kThreads: the block's threads.  Fewer threads, each holding more
//   pieces, launch fewer waves for the same bytes: with many tokens the
//   launch picks about a quarter of the row's pieces (64, 128 or 256).
template <bool kFusedScan, bool kFp8, int kHeld, int kThreads>
__global__ __launch_bounds__(kThreads) void dispatch_scatter_kernel(
    const uint4* __restrict__ x, int row_chunks, int N,
    const int32_t* __restrict__ topk_idx, int E, int K, int W, int64_t capacity, int tpb,
    const int32_t* __restrict__ block_counts, const int32_t* __restrict__ block_excl,
    const int32_t* __restrict__ local_rank, int32_t* __restrict__ offsets,
    int32_t* __restrict__ demand, int32_t* __restrict__ counts,
    int32_t* __restrict__ rank_offsets, void* __restrict__ x_perm,
    float* __restrict__ x_scale, int32_t* __restrict__ perm_token,
    int32_t* __restrict__ dest) {
  __shared__ int rows[MOE_MAX_TOPK];
  __shared__ int table[kFusedScan ? kFusedScanMaxCounts : 1];
  __shared__ int offs[kFusedScan ? kFusedScanMaxExperts + 1 : 1];
  __shared__ int base[kFusedScan ? kFusedScanMaxExperts : 1];
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int b = t / tpb;  // rank block

  const uint4* src = x + (size_t)t * row_chunks;
  // a buffer resource over the row: pieces past its end read as zero, so the
  // loads need no branch (a branch around each would make the compiler wait
  // for every load right after issuing it)
  const __amdgpu_buffer_rsrc_t row_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)src, 0, row_chunks * (int)sizeof(uint4), kRowBufferFlags);
  u32x4 held[kHeld];
#pragma unroll
  for (int u = 0; u < kHeld; ++u)
    held[u] = __builtin_amdgcn_raw_buffer_load_b128(
        row_rsrc, (tid + u * kThreads) * (int)sizeof(uint4), 0, 0);

  if (tid < kWave) {
    int e = -1, lr = 0;
    if (lane < K) {
      e = topk_idx[(size_t)t * K + lane];
      lr = local_rank[(size_t)t * K + lane];
    }
    int row = -1;
    if constexpr (kFusedScan) {
      // E <= 256: lane l owns experts 4l .. 4l + 3
      const int B = (N + tpb - 1) / tpb;
      // all of the table's loads are issued before any is waited for
      constexpr int kPer = kFusedScanMaxCounts / kWave;
      int cv[kPer];
#pragma unroll
      for (int m = 0; m < kPer; ++m) {
        const int i = lane + m * kWave;
        cv[m] = i < B * E ? block_counts[i] : 0;
      }
#pragma unroll
      for (int m = 0; m < kPer; ++m) {
        const int i = lane + m * kWave;
        if (i < B * E) table[i] = cv[m];
      }
      int kept[4];
      int lane_sum = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int ex = lane * 4 + j;
        int pre = 0, tot = 0;
        if (ex < E) {
          for (int bb = 0; bb < B; ++bb) {
            const int c = table[bb * E + ex];
            if (bb < b) pre += c;
            tot += c;
          }
          base[ex] = pre;
          if (t == 0) demand[ex] = tot;
        }
        kept[j] = capacity < 0 ? tot : (int)min((int64_t)tot, capacity);
        lane_sum += kept[j];
      }
      int incl = lane_sum;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const int o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
      }
      int run = incl - lane_sum;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int ex = lane * 4 + j;
        if (ex < E) {
          offs[ex] = run;
          if (t == 0) {
            counts[ex] = kept[j];
            offsets[ex] = run;
          }
        }
        run += kept[j];
      }
      if (lane == kWave - 1) {
        offs[E] = incl;
        if (t == 0) offsets[E] = incl;
      }
      if (t == 0) {
        const int per_rank = E / W;
        for (int r = lane; r <= W; r += kWave) rank_offsets[r] = offs[r * per_rank];
      }
      if ((unsigned)e < (unsigned)E) {
        const int r = lr + base[e];
        if (capacity < 0 || (int64_t)r < capacity) row = offs[e] + r;
      }
    } else {
      if ((unsigned)e < (unsigned)E) {
        const int r = lr + block_excl[(size_t)b * E + e];
        if (capacity < 0 || (int64_t)r < capacity) row = offsets[e] + r;
      }
    }
    // a row outside the N*K buffer rows can only come from a count table
    // that does not belong to this topk_idx (a misused plan); it is dropped,
    // so the stores below stay inside x_perm and perm_token
    if ((unsigned)row >= (unsigned)(N * K)) row = -1;
    if (lane < K) {
      rows[lane] = row;
      dest[(size_t)t * K + lane] = row;
      if (row >= 0) perm_token[row] = t;
    }
  }
  // wave 0's LDS writes are done before the barrier; the row loads stay in
  // flight across it
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  // One wait for all held pieces before the first store: a store counts in
  // the same counter as the loads, so a wait placed later would also wait
  // for the stores issued before it.
#pragma unroll
  for (int u = 0; u < kHeld; ++u) asm volatile("" ::"v"(held[u]));
  const int extra0 = tid + kHeld * kThreads;  // pieces beyond the held ones

  if constexpr (kFp8) {
    // row_chunks is a multiple of 16, so the lanes of a group are active
    // together
    constexpr int kPieces = kFp8Group / 8;
    const int groups = row_chunks / kPieces;
    uint2* q = static_cast<uint2*>(x_perm);
    uint2 codes[kHeld];
    float scale[kHeld];
#pragma unroll
    for (int u = 0; u < kHeld; ++u) {
      const int c = tid + u * kThreads;
      if (c < row_chunks) codes[u] = quantize_piece(__builtin_bit_cast(uint4, held[u]), &scale[u]);
    }
    for (int k = 0; k < K; ++k) {
      const int rk = rows[k];
      if (rk < 0) continue;
#pragma unroll
      for (int u = 0; u < kHeld; ++u) {
        const int c = tid + u * kThreads;
        if (c < row_chunks) {
          q[(size_t)rk * row_chunks + c] = codes[u];
          if (c % kPieces == 0) x_scale[(size_t)rk * groups + c / kPieces] = scale[u];
        }
      }
    }
    for (int c = extra0; c < row_chunks; c += kThreads) {
      float sc;
      const uint2 cd = quantize_piece(src[c], &sc);
      for (int k = 0; k < K; ++k) {
        const int rk = rows[k];
        if (rk < 0) continue;
        q[(size_t)rk * row_chunks + c] = cd;
        if (c % kPieces == 0) x_scale[(size_t)rk * groups + c / kPieces] = sc;
      }
    }
  } else {
    u32x4* dst = static_cast<u32x4*>(x_perm);
    for (int k = 0; k < K; ++k) {
      const int rk = rows[k];
      if (rk < 0) continue;
      u32x4* drow = dst + (size_t)rk * row_chunks;
#pragma unroll
      for (int u = 0; u < kHeld; ++u) {
        const int c = tid + u * kThreads;
        if (c < row_chunks) drow[c] = held[u];
      }
    }
    for (int c = extra0; c < row_chunks; c += kThreads) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(src + c);
      for (int k = 0; k < K; ++k) {
        const int rk = rows[k];
        if (rk >= 0) dst[(size_t)rk * row_chunks + c] = v;
      }
    }
  }
}

}  // namespace

size_t dispatch_workspace_bytes(int N, int E, int K) {
  const size_t B = (size_t)(N + kRankBlockTokens - 1) / kRankBlockTokens;
  return 2 * align_up(B * E * sizeof(int32_t), 256) +
         align_up((size_t)N * K * sizeof(int32_t), 256);
}

DispatchWorkspace dispatch_workspace(void* base, int N, int E, int K) {
  const size_t B = (size_t)(N + kRankBlockTokens - 1) / kRankBlockTokens;
  char* p = static_cast<char*>(base);
  DispatchWorkspace ws;
  ws.block_counts = reinterpret_cast<int32_t*>(p);
  p += align_up(B * E * sizeof(int32_t), 256);
  ws.block_excl = reinterpret_cast<int32_t*>(p);
  p += align_up(B * E * sizeof(int32_t), 256);
  ws.local_rank = reinterpret_cast<int32_t*>(p);
  return ws;
}

namespace {

// The scatter launch (threads, held pieces, fused scan and payload chosen
// from the sizes).
hipError_t launch_scatter(const void* x, size_t row_bytes, int N, const int32_t* topk_idx,
                          int E, int K, int W, int64_t capacity, int tpb, bool fused,
                          const int32_t* block_counts, const int32_t* block_excl,
                          const int32_t* local_rank, int32_t* offsets, int32_t* demand,
                          int32_t* counts, int32_t* rank_offsets, void* x_perm, float* x_scale,
                          int32_t* perm_token, int32_t* dest, hipStream_t stream) {
  // x_scale != nullptr: fp8 payload of a bf16 row (row_bytes = 2 d)
  const bool fp8 = x_scale != nullptr;
  const int row_chunks = (int)(row_bytes / 16);
  const uint4* xs = static_cast<const uint4*>(x);
  // threads per token: about a quarter of the row's pieces when there are
  // enough tokens to fill the GPU with the fewer waves (dense8's 512-piece
  // rows on 128 threads: cold dispatch 22.7 against 28.5 us on 256), else
  // all 256 (a few tokens of wide rows want every thread)
  const int threads = N < kScatterFewTokens || row_chunks > 2 * kScatterMaxThreads
                          ? kScatterMaxThreads
                          : row_chunks > kScatterMaxThreads ? 128 : 64;
  const int held = row_chunks <= threads ? 1 : row_chunks <= 2 * threads ? 2 : kMaxHeld;
  auto go = [&](auto fused_c, auto fp8_c, auto held_c, auto threads_c) {
    constexpr int kT = decltype(threads_c)::value;
    dispatch_scatter_kernel<decltype(fused_c)::value, decltype(fp8_c)::value,
                            decltype(held_c)::value, kT><<<N, kT, 0, stream>>>(
        xs, row_chunks, N, topk_idx, E, K, W, capacity, tpb, block_counts, block_excl,
        local_rank, offsets, demand, counts, rank_offsets, x_perm, fp8 ? x_scale : nullptr,
        perm_token, dest);
  };
  auto by_threads = [&](auto fused_c, auto fp8_c, auto held_c) {
    if (threads == 64) go(fused_c, fp8_c, held_c, std::integral_constant<int, 64>{});
    else if (threads == 128) go(fused_c, fp8_c, held_c, std::integral_constant<int, 128>{});
    else go(fused_c, fp8_c, held_c, std::integral_constant<int, kScatterMaxThreads>{});
  };
  auto by_held = [&](auto fused_c, auto fp8_c) {
    using I = std::integral_constant<int, 1>;
    using II = std::integral_constant<int, 2>;
    using IV = std::integral_constant<int, kMaxHeld>;
    if (held == 1) by_threads(fused_c, fp8_c, I{});
    else if (held == 2) by_threads(fused_c, fp8_c, II{});
    else by_threads(fused_c, fp8_c, IV{});
  };
  using T = std::true_type;
  using F = std::false_type;
  if (fused) {
    if (fp8) by_held(T{}, T{});
    else by_held(T{}, F{});
  } else {
    if (fp8) by_held(F{}, T{});
    else by_held(F{}, F{});
  }
  return hipGetLastError();
}

}  // namespace

namespace {

// Scan of a per-block count table (rows of tpb tokens) and the scatter: the
// scan kernel when the table is large, else every scatter block scans it;
// scanned: the table's scan is already in block_excl and the outputs.
hipError_t scan_and_scatter(const void* x, size_t row_bytes, int N, const int32_t* topk_idx,
                            int E, int K, int W, int64_t capacity, int tpb, bool scanned,
                            const int32_t* block_counts, int32_t* block_excl,
                            const int32_t* local_rank, void* x_perm, float* x_scale,
                            int32_t* perm_token, int32_t* dest, int32_t* demand, int32_t* counts,
                            int32_t* offsets, int32_t* rank_offsets, hipStream_t stream) {
  const int B = (N + tpb - 1) / tpb;
  const bool fused =
      !scanned && (int64_t)B * E <= kFusedScanMaxCounts && E <= kFusedScanMaxExperts;
  if (!fused && !scanned) {
    dispatch_scan_kernel<<<1, kRankScanThreads, 0, stream>>>(
        block_counts, B, E, W, capacity, block_excl, demand, counts, offsets, rank_offsets);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return launch_scatter(x, row_bytes, N, topk_idx, E, K, W, capacity, tpb, fused, block_counts,
                        block_excl, local_rank, offsets, demand, counts, rank_offsets, x_perm,
                        x_scale, perm_token, dest, stream);
}

}  // namespace

hipError_t launch_dispatch(const void* x, size_t row_bytes, int N,
                           const int32_t* topk_idx, int E, int K, int W,
                           int64_t capacity, void* x_perm, float* x_scale,
                           int32_t* perm_token, int32_t* dest,
                           int32_t* demand, int32_t* counts,
                           int32_t* offsets, int32_t* rank_offsets,
                           const DispatchWorkspace& ws, hipStream_t stream) {
  const int B = (N + kRankBlockTokens - 1) / kRankBlockTokens;
  const size_t lds = (size_t)kRankWaves * E * sizeof(unsigned long long);
  dispatch_rank_kernel<<<B, kRankBlockTokens, lds, stream>>>(
      topk_idx, N, E, K, ws.block_counts, ws.local_rank);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return scan_and_scatter(x, row_bytes, N, topk_idx, E, K, W, capacity, kRankBlockTokens,
                          false, ws.block_counts, ws.block_excl, ws.local_rank, x_perm, x_scale,
                          perm_token, dest, demand, counts, offsets, rank_offsets, stream);
}

hipError_t launch_dispatch_planned(const void* x, size_t row_bytes, int N,
                                   const int32_t* topk_idx, int E, int K, int W,
                                   int64_t capacity, const RoutePlan& plan, void* x_perm,
                                   float* x_scale, int32_t* perm_token, int32_t* dest,
                                   int32_t* demand, int32_t* counts, int32_t* offsets,
                                   int32_t* rank_offsets, hipStream_t stream) {
  static_assert(kPlanFusedMaxCounts == kFusedScanMaxCounts &&
                    kPlanFusedMaxExperts == kFusedScanMaxExperts,
                "the plan's scan modes follow the scatter's fused-scan limits");
  const bool scanned = plan_scan_mode(N, E) == PlanScan::kInRoute;
  return scan_and_scatter(x, row_bytes, N, topk_idx, E, K, W, capacity, route_plan_tokens(E),
                          scanned, plan.block_counts, plan.block_excl, plan.local_rank, x_perm, x_scale,
                          perm_token, dest, demand, counts, offsets, rank_offsets, stream);
}

hipError_t launch_rank_scan(const int32_t* idx, int N, int E, int K, int64_t capacity,
                            int32_t* block_counts, int32_t* block_excl,
                            int32_t* local_rank, int32_t* demand, int32_t* counts,
                            int32_t* offsets, int32_t* rank_offsets, hipStream_t stream) {
  const int B = (N + kRankBlockTokens - 1) / kRankBlockTokens;
  const size_t lds = (size_t)kRankWaves * E * sizeof(unsigned long long);
  dispatch_rank_kernel<<<B, kRankBlockTokens, lds, stream>>>(idx, N, E, K, block_counts,
                                                             local_rank);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  dispatch_scan_kernel<<<1, kRankScanThreads, 0, stream>>>(block_counts, B, E, 1, capacity,
                                                       block_excl, demand, counts, offsets,
                                                       rank_offsets);
  return hipGetLastError();
}

}  // namespace moe
