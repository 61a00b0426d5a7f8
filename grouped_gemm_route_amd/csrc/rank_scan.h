// Per-expert scan of a per-block count table, run by one block of
// kRankScanThreads threads (device helper of the dispatch's scan kernel and
// of the routing kernel's last block).
//
// "MoE 推理服务工程真相 2026", section 2.3: the dispatch counts the tokens of
// each expert, drops those beyond the capacity and groups the rest expert by
// expert (rank by rank); "MoE Inference Communication", section "MoE 计算核
// 优化", builds the token-to-expert table from a cumsum.  Here the counts
// come per block of tokens: block_counts[b][e] tokens of block b chose
// expert e, and the scan produces, per expert, the exclusive sum over the
// blocks before b (block_excl[b][e], so token t of block b with in-block
// rank r is the (block_excl[b][e] + r)-th token of e), the expert's total
// (demand), the kept count min(demand, capacity), and the exclusive scan of
// the kept counts over experts (offsets; rank_offsets[r] = offsets[r E / W]).
#pragma once

#include "moe_internal.h"
#include "block_scan.h"

namespace moe {

constexpr int kRankScanThreads = 1024;
// Table entries a thread loads before it waits for any of them; a thread's
// share of up to this many stays in registers between the two passes.
constexpr int kRankScanHeld = 32;
// Buffer descriptor word 3 for raw 32-bit accesses.
constexpr int kRankScanBufferFlags = 0x00020000;
// Cache policy of system scope (sc0 | sc1): stores are written through L1
// and L2 to memory and counted in vmcnt until they are there; loads read
// memory, not L1 or L2 lines.
constexpr int kRankScanCoherent = 1 | 16;

struct RankScanShared {
  int part[kRankScanThreads];        // part sums, then their exclusive scans
  int base[kRankScanThreads + 1];    // per expert: parts' scan at its first part
  int kept[kRankScanThreads + 1];
  int wave_sums[kRankScanThreads / kWave];
};

// Scan of block_counts [B][E] (E <= kRankScanThreads) by the calling block
// of kRankScanThreads threads.
//   1. Thread (e, p) = (tid % E, tid / E), p < P = kRankScanThreads / E,
//      sums the counts of expert e over its part p, a contiguous range of
//      blocks (rows read side by side by neighbouring threads), loading them
//      in batches of kRankScanHeld with every load of a batch issued before
//      the first is waited for.
//   2. One block-wide exclusive scan over the part sums taken expert by
//      expert (thread t holds part t % P of expert t / P): at each part it
//      gives the sum of all earlier experts' parts plus this expert's
//      earlier parts; minus its value at the expert's first part, that is
//      the expert's exclusive prefix over parts, and the differences of the
//      first-part values are the experts' totals (demand).
//   3. Each thread writes block_excl over its range from its part's prefix.
//   4. A second block-wide scan over experts of min(demand, capacity) gives
//      offsets and rank_offsets.
// kCoherent: the table was written by other blocks of the running kernel, so
// it is read with the system-scope policy (kRankScanCoherent).
template <bool kCoherent>
__device__ __forceinline__ void scan_rank_table(const int32_t* __restrict__ block_counts, int B,
                                                int E, int W, int64_t capacity,
                                                int32_t* __restrict__ block_excl,
                                                int32_t* __restrict__ demand,
                                                int32_t* __restrict__ counts,
                                                int32_t* __restrict__ offsets,
                                                int32_t* __restrict__ rank_offsets,
                                                RankScanShared& sh) {
  constexpr int kPolicy = kCoherent ? kRankScanCoherent : 0;
  const int tid = threadIdx.x;
  const int P = kRankScanThreads / E;
  const int e = tid % E;
  const int part = tid / E;
  const bool active = part < P;
  const int chunk = (B + P - 1) / P;
  const int b0 = active ? min(B, part * chunk) : B;
  const int n = active ? min(B, b0 + chunk) - b0 : 0;
  // loads past the table read zero (range-checked offset); entries of the
  // next part are masked out by i < n
  const __amdgpu_buffer_rsrc_t tr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)block_counts, 0, (uint32_t)((size_t)B * E * sizeof(int32_t)),
      kRankScanBufferFlags);
  auto load = [&](int i) __attribute__((always_inline)) {
    const int off = ((b0 + i) * E + e) * (int)sizeof(int32_t);
    return __builtin_amdgcn_raw_buffer_load_b32(tr, off, 0, kPolicy);
  };
  int held[kRankScanHeld];
#pragma unroll
  for (int i = 0; i < kRankScanHeld; ++i) held[i] = (int)load(i);
  int s = 0;
#pragma unroll
  for (int i = 0; i < kRankScanHeld; ++i) {
    held[i] = i < n ? held[i] : 0;
    s += held[i];
  }
  for (int i0 = kRankScanHeld; i0 < n; i0 += kRankScanHeld) {
    int v[kRankScanHeld];
#pragma unroll
    for (int i = 0; i < kRankScanHeld; ++i) v[i] = (int)load(i0 + i);
#pragma unroll
    for (int i = 0; i < kRankScanHeld; ++i) s += i0 + i < n ? v[i] : 0;
  }
  if (active) sh.part[part * E + e] = s;
  __syncthreads();

  // 2. expert-major scan of the part sums
  const int se = tid / P;
  const int sp = tid % P;
  const bool scanned = se < E;
  const int pv = scanned ? sh.part[sp * E + se] : 0;
  int all = 0;
  const int x = block_exclusive_scan(pv, sh.wave_sums, &all);
  if (scanned && sp == 0) sh.base[se] = x;
  if (tid == 0) sh.base[E] = all;
  __syncthreads();
  if (scanned) sh.part[sp * E + se] = x - sh.base[se];
  __syncthreads();

  // 3. block_excl over this thread's range
  if (active) {
    int run = sh.part[part * E + e];
#pragma unroll
    for (int i = 0; i < kRankScanHeld; ++i) {
      if (i < n) block_excl[(size_t)(b0 + i) * E + e] = run;
      run += held[i];
    }
    for (int i0 = kRankScanHeld; i0 < n; i0 += kRankScanHeld) {
      int v[kRankScanHeld];
#pragma unroll
      for (int i = 0; i < kRankScanHeld; ++i) v[i] = (int)load(i0 + i);
#pragma unroll
      for (int i = 0; i < kRankScanHeld; ++i) {
        if (i0 + i < n) {
          block_excl[(size_t)(b0 + i0 + i) * E + e] = run;
          run += v[i];
        }
      }
    }
  }

  // 4. kept counts and their scan over experts (threads 0 .. E - 1)
  int kept = 0;
  if (tid < E) {
    const int tot = sh.base[tid + 1] - sh.base[tid];
    demand[tid] = tot;
    kept = capacity < 0 ? tot : (int)min((int64_t)tot, capacity);
    counts[tid] = kept;
  }
  int total = 0;
  const int excl = block_exclusive_scan(tid < E ? kept : 0, sh.wave_sums, &total);
  if (tid < E) {
    offsets[tid] = excl;
    sh.kept[tid] = excl;
  }
  if (tid == 0) {
    offsets[E] = total;
    sh.kept[E] = total;
  }
  __syncthreads();
  const int per_rank = E / W;
  for (int r = tid; r <= W; r += blockDim.x) rank_offsets[r] = sh.kept[r * per_rank];
}

}  // namespace moe
