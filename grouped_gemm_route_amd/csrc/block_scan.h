// Block-wide exclusive scan of one int per thread (device helper).
#pragma once

#include "moe_internal.h"

namespace moe {

// Exclusive scan of up to kScanThreads values, one per thread, block-wide.
// Returns the exclusive prefix for this thread; *total receives the sum.
__device__ __forceinline__ int block_exclusive_scan(int v, int* wave_sums, int* total) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  int incl = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == kWave - 1) wave_sums[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    const int nw = blockDim.x / kWave;
    int s = lane < nw ? wave_sums[lane] : 0;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int o = __shfl_up(s, off);
      if (lane >= off) s += o;
    }
    if (lane < nw) wave_sums[lane] = s;  // inclusive wave prefix
  }
  __syncthreads();
  const int before = wave > 0 ? wave_sums[wave - 1] : 0;
  *total = wave_sums[blockDim.x / kWave - 1];
  return before + incl - v;
}


}  // namespace moe
