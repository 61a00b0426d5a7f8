// Virtual multi-source exchange: the two local permutations on either side
// of the expert-parallel all-to-all, for W source ranks on one GPU.
//
// "MoE 专家并行的 All-to-All 通信瓶颈", section "All-to-All 分发与回收的机制":
// every card packs its tokens by destination card (flowchart step 按目标卡
// 分组打包), the all-to-all moves them, and each card groups what it
// received by expert (各卡按专家分组).  Rank r owns experts
// [r*E/W, (r+1)*E/W) and source rank s owns the tokens
// [floor(s*N/W), floor((s+1)*N/W)).  The layouts:
//   send buffer  [source][expert][token]  (so [source][destination]...)
//   receive      [destination][source][expert][token]  (the all-to-all)
//   regrouped    [destination][expert][source][token]  = the one-source
//                dispatch's expert-contiguous order, because sources own
//                contiguous, ordered token ranges.
// "MoE Inference Communication", Aurora, Theorem 4.2: the traffic matrix
// D[s][r] (pairs sent by s to r) bounds the all-to-all time from below.
//
// The plan is computed from the one-source dispatch (perm_token, offsets,
// dest): the rows of expert e that come from source s are a contiguous run
// of the expert's rows (tokens ascend inside an expert), found by binary
// search.  Kernels:
//   counts  one thread per (source, expert): C[s][e] and the prefix P[s][e]
//           (rows of e from sources before s);
//   scan    one block: D, the per-source send bases, per-(source, expert)
//           send offsets, per-(destination, source) receive bases and the
//           per-(source, expert) offsets inside a receive chunk;
//   maps    one thread per row of the regrouped layout: its receive row and
//           send row; writes the three gather maps;
//   pairs   one thread per (token, slot): send row of each kept pair.
// moving rows: a gather / scatter kernel, one block per row, 16-byte pieces.
#include "moe_internal.h"
#include "block_scan.h"

namespace moe {
namespace {

// largest s with floor(s * N / W) <= t, i.e. the source rank owning token t
__device__ __forceinline__ int shard_of(int t, int N, int W) {
  return (int)((((int64_t)t + 1) * W - 1) / N);
}

// first index i in [lo, hi) with a[i] >= v (hi if none); a ascending
__device__ __forceinline__ int lower_bound(const int32_t* __restrict__ a, int lo, int hi, int v) {
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] < v) lo = mid + 1; else hi = mid;
  }
  return lo;
}

__global__ __launch_bounds__(256) void exchange_counts_kernel(
    const int32_t* __restrict__ perm_token, const int32_t* __restrict__ offsets, int N, int E,
    int W, int32_t* __restrict__ C, int32_t* __restrict__ P) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= W * E) return;
  const int s = i / E, e = i % E;
  const int a = offsets[e], b = offsets[e + 1];
  const int lo_tok = (int)(((int64_t)s * N) / W);
  const int hi_tok = (int)(((int64_t)(s + 1) * N) / W);
  const int p0 = lower_bound(perm_token, a, b, lo_tok);
  const int p1 = lower_bound(perm_token, p0, b, hi_tok);
  C[i] = p1 - p0;
  P[i] = p0 - a;
}

constexpr int kScanThreads = 1024;

// One block.  Layouts (all int32): C, soff, eoff [W][E]; D, roff [W][W];
// send_base, recv_base [W + 1].
__global__ __launch_bounds__(kScanThreads) void exchange_scan_kernel(
    const int32_t* __restrict__ C, int E, int W, int32_t* __restrict__ D,
    int32_t* __restrict__ soff, int32_t* __restrict__ eoff, int32_t* __restrict__ roff,
    int32_t* __restrict__ send_base, int32_t* __restrict__ recv_base) {
  const int tid = threadIdx.x;
  const int per_rank = E / W;
  // per (source, expert): offsets within the source's send rows and within
  // the source's chunk for the expert's rank
  for (int s = tid; s < W; s += kScanThreads) {
    int run = 0;
    for (int e = 0; e < E; ++e) {
      soff[s * E + e] = run;
      run += C[s * E + e];
    }
    for (int r = 0; r < W; ++r) {
      int c = 0;
      for (int e = r * per_rank; e < (r + 1) * per_rank; ++e) {
        eoff[s * E + e] = c;
        c += C[s * E + e];
      }
      D[s * W + r] = c;
    }
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int s = 0; s < W; ++s) {
      send_base[s] = run;
      for (int r = 0; r < W; ++r) run += D[s * W + r];
    }
    send_base[W] = run;
    run = 0;
    for (int r = 0; r < W; ++r) {
      recv_base[r] = run;
      for (int s = 0; s < W; ++s) {
        roff[r * W + s] = run - recv_base[r];
        run += D[s * W + r];
      }
    }
    recv_base[W] = run;
  }
}

__global__ __launch_bounds__(256) void exchange_maps_kernel(
    const int32_t* __restrict__ perm_token, const int32_t* __restrict__ offsets, int N, int E,
    int W, int max_rows, const int32_t* __restrict__ P, const int32_t* __restrict__ soff,
    const int32_t* __restrict__ eoff, const int32_t* __restrict__ roff,
    const int32_t* __restrict__ send_base, const int32_t* __restrict__ recv_base,
    int32_t* __restrict__ send_token, int32_t* __restrict__ a2a_src,
    int32_t* __restrict__ regroup_src) {
  const int p = blockIdx.x * blockDim.x + threadIdx.x;
  const int M = min(offsets[E], max_rows);
  if (p >= M) return;
  // expert of row p: largest e with offsets[e] <= p
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offsets[mid] <= p) lo = mid; else hi = mid;
  }
  const int e = lo;
  const int t = perm_token[p];
  const int s = shard_of(t, N, W);
  const int r = e / (E / W);
  const int jl = p - offsets[e] - P[s * E + e];
  const int q = send_base[s] + soff[s * E + e] + jl;
  const int rr = recv_base[r] + roff[r * W + s] + eoff[s * E + e] + jl;
  send_token[q] = t;
  a2a_src[rr] = q;
  regroup_src[p] = rr;
}

__global__ __launch_bounds__(256) void exchange_pairs_kernel(
    const int32_t* __restrict__ topk_idx, const int32_t* __restrict__ dest,
    const int32_t* __restrict__ offsets, int N, int E, int K, int W,
    const int32_t* __restrict__ P, const int32_t* __restrict__ soff,
    const int32_t* __restrict__ send_base, int32_t* __restrict__ send_row) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= N * K) return;
  const int p = dest[i];
  int q = -1;
  if (p >= 0) {
    const int e = topk_idx[i];
    const int s = shard_of(i / K, N, W);
    q = send_base[s] + soff[s * E + e] + (p - offsets[e] - P[s * E + e]);
  }
  send_row[i] = q;
}

// dst[i] = src[map[i]] (gather) or dst[map[i]] = src[i] (scatter) for the
// first min(*n_rows, max_rows) rows.  One block per row.
template <bool kScatter>
__global__ __launch_bounds__(256) void rows_permute_kernel(
    const uint4* __restrict__ src, uint4* __restrict__ dst, const int32_t* __restrict__ map,
    const int32_t* __restrict__ n_rows, int max_rows, int row_chunks) {
  const int i = blockIdx.x;
  if (i >= min(*n_rows, max_rows)) return;
  const int m = map[i];
  const uint4* s = src + (size_t)(kScatter ? i : m) * row_chunks;
  uint4* d = dst + (size_t)(kScatter ? m : i) * row_chunks;
  for (int c = threadIdx.x; c < row_chunks; c += blockDim.x) d[c] = s[c];
}

}  // namespace

size_t exchange_workspace_bytes(int E, int W) {
  const size_t we = (size_t)W * E, ww = (size_t)W * W;
  return (4 * align_up(we * 4, 256) + align_up(ww * 4, 256) + 2 * align_up((size_t)(W + 1) * 4, 256));
}

hipError_t launch_exchange_plan(const int32_t* topk_idx, const int32_t* dest,
                                const int32_t* perm_token, const int32_t* offsets, int N,
                                int E, int K, int W, int max_rows, int32_t* src_counts,
                                int32_t* traffic, int32_t* send_row, int32_t* send_token,
                                int32_t* a2a_src, int32_t* regroup_src, void* workspace,
                                hipStream_t stream) {
  const size_t we = (size_t)W * E, ww = (size_t)W * W;
  char* p = static_cast<char*>(workspace);
  auto take = [&](size_t bytes) {
    int32_t* q = reinterpret_cast<int32_t*>(p);
    p += align_up(bytes, 256);
    return q;
  };
  int32_t* P = take(we * 4);
  int32_t* soff = take(we * 4);
  int32_t* eoff = take(we * 4);
  take(we * 4);  // reserved
  int32_t* roff = take(ww * 4);
  int32_t* send_base = take((W + 1) * 4);
  int32_t* recv_base = take((W + 1) * 4);
  const int ce = (int)((we + 255) / 256);
  exchange_counts_kernel<<<ce, 256, 0, stream>>>(perm_token, offsets, N, E, W, src_counts, P);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  exchange_scan_kernel<<<1, kScanThreads, 0, stream>>>(src_counts, E, W, traffic, soff, eoff,
                                                       roff, send_base, recv_base);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (max_rows > 0) {
    exchange_maps_kernel<<<(max_rows + 255) / 256, 256, 0, stream>>>(
        perm_token, offsets, N, E, W, max_rows, P, soff, eoff, roff, send_base, recv_base,
        send_token, a2a_src, regroup_src);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  const int pairs = N * K;
  exchange_pairs_kernel<<<(pairs + 255) / 256, 256, 0, stream>>>(
      topk_idx, dest, offsets, N, E, K, W, P, soff, send_base, send_row);
  return hipGetLastError();
}

hipError_t launch_rows_permute(const void* src, void* dst, const int32_t* map,
                               const int32_t* n_rows, int max_rows, int row_bytes, bool scatter,
                               hipStream_t stream) {
  if (max_rows == 0) return hipSuccess;
  const int row_chunks = row_bytes / 16;
  const int threads = row_chunks >= 256 ? 256 : (row_chunks >= 128 ? 128 : 64);
  if (scatter)
    rows_permute_kernel<true><<<max_rows, threads, 0, stream>>>(
        static_cast<const uint4*>(src), static_cast<uint4*>(dst), map, n_rows, max_rows,
        row_chunks);
  else
    rows_permute_kernel<false><<<max_rows, threads, 0, stream>>>(
        static_cast<const uint4*>(src), static_cast<uint4*>(dst), map, n_rows, max_rows,
        row_chunks);
  return hipGetLastError();
}

}  // namespace moe
