// Tile schedule shared by the grouped-FFN GEMM kernels (grouped_ffn.hip:
// weights in their row-major layout; grouped_ffn_packed.hip: weights packed
// in MFMA operand order).
//
// A one-block kernel turns offsets[] (which stays on the device) into row
// tiles (expert, first row, end row) of at most tile_rows rows of one
// expert.  The blocks of a GEMM pass are (row tile, output-column tile)
// pairs; block b runs on XCD b % 8, and every XCD works through a list in
// which each column tile comes with all of its expert's row tiles, so the
// blocks resident on an XCD share one weight tile and a few activation
// tiles through its L2.  How the column tiles are dealt to the XCDs depends
// on how many a pass has (see map_unit):
//   - 8 or more: each expert's column tiles are dealt round-robin over the
//     XCDs, so all XCDs work on an expert at once, walk its row tiles in the
//     same order and share its activation tiles through the MALL (experts of
//     hundreds of row tiles, whose activations do not fit in one XCD's
//     caches, need this), and every XCD gets the same share of every expert;
//   - fewer: an expert's column tiles would land on a few XCDs only, which
//     with skewed routing leaves others idle, so each XCD instead takes one
//     contiguous eighth of the global order (expert by expert, column tile
//     by column tile) and gets the same number of blocks.
// The tiles of an XCD's partial last round are split along the reduction
// when that shortens the round enough.  Both GEMMs launch one block per CU
// that walks its XCD's list.
#pragma once

#include "moe_internal.h"
#include "block_scan.h"

namespace moe {
namespace {

// ---------------------------------------------------------------------------
// tile schedule
// ---------------------------------------------------------------------------

// Split reduction.  A block-tile grid rarely divides evenly among the
// resident block slots (one block per CU): the 576 blocks of an 8-expert
// down projection over 8192 rows with d = 4096 fill 256 CUs twice and then a
// quarter of them.  The tiles of such a last, partial round are split along
// the reduction into up to kMaxSplit pieces, so that the round fills the
// chip; each piece writes its fp32 accumulators to a workspace slot and the
// last piece to finish adds the pieces up in piece order (a fixed order, so
// results do not depend on which piece finishes last) and stores the tile.
constexpr int kMaxSplitUnits = 256;  // split pieces per launch (block slots)
constexpr int kMaxSplit = 8;         // pieces per tile
constexpr int kMinSplitTiles = 8;    // reduction tiles per piece, at least
// A split costs each piece a pass of its fp32 partials through memory, and
// the last piece to finish the sum of all of them: on MI355X at BM = 128 about
// 3 reduction tiles of compute for a piece and up to about 25 for the last of
// 8, so a tile is split only when that takes at least this many reduction
// tiles off the last round.
constexpr int kSplitMinSaved = 48;

// Workspace layout: [num_tiles | pad to 256 B][split counters: 2 x
// kMaxSplitUnits ints][XCD block tables: 2 passes x 8 XCDs x (E+1) ints |
// pad][tile_start[E+1] | pad][deal_rank[E+1] | pad][tiles | pad][split
// partials].
struct FfnWorkspace {
  int* num_tiles;
  int* split_cnt;   // arrival counters of split tiles: gate/up pass, then down
  int* xcd_start;   // [pass][xcd][E+1]: round-robin lists, the XCD's blocks for experts < e
  int* tile_start;  // tiles of expert e are slots [tile_start[e], tile_start[e+1])
  int* deal_rank;   // experts with tiles before expert e
  int4* tiles;      // (expert, first row, end row, 0)
  float* partial;   // kMaxSplitUnits fp32 accumulator tiles (one per block slot)
};

constexpr int kXcds = 8;  // block b runs on XCD b % 8
constexpr size_t kSplitCntBytes = 2 * kMaxSplitUnits * sizeof(int);

inline size_t ffn_xcd_table_bytes(int E) {
  return align_up((size_t)2 * kXcds * (E + 1) * sizeof(int), 256);
}

inline size_t ffn_tiles_offset(int E) {
  return 256 + kSplitCntBytes + ffn_xcd_table_bytes(E) +
         2 * align_up((size_t)(E + 1) * sizeof(int), 256);
}

inline FfnWorkspace ffn_workspace(void* base, int E, int max_tiles) {
  char* p = static_cast<char*>(base);
  FfnWorkspace ws;
  ws.num_tiles = reinterpret_cast<int*>(p);
  ws.split_cnt = reinterpret_cast<int*>(p + 256);
  ws.xcd_start = reinterpret_cast<int*>(p + 256 + kSplitCntBytes);
  ws.tile_start = reinterpret_cast<int*>(p + 256 + kSplitCntBytes + ffn_xcd_table_bytes(E));
  ws.deal_rank = ws.tile_start + align_up((size_t)(E + 1) * sizeof(int), 256) / sizeof(int);
  ws.tiles = reinterpret_cast<int4*>(p + ffn_tiles_offset(E));
  ws.partial = reinterpret_cast<float*>(
      p + ffn_tiles_offset(E) + align_up((size_t)max_tiles * sizeof(int4), 256));
  return ws;
}

// Round-robin dealing: column tiles n of an expert that XCD x runs are
// n = xcd_first_n(rank, x, n_tiles) + 8 k, rank = the expert's deal_rank
// (experts with tiles before it).  The column tiles of the experts that
// have rows are dealt round-robin over the XCDs, each expert continuing
// where the previous one with rows stopped (counting empty experts too
// would tie an expert's XCDs to its id).
__device__ __forceinline__ int xcd_first_n(int rank, int x, int n_tiles) {
  const int start = ((rank % kXcds) * (n_tiles % kXcds)) % kXcds;  // (rank * n_tiles) % 8
  return (x - start + kXcds) % kXcds;
}
__device__ __forceinline__ int xcd_groups(int rank, int x, int n_tiles) {
  const int f = xcd_first_n(rank, x, n_tiles);
  return f < n_tiles ? (n_tiles - f + kXcds - 1) / kXcds : 0;
}

// n_up, n_dn: column tiles of the two passes (a pass with at least 8 gets
// round-robin tables).
__global__ __launch_bounds__(1024) void ffn_schedule_kernel(
    const int32_t* __restrict__ offsets, int E, int tile_rows, int max_rows,
    int max_tiles, int n_up, int n_dn, int4* __restrict__ tiles,
    int* __restrict__ tile_start, int* __restrict__ num_tiles,
    int* __restrict__ split_cnt, int* __restrict__ xcd_start, int* __restrict__ deal_rank) {
  __shared__ int wave_sums[1024 / kWave];
  __shared__ int wave_sums2[1024 / kWave];
  const int e = threadIdx.x;
  if (e < 2 * kMaxSplitUnits) split_cnt[e] = 0;
  int a = 0, b = 0, nt = 0;
  if (e < E) {
    a = min(max(offsets[e], 0), max_rows);
    b = min(max(offsets[e + 1], a), max_rows);
    nt = (b - a + tile_rows - 1) / tile_rows;
  }
  int total = 0;
  const int base = block_exclusive_scan(nt, wave_sums, &total);
  if (e < E) tile_start[e] = min(base, max_tiles);
  if (e == 0) tile_start[E] = min(total, max_tiles);
  for (int i = 0; i < nt; ++i) {
    const int slot = base + i;
    if (slot < max_tiles) {
      const int r0 = a + i * tile_rows;
      tiles[slot] = make_int4(e, r0, min(b, r0 + tile_rows), 0);
    }
  }
  if (e == 0) *num_tiles = min(total, max_tiles);
  // Per round-robin pass and XCD, the exclusive scan over experts of the
  // XCD's blocks: wave w < 16 scans the table of pass w / 8 and XCD w % 8,
  // 64 experts at a time.
  __shared__ int cnt_s[1024];
  __shared__ int rank_s[1024];
  const int cnt = e < E ? min(base + nt, max_tiles) - min(base, max_tiles) : 0;
  cnt_s[e] = cnt;
  int with_rows = 0;
  rank_s[e] = block_exclusive_scan(cnt > 0 ? 1 : 0, wave_sums2, &with_rows);
  if (e < E) deal_rank[e] = rank_s[e];
  if (e == 0) deal_rank[E] = with_rows;
  __syncthreads();
  const int wave = e / kWave, lane = e % kWave;
  const int n_tiles = wave < kXcds ? n_up : n_dn;
  if (wave < 2 * kXcds && n_tiles >= kXcds) {
    const int x = wave % kXcds;
    int* P = xcd_start + wave * (E + 1);
    int run = 0;
    for (int c = 0; c < E; c += kWave) {
      const int ee = c + lane;
      const int v = ee < E ? xcd_groups(rank_s[ee], x, n_tiles) * cnt_s[ee] : 0;
      int incl = v;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const int o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
      }
      if (ee < E) P[ee] = run + incl - v;
      run += __shfl(incl, kWave - 1);
    }
    if (lane == 0) P[E] = run;
  }
}

inline int max_tiles_for(int64_t max_rows, int E, int tile_rows) {
  return (int)((max_rows + tile_rows - 1) / tile_rows +
               (max_rows < E ? max_rows : E));
}

// Block -> (tile slot, output column tile).  The first round_up(total, 8)
// blocks carry work; block b runs on XCD b % 8, so blocks are renumbered to
// give every XCD one contiguous run of the work order.  The work order is
// expert-major, then column tile, then the expert's row tiles, so the blocks
// that an XCD runs together read the same weight tile and the same few row
// tiles from its L2.  Returns false for blocks without work.
__device__ __forceinline__ bool map_block(const int* __restrict__ tile_start,
                                          const int* __restrict__ num_tiles_p,
                                          int E, int n_tiles, int* slot,
                                          int* n_tile) {
  const int total = n_tiles * *num_tiles_p;
  const int per_xcd = (total + 7) / 8;
  const int b = blockIdx.x;
  if (b >= per_xcd * 8) return false;
  const int L = (b % 8) * per_xcd + b / 8;
  if (L >= total) return false;
  int lo = 0, hi = E;  // largest e with n_tiles * tile_start[e] <= L
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (n_tiles * tile_start[mid] <= L) lo = mid; else hi = mid;
  }
  const int first = tile_start[lo];
  const int cnt = tile_start[lo + 1] - first;
  const int r = L - n_tiles * first;
  *n_tile = r / cnt;
  *slot = first + r % cnt;
  return true;
}

// Work unit of a bf16 GEMM block: a tile slot and column tile, and the range
// [kb, ke) of reduction tiles.  For a piece of a split tile, split >= 0
// numbers the tile's arrival counter, the tile is piece `piece` of `parts`
// and its pieces' partials go to workspace slots pslot0 + 0 .. parts - 1.
// half >= 0: a half-width unit, the column tile's half `half` (packed-weight
// kernel only); -1: the whole column tile.
struct Unit {
  int slot, n_tile, kb, ke, split, piece, parts, pslot0, half;
};

// Expert holding global block position L (0 <= L < n_tiles * tile_start[E]):
// the largest e with n_tiles * tile_start[e] <= L (an expert without tiles
// never matches, since the next expert starts at the same position).
__device__ __forceinline__ int expert_at(const int* __restrict__ tile_start, int E, int n_tiles,
                                         int L) {
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (n_tiles * tile_start[mid] <= L) lo = mid; else hi = mid;
  }
  return lo;
}

// First global block position of XCD x's range: x T / 8 (T = all blocks of
// the pass); x = 8 gives T.  The XCDs' block counts differ by at most one;
// a column tile whose row tiles straddle a cut is shared by two XCDs.
__device__ __forceinline__ int xcd_range(const int* __restrict__ tile_start, int E,
                                         int n_tiles, int x) {
  const int T = n_tiles * tile_start[E];
  return (int)((long long)x * T / kXcds);
}

// Block slot b -> work unit.  Block slot b runs on XCD x = b % 8 as that
// XCD's block i = b / 8 (b = blockIdx.x + k gridDim.x, gridDim.x a multiple
// of 8).  With n_tiles >= 8, XCD x's list is, expert by expert, its
// round-robin share of the expert's column tiles (xcd_first_n), each with
// all of the expert's row tiles, and P (the XCD's row of xcd_start) gives
// the list position of each expert's first block; with fewer, its list is
// the range [xcd_range(x), xcd_range(x + 1)) of the global order.
//
// With cps blocks resident per XCD, the first B - R entries of a list of B
// (R = B mod cps, the XCD's partial last round) are whole tiles; each of the
// last R tiles becomes s = min(cps / R, kMaxSplit, nk / kMinSplitTiles)
// pieces of consecutive reduction tiles, which take the XCD's block numbers
// after the whole tiles and so fill its last round, if that saves at least
// kSplitMinSaved reduction tiles of the round (nk - nk / s).  Otherwise, with
// kNarrow and a last round at most half full (2 R <= cps), each of the last R
// tiles becomes two half-width units (each half of its column tile's weight
// rows, the whole reduction: no partial sums), which take the block numbers
// after the whole tiles; else every tile stays whole.
template <bool kNarrow = false>
__device__ __forceinline__ bool map_unit(int b, const int* __restrict__ tile_start,
                                         const int* __restrict__ deal_rank,
                                         const int* __restrict__ xcd_start, int E,
                                         int n_tiles, int nk, int cps, Unit* w) {
  const int x = b % kXcds;
  const int i = b / kXcds;
  const bool rr = n_tiles >= kXcds;
  const int* __restrict__ P = xcd_start + x * (E + 1);
  const int S0 = rr ? 0 : xcd_range(tile_start, E, n_tiles, x);
  const int B = rr ? P[E] : xcd_range(tile_start, E, n_tiles, x + 1) - S0;
  const int R = B % cps;
  int s = R > 0 ? min(min(cps / R, kMaxSplit), nk / kMinSplitTiles) : 1;
  if (s < 2 || nk - nk / s < kSplitMinSaved) s = 1;
  const bool narrow = kNarrow && s == 1 && R > 0 && 2 * R <= cps;
  const int ways = s > 1 ? s : (narrow ? 2 : 1);  // units per tile of the last round
  const int whole = ways > 1 ? B - R : B;
  // (fields are set once, at the end: per-branch stores to a struct through
  // a pointer can end up in scratch memory)
  const bool is_piece = i >= whole;
  const int p = i - whole;
  if (is_piece && (ways == 1 || p >= R * ways)) return false;
  const int t = is_piece ? p / ways : 0;
  const int sub = is_piece ? p % ways : 0;
  const bool kpiece = is_piece && s > 1;  // a piece of a split tile
  const int piece = kpiece ? sub : 0;
  const int parts = kpiece ? s : 1;
  const int half = is_piece && narrow ? sub : -1;
  const int entry = is_piece ? whole + t : i;
  int e = 0, r = 0;
  if (rr) {
    int lo = 0, hi = E;  // P[lo] <= entry < P[hi]: expert lo has blocks here
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (P[mid] <= entry) lo = mid; else hi = mid;
    }
    e = lo;
    r = entry - P[lo];
  } else {
    const int L = S0 + entry;
    e = expert_at(tile_start, E, n_tiles, L);
    r = L - n_tiles * tile_start[e];
  }
  const int first = tile_start[e];
  const int cnt = tile_start[e + 1] - first;
  const int n_tile = rr ? xcd_first_n(deal_rank[e], x, n_tiles) + kXcds * (r / cnt) : r / cnt;
  *w = Unit{first + r % cnt,
            n_tile,
            piece * nk / parts,
            (piece + 1) * nk / parts,
            kpiece ? x * cps + t : -1,
            piece,
            parts,
            x * cps + t * s,
            half};
  return true;
}


// Split-piece partials travel between blocks through memory with
// system-scope cache policy (sc0 | sc1): a piece's stores go through the
// caches to memory and complete (vmcnt) only once there, and the last piece's
// loads bypass L1 and L2.  A piece then waits for its stores and counts
// itself in with the arrival atomic; no device-wide fence is needed, which
// on a multi-XCD GPU writes back (release) or invalidates (acquire) the
// whole L2 of the XCD.
constexpr int kCoherentPolicy = 1 | 16;

__device__ __forceinline__ void store_partial(__amdgpu_buffer_rsrc_t r, int voff, int soff,
                                              f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, voff, soff,
                                         kCoherentPolicy);
}
__device__ __forceinline__ f32x4 load_partial(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(f32x4,
                            __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kCoherentPolicy));
}

// ---------------------------------------------------------------------------
// operand staging helpers
// ---------------------------------------------------------------------------

// Buffer descriptor word 3 for raw (untyped) buffer loads on CDNA.
constexpr int kBufferFlags = 0x00020000;

// SwiGLU of one gate/up pair of fp32 accumulators: silu(g) * u, silu(g) =
// g / (1 + e^-g).  The quotient is taken with the hardware reciprocal
// (v_rcp_f32, within 1 ulp) instead of the correctly rounded division's
// dozen instructions: the bf16 rounding that follows is 2^15 times coarser.
// For g below about -88, e^-g = inf, the reciprocal is 0 and silu(g) = -0,
// as the exact quotient gives.
__device__ __forceinline__ float swiglu(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

constexpr int kBK = 64;             // reduction elements per stage
constexpr int kRowBytes = kBK * (int)sizeof(bf16);  // 128: one LDS row

typedef __attribute__((address_space(3))) void lds_void_t;

// Element offset of 16-byte chunk `chunk` (0..7) of LDS row `row`.  An MFMA
// operand read has 16 lanes in flight per LDS cycle (64 banks x 4 bytes),
// reading 16 consecutive 128-byte rows at one chunk; rows r and r + 1 fall
// in different halves of the 256-byte bank window, so XOR-ing the chunk
// with (row / 2) & 7 puts the 16 lanes on 16 different 16-byte bank groups.
__device__ __forceinline__ int swz_chunk(int row, int chunk) {
  return chunk ^ ((row >> 1) & 7);
}
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kBK + (swz_chunk(row, chunk) << 3);
}

}  // namespace

// Blocks of a bf16 GEMM resident at once on the current device: one per CU
// (the kernels take all of a CU's registers), capped at kMaxSplitUnits.
// Cached per device.
int ffn_resident_blocks();

}  // namespace moe
