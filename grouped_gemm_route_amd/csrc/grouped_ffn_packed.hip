// Ragged grouped-GEMM SwiGLU expert FFN on packed weights.
//
// Same operation as grouped_ffn.hip ("MoE 专家并行的 All-to-All 通信瓶颈",
// flowchart step "Grouped GEMM 专家计算": per expert e on its rows R,
// h = silu(R Wg[e]^T) * (R Wu[e]^T), y = h Wd[e]^T), for weights that were
// rearranged once, ahead of time, into the order in which the matrix cores
// consume them.  Expert weights are model parameters: they are packed when
// they are loaded, and every layer call after that streams them with
// contiguous 1 KB loads straight into registers.
//
// Packed layout.  A weight matrix of Nrows output features x Kdim reduction
// elements (bf16, reduction-contiguous rows) becomes panels of 128 rows; a
// panel holds, for each 16-wide reduction step s, four 1 KB fragments (32
// rows each), and fragment i of step s holds, for lane l = 0..63, the 8
// values W[row(i, l % 32)][16 s + 8 (l / 32) .. + 8]: exactly the MFMA
// v_mfma_f32_32x32x16_bf16 "A" operand of 32 rows x 16 reduction elements.
//   byte offset of (expert e, panel p, step s, fragment i, lane l) =
//     (((e * P + p) * S + s) * 4 + i) * 1024 + 16 l,   S = Kdim / 16.
//   gate/up: P = ffn / 64; panel p carries output features 64 p .. 64 p + 63
//     as fragments (gate 0..31, gate 32..63, up 0..31, up 32..63), so one
//     wave holds matching gate and up accumulators and applies SwiGLU in
//     registers.
//   down: P = ceil(d / 128); panel p carries rows 128 p .. 128 p + 127 of Wd
//     (rows past d are zero).
//
// GEMM (fp32 accumulate).  A block is 4 waves laid out along the weight
// rows: the block tile is BM tokens x 4 panels (512 weight rows; 256 output
// features in the gate/up pass), and each wave multiplies all BM tokens by
// its own panel (BM / 32 x 4 accumulators of 32 x 32; 256 AGPRs at BM = 128).
//   weights: each wave loads its panel's fragments global -> registers
//     (4 loads of 1 KB per 16-wide step) into a ring of 8 steps, kDist steps
//     ahead of use.  No weight byte passes through LDS, and every weight
//     byte is loaded once per block.
//   activations: the 4 waves fill a 4-stage LDS ring of BM x 64 tiles with
//     direct-to-LDS buffer loads, two reduction tiles ahead, and every wave
//     reads all BM rows from it (one 16-byte read per 32-token operand).
//     16-byte chunks are XOR-swizzled as in the row-major kernel.
// A half-width unit (a tile of an XCD's partial last round, ffn_tiles.h
// map_unit) covers half the column tile: two waves per panel, two fragments
// each.
// Compared with staging both operands through LDS (grouped_ffn.hip: 256 x
// 256 block tiles, each operand read from LDS by two waves), the LDS traffic
// per 64-wide reduction tile drops from 192 KB to 80 KB at the same MFMA
// work, which lowers the power drawn and lets the clock run higher; the
// texture path carries 80 KB instead of 64 KB.  128-row tiles also waste
// less on an expert's ragged last tile than 256-row tiles.
#include "ffn_tiles.h"

#include <mutex>
#include <type_traits>

namespace moe {
namespace {

constexpr int kPkWaves = 4;
constexpr int kPanelRows = 128;                   // weight rows per panel (one wave)
constexpr int kFragBytes = 1024;                  // 32 rows x 16 reduction elements
constexpr int kStepBytes = 4 * kFragBytes;        // one panel, one 16-wide step
constexpr int kPkCols = kPkWaves * kPanelRows;    // weight rows per block tile

// Output staging (epilogue): each wave's tile of BM rows x its output
// features (64 after SwiGLU, 128 in the down pass) in its own LDS region,
// rows 16 bytes longer than their data so that the 32 rows one register
// group writes fall on different LDS banks.
template <bool kDual>
constexpr int staged_row_bytes() {
  return (kDual ? 64 : kPanelRows) * (int)sizeof(bf16) + 16;
}
// LDS of a block: the activation stages during the main loop, the wave
// staging areas in the epilogue (the same bytes), then the arrival flag of
// split tiles.
template <int BM, bool kDual>
constexpr int packed_flag_offset() {
  return 4 * BM * kRowBytes > kPkWaves * BM * staged_row_bytes<kDual>()
             ? 4 * BM * kRowBytes
             : kPkWaves * BM * staged_row_bytes<kDual>();
}
template <int BM, bool kDual>
constexpr size_t packed_lds_bytes() {
  return (size_t)packed_flag_offset<BM, kDual>() + 256;
}

// One thread per 16-byte piece of the packed matrix, written in order.
__global__ __launch_bounds__(256) void pack_weights_kernel(
    const bf16* __restrict__ w0, const bf16* __restrict__ w1, int Nrows, int Kdim, int P,
    long long pieces, uint4* __restrict__ out) {
  const int S = Kdim / 16;
  for (long long idx = blockIdx.x * 256LL + threadIdx.x; idx < pieces;
       idx += (long long)gridDim.x * 256) {
    const int lane = (int)(idx & 63);
    const int frag = (int)((idx >> 6) & 3);
    long long r = idx >> 8;
    const int s = (int)(r % S);
    r /= S;
    const int p = (int)(r % P);
    const long long e = r / P;
    int row;
    const bf16* src;
    if (w1) {  // gate/up: fragments 0, 1 from w0 and 2, 3 from w1
      row = p * 64 + (frag & 1) * 32 + (lane & 31);
      src = frag < 2 ? w0 : w1;
    } else {
      row = p * kPanelRows + frag * 32 + (lane & 31);
      src = w0;
    }
    uint4 v = make_uint4(0, 0, 0, 0);
    if (row < Nrows)
      v = *reinterpret_cast<const uint4*>(src + ((size_t)e * Nrows + row) * Kdim + s * 16 +
                                          (lane >> 5) * 8);
    out[idx] = v;
  }
}

// Wait until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int BM, bool kDual>
__global__ __launch_bounds__(kPkWaves * kWave, 1) void ffn_gemm_packed_kernel(
    const bf16* __restrict__ act, int Kdim, const bf16* __restrict__ wpk, int Nout, int P,
    bf16* __restrict__ out, const int4* __restrict__ tiles, const int* __restrict__ tile_start,
    const int* __restrict__ deal_rank, const int* __restrict__ xcd_start, int E, int n_tiles,
    int cps, float* __restrict__ partial, int* __restrict__ split_cnt) {
  constexpr int NW = kPkWaves;
  constexpr int kTM = BM / 32;             // 32-token operands per wave (all BM rows)
  constexpr int kTW = 4;                   // 32-row weight operands per wave (one panel)
  constexpr int kRing = 8;                 // weight steps held in registers
  constexpr int kDist = 5;                 // weight loads run this many steps ahead
  constexpr int kStages = 4;               // activation LDS stages
  constexpr int kAStage = BM * kRowBytes;  // one BM x 64 activation tile
  constexpr int kAL = BM / (8 * NW);       // activation loads per wave per tile
  static_assert(kAL == kTM && kTM >= 1 && kTM <= 4, "tile shape");
  static_assert(kDist >= 4 && kDist < kRing, "weight ring");
  extern __shared__ __attribute__((aligned(16))) bf16 lds[];
  // One block per CU walks its XCD's list: block slot b = blockIdx.x + k
  // gridDim.x (gridDim.x is 8 x the blocks resident per XCD), so no block is
  // launched only to find no work.
  Unit unit;
  bool have = map_unit<true>(blockIdx.x, tile_start, deal_rank, xcd_start, E, n_tiles,
                             Kdim / kBK, cps, &unit);
  for (int vb = blockIdx.x; have; vb += gridDim.x) {
    // the previous unit's waves are done with the LDS stages
    __syncthreads();
    const int kofs = unit.kb * kBK;
    const int4 tile = tiles[unit.slot];
    const int e = tile.x;
    const int row0 = tile.y;
    const int rows = tile.z - tile.y;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    // A half-width unit (unit.half >= 0) covers panels 2 half, 2 half + 1 of
    // the column tile, two waves per panel, each wave two of the panel's four
    // fragments: the gate/up pass's matching gate and up fragments (SwiGLU
    // stays in registers), the down pass's 64 consecutive rows.
    const bool nar = unit.half >= 0;
    const int pn = nar ? unit.n_tile * NW + unit.half * 2 + (wave >> 1)
                       : unit.n_tile * NW + wave;  // this wave's panel
    const int nfrag0 = kDual ? (wave & 1) : 2 * (wave & 1);  // half-width: first fragment
    constexpr int kNStride = kDual ? 2 : 1;                  // and the step to the second
    const int S = Kdim / 16;
    const int nk = unit.ke - unit.kb;        // reduction tiles of this unit
    const int nsteps = nk * 4;

    // Buffer descriptors: this expert's packed weights and this tile's token
    // rows; loads past a descriptor's size return zeros.  The panel offset
    // rides in the per-lane offset, which the range check covers (the scalar
    // offset is not checked), so a wave whose panel lies past the expert's
    // last reads zeros; its results are never stored.
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(wpk + (size_t)e * P * S * (kStepBytes / sizeof(bf16))), 0,
        (uint32_t)((size_t)P * S * kStepBytes), kBufferFlags);
    const __amdgpu_buffer_rsrc_t ar = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(act + (size_t)row0 * Kdim), 0, (uint32_t)((size_t)rows * Kdim * sizeof(bf16)),
        kBufferFlags);
    const int w_lane = pn * S * kStepBytes + lane * 16;
    const int w_step0 = unit.kb * 4 * kStepBytes;
    // direct-to-LDS activation loads: as in grouped_ffn.hip, lane l fills
    // slot l % 8 of LDS row (group row + l / 8) with global chunk
    // swz_chunk(row, l % 8)
    const int grow = lane >> 3;
    int a_src[kAL];
#pragma unroll
    for (int l = 0; l < kAL; ++l) {
      const int lr = (l * NW + wave) * 8 + grow;
      a_src[l] = (lr * Kdim + swz_chunk(lr, lane & 7) * 8) * (int)sizeof(bf16);
    }
    char* const lds_bytes = reinterpret_cast<char*>(lds);
    const int lrow = lane & 31;
    const int lhalf = lane >> 5;
    // LDS byte offset of this lane's operand for step ks of 32-token operand
    // 0 (operands start at multiples of 32 rows, which share a swizzle)
    int abase[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) abase[ks] = swz(lrow, ks * 2 + lhalf) * (int)sizeof(bf16);
    const int jlim = min(kTM, (rows + 31) / 32);  // operands holding at least one row

    f32x16 acc[kTW][kTM];
#pragma unroll
    for (int i = 0; i < kTW; ++i)
#pragma unroll
      for (int j = 0; j < kTM; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    bf16x8 wf[kRing][kTW];  // weight fragments, ring of steps
    bf16x8 af[2][kTM];      // activation operands, double-buffered

    // (offsets go through locals: an array element or a conditional
    // expression as a buffer builtin's argument drops the kernel's host stub)
    auto load_w = [&](auto ktw_c, int slot, int i, int q) __attribute__((always_inline)) {
      constexpr int KTW = decltype(ktw_c)::value;
      const int frag = KTW == kTW ? i : nfrag0 + i * kNStride;
      const int voff = w_lane + frag * kFragBytes;
      const int soff = w_step0 + q * kStepBytes;
      wf[slot][i] =
          __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(wr, voff, soff, 0));
    };
    auto load_a = [&](int stage, int kt, int l) __attribute__((always_inline)) {
      const int voff = a_src[l];
      const int soff = (kofs + kt * kBK) * (int)sizeof(bf16);
      lds_void_t* dst =
          (lds_void_t*)(lds_bytes + stage * kAStage + (l * NW + wave) * 8 * kRowBytes);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, dst, 16, voff, soff, 0, 0);
    };
    auto read_a = [&](int buf, int stage, int ks, int j) __attribute__((always_inline)) {
      af[buf][j] = *reinterpret_cast<const bf16x8*>(lds_bytes + stage * kAStage + abase[ks] +
                                                    j * 32 * kRowBytes);
    };
    auto fence_free_barrier = []() __attribute__((always_inline)) {
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    };

    // One 16-wide reduction step ks of reduction tile kt (weights in ring
    // slot SL, activations on stage kt % 4), as kTW x kTM MFMA slots; a
    // scheduling fence after every slot keeps the order below.
    //   - the first slot of weight operand i loads fragment i of step
    //     q + kDist into ring slot (SL + kDist) % 8;
    //   - step 0 loads activation tile kt + 2 into stage (kt + 2) % 4 (last
    //     read by tile kt - 2), load l in the middle slot of weight operand l;
    //   - steps 0..2 read the next step's activation operands, one per 4
    //     slots; step 3 waits halfway (see below), meets the other waves at
    //     the barrier and then reads tile kt + 1's first operands.
    // Halfway through step 3 the wave needs tile kt + 1's activations, loaded
    // during step 0 of tile kt - 1.  Counting the loads issued after them
    // (4 - kAL weight loads later in that step, 12 in its steps 1..3, 4 + kAL
    // in step 0 of tile kt, 8 in its steps 1..2 and 2 before the wait) gives
    // 30 in every tile; the prologue issues more (4 kDist weight loads after
    // tile 1's activations), so vmcnt(30) is sufficient there too.  Weight
    // operands need no explicit wait: the compiler waits for each register's
    // own load.  Past the last tile the loads repeat the last step or tile
    // into ring slots and stages nobody reads again, so the body has no
    // branches.
    // A half-width unit's step has KTW = 2 weight operands: 2 kTM slots,
    // activation load l in slot 2 l + 1 of step 0 (after both weight loads of
    // that step), and 13 + kAL loads between tile kt + 1's activations and
    // the wait (none later in their step, 6 in steps 1..3, 2 + kAL in step 0
    // of tile kt, 4 in its steps 1..2 and 1 before the wait; the prologue
    // issues 2 x 7 weight loads after tile 1's).
    auto step = [&](auto ktw_c, auto jn_c, auto sl_c, auto ks_c, int kt)
                    __attribute__((always_inline)) {
      constexpr int KTW = decltype(ktw_c)::value;
      constexpr int JN = decltype(jn_c)::value;
      constexpr int SL = decltype(sl_c)::value;
      constexpr int KS = decltype(ks_c)::value;
      constexpr int n = KTW * kTM;                   // MFMA slots
      constexpr int kWaitN = KTW == kTW ? 30 : 13 + kAL;
      // half-width units hold half the weight bytes per step in flight: they
      // load 7 steps ahead (the ring's limit) instead of kDist
      constexpr int kD = KTW == kTW ? kDist : kRing - 1;
      constexpr int per_read = n / kTM;              // slots per operand read, steps 0..2
      constexpr int half = n / 2;
      constexpr int per_read3 = half / kTM > 0 ? half / kTM : 1;
      const int q = kt * 4 + KS;
      const int qw = min(q + kD, nsteps - 1);
      const int cur = (kt & (kStages - 1));
      const int nxt = ((kt + 1) & (kStages - 1));
      const int kt_a = min(kt + 2, nk - 1);
#pragma unroll
      for (int m = 0; m < n; ++m) {
        const int i = m / kTM, j = m % kTM;
        if (KS == 3 && m == half) {
          wait_vmcnt<kWaitN>();
          fence_free_barrier();
        }
        if (j == 0) load_w(ktw_c, (SL + kD) % kRing, i, qw);
        if (KTW == kTW) {
          if (KS == 0 && j == kTM / 2 && i < kAL) load_a((kt + 2) & (kStages - 1), kt_a, i);
        } else {
          if (KS == 0 && m % 2 == 1) load_a((kt + 2) & (kStages - 1), kt_a, m / 2);
        }
        if (KS < 3) {
          if (m % per_read == 1 % per_read && m / per_read < JN)
            read_a((KS + 1) & 1, cur, KS + 1, m / per_read);
        } else if (m >= half) {
          const int r = m - half;
          if (r % per_read3 == (per_read3 > 1 ? 1 : 0) && r / per_read3 < JN)
            read_a(0, nxt, 0, r / per_read3);
        }
        if (j < JN)  // 32-token operands past the tile's last row are skipped
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[SL][i], af[KS & 1][j],
                                                              acc[i][j], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    using C0 = std::integral_constant<int, 0>;
    using C1 = std::integral_constant<int, 1>;
    using C2 = std::integral_constant<int, 2>;
    using C3 = std::integral_constant<int, 3>;
    // tile kt uses ring slots (kt % 2) * 4 + ks
    auto tile_fn = [&](auto ktw_c, auto jn_c, auto ph_c, int kt) __attribute__((always_inline)) {
      constexpr int PH = decltype(ph_c)::value;
      step(ktw_c, jn_c, std::integral_constant<int, PH + 0>{}, C0{}, kt);
      step(ktw_c, jn_c, std::integral_constant<int, PH + 1>{}, C1{}, kt);
      step(ktw_c, jn_c, std::integral_constant<int, PH + 2>{}, C2{}, kt);
      step(ktw_c, jn_c, std::integral_constant<int, PH + 3>{}, C3{}, kt);
    };
    using P0 = std::integral_constant<int, 0>;
    using P4 = std::integral_constant<int, 4>;
    // JN: 32-token operands that hold rows (a ragged last tile of an expert
    // multiplies fewer; a run-time test per MFMA would force the accumulators
    // out of registers, so the loop comes in one variant per JN)
    auto main_loop = [&](auto ktw_c, auto jn_c) __attribute__((always_inline)) {
      constexpr int KTW = decltype(ktw_c)::value;
      constexpr int JN = decltype(jn_c)::value;
      constexpr int kD = KTW == kTW ? kDist : kRing - 1;
      // prologue: activation tiles 0 and 1, weight steps 0 .. kD - 1; wait
      // for tile 0 (after it: kAL + KTW kD loads)
#pragma unroll
      for (int l = 0; l < kAL; ++l) load_a(0, 0, l);
#pragma unroll
      for (int l = 0; l < kAL; ++l) load_a(1, min(1, nk - 1), l);
#pragma unroll
      for (int s = 0; s < kD; ++s)
#pragma unroll
        for (int i = 0; i < KTW; ++i) load_w(ktw_c, s, i, min(s, nsteps - 1));
      wait_vmcnt<kAL + KTW * kD>();
      fence_free_barrier();
#pragma unroll
      for (int j = 0; j < kTM; ++j)
        if (j < JN) read_a(0, 0, 0, j);
      if (nk & 1) {
        tile_fn(ktw_c, jn_c, P0{}, 0);
        for (int kt = 1; kt < nk; kt += 2) {
          tile_fn(ktw_c, jn_c, P4{}, kt);
          tile_fn(ktw_c, jn_c, P0{}, kt + 1);
        }
      } else {
        for (int kt = 0; kt < nk; kt += 2) {
          tile_fn(ktw_c, jn_c, P0{}, kt);
          tile_fn(ktw_c, jn_c, P4{}, kt + 1);
        }
      }
      // the trailing repeat loads land before the block can end (and its LDS
      // be handed to another block)
      wait_vmcnt<0>();
    };
    auto run_loop = [&](auto ktw_c) __attribute__((always_inline)) {
      if (jlim >= kTM)
        main_loop(ktw_c, std::integral_constant<int, kTM>{});
      else if (kTM > 2 && jlim == 3)
        main_loop(ktw_c, std::integral_constant<int, (kTM > 2 ? 3 : kTM)>{});
      else if (kTM > 1 && jlim == 2)
        main_loop(ktw_c, std::integral_constant<int, (kTM > 1 ? 2 : kTM)>{});
      else
        main_loop(ktw_c, C1{});
    };
    if (nar)
      run_loop(std::integral_constant<int, 2>{});
    else
      run_loop(std::integral_constant<int, kTW>{});

    // A piece of a split tile (map_unit): its fp32 accumulators go to its
    // workspace slot in register order (each store instruction writes one
    // contiguous 1 KB run, lanes side by side, so only whole cache lines
    // travel; with the coherent policy of
    // store_partial), and once they are in memory the piece counts itself in;
    // the piece that arrives last adds the pieces in piece order, re-arms the
    // counter and stores the tile.  The arrival flag sits past the activation
    // stages and the epilogue's staging areas.
    // The next unit's mapping (a chain of dependent schedule reads) is taken
    // here, so that its latency passes during this unit's epilogue.
    Unit next;
    const bool more = map_unit<true>(vb + (int)gridDim.x, tile_start, deal_rank, xcd_start, E,
                                     n_tiles, Kdim / kBK, cps, &next);
    if (unit.parts > 1) {
      constexpr int kUnitFloats = NW * kTW * kTM * kWave * 16;
      constexpr int kUnitBytes = kUnitFloats * (int)sizeof(float);
      const __amdgpu_buffer_rsrc_t pr = __builtin_amdgcn_make_buffer_rsrc(
          partial + (size_t)unit.pslot0 * kUnitFloats, 0, (uint32_t)(unit.parts * kUnitBytes),
          kBufferFlags);
      const int lane_off =
          (wave * (kTW * kTM * kWave * 16) + lane * 4) * (int)sizeof(float);
      const int mine = unit.piece * kUnitBytes;
#pragma unroll
      for (int i = 0; i < kTW; ++i)
#pragma unroll
        for (int j = 0; j < kTM; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            f32x4 v;
#pragma unroll
            for (int c = 0; c < 4; ++c) v[c] = acc[i][j][q * 4 + c];
            const int voff = lane_off + ((i * kTM + j) * 4 + q) * kWave * 4 * (int)sizeof(float);
            store_partial(pr, voff, mine, v);
          }
      wait_vmcnt<0>();
      __syncthreads();
      int* const flag = reinterpret_cast<int*>(lds_bytes + packed_flag_offset<BM, kDual>());
      if (threadIdx.x == 0) *flag = atomicAdd(&split_cnt[unit.split], 1);
      __syncthreads();
      if (*flag != unit.parts - 1) {
        unit = next;
        have = more;
        continue;
      }
      // the partials of one weight operand (all kTM token operands) of one
      // piece are loaded together, so a piece costs one memory round trip per
      // weight operand
#pragma unroll
      for (int i = 0; i < kTW; ++i) {
        f32x16 sum[kTM];
#pragma unroll
        for (int j = 0; j < kTM; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) sum[j][r] = 0.0f;
        for (int p = 0; p < unit.parts; ++p) {
          const int soff = p * kUnitBytes;
          f32x4 v[kTM][4];
#pragma unroll
          for (int j = 0; j < kTM; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int voff =
                  lane_off + ((i * kTM + j) * 4 + q) * kWave * 4 * (int)sizeof(float);
              v[j][q] = load_partial(pr, voff, soff);
            }
#pragma unroll
          for (int j = 0; j < kTM; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
              for (int c = 0; c < 4; ++c) sum[j][q * 4 + c] += v[j][q][c];
        }
#pragma unroll
        for (int j = 0; j < kTM; ++j) acc[i][j] = sum[j];
      }
      if (threadIdx.x == 0) split_cnt[unit.split] = 0;
    }

    // Epilogue.  Accumulator register r of lane l holds weight row
    // (r / 4) * 8 + (l / 32) * 4 + r % 4 of its 32-row fragment and token
    // l % 32 of its 32-token operand: runs of 4 consecutive output features,
    // one per row for 32 rows.  Stored from the registers, each 8-byte run
    // would be a write of its own (a store instruction then touches 32 rows
    // and takes about 0.2 us); instead each wave stages its tile, rounded to
    // bf16 (after SwiGLU in the gate/up pass), row by row in its own LDS
    // region, and then stores whole row segments: 16 bytes per lane, a row's
    // features side by side.  The staging areas cover activation stages:
    // the barrier lets every wave's last direct-to-LDS loads land first
    // (each wave waits for its own at the end of the main loop), and the next
    // unit's loads start after the block barrier at its top.
    // A half-width unit's wave holds half as many output features (32 after
    // SwiGLU, 64 in the down pass) and stages them in the first half of each
    // of its rows.
    auto epilogue = [&](auto nar_c) __attribute__((always_inline)) {
      constexpr bool kNar = decltype(nar_c)::value;
      constexpr int kWF = (kDual ? 64 : kPanelRows) / (kNar ? 2 : 1);  // output features of a wave
      constexpr int kSRow = staged_row_bytes<kDual>();
      char* const st = lds_bytes + wave * (BM * kSRow);
      __syncthreads();
#pragma unroll
      for (int j = 0; j < kTM; ++j) {
        char* const srow = st + (j * 32 + lrow) * kSRow;
        if (kDual) {
          constexpr int kPairs = kNar ? 1 : 2;  // gate operands; up operand i + kPairs
#pragma unroll
          for (int i = 0; i < kPairs; ++i) {
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
              bf16x4 o;
#pragma unroll
              for (int c = 0; c < 4; ++c) {
                const float g = acc[i][j][r4 * 4 + c];
                const float u = acc[i + kPairs][j][r4 * 4 + c];
                o[c] = (bf16)swiglu(g, u);
              }
              const int fl = i * 32 + r4 * 8 + lhalf * 4;
              *reinterpret_cast<bf16x4*>(srow + fl * (int)sizeof(bf16)) = o;
            }
          }
        } else {
#pragma unroll
          for (int i = 0; i < (kNar ? 2 : kTW); ++i) {
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
              bf16x4 o;
#pragma unroll
              for (int c = 0; c < 4; ++c) o[c] = (bf16)acc[i][j][r4 * 4 + c];
              const int fl = i * 32 + r4 * 8 + lhalf * 4;
              *reinterpret_cast<bf16x4*>(srow + fl * (int)sizeof(bf16)) = o;
            }
          }
        }
      }
      // this wave's LDS writes are done before its lanes read other lanes' rows
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      constexpr int kLPR = kWF / 8;       // lanes per row (16 bytes each)
      constexpr int kRPI = kWave / kLPR;  // rows per store instruction
      const int f0 = kNar ? pn * (kDual ? 64 : kPanelRows) + (wave & 1) * kWF : pn * kWF;
      const int fo = f0 + (lane % kLPR) * 8;  // this lane's first output feature
#pragma unroll 4
      for (int r0 = 0; r0 < BM; r0 += kRPI) {
        if (r0 >= rows) break;
        const int m_local = r0 + lane / kLPR;
        if (m_local < rows && fo < Nout) {
          const uint4 v =
              *reinterpret_cast<const uint4*>(st + m_local * kSRow + (lane % kLPR) * 16);
          *reinterpret_cast<uint4*>(out + (size_t)(row0 + m_local) * Nout + fo) = v;
        }
      }
    };
    if (nar)
      epilogue(std::true_type{});
    else
      epilogue(std::false_type{});
    unit = next;
    have = more;
  }
}

template <int BM, bool kDual>
hipError_t launch_packed_gemm(const bf16* act, int Kdim, const bf16* wpk, int Nout, int P,
                              bf16* out, const FfnWorkspace& ws, int E, int max_tiles,
                              hipStream_t stream) {
  static std::once_flag once;
  static hipError_t attr = hipSuccess;
  std::call_once(once, [] {
    attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&ffn_gemm_packed_kernel<BM, kDual>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)packed_lds_bytes<BM, kDual>());
  });
  if (attr != hipSuccess) return attr;
  const int n_tiles = (P + kPkWaves - 1) / kPkWaves;
  // one block per CU (the kernel takes a CU's registers), 8 per XCD row
  const int cps = ffn_resident_blocks() / kXcds > 0 ? ffn_resident_blocks() / kXcds : 1;
  const int grid = cps * kXcds;
  (void)max_tiles;
  const int* xcd_start = ws.xcd_start + (kDual ? 0 : kXcds * (E + 1));
  ffn_gemm_packed_kernel<BM, kDual><<<grid, kPkWaves * kWave, packed_lds_bytes<BM, kDual>(), stream>>>(
      act, Kdim, wpk, Nout, P, out, ws.tiles, ws.tile_start, ws.deal_rank, xcd_start, E,
      n_tiles, cps, ws.partial, ws.split_cnt + (kDual ? 0 : kMaxSplitUnits));
  return hipGetLastError();
}

template <int BM>
hipError_t launch_packed_ffn(const void* x_perm, int d, int ffn, int E, const void* packed_up,
                             const void* packed_down, void* h, void* y_perm,
                             const FfnWorkspace& ws, int max_tiles, hipStream_t stream) {
  hipError_t err = launch_packed_gemm<BM, true>(
      static_cast<const bf16*>(x_perm), d, static_cast<const bf16*>(packed_up), ffn,
      packed_panels(d, ffn, true), static_cast<bf16*>(h), ws, E, max_tiles, stream);
  if (err != hipSuccess) return err;
  return launch_packed_gemm<BM, false>(
      static_cast<const bf16*>(h), ffn, static_cast<const bf16*>(packed_down), d,
      packed_panels(d, ffn, false), static_cast<bf16*>(y_perm), ws, E, max_tiles, stream);
}

}  // namespace

int packed_panels(int d, int ffn, bool gate_up) {
  return gate_up ? ffn / 64 : (d + kPanelRows - 1) / kPanelRows;
}

size_t packed_ffn_weight_bytes(int E, int d, int ffn, bool gate_up) {
  const int S = (gate_up ? d : ffn) / 16;
  return (size_t)E * packed_panels(d, ffn, gate_up) * S * kStepBytes;
}

int packed_ffn_tile_rows(int64_t max_rows, int E) {
  const int64_t used = max_rows < E ? max_rows : E;
  const int64_t mean = used > 0 ? max_rows / used : 0;
  if (mean >= 96) return 128;
  if (mean >= 40) return 64;
  return 32;
}

size_t packed_ffn_partial_bytes(int64_t max_rows, int E) {
  return (size_t)kMaxSplitUnits * packed_ffn_tile_rows(max_rows, E) * kPkCols * sizeof(float);
}

hipError_t launch_pack_ffn_weights(const void* w_gate, const void* w_up, const void* w_down,
                                   int E, int d, int ffn, void* packed_up, void* packed_down,
                                   hipStream_t stream) {
  const long long up_pieces = (long long)(packed_ffn_weight_bytes(E, d, ffn, true) / 16);
  const long long dn_pieces = (long long)(packed_ffn_weight_bytes(E, d, ffn, false) / 16);
  pack_weights_kernel<<<4096, 256, 0, stream>>>(
      static_cast<const bf16*>(w_gate), static_cast<const bf16*>(w_up), ffn, d,
      packed_panels(d, ffn, true), up_pieces, static_cast<uint4*>(packed_up));
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  pack_weights_kernel<<<4096, 256, 0, stream>>>(
      static_cast<const bf16*>(w_down), nullptr, d, ffn, packed_panels(d, ffn, false),
      dn_pieces, static_cast<uint4*>(packed_down));
  return hipGetLastError();
}

hipError_t launch_grouped_ffn_packed(const void* x_perm, int d, int ffn, int E,
                                     const int32_t* offsets, int64_t max_rows,
                                     const void* packed_up, const void* packed_down, void* h,
                                     void* y_perm, void* workspace, hipStream_t stream) {
  if (max_rows == 0) return hipSuccess;
  const int tr = packed_ffn_tile_rows(max_rows, E);
  const int max_tiles = max_tiles_for(max_rows, E, tr);
  const FfnWorkspace ws = ffn_workspace(workspace, E, max_tiles);
  const int n_up = (packed_panels(d, ffn, true) + kPkWaves - 1) / kPkWaves;
  const int n_dn = (packed_panels(d, ffn, false) + kPkWaves - 1) / kPkWaves;
  ffn_schedule_kernel<<<1, 1024, 0, stream>>>(offsets, E, tr, (int)max_rows, max_tiles, n_up,
                                              n_dn, ws.tiles, ws.tile_start, ws.num_tiles,
                                              ws.split_cnt, ws.xcd_start, ws.deal_rank);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (tr == 128)
    return launch_packed_ffn<128>(x_perm, d, ffn, E, packed_up, packed_down, h, y_perm, ws,
                                  max_tiles, stream);
  if (tr == 64)
    return launch_packed_ffn<64>(x_perm, d, ffn, E, packed_up, packed_down, h, y_perm, ws,
                                 max_tiles, stream);
  return launch_packed_ffn<32>(x_perm, d, ffn, E, packed_up, packed_down, h, y_perm, ws,
                               max_tiles, stream);
}

}  // namespace moe
