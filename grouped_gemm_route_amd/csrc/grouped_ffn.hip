// Ragged grouped-GEMM SwiGLU expert FFN.
//
// "MoE 专家并行的 All-to-All 通信瓶颈", flowchart step "Grouped GEMM 专家计算"
// and section "容量因子、专家复制与 dropless 的取舍": each expert multiplies
// its own, variable number of token rows, all experts in one call, with no
// padding of the token count.  Per expert e on rows R = x_perm[offsets[e] :
// offsets[e+1]]:  h = silu(R Wg[e]^T) * (R Wu[e]^T);  y = h Wd[e]^T.
//
// Weights in their row-major layout ([E, ffn, d] gate and up, [E, d, ffn]
// down).  Tiles are scheduled as in ffn_tiles.h; grouped_ffn_packed.hip
// holds the variant for weights packed in MFMA operand order.
//
// bf16 GEMM (gfx950 MFMA v_mfma_f32_32x32x16_bf16, fp32 accumulate).  Both
// operands are contiguous along the reduction dimension (x_perm and h rows;
// weight rows), so every MFMA operand is one 16-byte LDS read.  The weight
// is the MFMA "A" operand (32 output features) and the activations the "B"
// operand (32 tokens): each lane's accumulator then holds runs of 4
// consecutive features of one token, which the epilogue stores as 8 bytes.
//   block tile: BM tokens x 256 weight rows x 64 reduction elements, BM =
//     256 / 128 / 32 chosen from the mean rows per expert; the gate/up pass
//     loads 128 gate rows and the same 128 up rows, so a wave holds matching
//     gate and up accumulators and applies SwiGLU in registers; the down
//     pass loads 256 rows of Wd.
//   4 waves; at BM = 256 each wave owns 128 tokens x 128 weight rows
//     (16 accumulators of 32 x 32, 256 AGPRs).
//   LDS: two activation stages and a ring of three 32 KB weight slots (160
//     KB at BM = 256), filled by direct-to-LDS buffer loads; 16-byte chunks
//     XOR-swizzled by (row / 2) & 7, which keeps the 16 lanes of an LDS read
//     phase on 16 different bank groups.  Tiles of at most 64 rows (32 at
//     BM = 32) use four-deep rings for both operands instead.
//   pipeline: the next tiles' loads and the next step's operand reads are
//     interleaved one by one with the MFMAs (scheduling fences keep the
//     order); one fence-free barrier per reduction tile.
// fp32 path: a plain LDS-tiled FMA kernel (64 x 64 tiles), used for fp32
// layers, which are small.
#include "ffn_tiles.h"

#include <mutex>
#include <type_traits>

namespace moe {
namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------------------
// bf16 MFMA GEMM
// ---------------------------------------------------------------------------

constexpr int kBW = 256;            // weight rows per block tile

// Geometry of a block tile of BM token rows x 256 weight rows, NW waves laid
// out WM (along tokens) x NW/WM (along weight rows).
template <int BM, int WM, int NW>
struct TileGeo {
  static constexpr int kWaves = NW;
  static constexpr int kWN = NW / WM;
  static constexpr int kTM = BM / WM / 32;   // 32-token MFMA tiles per wave
  static constexpr int kTW = kBW / kWN / 32; // 32-row weight MFMA tiles per wave
  // LDS: two activation stages, then a ring of three weight slots
  static constexpr int kAStageBytes = BM * kRowBytes;
  static constexpr int kWSlotBytes = kBW * kRowBytes;
  static constexpr int kWRegion = 2 * kAStageBytes;
  // one wave-wide direct-to-LDS load moves 64 lanes x 16 bytes = 8 LDS rows;
  // the NW waves together fill 8 NW rows per round
  static constexpr int kWLoads = kBW / (8 * NW);
  static constexpr int kALoads = BM / (8 * NW);
  static constexpr size_t kMainLds = (size_t)kWRegion + 3 * (size_t)kWSlotBytes;
  // Thin tiles (at most kThinRows token rows: an expert's ragged last tile,
  // or every tile of a decode-sized layer) do few MFMAs per reduction tile
  // and would wait on load latency, so they use rings four deep for both
  // operands, loaded three reduction tiles ahead: kThinRows-row activation
  // slots, then four weight slots (160 KB with 64-row slots, 144 KB with
  // 32).  A thin activation slot is kThinALoads loads per wave.
  static constexpr int kThinRows = BM >= 128 ? 64 : 32;
  static constexpr bool kThin = NW == 4 && kThinRows <= BM / WM;
  static constexpr int kThinALoads = kThinRows / (8 * NW);
  static constexpr int kThinABytes = kThinRows * kRowBytes;
  static constexpr int kThinWRegion = 4 * kThinABytes;
  static constexpr size_t kThinLds = (size_t)kThinWRegion + 4 * (size_t)kWSlotBytes;
  static constexpr size_t kLds = kThin && kThinLds > kMainLds ? kThinLds : kMainLds;
  static_assert(kALoads >= 1 && kTM >= 1 && kTW >= 2, "tile shape");
};

template <int BM, int WM, int NW, bool kDual>
__global__ __launch_bounds__(NW * kWave, 1) void ffn_gemm_bf16_kernel(
    const bf16* __restrict__ act, int Kdim, const bf16* __restrict__ w0,
    const bf16* __restrict__ w1, int Nout, bf16* __restrict__ out,
    const int4* __restrict__ tiles, const int* __restrict__ tile_start,
    const int* __restrict__ deal_rank, const int* __restrict__ xcd_start, int E, int n_tiles,
    int cps, float* __restrict__ partial, int* __restrict__ split_cnt) {
  using G = TileGeo<BM, WM, NW>;
  extern __shared__ __attribute__((aligned(16))) bf16 lds[];
  // One block per CU walks its XCD's range: block slot b = blockIdx.x + k
  // gridDim.x (gridDim.x is 8 x the blocks resident per XCD).
  for (int vb = blockIdx.x;; vb += gridDim.x) {
    Unit unit;
    if (!map_unit(vb, tile_start, deal_rank, xcd_start, E, n_tiles, Kdim / kBK, cps, &unit))
      break;
    // the previous unit's waves are done with LDS
    __syncthreads();
    const int slot = unit.slot;
    const int n_tile = unit.n_tile;
    const int kofs = unit.kb * kBK;  // first reduction element of this unit
    const int4 tile = tiles[slot];
    const int e = tile.x;
    const int row0 = tile.y;
    const int rows = tile.z - tile.y;
    constexpr int kNOut = kDual ? kBW / 2 : kBW;  // output columns per block
    const int n0 = n_tile * kNOut;

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);

    // Global -> LDS.  Loads go straight into LDS (buffer_load ... lds): a
    // wave-wide load writes its 64 lanes' 16-byte pieces to 1 KB of
    // consecutive LDS, i.e. 8 rows of 128 bytes.  Lane l fills slot l % 8 of
    // row r = (its group's first row) + l / 8, and since slot s of row r must
    // hold the chunk that swz_chunk maps to s (an involution), the lane
    // fetches global chunk swz_chunk(r, l % 8).
    // Sources are buffer descriptors (one per weight matrix of this expert,
    // one for this tile's token rows); a load past a descriptor's size
    // returns zeros, so edge rows (weight rows >= Nout, token rows >= rows)
    // need no clamping and their results are never stored.  Per-lane byte
    // offsets stay fixed; the reduction position rides in the scalar offset.
    const size_t wexp = (size_t)e * Nout * Kdim;
    const uint32_t wbytes = (uint32_t)((size_t)Nout * Kdim * sizeof(bf16));
    const __amdgpu_buffer_rsrc_t wr0 =
        __builtin_amdgcn_make_buffer_rsrc((void*)(w0 + wexp), 0, wbytes, kBufferFlags);
    const __amdgpu_buffer_rsrc_t wr1 = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((kDual ? w1 : w0) + wexp), 0, wbytes, kBufferFlags);
    const __amdgpu_buffer_rsrc_t ar = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(act + (size_t)row0 * Kdim), 0,
        (uint32_t)((size_t)rows * Kdim * sizeof(bf16)), kBufferFlags);
    const int grow = lane >> 3;                   // row within the wave's 8
    int w_src[G::kWLoads];
#pragma unroll
    for (int i = 0; i < G::kWLoads; ++i) {
      const int lr = (i * NW + wave) * 8 + grow;
      const int n = kDual ? n0 + (lr & (kBW / 2 - 1)) : n0 + lr;
      w_src[i] = (n * Kdim + swz_chunk(lr, lane & 7) * 8) * (int)sizeof(bf16);
    }
    int a_src[G::kALoads];
#pragma unroll
    for (int i = 0; i < G::kALoads; ++i) {
      const int lr = (i * NW + wave) * 8 + grow;
      a_src[i] = (lr * Kdim + swz_chunk(lr, lane & 7) * 8) * (int)sizeof(bf16);
    }
    char* const lds_bytes = reinterpret_cast<char*>(lds);
    // (offsets go through locals and each descriptor has its own call: an
    // array element or a conditional expression of descriptor type as a
    // builtin argument here drops the kernel's host-side stub)
    // (LDS destinations and operand sources are byte offsets of a ring slot)
    auto issue_wload = [&](int woff, int k0, int i) __attribute__((always_inline)) {
      const int voff = w_src[i];
      const int soff = (kofs + k0) * (int)sizeof(bf16);
      lds_void_t* dst = (lds_void_t*)(lds_bytes + woff + (i * NW + wave) * 8 * kRowBytes);
      if (kDual && i >= G::kWLoads / 2)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wr1, dst, 16, voff, soff, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wr0, dst, 16, voff, soff, 0, 0);
    };
    auto issue_aload = [&](int aoff, int k0, int i) __attribute__((always_inline)) {
      const int voff = a_src[i];
      const int soff = (kofs + k0) * (int)sizeof(bf16);
      lds_void_t* dst = (lds_void_t*)(lds_bytes + aoff + (i * NW + wave) * 8 * kRowBytes);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, dst, 16, voff, soff, 0, 0);
    };

    // Wave tiling.  In the gate/up pass the first half of a wave's weight
    // tiles are gate rows and the second half the up rows of the same output
    // features, so SwiGLU pairs accumulator i with i + kTW / 2.
    const int wm = wave % WM;
    const int wn = wave / WM;
    int wrow[G::kTW];
#pragma unroll
    for (int i = 0; i < G::kTW; ++i) {
      if (kDual) {
        constexpr int kHalf = G::kTW / 2;
        wrow[i] = (i / kHalf) * (kBW / 2) + wn * (kBW / 2 / G::kWN) + (i % kHalf) * 32;
      } else {
        wrow[i] = wn * (kBW / G::kWN) + i * 32;
      }
    }
    const int arow0 = wm * (BM / WM);
    // this wave's 32-token subtiles that hold at least one of the tile's rows
    const int jlim = min(G::kTM, max(0, (rows - arow0 + 31) / 32));
    const int lrow = lane & 31;
    const int lhalf = lane >> 5;

    f32x16 acc[G::kTW][G::kTM];
#pragma unroll
    for (int i = 0; i < G::kTW; ++i)
#pragma unroll
      for (int j = 0; j < G::kTM; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // LDS byte addresses of this lane's MFMA operands.  Operand tiles start
    // at multiples of 32 rows, so the swizzle of row (tile + lane % 32) is
    // that of lane % 32 and one per-lane base per reduction step ks covers
    // every operand tile.
    int wbase[kBK / 16], abase[kBK / 16];
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      const int chunk = ks * 2 + lhalf;
      wbase[ks] = swz(wrow[0] + lrow, chunk) * (int)sizeof(bf16);
      abase[ks] = swz(arow0 + lrow, chunk) * (int)sizeof(bf16);
    }

    // MFMA operands of one 16-wide reduction step, double-buffered in
    // registers: the LDS reads of step ks + 1 are spread between the MFMAs of
    // step ks.
    bf16x8 wf[2][G::kTW], af[2][G::kTM];
    constexpr int kFrags = G::kTW + G::kTM;  // LDS reads per step
    auto read_frag = [&](int aoff, int woff, int ks, int buf, int r) __attribute__((always_inline)) {
      if (r < G::kTW)
        wf[buf][r] = *reinterpret_cast<const bf16x8*>(
            lds_bytes + woff + wbase[ks] + (wrow[r] - wrow[0]) * kRowBytes);
      else
        af[buf][r - G::kTW] = *reinterpret_cast<const bf16x8*>(
            lds_bytes + aoff + abase[ks] + (r - G::kTW) * 32 * kRowBytes);
    };
    // MFMAs of weight tiles [I0, I1) on operand buffer `buf`, for the first
    // JN token subtiles.  If kReads, the operand reads of reduction step ks
    // from the ring slots at byte offsets (aoff, woff) into buffer rbuf are
    // spread evenly between them (reads of subtiles that are skipped are left
    // out), and so are the activation loads [A0, A1) into the slot at aoff_ld
    // and the weight loads [W0, W1) into the slot at woff_ld of later tiles.
    // A scheduling fence after every MFMA slot keeps this exact order: left
    // alone, the compiler sinks each read next to its first use and bunches
    // the loads, leaving the matrix cores idle meanwhile.
    auto mfma_step = [&](auto jn_c, auto i0_c, auto i1_c, auto reads_c, auto a0_c, auto a1_c,
                         auto w0_c, auto w1_c, int buf, int aoff, int woff, int ks, int rbuf,
                         int aoff_ld, int ak0, int woff_ld, int wk0) __attribute__((always_inline)) {
      constexpr int JN = decltype(jn_c)::value;
      constexpr int I0 = decltype(i0_c)::value;
      constexpr int I1 = decltype(i1_c)::value;
      constexpr bool kReads = decltype(reads_c)::value && JN > 0;
      constexpr int A0 = decltype(a0_c)::value, A1 = decltype(a1_c)::value;
      constexpr int W0 = decltype(w0_c)::value, W1 = decltype(w1_c)::value;
      constexpr int n = (I1 - I0) * G::kTM;
#pragma unroll
      for (int m = 0; m < n; ++m) {
#pragma unroll
        for (int l = A0 + (m * (A1 - A0) + n - 1) / n; l < A0 + ((m + 1) * (A1 - A0) + n - 1) / n;
             ++l)
          issue_aload(aoff_ld, ak0, l);
#pragma unroll
        for (int l = W0 + (m * (W1 - W0) + n - 1) / n; l < W0 + ((m + 1) * (W1 - W0) + n - 1) / n;
             ++l)
          issue_wload(woff_ld, wk0, l);
        if (kReads) {
#pragma unroll
          for (int r = (m * kFrags + n - 1) / n; r < ((m + 1) * kFrags + n - 1) / n; ++r)
            if (r < G::kTW + JN) read_frag(aoff, woff, ks, rbuf, r);
        }
        const int i = I0 + m / G::kTM;
        const int j = m % G::kTM;
        if (j < JN)  // 32-token subtiles past the tile's last row are skipped
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[buf][i], af[buf][j],
                                                              acc[i][j], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    using IC0 = std::integral_constant<int, 0>;
    using IC1 = std::integral_constant<int, 1>;
    using ICH = std::integral_constant<int, G::kTW / 2>;
    using ICW = std::integral_constant<int, G::kTW>;
    using AA = std::integral_constant<int, G::kALoads>;
    using WA = std::integral_constant<int, G::kWLoads>;
    using YES = std::true_type;
    using NO = std::false_type;
    auto wslot_off = [](int u) __attribute__((always_inline)) {
      return G::kWRegion + u * G::kWSlotBytes;
    };
    auto fence_free_barrier = []() __attribute__((always_inline)) {
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    };

    // One reduction tile kt: activations on LDS stage S = kt % 2, weights in
    // slot u = kt % 3 of a three-slot ring.  Step 0 loads tile kt + 1's
    // activations into the other stage and step 1 loads tile kt + 2's weights
    // into slot (u + 2) % 3; both targets were last read by tile kt - 1, which
    // every wave finished ahead of the barrier that closed it.  Halfway
    // through the last step this wave waits until only the weight loads of
    // tile kt + 2 may be outstanding (so tile kt + 1 has landed) and meets the
    // others at a barrier, after which every wave's loads of tile kt + 1 are
    // visible; tile kt + 1's first operands are then read between the last
    // MFMAs.  Weights, which come from HBM more often, thus get two tiles'
    // time to arrive.  The barrier has no memory fence: a fence would also
    // wait for the weight loads still in flight.  The body has no branches:
    // past the last tile the loads repeat the last tile (into buffers no one
    // reads again) and the trailing reads go unused.
    static_assert(kBK / 16 == 4, "four reduction steps per tile");
    static_assert(G::kWLoads == 8 || G::kWLoads == 4, "vmcnt immediate");
    const int nk = unit.ke - unit.kb;  // reduction tiles of this unit
    auto tile_step = [&](auto jn_c, auto stage_c, int kt, int u) __attribute__((always_inline)) {
      constexpr int S = decltype(stage_c)::value;
      constexpr int ao = S * G::kAStageBytes, ao1 = (1 - S) * G::kAStageBytes;
      const int ak0 = min(kt + 1, nk - 1) * kBK;
      const int wk0 = min(kt + 2, nk - 1) * kBK;
      const int wo = wslot_off(u);
      const int wo1 = wslot_off(u == 2 ? 0 : u + 1);
      const int wo2 = wslot_off(u == 0 ? 2 : u - 1);
      mfma_step(jn_c, IC0{}, ICW{}, YES{}, IC0{}, AA{}, IC0{}, IC0{}, 0, ao, wo, 1, 1, ao1, ak0, 0, 0);
      mfma_step(jn_c, IC0{}, ICW{}, YES{}, IC0{}, IC0{}, IC0{}, WA{}, 1, ao, wo, 2, 0, 0, 0, wo2, wk0);
      mfma_step(jn_c, IC0{}, ICW{}, YES{}, IC0{}, IC0{}, IC0{}, IC0{}, 0, ao, wo, 3, 1, 0, 0, 0, 0);
      mfma_step(jn_c, IC0{}, ICH{}, NO{}, IC0{}, IC0{}, IC0{}, IC0{}, 1, 0, 0, 0, 0, 0, 0, 0, 0);
      if constexpr (G::kWLoads == 8)
        asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
      else
        asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
      fence_free_barrier();
      mfma_step(jn_c, ICH{}, ICW{}, YES{}, IC0{}, IC0{}, IC0{}, IC0{}, 1, ao1, wo1, 0, 0, 0, 0, 0,
                0);
    };
    using St0 = std::integral_constant<int, 0>;
    using St1 = std::integral_constant<int, 1>;

    // Tiles in pairs (stage 0, stage 1); an odd count starts with one tile
    // on stage 0 and pairs (stage 1, stage 0) after it.  JN is the number of
    // this wave's 32-token subtiles that are multiplied: a ragged last tile of
    // an expert has all-zero subtiles past its last row, and the loop comes in
    // variants that skip them (a run-time test per MFMA would force the
    // accumulators out of registers).
    auto main_loop = [&](auto jn_c) __attribute__((always_inline)) {
      // prologue: weights of tile 0, activations of tile 0, weights of tile
      // 1; wait for the first two
#pragma unroll
      for (int l = 0; l < G::kWLoads; ++l) issue_wload(wslot_off(0), 0, l);
#pragma unroll
      for (int l = 0; l < G::kALoads; ++l) issue_aload(0, 0, l);
#pragma unroll
      for (int l = 0; l < G::kWLoads; ++l) issue_wload(wslot_off(1), min(1, nk - 1) * kBK, l);
      if constexpr (G::kWLoads == 8)
        asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
      else
        asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
      fence_free_barrier();
      constexpr int JN = decltype(jn_c)::value;
#pragma unroll
      for (int r = 0; r < kFrags; ++r)
        if (JN > 0 && r < G::kTW + JN) read_frag(0, wslot_off(0), 0, 0, r);
      int u = 0;  // weight slot of the current tile, kt % 3
      auto next = [](int v) { return v == 2 ? 0 : v + 1; };
      if (nk & 1) {
        tile_step(jn_c, St0{}, 0, u);
        u = next(u);
        for (int kt = 1; kt < nk; kt += 2) {
          tile_step(jn_c, St1{}, kt, u);
          u = next(u);
          tile_step(jn_c, St0{}, kt + 1, u);
          u = next(u);
        }
      } else {
        for (int kt = 0; kt < nk; kt += 2) {
          tile_step(jn_c, St0{}, kt, u);
          u = next(u);
          tile_step(jn_c, St1{}, kt + 1, u);
          u = next(u);
        }
      }
    };

    // Thin tiles: reduction tile kt has both operands in slot u = kt % 4 of
    // four-slot rings.  Steps 0 and 1 load tile kt + 3's activations and
    // weights into slot (u + 3) % 4, last read by tile kt - 1; halfway through
    // the last step the wave waits until only the loads of tiles kt + 2 and
    // kt + 3 may be outstanding, then meets the others at the barrier, as
    // above.
    using TA = std::integral_constant<int, G::kThinALoads>;
    auto thin_wait = []() __attribute__((always_inline)) {
      // the loads of two tiles, 2 x (kThinALoads + 8) per wave, may be in flight
      if constexpr (G::kThinALoads == 2)
        asm volatile("s_waitcnt vmcnt(20)" ::: "memory");
      else
        asm volatile("s_waitcnt vmcnt(18)" ::: "memory");
    };
    auto thin_step = [&](auto jn_c, int kt, int u) __attribute__((always_inline)) {
      const int k3 = min(kt + 3, nk - 1) * kBK;
      const int ao = u * G::kThinABytes, wo = G::kThinWRegion + u * G::kWSlotBytes;
      const int u1 = (u + 1) & 3, u3 = (u + 3) & 3;
      const int ao3 = u3 * G::kThinABytes, wo3 = G::kThinWRegion + u3 * G::kWSlotBytes;
      mfma_step(jn_c, IC0{}, ICW{}, YES{}, IC0{}, TA{}, IC0{}, IC0{}, 0, ao, wo, 1, 1, ao3, k3, 0, 0);
      mfma_step(jn_c, IC0{}, ICW{}, YES{}, IC0{}, IC0{}, IC0{}, WA{}, 1, ao, wo, 2, 0, 0, 0, wo3, k3);
      mfma_step(jn_c, IC0{}, ICW{}, YES{}, IC0{}, IC0{}, IC0{}, IC0{}, 0, ao, wo, 3, 1, 0, 0, 0, 0);
      mfma_step(jn_c, IC0{}, ICH{}, NO{}, IC0{}, IC0{}, IC0{}, IC0{}, 1, 0, 0, 0, 0, 0, 0, 0, 0);
      thin_wait();
      fence_free_barrier();
      mfma_step(jn_c, ICH{}, ICW{}, YES{}, IC0{}, IC0{}, IC0{}, IC0{}, 1, u1 * G::kThinABytes,
                G::kThinWRegion + u1 * G::kWSlotBytes, 0, 0, 0, 0, 0, 0);
    };
    auto thin_loop = [&](auto jn_c) __attribute__((always_inline)) {
      static_assert(G::kWLoads == 8, "vmcnt immediate");
      // prologue: tiles 0, 1 and 2 (activations, then weights); wait for tile 0
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        const int k0 = min(t, nk - 1) * kBK;
#pragma unroll
        for (int l = 0; l < G::kThinALoads; ++l) issue_aload(t * G::kThinABytes, k0, l);
#pragma unroll
        for (int l = 0; l < G::kWLoads; ++l)
          issue_wload(G::kThinWRegion + t * G::kWSlotBytes, k0, l);
      }
      thin_wait();
      fence_free_barrier();
      constexpr int JN = decltype(jn_c)::value;
#pragma unroll
      for (int r = 0; r < kFrags; ++r)
        if (JN > 0 && r < G::kTW + JN) read_frag(0, G::kThinWRegion, 0, 0, r);
      for (int kt = 0; kt < nk; ++kt) thin_step(jn_c, kt, kt & 3);
    };

    constexpr int kTM = G::kTM;
    if constexpr (G::kThin) {
      if (rows <= G::kThinRows) {
        // only the first kThinRows / 32 token subtiles of wave row 0 hold rows
        if (G::kThinRows > 32 && jlim >= 2)
          thin_loop(std::integral_constant<int, (G::kThinRows > 32 ? 2 : 1)>{});
        else if (jlim >= 1)
          thin_loop(IC1{});
        else
          thin_loop(IC0{});
      } else if constexpr (kTM > 1) {
        if (jlim >= kTM || (kTM > 2 && jlim > 2))
          main_loop(std::integral_constant<int, kTM>{});
        else if (kTM > 2 && jlim == 2)
          main_loop(std::integral_constant<int, (kTM > 2 ? 2 : kTM)>{});
        else if (jlim == 1)
          main_loop(IC1{});
        else
          main_loop(IC0{});
      }
    } else {
      if (jlim >= kTM || (kTM > 2 && jlim > 2))
        main_loop(std::integral_constant<int, kTM>{});
      else if (kTM > 2 && jlim == 2)
        main_loop(std::integral_constant<int, (kTM > 2 ? 2 : kTM)>{});
      else if (kTM > 1 && jlim == 1)
        main_loop(std::integral_constant<int, (kTM > 1 ? 1 : kTM)>{});
      else
        main_loop(IC0{});
    }

    // The trailing repeat loads of the reduction loop land before this unit
    // ends: the next unit's loads reuse the same LDS.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // A piece of a split tile.  Its accumulators go to its workspace slot in
    // register order (each store instruction writes one contiguous 1 KB run,
    // lanes side by side, so only whole cache lines travel), with the
    // coherent policy of store_partial; once they are in memory the block
    // counts itself in, so
    // the piece that arrives last sees every piece, adds them in piece order
    // into its accumulators, re-arms the counter for the next launch and goes
    // on to the ordinary epilogue.  No block waits on another.
    if (unit.parts > 1) {
      constexpr int kUnitFloats = NW * G::kTW * G::kTM * kWave * 16;
      constexpr int kUnitBytes = kUnitFloats * (int)sizeof(float);
      const __amdgpu_buffer_rsrc_t pr = __builtin_amdgcn_make_buffer_rsrc(
          partial + (size_t)unit.pslot0 * kUnitFloats, 0, (uint32_t)(unit.parts * kUnitBytes),
          kBufferFlags);
      const int lane_off =
          (wave * (G::kTW * G::kTM * kWave * 16) + lane * 4) * (int)sizeof(float);
      const int mine = unit.piece * kUnitBytes;
#pragma unroll
      for (int i = 0; i < G::kTW; ++i)
#pragma unroll
        for (int j = 0; j < G::kTM; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            f32x4 v;
#pragma unroll
            for (int c = 0; c < 4; ++c) v[c] = acc[i][j][q * 4 + c];
            const int voff =
                lane_off + ((i * G::kTM + j) * 4 + q) * kWave * 4 * (int)sizeof(float);
            store_partial(pr, voff, mine, v);
          }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();  // also: every wave is done reading operand LDS
      int* const flag = reinterpret_cast<int*>(lds);
      if (threadIdx.x == 0) *flag = atomicAdd(&split_cnt[unit.split], 1);
      __syncthreads();
      if (*flag != unit.parts - 1) continue;
      // the partials of one weight operand (all G::kTM token operands) of one
      // piece are loaded together, so a piece costs one memory round trip per
      // weight operand
#pragma unroll
      for (int i = 0; i < G::kTW; ++i) {
        f32x16 sum[G::kTM];
#pragma unroll
        for (int j = 0; j < G::kTM; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) sum[j][r] = 0.0f;
        for (int p = 0; p < unit.parts; ++p) {
          const int soff = p * kUnitBytes;
          f32x4 v[G::kTM][4];
#pragma unroll
          for (int j = 0; j < G::kTM; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int voff =
                  lane_off + ((i * G::kTM + j) * 4 + q) * kWave * 4 * (int)sizeof(float);
              v[j][q] = load_partial(pr, voff, soff);
            }
#pragma unroll
          for (int j = 0; j < G::kTM; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
              for (int c = 0; c < 4; ++c) sum[j][q * 4 + c] += v[j][q][c];
        }
#pragma unroll
        for (int j = 0; j < G::kTM; ++j) acc[i][j] = sum[j];
      }
      if (threadIdx.x == 0) split_cnt[unit.split] = 0;
    }

    // Epilogue.  Accumulator register r of lane l holds weight row
    // (r / 4) * 8 + (l / 32) * 4 + r % 4 of its 32-row weight tile and token
    // l % 32 of its 32-row token tile: runs of 4 consecutive output features,
    // one per row for 32 rows.  As in the packed-weight kernel, each wave
    // stages its tile (its kTM x 32 rows by its output features, contiguous:
    // wrow[0] onwards), rounded to bf16 after SwiGLU in the gate/up pass, in
    // its own LDS region with rows 16 bytes longer than their data, and then
    // stores whole row segments of 16 bytes per lane.  The staging regions
    // cover the operand stages: every wave's loads land and its operand
    // reads end before the barrier.
    {
      constexpr int kHalf = G::kTW / 2;
      constexpr int kWF = (kDual ? kHalf : G::kTW) * 32;  // output features of a wave
      constexpr int kSRow = kWF * (int)sizeof(bf16) + 16;
      constexpr int kRows = G::kTM * 32;
      static_assert((size_t)G::kWaves * kRows * kSRow <= G::kLds, "staging fits the LDS");
      char* const st = lds_bytes + wave * (kRows * kSRow);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
#pragma unroll
      for (int j = 0; j < G::kTM; ++j) {
        char* const srow = st + (j * 32 + lrow) * kSRow;
#pragma unroll
        for (int i = 0; i < (kDual ? kHalf : G::kTW); ++i) {
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            bf16x4 o;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              if (kDual)
                o[q] = (bf16)swiglu(acc[i][j][r4 * 4 + q], acc[i + kHalf][j][r4 * 4 + q]);
              else
                o[q] = (bf16)acc[i][j][r4 * 4 + q];
            }
            const int fl = i * 32 + r4 * 8 + lhalf * 4;
            *reinterpret_cast<bf16x4*>(srow + fl * (int)sizeof(bf16)) = o;
          }
        }
      }
      // this wave's LDS writes are done before its lanes read other lanes' rows
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      constexpr int kLPR = kWF / 8;       // lanes per row (16 bytes each)
      constexpr int kRPI = kWave / kLPR;  // rows per store instruction
      const int fo = n0 + wrow[0] + (lane % kLPR) * 8;  // this lane's first output feature
#pragma unroll 4
      for (int r0 = 0; r0 < kRows; r0 += kRPI) {
        if (arow0 + r0 >= rows) break;
        const int m_local = arow0 + r0 + lane / kLPR;
        if (m_local < rows && fo < Nout) {
          const uint4 v =
              *reinterpret_cast<const uint4*>(st + (r0 + lane / kLPR) * kSRow + (lane % kLPR) * 16);
          *reinterpret_cast<uint4*>(out + (size_t)(row0 + m_local) * Nout + fo) = v;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 FMA GEMM (small layers)
// ---------------------------------------------------------------------------
// Block tile 32 tokens x 32 output features (x 2 for gate and up), the
// reduction in chunks of up to 128 staged in LDS: 256 threads, thread t
// owning token t / 8 and features 4 (t % 8) .. + 4.  Small layers are bound
// by load latency, so a tile is small (more blocks) and the next chunk's
// loads are in flight while the current one is multiplied.  Each operand
// row is loaded as 16-byte pieces (Kdim is a multiple of 8); thread t loads
// row t % 32 of a 32-row operand, pieces t / 32 + 8 i, and writes them
// transposed into LDS ([k][row], conflict-free).  Rows past the tile or the
// output width are clamped to the last valid one and never stored; pieces
// past Kdim are zero.

constexpr int kFM = kF32TileRows;  // 32 tokens
constexpr int kFN = 32;            // output features
constexpr int kFK = 128;           // reduction elements per chunk
constexpr int kFP = kFK / 4 / (kThreads / 32);  // 16-byte pieces per thread and operand

template <bool kDual>
__global__ __launch_bounds__(kThreads) void ffn_gemm_f32_kernel(
    const float* __restrict__ act, int Kdim, const float* __restrict__ w0,
    const float* __restrict__ w1, int Nout, float* __restrict__ out,
    const int4* __restrict__ tiles, const int* __restrict__ tile_start,
    const int* __restrict__ num_tiles, int E, int n_tiles) {
  static_assert(kFM == 32 && kFN == 32 && kFP * 4 * (kThreads / 32) == kFK, "fp32 tile");
  __shared__ float a_s[kFK][kFM];
  __shared__ float w0_s[kFK][kFN];
  __shared__ float w1_s[kDual ? kFK : 1][kFN];
  int slot, n_tile;
  if (!map_block(tile_start, num_tiles, E, n_tiles, &slot, &n_tile)) return;
  const int4 tile = tiles[slot];
  const int e = tile.x;
  const int row0 = tile.y;
  const int rows = tile.z - tile.y;
  const int n0 = n_tile * kFN;
  const int tid = threadIdx.x;
  const int tx = tid % 8;   // features 4 tx ..
  const int ty = tid / 8;   // token ty
  const int lr = tid % 32;  // operand row this thread loads
  const int lp = tid / 32;  // its first 16-byte piece of a chunk
  const size_t wbase = (size_t)e * Nout * Kdim;
  const float* arow = act + (size_t)(row0 + min(lr, rows - 1)) * Kdim;
  const float* w0row = w0 + wbase + (size_t)min(n0 + lr, Nout - 1) * Kdim;
  const float* w1row = kDual ? w1 + wbase + (size_t)min(n0 + lr, Nout - 1) * Kdim : nullptr;

  float4 ra[kFP], rw0[kFP], rw1[kDual ? kFP : 1];
  auto load = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kFP; ++i) {
      const int k = k0 + (lp + 8 * i) * 4;
      const bool in = k < Kdim;
      ra[i] = in ? *reinterpret_cast<const float4*>(arow + k) : float4{0, 0, 0, 0};
      rw0[i] = in ? *reinterpret_cast<const float4*>(w0row + k) : float4{0, 0, 0, 0};
      if (kDual) rw1[i] = in ? *reinterpret_cast<const float4*>(w1row + k) : float4{0, 0, 0, 0};
    }
  };
  float acc0[4] = {}, acc1[4] = {};
  load(0);
  for (int k0 = 0; k0 < Kdim; k0 += kFK) {
    __syncthreads();  // every thread is done with the previous chunk
#pragma unroll
    for (int i = 0; i < kFP; ++i) {
      const int kk = (lp + 8 * i) * 4;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        a_s[kk + c][lr] = ra[i][c];
        w0_s[kk + c][lr] = rw0[i][c];
        if (kDual) w1_s[kk + c][lr] = rw1[i][c];
      }
    }
    __syncthreads();
    if (k0 + kFK < Kdim) load(k0 + kFK);  // in flight during this chunk
    const int kc = min(kFK, Kdim - k0);
    for (int kk = 0; kk < kc; ++kk) {
      const float a = a_s[kk][ty];
      const float4 b0 = *reinterpret_cast<const float4*>(&w0_s[kk][tx * 4]);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc0[j] = fmaf(a, b0[j], acc0[j]);
      if (kDual) {
        const float4 b1 = *reinterpret_cast<const float4*>(&w1_s[kk][tx * 4]);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc1[j] = fmaf(a, b1[j], acc1[j]);
      }
    }
  }
  if (ty >= rows) return;
  float* orow = out + (size_t)(row0 + ty) * Nout;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = n0 + tx * 4 + j;
    if (n >= Nout) continue;
    float v = acc0[j];
    if (kDual) v = v / (1.0f + __expf(-v)) * acc1[j];
    orow[n] = v;
  }
}

template <int BM, int WM, int NW, bool kDual>
hipError_t launch_bf16_gemm(const bf16* act, int Kdim, const bf16* w0,
                            const bf16* w1, int Nout, bf16* out,
                            const FfnWorkspace& ws, int E, int max_tiles,
                            hipStream_t stream) {
  using G = TileGeo<BM, WM, NW>;
  static std::once_flag once;
  static hipError_t attr = hipSuccess;
  std::call_once(once, [] {
    attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&ffn_gemm_bf16_kernel<BM, WM, NW, kDual>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)G::kLds);
  });
  if (attr != hipSuccess) return attr;
  constexpr int kNOut = kDual ? kBW / 2 : kBW;
  const int n_tiles = (Nout + kNOut - 1) / kNOut;
  // one block per CU (the kernel takes a CU's LDS), 8 per XCD row
  const int cps = ffn_resident_blocks() / kXcds > 0 ? ffn_resident_blocks() / kXcds : 1;
  const int grid = cps * kXcds;
  (void)max_tiles;
  const int* xcd_start = ws.xcd_start + (kDual ? 0 : kXcds * (E + 1));
  ffn_gemm_bf16_kernel<BM, WM, NW, kDual><<<grid, NW * kWave, G::kLds, stream>>>(
      act, Kdim, w0, w1, Nout, out, ws.tiles, ws.tile_start, ws.deal_rank, xcd_start, E,
      n_tiles, cps, ws.partial, ws.split_cnt + (kDual ? 0 : kMaxSplitUnits));
  return hipGetLastError();
}

template <int BM, int WM, int NW>
hipError_t launch_bf16_ffn(const void* x_perm, int d, int ffn, int E,
                           const void* w_gate, const void* w_up,
                           const void* w_down, void* h, void* y_perm,
                           const FfnWorkspace& ws, int max_tiles,
                           hipStream_t stream) {
  hipError_t err = launch_bf16_gemm<BM, WM, NW, true>(
      static_cast<const bf16*>(x_perm), d, static_cast<const bf16*>(w_gate),
      static_cast<const bf16*>(w_up), ffn, static_cast<bf16*>(h), ws, E,
      max_tiles, stream);
  if (err != hipSuccess) return err;
  return launch_bf16_gemm<BM, WM, NW, false>(
      static_cast<const bf16*>(h), ffn, static_cast<const bf16*>(w_down),
      nullptr, d, static_cast<bf16*>(y_perm), ws, E, max_tiles, stream);
}

// Row-tile height for the bf16 path, from what the host knows: the mean
// rows per expert if every row bound were used.  Decode-sized layers (a few
// rows per expert) take 32-row tiles, mid-sized 128, large 256.
int bf16_tile_rows(int64_t max_rows, int E) {
  const int64_t used = max_rows < E ? max_rows : E;
  const int64_t mean = used > 0 ? max_rows / used : 0;
  if (mean >= 192) return 256;
  if (mean >= 48) return 128;
  return 32;
}

}  // namespace

int ffn_resident_blocks() {
  constexpr int kMaxDevices = 64;
  static int cache[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return kMaxSplitUnits;
  if (dev < kMaxDevices && cache[dev] > 0) return cache[dev];
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = kMaxSplitUnits;
  cus = cus < kMaxSplitUnits ? cus : kMaxSplitUnits;
  if (dev < kMaxDevices) cache[dev] = cus;
  return cus;
}

size_t grouped_ffn_workspace_bytes(int64_t max_rows, int E, bool bf16_data) {
  // the tile table is sized for the smallest row tile, so it covers every
  // tile choice; split partials hold kMaxSplitUnits fp32 block tiles, of
  // BM x 256 here and of BM x 512 in the packed-weight kernel (one
  // workspace serves both)
  const int tr = bf16_data ? 32 : kF32TileRows;
  const size_t table = ffn_tiles_offset(E) +
                       align_up((size_t)max_tiles_for(max_rows, E, tr) * sizeof(int4), 256);
  if (!bf16_data) return table;
  const size_t mine = (size_t)kMaxSplitUnits * bf16_tile_rows(max_rows, E) * kBW * sizeof(float);
  const size_t packed = packed_ffn_partial_bytes(max_rows, E);
  return table + (mine > packed ? mine : packed);
}

hipError_t launch_grouped_ffn(const void* x_perm, bool bf16_data, int d,
                              int ffn, int E, const int32_t* offsets,
                              int64_t max_rows, const void* w_gate,
                              const void* w_up, const void* w_down, void* h,
                              void* y_perm, void* workspace,
                              hipStream_t stream) {
  if (max_rows == 0) return hipSuccess;
  const int tr = bf16_data ? bf16_tile_rows(max_rows, E) : kF32TileRows;
  const int max_tiles = max_tiles_for(max_rows, E, tr);
  const FfnWorkspace ws = ffn_workspace(workspace, E, max_tiles);
  // column tiles of the bf16 passes (the round-robin tables serve only those)
  const int n_up = (ffn + kBW / 2 - 1) / (kBW / 2);
  const int n_dn = (d + kBW - 1) / kBW;
  ffn_schedule_kernel<<<1, 1024, 0, stream>>>(offsets, E, tr, (int)max_rows, max_tiles,
                                              n_up, n_dn, ws.tiles, ws.tile_start,
                                              ws.num_tiles, ws.split_cnt, ws.xcd_start,
                                              ws.deal_rank);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  if (bf16_data) {
    if (tr == 256)
      return launch_bf16_ffn<256, 2, 4>(x_perm, d, ffn, E, w_gate, w_up, w_down, h,
                                     y_perm, ws, max_tiles, stream);
    if (tr == 128)
      return launch_bf16_ffn<128, 2, 4>(x_perm, d, ffn, E, w_gate, w_up, w_down, h,
                                     y_perm, ws, max_tiles, stream);
    return launch_bf16_ffn<32, 1, 4>(x_perm, d, ffn, E, w_gate, w_up, w_down, h,
                                  y_perm, ws, max_tiles, stream);
  }
  const int f_up = (ffn + kFN - 1) / kFN;
  const int g_up = (int)(((long long)f_up * max_tiles + 7) / 8 * 8);
  ffn_gemm_f32_kernel<true><<<g_up, kThreads, 0, stream>>>(
      static_cast<const float*>(x_perm), d, static_cast<const float*>(w_gate),
      static_cast<const float*>(w_up), ffn, static_cast<float*>(h), ws.tiles,
      ws.tile_start, ws.num_tiles, E, f_up);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int f_dn = (d + kFN - 1) / kFN;
  const int g_dn = (int)(((long long)f_dn * max_tiles + 7) / 8 * 8);
  ffn_gemm_f32_kernel<false><<<g_dn, kThreads, 0, stream>>>(
      static_cast<const float*>(h), ffn, static_cast<const float*>(w_down),
      nullptr, d, static_cast<float*>(y_perm), ws.tiles, ws.tile_start,
      ws.num_tiles, E, f_dn);
  return hipGetLastError();
}

}  // namespace moe
