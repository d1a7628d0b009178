// gemm_standard.hip -- Standard (and Split-K) variant of the blockwise-scaled
// FP8 GEMM for gfx950 (scaled_mm_blockwise, Block_FP8 scaling: page "Helion:
// improving vLLM inference with autotuning", sections "Helion Linear Backend"
// / "Scope" and "Kernel Implementation").
//
//   y[m][n] = bf16( sum_kb sa[m][kb] * sw[n/128][kb] * P_kb[m][n] )
//
// Design (MFMA-bound at large M):
//   * A workgroup owns a BM x BN output tile; its waves tile it as
//     (BM/WM) x (BN/WN), each wave WM x WN = (WM/16) x (WN/16) 16x16 tiles.
//   * Per 128-wide K block the fp8 tiles a[BM][128] and w[BN][128] and the
//     activation scales sa[BM][kb] go HBM -> LDS with the buffer form of the
//     direct-to-LDS load (the data never passes through VGPRs).  Two to four
//     LDS stages: the loads of block kb+1 are in flight while the matrix
//     cores work on block kb.
//   * LDS rows are 128 bytes = eight 16-byte chunks; chunk c of row r is
//     stored at c ^ g(r), g(r) = (r & 7) ^ ((r >> 3) & 1).  A fragment read
//     (ds_read_b128; lane l: row l & 15, chunk 2 (l >> 4) [+1]) then puts
//     lanes 0-31 and lanes 32-63 each on 32 distinct 16-byte slots modulo
//     512 bytes, which is what gfx950's LDS needs to serve the read without
//     bank conflicts (measured: 231 B/clk vs 126 B/clk for an XOR with
//     r & 7 alone).  One direct-to-LDS instruction fills 8 rows (1 KiB, lane
//     L at offset 16 L); lane L therefore fetches chunk (L & 7) ^ g(row).
//   * One v_mfma_f32_16x16x128_f8f6f4 per 16x16 tile and K block gives the
//     complete block partial P_kb; it is folded into the fp32 accumulator
//     with one FMA by sa[m][kb] * sw[nb][kb] (a wave's N range lies inside one
//     128-row weight block, so sw is a scalar per wave and K block).  The
//     matrix core computes the tile transposed (weight fragment as its A
//     operand, activation fragment as its B): a lane then holds one row m
//     and four consecutive columns n, so the rescale needs one activation
//     scale per lane and tile row, and the output leaves in 8-byte stores.
//   * Tile order: blocks are remapped so that each XCD (blocks are dealt
//     round-robin to the 8 XCDs) owns a contiguous range of tiles, and tiles
//     are walked in column groups of GROUP_M tile-rows, so the workgroups
//     resident on one XCD share A and W slices in that XCD's L2.
//   * Split-K: grid x split_k; split s covers a contiguous range of K blocks
//     and writes fp32 partials to the workspace [split][M][N]; a separate
//     kernel sums them in split order.  Split tail: when the tiles fill
//     R >= 1 whole rounds of resident workgroups and leave a partial round,
//     the tiles of the whole rounds run unsplit (bf16 out, no workspace)
//     and only the remaining tiles are split, so the last round is filled
//     with split_k times as many, shorter, workgroups; the sum then covers
//     those tiles only.
#include <atomic>
#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"

namespace fp8blk {
namespace {

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ int swz_g(int row) { return (row & 7) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int swz_off(int row, int chunk) { return row * 128 + ((chunk ^ swz_g(row)) << 4); }

struct StdParams {
  GemmArgs g;
  int tiles_m, tiles_n;
  int kb_total, kb_per_split;
  int tiles_dp;  // leading tiles (in walk order) computed unsplit; blocks [0, tiles_dp)
  int tail;      // tiles after them, each split into split_k blocks
  int remap_dp;  // 1: XCD-contiguous remap of the unsplit blocks (count divisible by 8)
  int remap;     // 1: XCD-contiguous remap of the split blocks (count divisible by 8)
};

constexpr int kGroupM = 8;
// Word 3 of a raw buffer resource on gfx9-family parts (32-bit untyped data).
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kXcds = 8;

// Block b of a group of n blocks -> its tile slot, so that XCD x (blocks
// are dealt round-robin to the 8 XCDs) takes slots [x n/8, (x+1) n/8).
__device__ __forceinline__ int xcd_remap(int b, int n) { return (b % kXcds) * (n / kXcds) + b / kXcds; }

// Tile t of the walk -> (tile row, tile column): column groups of kGroupM
// tile-rows, column by column inside a group.
__device__ __forceinline__ void walk_tile(int t, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int group = kGroupM * tiles_n;
  const int first_m = (t / group) * kGroupM;
  const int gm = min(kGroupM, tiles_m - first_m);
  tm = first_m + (t % group) % gm;
  tn = (t % group) / gm;
}

template <int BM, int BN, int WM, int WN>
struct Shape {
  static constexpr int WAVES_M = BM / WM;
  static constexpr int WAVES_N = BN / WN;
  static constexpr int WAVES = WAVES_M * WAVES_N;
  static constexpr int NT = WAVES * 64;
  static constexpr int TM = WM / 16;
  static constexpr int TN = WN / 16;
  static constexpr int A_INSTR = BM / 8 / WAVES;  // 1 KiB direct-to-LDS loads per wave per K block
  static constexpr int B_INSTR = BN / 8 / WAVES;
  static constexpr int SA_INSTR = BM / 64;        // 256-byte activation-scale loads, one per wave
  static constexpr int SW_WAVE = SA_INSTR;        // the wave that loads the weight scales
  static constexpr int S_FLOATS = BM + 64;        // per-stage scale buffer: sa[BM], sw[BN/128] (+pad)
  static constexpr int SW_N = BN >= 128 ? BN / 128 : 1;  // weight-scale blocks a tile spans
  static_assert((BM / 8) % WAVES == 0 && (BN / 8) % WAVES == 0, "row groups must divide over waves");
  static_assert(128 % WN == 0, "a wave's N range must sit inside one 128-row weight block");
  static_assert(SW_WAVE < WAVES, "one scale load per wave at most");
};

template <int I>
using ic = std::integral_constant<int, I>;

// f(ic<0>{}), ..., f(ic<N-1>{}) in order: every stage index is a constant.
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (N > 0) {
    static_for<N - 1>(f);
    f(ic<N - 1>{});
  }
}

// s_waitcnt vmcnt(n) (expcnt and lgkmcnt left unconstrained).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit count");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// NS LDS stages: the direct-to-LDS loads of K blocks kb+1 .. kb+NS-1 are in
// flight while the matrix cores work on block kb.  Two stages suit the
// MFMA-bound tiles; decode-sized problems, where each workgroup does little
// work per K block and the loop would otherwise wait one memory latency per
// block, use three or four.
//
// SM: 0 = blockwise fp32 scales (one VALU rescale per K block), 1 = P2,
// 2 = CH (per-token / per-channel scales, FP8_Dynamic: the K loop is plain
// matrix-core accumulation and the epilogue multiplies by sa[m] * sw[n]).
//
// P2 (power-of-two scales, the UE8M0 mode): every sa and sw is 2^e, so the
// K-block scaling is exact in the matrix core itself:
// v_mfma_scale_f32_16x16x128_f8f6f4 takes an E8M0 exponent per row of its A
// operand (here the weight rows: one exponent for the wave's 128-row weight
// block) and per column of its B operand (here the activation rows: lane
// l & 15 passes sa's exponent for its row; the same for the lane's four
// 32-wide K sub-blocks), multiplies the block product by 2^(ea + eb - 254)
// and accumulates into the fp32 tile directly.  No VALU rescale and no
// product registers.
template <int BM, int BN, int WM, int WN, bool SPLIT, int NS, int SM>
__global__ __launch_bounds__(BM / WM * (BN / WN) * 64) void k_gemm_lds(StdParams p) {
  using S = Shape<BM, BN, WM, WN>;
  constexpr bool P2 = SM == 1;
  constexpr bool CH = SM == 2;
  static_assert(NS >= 2 && NS <= 4, "2 to 4 LDS stages");
  // separate objects per stage, so that the compiler sees that the stage
  // being filled and the stage being read never alias
  __shared__ __attribute__((aligned(1024))) uint8_t lds_a0[BM * 128];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_a1[BM * 128];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_a2[NS > 2 ? BM * 128 : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_a3[NS > 3 ? BM * 128 : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_b0[BN * 128];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_b1[BN * 128];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_b2[NS > 2 ? BN * 128 : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_b3[NS > 3 ? BN * 128 : 16];
  __shared__ __attribute__((aligned(256))) float lds_s0[S::S_FLOATS];
  __shared__ __attribute__((aligned(256))) float lds_s1[S::S_FLOATS];
  __shared__ __attribute__((aligned(256))) float lds_s2[NS > 2 ? S::S_FLOATS : 4];
  __shared__ __attribute__((aligned(256))) float lds_s3[NS > 3 ? S::S_FLOATS : 4];
  auto stage_a = [&](auto st) __attribute__((always_inline)) -> uint8_t* {
    constexpr int i = decltype(st)::value;
    if constexpr (i == 0) return lds_a0;
    else if constexpr (i == 1) return lds_a1;
    else if constexpr (i == 2) return lds_a2;
    else return lds_a3;
  };
  auto stage_b = [&](auto st) __attribute__((always_inline)) -> uint8_t* {
    constexpr int i = decltype(st)::value;
    if constexpr (i == 0) return lds_b0;
    else if constexpr (i == 1) return lds_b1;
    else if constexpr (i == 2) return lds_b2;
    else return lds_b3;
  };
  auto stage_s = [&](auto st) __attribute__((always_inline)) -> float* {
    constexpr int i = decltype(st)::value;
    if constexpr (i == 0) return lds_s0;
    else if constexpr (i == 1) return lds_s1;
    else if constexpr (i == 2) return lds_s2;
    else return lds_s3;
  };
  constexpr int PER = S::A_INSTR + S::B_INSTR + (CH ? 0 : 1);  // direct-to-LDS instructions per wave and stage

  const GemmArgs& g = p.g;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wave_m = wave % S::WAVES_M;
  const int wave_n = wave / S::WAVES_M;

  // ---- tile of this workgroup: blocks [0, tiles_dp) take the leading tiles
  // whole; the others take split (b / tail) of tile tiles_dp + b % tail ----
  const bool whole = SPLIT && (int)blockIdx.x < p.tiles_dp;  // unsplit tile of a split launch
  int t, split;
  if (whole) {
    t = p.remap_dp ? xcd_remap(blockIdx.x, p.tiles_dp) : (int)blockIdx.x;
    split = 0;
  } else {
    const int nb = (int)gridDim.x - p.tiles_dp;
    int b = (int)blockIdx.x - p.tiles_dp;
    if (p.remap) b = xcd_remap(b, nb);
    split = b / p.tail;
    t = p.tiles_dp + (b - split * p.tail);
  }
  int tm, tn;
  walk_tile(t, p.tiles_m, p.tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM;
  const int64_t n0 = (int64_t)tn * BN;
  const int kb0 = whole ? 0 : split * p.kb_per_split;
  const int kb1 = whole ? p.kb_total : min(kb0 + p.kb_per_split, p.kb_total);
  const int64_t mlast = g.M - 1;

  // ---- direct-to-LDS sources: wave-uniform tile bases + 32-bit lane offsets
  // (row pitches are below 2^24, so every offset inside a tile fits) ----
  // instruction i of this wave fills rows 8 * (wave + i * WAVES) .. +7
  const int lrow = lane >> 3;
  const int lch = lane & 7;
  const int rows_valid = (int)min((int64_t)BM, g.M - m0);  // rows past M re-read the last row
  const uint8_t* a_base = g.a + m0 * g.lda;
  const uint8_t* b_base = g.w + n0 * g.ldw;
  uint32_t a_off[S::A_INSTR];
#pragma unroll
  for (int i = 0; i < S::A_INSTR; ++i) {
    const int row = 8 * (wave + i * S::WAVES) + lrow;
    a_off[i] = (uint32_t)min(row, rows_valid - 1) * (uint32_t)g.lda + ((lch ^ swz_g(row)) << 4);
  }
  uint32_t b_off[S::B_INSTR];
#pragma unroll
  for (int i = 0; i < S::B_INSTR; ++i) {
    const int row = 8 * (wave + i * S::WAVES) + lrow;
    b_off[i] = (uint32_t)row * (uint32_t)g.ldw + ((lch ^ swz_g(row)) << 4);
  }
  const float* sa_base = g.sa + m0 * g.sa_row;
  const uint32_t sa_off = (uint32_t)min((wave * 64 + lane) % BM, rows_valid - 1) * (uint32_t)g.sa_row;
  const float* sw_base = g.sw + (n0 >> 7) * g.ldsw;
  const uint32_t sw_off = (uint32_t)min(lane, S::SW_N - 1) * (uint32_t)g.ldsw;
  const int sw_slot = BM + ((wave_n * WN) >> 7);  // this wave's weight scale in the stage buffer
  const bool sa_wave = wave < S::SA_INSTR;
  const float* sc_base = sa_wave ? sa_base : sw_base;
  const uint32_t sc_off = sa_wave ? sa_off : sw_off;
  // bytes from one K block's scales to the next: sa_kb floats for the
  // activation scales (1 row-major; the token pitch when token-contiguous, so
  // that a wave's 64 rows are one contiguous 256-byte run), 1 for the weight's
  const uint32_t sc_kb = sa_wave ? (uint32_t)g.sa_kb * 4u : 4u;
  const int sc_dst = sa_wave ? wave * 64 : BM;

  // Buffer resources over the tile bases (raw, byte-addressed; offsets are
  // below 2^32 as above).  The buffer form of the direct-to-LDS load keeps
  // LDS-read waits exact: the compiler treats the global form as a flat
  // access that may also count on the LDS counter, and then waits for every
  // outstanding LDS read wherever it needs one.
  const __amdgpu_buffer_rsrc_t rs_a = __builtin_amdgcn_make_buffer_rsrc((void*)a_base, (short)0, -1, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rs_b = __builtin_amdgcn_make_buffer_rsrc((void*)b_base, (short)0, -1, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rs_s = __builtin_amdgcn_make_buffer_rsrc((void*)sc_base, (short)0, -1, kRsrcWord3);

  // The PER direct-to-LDS loads of one stage, numbered A tile rows, B tile
  // rows, scales; issue_part issues those numbered [LO, HI).
  auto issue_part = [&](auto lo_c, auto hi_c, uint8_t* la, uint8_t* lb, float* ls, int kb)
                        __attribute__((always_inline)) {
    constexpr int LO = decltype(lo_c)::value, HI = decltype(hi_c)::value;
    const int kbyte = kb * 128;
#pragma unroll
    for (int i = 0; i < S::A_INSTR; ++i)
      if (i >= LO && i < HI)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_a, (lds_void*)(la + (wave + i * S::WAVES) * 1024), 16,
                                                 (int)a_off[i], kbyte, 0, 0);
#pragma unroll
    for (int i = 0; i < S::B_INSTR; ++i)
      if (S::A_INSTR + i >= LO && S::A_INSTR + i < HI)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_b, (lds_void*)(lb + (wave + i * S::WAVES) * 1024), 16,
                                                 (int)b_off[i], kbyte, 0, 0);
    // one 4-byte scale load per wave: waves < SA_INSTR load activation
    // scales, the others the weight scales (the same values, harmless)
    constexpr int IS = S::A_INSTR + S::B_INSTR;
    if constexpr (!CH && IS >= LO && IS < HI)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_s, (lds_void*)(ls + sc_dst), 4, (int)(sc_off * 4u),
                                               (int)((uint32_t)kb * sc_kb), 0, 0);
  };
  auto issue = [&](uint8_t* la, uint8_t* lb, float* ls, int kb) __attribute__((always_inline)) {
    issue_part(ic<0>{}, ic<PER>{}, la, lb, ls, kb);
  };
  // A stage's loads are spread over the first DMA_ROWS tile rows of the
  // block before (DMA_PER per row) rather than issued in one burst: eight
  // waves issuing all of theirs at once after a barrier stall on the
  // vector-memory queue instead of feeding the matrix cores.
  constexpr int DMA_ROWS = S::TM < 4 ? S::TM : 4;
  constexpr int DMA_PER = (PER + DMA_ROWS - 1) / DMA_ROWS;
  auto issue_row = [&](auto row_c, uint8_t* la, uint8_t* lb, float* ls, int kb) __attribute__((always_inline)) {
    constexpr int R = decltype(row_c)::value;
    constexpr int LO = R * DMA_PER, HI = (R + 1) * DMA_PER < PER ? (R + 1) * DMA_PER : PER;
    if constexpr (LO < PER) issue_part(ic<LO>{}, ic<HI>{}, la, lb, ls, kb);
  };

  v4f acc[S::TM][S::TN];
#pragma unroll
  for (int i = 0; i < S::TM; ++i)
#pragma unroll
    for (int j = 0; j < S::TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const int frow = lane & 15;
  const int fch = (lane >> 4) * 2;
  const int orow = (lane >> 4) * 4;

  // Per K block, software-pipelined over the wave's 16-row tile rows i:
  // while the matrix cores compute the TN products of row i, the VALU folds
  // the products of row i-1 into their accumulators (one FMA per element,
  // factor sa[m][kb] * sw[nb][kb]) and the A fragment and activation scales
  // of row i+1 are read from LDS.  The products of two rows are live at a
  // time; the order (the next row's LDS reads, then 1 MFMA : 4 FMA) is
  // requested from the scheduler per step.  The first rows also issue the
  // direct-to-LDS loads that refill the stage the previous block consumed.
  // The pipeline runs across K blocks.  When the stage's loads are all
  // issued before the last row (EARLY: more tile rows than DMA rows), the
  // wave passes the stage barrier before that row, whose A fragment is
  // already in registers, and reads the next block's first A fragment and
  // activation scale during the row's products, and the next block's B
  // fragment j right after its product j of the row (the fragment register
  // is free once the product has been issued); the weight scale follows, and
  // the last row's products are folded while those reads are in flight.
  // Otherwise the barrier and all of the next block's first reads follow
  // the last row's products.
  static_assert(S::TM % 2 == 0, "row pipeline assumes an even number of tile rows");
  const int arow = wave_m * WM + frow;
  const int a_lo = swz_off(arow, fch), a_hi = swz_off(arow, fch + 1);  // + 2048 per tile row
  const int srow = wave_m * WM + frow;                                 // + 16 per tile row
  v8i bf[S::TN];
  v8i af[2];
  float scl;    // activation scale of this lane's row in the tile row read last
  float gq[2];  // factors sa * sw of the tile rows in flight
  v4f P[2][S::TN];
  float swv;
  float ear;  // P2: sa of row frow of the tile row read last (its exponent bits are the E8M0 scale)

  // LDS reads complete in issue order, so the reads are issued in the order
  // of use (pinned by scheduling barriers): the first MFMA waits only for
  // the first A and B fragments, not for the whole burst.
  auto read_bj = [&](int j, const uint8_t* lb) __attribute__((always_inline)) {
    const int r = wave_n * WN + j * 16 + frow;
    bf[j] = make_v8i(*(const u32x4*)(lb + swz_off(r, fch)), *(const u32x4*)(lb + swz_off(r, fch + 1)));
  };
  auto read_b = [&](const uint8_t* lb, const float* ls) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < S::TN; ++j) {
      read_bj(j, lb);
      __builtin_amdgcn_sched_barrier(0);
    }
    swv = ls[sw_slot];
  };
  auto read_first = [&](const uint8_t* la, const uint8_t* lb, const float* ls) __attribute__((always_inline)) {
    af[0] = make_v8i(*(const u32x4*)(la + a_lo), *(const u32x4*)(la + a_hi));
    __builtin_amdgcn_sched_barrier(0);
    read_b(lb, ls);
    if constexpr (P2)
      ear = ls[srow];
    else if constexpr (!CH)
      scl = ls[srow];
  };
  // Before the last tile row of a block: this wave's loads into the next
  // stage have landed (the NS-2 younger stages may still be in flight);
  // after the barrier every wave's have, and the last reads of the stage
  // being consumed (the last row's A fragment and scale, read during the row
  // before) are complete, so nobody reads it any more.
  auto stage_barrier = [&]() __attribute__((always_inline)) {
    wait_vmcnt<(NS - 2) * PER>();
    __syncthreads();
  };
  constexpr bool EARLY = S::TM > DMA_ROWS;

  // The loads due in tile row i (none past the first DMA_ROWS rows).
  auto dma_row = [&](int i, uint8_t* ra, uint8_t* rb, float* rs, int kb_refill) __attribute__((always_inline)) {
    static_for<DMA_ROWS>([&](auto r) __attribute__((always_inline)) {
      if (i == decltype(r)::value) issue_row(r, ra, rb, rs, kb_refill);  // i is a constant once unrolled
    });
  };
  // One K block from the stage (la, ls) whose first fragments are already in
  // registers; over its first rows it fills the stage (ra, rb, rs), which the
  // block before consumed, with block kb_refill, and at its end it reads the
  // first fragments of the next stage (na, nb, ns).
  auto kblock = [&](const uint8_t* la, const float* ls, uint8_t* ra, uint8_t* rb, float* rs,
                    int kb_refill, const uint8_t* na, const uint8_t* nb, const float* ns)
                    __attribute__((always_inline)) {
    if constexpr (P2 || CH) {
      const uint32_t eb = P2 ? __float_as_uint(swv) >> 23 : 0u;  // this wave's 128 columns share sw
#pragma unroll
      for (int i = 0; i < S::TM; ++i) {
        const int cur = i & 1, prv = cur ^ 1;
        const uint32_t eac = __float_as_uint(ear) >> 23;
        dma_row(i, ra, rb, rs, kb_refill);
        if (i + 1 < S::TM) {
          af[prv] = make_v8i(*(const u32x4*)(la + a_lo + (i + 1) * 2048),
                             *(const u32x4*)(la + a_hi + (i + 1) * 2048));
          if constexpr (P2) ear = ls[srow + (i + 1) * 16];
        } else if constexpr (EARLY) {  // the next block's first A fragment (and its scale)
          stage_barrier();
          af[prv] = make_v8i(*(const u32x4*)(na + a_lo), *(const u32x4*)(na + a_hi));
          if constexpr (P2) ear = ns[srow];
        }
        const bool refill_b = EARLY && i + 1 == S::TM;  // the last row reads the next block's B fragments
#pragma unroll
        for (int j = 0; j < S::TN; ++j) {
          if constexpr (P2)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[j], af[cur], acc[i][j], 0, 0, 0,
                                                                         (int)eb, 0, (int)eac);
          else  // unscaled accumulate (zero scale operands select the plain instruction)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[j], af[cur], acc[i][j], 0, 0, 0,
                                                                         0, 0, 0);
          if (refill_b) read_bj(j, nb);
        }
        if (EARLY || i + 1 < S::TM) __builtin_amdgcn_sched_group_barrier(0x100, P2 ? 3 : 2, 0);  // next row's reads first
        if (refill_b) {
#pragma unroll
          for (int j = 0; j < S::TN; ++j) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // product j, then the reads that refill bf[j]
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          }
        } else {
          __builtin_amdgcn_sched_group_barrier(0x008, S::TN, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (EARLY) {
        swv = ns[sw_slot];
      } else {
        stage_barrier();
        read_first(na, nb, ns);
      }
      __builtin_amdgcn_sched_barrier(0);
      return;
    }
    float scn = 0.f;  // activation scale of row i+1 (read during row i)
#pragma unroll
    for (int i = 0; i < S::TM; ++i) {
      const int cur = i & 1, prv = cur ^ 1;
      dma_row(i, ra, rb, rs, kb_refill);
      if (i + 1 < S::TM) {
        af[prv] = make_v8i(*(const u32x4*)(la + a_lo + (i + 1) * 2048),
                           *(const u32x4*)(la + a_hi + (i + 1) * 2048));
        scn = ls[srow + (i + 1) * 16];
      } else if constexpr (EARLY) {  // the next block's first A fragment and activation scale
        stage_barrier();
        af[prv] = make_v8i(*(const u32x4*)(na + a_lo), *(const u32x4*)(na + a_hi));
        scn = ns[srow];
      }
      // The last row of an EARLY block reads each B fragment of the next
      // block as soon as its own product with that fragment has been
      // issued, so that the next block's first products find their operands
      // in registers instead of waiting for eight fragment reads issued
      // after the last product (2-2.4 % on the prefill layers).
      const bool refill_b = EARLY && i + 1 == S::TM;
#pragma unroll
      for (int j = 0; j < S::TN; ++j) {
        P[cur][j] = mfma16x16x128(bf[j], af[cur]);
        if (refill_b) read_bj(j, nb);
        if (i > 0) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            acc[i - 1][j][q] = __builtin_fmaf(P[prv][j][q], gq[prv], acc[i - 1][j][q]);
        }
      }
      if (i > 0) {
        if (EARLY || i + 1 < S::TM) __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);  // next row's LDS reads first
#pragma unroll
        for (int j = 0; j < S::TN; ++j) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
          if (refill_b) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // the reads that refill bf[j]
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // 4 VALU
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      gq[cur] = scl * swv;  // row i's factor, folded during row i+1
      scl = scn;
    }
    if constexpr (EARLY) {
      swv = ns[sw_slot];  // after the last row's factor has used this block's
    } else {
      stage_barrier();
      read_first(na, nb, ns);
    }
    __builtin_amdgcn_sched_barrier(0);
    constexpr int last = S::TM - 1, lc = (S::TM - 1) & 1;
#pragma unroll
    for (int j = 0; j < S::TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        acc[last][j][q] = __builtin_fmaf(P[lc][j][q], gq[lc], acc[last][j][q]);
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- epilogue of one tile row i (rows wave_m WM + 16 i + frow): lane
  // holds row frow and columns orow..orow+3 of each tile (the products are
  // computed as W A^T, so a lane's four values are consecutive in n); fp32
  // split-K partials leave in one 16-byte store per tile ----
  v4f swc[S::TN];  // CH: per-channel weight scales of this lane's columns
  auto load_swc = [&]() __attribute__((always_inline)) {
    if constexpr (CH) {
#pragma unroll
      for (int j = 0; j < S::TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) swc[j][q] = g.sw[n0 + wave_n * WN + j * 16 + orow + q];
    }
  };
  // Rows past M hold exactly the values of row M-1 (their A rows and scales
  // re-read row M-1), so they are stored there again rather than skipped: the
  // same bytes, and no branch in the pipeline.
  //
  // bf16 output leaves in 16-byte stores of 8 consecutive columns: for each
  // pair of tiles (j, j+1) the lanes l and l ^ 16 (same row, column groups
  // 4g and 4g + 4 of both tiles) trade halves, so that the even-group lane
  // holds 8 columns of tile j and the odd-group lane 8 columns of tile j+1,
  // and one store instruction writes 64 contiguous bytes of each of its 16
  // rows (half as many store instructions as 8-byte pieces; 4-5 % faster
  // on the prefill layers).
  auto store_row = [&](auto partial_c, int i) __attribute__((always_inline)) {
    constexpr bool PARTIAL = decltype(partial_c)::value;  // fp32 split-K partials, else bf16
    const int64_t m = min(m0 + wave_m * WM + i * 16 + frow, mlast);
    const float sam = CH ? g.sa[m] : 1.0f;
    auto scaled = [&](int j) __attribute__((always_inline)) {
      v4f v = acc[i][j];
      if constexpr (CH) {
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = v[q] * sam * swc[j][q];
      }
      return v;
    };
    if constexpr (!PARTIAL && S::TN % 2 == 0) {
      const bool odd = (lane >> 4) & 1;
      const int c8 = ((lane >> 5) & 1) * 8;  // this lane pair's 8 columns within a tile
#pragma unroll
      for (int j = 0; j < S::TN; j += 2) {
        const v4f v0 = scaled(j), v1 = scaled(j + 1);
        const uint32_t a0 = bf16x2_bits(v0[0], v0[1]), a1 = bf16x2_bits(v0[2], v0[3]);
        const uint32_t b0 = bf16x2_bits(v1[0], v1[1]), b1 = bf16x2_bits(v1[2], v1[3]);
        // the even lane sends its tile-(j+1) columns, the odd lane its tile-j ones
        const uint32_t r0 = (uint32_t)__shfl_xor((int)(odd ? a0 : b0), 16);
        const uint32_t r1 = (uint32_t)__shfl_xor((int)(odd ? a1 : b1), 16);
        const u32x4 d = odd ? u32x4{r0, r1, b0, b1} : u32x4{a0, a1, r0, r1};
        const int64_t n = n0 + wave_n * WN + (j + (odd ? 1 : 0)) * 16 + c8;
        *(u32x4*)(g.y + m * g.ldy + n) = d;
      }
    } else {
#pragma unroll
      for (int j = 0; j < S::TN; ++j) {
        const int64_t n = n0 + wave_n * WN + j * 16 + orow;
        const v4f v = scaled(j);
        if constexpr (PARTIAL) {
          *(v4f*)(g.ws + ((int64_t)split * g.M + m) * g.N + n) = v;
        } else {
          const uint32_t lo = bf16x2_bits(v[0], v[1]);
          const uint32_t hi = bf16x2_bits(v[2], v[3]);
          *(uint2*)(g.y + m * g.ldy + n) = make_uint2(lo, hi);
        }
      }
    }
  };

  // The last block's bf16 rows through LDS (two stages, 64-column wave
  // tiles): the other stage is free by then (its block passed its stage
  // barrier and nothing refills it), so each wave writes its 16 x 64
  // output values of tile row i into a private 16-row patch of it (rows
  // padded to 144 bytes against bank conflicts) and reads them back as
  // 16 bytes per lane, 8 lanes per row: each store instruction then writes
  // 8 whole 128-byte rows.  LDS instructions of one wave complete in order;
  // the wave barriers keep the compiler from moving the reads above the
  // writes of other lanes, or the next row's writes above these reads.
  constexpr int kOutPitch = 144;
  constexpr int kOutBytes = S::WAVES * 16 * kOutPitch;
  constexpr bool OUT_IN_B = kOutBytes <= BN * 128;  // the free stage's B buffer holds the patches
  constexpr bool LDS_OUT = !SPLIT && NS == 2 && WN == 64 && (OUT_IN_B || kOutBytes <= BM * 128);
  auto store_row_lds = [&](int i, uint8_t* scratch) __attribute__((always_inline)) {
    uint8_t* patch = scratch + wave * (16 * kOutPitch);
    const float sam = CH ? g.sa[min(m0 + wave_m * WM + i * 16 + frow, mlast)] : 1.0f;
#pragma unroll
    for (int j = 0; j < S::TN; ++j) {
      v4f v = acc[i][j];
      if constexpr (CH) {
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = v[q] * sam * swc[j][q];
      }
      *(uint2*)(patch + frow * kOutPitch + (j * 16 + orow) * 2) =
          make_uint2(bf16x2_bits(v[0], v[1]), bf16x2_bits(v[2], v[3]));
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int r = (lane >> 3) + 8 * k;
      const u32x4 d = *(const u32x4*)(patch + r * kOutPitch + (lane & 7) * 16);
      const int64_t m = min(m0 + wave_m * WM + i * 16 + r, mlast);
      *(u32x4*)(g.y + m * g.ldy + n0 + wave_n * WN + (lane & 7) * 8) = d;
    }
    __builtin_amdgcn_wave_barrier();
  };

  // The last K block: the same row pipeline without a refill, a stage
  // barrier or the next block's reads, and each tile row leaves as soon as
  // its accumulators are final (during the next row's products), so the
  // workgroup's output stores overlap its last block instead of following
  // it in one burst.
  auto kblock_last = [&](auto partial_c, const uint8_t* la, const float* ls, uint8_t* scratch) __attribute__((always_inline)) {
    auto out_row = [&](int i) __attribute__((always_inline)) {
      if constexpr (LDS_OUT && !decltype(partial_c)::value)
        store_row_lds(i, scratch);
      else
        store_row(partial_c, i);
    };
    load_swc();
    if constexpr (P2 || CH) {
      const uint32_t eb = P2 ? __float_as_uint(swv) >> 23 : 0u;
#pragma unroll
      for (int i = 0; i < S::TM; ++i) {
        const int cur = i & 1, prv = cur ^ 1;
        const uint32_t eac = __float_as_uint(ear) >> 23;
        if (i + 1 < S::TM) {
          af[prv] = make_v8i(*(const u32x4*)(la + a_lo + (i + 1) * 2048),
                             *(const u32x4*)(la + a_hi + (i + 1) * 2048));
          if constexpr (P2) ear = ls[srow + (i + 1) * 16];
        }
#pragma unroll
        for (int j = 0; j < S::TN; ++j) {
          if constexpr (P2)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[j], af[cur], acc[i][j], 0, 0, 0,
                                                                         (int)eb, 0, (int)eac);
          else
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[j], af[cur], acc[i][j], 0, 0, 0,
                                                                         0, 0, 0);
        }
        if (i + 1 < S::TM) __builtin_amdgcn_sched_group_barrier(0x100, P2 ? 3 : 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, S::TN, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (i > 0) out_row(i - 1);  // its products finished during this row's
        __builtin_amdgcn_sched_barrier(0);
      }
      out_row(S::TM - 1);
      return;
    }
    float scn = 0.f;
#pragma unroll
    for (int i = 0; i < S::TM; ++i) {
      const int cur = i & 1, prv = cur ^ 1;
      if (i + 1 < S::TM) {
        af[prv] = make_v8i(*(const u32x4*)(la + a_lo + (i + 1) * 2048),
                           *(const u32x4*)(la + a_hi + (i + 1) * 2048));
        scn = ls[srow + (i + 1) * 16];
      }
#pragma unroll
      for (int j = 0; j < S::TN; ++j) {
        P[cur][j] = mfma16x16x128(bf[j], af[cur]);
        if (i > 0) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            acc[i - 1][j][q] = __builtin_fmaf(P[prv][j][q], gq[prv], acc[i - 1][j][q]);
        }
      }
      if (i > 0) {
        if (i + 1 < S::TM) __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
        for (int j = 0; j < S::TN; ++j) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      gq[cur] = scl * swv;
      scl = scn;
      if (i > 0) out_row(i - 1);  // folded during this row
      __builtin_amdgcn_sched_barrier(0);
    }
    constexpr int last = S::TM - 1, lc = (S::TM - 1) & 1;
#pragma unroll
    for (int j = 0; j < S::TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        acc[last][j][q] = __builtin_fmaf(P[lc][j][q], gq[lc], acc[last][j][q]);
    out_row(last);
  };


  // Stage s <- block kb0+s for s < NS-1; stage 0 is waited for, the others
  // stay in flight.  The block in stage s is consumed by kblock(s), which
  // meanwhile fills stage s-1 (consumed one block earlier; that block's
  // stage barrier has released it) with the block NS-1 ahead.  NS K
  // blocks per trip so that every LDS buffer is a static object (the
  // compiler then knows the stage being read and the stages being filled
  // never alias and inserts no early wait); no branch inside a trip: block
  // indices are clamped to the last block (re-loading it into an idle stage
  // is harmless).  An empty K range (a trailing split) loads the last block
  // and computes nothing.
  const int kblast = kb1 - 1;
  static_for<NS - 1>([&](auto st) __attribute__((always_inline)) {
    issue(stage_a(st), stage_b(st), stage_s(st), min(kb0 + (int)decltype(st)::value, kblast));
  });
  wait_vmcnt<(NS - 2) * PER>();
  __syncthreads();
  read_first(lds_a0, lds_b0, lds_s0);
  int kb = kb0;
  if constexpr (SPLIT) {
    // Split launches (fp32 partials or bf16 per workgroup): every block
    // refills, and the output leaves after the last one.
    for (; kb + NS - 1 < kb1; kb += NS) {
      static_for<NS>([&](auto st) __attribute__((always_inline)) {
        constexpr int i = decltype(st)::value;
        constexpr int nx = (i + 1) % NS, pv = (i + NS - 1) % NS;
        kblock(stage_a(st), stage_s(st), stage_a(ic<pv>{}), stage_b(ic<pv>{}), stage_s(ic<pv>{}),
               min(kb + i + NS - 1, kblast), stage_a(ic<nx>{}), stage_b(ic<nx>{}), stage_s(ic<nx>{}));
      });
    }
    static_for<NS - 1>([&](auto st) __attribute__((always_inline)) {  // the remaining kb1 - kb < NS blocks
      constexpr int i = decltype(st)::value;
      constexpr int nx = (i + 1) % NS, pv = (i + NS - 1) % NS;
      if (kb + i < kb1)
        kblock(stage_a(st), stage_s(st), stage_a(ic<pv>{}), stage_b(ic<pv>{}), stage_s(ic<pv>{}), kblast,
               stage_a(ic<nx>{}), stage_b(ic<nx>{}), stage_s(ic<nx>{}));
    });
    wait_vmcnt<0>();
    load_swc();
#pragma unroll
    for (int i = 0; i < S::TM; ++i) {
      if (!whole)
        store_row(std::true_type{}, i);
      else
        store_row(std::false_type{}, i);
    }
  } else {
    for (; kb + NS < kb1; kb += NS) {  // whole trips while more than NS blocks remain
      static_for<NS>([&](auto st) __attribute__((always_inline)) {
        constexpr int i = decltype(st)::value;
        constexpr int nx = (i + 1) % NS, pv = (i + NS - 1) % NS;
        kblock(stage_a(st), stage_s(st), stage_a(ic<pv>{}), stage_b(ic<pv>{}), stage_s(ic<pv>{}),
               min(kb + i + NS - 1, kblast), stage_a(ic<nx>{}), stage_b(ic<nx>{}), stage_s(ic<nx>{}));
      });
    }
    // The remaining R = 1 .. NS blocks (stages 0 .. R-1), the last one
    // storing the output as it goes: one straight-line path per R, so that
    // nothing the refills need stays live into the last block.  (Only a
    // split launch can have an empty K range.)
    const int rem = kb1 - kb;
    static_for<NS>([&](auto rc) __attribute__((always_inline)) {
      constexpr int R = decltype(rc)::value + 1;
      if (rem == R) {
        static_for<R>([&](auto st) __attribute__((always_inline)) {
          constexpr int i = decltype(st)::value;
          constexpr int nx = (i + 1) % NS, pv = (i + NS - 1) % NS;
          if constexpr (i + 1 < R)
            kblock(stage_a(st), stage_s(st), stage_a(ic<pv>{}), stage_b(ic<pv>{}), stage_s(ic<pv>{}), kblast,
                   stage_a(ic<nx>{}), stage_b(ic<nx>{}), stage_s(ic<nx>{}));
          else
            kblock_last(std::false_type{}, stage_a(st), stage_s(st),
                        OUT_IN_B ? stage_b(ic<(i + 1) % NS>{}) : stage_a(ic<(i + 1) % NS>{}));
        });
      }
    });
    // Two stages: nothing but stores is outstanding here (the last block's
    // data was waited for before it was read, and the last block refills
    // nothing).  More stages: refills of clamped blocks may still be in
    // flight into LDS, which must land before the workgroup ends.
    if constexpr (NS > 2) wait_vmcnt<0>();
  }

}

// Sum of the split_k fp32 partials of the tail tiles (walk order tiles_dp
// .. tiles_dp + gridDim.x / (BM / 16) - 1) -> bf16, in increasing split
// order like the whole-output sum.  Workgroup: 16 rows of one tile.
template <int BM, int BN>
__global__ __launch_bounds__(256) void k_tail_reduce(const float* __restrict__ ws, int S, int64_t M, int64_t N,
                                                     uint16_t* __restrict__ y, int64_t ldy, int tiles_m,
                                                     int tiles_n, int tiles_dp) {
  constexpr int CPR = BN / 4;          // threads per row (four columns each)
  constexpr int RPP = 256 / CPR;       // rows per pass
  const int u = (int)blockIdx.x / (BM / 16);
  const int c = (int)blockIdx.x % (BM / 16);
  int tm, tn;
  walk_tile(tiles_dp + u, tiles_m, tiles_n, tm, tn);
  const int64_t n = (int64_t)tn * BN + (threadIdx.x % CPR) * 4;
#pragma unroll
  for (int r = (int)threadIdx.x / CPR; r < 16; r += RPP) {
    const int64_t m = (int64_t)tm * BM + c * 16 + r;
    if (m >= M) break;
    float4 acc = *(const float4*)(ws + m * N + n);
    for (int s = 1; s < S; ++s) {
      const float4 v = *(const float4*)(ws + ((int64_t)s * M + m) * N + n);
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    *(uint2*)(y + m * ldy + n) = make_uint2(bf16x2_bits(acc.x, acc.y), bf16x2_bits(acc.z, acc.w));
  }
}

// Workgroups of one kernel resident at once on the current device (CUs x
// workgroups per CU).  Cached per kernel for the last device asked about, as
// (device << 32) | count in one atomic word.
int resident_blocks(const void* kernel, int threads, std::atomic<uint64_t>& cache) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  const uint64_t c = cache.load(std::memory_order_relaxed);
  if (c != 0 && (int)(c >> 32) == dev) return (int)(uint32_t)c;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess) return 0;
  const int n = cus * per_cu;
  if (n > 0) cache.store(((uint64_t)(uint32_t)dev << 32) | (uint32_t)n, std::memory_order_relaxed);
  return n;
}

template <int BM, int BN, int WM, int WN, int NS, int SM>
hipError_t run_p(const GemmArgs& g, int split_k, bool split_tail, hipStream_t stream) {
  using S = Shape<BM, BN, WM, WN>;
  StdParams p;
  p.g = g;
  p.tiles_m = (int)((g.M + BM - 1) / BM);
  p.tiles_n = (int)(g.N / BN);
  p.kb_total = (int)(g.K / 128);
  p.kb_per_split = (p.kb_total + split_k - 1) / split_k;
  const int tiles = p.tiles_m * p.tiles_n;
  p.tiles_dp = 0;
  if (split_k > 1 && split_tail) {
    static std::atomic<uint64_t> cache{0};
    const int slots = resident_blocks((const void*)k_gemm_lds<BM, BN, WM, WN, true, NS, SM>, S::NT, cache);
    if (slots <= 0) return hipErrorInvalidDevice;
    p.tiles_dp = tiles / slots * slots;
    if (p.tiles_dp == tiles) split_k = 1;  // whole rounds only: nothing to split
  }
  p.tail = tiles - p.tiles_dp;
  p.remap_dp = (p.tiles_dp % kXcds == 0) ? 1 : 0;
  const int64_t blocks = (int64_t)p.tiles_dp + (int64_t)p.tail * split_k;
  p.remap = (split_k == 1 ? tiles : (int64_t)p.tail * split_k) % kXcds == 0 ? 1 : 0;
  if (split_k == 1) {
    p.tiles_dp = 0;
    p.tail = tiles;
    p.kb_per_split = p.kb_total;
    hipLaunchKernelGGL((k_gemm_lds<BM, BN, WM, WN, false, NS, SM>), dim3((unsigned)tiles), dim3(S::NT), 0, stream, p);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((k_gemm_lds<BM, BN, WM, WN, true, NS, SM>), dim3((unsigned)blocks), dim3(S::NT), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.tiles_dp == 0) return launch_splitk_reduce(g.ws, split_k, g.M, g.N, g.y, g.ldy, stream);
  hipLaunchKernelGGL((k_tail_reduce<BM, BN>), dim3((unsigned)(p.tail * (BM / 16))), dim3(256), 0, stream, g.ws,
                     split_k, g.M, g.N, g.y, g.ldy, p.tiles_m, p.tiles_n, p.tiles_dp);
  return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, int NS>
hipError_t run(const GemmArgs& g, int split_k, bool split_tail, int sm, hipStream_t stream) {
  if (sm == 1) return run_p<BM, BN, WM, WN, NS, 1>(g, split_k, split_tail, stream);
  if (sm == 2) return run_p<BM, BN, WM, WN, NS, 2>(g, split_k, split_tail, stream);
  return run_p<BM, BN, WM, WN, NS, 0>(g, split_k, split_tail, stream);
}

}  // namespace

// (tile_m, tile_n, LDS stages, kwaves) combinations that are compiled;
// stages 0 means the default, 2.  kwaves 2 doubles the waves of the 64x64,
// 64x128 and 128x128 tiles (each wave 32 columns wide instead of 64): two
// waves per SIMD hide each other's latencies when the grid holds only one
// workgroup per CU (M of a few hundred to a few thousand).  The 64x64 tile
// (a 64-wide weight range inside one 128-row scale block) gives decode-sized
// layers with many weight rows enough workgroups without splitting K, so
// that no partial sums and no second kernel are needed.
bool standard_tile_supported(int tile_m, int tile_n, int stages, int kwaves) {
  const int ns = stages == 0 ? 2 : stages;
  if (tile_m == 64 && tile_n == 64) return (kwaves == 1 || kwaves == 2) && ns >= 2 && ns <= 4;
  if (kwaves == 2) {
    if (tile_m == 64 && tile_n == 128) return ns >= 2 && ns <= 4;
    if (tile_m == 128 && tile_n == 128) return ns == 2 || ns == 3;
    return false;
  }
  if (kwaves != 1) return false;
  if (tile_m == 64 && tile_n == 128) return ns >= 2 && ns <= 4;
  if (tile_m == 128 && tile_n == 128) return ns == 2 || ns == 3;
  if (tile_m == 256 && tile_n == 128) return ns == 2 || ns == 3;
  if (tile_m == 128 && tile_n == 256) return ns == 2;
  if (tile_m == 256 && tile_n == 256) return ns == 2;
  return false;
}

hipError_t launch_gemm_standard(const GemmArgs& g, int tile_m, int tile_n, int split_k, bool split_tail, int stages,
                                int kwaves, int scale_mode, hipStream_t stream) {
  const int sm = scale_mode;  // 0 block fp32, 1 block power-of-two, 2 per-token / per-channel
  const int ns = stages == 0 ? 2 : stages;
  hipError_t e = hipErrorInvalidValue;
  if (tile_m == 64 && tile_n == 64) {
    if (kwaves == 2)
      e = ns == 4 ? run<64, 64, 32, 32, 4>(g, split_k, split_tail, sm, stream)
        : ns == 3 ? run<64, 64, 32, 32, 3>(g, split_k, split_tail, sm, stream)
                  : run<64, 64, 32, 32, 2>(g, split_k, split_tail, sm, stream);
    else if (kwaves == 1)
      e = ns == 4 ? run<64, 64, 32, 64, 4>(g, split_k, split_tail, sm, stream)
        : ns == 3 ? run<64, 64, 32, 64, 3>(g, split_k, split_tail, sm, stream)
                  : run<64, 64, 32, 64, 2>(g, split_k, split_tail, sm, stream);
  } else if (kwaves == 2) {
    if (tile_m == 64 && tile_n == 128)
      e = ns == 4 ? run<64, 128, 32, 32, 4>(g, split_k, split_tail, sm, stream)
        : ns == 3 ? run<64, 128, 32, 32, 3>(g, split_k, split_tail, sm, stream)
                  : run<64, 128, 32, 32, 2>(g, split_k, split_tail, sm, stream);
    else if (tile_m == 128 && tile_n == 128)
      e = ns == 3 ? run<128, 128, 64, 32, 3>(g, split_k, split_tail, sm, stream) : run<128, 128, 64, 32, 2>(g, split_k, split_tail, sm, stream);
  } else if (tile_m == 64 && tile_n == 128) {
    e = ns == 4 ? run<64, 128, 32, 64, 4>(g, split_k, split_tail, sm, stream)
      : ns == 3 ? run<64, 128, 32, 64, 3>(g, split_k, split_tail, sm, stream)
                : run<64, 128, 32, 64, 2>(g, split_k, split_tail, sm, stream);
  } else if (tile_m == 128 && tile_n == 128) {
    e = ns == 3 ? run<128, 128, 64, 64, 3>(g, split_k, split_tail, sm, stream) : run<128, 128, 64, 64, 2>(g, split_k, split_tail, sm, stream);
  } else if (tile_m == 256 && tile_n == 128) {
    e = ns == 3 ? run<256, 128, 64, 64, 3>(g, split_k, split_tail, sm, stream) : run<256, 128, 64, 64, 2>(g, split_k, split_tail, sm, stream);
  } else if (tile_m == 128 && tile_n == 256) {
    e = run<128, 256, 64, 64, 2>(g, split_k, split_tail, sm, stream);
  } else if (tile_m == 256 && tile_n == 256) {
    e = run<256, 256, 128, 64, 2>(g, split_k, split_tail, sm, stream);
  }
  return e;
}

}  // namespace fp8blk
