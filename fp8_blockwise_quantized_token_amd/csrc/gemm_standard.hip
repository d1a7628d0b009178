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
//     activation scales sa[BM][kb] go HBM -> LDS with global_load_lds (the
//     data never passes through VGPRs).  Two LDS stages: the loads of block
//     kb+1 are in flight while the matrix cores work on block kb.
//   * LDS rows are 128 bytes = eight 16-byte chunks; chunk c of row r is
//     stored at c ^ g(r), g(r) = ((r >> 1) & 7) ^ ((r & 1) << 2), so the
//     ds_read_b128 of a fragment (16 consecutive rows, one chunk) hit 16
//     distinct 16-byte bank groups of a 256-byte window (and 8 distinct ones
//     of any 128-byte window).  One direct-to-LDS instruction fills 8 rows
//     (1 KiB, lane L at offset 16 L); lane L therefore fetches chunk
//     (L & 7) ^ g(row) of its row.
//   * One v_mfma_f32_16x16x128_f8f6f4 per 16x16 tile and K block gives the
//     complete block partial P_kb; it is folded into the fp32 accumulator
//     with one FMA by sa[m][kb] * sw[nb][kb] (a wave's N range lies inside one
//     128-row weight block, so sw is a scalar per wave and K block).
//   * Tile order: blocks are remapped so that each XCD (blocks are dealt
//     round-robin to the 8 XCDs) owns a contiguous range of tiles, and tiles
//     are walked in column groups of GROUP_M tile-rows, so the workgroups
//     resident on one XCD share A and W slices in that XCD's L2.
//   * Split-K: grid x split_k; split s covers a contiguous range of K blocks
//     and writes fp32 partials to the workspace [split][M][N]; a separate
//     kernel sums them in split order.
#include "device_common.hpp"
#include "launch.hpp"

namespace fp8blk {
namespace {

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ int swz_g(int row) { return ((row >> 1) & 7) ^ ((row & 1) << 2); }
__device__ __forceinline__ int swz_off(int row, int chunk) { return row * 128 + ((chunk ^ swz_g(row)) << 4); }

struct StdParams {
  GemmArgs g;
  int tiles_m, tiles_n;
  int kb_total, kb_per_split;
  int remap;  // 1: XCD-contiguous remap (block count divisible by 8)
};

constexpr int kGroupM = 8;
constexpr int kXcds = 8;

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
  static_assert((BM / 8) % WAVES == 0 && (BN / 8) % WAVES == 0, "row groups must divide over waves");
  static_assert(128 % WN == 0, "a wave's N range must sit inside one 128-row weight block");
  static_assert(SW_WAVE < WAVES, "one scale load per wave at most");
};

template <int BM, int BN, int WM, int WN, bool SPLIT>
__global__ __launch_bounds__(BM / WM * (BN / WN) * 64) void k_gemm_lds(StdParams p) {
  using S = Shape<BM, BN, WM, WN>;
  __shared__ __attribute__((aligned(1024))) uint8_t lds_a0[BM * 128];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_a1[BM * 128];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_b0[BN * 128];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_b1[BN * 128];
  __shared__ __attribute__((aligned(256))) float lds_s0[S::S_FLOATS];
  __shared__ __attribute__((aligned(256))) float lds_s1[S::S_FLOATS];

  const GemmArgs& g = p.g;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wave_m = wave % S::WAVES_M;
  const int wave_n = wave / S::WAVES_M;

  // ---- tile of this workgroup ----
  const int tiles = p.tiles_m * p.tiles_n;
  int bid = blockIdx.x;
  if (p.remap) {
    const int per_xcd = (int)(gridDim.x / kXcds);
    bid = (bid % kXcds) * per_xcd + bid / kXcds;
  }
  const int split = bid / tiles;
  const int t = bid - split * tiles;
  const int group = kGroupM * p.tiles_n;
  const int first_m = (t / group) * kGroupM;
  const int gm = min(kGroupM, p.tiles_m - first_m);
  const int tm = first_m + (t % group) % gm;
  const int tn = (t % group) / gm;
  const int64_t m0 = (int64_t)tm * BM;
  const int64_t n0 = (int64_t)tn * BN;
  const int kb0 = split * p.kb_per_split;
  const int kb1 = min(kb0 + p.kb_per_split, p.kb_total);
  const int64_t mlast = g.M - 1;

  // ---- direct-to-LDS source addresses (per lane) ----
  // instruction i of this wave fills rows 8 * (wave + i * WAVES) .. +7
  const int lrow = lane >> 3;
  const int lch = lane & 7;
  const uint8_t* a_src[S::A_INSTR];
#pragma unroll
  for (int i = 0; i < S::A_INSTR; ++i) {
    const int row = 8 * (wave + i * S::WAVES) + lrow;
    const int64_t m = min(m0 + row, mlast);
    a_src[i] = g.a + m * g.lda + ((lch ^ swz_g(row)) << 4);
  }
  const uint8_t* b_src[S::B_INSTR];
#pragma unroll
  for (int i = 0; i < S::B_INSTR; ++i) {
    const int row = 8 * (wave + i * S::WAVES) + lrow;
    b_src[i] = g.w + (n0 + row) * g.ldw + ((lch ^ swz_g(row)) << 4);
  }
  const float* sa_src = g.sa + min(m0 + (wave * 64 + lane) % BM, mlast) * g.ldsa;
  const float* sw_src = g.sw + ((n0 >> 7) + min(lane, BN / 128 - 1)) * g.ldsw;
  const int sw_slot = BM + ((wave_n * WN) >> 7);  // this wave's weight scale in the stage buffer

  auto issue = [&](uint8_t* la, uint8_t* lb, float* ls, int kb) {
    const int64_t ko = (int64_t)kb * 128;
#pragma unroll
    for (int i = 0; i < S::A_INSTR; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(a_src[i] + ko),
                                       (lds_void*)(la + (wave + i * S::WAVES) * 1024), 16, 0, 0);
#pragma unroll
    for (int i = 0; i < S::B_INSTR; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(b_src[i] + ko),
                                       (lds_void*)(lb + (wave + i * S::WAVES) * 1024), 16, 0, 0);
    if (wave < S::SA_INSTR)
      __builtin_amdgcn_global_load_lds((const void*)(sa_src + kb), (lds_void*)(ls + wave * 64), 4, 0, 0);
    else if (wave == S::SW_WAVE)
      __builtin_amdgcn_global_load_lds((const void*)(sw_src + kb), (lds_void*)(ls + BM), 4, 0, 0);
  };

  v4f acc[S::TM][S::TN];
#pragma unroll
  for (int i = 0; i < S::TM; ++i)
#pragma unroll
    for (int j = 0; j < S::TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const int frow = lane & 15;
  const int fch = (lane >> 4) * 2;
  const int orow = (lane >> 4) * 4;

  auto compute = [&](const uint8_t* la, const uint8_t* lb, const float* ls) {
    const float swv = ls[sw_slot];
    v8i bf[S::TN];
#pragma unroll
    for (int j = 0; j < S::TN; ++j) {
      const int r = wave_n * WN + j * 16 + frow;
      bf[j] = make_v8i(*(const u32x4*)(lb + swz_off(r, fch)), *(const u32x4*)(lb + swz_off(r, fch + 1)));
    }
#pragma unroll
    for (int i = 0; i < S::TM; ++i) {
      const int r = wave_m * WM + i * 16 + frow;
      const v8i af = make_v8i(*(const u32x4*)(la + swz_off(r, fch)), *(const u32x4*)(la + swz_off(r, fch + 1)));
      const v4f sa4 = *(const v4f*)(ls + wave_m * WM + i * 16 + orow);
      const float g0 = sa4[0] * swv, g1 = sa4[1] * swv, g2 = sa4[2] * swv, g3 = sa4[3] * swv;
#pragma unroll
      for (int j = 0; j < S::TN; ++j) {
        const v4f P = mfma16x16x128(af, bf[j]);
        acc[i][j][0] = __builtin_fmaf(P[0], g0, acc[i][j][0]);
        acc[i][j][1] = __builtin_fmaf(P[1], g1, acc[i][j][1]);
        acc[i][j][2] = __builtin_fmaf(P[2], g2, acc[i][j][2]);
        acc[i][j][3] = __builtin_fmaf(P[3], g3, acc[i][j][3]);
      }
    }
  };

  if (kb0 < kb1) issue(lds_a0, lds_b0, lds_s0, kb0);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads have landed
  __syncthreads();
  for (int kb = kb0; kb < kb1; ++kb) {
    const bool odd = ((kb - kb0) & 1) != 0;
    uint8_t* ca = odd ? lds_a1 : lds_a0;
    uint8_t* cb = odd ? lds_b1 : lds_b0;
    float* cs = odd ? lds_s1 : lds_s0;
    if (kb + 1 < kb1) issue(odd ? lds_a0 : lds_a1, odd ? lds_b0 : lds_b1, odd ? lds_s0 : lds_s1, kb + 1);
    compute(ca, cb, cs);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
  }

  // ---- epilogue: lane holds rows orow..orow+3 and column frow of each tile ----
#pragma unroll
  for (int i = 0; i < S::TM; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t m = m0 + wave_m * WM + i * 16 + orow + q;
      if (m >= g.M) continue;
#pragma unroll
      for (int j = 0; j < S::TN; ++j) {
        const int64_t n = n0 + wave_n * WN + j * 16 + frow;
        if (SPLIT)
          g.ws[((int64_t)split * g.M + m) * g.N + n] = acc[i][j][q];
        else
          g.y[m * g.ldy + n] = (uint16_t)f32_to_bf16_bits(acc[i][j][q]);
      }
    }
  }
}

template <int BM, int BN, int WM, int WN>
hipError_t run(const GemmArgs& g, int split_k, hipStream_t stream) {
  using S = Shape<BM, BN, WM, WN>;
  StdParams p;
  p.g = g;
  p.tiles_m = (int)((g.M + BM - 1) / BM);
  p.tiles_n = (int)(g.N / BN);
  p.kb_total = (int)(g.K / 128);
  p.kb_per_split = (p.kb_total + split_k - 1) / split_k;
  const int64_t blocks = (int64_t)p.tiles_m * p.tiles_n * split_k;
  p.remap = (blocks % kXcds == 0) ? 1 : 0;
  if (split_k > 1)
    hipLaunchKernelGGL((k_gemm_lds<BM, BN, WM, WN, true>), dim3((unsigned)blocks), dim3(S::NT), 0, stream, p);
  else
    hipLaunchKernelGGL((k_gemm_lds<BM, BN, WM, WN, false>), dim3((unsigned)blocks), dim3(S::NT), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

bool standard_tile_supported(int tile_m, int tile_n) {
  return (tile_m == 64 && tile_n == 128) || (tile_m == 128 && tile_n == 128) ||
         (tile_m == 256 && tile_n == 128) || (tile_m == 128 && tile_n == 256) ||
         (tile_m == 256 && tile_n == 256);
}

hipError_t launch_gemm_standard(const GemmArgs& g, int tile_m, int tile_n, int split_k,
                                hipStream_t stream) {
  hipError_t e = hipErrorInvalidValue;
  if (tile_m == 64 && tile_n == 128)
    e = run<64, 128, 32, 64>(g, split_k, stream);
  else if (tile_m == 128 && tile_n == 128)
    e = run<128, 128, 64, 64>(g, split_k, stream);
  else if (tile_m == 256 && tile_n == 128)
    e = run<256, 128, 64, 64>(g, split_k, stream);
  else if (tile_m == 128 && tile_n == 256)
    e = run<128, 256, 64, 64>(g, split_k, stream);
  else if (tile_m == 256 && tile_n == 256)
    e = run<256, 256, 128, 64>(g, split_k, stream);
  if (e != hipSuccess || split_k == 1) return e;
  return launch_splitk_reduce(g.ws, split_k, g.M, g.N, g.y, g.ldy, stream);
}

}  // namespace fp8blk
