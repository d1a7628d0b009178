// gemm.hip -- blockwise-scaled FP8 GEMM for gfx950 (scaled_mm_blockwise).
//
//   y[m][n] = bf16( sum_kb sa[m][kb] * sw[n/128][kb] * P_kb[m][n] ),
//   P_kb = sum over the 128 K of block kb of a[m][k] * w[n][k]   (fp8 x fp8 -> fp32)
//
// Block_FP8 scaling (page "Helion: improving vLLM inference with
// autotuning", section "Helion Linear Backend" / "Scope"); the variants
// Standard, Split-K and Swap-AB and their tunables (split_k a power of two up
// to 256, swap_ab a boolean) follow section "Kernel Implementation" of the
// same page.
//
// The K-block of the scales (128) equals the K depth of one
// v_mfma_f32_16x16x128_f8f6f4, so each matrix-core instruction produces one
// complete block partial P_kb for a 16x16 tile; it is folded into the fp32
// accumulator with one FMA per element by the factor sa[m][kb] * sw[nb][kb]
// (the per-K-block rescale).  Split-K here writes fp32 partials to a
// caller-provided workspace and a second kernel sums them in a fixed order,
// instead of zeroing the output and adding with atomics: results are
// bitwise deterministic and the output needs no pre-zeroing.
#include "device_common.hpp"
#include "launch.hpp"

namespace fp8blk {
namespace {

// ---------------------------------------------------------------------------
// Standard variant
// ---------------------------------------------------------------------------
// A workgroup computes a BM x BN tile of y over its range of K blocks.  Per
// K block it stages a[BM][128] and w[BN][128] (fp8) plus sa[BM][kb] in LDS,
// double-buffered: the global loads of block kb+1 are in flight while the
// matrix cores work on block kb.  LDS rows are 128 bytes; 16-byte chunk c of
// row r lives at chunk c ^ (r & 7) so that the ds_read_b128 of a fragment
// (16 rows, same chunk) touch distinct banks.  Waves tile the block as
// (BM/WM) x (BN/WN); a wave's WM x WN tile is (WM/16) x (WN/16) 16x16
// matrix-core tiles.

__device__ __forceinline__ int swz(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }

__device__ __forceinline__ u32x4 lds_load16(const uint8_t* p) { return *(const u32x4*)p; }

template <int N>
__device__ __forceinline__ void gload_rows(u32x4 (&r)[N], const uint8_t* const (&src)[N], int kb) {
#pragma unroll
  for (int i = 0; i < N; ++i) r[i] = *(const u32x4*)(src[i] + (int64_t)kb * 128);
}

template <int N>
__device__ __forceinline__ void lstore_rows(uint8_t* lds, const u32x4 (&r)[N], const int (&dst)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) *(u32x4*)(lds + dst[i]) = r[i];
}

struct StdParams {
  GemmArgs g;
  int tiles_m, tiles_n;
  int kb_total, kb_per_split;
};

template <int BM, int BN, int WM, int WN>
struct StdShape {
  static constexpr int WAVES_M = BM / WM;
  static constexpr int WAVES_N = BN / WN;
  static constexpr int NT = WAVES_M * WAVES_N * 64;
  static constexpr int TM = WM / 16;
  static constexpr int TN = WN / 16;
  static constexpr int A_CHUNKS = BM * 8 / NT;
  static constexpr int B_CHUNKS = BN * 8 / NT;
  static_assert(BM * 8 % NT == 0 && BN * 8 % NT == 0, "tile not divisible by threads");
  static_assert(128 % WN == 0, "a wave's N range must sit inside one 128-row weight block");
  static_assert(BM <= NT, "one thread per row loads the activation scales");
};

template <int BM, int BN, int WM, int WN, bool SPLIT>
__global__ __launch_bounds__(BM / WM * (BN / WN) * 64) void k_gemm_std(StdParams p) {
  using S = StdShape<BM, BN, WM, WN>;
  __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][BM * 128];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b[2][BN * 128];
  __shared__ float lds_sa[2][BM];

  const GemmArgs& g = p.g;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wave_m = wave % S::WAVES_M;
  const int wave_n = wave / S::WAVES_M;

  const int tiles = p.tiles_m * p.tiles_n;
  const int split = blockIdx.x / tiles;
  const int t = blockIdx.x - split * tiles;
  const int tm = t % p.tiles_m;
  const int tn = t / p.tiles_m;
  const int64_t m0 = (int64_t)tm * BM;
  const int64_t n0 = (int64_t)tn * BN;
  const int kb0 = split * p.kb_per_split;
  const int kb1 = min(kb0 + p.kb_per_split, p.kb_total);
  const int64_t mlast = g.M - 1;

  // global -> LDS assignment (rows past M re-read row M-1; never stored)
  const uint8_t* a_src[S::A_CHUNKS];
  int a_dst[S::A_CHUNKS];
#pragma unroll
  for (int i = 0; i < S::A_CHUNKS; ++i) {
    const int c = tid + i * S::NT;
    const int row = c >> 3, ch = c & 7;
    const int64_t m = min(m0 + row, mlast);
    a_src[i] = g.a + m * g.lda + ch * 16;
    a_dst[i] = swz(row, ch);
  }
  const uint8_t* b_src[S::B_CHUNKS];
  int b_dst[S::B_CHUNKS];
#pragma unroll
  for (int i = 0; i < S::B_CHUNKS; ++i) {
    const int c = tid + i * S::NT;
    const int row = c >> 3, ch = c & 7;
    b_src[i] = g.w + (n0 + row) * g.ldw + ch * 16;
    b_dst[i] = swz(row, ch);
  }
  const float* sa_src = g.sa + min(m0 + (tid < BM ? tid : 0), mlast) * g.ldsa;
  const float* sw_src = g.sw + ((n0 + wave_n * WN) >> 7) * g.ldsw;

  u32x4 ra[S::A_CHUNKS], rb[S::B_CHUNKS];
  float rsa = 0.f;
  v4f acc[S::TM][S::TN];
#pragma unroll
  for (int i = 0; i < S::TM; ++i)
#pragma unroll
    for (int j = 0; j < S::TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const int frow = lane & 15;
  const int fch = (lane >> 4) * 2;
  const int orow = (lane >> 4) * 4;

  if (kb0 < kb1) {
    gload_rows(ra, a_src, kb0);
    gload_rows(rb, b_src, kb0);
    if (tid < BM) rsa = sa_src[kb0];
    lstore_rows(&lds_a[0][0], ra, a_dst);
    lstore_rows(&lds_b[0][0], rb, b_dst);
    if (tid < BM) lds_sa[0][tid] = rsa;
  }
  __syncthreads();
  for (int kb = kb0; kb < kb1; ++kb) {
    const int buf = (kb - kb0) & 1;
    if (kb + 1 < kb1) {
      gload_rows(ra, a_src, kb + 1);
      gload_rows(rb, b_src, kb + 1);
      if (tid < BM) rsa = sa_src[kb + 1];
    }
    const float swv = sw_src[kb];
    v8i bf[S::TN];
#pragma unroll
    for (int j = 0; j < S::TN; ++j) {
      const int r = wave_n * WN + j * 16 + frow;
      bf[j] = make_v8i(lds_load16(&lds_b[buf][swz(r, fch)]), lds_load16(&lds_b[buf][swz(r, fch + 1)]));
    }
#pragma unroll
    for (int i = 0; i < S::TM; ++i) {
      const int r = wave_m * WM + i * 16 + frow;
      const v8i af = make_v8i(lds_load16(&lds_a[buf][swz(r, fch)]), lds_load16(&lds_a[buf][swz(r, fch + 1)]));
      float gsc[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) gsc[q] = lds_sa[buf][wave_m * WM + i * 16 + orow + q] * swv;
#pragma unroll
      for (int j = 0; j < S::TN; ++j) {
        const v4f P = mfma16x16x128(af, bf[j]);
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[i][j][q] = __builtin_fmaf(P[q], gsc[q], acc[i][j][q]);
      }
    }
    if (kb + 1 < kb1) {
      lstore_rows(&lds_a[buf ^ 1][0], ra, a_dst);
      lstore_rows(&lds_b[buf ^ 1][0], rb, b_dst);
      if (tid < BM) lds_sa[buf ^ 1][tid] = rsa;
    }
    __syncthreads();
  }

  // epilogue: lane holds rows orow..orow+3, column frow of every 16x16 tile
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

// ---------------------------------------------------------------------------
// Swap-AB variant (small M)
// ---------------------------------------------------------------------------
// Computes y^T = w a^T: 16-row slices of the weight are the matrix-core "A"
// operand and up to 16 tokens are the "B" operand, so one instruction covers
// 16 weight rows x 16 tokens x one 128-wide K block and no row of the
// instruction is wasted on padding tokens.  A workgroup owns RN*16 weight
// rows and all (<= 16*TOKT) tokens; its kwaves waves split the workgroup's K
// range and their fp32 tiles are summed in LDS in a fixed wave order.  Weight
// fragments are read straight from HBM (each weight byte is used by exactly
// one workgroup), two K blocks at a time per wave to keep loads in flight;
// activations and their scales are small and come from L2.

struct SwapParams {
  GemmArgs g;
  int kb_total, kb_per_split;
};

__device__ __forceinline__ u32x4 gload16(const uint8_t* p) { return *(const u32x4*)p; }

template <int TOKT, int RN, bool SPLIT>
__global__ __launch_bounds__(512) void k_gemm_swapab(SwapParams p) {
  constexpr int UNR = 2;
  __shared__ float red[8 * RN * TOKT * 4 * 64];
  const GemmArgs& g = p.g;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int kw = blockDim.x >> 6;
  const int64_t n0 = (int64_t)blockIdx.x * 16 * RN;
  const int split = blockIdx.y;
  const int kbs0 = split * p.kb_per_split;
  const int kbs1 = min(kbs0 + p.kb_per_split, p.kb_total);
  const int per = (kbs1 - kbs0 + kw - 1) / kw;
  const int kb0 = kbs0 + wave * per;
  const int kb1 = min(kb0 + per, kbs1);

  const int row = lane & 15;
  const int kq = (lane >> 4) * 32;
  const uint8_t* wsrc[RN];
#pragma unroll
  for (int r = 0; r < RN; ++r) wsrc[r] = g.w + (n0 + r * 16 + row) * g.ldw + kq;
  const uint8_t* xsrc[TOKT];
  const float* sasrc[TOKT];
  bool tvalid[TOKT];
#pragma unroll
  for (int t = 0; t < TOKT; ++t) {
    const int64_t m = t * 16 + row;
    tvalid[t] = m < g.M;
    const int64_t mc = tvalid[t] ? m : 0;
    xsrc[t] = g.a + mc * g.lda + kq;
    sasrc[t] = g.sa + mc * g.ldsa;
  }
  const float* swsrc = g.sw + (n0 >> 7) * g.ldsw;

  v4f acc[RN][TOKT];
#pragma unroll
  for (int r = 0; r < RN; ++r)
#pragma unroll
    for (int t = 0; t < TOKT; ++t) acc[r][t] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int kb = kb0; kb < kb1; kb += UNR) {
    v8i wf[UNR][RN], xf[UNR][TOKT];
    float gsc[UNR][TOKT];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int k = kb + u;
      const bool kval = k < kb1;
      const int64_t ko = (int64_t)(kval ? k : kb) * 128;
#pragma unroll
      for (int r = 0; r < RN; ++r)
        wf[u][r] = make_v8i(load_nt16(wsrc[r] + ko), load_nt16(wsrc[r] + ko + 16));
      const float swv = kval ? swsrc[kval ? k : kb] : 0.f;
#pragma unroll
      for (int t = 0; t < TOKT; ++t) {
        if (tvalid[t]) {
          xf[u][t] = make_v8i(gload16(xsrc[t] + ko), gload16(xsrc[t] + ko + 16));
          gsc[u][t] = sasrc[t][kval ? k : kb] * swv;
        } else {
          xf[u][t] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
          gsc[u][t] = 0.f;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
#pragma unroll
      for (int r = 0; r < RN; ++r)
#pragma unroll
        for (int t = 0; t < TOKT; ++t) {
          const v4f P = mfma16x16x128(wf[u][r], xf[u][t]);
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[r][t][q] = __builtin_fmaf(P[q], gsc[u][t], acc[r][t][q]);
        }
    }
  }

  // lane holds weight rows n0 + 16r + 4*(lane>>4) + q (q = 0..3) for token
  // 16t + (lane & 15)
  if (kw > 1) {
#pragma unroll
    for (int r = 0; r < RN; ++r)
#pragma unroll
      for (int t = 0; t < TOKT; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q) red[((wave * RN + r) * TOKT + t) * 256 + q * 64 + lane] = acc[r][t][q];
    __syncthreads();
    for (int idx = threadIdx.x; idx < RN * TOKT * 64; idx += blockDim.x) {
      const int rt = idx >> 6, ln = idx & 63;
      float v[4] = {0.f, 0.f, 0.f, 0.f};
      for (int w2 = 0; w2 < kw; ++w2)
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] += red[(w2 * RN * TOKT + rt) * 256 + q * 64 + ln];
      const int r = rt / TOKT, t = rt - (rt / TOKT) * TOKT;
      const int64_t m = t * 16 + (ln & 15);
      const int64_t n = n0 + r * 16 + (ln >> 4) * 4;
      if (m < g.M) {
        if (SPLIT)
          *(float4*)(g.ws + ((int64_t)split * g.M + m) * g.N + n) = make_float4(v[0], v[1], v[2], v[3]);
        else
          *(uint2*)(g.y + m * g.ldy + n) =
              make_uint2(f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16),
                         f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16));
      }
    }
  } else {
#pragma unroll
    for (int r = 0; r < RN; ++r)
#pragma unroll
      for (int t = 0; t < TOKT; ++t) {
        const int64_t m = t * 16 + row;
        const int64_t n = n0 + r * 16 + (lane >> 4) * 4;
        if (m < g.M) {
          const v4f v = acc[r][t];
          if (SPLIT)
            *(float4*)(g.ws + ((int64_t)split * g.M + m) * g.N + n) = make_float4(v[0], v[1], v[2], v[3]);
          else
            *(uint2*)(g.y + m * g.ldy + n) =
                make_uint2(f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16),
                           f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16));
        }
      }
  }
}

// ---------------------------------------------------------------------------
// Split-K reduction: y = bf16(sum_s ws[s]) in increasing s.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_splitk_reduce(const float* __restrict__ ws, int S,
                                                       int64_t M, int64_t N,
                                                       uint16_t* __restrict__ y, int64_t ldy) {
  const int64_t n = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (n >= N) return;
  for (int64_t m = blockIdx.y; m < M; m += gridDim.y) {
    float4 acc = *(const float4*)(ws + m * N + n);
    for (int s = 1; s < S; ++s) {
      const float4 v = *(const float4*)(ws + ((int64_t)s * M + m) * N + n);
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    *(uint2*)(y + m * ldy + n) = make_uint2(f32_to_bf16_bits(acc.x) | (f32_to_bf16_bits(acc.y) << 16),
                                            f32_to_bf16_bits(acc.z) | (f32_to_bf16_bits(acc.w) << 16));
  }
}

template <int BM, int BN, int WM, int WN>
hipError_t run_std(const GemmArgs& g, int split_k, hipStream_t stream) {
  using S = StdShape<BM, BN, WM, WN>;
  StdParams p;
  p.g = g;
  p.tiles_m = (int)((g.M + BM - 1) / BM);
  p.tiles_n = (int)(g.N / BN);
  p.kb_total = (int)(g.K / 128);
  p.kb_per_split = (p.kb_total + split_k - 1) / split_k;
  const int64_t blocks = (int64_t)p.tiles_m * p.tiles_n * split_k;
  if (split_k > 1)
    hipLaunchKernelGGL((k_gemm_std<BM, BN, WM, WN, true>), dim3((unsigned)blocks), dim3(S::NT), 0, stream, p);
  else
    hipLaunchKernelGGL((k_gemm_std<BM, BN, WM, WN, false>), dim3((unsigned)blocks), dim3(S::NT), 0, stream, p);
  return hipGetLastError();
}

template <int TOKT, int RN>
hipError_t run_swap(const GemmArgs& g, int kwaves, int split_k, hipStream_t stream) {
  SwapParams p;
  p.g = g;
  p.kb_total = (int)(g.K / 128);
  p.kb_per_split = (p.kb_total + split_k - 1) / split_k;
  dim3 grid((unsigned)(g.N / (16 * RN)), (unsigned)split_k);
  if (split_k > 1)
    hipLaunchKernelGGL((k_gemm_swapab<TOKT, RN, true>), grid, dim3(64 * kwaves), 0, stream, p);
  else
    hipLaunchKernelGGL((k_gemm_swapab<TOKT, RN, false>), grid, dim3(64 * kwaves), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

bool standard_tile_supported(int tile_m, int tile_n) {
  return (tile_m == 64 && tile_n == 128) || (tile_m == 128 && tile_n == 128) ||
         (tile_m == 256 && tile_n == 128) || (tile_m == 128 && tile_n == 256);
}

hipError_t launch_gemm_standard(const GemmArgs& g, int tile_m, int tile_n, int split_k,
                                hipStream_t stream) {
  hipError_t e = hipErrorInvalidValue;
  if (tile_m == 64 && tile_n == 128)
    e = run_std<64, 128, 32, 64>(g, split_k, stream);
  else if (tile_m == 128 && tile_n == 128)
    e = run_std<128, 128, 64, 64>(g, split_k, stream);
  else if (tile_m == 256 && tile_n == 128)
    e = run_std<256, 128, 64, 64>(g, split_k, stream);
  else if (tile_m == 128 && tile_n == 256)
    e = run_std<128, 256, 64, 64>(g, split_k, stream);
  if (e != hipSuccess || split_k == 1) return e;
  return launch_splitk_reduce(g.ws, split_k, g.M, g.N, g.y, g.ldy, stream);
}

bool swapab_tile_supported(int tile_m, int tile_n, int kwaves) {
  const bool tm = tile_m == 16 || tile_m == 32 || tile_m == 64;
  const bool tn = tile_n == 16 || tile_n == 32 || (tile_n == 64 && tile_m <= 32);
  const bool kwv = kwaves == 1 || kwaves == 2 || kwaves == 4 || kwaves == 8;
  return tm && tn && kwv;
}

hipError_t launch_gemm_swapab(const GemmArgs& g, int tile_m, int tile_n, int kwaves, int split_k,
                              hipStream_t stream) {
  const int tokt = tile_m / 16, rn = tile_n / 16;
  hipError_t e = hipErrorInvalidValue;
#define FP8BLK_SWAP_CASE(T, R) \
  if (tokt == T && rn == R) e = run_swap<T, R>(g, kwaves, split_k, stream);
  FP8BLK_SWAP_CASE(1, 1)
  FP8BLK_SWAP_CASE(1, 2)
  FP8BLK_SWAP_CASE(1, 4)
  FP8BLK_SWAP_CASE(2, 1)
  FP8BLK_SWAP_CASE(2, 2)
  FP8BLK_SWAP_CASE(2, 4)
  FP8BLK_SWAP_CASE(4, 1)
  FP8BLK_SWAP_CASE(4, 2)
#undef FP8BLK_SWAP_CASE
  if (e != hipSuccess || split_k == 1) return e;
  return launch_splitk_reduce(g.ws, split_k, g.M, g.N, g.y, g.ldy, stream);
}

hipError_t launch_splitk_reduce(const float* ws, int split_k, int64_t M, int64_t N, uint16_t* y,
                                int64_t ldy, hipStream_t stream) {
  const int64_t gx = (N / 4 + 255) / 256;
  const int64_t gy = M < 65535 ? M : 65535;
  hipLaunchKernelGGL(k_splitk_reduce, dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, stream, ws,
                     split_k, M, N, y, ldy);
  return hipGetLastError();
}

}  // namespace fp8blk
