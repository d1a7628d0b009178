// gemm.hip -- Swap-AB variant and the Split-K reduction of the
// blockwise-scaled FP8 GEMM for gfx950 (scaled_mm_blockwise); the Standard
// variant is in gemm_standard.hip.
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
