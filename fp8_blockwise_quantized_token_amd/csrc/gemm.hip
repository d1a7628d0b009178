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

// The fused quantizer must round exactly like fp8_group_quant: no FMA
// contraction of separate multiplies and adds.
#pragma clang fp contract(off)

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
// fragments are read straight from HBM into registers (each weight byte is
// used by exactly one workgroup; plain loads, which measure faster here than
// non-temporal ones), two K blocks at a time per wave to keep loads in flight;
// activations and their scales are small and come from L2.

struct SwapParams {
  GemmArgs g;
  int kb_total, kb_per_split;
};

__device__ __forceinline__ u32x4 gload16(const uint8_t* p) { return *(const u32x4*)p; }

// Fused variants (FQ != 0): the activation operand is quantized here from
// bf16 x with exactly the group rule of fp8_group_quant (same amax, scale,
// division and encoder), so the GEMM sees the bytes and scales the separate
// quantizer would have produced.
//   FQ = 16: lane l holds 32 of the 128 values of group (token l & 15, kb)
//     in operand order; the group amax is reduced over the four lanes l,
//     l^16, l^32, l^48 that hold the same token.
//   FQ = 1, 2, 4, 8 (M <= FQ, one token tile): only the FQ tokens that can
//     be valid are quantized, 64/FQ lanes per token and 2 FQ values per lane
//     (the work of the 16 - FQ padding rows is not done); the codes go to a
//     wave-private 16 x 128-byte LDS tile (rows >= FQ stay zero) and are
//     read back in operand order.
//
// CH: per-token / per-channel scales (FP8_Dynamic, separate quantizer): the
// K loop accumulates in the matrix core without rescaling and the epilogue
// multiplies by sw[n] * sa[m].
template <int TOKT, int RN, bool SPLIT, int FQ, bool CH>
__global__ __launch_bounds__(512) void k_gemm_swapab(SwapParams p) {
  static_assert(!CH || FQ == 0, "per-token scales need the whole row: quantize first");
  constexpr bool FUSED = FQ != 0;
  constexpr bool LEAN = FQ > 0 && FQ < 16;
  static_assert(!LEAN || TOKT == 1, "the lean quantizer serves one token tile");
  constexpr int LPT = LEAN ? 64 / FQ : 1;      // lanes per token
  constexpr int EPL = LEAN ? 128 / LPT : 2;    // values per lane (2 FQ)
  constexpr int UNR = (RN + TOKT <= 3) ? 2 : 1;  // K blocks per register batch
  __shared__ float red[8 * RN * TOKT * 4 * 64];
  __shared__ __attribute__((aligned(16))) uint8_t xq_all[LEAN ? 8 * 2112 : 16];  // per wave: codes, scales
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

  // Matrix-core operands: lane l holds row l & 15 and 32 bytes of the K
  // block.  Only the pairing of A and B bytes matters, so both operands use
  // the same K order: lane group g = l >> 4 takes bytes [16g, 16g+16) and
  // [64+16g, 64+16g+16).  Each 16-byte load instruction then reads 64
  // contiguous bytes of each of its 16 rows.
  const int row = lane & 15;
  const int kq = (lane >> 4) * 16;
  const uint8_t* wsrc[RN];
#pragma unroll
  for (int r = 0; r < RN; ++r) wsrc[r] = g.w + (n0 + r * 16 + row) * g.ldw + kq;
  const uint8_t* xsrc[TOKT];
  const uint16_t* xbsrc[TOKT];  // fused: bf16 activations, element 16g of the block
  const float* sasrc[TOKT];
  bool tvalid[TOKT];
#pragma unroll
  for (int t = 0; t < TOKT; ++t) {
    const int64_t m = t * 16 + row;
    tvalid[t] = m < g.M;
    const int64_t mc = tvalid[t] ? m : 0;
    if (FUSED) {
      xbsrc[t] = g.x + mc * g.ldx + kq;
    } else {
      xsrc[t] = g.a + mc * g.lda + kq;
      sasrc[t] = g.sa + mc * g.sa_row;
    }
  }
  const float* swsrc = g.sw + (n0 >> 7) * g.ldsw;

  // lean quantizer: lane (lt, lp) loads values [lp EPL, (lp+1) EPL) of token lt
  const int lt = lane / LPT, lp = lane % LPT;
  const bool lvalid = lt < g.M;
  const uint16_t* lsrc = LEAN ? g.x + (int64_t)(lvalid ? lt : 0) * g.ldx + lp * EPL : nullptr;
  uint8_t* xq = xq_all + (LEAN ? wave * 2112 : 0);  // 16 rows x 128 code bytes, then 16 scales
  if (LEAN) {
    u32x4* z = (u32x4*)xq;
    z[lane] = u32x4{0u, 0u, 0u, 0u};
    z[lane + 64] = u32x4{0u, 0u, 0u, 0u};
    if (lane < 4) z[128 + lane] = u32x4{0u, 0u, 0u, 0u};
  }

  v4f acc[RN][TOKT];
#pragma unroll
  for (int r = 0; r < RN; ++r)
#pragma unroll
    for (int t = 0; t < TOKT; ++t) acc[r][t] = v4f{0.f, 0.f, 0.f, 0.f};

  // Two register batches of UNR K blocks each: the loads of the next batch
  // are issued before the matrix-core work of the current one, so every
  // wave keeps 2 * UNR K blocks of weight in flight.  Inside a batch, K
  // blocks past the wave's range re-read its last block (in-bounds, an L2
  // hit) and get a zero factor.
  struct Batch {
    v8i wf[UNR][RN];
    v8i xf[UNR][TOKT];       // quantized operands (separate-quant path)
    float gsc[UNR][TOKT];
    u32x4 xr[UNR][TOKT][4];             // fused (FQ = 16): 32 raw bf16 values of this lane
    u32x4 xl[UNR][LEAN && FQ == 8 ? 2 : 1];  // lean: 2 FQ raw bf16 values
    float swv[UNR];
  };
  const int kblast = kb1 - 1;
  // The activation bytes and the scales of a batch are requested before its
  // weight fragments: loads complete in order, so the activation operand
  // (and the fused quantizer's work on it) is ready while the weights are
  // still streaming in.
  auto load = [&](Batch& b, int kb) {
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int k = kb + u;
      const int kc = max(min(k, kblast), 0);
      const int64_t ko = (int64_t)kc * 128;
      const float swv = CH ? 0.f : (k <= kblast ? swsrc[kc] : 0.f);
      if (FUSED) b.swv[u] = swv;
      if (LEAN) {
        u32x4 v0 = u32x4{0u, 0u, 0u, 0u}, v1 = u32x4{0u, 0u, 0u, 0u};
        if (lvalid) {
          const uint16_t* src = lsrc + ko;
          if (FQ == 1) {
            v0.x = *(const uint32_t*)src;
          } else if (FQ == 2) {
            const uint2 t2 = *(const uint2*)src;
            v0.x = t2.x;
            v0.y = t2.y;
          } else {
            v0 = *(const u32x4*)src;
            if (FQ == 8) v1 = *(const u32x4*)(src + 8);
          }
        }
        b.xl[u][0] = v0;
        if (FQ == 8) b.xl[u][LEAN && FQ == 8 ? 1 : 0] = v1;
        continue;
      }
#pragma unroll
      for (int t = 0; t < TOKT; ++t) {
        if (FUSED) {
          if (tvalid[t]) {
            const uint16_t* src = xbsrc[t] + ko;
            b.xr[u][t][0] = *(const u32x4*)(src);
            b.xr[u][t][1] = *(const u32x4*)(src + 8);
            b.xr[u][t][2] = *(const u32x4*)(src + 64);
            b.xr[u][t][3] = *(const u32x4*)(src + 72);
          } else {
#pragma unroll
            for (int c = 0; c < 4; ++c) b.xr[u][t][c] = u32x4{0u, 0u, 0u, 0u};
          }
        } else if (tvalid[t]) {
          b.xf[u][t] = make_v8i(gload16(xsrc[t] + ko), gload16(xsrc[t] + ko + 64));
          // CH: no per-block factor; a K block past the range must add nothing
          b.gsc[u][t] = CH ? (k <= kblast ? 1.f : 0.f) : sasrc[t][kc * g.sa_kb] * swv;
        } else {
          b.xf[u][t] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
          b.gsc[u][t] = 0.f;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int64_t ko = (int64_t)max(min(kb + u, kblast), 0) * 128;
#pragma unroll
      for (int r = 0; r < RN; ++r)
        b.wf[u][r] = make_v8i(load16(wsrc[r] + ko), load16(wsrc[r] + ko + 64));
    }
  };
  // fused: quantize one lane's 32 values of group (token, kb) -> operand, scale
  auto quant_operand = [&](const u32x4 (&xr)[4], v8i& op, float& sc) {
    uint32_t am = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const u32x4 w = xr[c];
      am = max(am, max(max(w.x & 0x7FFFu, w.x >> 16 & 0x7FFFu), max(w.y & 0x7FFFu, w.y >> 16 & 0x7FFFu)));
      am = max(am, max(max(w.z & 0x7FFFu, w.z >> 16 & 0x7FFFu), max(w.w & 0x7FFFu, w.w >> 16 & 0x7FFFu)));
    }
    am = max(am, (uint32_t)__shfl_xor((int)am, 16));
    am = max(am, (uint32_t)__shfl_xor((int)am, 32));
    sc = scale_from_amax(__uint_as_float(am << 16), g.eps, g.ue8m0 != 0);
    const float rc = 1.0f / sc;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const u32x4 w = xr[c];
      op[2 * c] = (int)encode4_q(div_by_scale(bf16_lo(w.x), sc, rc), div_by_scale(bf16_hi(w.x), sc, rc),
                               div_by_scale(bf16_lo(w.y), sc, rc), div_by_scale(bf16_hi(w.y), sc, rc));
      op[2 * c + 1] = (int)encode4_q(div_by_scale(bf16_lo(w.z), sc, rc), div_by_scale(bf16_hi(w.z), sc, rc),
                                   div_by_scale(bf16_lo(w.w), sc, rc), div_by_scale(bf16_hi(w.w), sc, rc));
    }
  };
  // lean: quantize this lane's 2 FQ values, stage the codes and the scale in
  // the wave's LDS tile, read back this lane's operand row and its scale
  auto lean_operand = [&](const u32x4 (&xl)[LEAN && FQ == 8 ? 2 : 1], v8i& op, float& sc) {
    constexpr int NW = EPL / 2;  // 32-bit words of bf16 pairs
    uint32_t wd[NW];
#pragma unroll
    for (int i = 0; i < NW; ++i) wd[i] = xl[i >> 2][i & 3];
    uint32_t am = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) am = max(am, max(wd[i] & 0x7FFFu, wd[i] >> 16 & 0x7FFFu));
    // maximum over the LPT lanes of this token: DPP inside 16-lane rows,
    // then across rows through scalar reads of one lane per row
    am = max(am, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)am, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
    am = max(am, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)am, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
    am = max(am, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)am, 0x141, 0xF, 0xF, false));  // row_half_mirror
    if (LPT >= 16) am = max(am, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)am, 0x140, 0xF, 0xF, false));  // row_mirror
    if (LPT == 32) {
      const uint32_t r0 = max((uint32_t)__builtin_amdgcn_readlane((int)am, 0), (uint32_t)__builtin_amdgcn_readlane((int)am, 16));
      const uint32_t r1 = max((uint32_t)__builtin_amdgcn_readlane((int)am, 32), (uint32_t)__builtin_amdgcn_readlane((int)am, 48));
      am = lane < 32 ? r0 : r1;
    } else if (LPT == 64) {
      am = max(max((uint32_t)__builtin_amdgcn_readlane((int)am, 0), (uint32_t)__builtin_amdgcn_readlane((int)am, 16)),
               max((uint32_t)__builtin_amdgcn_readlane((int)am, 32), (uint32_t)__builtin_amdgcn_readlane((int)am, 48)));
    }
    const float s_own = scale_from_amax(__uint_as_float(am << 16), g.eps, g.ue8m0 != 0);
    const float rc = 1.0f / s_own;
    uint32_t code[NW / 2 > 0 ? NW / 2 : 1];
    if (NW == 1) {
      code[0] = encode4_q(div_by_scale(bf16_lo(wd[0]), s_own, rc), div_by_scale(bf16_hi(wd[0]), s_own, rc), 0.f, 0.f);
    } else {
#pragma unroll
      for (int i = 0; i < NW / 2; ++i)
        code[i] = encode4_q(div_by_scale(bf16_lo(wd[2 * i]), s_own, rc), div_by_scale(bf16_hi(wd[2 * i]), s_own, rc),
                          div_by_scale(bf16_lo(wd[2 * i + 1]), s_own, rc),
                          div_by_scale(bf16_hi(wd[2 * i + 1]), s_own, rc));
    }
    uint8_t* dst = xq + lt * 128 + lp * EPL;
    if (FQ == 1) {
      *(uint16_t*)dst = (uint16_t)code[0];
    } else if (FQ == 2) {
      *(uint32_t*)dst = code[0];
    } else if (FQ == 4) {
      *(uint2*)dst = make_uint2(code[0], code[NW / 2 > 1 ? 1 : 0]);
    } else {
      *(u32x4*)dst = u32x4{code[0], code[NW / 2 > 1 ? 1 : 0], code[NW / 2 > 2 ? 2 : 0], code[NW / 2 > 3 ? 3 : 0]};
    }
    if (lp == 0) *(float*)(xq + 2048 + lt * 4) = s_own;
    __builtin_amdgcn_wave_barrier();
    op = make_v8i(*(const u32x4*)(xq + row * 128 + kq), *(const u32x4*)(xq + row * 128 + kq + 64));
    sc = *(const float*)(xq + 2048 + row * 4);
    __builtin_amdgcn_wave_barrier();
  };
  auto comp = [&](const Batch& b) {
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      v8i xo[TOKT];
      float gs[TOKT];
#pragma unroll
      for (int t = 0; t < TOKT; ++t) {
        if constexpr (LEAN) {
          float sc;
          lean_operand(b.xl[u], xo[t], sc);
          gs[t] = sc * b.swv[u];
        } else if constexpr (FUSED) {
          float sc;
          quant_operand(b.xr[u][t], xo[t], sc);
          gs[t] = sc * b.swv[u];
        } else {
          xo[t] = b.xf[u][t];
          gs[t] = b.gsc[u][t];
        }
      }
#pragma unroll
      for (int r = 0; r < RN; ++r)
#pragma unroll
        for (int t = 0; t < TOKT; ++t) {
          const v4f P = mfma16x16x128(b.wf[u][r], xo[t]);
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[r][t][q] = __builtin_fmaf(P[q], gs[t], acc[r][t][q]);
        }
    }
  };
  Batch b0, b1;
  load(b0, kb0);
  for (int kb = kb0; kb < kb1; kb += 2 * UNR) {
    const bool more1 = kb + UNR < kb1;  // wave-uniform
    if (more1) load(b1, kb + UNR);
    __builtin_amdgcn_sched_barrier(0);
    comp(b0);
    __builtin_amdgcn_sched_barrier(0);
    if (!more1) break;
    if (kb + 2 * UNR < kb1) load(b0, kb + 2 * UNR);
    __builtin_amdgcn_sched_barrier(0);
    comp(b1);
    __builtin_amdgcn_sched_barrier(0);
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
        if (CH) {
          const float sam = g.sa[m];
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = v[q] * sam * g.sw[n + q];
        }
        if (SPLIT)
          *(float4*)(g.ws + ((int64_t)split * g.M + m) * g.N + n) = make_float4(v[0], v[1], v[2], v[3]);
        else
          *(uint2*)(g.y + m * g.ldy + n) =
              make_uint2(bf16x2_bits(v[0], v[1]),
                         bf16x2_bits(v[2], v[3]));
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
          v4f v = acc[r][t];
          if (CH) {
            const float sam = g.sa[m];
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = v[q] * sam * g.sw[n + q];
          }
          if (SPLIT)
            *(float4*)(g.ws + ((int64_t)split * g.M + m) * g.N + n) = make_float4(v[0], v[1], v[2], v[3]);
          else
            *(uint2*)(g.y + m * g.ldy + n) =
                make_uint2(bf16x2_bits(v[0], v[1]),
                           bf16x2_bits(v[2], v[3]));
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
    *(uint2*)(y + m * ldy + n) = make_uint2(bf16x2_bits(acc.x, acc.y),
                                            bf16x2_bits(acc.z, acc.w));
  }
}

template <int TOKT, int RN, int FQ, bool CH = false>
hipError_t run_swap3(const SwapParams& p, dim3 grid, int kwaves, bool split, hipStream_t stream) {
  if (split)
    hipLaunchKernelGGL((k_gemm_swapab<TOKT, RN, true, FQ, CH>), grid, dim3(64 * kwaves), 0, stream, p);
  else
    hipLaunchKernelGGL((k_gemm_swapab<TOKT, RN, false, FQ, CH>), grid, dim3(64 * kwaves), 0, stream, p);
  return hipGetLastError();
}

template <int TOKT, int RN>
hipError_t run_swap(const GemmArgs& g, int kwaves, int split_k, bool ch, hipStream_t stream) {
  SwapParams p;
  p.g = g;
  p.kb_total = (int)(g.K / 128);
  p.kb_per_split = (p.kb_total + split_k - 1) / split_k;
  dim3 grid((unsigned)(g.N / (16 * RN)), (unsigned)split_k);
  const bool sp = split_k > 1;
  if (ch) return run_swap3<TOKT, RN, 0, true>(p, grid, kwaves, sp, stream);
  if (g.x == nullptr) return run_swap3<TOKT, RN, 0>(p, grid, kwaves, sp, stream);
  if constexpr (TOKT == 1) {  // fused: quantize only the tokens that can be valid
    if (g.M <= 1) return run_swap3<TOKT, RN, 1>(p, grid, kwaves, sp, stream);
    if (g.M <= 2) return run_swap3<TOKT, RN, 2>(p, grid, kwaves, sp, stream);
    if (g.M <= 4) return run_swap3<TOKT, RN, 4>(p, grid, kwaves, sp, stream);
    if (g.M <= 8) return run_swap3<TOKT, RN, 8>(p, grid, kwaves, sp, stream);
    return run_swap3<TOKT, RN, 16>(p, grid, kwaves, sp, stream);
  } else if constexpr (TOKT == 2 || RN == 1) {
    return run_swap3<TOKT, RN, 16>(p, grid, kwaves, sp, stream);
  }
  // four token tiles fuse only with 16 weight rows per workgroup: with more,
  // the raw activations and the weight fragments exceed the registers
  return hipErrorInvalidValue;
}

}  // namespace

bool swapab_tile_supported(int tile_m, int tile_n, int kwaves) {
  const bool tm = tile_m == 16 || tile_m == 32 || tile_m == 64;
  const bool tn = tile_n == 16 || tile_n == 32 || (tile_n == 64 && tile_m <= 32);
  const bool kwv = kwaves == 1 || kwaves == 2 || kwaves == 4 || kwaves == 8;
  return tm && tn && kwv;
}

hipError_t launch_gemm_swapab(const GemmArgs& g, int tile_m, int tile_n, int kwaves, int split_k,
                              hipStream_t stream, bool channel_scales) {
  const int tokt = tile_m / 16, rn = tile_n / 16;
  hipError_t e = hipErrorInvalidValue;
#define FP8BLK_SWAP_CASE(T, R) \
  if (tokt == T && rn == R) e = run_swap<T, R>(g, kwaves, split_k, channel_scales, stream);
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
