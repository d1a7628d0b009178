// fused.hip -- the producers of the GEMM's activation operand, fused with
// the 1x128 group quantizer, for gfx950:
//   rms_norm_per_block_quant      RMSNorm, then group quantization
//   silu_and_mul_per_block_quant  SiLU(gate) * up, then group quantization
// (page "Helion-Kernel in vLLM: PyTorch FP8 ohne CUDA", section "Welche
// Kernel wurden in vLLM integriert"; page "[RFC]: Using Helion for Selected
// vLLM CustomOps", section "Motivation").
//
// Both are HBM-bound streams (RMSNorm: 2 bytes in, 1 + 4/128 out per
// element; SiLU-and-mul: 4 in, 1 + 4/128 out).  A 128-group is owned by 8
// lanes holding 16 contiguous values each (16 lanes of 8 where the row
// length does not allow it), the group amax reduced with DPP inside the
// lanes' DPP row, the scale and its float64 reciprocal computed once per
// group, every fp32 value divided by the scale as IEEE division would (a
// float64 product rounded to fp32: three instructions), two values per fp8
// convert.
//
// RMSNorm (the fp8 RMSNorm example of the Chinese Helion article, section
// "自己写一个 Helion kernel 并接入 vLLM": variance = mean of squares,
// rms = sqrt(variance + eps), y = x / rms * weight):
//   - a row is spread over one, two or four waves and held in registers, so
//     the normalization pass costs no second HBM read;
//   - the sum of squares is accumulated in fp64 (every square of a bf16
//     value is exact there), then 1/sqrt(variance + eps) in fp64 with
//     correctly rounded sqrt and division, rounded once to fp32;
//   - y = (x * (1/rms)) * weight in fp32, quantized straight from fp32
//     (no bf16 rounding in between).
//   Rows are walked grid-stride and the next row is loaded while the
//   current one is reduced and quantized.
//
// SiLU-and-mul: x row = [gate (I values) | up (I values)]; y = silu(g) * u
// from a float64 product with a correctly rounded float64 logistic table,
// rounded once to fp32 and quantized from fp32.
#include "device_common.hpp"
#include "launch.hpp"

#pragma clang fp contract(off)

namespace fp8blk {
namespace {

// Stores the scale of group `col` of row `row` in the requested layout:
// bit 0 of fmt = MN-major ([H/128][lds]), bit 1 = one E8M0 byte per scale.
__device__ __forceinline__ void store_scale(void* s, int fmt, int64_t lds, int64_t row, int64_t col,
                                            float sc) {
  const int64_t o = (fmt & 1) ? col * lds + row : row * lds + col;
  if (fmt & 2)
    ((uint8_t*)s)[o] = (uint8_t)(__float_as_uint(sc) >> 23);
  else
    ((float*)s)[o] = sc;
}

// Group quantization of 8 fp32 values per lane, 16 lanes per group (one DPP
// row): amax, scale, codes.  Returns the 8 codes; *sc_out gets the scale.
// The values are results of fp32 arithmetic (canonical, finite), so their
// magnitudes are compared as floats.
__device__ __forceinline__ uint2 quant8(const float (&y)[8], float eps, bool ue8m0, float* sc_out) {
  float m = fmaxf(fmaxf(fabsf(y[0]), fabsf(y[1])), fmaxf(fabsf(y[2]), fabsf(y[3])));
  m = fmaxf(m, fmaxf(fmaxf(fabsf(y[4]), fabsf(y[5])), fmaxf(fabsf(y[6]), fabsf(y[7]))));
  const uint32_t am = row16_max_u32(__float_as_uint(m));
  const float sc = scale_from_amax(__uint_as_float(am), eps, ue8m0);
  const double d = recip_f64(sc);
  *sc_out = sc;
  const uint32_t lo = encode4_q(div_by_scale_f64(y[0], d), div_by_scale_f64(y[1], d),
                                div_by_scale_f64(y[2], d), div_by_scale_f64(y[3], d));
  const uint32_t hi = encode4_q(div_by_scale_f64(y[4], d), div_by_scale_f64(y[5], d),
                                div_by_scale_f64(y[6], d), div_by_scale_f64(y[7], d));
  return make_uint2(lo, hi);
}

// Maximum over the 8 lanes of each half DPP row (lanes 8k .. 8k+7).
__device__ __forceinline__ uint32_t row8_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));  // quad_perm 1,0,3,2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));  // quad_perm 2,3,0,1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false)); // row_half_mirror
  return v;
}

// quant8 for 16 values per lane and 8 lanes per group: the per-group work
// (amax reduction, scale, reciprocal) is shared by twice as many values.
__device__ __forceinline__ u32x4 quant16(const float (&y)[16], float eps, bool ue8m0, float* sc_out) {
  float m[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
    m[k] = fmaxf(fmaxf(fabsf(y[4 * k]), fabsf(y[4 * k + 1])), fmaxf(fabsf(y[4 * k + 2]), fabsf(y[4 * k + 3])));
  const uint32_t am = row8_max_u32(__float_as_uint(fmaxf(fmaxf(m[0], m[1]), fmaxf(m[2], m[3]))));
  const float sc = scale_from_amax(__uint_as_float(am), eps, ue8m0);
  const double d = recip_f64(sc);
  *sc_out = sc;
  u32x4 c;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    c[k] = encode4_q(div_by_scale_f64(y[4 * k], d), div_by_scale_f64(y[4 * k + 1], d),
                     div_by_scale_f64(y[4 * k + 2], d), div_by_scale_f64(y[4 * k + 3], d));
  return c;
}

// 64-bit DPP move of a double (each 32-bit half moved with the same control).
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, 0xF, 0xF, false);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ double readlane_f64(double v, int l) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), l);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Sum over the 64 lanes, the same value in every lane: DPP inside each
// 16-lane row (quad swaps, half-row and row mirrors), then the four row sums
// read out and added in a fixed order.
__device__ __forceinline__ double wave_sum_f64(double v) {
  v += dpp_f64<0xB1>(v);   // quad_perm 1,0,3,2
  v += dpp_f64<0x4E>(v);   // quad_perm 2,3,0,1
  v += dpp_f64<0x141>(v);  // row_half_mirror
  v += dpp_f64<0x140>(v);  // row_mirror
  return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}

// ---------------------------------------------------------------- RMSNorm
//
// WPR waves per row (1, 2 or 4; 4 / WPR rows per workgroup), VPL vectors of
// 8 values per lane (placement in rms_elem: with an even VPL a lane holds 16
// consecutive values of one group, so a group's amax, scale and reciprocal
// are shared by 16 values per lane instead of 8).  A row covers
// WPR * 512 * VPL elements; FULL when that is exactly H, else groups past H
// are masked (the lanes of a group agree).  Workgroups walk their row slots grid-stride (one round of
// resident workgroups), the next rows' loads issued before the current rows
// are reduced and quantized (two register buffers used in turn), so HBM
// reads overlap the arithmetic.  The walk is uniform over the workgroup
// (its barriers); waves whose row is past M compute on a copy of the last
// row and store nothing.
// Loads one row's vectors.  Loads are never predicated (so the compiler can
// count them and wait for exactly the ones it needs): a row past M reads the
// last row instead, and in masked shapes a vector past H reads the row's
// last vector and is then zeroed.
// First element of vector i of wave wv (of its row), lane `lane`.  Even VPL:
// vectors go in pairs and lane l of pair p holds the 16 consecutive values
// 16 * ((p * WPR + wv) * 64 + l) .. +16 (8 lanes per group; the two loads of
// a pair read 16-byte pieces 32 bytes apart, together a contiguous 2 KiB).
// Odd VPL: lane l of vector i holds 8 values, 16 lanes per group.
template <int VPL, int WPR>
__device__ __forceinline__ int rms_elem(int i, int wv, int lane) {
  if constexpr (VPL % 2 == 0)
    return 16 * (((i >> 1) * WPR + wv) * 64 + lane) + 8 * (i & 1);
  else
    return 8 * ((i * WPR + wv) * 64 + lane);
}

template <int VPL, int WPR, bool FULL>
__device__ __forceinline__ void rms_load_row(u32x4 (&v)[VPL], const uint16_t* x, int64_t ldx, int64_t row,
                                             int64_t M, int wv, int lane, int H) {
  const uint16_t* xr = x + (row < M ? row : M - 1) * ldx;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = rms_elem<VPL, WPR>(i, wv, lane);
    if (FULL) {
      v[i] = load16(xr + e);
    } else {
      const u32x4 t = load16(xr + (e < H ? e : H - 8));
      v[i] = e < H ? t : u32x4{0u, 0u, 0u, 0u};
    }
  }
}

// WL: the weight is staged once per workgroup in LDS (rows up to 8192
// values), so the row loop issues no global loads besides the rows' own.
template <int VPL, int WPR, bool FULL>
__global__ __launch_bounds__(256) void k_rms_norm_quant(
    const uint16_t* __restrict__ x, int64_t ldx, const float* __restrict__ w, uint8_t* __restrict__ q,
    int64_t ldq, void* __restrict__ s, int64_t lds, int64_t M, int H, float eps_norm, float eps,
    int ue8m0, int fmt) {
  constexpr int kCover = VPL * WPR * 512;
  constexpr bool WL = kCover <= 8192;
  constexpr int VPU = VPL % 2 == 0 ? 2 : 1;  // vectors per group share of a lane
  constexpr int NU = VPL / VPU;              // group shares per lane and row
  constexpr int LPG = 16 / VPU;              // lanes per group
  __shared__ double red[2][4];
  __shared__ float4 wl[WL ? kCover / 4 : 1];
  constexpr int kRowsPerBlock = 4 / WPR;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int slot = wave / WPR;  // row slot of this wave in the workgroup
  const int wv = wave % WPR;    // this wave's part of the row
  const int ngroups = H / kGroup;
  const int64_t rstep = (int64_t)gridDim.x * kRowsPerBlock;
  int64_t base = (int64_t)blockIdx.x * kRowsPerBlock;
  if (base >= M) return;  // uniform over the workgroup

  u32x4 va[VPL], vb[VPL];
  rms_load_row<VPL, WPR, FULL>(va, x, ldx, base + slot, M, wv, lane, H);
  if (WL) {
    for (int i = threadIdx.x; i < H / 4; i += 256) wl[i] = ((const float4*)w)[i];
    __syncthreads();
  }

  auto process = [&](const u32x4(&v)[VPL], int64_t row, int it) __attribute__((always_inline)) {
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const uint32_t c[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const double a = (double)bf16_lo(c[k]), b = (double)bf16_hi(c[k]);
        ss = __builtin_fma(a, a, ss);
        ss = __builtin_fma(b, b, ss);
      }
    }
    ss = wave_sum_f64(ss);
    if (WPR > 1) {
      // two buffers: a wave overwrites one only after every wave has passed
      // the barrier of the iteration in between
      if (lane == 0) red[it & 1][wave] = ss;
      __syncthreads();
      const double* rr = &red[it & 1][slot * WPR];
      ss = WPR == 2 ? rr[0] + rr[1] : (rr[0] + rr[1]) + (rr[2] + rr[3]);
    }
    if (row >= M) return;
    const float r = (float)(1.0 / __builtin_sqrt(ss / (double)H + (double)eps_norm));
    uint8_t* qr = q + row * ldq;
    auto weight4 = [&](int e) __attribute__((always_inline)) -> float4 {
      return WL ? wl[e / 4] : *(const float4*)(w + e);
    };
    // scales are kept and stored together after the row (one masked region)
    float scs[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int e = rms_elem<VPL, WPR>(u * VPU, wv, lane);
      scs[u] = 0.f;
      if (!FULL && (e >> 7) >= ngroups) continue;  // the lanes of a group agree
      if constexpr (VPU == 2) {
        const float4 w0 = weight4(e), w1 = weight4(e + 4), w2 = weight4(e + 8), w3 = weight4(e + 12);
        const float wj[16] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w,
                              w2.x, w2.y, w2.z, w2.w, w3.x, w3.y, w3.z, w3.w};
        const uint32_t c[8] = {v[2 * u].x, v[2 * u].y, v[2 * u].z, v[2 * u].w,
                               v[2 * u + 1].x, v[2 * u + 1].y, v[2 * u + 1].z, v[2 * u + 1].w};
        float y[16];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          y[2 * k] = (bf16_lo(c[k]) * r) * wj[2 * k];
          y[2 * k + 1] = (bf16_hi(c[k]) * r) * wj[2 * k + 1];
        }
        *(u32x4*)(qr + e) = quant16(y, eps, ue8m0 != 0, &scs[u]);
      } else {
        const float4 w0 = weight4(e), w1 = weight4(e + 4);
        const float wj[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
        const uint32_t c[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
        float y[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          y[2 * k] = (bf16_lo(c[k]) * r) * wj[2 * k];
          y[2 * k + 1] = (bf16_hi(c[k]) * r) * wj[2 * k + 1];
        }
        *(uint2*)(qr + e) = quant8(y, eps, ue8m0 != 0, &scs[u]);
      }
    }
    if ((lane & (LPG - 1)) == 0) {
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int g = rms_elem<VPL, WPR>(u * VPU, wv, lane) >> 7;
        if (FULL || g < ngroups) store_scale(s, fmt, lds, row, g, scs[u]);
      }
    }
  };

  for (int it = 0;; it += 2) {
    int64_t nbase = base + rstep;
    rms_load_row<VPL, WPR, FULL>(vb, x, ldx, nbase + slot, M, wv, lane, H);
    process(va, base + slot, it);
    base = nbase;
    if (base >= M) break;
    nbase = base + rstep;
    rms_load_row<VPL, WPR, FULL>(va, x, ldx, nbase + slot, M, wv, lane, H);
    process(vb, base + slot, it + 1);
    base = nbase;
    if (base >= M) break;
  }
}

int cu_count() {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      cus = v;
  }
  return cus;
}


// Workgroups of an RMSNorm kernel instance that fit the device at once
// (occupancy x CUs), queried once per instance (the devices this library
// runs on are all the same part).
template <int VPL, int WPR, bool FULL>
int rms_resident_blocks() {
  static const int cached = [] {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_rms_norm_quant<VPL, WPR, FULL>, 256, 0) !=
            hipSuccess ||
        per_cu < 1)
      per_cu = 1;
    return per_cu * cu_count();
  }();
  return cached;
}

template <int VPL, int WPR, bool FULL>
hipError_t launch_rms(const uint16_t* x, int64_t ldx, const float* w, uint8_t* q, int64_t ldq, void* s,
                      int64_t lds, int64_t M, int H, float eps_norm, float eps, int ue8m0, int fmt,
                      hipStream_t stream) {
  constexpr int rpb = 4 / WPR;
  int64_t blocks = (M + rpb - 1) / rpb;
  // persistent: one round of resident workgroups, each walking its row slots
  const int max_blocks = rms_resident_blocks<VPL, WPR, FULL>();
  if (blocks > max_blocks) blocks = max_blocks;
  hipLaunchKernelGGL((k_rms_norm_quant<VPL, WPR, FULL>), dim3((unsigned)blocks), dim3(256), 0, stream, x,
                     ldx, w, q, ldq, s, lds, M, H, eps_norm, eps, ue8m0, fmt);
  return hipGetLastError();
}

// ------------------------------------------------------------ SiLU and mul
//
// 8 lanes per group and 16 consecutive values per lane (two 16-byte loads
// 16 bytes apart per operand, one 16-byte code store), so a group's amax
// reduction, scale and reciprocal are shared by 16 values; U groups per
// 8-lane slot in flight (two on the LDS-table path, one on the small-problem
// path, which needs its workgroups more than its registers) (group k of a slot is base + k * slots +
// slot).  Against 16 lanes of 8 values: 13 % fewer VALU instructions and
// half the store instructions, 4-5 % faster at the Qwen3-8B/32B sizes.
// Groups are numbered row-major over (row, group column) and split into chunks of
// fewer than 2^24 groups so that row = (g * ceil(2^40 / gpr)) >> 40 is exact.
// Grid-stride over the groups, the next iteration's loads issued before the
// current groups are computed.
//
// The logistic function comes from a table of t(a) = 1 / (1 + e^a) for
// every bf16 magnitude a, correctly rounded to float64 (sigmoid_table.inc):
// s(g) = t(|g|) for g <= 0 and 1 - t(|g|) for g > 0, and y = (g u) s(g) in
// float64 (g u exact there), rounded once to float32.  The float64 value is
// within 2^-51 (relative) of the exact silu(g) u, so the float32 y is the
// correctly rounded one except next to a rounding midpoint.  Large problems
// copy the table (61 KB) into LDS once per workgroup (TAB); small ones,
// where that copy would not pay, read it from global memory (L2).
constexpr int kSiluUnrollTab = 2;  // U on the LDS-table path
constexpr int kSiluLanes = 8;

#include "sigmoid_table.inc"

// silu(g) * u for the gate and up values widened to fp32 (gb: the gate's
// fp32 bits).  With q = |g| u (exact in float64) and c = 1 for a positive
// sign bit, 0 for a negative one: s(g) = c - t(|g|) for g > 0 and
// -(c - t) = t for g < 0, so silu(g) u = g u s(g) = q (c - t) in both cases,
// with one float64 subtraction (exact for g < 0), one product and one
// rounding to fp32.  Signed zeros come out right as well: g = +0 gives
// q (1 - 1/2), g = -0 gives q (0 - 1/2), i.e. the sign of g u.
__device__ __forceinline__ float silu_mul64(uint32_t gb, float g, float u, const double* tab) {
  const uint32_t mag = (gb >> 16) & 0x7FFFu;
  const uint32_t i = min(max(mag, (uint32_t)kSigmoidBase), (uint32_t)(kSigmoidBase + kSigmoidSpan - 1));
  const double t = tab[i - (uint32_t)kSigmoidBase];
  const uint32_t c_hi = (int32_t)gb < 0 ? 0u : 0x3FF00000u;  // 1.0 or 0.0
  const double c = __builtin_bit_cast(double, (uint64_t)c_hi << 32);
  const double q = __builtin_fabs((double)g) * (double)u;
  return (float)(q * (c - t));
}

// One iteration's inputs for U groups per 8-lane slot, with each
// group's row, column and offset in q (32-bit offsets: a launch covers
// fewer than 2^31 elements of x and of q).
template <int U>
struct SiluFrag {
  u32x4 gv[U][2], uv[U][2];
  uint32_t qo[U];
  uint32_t row[U], col[U];
};

// Group k of a lane is base + k * NS + slot (NS = 8-lane slots per
// workgroup), so one iteration covers NS * U consecutive groups.
template <uint32_t NS, int U>
__device__ __forceinline__ void silu_load(SiluFrag<U>& f, const uint16_t* __restrict__ x, uint32_t ldx,
                                          uint32_t ldq, uint32_t base, uint32_t slot, uint32_t sub,
                                          uint32_t total, uint32_t gpr, uint64_t magic, uint32_t I) {
#pragma unroll
  for (int k = 0; k < U; ++k) {
    // groups past the end load the last group again (in bounds, unused:
    // their stores are skipped), which keeps the loads unpredicated
    const uint32_t g = min(base + k * NS + slot, total - 1u);
    const uint32_t row = (uint32_t)(((uint64_t)g * magic) >> 40);
    const uint32_t col = g - row * gpr;
    f.row[k] = row;
    f.col[k] = col;
    const uint32_t xo = row * ldx + col * kGroup + sub * 16;  // elements
    f.qo[k] = row * ldq + col * kGroup + sub * 16;
    f.gv[k][0] = load_nt16((const char*)x + 2u * xo);
    f.gv[k][1] = load_nt16((const char*)x + 2u * (xo + 8));
    f.uv[k][0] = load_nt16((const char*)x + 2u * (xo + I));
    f.uv[k][1] = load_nt16((const char*)x + 2u * (xo + I + 8));
  }
}

template <uint32_t NS, int U>
__device__ __forceinline__ void silu_compute_store(const SiluFrag<U>& f, uint32_t base, uint32_t slot,
                                                   uint32_t sub, uint32_t total, const double* tab,
                                                   uint8_t* __restrict__ q, void* __restrict__ s,
                                                   int64_t lds, int64_t row0, float eps, int ue8m0,
                                                   int fmt) {
#pragma unroll
  for (int k = 0; k < U; ++k) {
    const uint32_t g = base + k * NS + slot;
    const uint32_t gc[8] = {f.gv[k][0].x, f.gv[k][0].y, f.gv[k][0].z, f.gv[k][0].w,
                            f.gv[k][1].x, f.gv[k][1].y, f.gv[k][1].z, f.gv[k][1].w};
    const uint32_t uc[8] = {f.uv[k][0].x, f.uv[k][0].y, f.uv[k][0].z, f.uv[k][0].w,
                            f.uv[k][1].x, f.uv[k][1].y, f.uv[k][1].z, f.uv[k][1].w};
    float y[16];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float g0 = bf16_lo(gc[j]), g1 = bf16_hi(gc[j]);
      y[2 * j] = silu_mul64(__float_as_uint(g0), g0, bf16_lo(uc[j]), tab);
      y[2 * j + 1] = silu_mul64(__float_as_uint(g1), g1, bf16_hi(uc[j]), tab);
    }
    float sc;
    const u32x4 codes = quant16(y, eps, ue8m0 != 0, &sc);
    if (g < total) {
      *(u32x4*)(q + f.qo[k]) = codes;
      if (sub == 0) store_scale(s, fmt, lds, row0 + f.row[k], f.col[k], sc);
    }
  }
}

// x and q point at the launch's first row; row0 is that row's index (for
// the scales).
template <bool TAB, int NT>
__global__ __launch_bounds__(NT) void k_silu_mul_quant(
    const uint16_t* __restrict__ x, uint32_t ldx, uint8_t* __restrict__ q, uint32_t ldq,
    void* __restrict__ s, int64_t lds, int64_t row0, uint32_t total, uint32_t gpr, uint64_t magic,
    uint32_t I, float eps, int ue8m0, int fmt) {
  constexpr uint32_t kSlots = NT / kSiluLanes;
  constexpr int U = TAB ? kSiluUnrollTab : 1;
  constexpr uint32_t kPerIter = kSlots * U;
  __shared__ double lds_tab[TAB ? kSigmoidSpan : 1];
  const double* tab = TAB ? lds_tab : kSigmoidTable;
  const uint32_t sub = threadIdx.x & (kSiluLanes - 1u);
  const uint32_t slot = threadIdx.x / kSiluLanes;
  const uint32_t step = gridDim.x * kPerIter;
  uint32_t base = blockIdx.x * kPerIter;
  if (base >= total) return;  // uniform over the workgroup
  SiluFrag<U> fa, fb;
  silu_load<kSlots, U>(fa, x, ldx, ldq, base, slot, sub, total, gpr, magic, I);
  if (TAB) {
    for (int i = threadIdx.x; i < kSigmoidSpan; i += NT) lds_tab[i] = kSigmoidTable[i];
    __syncthreads();
  }
  // two fragments used in turn: the loads of one are in flight while the
  // other is computed (total + step < 2^26: no wrap)
  for (;;) {
    uint32_t nb = base + step;
    if (nb < total) silu_load<kSlots, U>(fb, x, ldx, ldq, nb, slot, sub, total, gpr, magic, I);
    silu_compute_store<kSlots, U>(fa, base, slot, sub, total, tab, q, s, lds, row0, eps, ue8m0, fmt);
    base = nb;
    if (base >= total) break;
    nb = base + step;
    if (nb < total) silu_load<kSlots, U>(fa, x, ldx, ldq, nb, slot, sub, total, gpr, magic, I);
    silu_compute_store<kSlots, U>(fb, base, slot, sub, total, tab, q, s, lds, row0, eps, ue8m0, fmt);
    base = nb;
    if (base >= total) break;
  }
}

}  // namespace

hipError_t launch_rms_norm_quant(const uint16_t* x, int64_t M, int64_t H, int64_t ldx, const float* w,
                                 float eps_norm, uint8_t* q, int64_t ldq, void* s, int64_t lds,
                                 float eps, bool ue8m0, int scale_format, hipStream_t stream) {
  const int h = (int)H;
  const int u = ue8m0 ? 1 : 0;
  // one launch covers at most 2^31 - 1 workgroups; rows beyond go in chunks
  const int64_t chunk = int64_t(1) << 30;
  for (int64_t r0 = 0; r0 < M; r0 += chunk) {
    const int64_t rows = (M - r0) < chunk ? (M - r0) : chunk;
    const uint16_t* xr = x + r0 * ldx;
    uint8_t* qr = q + r0 * ldq;
    const int64_t selt = (scale_format & 2) ? 1 : 4;
    void* sr = (char*)s + ((scale_format & 1) ? r0 : r0 * lds) * selt;
    hipError_t e;
    // Many rows (more than fill the GPU with one wave each): exact fits for H
    // a multiple of 512 with one wave per row up to 4096 values, two waves up
    // to 8192, four beyond, at most 8 vectors per lane (two rows in registers
    // at 3 or more waves per SIMD).  Few rows (decode): four waves per row
    // where H allows (each row's latency chain is then a quarter as long:
    // 3.3 us instead of 5.4 us for one 4096-value row), else two.  Other H
    // (multiples of 128): masked shapes that round the row up.
#define FP8BLK_RMS(V, W, F) launch_rms<V, W, F>(xr, ldx, w, qr, ldq, sr, lds, rows, h, eps_norm, eps, u, scale_format, stream)
    const bool few = rows <= 1024;
    const int c512 = H % 512 == 0 ? (int)(H / 512) : 0;
    const int c2048 = H % 2048 == 0 ? (int)(H / 2048) : 0;
    const int c1024 = H % 1024 == 0 ? (int)(H / 1024) : 0;
    if (few && c2048 >= 1 && c2048 <= 8) {
      switch (c2048) {
        case 1: e = FP8BLK_RMS(1, 4, true); break;
        case 2: e = FP8BLK_RMS(2, 4, true); break;
        case 3: e = FP8BLK_RMS(3, 4, true); break;
        case 4: e = FP8BLK_RMS(4, 4, true); break;
        case 5: e = FP8BLK_RMS(5, 4, true); break;
        case 6: e = FP8BLK_RMS(6, 4, true); break;
        case 7: e = FP8BLK_RMS(7, 4, true); break;
        default: e = FP8BLK_RMS(8, 4, true); break;
      }
    } else if (few && c1024 >= 5 && c1024 <= 8 && c2048 == 0) {
      switch (c1024) {
        case 5: e = FP8BLK_RMS(5, 2, true); break;
        default: e = FP8BLK_RMS(7, 2, true); break;
      }
    } else {
      switch (c512) {
        case 1: e = FP8BLK_RMS(1, 1, true); break;
        case 2: e = FP8BLK_RMS(2, 1, true); break;
        case 3: e = FP8BLK_RMS(3, 1, true); break;
        case 4: e = FP8BLK_RMS(4, 1, true); break;
        case 5: e = FP8BLK_RMS(5, 1, true); break;
        case 6: e = FP8BLK_RMS(6, 1, true); break;
        case 7: e = FP8BLK_RMS(7, 1, true); break;
        case 8: e = FP8BLK_RMS(8, 1, true); break;
        case 10: e = FP8BLK_RMS(5, 2, true); break;
        case 12: e = FP8BLK_RMS(6, 2, true); break;
        case 14: e = FP8BLK_RMS(7, 2, true); break;
        case 16: e = FP8BLK_RMS(8, 2, true); break;
        case 20: e = FP8BLK_RMS(5, 4, true); break;
        case 24: e = FP8BLK_RMS(6, 4, true); break;
        case 28: e = FP8BLK_RMS(7, 4, true); break;
        case 32: e = FP8BLK_RMS(8, 4, true); break;
        case 64: e = FP8BLK_RMS(16, 4, true); break;
        default:
          if (H <= 1024) e = FP8BLK_RMS(2, 1, false);
          else if (H <= 4096) e = FP8BLK_RMS(8, 1, false);
          else if (H <= 8192) e = FP8BLK_RMS(8, 2, false);
          else if (H <= 16384) e = FP8BLK_RMS(8, 4, false);
          else e = FP8BLK_RMS(16, 4, false);
      }
    }
#undef FP8BLK_RMS
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_silu_mul_quant(const uint16_t* x, int64_t M, int64_t I, int64_t ldx, uint8_t* q,
                                 int64_t ldq, void* s, int64_t lds, float eps, bool ue8m0,
                                 int scale_format, hipStream_t stream) {
  const int64_t gpr = I / kGroup;
  // chunks of rows: fewer than 2^24 groups (exact row division) and fewer
  // than 2^31 elements of x and of q (32-bit offsets)
  const int64_t pitch = ldx > ldq ? ldx : ldq;
  int64_t rows_per_chunk = (int64_t(1) << 24) / gpr;
  const int64_t by_offset = ((int64_t(1) << 31) - 1) / pitch;
  if (rows_per_chunk > by_offset) rows_per_chunk = by_offset;
  if (rows_per_chunk < 1) rows_per_chunk = 1;
  const uint64_t magic = ((uint64_t(1) << 40) + (uint64_t)gpr - 1) / (uint64_t)gpr;
  const int cus = cu_count();
  for (int64_t r0 = 0; r0 < M; r0 += rows_per_chunk) {
    const int64_t rows = (M - r0) < rows_per_chunk ? (M - r0) : rows_per_chunk;
    const uint32_t total = (uint32_t)(rows * gpr);
    // the LDS table pays off once every resident workgroup has several
    // iterations to run (2 workgroups of 512 threads per CU: 61 KB of LDS each)
    const bool tab = total >= (uint32_t)cus * 2 * (512 / kSiluLanes) * kSiluUnrollTab * 2;
    const int nt = tab ? 512 : 256;
    const uint32_t per_iter = (uint32_t)(nt / kSiluLanes) * (tab ? kSiluUnrollTab : 1);
    int64_t blocks = (total + per_iter - 1) / per_iter;
    const int64_t max_blocks = (int64_t)cus * (tab ? 2 : 8);
    if (blocks > max_blocks) blocks = max_blocks;
    const int u = ue8m0 ? 1 : 0;
    const uint16_t* xr = x + r0 * ldx;
    uint8_t* qr = q + r0 * ldq;
    if (tab)
      hipLaunchKernelGGL((k_silu_mul_quant<true, 512>), dim3((unsigned)blocks), dim3(512), 0, stream, xr,
                         (uint32_t)ldx, qr, (uint32_t)ldq, s, lds, r0, total, (uint32_t)gpr, magic,
                         (uint32_t)I, eps, u, scale_format);
    else
      hipLaunchKernelGGL((k_silu_mul_quant<false, 256>), dim3((unsigned)blocks), dim3(256), 0, stream, xr,
                         (uint32_t)ldx, qr, (uint32_t)ldq, s, lds, r0, total, (uint32_t)gpr, magic,
                         (uint32_t)I, eps, u, scale_format);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace fp8blk
