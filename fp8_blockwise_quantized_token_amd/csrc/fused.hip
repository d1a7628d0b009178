// fused.hip -- the producers of the GEMM's activation operand, fused with
// the 1x128 group quantizer, for gfx950:
//   rms_norm_per_block_quant      RMSNorm, then group quantization
//   silu_and_mul_per_block_quant  SiLU(gate) * up, then group quantization
// (page "Helion-Kernel in vLLM: PyTorch FP8 ohne CUDA", section "Welche
// Kernel wurden in vLLM integriert"; page "[RFC]: Using Helion for Selected
// vLLM CustomOps", section "Motivation").
//
// Both are HBM-bound streams (RMSNorm: 2 bytes in, 1 + 4/128 out per
// element; SiLU-and-mul: 4 in, 1 + 4/128 out) and keep the quantizer's
// lane layout: 16 lanes own one 128-group, 8 contiguous values per lane
// loaded with one 16-byte load, the group amax reduced with DPP inside the
// 16-lane row, the scale computed once per group, every value divided with
// the 3-instruction correctly rounded division, two values per fp8 convert.
//
// RMSNorm (the fp8 RMSNorm example of the Chinese Helion article, section
// "自己写一个 Helion kernel 并接入 vLLM": variance = mean of squares,
// rms = sqrt(variance + eps), y = x / rms * weight):
//   - one wave per row: the row is read once and held in registers, so the
//     normalization pass costs no second HBM read;
//   - the sum of squares is accumulated in fp64 (every square of a bf16
//     value is exact there), then 1/sqrt(variance + eps) in fp64 with
//     correctly rounded sqrt and division, rounded once to fp32;
//   - y = (x * (1/rms)) * weight in fp32, quantized straight from fp32
//     (no bf16 rounding in between).
//   Rows longer than 8192 are split over the four waves of the workgroup,
//   whose partial sums meet in LDS.
//
// SiLU-and-mul: x row = [gate (I values) | up (I values)]; y = silu(g) * u
// = (g u) / (1 + exp(-g)) in fp32 with the library expf (within an ulp) and
// one corrected reciprocal division, quantized from fp32.
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
__device__ __forceinline__ uint2 quant8(const float (&y)[8], float eps, bool ue8m0, float* sc_out) {
  uint32_t am = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) am = max(am, __float_as_uint(y[j]) & 0x7FFFFFFFu);
  am = row16_max_u32(am);
  const float sc = scale_from_amax(__uint_as_float(am), eps, ue8m0);
  const float rc = 1.0f / sc;
  *sc_out = sc;
  const uint32_t lo = encode4(div_by_scale(y[0], sc, rc), div_by_scale(y[1], sc, rc),
                              div_by_scale(y[2], sc, rc), div_by_scale(y[3], sc, rc));
  const uint32_t hi = encode4(div_by_scale(y[4], sc, rc), div_by_scale(y[5], sc, rc),
                              div_by_scale(y[6], sc, rc), div_by_scale(y[7], sc, rc));
  return make_uint2(lo, hi);
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// ---------------------------------------------------------------- RMSNorm
//
// WPR waves per row (1 or 4), VPL vectors of 8 values per lane: vector i of
// wave w, lane l covers elements 8 * ((i * WPR + w) * 64 + l) .. +8, i.e.
// each vector instruction of a wave reads 4 whole groups (1 KiB).  A row
// covers WPR * 512 * VPL elements; groups past H are masked (per 16 lanes).
template <int VPL, int WPR>
__global__ __launch_bounds__(256) void k_rms_norm_quant(
    const uint16_t* __restrict__ x, int64_t ldx, const float* __restrict__ w, uint8_t* __restrict__ q,
    int64_t ldq, void* __restrict__ s, int64_t lds, int64_t M, int H, float eps_norm, float eps,
    int ue8m0, int fmt) {
  __shared__ double red[4];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  constexpr int kRowsPerBlock = 4 / WPR;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (WPR == 1 ? wave : 0);
  const int wv = WPR == 1 ? 0 : wave;
  const int ngroups = H / kGroup;
  // WPR == 1: a wave whose row is past M has nothing to do (no barrier below)
  if (WPR == 1 && row >= M) return;
  const uint16_t* xr = x + row * ldx;
  u32x4 v[VPL];
  double ss = 0.0;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = ((i * WPR + wv) * 64 + lane) * 8;
    v[i] = (e >> 7) < ngroups ? load_nt16(xr + e) : u32x4{0u, 0u, 0u, 0u};
  }
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
    if (lane == 0) red[wave] = ss;
    __syncthreads();
    ss = (red[0] + red[1]) + (red[2] + red[3]);
  }
  const float r = (float)(1.0 / __builtin_sqrt(ss / (double)H + (double)eps_norm));
  uint8_t* qr = q + row * ldq;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = ((i * WPR + wv) * 64 + lane) * 8;
    const int g = e >> 7;
    if (g >= ngroups) continue;  // the 16 lanes of a group agree
    const float4 w0 = *(const float4*)(w + e);
    const float4 w1 = *(const float4*)(w + e + 4);
    const float wj[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    const uint32_t c[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
    float y[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      y[2 * k] = (bf16_lo(c[k]) * r) * wj[2 * k];
      y[2 * k + 1] = (bf16_hi(c[k]) * r) * wj[2 * k + 1];
    }
    float sc;
    const uint2 codes = quant8(y, eps, ue8m0 != 0, &sc);
    *(uint2*)(qr + e) = codes;
    if ((lane & 15) == 0) store_scale(s, fmt, lds, row, g, sc);
  }
}

template <int VPL, int WPR>
hipError_t launch_rms(const uint16_t* x, int64_t ldx, const float* w, uint8_t* q, int64_t ldq, void* s,
                      int64_t lds, int64_t M, int H, float eps_norm, float eps, int ue8m0, int fmt,
                      hipStream_t stream) {
  constexpr int rpb = 4 / WPR;
  const int64_t blocks = (M + rpb - 1) / rpb;
  hipLaunchKernelGGL((k_rms_norm_quant<VPL, WPR>), dim3((unsigned)blocks), dim3(256), 0, stream, x, ldx,
                     w, q, ldq, s, lds, M, H, eps_norm, eps, ue8m0, fmt);
  return hipGetLastError();
}

// ------------------------------------------------------------ SiLU and mul
//
// 16 lanes per group, kSiluUnroll groups per 16 lanes in flight; groups are
// numbered row-major over (row, group column) and split into chunks of
// fewer than 2^24 groups so that row = (g * ceil(2^40 / gpr)) >> 40 is exact.
constexpr int kSiluThreads = 256;
constexpr int kSiluUnroll = 2;
constexpr uint32_t kSiluGroupsPerIter = (kSiluThreads / 16) * kSiluUnroll;

// silu(g) * u = (g u) / (1 + e^-g).  g u is exact in fp32 (two 8-bit
// significands).  1 + e is rounded to d with its error t recovered exactly
// (Fast2Sum on the larger and smaller of 1 and e), the quotient by d taken
// from the hardware reciprocal and corrected once with the exact residual
// g u - q d, less q t for the rounding of the divisor.  The result is within
// a fraction of an ulp of (g u) / (1 + e), so only exp's error remains
// (within an ulp: the library expf, not the bare hardware exp2).  e^-g is
// capped at e^80 so that d and 1/d stay normal; for g < -80 the true value
// is below 1e-30 |g u| either way.  The sign is that of g u.
__device__ __forceinline__ float silu_mul(float g, float u) {
  const float gu = g * u;
  const float e = expf(fminf(-g, 80.0f));
  const float a = fmaxf(1.0f, e), b = fminf(1.0f, e);
  const float d = a + b;
  const float t = b - (d - a);
  const float rd = __builtin_amdgcn_rcpf(d);
  const float q = gu * rd;
  const float r = __builtin_fmaf(-q, d, gu);
  const float r2 = __builtin_fmaf(-q, t, r);
  return __builtin_copysignf(__builtin_fmaf(r2, rd, q), gu);
}

__global__ __launch_bounds__(kSiluThreads) void k_silu_mul_quant(
    const uint16_t* __restrict__ x, int64_t ldx, uint8_t* __restrict__ q, int64_t ldq,
    void* __restrict__ s, int64_t lds, int64_t row0, uint32_t total, uint32_t gpr, uint64_t magic,
    int I, float eps, int ue8m0, int fmt) {
  const uint32_t sub = threadIdx.x & 15u;
  const uint32_t slot = threadIdx.x >> 4;
  const uint32_t step = gridDim.x * kSiluGroupsPerIter;
  for (uint32_t base = blockIdx.x * kSiluGroupsPerIter; base < total; base += step) {
    u32x4 gv[kSiluUnroll], uv[kSiluUnroll];
    uint32_t rows[kSiluUnroll], cols[kSiluUnroll];
    bool valid[kSiluUnroll];
#pragma unroll
    for (int k = 0; k < kSiluUnroll; ++k) {
      const uint32_t g = base + k * 16u + slot;
      valid[k] = g < total;
      rows[k] = (uint32_t)(((uint64_t)g * magic) >> 40);
      cols[k] = g - rows[k] * gpr;
      const uint16_t* p = x + (int64_t)rows[k] * ldx + (int64_t)cols[k] * kGroup + sub * 8;
      gv[k] = valid[k] ? load_nt16(p) : u32x4{0u, 0u, 0u, 0u};
      uv[k] = valid[k] ? load_nt16(p + I) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int k = 0; k < kSiluUnroll; ++k) {
      const uint32_t gc[4] = {gv[k].x, gv[k].y, gv[k].z, gv[k].w};
      const uint32_t uc[4] = {uv[k].x, uv[k].y, uv[k].z, uv[k].w};
      float y[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        y[2 * j] = silu_mul(bf16_lo(gc[j]), bf16_lo(uc[j]));
        y[2 * j + 1] = silu_mul(bf16_hi(gc[j]), bf16_hi(uc[j]));
      }
      float sc;
      const uint2 codes = quant8(y, eps, ue8m0 != 0, &sc);
      if (valid[k]) {
        const int64_t rr = row0 + rows[k];
        *(uint2*)(q + rr * ldq + (int64_t)cols[k] * kGroup + sub * 8) = codes;
        if (sub == 0) store_scale(s, fmt, lds, rr, cols[k], sc);
      }
    }
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
    if (H <= 512) e = launch_rms<1, 1>(xr, ldx, w, qr, ldq, sr, lds, rows, h, eps_norm, eps, u, scale_format, stream);
    else if (H <= 1024) e = launch_rms<2, 1>(xr, ldx, w, qr, ldq, sr, lds, rows, h, eps_norm, eps, u, scale_format, stream);
    else if (H <= 2048) e = launch_rms<4, 1>(xr, ldx, w, qr, ldq, sr, lds, rows, h, eps_norm, eps, u, scale_format, stream);
    else if (H <= 4096) e = launch_rms<8, 1>(xr, ldx, w, qr, ldq, sr, lds, rows, h, eps_norm, eps, u, scale_format, stream);
    else if (H <= 6144) e = launch_rms<12, 1>(xr, ldx, w, qr, ldq, sr, lds, rows, h, eps_norm, eps, u, scale_format, stream);
    else if (H <= 8192) e = launch_rms<16, 1>(xr, ldx, w, qr, ldq, sr, lds, rows, h, eps_norm, eps, u, scale_format, stream);
    else if (H <= 16384) e = launch_rms<8, 4>(xr, ldx, w, qr, ldq, sr, lds, rows, h, eps_norm, eps, u, scale_format, stream);
    else e = launch_rms<16, 4>(xr, ldx, w, qr, ldq, sr, lds, rows, h, eps_norm, eps, u, scale_format, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_silu_mul_quant(const uint16_t* x, int64_t M, int64_t I, int64_t ldx, uint8_t* q,
                                 int64_t ldq, void* s, int64_t lds, float eps, bool ue8m0,
                                 int scale_format, hipStream_t stream) {
  const int64_t gpr = I / kGroup;
  int64_t rows_per_chunk = (int64_t(1) << 24) / gpr;
  if (rows_per_chunk < 1) rows_per_chunk = 1;
  const uint64_t magic = ((uint64_t(1) << 40) + (uint64_t)gpr - 1) / (uint64_t)gpr;
  const int max_blocks = cu_count() * 8;
  for (int64_t r0 = 0; r0 < M; r0 += rows_per_chunk) {
    const int64_t rows = (M - r0) < rows_per_chunk ? (M - r0) : rows_per_chunk;
    const uint32_t total = (uint32_t)(rows * gpr);
    int64_t blocks = (total + kSiluGroupsPerIter - 1) / kSiluGroupsPerIter;
    if (blocks > max_blocks) blocks = max_blocks;
    hipLaunchKernelGGL(k_silu_mul_quant, dim3((unsigned)blocks), dim3(kSiluThreads), 0, stream,
                       x + r0 * ldx, ldx, q, ldq, s, lds, r0, total, (uint32_t)gpr, magic, (int)I, eps,
                       ue8m0 ? 1 : 0, scale_format);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace fp8blk
