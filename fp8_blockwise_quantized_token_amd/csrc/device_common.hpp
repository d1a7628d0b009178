// device_common.hpp -- gfx950 device helpers shared by the library's kernels.
//
// Quantization rule (Block_FP8, 1x128 activation / 128x128 weight scaling:
// page "Helion: improving vLLM inference with autotuning", section "Helion
// Linear Backend" / "Scope"): scale = max(amax, eps) / 448, optionally
// rounded up to a power of two (UE8M0: page "Helion-Kernel in vLLM: PyTorch
// FP8 ohne CUDA", section "Praktische Einschränkungen"), then every value is
// divided by the scale in fp32, clamped to +-448 and rounded to the nearest
// e4m3fn code (ties to even).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8blk {

constexpr int kGroup = 128;
constexpr float kE4M3Max = 448.0f;

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// bf16 halves of a packed dword, widened exactly to fp32.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two fp32 values -> two bf16 (round to nearest even, subnormals kept) in
// one word, lo in bits 0..15: gfx950's v_cvt_pk_bf16_f32, one instruction
// for the pair.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_bits(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// Maximum over the 16 lanes of a DPP row (lanes 16r .. 16r+15): two quad
// permutations, then the half-row and row mirrors.  Every lane of the row
// ends with the row maximum.  Operates on non-negative fp32 bit patterns,
// which order like unsigned integers.
__device__ __forceinline__ uint32_t row16_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));  // quad_perm 1,0,3,2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));  // quad_perm 2,3,0,1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false)); // row_half_mirror
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false)); // row_mirror
  return v;
}

// RN(1/448) in fp32.
constexpr float kInv448 = 0x1.24924ap-9f;

// x / s, correctly rounded, from y = RN(1/s), for x with a significand of
// at most 8 bits (bf16 values): q0 = RN(x y) is within one ulp of x/s, the
// residual q0 s - x is exact under an FMA, and one correction
// step RN(q0 - r y) rounds to RN(x/s) (Markstein's division theorem).  The
// residual is taken as q0 s - x (not x - q0 s) so that the correction keeps
// the sign IEEE division gives a zero or an underflowing quotient: x = -0
// gives -0 + (-0) = -0, x = +0 gives +0.  The test-suite checks this against
// IEEE division for every pair of bf16 value and bf16-derived scale
// significands and for the signed-zero and tiny cases.
__device__ __forceinline__ float div_by_scale(float x, float s, float y) {
  const float q0 = x * y;
  const float r = __builtin_fmaf(q0, s, -x);
  return __builtin_fmaf(-r, y, q0);
}

// 1/s in float64 for a positive normal fp32 s, to within 2^-52 (relative):
// the hardware reciprocal, then three Newton steps with FMA.  Each step
// squares the relative error and the last one is limited by its own
// rounding, so the bound holds for any starting approximation within 2^-8
// (host test); the steps cost 6 instructions per 128-value group.
__device__ __forceinline__ double recip_f64(float s) {
  const double b = (double)s;
  double d = __builtin_amdgcn_rcp(b);
#pragma unroll
  for (int i = 0; i < 3; ++i) d = __builtin_fma(d, __builtin_fma(-b, d, 1.0), d);
  return d;
}

// x / s rounded to fp32 exactly as IEEE division, for any fp32 x, from
// d = recip_f64(s): z = RN64(x d) is within 2^-51 (relative) of x / s, and a
// quotient of two fp32 values in the normal range lies at least 2^-49
// (relative) away from every fp32 rounding midpoint (a midpoint has a
// 25-bit odd significand, and its product with the scale's significand
// cannot fit in x's 24 bits), so z rounds to the same fp32 value as x / s.
// Below 2^-126 the last bit may differ, far below the smallest e4m3 code:
// both encode to the same signed zero.  x = +-0 gives +-0.  Three
// operations per value (two conversions and a product).
__device__ __forceinline__ float div_by_scale_f64(float x, double d) { return (float)((double)x * d); }

// scale = max(amax, eps) / 448, correctly rounded, with the optional
// power-of-two ceiling done on the exponent field.  The division by 448 is
// the one-step corrected product with RN(1/448) (3 operations instead of
// an IEEE divide): for the divisor 448 its residual is exact and its result
// equals IEEE division for every fp32 significand (checked exhaustively by
// the test-suite; exponents scale every step exactly) from 2^-100 up.  The
// entry points accept eps >= 2^-80 only, so max(amax, eps) is always in
// that range.  No branch: the work of several groups schedules together.
__device__ __forceinline__ float scale_from_amax(float amax, float eps, bool ue8m0) {
  const float a = amax > eps ? amax : eps;
  float s = div_by_scale(a, kE4M3Max, kInv448);
  if (ue8m0) {
    uint32_t b = __float_as_uint(s);
    b = (b & 0x007FFFFFu) ? (b & 0x7F800000u) + 0x00800000u : b;
    s = __uint_as_float(b);
  }
  return s;
}

// Four already-scaled values -> four e4m3fn codes (byte i = value i), clamp
// to +-448 first.  gfx950's v_cvt_pk_fp8_f32 rounds to nearest even into the
// OCP e4m3fn format.
__device__ __forceinline__ uint32_t encode4(float a, float b, float c, float d) {
  a = __builtin_amdgcn_fmed3f(a, -kE4M3Max, kE4M3Max);
  b = __builtin_amdgcn_fmed3f(b, -kE4M3Max, kE4M3Max);
  c = __builtin_amdgcn_fmed3f(c, -kE4M3Max, kE4M3Max);
  d = __builtin_amdgcn_fmed3f(d, -kE4M3Max, kE4M3Max);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// encode4 for quotients of the group rule: each is RN(x / s) with |x| <= amax
// and s >= RN(amax / 448) (or the power-of-two ceiling), so |q| <= 448 (1 +
// 2^-23) < 464, which gfx950's conversion rounds to 448 (0x7E): the clamp can
// be left out.  (It turns values from 464 up into the NaN code; the
// encoder for arbitrary values keeps the clamp.)
__device__ __forceinline__ uint32_t encode4_q(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// 16x16x128 fp8 x fp8 -> fp32 matrix-core product (no block scaling).
// Operand layout: lane l supplies row (l & 15) of its matrix and the 32
// consecutive K bytes starting at 32 * (l >> 4).  Result: lane l holds
// column (l & 15), rows 4 * (l >> 4) + 0..3.
__device__ __forceinline__ v4f mfma16x16x128(const v8i& a, const v8i& b) {
  v4f z = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 0, 0, 0, 0, 0, 0);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming load (non-temporal: data used once, keep it out of the
// caches' way).  The quantizer and the SiLU producer read with it; the RMSNorm
// rows and the decode GEMM's weight stream measure faster with plain loads.
__device__ __forceinline__ u32x4 load_nt16(const void* p) {
  return __builtin_nontemporal_load((const u32x4*)p);
}

// 16-byte load through the caches.
__device__ __forceinline__ u32x4 load16(const void* p) { return *(const u32x4*)p; }

__device__ __forceinline__ v8i make_v8i(u32x4 lo, u32x4 hi) {
  v8i r;
  r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
  r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
  return r;
}

}  // namespace fp8blk
