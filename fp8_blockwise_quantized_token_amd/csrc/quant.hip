// quant.hip -- per-token 1x128 group quantizer, 128x128 weight block
// quantizer and the bare e4m3fn encoder for gfx950.
//
// per_token_group_fp8_quant (page "[RFC]: Using Helion for Selected vLLM
// CustomOps", section "Motivation"; Block_FP8 1x128 activation scaling on
// page "Helion: improving vLLM inference with autotuning", section "Helion
// Linear Backend" / "Scope").
//
// Group quantizer design (HBM-bound: 2 bytes in, 1 byte + 4/128 out per
// element):
//   - 16 lanes (one DPP row) own one 128-element group; each lane loads 16
//     contiguous bytes (8 bf16) with one global_load_dwordx4, so a wave reads
//     four whole groups = 1 KiB of contiguous HBM per load instruction.
//   - U = 4 groups per lane are loaded before any is used, keeping 4 KiB per
//     wave in flight.
//   - amax: packed u16 max of |bf16| bit patterns in registers, then a 4-step
//     DPP reduction inside the row (no LDS, no barriers).
//   - scale = max(amax, eps)/448 once per group (the corrected product with
//     RN(1/448), equal to IEEE division for eps >= 2^-80), 1/scale once per
//     group, and every element divided by the scale with a 3-instruction
//     correctly rounded division (Markstein) instead of a full IEEE divide.
//   - clamp with v_med3 and encode two values per v_cvt_pk_fp8_f32; 8 bytes
//     stored per lane.
#include "device_common.hpp"
#include "launch.hpp"

#pragma clang fp contract(off)

namespace fp8blk {
namespace {

typedef unsigned short us2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t amax8_bits(u32x4 v) {
  // |bf16| bit patterns order like their magnitudes.
  us2 a = __builtin_bit_cast(us2, v.x & 0x7FFF7FFFu);
  us2 b = __builtin_bit_cast(us2, v.y & 0x7FFF7FFFu);
  us2 c = __builtin_bit_cast(us2, v.z & 0x7FFF7FFFu);
  us2 d = __builtin_bit_cast(us2, v.w & 0x7FFF7FFFu);
  us2 m = __builtin_elementwise_max(__builtin_elementwise_max(a, b), __builtin_elementwise_max(c, d));
  uint32_t mm = m.x > m.y ? m.x : m.y;
  return mm << 16;
}

constexpr int kQuantThreads = 256;
constexpr int kQuantUnroll = 4;
constexpr uint32_t kGroupsPerIter = (kQuantThreads / 16) * kQuantUnroll;

// SF (scale output format): 0 fp32 [M][lds]; 1 fp32 MN-major [K/128][lds];
// 2 and 3: the same layouts with one E8M0 byte per scale (the biased
// exponent of a power-of-two scale, value 2^(b - 127)).
//
// Walk.  Row-major layouts take the groups row by row: group g of a launch
// is (g / div, g % div) with div = groups per row.  MN-major layouts take
// tiles of kTileR rows x kTileC group columns, one tile per workgroup
// iteration: g = 64 t + k is row kTileR (t / div) + k / kTileC and column
// kTileC (t % div) + k % kTileC, div = tiles per row band (groups outside
// the rows x cols of the launch are skipped).  A column's kTileR = 32 scales
// of a tile are then one whole 128-byte line stored from one workgroup,
// instead of pieces of a line stored from workgroups on different XCDs (that
// cost 15-20 % at prefill sizes), while each row still reads kTileC
// consecutive groups.  Either quotient is (n * magic) >> 40 with magic =
// ceil(2^40 / div), exact for n < 2^24 and div <= 2^16.
constexpr uint32_t kTileR = 32;
constexpr uint32_t kTileC = kGroupsPerIter / kTileR;

template <bool UE8M0, bool CONTIG, int SF>
__global__ __launch_bounds__(kQuantThreads) void k_group_quant(
    const uint16_t* __restrict__ x, uint8_t* __restrict__ q, void* __restrict__ s,
    uint32_t total_groups, uint32_t div, uint64_t magic, int64_t ldx, int64_t ldq,
    int64_t lds, float eps, uint32_t rows, uint32_t cols) {
  constexpr bool MN = (SF & 1) != 0;
  constexpr bool E8M0 = (SF & 2) != 0;
  const uint32_t sub = threadIdx.x & 15u;
  const uint32_t slot = threadIdx.x >> 4;
  const uint32_t step = gridDim.x * kGroupsPerIter;
  for (uint32_t base = blockIdx.x * kGroupsPerIter; base < total_groups; base += step) {
    u32x4 v[kQuantUnroll];
    int64_t qo[kQuantUnroll], so[kQuantUnroll];
    bool valid[kQuantUnroll];
#pragma unroll
    for (int u = 0; u < kQuantUnroll; ++u) {
      const uint32_t g = base + u * 16u + slot;
      valid[u] = g < total_groups;
      int64_t xo;
      if (CONTIG) {
        xo = (int64_t)g * kGroup + sub * 8;
        qo[u] = xo;
        so[u] = g;
      } else {
        uint32_t row, col;
        if (MN) {
          const uint32_t t = g / kGroupsPerIter, k = g % kGroupsPerIter;
          const uint32_t tr = (uint32_t)(((uint64_t)t * magic) >> 40);
          row = tr * kTileR + k / kTileC;
          col = (t - tr * div) * kTileC + k % kTileC;
          valid[u] = valid[u] && row < rows && col < cols;
        } else {
          row = (uint32_t)(((uint64_t)g * magic) >> 40);
          col = g - row * div;
        }
        xo = (int64_t)row * ldx + (int64_t)col * kGroup + sub * 8;
        qo[u] = (int64_t)row * ldq + (int64_t)col * kGroup + sub * 8;
        so[u] = MN ? (int64_t)col * lds + row : (int64_t)row * lds + col;
      }
      v[u] = valid[u] ? load_nt16(x + xo) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kQuantUnroll; ++u) {
      const float amax = __uint_as_float(row16_max_u32(amax8_bits(v[u])));
      const float sc = scale_from_amax(amax, eps, UE8M0);
      const float rc = 1.0f / sc;
      const u32x4 w = v[u];
      const uint32_t lo = encode4_q(div_by_scale(bf16_lo(w.x), sc, rc), div_by_scale(bf16_hi(w.x), sc, rc),
                                  div_by_scale(bf16_lo(w.y), sc, rc), div_by_scale(bf16_hi(w.y), sc, rc));
      const uint32_t hi = encode4_q(div_by_scale(bf16_lo(w.z), sc, rc), div_by_scale(bf16_hi(w.z), sc, rc),
                                  div_by_scale(bf16_lo(w.w), sc, rc), div_by_scale(bf16_hi(w.w), sc, rc));
      if (valid[u]) {
        *(uint2*)(q + qo[u]) = make_uint2(lo, hi);
        if (sub == 0) {
          if (E8M0)
            ((uint8_t*)s)[so[u]] = (uint8_t)(__float_as_uint(sc) >> 23);
          else
            ((float*)s)[so[u]] = sc;
        }
      }
    }
  }
}

// One workgroup per 128x128 block: thread t owns half a row (64 floats).
template <bool UE8M0>
__global__ __launch_bounds__(256) void k_weight_block_quant(
    const float* __restrict__ w, int64_t ldw, uint8_t* __restrict__ q, int64_t ldq,
    float* __restrict__ s, int64_t lds, float eps) {
  __shared__ float red[4];
  const int kb = blockIdx.x;
  const int64_t nb = blockIdx.y;
  const int t = threadIdx.x;
  const int row = t >> 1, half = t & 1;
  const float4* src = (const float4*)(w + (nb * kGroup + row) * ldw + (int64_t)kb * kGroup + half * 64);
  float4 v[16];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    v[i] = src[i];
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)), fmaxf(fabsf(v[i].z), fabsf(v[i].w))));
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if ((t & 63) == 0) red[t >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float sc = scale_from_amax(amax, eps, UE8M0);
  uint4* dst = (uint4*)(q + (nb * kGroup + row) * ldq + (int64_t)kb * kGroup + half * 64);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint4 o;
    o.x = encode4_q(v[4 * i].x / sc, v[4 * i].y / sc, v[4 * i].z / sc, v[4 * i].w / sc);
    o.y = encode4_q(v[4 * i + 1].x / sc, v[4 * i + 1].y / sc, v[4 * i + 1].z / sc, v[4 * i + 1].w / sc);
    o.z = encode4_q(v[4 * i + 2].x / sc, v[4 * i + 2].y / sc, v[4 * i + 2].z / sc, v[4 * i + 2].w / sc);
    o.w = encode4_q(v[4 * i + 3].x / sc, v[4 * i + 3].y / sc, v[4 * i + 3].z / sc, v[4 * i + 3].w / sc);
    dst[i] = o;
  }
  if (t == 0) s[nb * lds + kb] = sc;
}

// Per-token / per-channel quantization (FP8_Dynamic): one workgroup per
// row, the row held in registers (read once): up to 16 vectors of 16 bytes
// per thread.  amax over the row: |x| bit patterns (ordered like the
// magnitudes) reduced with DPP inside 16-lane rows, readlane across rows and
// LDS across waves; one scale; every value divided and encoded.  bf16 rows
// use the 3-instruction correctly rounded division (exact for 8-bit
// significands); fp32 rows (weights, offline) use IEEE division.
constexpr int kRowVec = 16;

template <bool BF16, bool UE8M0, int NT>
__global__ __launch_bounds__(NT) void k_row_quant(const uint8_t* __restrict__ x, int64_t ldx_bytes,
                                                  uint8_t* __restrict__ q, int64_t ldq,
                                                  float* __restrict__ s, int nvec, float eps) {
  __shared__ uint32_t red[NT / 64];
  constexpr int EV = BF16 ? 8 : 4;  // values per 16-byte vector
  const int64_t row = blockIdx.x;
  const int t = threadIdx.x;
  const uint8_t* src = x + row * ldx_bytes;
  u32x4 v[kRowVec];
  uint32_t am = 0;
#pragma unroll
  for (int i = 0; i < kRowVec; ++i) {
    const int idx = t + i * NT;
    v[i] = idx < nvec ? load_nt16(src + (int64_t)idx * 16) : u32x4{0u, 0u, 0u, 0u};
    if (BF16) {
      const uint32_t a = max(max(v[i].x & 0x7FFFu, v[i].x >> 16 & 0x7FFFu), max(v[i].y & 0x7FFFu, v[i].y >> 16 & 0x7FFFu));
      const uint32_t b = max(max(v[i].z & 0x7FFFu, v[i].z >> 16 & 0x7FFFu), max(v[i].w & 0x7FFFu, v[i].w >> 16 & 0x7FFFu));
      am = max(am, max(a, b) << 16);
    } else {
      am = max(am, max(max(v[i].x & 0x7FFFFFFFu, v[i].y & 0x7FFFFFFFu), max(v[i].z & 0x7FFFFFFFu, v[i].w & 0x7FFFFFFFu)));
    }
  }
  am = row16_max_u32(am);
  am = max(max((uint32_t)__builtin_amdgcn_readlane((int)am, 0), (uint32_t)__builtin_amdgcn_readlane((int)am, 16)),
           max((uint32_t)__builtin_amdgcn_readlane((int)am, 32), (uint32_t)__builtin_amdgcn_readlane((int)am, 48)));
  if ((t & 63) == 0) red[t >> 6] = am;
  __syncthreads();
  am = red[0];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) am = max(am, red[w]);
  const float sc = scale_from_amax(__uint_as_float(am), eps, UE8M0);
  const float rc = 1.0f / sc;
  uint8_t* dst = q + row * ldq;
#pragma unroll
  for (int i = 0; i < kRowVec; ++i) {
    const int idx = t + i * NT;
    if (idx >= nvec) continue;
    const u32x4 w = v[i];
    if (BF16) {
      const uint32_t lo = encode4_q(div_by_scale(bf16_lo(w.x), sc, rc), div_by_scale(bf16_hi(w.x), sc, rc),
                                  div_by_scale(bf16_lo(w.y), sc, rc), div_by_scale(bf16_hi(w.y), sc, rc));
      const uint32_t hi = encode4_q(div_by_scale(bf16_lo(w.z), sc, rc), div_by_scale(bf16_hi(w.z), sc, rc),
                                  div_by_scale(bf16_lo(w.w), sc, rc), div_by_scale(bf16_hi(w.w), sc, rc));
      *(uint2*)(dst + (int64_t)idx * EV) = make_uint2(lo, hi);
    } else {
      *(uint32_t*)(dst + (int64_t)idx * EV) =
          encode4_q(__uint_as_float(w.x) / sc, __uint_as_float(w.y) / sc, __uint_as_float(w.z) / sc,
                  __uint_as_float(w.w) / sc);
    }
  }
  if (t == 0) s[row] = sc;
}

__global__ __launch_bounds__(256) void k_e4m3_encode(const float* __restrict__ t,
                                                     uint8_t* __restrict__ q, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x * 4;
  for (int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4; i < n; i += stride) {
    if (i + 4 <= n) {
      const float4 v = *(const float4*)(t + i);
      *(uint32_t*)(q + i) = encode4(v.x, v.y, v.z, v.w);
    } else {
      for (int64_t j = i; j < n; ++j) q[j] = (uint8_t)(encode4(t[j], 0.f, 0.f, 0.f) & 0xFFu);
    }
  }
}

int device_cu_count() {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      cus = v;
  }
  return cus;
}

}  // namespace

template <bool UE8M0, bool CONTIG, int SF>
void launch_gq(dim3 grid, dim3 block, hipStream_t stream, const uint16_t* xr, uint8_t* qr, void* sr,
               uint32_t total, uint32_t div, uint64_t magic, int64_t ldx, int64_t ldq, int64_t lds,
               float eps, uint32_t rows, uint32_t cols) {
  hipLaunchKernelGGL((k_group_quant<UE8M0, CONTIG, SF>), grid, block, 0, stream, xr, qr, sr, total, div,
                     magic, ldx, ldq, lds, eps, rows, cols);
}

hipError_t launch_group_quant(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* q,
                              int64_t ldq, void* s, int64_t lds, float eps, bool ue8m0,
                              int scale_format, hipStream_t stream) {
  const int64_t gpr = K / kGroup;
  const bool mn = (scale_format & 1) != 0;
  const int64_t selt = (scale_format & 2) ? 1 : 4;  // bytes per stored scale
  const bool contig = scale_format == 0 && (ldx == K) && (ldq == K) && (lds == gpr);
  const int max_blocks = device_cu_count() * 8;
  // Contiguous: one flat launch per 2^31 groups.  Otherwise row chunks of
  // fewer than 2^24 groups, so that the kernel's quotients are exact (the
  // tiled MN-major walk divides tile numbers, below 2^18 then).
  const int64_t chunk_groups = contig ? (int64_t(1) << 31) : (int64_t(1) << 24);
  int64_t rows_per_chunk = chunk_groups / gpr;
  if (mn) rows_per_chunk = rows_per_chunk / kTileR * kTileR;  // whole row bands per chunk
  if (rows_per_chunk < 1) rows_per_chunk = 1;
  const int64_t tiles_c = (gpr + kTileC - 1) / kTileC;
  const uint64_t div = (!contig && mn) ? (uint64_t)tiles_c : (uint64_t)gpr;
  const uint64_t magic = ((uint64_t(1) << 40) + div - 1) / div;
  for (int64_t r0 = 0; r0 < M; r0 += rows_per_chunk) {
    const int64_t rows = (M - r0) < rows_per_chunk ? (M - r0) : rows_per_chunk;
    const uint32_t total = (uint32_t)((!contig && mn) ? ((rows + kTileR - 1) / kTileR) * tiles_c * kGroupsPerIter
                                                      : rows * gpr);
    int64_t blocks = (total + kGroupsPerIter - 1) / kGroupsPerIter;
    if (blocks > max_blocks) blocks = max_blocks;
    const uint16_t* xr = x + r0 * ldx;
    uint8_t* qr = q + r0 * ldq;
    void* sr = (char*)s + (mn ? r0 : r0 * lds) * selt;
    dim3 grid((unsigned)blocks), block(kQuantThreads);
    const uint32_t d32 = (uint32_t)div, r32 = (uint32_t)rows, c32 = (uint32_t)gpr;
#define FP8BLK_GQ(U, C, F) \
  launch_gq<U, C, F>(grid, block, stream, xr, qr, sr, total, d32, magic, ldx, ldq, lds, eps, r32, c32)
    if (contig) {
      if (ue8m0) FP8BLK_GQ(true, true, 0); else FP8BLK_GQ(false, true, 0);
    } else if (ue8m0) {
      switch (scale_format) {
        case 0: FP8BLK_GQ(true, false, 0); break;
        case 1: FP8BLK_GQ(true, false, 1); break;
        case 2: FP8BLK_GQ(true, false, 2); break;
        default: FP8BLK_GQ(true, false, 3); break;
      }
    } else {
      if (mn) FP8BLK_GQ(false, false, 1); else FP8BLK_GQ(false, false, 0);
    }
#undef FP8BLK_GQ
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_weight_block_quant(const float* w, int64_t N, int64_t K, int64_t ldw, uint8_t* q,
                                     int64_t ldq, float* s, int64_t lds, float eps, bool ue8m0,
                                     hipStream_t stream) {
  // grid.y is limited to 65535 row bands per launch
  const int64_t nbands = N / kGroup;
  for (int64_t b0 = 0; b0 < nbands; b0 += 65535) {
    const int64_t nb = (nbands - b0) < 65535 ? (nbands - b0) : 65535;
    dim3 grid((unsigned)(K / kGroup), (unsigned)nb), block(256);
    const float* wb = w + b0 * kGroup * ldw;
    uint8_t* qb = q + b0 * kGroup * ldq;
    float* sb = s + b0 * lds;
    if (ue8m0)
      hipLaunchKernelGGL(k_weight_block_quant<true>, grid, block, 0, stream, wb, ldw, qb, ldq, sb, lds, eps);
    else
      hipLaunchKernelGGL(k_weight_block_quant<false>, grid, block, 0, stream, wb, ldw, qb, ldq, sb, lds, eps);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_row_quant(const void* x, bool bf16, int64_t rows, int64_t K, int64_t ldx,
                            uint8_t* q, int64_t ldq, float* s, float eps, bool ue8m0,
                            hipStream_t stream) {
  const int ev = bf16 ? 8 : 4;
  const int nvec = (int)(K / ev);
  const int64_t ldx_bytes = ldx * (bf16 ? 2 : 4);
  for (int64_t r0 = 0; r0 < rows; r0 += 2147483647) {
    const int64_t nr = (rows - r0) < 2147483647 ? (rows - r0) : 2147483647;
    const uint8_t* xr = (const uint8_t*)x + r0 * ldx_bytes;
    uint8_t* qr = q + r0 * ldq;
    float* sr = s + r0;
    if (bf16) {
      if (ue8m0)
        hipLaunchKernelGGL((k_row_quant<true, true, 256>), dim3((unsigned)nr), dim3(256), 0, stream, xr, ldx_bytes, qr, ldq, sr, nvec, eps);
      else
        hipLaunchKernelGGL((k_row_quant<true, false, 256>), dim3((unsigned)nr), dim3(256), 0, stream, xr, ldx_bytes, qr, ldq, sr, nvec, eps);
    } else {
      if (ue8m0)
        hipLaunchKernelGGL((k_row_quant<false, true, 512>), dim3((unsigned)nr), dim3(512), 0, stream, xr, ldx_bytes, qr, ldq, sr, nvec, eps);
      else
        hipLaunchKernelGGL((k_row_quant<false, false, 512>), dim3((unsigned)nr), dim3(512), 0, stream, xr, ldx_bytes, qr, ldq, sr, nvec, eps);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_e4m3_encode(const float* t, uint8_t* q, int64_t n, hipStream_t stream) {
  int64_t blocks = (n + 1023) / 1024;
  const int64_t max_blocks = (int64_t)device_cu_count() * 16;
  if (blocks > max_blocks) blocks = max_blocks;
  hipLaunchKernelGGL(k_e4m3_encode, dim3((unsigned)blocks), dim3(256), 0, stream, t, q, n);
  return hipGetLastError();
}

}  // namespace fp8blk
