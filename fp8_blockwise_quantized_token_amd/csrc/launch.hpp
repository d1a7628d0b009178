// launch.hpp -- host-side launchers of the gfx950 kernels (internal).
// Arguments are validated by the C ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8blk {

// scale_format: bit 0 = MN-major scales [K/128][lds], bit 1 = E8M0 bytes.
hipError_t launch_group_quant(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                              uint8_t* q, int64_t ldq, void* s, int64_t lds,
                              float eps, bool ue8m0, int scale_format, hipStream_t stream);

hipError_t launch_weight_block_quant(const float* w, int64_t N, int64_t K, int64_t ldw,
                                     uint8_t* q, int64_t ldq, float* s, int64_t lds,
                                     float eps, bool ue8m0, hipStream_t stream);

hipError_t launch_e4m3_encode(const float* t, uint8_t* q, int64_t n, hipStream_t stream);

// One scale per row (per token for bf16 activations, per channel for fp32
// weights); K <= kRowQuantMaxK (the row is held in registers).
constexpr int64_t kRowQuantMaxK = 32768;
hipError_t launch_row_quant(const void* x, bool bf16, int64_t rows, int64_t K, int64_t ldx,
                            uint8_t* q, int64_t ldq, float* s, float eps, bool ue8m0,
                            hipStream_t stream);

// Fused producers of the activation operand: RMSNorm (H <= kRmsMaxH) or
// SiLU(gate) * up, then 1x128 group quantization (scale_format as above).
constexpr int64_t kRmsMaxH = 32768;
hipError_t launch_rms_norm_quant(const uint16_t* x, int64_t M, int64_t H, int64_t ldx, const float* w,
                                 float eps_norm, uint8_t* q, int64_t ldq, void* s, int64_t lds,
                                 float eps, bool ue8m0, int scale_format, hipStream_t stream);
hipError_t launch_silu_mul_quant(const uint16_t* x, int64_t M, int64_t I, int64_t ldx, uint8_t* q,
                                 int64_t ldq, void* s, int64_t lds, float eps, bool ue8m0,
                                 int scale_format, hipStream_t stream);

struct GemmArgs {
  const uint8_t* a;
  const float* sa;
  int64_t lda, ldsa;
  // Activation scale (m, kb) is sa[m * sa_row + kb * sa_kb] (floats): row-major
  // [M][K/128] has (ldsa, 1), token-contiguous [K/128][ldsa] has (1, ldsa).
  // Unused by the per-token scale mode.
  int64_t sa_row, sa_kb;
  const uint8_t* w;
  const float* sw;
  int64_t ldw, ldsw;
  uint16_t* y;
  int64_t ldy;
  int64_t M, N, K;
  float* ws;  // split-K partials [split][M][N], or nullptr
  // Fused activation quantization (Swap-AB only): when x is set, the
  // activation operand is quantized from bf16 x in the GEMM itself and a/sa
  // are unused.
  const uint16_t* x;
  int64_t ldx;
  float eps;
  int ue8m0;
};

// Standard variant: (tile_m, tile_n, LDS stages, wave layout) among the
// compiled ones; kwaves 1 = the tile's default waves, 2 = twice as many
// waves, each half as wide in N (64x128 and 128x128 tiles).
// scale_mode: kScalesBlock (sa [M][K/128], sw [N/128][K/128], any fp32),
// kScalesBlockPow2 (same layout, every scale a power of two, applied by the
// matrix core), kScalesChannel (sa [M], sw [N]: per token / per channel).
constexpr int kScalesBlock = 0, kScalesBlockPow2 = 1, kScalesChannel = 2;
bool standard_tile_supported(int tile_m, int tile_n, int stages, int kwaves);
// split_tail: split only the tiles past the last whole round of resident
// workgroups (the reduction then covers those tiles only).
hipError_t launch_gemm_standard(const GemmArgs& g, int tile_m, int tile_n, int split_k, bool split_tail,
                                int stages, int kwaves, int scale_mode, hipStream_t stream);

// Swap-AB variant.
bool swapab_tile_supported(int tile_m, int tile_n, int kwaves);
hipError_t launch_gemm_swapab(const GemmArgs& g, int tile_m, int tile_n, int kwaves,
                              int split_k, hipStream_t stream, bool channel_scales = false);  // fused when g.x != nullptr

// Fixed-order sum of split_k fp32 partials -> bf16.
hipError_t launch_splitk_reduce(const float* ws, int split_k, int64_t M, int64_t N,
                                uint16_t* y, int64_t ldy, hipStream_t stream);

}  // namespace fp8blk
