// api.hip -- the C ABI of libfp8blk (declared in include/fp8blk.h).
//
// Every entry point validates its arguments completely before touching the
// HIP runtime, so that a bad call returns an error code with nothing
// launched.  No entry point allocates, synchronizes or reads device memory.
#include <math.h>
#include <stdint.h>

#include <atomic>

#include "../../include/fp8blk.h"
#include "dispatch.hpp"
#include "launch.hpp"

namespace {

constexpr int64_t kG = FP8BLK_GROUP;
constexpr int64_t kMaxDim = int64_t(1) << 31;  // every extent fits int32 index math
constexpr int64_t kMaxK = int64_t(1) << 22;    // the strided quantizer's row division
constexpr int64_t kMaxPitch = int64_t(1) << 24;  // GEMM operand row pitch in bytes: a tile spans < 2^32 bytes

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

int to_status(hipError_t e) { return e == hipSuccess ? FP8BLK_OK : FP8BLK_ERR_HIP; }

// scale_mode without the activation-scale layout bit
int scale_rule(const fp8blk_gemm_config& c) { return c.scale_mode & ~FP8BLK_SCALES_SA_MN_MAJOR; }
bool sa_mn_major(const fp8blk_gemm_config& c) { return (c.scale_mode & FP8BLK_SCALES_SA_MN_MAJOR) != 0; }

int check_config(const fp8blk_gemm_config& c, int64_t M, int64_t N, int64_t K) {
  const int64_t kb = K / kG;
  if (c.split_tail != 0 && (c.split_tail != 1 || c.variant != FP8BLK_STANDARD)) return FP8BLK_ERR_BAD_CONFIG;
  if (c.scale_mode < 0 || (scale_rule(c) != FP8BLK_SCALES_FP32 && scale_rule(c) != FP8BLK_SCALES_POW2))
    return FP8BLK_ERR_BAD_CONFIG;
  if (scale_rule(c) == FP8BLK_SCALES_POW2 && c.variant != FP8BLK_STANDARD) return FP8BLK_ERR_BAD_CONFIG;
  if (c.split_k < 1 || c.split_k > 256 || c.split_k > kb) return FP8BLK_ERR_BAD_CONFIG;
  if (c.variant == FP8BLK_STANDARD) {
    if (!fp8blk::standard_tile_supported(c.tile_m, c.tile_n, c.stages, c.kwaves == 0 ? 1 : c.kwaves))
      return FP8BLK_ERR_BAD_CONFIG;
    if (N % c.tile_n != 0) return FP8BLK_ERR_BAD_CONFIG;
    // one workgroup per (tile, split): the grid must fit a 32-bit count
    const int64_t blocks = ((M + c.tile_m - 1) / c.tile_m) * (N / c.tile_n) * c.split_k;
    if (blocks > 2147483647) return FP8BLK_ERR_BAD_SHAPE;
    return FP8BLK_OK;
  }
  if (c.variant == FP8BLK_SWAPAB) {
    if (!fp8blk::swapab_tile_supported(c.tile_m, c.tile_n, c.kwaves) || c.stages != 0)
      return FP8BLK_ERR_BAD_CONFIG;
    if (M > c.tile_m) return FP8BLK_ERR_BAD_CONFIG;
    return FP8BLK_OK;
  }
  return FP8BLK_ERR_BAD_CONFIG;
}

int check_gemm_shape(int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N <= 0 || K <= 0) return FP8BLK_ERR_BAD_SHAPE;
  if (K % kG != 0 || N % kG != 0) return FP8BLK_ERR_BAD_SHAPE;
  if (M >= kMaxDim || N >= kMaxDim || K >= kMaxDim) return FP8BLK_ERR_BAD_SHAPE;
  return FP8BLK_OK;
}

int kernel_scale_mode(const fp8blk_gemm_config& c) {
  return scale_rule(c) == FP8BLK_SCALES_POW2 ? fp8blk::kScalesBlockPow2 : fp8blk::kScalesBlock;
}

// Activation scales of fp8_block_gemm: row-major [M][ldsa] (ldsa >= K/128) or
// token-contiguous [K/128][ldsa] (ldsa >= M); a K block's offset kb * ldsa * 4
// must stay below 2^31 bytes (the kernels' 32-bit scalar offsets).
int set_sa_layout(fp8blk::GemmArgs& g, bool mn, int64_t ldsa, int64_t M, int64_t K) {
  if (mn) {
    if (ldsa < M) return FP8BLK_ERR_BAD_STRIDE;
    if ((K / kG) * ldsa * 4 >= (int64_t(1) << 31)) return FP8BLK_ERR_BAD_STRIDE;
    g.sa_row = 1;
    g.sa_kb = ldsa;
  } else {
    if (ldsa < K / kG) return FP8BLK_ERR_BAD_STRIDE;
    g.sa_row = ldsa;
    g.sa_kb = 1;
  }
  return FP8BLK_OK;
}

int64_t workspace_for(const fp8blk_gemm_config& c, int64_t M, int64_t N) {
  return c.split_k > 1 ? (int64_t)c.split_k * M * N * 4 : 0;
}

int64_t round256(int64_t v) { return (v + 255) / 256 * 256; }

// fp8_linear's workspace: Swap-AB with up to two token tiles (tile_m <= 32),
// or four with 16 weight rows per workgroup (tile_m 64, tile_n 16; wider
// tiles would not fit the raw activations in registers), quantizes in the
// GEMM and needs only the split-K partials; the other
// configurations first quantize into the workspace:
// [q: M x K bytes][s: M x K/128 floats][split-K partials], each 256-aligned.
struct LinearLayout {
  bool fused;
  int64_t q_off, s_off, ws_off, total;
};

LinearLayout linear_layout(const fp8blk_gemm_config& c, int64_t M, int64_t N, int64_t K) {
  LinearLayout L;
  L.fused = c.variant == FP8BLK_SWAPAB && (c.tile_m <= 32 || (c.tile_m == 64 && c.tile_n == 16));
  const int64_t split = workspace_for(c, M, N);
  if (L.fused) {
    L.q_off = L.s_off = L.ws_off = 0;
    L.total = split;
    return L;
  }
  L.q_off = 0;
  L.s_off = round256(M * K);
  L.ws_off = L.s_off + round256(M * (K / kG) * 4);
  L.total = L.ws_off + split;
  return L;
}

// Scale output of the group quantizers: flags, layout and pitch.  *fmt gets
// bit 0 = MN-major, bit 1 = E8M0 bytes.
int check_group_scales(uint32_t flags, int64_t M, int64_t K, int64_t lds, int* fmt) {
  const uint32_t known = FP8BLK_FLAG_UE8M0 | FP8BLK_FLAG_SCALE_E8M0 | FP8BLK_FLAG_SCALE_MN_MAJOR;
  if ((flags & ~known) != 0) return FP8BLK_ERR_BAD_CONFIG;
  const bool e8m0 = (flags & FP8BLK_FLAG_SCALE_E8M0) != 0;
  const bool mn = (flags & FP8BLK_FLAG_SCALE_MN_MAJOR) != 0;
  if (e8m0 && !(flags & FP8BLK_FLAG_UE8M0)) return FP8BLK_ERR_BAD_CONFIG;  // E8M0 holds powers of two only
  if (lds < (mn ? M : K / kG)) return FP8BLK_ERR_BAD_STRIDE;
  *fmt = (mn ? 1 : 0) | (e8m0 ? 2 : 0);
  return FP8BLK_OK;
}

int check_quant_args(float eps, uint32_t flags) {
  if (!(eps >= FP8BLK_MIN_EPS) || !isfinite(eps)) return FP8BLK_ERR_BAD_SHAPE;
  if ((flags & ~FP8BLK_FLAG_UE8M0) != 0) return FP8BLK_ERR_BAD_CONFIG;
  return FP8BLK_OK;
}

// ---- the scratch array of fp8_linear_noalloc ----
// One array per GPU, allocated with the code object and held until the
// process ends.  In host code its name is only a stand-in: the device
// address is looked up once per device (hipGetSymbolAddress with that device
// current) and used instead everywhere.
constexpr int64_t kScratchBytes = int64_t(FP8BLK_NOALLOC_SCRATCH_BYTES);
static __device__ __align__(256) uint8_t scratch[FP8BLK_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 256;
std::atomic<void*> scratch_ptr[kMaxDevices];  // device address per device id (nullptr: not looked up yet)

int scratch_of_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FP8BLK_ERR_HIP;
  void* p = scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return FP8BLK_ERR_HIP;
    scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return FP8BLK_OK;
}

// fp8_linear's work for both of its entry points.  from_scratch: the
// workspace is this device's scratch array (fp8_linear_noalloc), looked up
// after the arguments are validated and the size is checked against it.
int linear_call(const uint16_t* x, int64_t ldx, const uint8_t* w, const float* sw, int64_t ldw,
                int64_t ldsw, uint16_t* y, int64_t ldy, int64_t M, int64_t N, int64_t K, float eps,
                uint32_t flags, const fp8blk_gemm_config* cfg, void* workspace, int64_t workspace_bytes,
                bool from_scratch, void* stream) {
  int st = check_gemm_shape(M, N, K);
  if (st != FP8BLK_OK) return st;
  if (K > kMaxK) return FP8BLK_ERR_BAD_SHAPE;
  st = check_quant_args(eps, flags & ~FP8BLK_FLAG_WEIGHT_POW2);
  if (st != FP8BLK_OK) return st;
  fp8blk_gemm_config c;
  if (cfg) {
    c = *cfg;
  } else {
    fp8blk::select_config(M, N, K, flags, &c);
  }
  st = check_config(c, M, N, K);
  if (st != FP8BLK_OK) return st;
  // the matrix core keeps only the exponent bits of every scale: both the
  // quantizer's scales and the caller's weight scales must be powers of two
  const uint32_t pow2_flags = FP8BLK_FLAG_UE8M0 | FP8BLK_FLAG_WEIGHT_POW2;
  if (scale_rule(c) == FP8BLK_SCALES_POW2 && (flags & pow2_flags) != pow2_flags) return FP8BLK_ERR_BAD_CONFIG;
  if (ldx < K || ldw < K || ldy < N || ldsw < K / kG) return FP8BLK_ERR_BAD_STRIDE;
  if (ldw >= kMaxPitch || ldsw * 4 >= kMaxPitch) return FP8BLK_ERR_BAD_STRIDE;
  const LinearLayout L = linear_layout(c, M, N, K);
  if (from_scratch) {
    if (L.total > kScratchBytes) return FP8BLK_ERR_WORKSPACE;
    st = scratch_of_current_device(&workspace);
    if (st != FP8BLK_OK) return st;
    workspace_bytes = kScratchBytes;
  }
  if (M == 0) return FP8BLK_OK;
  if (!x || !w || !sw || !y) return FP8BLK_ERR_NULL_PTR;
  if (!aligned16(x) || !aligned16(w) || !aligned16(y) || !aligned4(sw) || (ldx * 2) % 16 != 0 ||
      ldw % 16 != 0 || (ldy * 2) % 16 != 0)
    return FP8BLK_ERR_MISALIGNED;
  if (L.total > 0) {
    if (!workspace || workspace_bytes < L.total) return FP8BLK_ERR_WORKSPACE;
    if (!aligned16(workspace)) return FP8BLK_ERR_MISALIGNED;
  }
  const bool ue8m0 = (flags & FP8BLK_FLAG_UE8M0) != 0;
  hipStream_t s = (hipStream_t)stream;
  char* base = (char*)workspace;
  fp8blk::GemmArgs g{};
  g.w = w;
  g.sw = sw;
  g.ldw = ldw;
  g.ldsw = ldsw;
  g.y = y;
  g.ldy = ldy;
  g.M = M;
  g.N = N;
  g.K = K;
  g.ws = c.split_k > 1 ? (float*)(base + L.ws_off) : nullptr;
  if (L.fused) {
    g.x = x;
    g.ldx = ldx;
    g.eps = eps;
    g.ue8m0 = ue8m0 ? 1 : 0;
    return to_status(fp8blk::launch_gemm_swapab(g, c.tile_m, c.tile_n, c.kwaves, c.split_k, s));
  }
  uint8_t* q = (uint8_t*)(base + L.q_off);
  float* sc = (float*)(base + L.s_off);
  // The scales go to the workspace token-contiguous ([K/128][M]): a Standard
  // tile then loads each K block's 256 activation scales as one contiguous
  // run instead of 256 scattered words (row-major when a K block's offset
  // would not fit 31 bits).
  const bool mn = (K / kG) * M * 4 < (int64_t(1) << 31);
  hipError_t e = fp8blk::launch_group_quant(x, M, K, ldx, q, K, sc, mn ? M : K / kG, eps, ue8m0, mn ? 1 : 0, s);
  if (e != hipSuccess) return FP8BLK_ERR_HIP;
  g.a = q;
  g.sa = sc;
  g.lda = K;
  g.ldsa = mn ? M : K / kG;
  set_sa_layout(g, mn, g.ldsa, M, K);
  if (c.variant == FP8BLK_SWAPAB)
    return to_status(fp8blk::launch_gemm_swapab(g, c.tile_m, c.tile_n, c.kwaves, c.split_k, s));
  return to_status(fp8blk::launch_gemm_standard(g, c.tile_m, c.tile_n, c.split_k, c.split_tail != 0, c.stages,
                                                c.kwaves == 0 ? 1 : c.kwaves, kernel_scale_mode(c), s));
}


}  // namespace

extern "C" {

int fp8_abi_version(void) { return FP8BLK_ABI_VERSION; }

const char* fp8_status_string(int status) {
  switch (status) {
    case FP8BLK_OK: return "ok";
    case FP8BLK_ERR_NULL_PTR: return "null pointer";
    case FP8BLK_ERR_BAD_SHAPE: return "unsupported shape";
    case FP8BLK_ERR_MISALIGNED: return "misaligned pointer or row pitch";
    case FP8BLK_ERR_BAD_STRIDE: return "leading dimension too small";
    case FP8BLK_ERR_WORKSPACE: return "workspace missing or too small";
    case FP8BLK_ERR_BAD_CONFIG: return "unsupported GEMM configuration";
    case FP8BLK_ERR_HIP: return "HIP launch failure";
    default: return "unknown status";
  }
}

int fp8_group_quant(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* q, int64_t ldq,
                    void* s, int64_t lds, int32_t group, float eps, uint32_t flags, void* stream) {
  if (group != kG) return FP8BLK_ERR_BAD_SHAPE;
  if (M < 0 || K <= 0 || K % kG != 0 || K > kMaxK || M >= kMaxDim) return FP8BLK_ERR_BAD_SHAPE;
  if (!(eps >= FP8BLK_MIN_EPS) || !isfinite(eps)) return FP8BLK_ERR_BAD_SHAPE;
  int fmt = 0;
  const int st = check_group_scales(flags, M, K, lds, &fmt);
  if (st != FP8BLK_OK) return st;
  if (ldx < K || ldq < K) return FP8BLK_ERR_BAD_STRIDE;
  if (M == 0) return FP8BLK_OK;
  if (!x || !q || !s) return FP8BLK_ERR_NULL_PTR;
  if (!aligned16(x) || !aligned16(q) || (!(fmt & 2) && !aligned4(s)) || (ldx * 2) % 16 != 0 || ldq % 16 != 0)
    return FP8BLK_ERR_MISALIGNED;
  return to_status(fp8blk::launch_group_quant(x, M, K, ldx, q, ldq, s, lds, eps,
                                              (flags & FP8BLK_FLAG_UE8M0) != 0, fmt, (hipStream_t)stream));
}

int fp8_weight_block_quant(const float* w, int64_t N, int64_t K, int64_t ldw, uint8_t* q,
                           int64_t ldq, float* s, int64_t lds, float eps, uint32_t flags,
                           void* stream) {
  if (N < 0 || K < 0 || N % kG != 0 || K % kG != 0 || N >= kMaxDim || K >= kMaxDim)
    return FP8BLK_ERR_BAD_SHAPE;
  if (!(eps >= FP8BLK_MIN_EPS) || !isfinite(eps)) return FP8BLK_ERR_BAD_SHAPE;
  if ((flags & ~FP8BLK_FLAG_UE8M0) != 0) return FP8BLK_ERR_BAD_CONFIG;
  if (ldw < K || ldq < K || lds < K / kG) return FP8BLK_ERR_BAD_STRIDE;
  if (N == 0 || K == 0) return FP8BLK_OK;
  if (!w || !q || !s) return FP8BLK_ERR_NULL_PTR;
  if (!aligned16(w) || !aligned16(q) || !aligned4(s) || (ldw * 4) % 16 != 0 || ldq % 16 != 0)
    return FP8BLK_ERR_MISALIGNED;
  if (K / kG > 2147483647 || N / kG > 2147483647) return FP8BLK_ERR_BAD_SHAPE;
  return to_status(fp8blk::launch_weight_block_quant(w, N, K, ldw, q, ldq, s, lds, eps,
                                                     (flags & FP8BLK_FLAG_UE8M0) != 0,
                                                     (hipStream_t)stream));
}

int fp8_e4m3_encode(const float* t, uint8_t* q, int64_t n, void* stream) {
  if (n < 0) return FP8BLK_ERR_BAD_SHAPE;
  if (n == 0) return FP8BLK_OK;
  if (!t || !q) return FP8BLK_ERR_NULL_PTR;
  if (!aligned16(t) || !aligned16(q)) return FP8BLK_ERR_MISALIGNED;
  return to_status(fp8blk::launch_e4m3_encode(t, q, n, (hipStream_t)stream));
}

int fp8_block_gemm_select(int64_t M, int64_t N, int64_t K, uint32_t flags, fp8blk_gemm_config* out) {
  if (!out) return FP8BLK_ERR_NULL_PTR;
  const int st = check_gemm_shape(M, N, K);
  if (st != FP8BLK_OK) return st;
  if ((flags & ~(FP8BLK_FLAG_UE8M0 | FP8BLK_FLAG_WEIGHT_POW2)) != 0) return FP8BLK_ERR_BAD_CONFIG;
  fp8blk::select_config(M, N, K, flags, out);
  return FP8BLK_OK;
}

int64_t fp8_block_gemm_workspace_size(int64_t M, int64_t N, int64_t K, const fp8blk_gemm_config* cfg) {
  const int st = check_gemm_shape(M, N, K);
  if (st != FP8BLK_OK) return st;
  fp8blk_gemm_config c;
  if (cfg) {
    c = *cfg;
    const int cs = check_config(c, M, N, K);
    if (cs != FP8BLK_OK) return cs;
  } else {
    fp8blk::select_config(M, N, K, 0, &c);
  }
  return workspace_for(c, M, N);
}

int fp8_block_gemm(const uint8_t* a, const float* sa, int64_t lda, int64_t ldsa, const uint8_t* w,
                   const float* sw, int64_t ldw, int64_t ldsw, uint16_t* y, int64_t ldy, int64_t M,
                   int64_t N, int64_t K, const fp8blk_gemm_config* cfg, void* workspace,
                   int64_t workspace_bytes, void* stream) {
  int st = check_gemm_shape(M, N, K);
  if (st != FP8BLK_OK) return st;
  fp8blk_gemm_config c;
  if (cfg) {
    c = *cfg;
  } else {
    fp8blk::select_config(M, N, K, 0, &c);
  }
  st = check_config(c, M, N, K);
  if (st != FP8BLK_OK) return st;
  if (lda < K || ldw < K || ldy < N || ldsw < K / kG) return FP8BLK_ERR_BAD_STRIDE;
  if (lda >= kMaxPitch || ldw >= kMaxPitch || ldsa * 4 >= kMaxPitch || ldsw * 4 >= kMaxPitch)
    return FP8BLK_ERR_BAD_STRIDE;
  fp8blk::GemmArgs g{};
  st = set_sa_layout(g, sa_mn_major(c), ldsa, M, K);
  if (st != FP8BLK_OK) return st;
  if (M == 0) return FP8BLK_OK;
  if (!a || !sa || !w || !sw || !y) return FP8BLK_ERR_NULL_PTR;
  if (!aligned16(a) || !aligned16(w) || !aligned16(y) || !aligned4(sa) || !aligned4(sw) ||
      lda % 16 != 0 || ldw % 16 != 0 || (ldy * 2) % 16 != 0)
    return FP8BLK_ERR_MISALIGNED;
  const int64_t need = workspace_for(c, M, N);
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return FP8BLK_ERR_WORKSPACE;
    if (!aligned16(workspace)) return FP8BLK_ERR_MISALIGNED;
  }
  g.a = a;
  g.sa = sa;
  g.lda = lda;
  g.ldsa = ldsa;
  g.w = w;
  g.sw = sw;
  g.ldw = ldw;
  g.ldsw = ldsw;
  g.y = y;
  g.ldy = ldy;
  g.M = M;
  g.N = N;
  g.K = K;
  g.ws = need > 0 ? (float*)workspace : nullptr;
  hipStream_t s = (hipStream_t)stream;
  if (c.variant == FP8BLK_STANDARD)
    return to_status(fp8blk::launch_gemm_standard(g, c.tile_m, c.tile_n, c.split_k, c.split_tail != 0, c.stages,
                                                  c.kwaves == 0 ? 1 : c.kwaves, kernel_scale_mode(c), s));
  return to_status(fp8blk::launch_gemm_swapab(g, c.tile_m, c.tile_n, c.kwaves, c.split_k, s));
}

int64_t fp8_linear_workspace_size(int64_t M, int64_t N, int64_t K, const fp8blk_gemm_config* cfg) {
  const int st = check_gemm_shape(M, N, K);
  if (st != FP8BLK_OK) return st;
  if (K > kMaxK) return FP8BLK_ERR_BAD_SHAPE;
  fp8blk_gemm_config c;
  if (cfg) {
    c = *cfg;
    const int cs = check_config(c, M, N, K);
    if (cs != FP8BLK_OK) return cs;
  } else {
    fp8blk::select_config(M, N, K, 0, &c);
  }
  return linear_layout(c, M, N, K).total;
}

int fp8_linear(const uint16_t* x, int64_t ldx, const uint8_t* w, const float* sw, int64_t ldw,
               int64_t ldsw, uint16_t* y, int64_t ldy, int64_t M, int64_t N, int64_t K, float eps,
               uint32_t flags, const fp8blk_gemm_config* cfg, void* workspace,
               int64_t workspace_bytes, void* stream) {
  return linear_call(x, ldx, w, sw, ldw, ldsw, y, ldy, M, N, K, eps, flags, cfg, workspace, workspace_bytes,
                     false, stream);
}

int fp8_linear_noalloc(const uint16_t* x, int64_t ldx, const uint8_t* w, const float* sw, int64_t ldw,
                       int64_t ldsw, uint16_t* y, int64_t ldy, int64_t M, int64_t N, int64_t K, float eps,
                       uint32_t flags, const fp8blk_gemm_config* cfg, void* stream) {
  return linear_call(x, ldx, w, sw, ldw, ldsw, y, ldy, M, N, K, eps, flags, cfg, nullptr, 0, true, stream);
}

int fp8_token_quant(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* q, int64_t ldq,
                    float* s, float eps, uint32_t flags, void* stream) {
  if (M < 0 || K <= 0 || K % kG != 0 || K > fp8blk::kRowQuantMaxK || M >= kMaxDim) return FP8BLK_ERR_BAD_SHAPE;
  const int st = check_quant_args(eps, flags);
  if (st != FP8BLK_OK) return st;
  if (ldx < K || ldq < K) return FP8BLK_ERR_BAD_STRIDE;
  if (M == 0) return FP8BLK_OK;
  if (!x || !q || !s) return FP8BLK_ERR_NULL_PTR;
  if (!aligned16(x) || !aligned16(q) || !aligned4(s) || (ldx * 2) % 16 != 0 || ldq % 16 != 0)
    return FP8BLK_ERR_MISALIGNED;
  return to_status(fp8blk::launch_row_quant(x, true, M, K, ldx, q, ldq, s, eps,
                                            (flags & FP8BLK_FLAG_UE8M0) != 0, (hipStream_t)stream));
}

int fp8_weight_channel_quant(const float* w, int64_t N, int64_t K, int64_t ldw, uint8_t* q,
                             int64_t ldq, float* s, float eps, uint32_t flags, void* stream) {
  if (N < 0 || K <= 0 || K % kG != 0 || K > fp8blk::kRowQuantMaxK || N >= kMaxDim) return FP8BLK_ERR_BAD_SHAPE;
  const int st = check_quant_args(eps, flags);
  if (st != FP8BLK_OK) return st;
  if (ldw < K || ldq < K) return FP8BLK_ERR_BAD_STRIDE;
  if (N == 0) return FP8BLK_OK;
  if (!w || !q || !s) return FP8BLK_ERR_NULL_PTR;
  if (!aligned16(w) || !aligned16(q) || !aligned4(s) || (ldw * 4) % 16 != 0 || ldq % 16 != 0)
    return FP8BLK_ERR_MISALIGNED;
  return to_status(fp8blk::launch_row_quant(w, false, N, K, ldw, q, ldq, s, eps,
                                            (flags & FP8BLK_FLAG_UE8M0) != 0, (hipStream_t)stream));
}

int fp8_scaled_mm(const uint8_t* a, const float* sa, int64_t lda, const uint8_t* w, const float* sw,
                  int64_t ldw, uint16_t* y, int64_t ldy, int64_t M, int64_t N, int64_t K,
                  const fp8blk_gemm_config* cfg, void* workspace, int64_t workspace_bytes,
                  void* stream) {
  int st = check_gemm_shape(M, N, K);
  if (st != FP8BLK_OK) return st;
  fp8blk_gemm_config c;
  if (cfg) {
    c = *cfg;
  } else {
    fp8blk::select_config(M, N, K, 0, &c);
  }
  st = check_config(c, M, N, K);
  if (st != FP8BLK_OK) return st;
  if (c.scale_mode != FP8BLK_SCALES_FP32) return FP8BLK_ERR_BAD_CONFIG;  // the scale layout is fixed here
  if (lda < K || ldw < K || ldy < N) return FP8BLK_ERR_BAD_STRIDE;
  if (lda >= kMaxPitch || ldw >= kMaxPitch) return FP8BLK_ERR_BAD_STRIDE;
  if (M == 0) return FP8BLK_OK;
  if (!a || !sa || !w || !sw || !y) return FP8BLK_ERR_NULL_PTR;
  if (!aligned16(a) || !aligned16(w) || !aligned16(y) || !aligned4(sa) || !aligned4(sw) ||
      lda % 16 != 0 || ldw % 16 != 0 || (ldy * 2) % 16 != 0)
    return FP8BLK_ERR_MISALIGNED;
  const int64_t need = workspace_for(c, M, N);
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return FP8BLK_ERR_WORKSPACE;
    if (!aligned16(workspace)) return FP8BLK_ERR_MISALIGNED;
  }
  fp8blk::GemmArgs g{};
  g.a = a;
  g.sa = sa;
  g.lda = lda;
  g.sa_row = 1;
  g.sa_kb = 0;
  g.w = w;
  g.sw = sw;
  g.ldw = ldw;
  g.y = y;
  g.ldy = ldy;
  g.M = M;
  g.N = N;
  g.K = K;
  g.ws = need > 0 ? (float*)workspace : nullptr;
  hipStream_t s = (hipStream_t)stream;
  if (c.variant == FP8BLK_STANDARD)
    return to_status(fp8blk::launch_gemm_standard(g, c.tile_m, c.tile_n, c.split_k, c.split_tail != 0, c.stages, c.kwaves == 0 ? 1 : c.kwaves,
                                                  fp8blk::kScalesChannel, s));
  return to_status(fp8blk::launch_gemm_swapab(g, c.tile_m, c.tile_n, c.kwaves, c.split_k, s, true));
}

int fp8_rms_norm_per_block_quant(const uint16_t* x, int64_t M, int64_t H, int64_t ldx, const float* weight,
                                 float eps_norm, uint8_t* q, int64_t ldq, void* s, int64_t lds, float eps,
                                 uint32_t flags, void* stream) {
  if (M < 0 || H <= 0 || H % kG != 0 || H > fp8blk::kRmsMaxH || M >= kMaxDim) return FP8BLK_ERR_BAD_SHAPE;
  if (!(eps >= FP8BLK_MIN_EPS) || !isfinite(eps) || !(eps_norm >= 0.0f) || !isfinite(eps_norm))
    return FP8BLK_ERR_BAD_SHAPE;
  int fmt = 0;
  const int st = check_group_scales(flags, M, H, lds, &fmt);
  if (st != FP8BLK_OK) return st;
  if (ldx < H || ldq < H) return FP8BLK_ERR_BAD_STRIDE;
  if (M == 0) return FP8BLK_OK;
  if (!x || !weight || !q || !s) return FP8BLK_ERR_NULL_PTR;
  if (!aligned16(x) || !aligned16(weight) || !aligned16(q) || (!(fmt & 2) && !aligned4(s)) ||
      (ldx * 2) % 16 != 0 || ldq % 16 != 0)
    return FP8BLK_ERR_MISALIGNED;
  return to_status(fp8blk::launch_rms_norm_quant(x, M, H, ldx, weight, eps_norm, q, ldq, s, lds, eps,
                                                 (flags & FP8BLK_FLAG_UE8M0) != 0, fmt, (hipStream_t)stream));
}

int fp8_silu_and_mul_per_block_quant(const uint16_t* x, int64_t M, int64_t I, int64_t ldx, uint8_t* q,
                                     int64_t ldq, void* s, int64_t lds, float eps, uint32_t flags,
                                     void* stream) {
  if (M < 0 || I <= 0 || I % kG != 0 || I > kMaxK || M >= kMaxDim) return FP8BLK_ERR_BAD_SHAPE;
  if (!(eps >= FP8BLK_MIN_EPS) || !isfinite(eps)) return FP8BLK_ERR_BAD_SHAPE;
  int fmt = 0;
  const int st = check_group_scales(flags, M, I, lds, &fmt);
  if (st != FP8BLK_OK) return st;
  if (ldx < 2 * I || ldq < I) return FP8BLK_ERR_BAD_STRIDE;
  if (M == 0) return FP8BLK_OK;
  if (!x || !q || !s) return FP8BLK_ERR_NULL_PTR;
  if (!aligned16(x) || !aligned16(q) || (!(fmt & 2) && !aligned4(s)) || (ldx * 2) % 16 != 0 || ldq % 16 != 0)
    return FP8BLK_ERR_MISALIGNED;
  return to_status(fp8blk::launch_silu_mul_quant(x, M, I, ldx, q, ldq, s, lds, eps,
                                                 (flags & FP8BLK_FLAG_UE8M0) != 0, fmt, (hipStream_t)stream));
}

}  // extern "C"
