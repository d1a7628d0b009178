/*
 * fp8blk.h -- C ABI of the MI355X (gfx950) FP8 blockwise-quantized linear layer.
 *
 * The operation is the "Block_FP8" quantized linear layer: FP8 e4m3fn
 * activations with one scale per token and 128-wide K group (1x128), FP8
 * e4m3fn weights with one scale per 128x128 block, fp32 accumulation, bf16
 * output.  Format named on page "Helion: improving vLLM inference with
 * autotuning", section "Helion Linear Backend" / "Scope".  The activation
 * quantizer is per_token_group_fp8_quant and the GEMM is scaled_mm_blockwise
 * (page "Helion-Kernel in vLLM: PyTorch FP8 ohne CUDA", section "Welche
 * Kernel wurden in vLLM integriert"; page "[RFC]: Using Helion for Selected
 * vLLM CustomOps", section "Motivation").  The GEMM variants Standard,
 * Split-K and Swap-AB and their selection per shape follow the sections
 * "Kernel Implementation", "Hybrid Dispatch" and "Per-shape Config Tuning"
 * of the autotuning page.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers on the current HIP device.
 *     bf16 is passed as uint16_t bit patterns, fp8 e4m3fn as uint8_t codes.
 *   - Row-major 2-D layouts with an explicit leading dimension ("ld", in
 *     elements).  Activations X/Q/A are [M][K], weights W are [N][K] (K
 *     contiguous), the output Y is [M][N]; Y = A * W^T.
 *   - Activation scales are [M][K/128] (row pitch ldsa/lds floats), weight
 *     scales are [N/128][K/128] (row pitch ldsw floats); groups and blocks
 *     start at k = 0 and n = 0.
 *   - The caller owns every buffer.  The library never allocates device or
 *     host memory, never synchronizes, never reads device memory on the host
 *     and keeps no mutable global state besides caches of device properties
 *     (how many workgroups of a kernel fit the device at once, queried from
 *     the runtime on first use; not stream operations): calls are
 *     thread-safe and can be captured into a HIP graph.  Work is ordered on the given stream
 *     (a hipStream_t passed as void*; NULL is the default stream).
 *   - Outputs are fully overwritten; inputs are never modified.
 *   - Invalid arguments return a negative status before anything is
 *     launched.  A launch failure reported by the HIP runtime returns
 *     FP8BLK_ERR_HIP.  M == 0 (or n == 0) is a no-op returning FP8BLK_OK.
 *   - Required alignment: every base pointer 16 bytes, every fp8/bf16 row
 *     pitch a multiple of 16 bytes; scale pointers 4 bytes.
 *   - GEMM operand row pitches (A, W and their scale arrays, in bytes) are
 *     below 2^24, so that a 256-row tile spans less than 2^32 bytes
 *     (FP8BLK_ERR_BAD_STRIDE otherwise).
 *   - Inputs must be finite; NaN/Inf inputs give unspecified (but memory-safe)
 *     results.
 */
#ifndef FP8BLK_H
#define FP8BLK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP8BLK_ABI_VERSION 6
#define FP8BLK_GROUP 128      /* K-group width and weight block edge */
#define FP8BLK_E4M3_MAX 448.0f
/* Smallest accepted eps (2^-80, about 8.3e-25).  With eps at least this,
   every scale is at least 2^-88.8, which keeps the kernels' shortcut
   divisions (x / s from a reciprocal and one exact-residual correction)
   exact for every quotient that can reach an fp8 code; smaller eps values
   return FP8BLK_ERR_BAD_SHAPE.  The pages' value is 1e-10. */
#define FP8BLK_MIN_EPS 8.271806125530277e-25f /* 2^-80 */

/* status codes */
#define FP8BLK_OK 0
#define FP8BLK_ERR_NULL_PTR (-1)    /* a required pointer is NULL */
#define FP8BLK_ERR_BAD_SHAPE (-2)   /* K%128, N%128, negative sizes, group != 128, too large */
#define FP8BLK_ERR_MISALIGNED (-3)  /* pointer or row pitch not 16-byte aligned */
#define FP8BLK_ERR_BAD_STRIDE (-4)  /* leading dimension smaller than the row */
#define FP8BLK_ERR_WORKSPACE (-5)   /* workspace missing or smaller than required */
#define FP8BLK_ERR_BAD_CONFIG (-6)  /* unknown variant or unsupported tile/split */
#define FP8BLK_ERR_HIP (-7)         /* the HIP runtime rejected a launch */

/* flags */
#define FP8BLK_FLAG_UE8M0 1u /* scales rounded up to a power of two ("UE8M0",
                                "float32 ceiling E8M0"): page "Helion-Kernel in
                                vLLM", section "Praktische Einschränkungen";
                                RFC page, H100 end-to-end settings */
#define FP8BLK_FLAG_WEIGHT_POW2 8u /* fp8_linear, fp8_block_gemm_select: the caller
                                guarantees that every weight scale sw is a power of
                                two (weights quantized with FP8BLK_FLAG_UE8M0).
                                Together with FP8BLK_FLAG_UE8M0 it lets STANDARD
                                configurations use FP8BLK_SCALES_POW2. */

/* How the GEMM applies the K-block scales (fp8blk_gemm_config.scale_mode) */
#define FP8BLK_SCALES_FP32 0 /* any fp32 scales: one fp32 rescale per K block */
#define FP8BLK_SCALES_POW2 1 /* every sa and sw is a power of two (UE8M0):
                                applied exactly by the matrix core (STANDARD
                                only; results unspecified for other scales:
                                only the exponent bits of each scale are used) */
#define FP8BLK_SCALES_SA_MN_MAJOR 2 /* bit OR-ed into either mode: fp8_block_gemm's
                                activation scales are token-contiguous,
                                sa[K/128][ldsa] with ldsa >= M, as fp8_group_quant
                                writes them with FP8BLK_FLAG_SCALE_MN_MAJOR (a
                                Standard tile then loads each K block's scales
                                as one contiguous run); requires
                                (K/128) * ldsa * 4 < 2^31.  fp8_linear ignores
                                it (it lays out its own scales). */

/* Scale output of fp8_group_quant for other consumers (German page,
 * "Praktische Einschränkungen": UE8M0 scales for GEMMs that take them) */
#define FP8BLK_FLAG_SCALE_E8M0 2u     /* one byte per scale: the biased exponent
                                        b of the power-of-two scale 2^(b-127);
                                        requires FP8BLK_FLAG_UE8M0 */
#define FP8BLK_FLAG_SCALE_MN_MAJOR 4u /* scales stored [K/128][lds] (token index
                                        contiguous), lds >= M */

/* GEMM variants (autotuning page, section "Kernel Implementation") */
#define FP8BLK_STANDARD 0 /* tiles over (M, N), loop over K */
#define FP8BLK_SWAPAB 1   /* computes (W A^T)^T: weight rows on the matrix-core
                             row side, tokens on the column side (small M) */

/* A GEMM configuration.  split_k > 1 is the Split-K variant: the K blocks
 * are divided among split_k groups of workgroups, each writing an fp32
 * partial product to the workspace, then a second kernel sums the partials
 * in a fixed order and writes bf16 (deterministic, no atomics).
 *   STANDARD: tile_m x tile_n in {64x64, 64x128, 128x128, 256x128,
 *             128x256, 256x256}; stages = LDS pipeline depth (K blocks
 *             staged ahead): 0 (default, = 2) or 2..4 where compiled (64x64,
 *             64x128: 2-4; 128x128, 256x128: 2-3; others: 2).  Deeper
 *             pipelines hide memory latency in decode-sized problems.
 *             kwaves 1 (or 0): the tile's default waves; 2: twice the
 *             waves, each half as wide (64x64 and 64x128 with stages 2-4,
 *             128x128 with stages 2-3), for grids of about one workgroup
 *             per CU.
 *   SWAPAB:   tile_m (tokens per workgroup) in {16, 32, 64} and >= M,
 *             tile_n (weight rows per workgroup) in {16, 32, 64},
 *             kwaves (waves sharing one tile, each on its own K range,
 *             summed in the workgroup) in {1, 2, 4, 8}; stages must be 0.
 *   split_k: 1 .. min(256, K/128).
 *   split_tail (STANDARD only; 0 or 1): 1 splits only the tiles that do not
 *             fill a whole round of resident workgroups (CUs x workgroups
 *             per CU on the current device; tiles are taken in the kernel's
 *             walk order): the tiles of the whole rounds run over the full
 *             K range and write bf16 directly, the remaining ones run as
 *             split_k shorter workgroups each, so the last round is full.
 *             With fewer tiles than one round this is plain Split-K; with
 *             an exact number of rounds nothing is split.  The workspace
 *             requirement is the same as for split_k alone. */
typedef struct fp8blk_gemm_config {
    int32_t variant;
    int32_t tile_m;
    int32_t tile_n;
    int32_t split_k;
    int32_t kwaves;
    int32_t stages;
    int32_t scale_mode;  /* FP8BLK_SCALES_FP32 or FP8BLK_SCALES_POW2, optionally
                            | FP8BLK_SCALES_SA_MN_MAJOR */
    int32_t split_tail;  /* 0 or 1, see above */
} fp8blk_gemm_config;

/* Library ABI version (FP8BLK_ABI_VERSION of the build). */
int fp8_abi_version(void);

/* Human-readable name of a status code; never NULL, static storage. */
const char *fp8_status_string(int status);

/*
 * per_token_group_fp8_quant -- dynamic activation quantization.
 *
 * For every row m and group g (128 consecutive K elements from k = 128 g):
 *   amax = max_j |x[m][128g + j]|                 (bf16 -> fp32 exactly)
 *   s    = max(amax, eps) / 448                   (fp32, correctly rounded)
 *   if (flags & FP8BLK_FLAG_UE8M0) s = 2^ceil(log2 s)  (power-of-two ceiling)
 *   q[m][128g + j] = e4m3fn_rne(clamp(x / s, -448, 448))  (fp32 quotient,
 *                                                  ties to even, sign of zero kept)
 *   s_out[m][g] = s
 * Format: autotuning page, "Helion Linear Backend" / "Scope" (Block_FP8, 1x128
 * activation scaling).  eps guards the all-zero group (pages silent; 1e-10
 * is the suggested value).
 *
 *   x     bf16 [M][ldx], ldx >= K        q  uint8 [M][ldq], ldq >= K
 *   s     fp32 [M][lds], lds >= K/128    group must be 128
 *         (FP8BLK_FLAG_SCALE_MN_MAJOR: [K/128][lds], lds >= M;
 *          FP8BLK_FLAG_SCALE_E8M0: uint8 E8M0 bytes in that layout)
 *   flags: FP8BLK_FLAG_UE8M0 | FP8BLK_FLAG_SCALE_E8M0 | FP8BLK_FLAG_SCALE_MN_MAJOR.
 *   Requires K % 128 == 0, M >= 0, eps >= FP8BLK_MIN_EPS and finite.
 */
int fp8_group_quant(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                    uint8_t *q, int64_t ldq, void *s, int64_t lds,
                    int32_t group, float eps, uint32_t flags, void *stream);

/*
 * 128x128 weight block quantization (offline preparation of W; same rule as
 * fp8_group_quant over 128x128 blocks of an fp32 matrix):
 *   s = max(amax_block, eps) / 448 [power-of-two ceiling if UE8M0],
 *   q = e4m3fn_rne(clamp(w / s, -448, 448)).
 * Format: autotuning page, "Helion Linear Backend" / "Scope" (128x128
 * weight scaling).
 *   w fp32 [N][ldw], ldw >= K;  q uint8 [N][ldq];  s fp32 [N/128][lds], lds >= K/128.
 *   Requires N % 128 == 0, K % 128 == 0, eps >= FP8BLK_MIN_EPS and finite.
 */
int fp8_weight_block_quant(const float *w, int64_t N, int64_t K, int64_t ldw,
                           uint8_t *q, int64_t ldq, float *s, int64_t lds,
                           float eps, uint32_t flags, void *stream);

/*
 * The encoding step on its own: q[i] = e4m3fn_rne(clamp(t[i], -448, 448))
 * for n contiguous fp32 values (same encoder as the quantizers).
 *   t fp32 [n], q uint8 [n]; n >= 0; both pointers 16-byte aligned.
 */
int fp8_e4m3_encode(const float *t, uint8_t *q, int64_t n, void *stream);

/*
 * Per-shape dispatch: the configuration fp8_block_gemm uses when cfg is NULL.
 * A table tuned on MI355X keyed on (N, K) and a bucket of M, with a
 * heuristic for shapes not in the table (autotuning page, "Hybrid Dispatch"
 * and "Per-shape Config Tuning").  flags: FP8BLK_FLAG_UE8M0 (the activation
 * scales are powers of two) and FP8BLK_FLAG_WEIGHT_POW2 (the weight scales
 * are powers of two); with both, STANDARD choices get scale_mode =
 * FP8BLK_SCALES_POW2.  Deterministic, host-only: a binary search over the
 * tabled weight shapes, then a scan of that shape's M buckets.
 * Returns FP8BLK_OK, or FP8BLK_ERR_BAD_SHAPE / FP8BLK_ERR_NULL_PTR /
 * FP8BLK_ERR_BAD_CONFIG (unknown flags).
 */
int fp8_block_gemm_select(int64_t M, int64_t N, int64_t K, uint32_t flags,
                          fp8blk_gemm_config *out);

/*
 * Workspace bytes fp8_block_gemm needs for this shape and configuration
 * (cfg NULL: the dispatched one).  Split-K needs split_k * M * N * 4 bytes;
 * the other variants need 0.  Returns a negative status on a bad argument.
 */
int64_t fp8_block_gemm_workspace_size(int64_t M, int64_t N, int64_t K,
                                      const fp8blk_gemm_config *cfg);

/*
 * scaled_mm_blockwise -- blockwise-scaled FP8 GEMM, bf16 out:
 *   y[m][n] = bf16_rne( sum_kb  sa[m][kb] * sw[n/128][kb] *
 *                       sum_{k in block kb} dec(a[m][k]) * dec(w[n][k]) )
 * with fp32 accumulation (autotuning page, "Kernel Implementation": the
 * quantized GEMM follows the unified GEMM with scaling added; "Scope":
 * 1x128 / 128x128 scales).
 *   a  uint8 e4m3fn [M][lda], lda >= K      sa fp32 [M][ldsa], ldsa >= K/128
 *                                           (FP8BLK_SCALES_SA_MN_MAJOR in the
 *                                           configuration: [K/128][ldsa], ldsa >= M)
 *   w  uint8 e4m3fn [N][ldw], ldw >= K      sw fp32 [N/128][ldsw], ldsw >= K/128
 *   y  bf16 [M][ldy], ldy >= N
 *   cfg NULL selects through fp8_block_gemm_select (flags 0: fp32 scale
 *   mode; pass a configuration from fp8_block_gemm_select(..., UE8M0, ...)
 *   to use the power-of-two mode).
 *   workspace: device buffer of at least fp8_block_gemm_workspace_size bytes
 *   (may be NULL when that is 0).  Concurrent calls must not share one.
 * Requires K % 128 == 0, N % 128 == 0, M >= 0.
 */
int fp8_block_gemm(const uint8_t *a, const float *sa, int64_t lda, int64_t ldsa,
                   const uint8_t *w, const float *sw, int64_t ldw, int64_t ldsw,
                   uint16_t *y, int64_t ldy, int64_t M, int64_t N, int64_t K,
                   const fp8blk_gemm_config *cfg, void *workspace,
                   int64_t workspace_bytes, void *stream);

/*
 * The whole FP8 linear layer in one call: y = scaled_mm_blockwise(
 * per_token_group_fp8_quant(x), w), i.e. exactly fp8_group_quant(x) (group
 * 128, this eps and flags) followed by fp8_block_gemm on its output.
 * Fusing the quantizer into the GEMM removes a launch: at a few tokens the
 * quantizer is launch-bound (RFC page "[RFC]: Using Helion for Selected vLLM
 * CustomOps", the SM120 benchmark comment), and the pages count kernel
 * launches per forward pass as the cost fusion cuts (page "Helion-Kernel in
 * vLLM", section "Welche Kernel wurden in vLLM integriert").
 *   SWAPAB configurations with tile_m <= 32, or tile_m 64 with tile_n 16
 *   (M <= 64, the small-M choices of the dispatcher), quantize each 1x128
 *   group of x inside the GEMM's operand load: one kernel (plus the split-K
 *   sum), and no fp8 copy of x is written.  Codes and scales are the ones fp8_group_quant would produce,
 *   bit for bit.  Other configurations run fp8_group_quant into the
 *   workspace, then the GEMM.
 *   x  bf16 [M][ldx], ldx >= K            w, sw, y, ldw, ldsw, ldy as in
 *                                           fp8_block_gemm
 *   eps as in fp8_group_quant.  flags: FP8BLK_FLAG_UE8M0 (power-of-two
 *   activation scales, as in fp8_group_quant) and FP8BLK_FLAG_WEIGHT_POW2
 *   (the caller's weight scales sw are powers of two).  The power-of-two
 *   GEMM mode needs both: cfg NULL selects through fp8_block_gemm_select with
 *   these flags (so UE8M0 activations with fp32 weight scales keep the fp32
 *   mode), and a caller cfg with scale_mode = FP8BLK_SCALES_POW2 without
 *   both flags returns FP8BLK_ERR_BAD_CONFIG.
 *   workspace: device buffer of at least fp8_linear_workspace_size bytes,
 *   16-byte aligned (may be NULL when that is 0); concurrent calls must not
 *   share one.  Layout: fp8 x [M][K] and its scales [M][K/128] (unless the
 *   quantizer is fused), then the split-K partials, each at a 256-byte
 *   boundary.
 * Requires K % 128 == 0, K <= 2^22, N % 128 == 0, M >= 0.
 */
int64_t fp8_linear_workspace_size(int64_t M, int64_t N, int64_t K,
                                  const fp8blk_gemm_config *cfg);

int fp8_linear(const uint16_t *x, int64_t ldx, const uint8_t *w, const float *sw,
               int64_t ldw, int64_t ldsw, uint16_t *y, int64_t ldy, int64_t M,
               int64_t N, int64_t K, float eps, uint32_t flags,
               const fp8blk_gemm_config *cfg, void *workspace,
               int64_t workspace_bytes, void *stream);

/*
 * fp8_linear without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, serving loops that may not
 * call hipMalloc, harnesses that forbid allocation.  Same arguments (minus
 * the workspace), results and configuration choice as fp8_linear.  The
 * workspace is instead a scratch array of FP8BLK_NOALLOC_SCRATCH_BYTES
 * (64 MiB) that the library holds on every GPU it runs on until the process
 * ends; nothing is allocated, freed or synchronized by the call.
 *   - A call whose workspace need (fp8_linear_workspace_size for the same
 *     M, N, K and configuration) exceeds that size returns
 *     FP8BLK_ERR_WORKSPACE with nothing launched.  Every dispatched
 *     configuration of the tabled Qwen3 shapes up to M = 256 fits (decode
 *     M <= 64 needs at most 15.3 MiB); large prefill calls generally do not.
 *   - The array is shared by every call on one GPU and keeps the last
 *     call's contents (nothing in it needs to start at zero): calls that may
 *     overlap on one GPU (several streams or host threads) race on it and
 *     must be serialized by the caller.
 *   - The first call on a device looks up the array's device address there
 *     (with that device current; no stream work).  A call with M = 0 does
 *     only that and returns FP8BLK_OK, so one such call per device before a
 *     graph capture keeps the lookup out of the capture.  FP8BLK_ERR_HIP if
 *     the lookup fails.
 */
#define FP8BLK_NOALLOC_SCRATCH_BYTES (64u << 20)
int fp8_linear_noalloc(const uint16_t *x, int64_t ldx, const uint8_t *w, const float *sw,
                       int64_t ldw, int64_t ldsw, uint16_t *y, int64_t ldy, int64_t M,
                       int64_t N, int64_t K, float eps, uint32_t flags,
                       const fp8blk_gemm_config *cfg, void *stream);

/*
 * FP8_Dynamic: per-token activation scales and per-channel weight scales
 * (autotuning page, "Helion Linear Backend" / "Scope": the first of its
 * three formats).  Quantizer dynamic_per_token_scaled_fp8_quant and GEMM
 * scaled_mm (German page, "Welche Kernel wurden in vLLM integriert").
 */

/*
 * dynamic_per_token_scaled_fp8_quant: the group rule of fp8_group_quant with
 * the whole row as one group -- for every row m: amax over its K values,
 * s[m] = max(amax, eps)/448 (power-of-two ceiling with FP8BLK_FLAG_UE8M0),
 * q[m][k] = e4m3fn_rne(clamp(x / s[m], -448, 448)).
 *   x bf16 [M][ldx], ldx >= K;  q uint8 [M][ldq], ldq >= K;  s fp32 [M].
 *   Requires K % 128 == 0, K <= 32768 (a row is held in registers) and
 *   eps >= FP8BLK_MIN_EPS;
 *   x and q 16-byte aligned with 16-byte row pitches, s 4-byte aligned.
 */
int fp8_token_quant(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                    uint8_t *q, int64_t ldq, float *s, float eps,
                    uint32_t flags, void *stream);

/*
 * Per-channel weight quantization (offline preparation of FP8_Dynamic
 * weights): for every row n of W, s[n] = max(amax_row, eps)/448 [power-of-
 * two ceiling], q = e4m3fn_rne(clamp(w / s[n], -448, 448)) (IEEE division).
 *   w fp32 [N][ldw], ldw >= K;  q uint8 [N][ldq];  s fp32 [N].
 *   Requires K % 128 == 0, K <= 32768 and eps >= FP8BLK_MIN_EPS.
 */
int fp8_weight_channel_quant(const float *w, int64_t N, int64_t K, int64_t ldw,
                             uint8_t *q, int64_t ldq, float *s, float eps,
                             uint32_t flags, void *stream);

/*
 * scaled_mm with per-token / per-channel scales, bf16 out:
 *   y[m][n] = bf16_rne( (sum_k dec(a[m][k]) * dec(w[n][k])) * sa[m] * sw[n] )
 * with fp32 accumulation.  The K loop is plain matrix-core accumulation; the
 * scales are applied once in the epilogue.
 *   a uint8 [M][lda], sa fp32 [M];  w uint8 [N][ldw], sw fp32 [N];
 *   y bf16 [M][ldy].  cfg as in fp8_block_gemm (NULL: fp8_block_gemm_select;
 *   scale_mode must be FP8BLK_SCALES_FP32); the workspace size is
 *   fp8_block_gemm_workspace_size's for the same configuration.
 * Requires K % 128 == 0, N % 128 == 0, M >= 0.
 */
int fp8_scaled_mm(const uint8_t *a, const float *sa, int64_t lda,
                  const uint8_t *w, const float *sw, int64_t ldw,
                  uint16_t *y, int64_t ldy, int64_t M, int64_t N, int64_t K,
                  const fp8blk_gemm_config *cfg, void *workspace,
                  int64_t workspace_bytes, void *stream);

/*
 * rms_norm_per_block_quant -- RMSNorm fused with the 1x128 group quantizer
 * (German page, "Welche Kernel wurden in vLLM integriert"; RFC page,
 * "Motivation").  RMSNorm as in the fp8 RMSNorm example of the Chinese
 * Helion article ("自己写一个 Helion kernel 并接入 vLLM"):
 *   r       = fp32( 1 / sqrt( (sum_j x[m][j]^2) / H + eps_norm ) )   (fp64)
 *   y[m][j] = (x[m][j] * r) * weight[j]                              (fp32)
 * then, per 128-group of y, exactly fp8_group_quant's rule (the scale from
 * the fp32 amax of y; the codes of y / s).  y is never stored.
 *   x      bf16 [M][ldx], ldx >= H        weight fp32 [H]
 *   q      uint8 [M][ldq], ldq >= H
 *   s      as fp8_group_quant's with K = H (fp32 [M][lds], lds >= H/128;
 *          MN-major / E8M0 by the same flags)
 *   Requires H % 128 == 0, H <= 32768, M >= 0, eps >= FP8BLK_MIN_EPS, eps_norm >= 0
 *   (both finite).  x, weight, q 16-byte aligned; ldx * 2 and ldq multiples
 *   of 16.  Finite inputs only.
 */
int fp8_rms_norm_per_block_quant(const uint16_t *x, int64_t M, int64_t H, int64_t ldx,
                                 const float *weight, float eps_norm,
                                 uint8_t *q, int64_t ldq, void *s, int64_t lds,
                                 float eps, uint32_t flags, void *stream);

/*
 * silu_and_mul_per_block_quant -- SiLU(gate) * up fused with the 1x128
 * group quantizer (German page, "Welche Kernel wurden in vLLM integriert";
 * RFC page, "Motivation").  Row m of x holds [gate | up], I values each:
 *   y[m][j] = silu(g) * u = g * u / (1 + exp(-g)),  g = x[m][j], u = x[m][I + j]
 * as the fp32 rounding of a float64 value within 2^-51 (relative) of the
 * exact one: g * u exact in float64, times the logistic function taken from
 * a correctly rounded float64 table of 1 / (1 + e^|g|) (1 minus it for
 * g > 0).  y is thus the correctly rounded fp32 value except where the
 * exact value lies within 2^-51 of a rounding midpoint.  Then
 * fp8_group_quant's rule on every 128-group of y.
 *   x  bf16 [M][ldx], ldx >= 2I          q uint8 [M][ldq], ldq >= I
 *   s  as fp8_group_quant's with K = I
 *   Requires I % 128 == 0, I <= 4194304, M >= 0, eps >= FP8BLK_MIN_EPS and finite; alignment as
 *   fp8_group_quant.  Finite inputs only.
 */
int fp8_silu_and_mul_per_block_quant(const uint16_t *x, int64_t M, int64_t I, int64_t ldx,
                                     uint8_t *q, int64_t ldq, void *s, int64_t lds,
                                     float eps, uint32_t flags, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8BLK_H */
