/*
 * oracle.c -- plain CPU reference of the FP8 blockwise-quantized linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this file; only the test-suite, the smoke check and the CPU
 * baseline leg of the benchmark do.  It shares no source with the GPU library
 * (no headers, no helpers, no tables).
 *
 * What it computes, and where that is defined:
 *   - "Block_FP8": FP8 with 1x128 activation scaling and 128x128 weight
 *     scaling.  Page "Helion: improving vLLM inference with autotuning",
 *     section "Helion Linear Backend" / "Scope".
 *   - The activation quantizer per_token_group_fp8_quant (named among the
 *     nine kernels of page "Helion-Kernel in vLLM: PyTorch FP8 ohne CUDA",
 *     section "Welche Kernel wurden in vLLM integriert", and as the first
 *     rollout kernel of page "[RFC]: Using Helion for Selected vLLM
 *     CustomOps", section "Motivation").
 *   - The power-of-two ("UE8M0", "float32 ceiling E8M0") scale option: page
 *     "Helion-Kernel in vLLM", section "Praktische Einschränkungen", and the
 *     H100 settings of the RFC page, section "End-to-End Model Performance".
 *   - The blockwise-scaled GEMM scaled_mm_blockwise: same structure as the
 *     plain GEMM of the "Kernel Implementation" section of the autotuning
 *     page, plus the quantization scales.
 *
 *   - "FP8_Dynamic": FP8 with per-token activation scaling and per-channel
 *     weight scaling (same page and section as Block_FP8).  Its activation
 *     quantizer is dynamic_per_token_scaled_fp8_quant and its GEMM scaled_mm
 *     (both among the nine kernels of the German page, section "Welche
 *     Kernel wurden in vLLM integriert").  Here: one scale per row of X (the
 *     group is the whole row) and one per row of W, the same amax / scale /
 *     encode rule as the group quantizer.
 *
 *   - The fused producers rms_norm_per_block_quant and
 *     silu_and_mul_per_block_quant (German page, section "Welche Kernel
 *     wurden in vLLM integriert"; RFC page, section "Motivation"): RMSNorm,
 *     respectively SiLU(gate) * up, followed by the 1x128 group quantizer.
 *     RMSNorm follows the fp8 RMSNorm example of the Chinese Helion article
 *     (zdabc.icu), section "自己写一个 Helion kernel 并接入 vLLM": variance =
 *     sum of squares / hidden size, rms = sqrt(variance + eps), normalized =
 *     x / rms times the weight, the weight in fp32 as in that example.  The
 *     pages fix no precision, so: the variance and
 *     1/rms in double, 1/rms rounded once to float, then (x * (1/rms)) * w in
 *     float; SiLU(g) * u = g / (1 + exp(-g)) * u in double, rounded once to
 *     float.  The quantizer then divides by the scale in IEEE float.
 *
 * The pages do not print the e4m3fn bit layout, the rounding mode, the
 * saturation rule, the all-zero-group rule or the scale layouts.  The
 * readings taken here (OCP e4m3fn, round to nearest with ties to even,
 * clamp to +-448 before encoding, amax clamped below by eps, scales stored
 * row-major as [M][K/128] and [N/128][K/128], weights as W[N][K]) are the
 * documented conventions of this project.
 *
 * Floating point: fp32 steps use C float arithmetic (SSE on x86-64, IEEE
 * single, correctly rounded division); build with -ffp-contract=off so that
 * no multiply-add is fused.  The GEMM reference is accumulated in fp64.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_GROUP 128
#define ORC_E4M3_MAX 448.0f

/* ------------------------------------------------------------------ */
/* e4m3fn codec                                                        */
/* ------------------------------------------------------------------ */

/* Value of an e4m3fn code: sign bit, 4 exponent bits (bias 7), 3 mantissa
 * bits; exponent field 0 is the subnormal range m * 2^-9; code 0x7F / 0xFF
 * is NaN; there is no infinity. */
double orc_e4m3_decode(uint8_t c)
{
    int sign = (c >> 7) & 1;
    int e = (c >> 3) & 0xF;
    int m = c & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp((double)(8 + m), e - 10); /* (1 + m/8) * 2^(e-7) */
    return sign ? -v : v;
}

/* Round |t| <= 448 to the nearest e4m3fn value, ties to the code whose
 * mantissa is even.  Written as the definition: the non-negative codes
 * 0x00..0x7E are in increasing order of value, so find the pair that
 * brackets |t| and compare |t| with their midpoint exactly (2|t| and the
 * sum of two e4m3 values are exact in double).  The sign of t (also of -0)
 * is kept in bit 7.  Values beyond 448 are the caller's to clamp. */
uint8_t orc_e4m3_encode(float t)
{
    int neg = signbit(t) ? 1 : 0;
    double a = fabs((double)t);
    int lo = 0, hi = 126, code;
    if (a >= 448.0) {
        code = 126;
    } else {
        /* largest code c with value(c) <= a */
        while (lo < hi) {
            int mid = (lo + hi + 1) / 2;
            if (orc_e4m3_decode((uint8_t)mid) <= a)
                lo = mid;
            else
                hi = mid - 1;
        }
        {
            double vlo = orc_e4m3_decode((uint8_t)lo);
            double vhi = orc_e4m3_decode((uint8_t)(lo + 1));
            double twice = 2.0 * a;
            double mids = vlo + vhi;
            if (twice < mids)
                code = lo;
            else if (twice > mids)
                code = lo + 1;
            else
                code = (lo & 1) ? lo + 1 : lo; /* mantissa LSB is the code LSB */
        }
    }
    return (uint8_t)((neg << 7) | code);
}

void orc_e4m3_encode_array(const float *t, uint8_t *q, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        q[i] = orc_e4m3_encode(t[i]);
}

/* ------------------------------------------------------------------ */
/* scales                                                              */
/* ------------------------------------------------------------------ */

/* bf16 is the upper half of an IEEE binary32. */
static float bf16_value(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Power-of-two ceiling of a positive normal float: s = f * 2^e with
 * f in [0.5, 1); s is already a power of two iff f == 0.5. */
float orc_pow2_ceil(float s)
{
    int e;
    float f = frexpf(s, &e);
    if (f == 0.5f)
        return s;
    return ldexpf(1.0f, e);
}

/* scale = max(amax, eps) / 448, then optionally its power-of-two ceiling. */
float orc_scale_from_amax(float amax, float eps, int ue8m0)
{
    float a = amax > eps ? amax : eps;
    float s = a / ORC_E4M3_MAX;
    if (ue8m0)
        s = orc_pow2_ceil(s);
    return s;
}

/* Encode one value with a given scale: t = v / s in fp32, clamped to
 * [-448, 448] (a value inside the range, -0 included, passes unchanged). */
static uint8_t quantize_one(float v, float s)
{
    float t = v / s;
    if (t > ORC_E4M3_MAX)
        t = ORC_E4M3_MAX;
    else if (t < -ORC_E4M3_MAX)
        t = -ORC_E4M3_MAX;
    return orc_e4m3_encode(t);
}

/* ------------------------------------------------------------------ */
/* per-token 1x128 group quantizer                                     */
/* ------------------------------------------------------------------ */

/* x: bf16 bits [M][ldx]; q: [M][ldq]; s: [M][lds], one scale per group of
 * 128 consecutive K elements starting at k = 0.  K % 128 == 0. */
void orc_group_quant(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                     uint8_t *q, int64_t ldq, float *s, int64_t lds,
                     float eps, int ue8m0)
{
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t g = 0; g < K / ORC_GROUP; ++g) {
            const uint16_t *xg = x + m * ldx + g * ORC_GROUP;
            float v[ORC_GROUP];
            float amax = 0.0f;
            for (int j = 0; j < ORC_GROUP; ++j) {
                v[j] = bf16_value(xg[j]);
                if (fabsf(v[j]) > amax)
                    amax = fabsf(v[j]);
            }
            float sc = orc_scale_from_amax(amax, eps, ue8m0);
            s[m * lds + g] = sc;
            for (int j = 0; j < ORC_GROUP; ++j)
                q[m * ldq + g * ORC_GROUP + j] = quantize_one(v[j], sc);
        }
    }
}

/* ------------------------------------------------------------------ */
/* per-token and per-channel quantizers (FP8_Dynamic)                  */
/* ------------------------------------------------------------------ */

/* One row of n values, already converted to float: amax over the row,
 * scale, then every value encoded with that scale. */
static float quantize_row(const float *v, int64_t n, uint8_t *q, float eps, int ue8m0)
{
    float amax = 0.0f;
    for (int64_t j = 0; j < n; ++j)
        if (fabsf(v[j]) > amax)
            amax = fabsf(v[j]);
    float sc = orc_scale_from_amax(amax, eps, ue8m0);
    for (int64_t j = 0; j < n; ++j)
        q[j] = quantize_one(v[j], sc);
    return sc;
}

/* dynamic_per_token_scaled_fp8_quant: x bf16 bits [M][ldx] -> q [M][ldq],
 * s [M] (one scale per token, over all K values of its row). */
void orc_token_quant(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                     uint8_t *q, int64_t ldq, float *s, float eps, int ue8m0)
{
    float *v = (float *)malloc((size_t)(K > 0 ? K : 1) * sizeof(float));
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t k = 0; k < K; ++k)
            v[k] = bf16_value(x[m * ldx + k]);
        s[m] = quantize_row(v, K, q + m * ldq, eps, ue8m0);
    }
    free(v);
}

/* Per-channel weight quantization: w fp32 [N][K] -> q [N][K], s [N]. */
void orc_channel_quant(const float *w, int64_t N, int64_t K, uint8_t *q, float *s,
                       float eps, int ue8m0)
{
    for (int64_t n = 0; n < N; ++n)
        s[n] = quantize_row(w + n * K, K, q + n * K, eps, ue8m0);
}

/* ------------------------------------------------------------------ */
/* fused producers: RMSNorm / SiLU-and-mul, then the group quantizer   */
/* ------------------------------------------------------------------ */

/* Group quantization of one row of float values already computed. */
static void group_quant_row(const float *y, int64_t n, uint8_t *q, float *s, float eps, int ue8m0)
{
    for (int64_t g = 0; g < n / ORC_GROUP; ++g)
        s[g] = quantize_row(y + g * ORC_GROUP, ORC_GROUP, q + g * ORC_GROUP, eps, ue8m0);
}

/* Group quantization of M rows of K float values (the group rule on values
 * already computed in float): q [M][K], s [M][K/128]. */
void orc_group_quant_f32(const float *y, int64_t M, int64_t K, uint8_t *q, float *s,
                         float eps, int ue8m0)
{
    for (int64_t m = 0; m < M; ++m)
        group_quant_row(y + m * K, K, q + m * K, s + m * (K / ORC_GROUP), eps, ue8m0);
}

/* RMSNorm's 1/rms of one row, in double (before its rounding to float):
 * variance = sum of squares / H, 1 / sqrt(variance + eps_norm). */
static double rms_inv_rms_row(const uint16_t *xr, int64_t H, float eps_norm)
{
    double ss = 0.0;
    for (int64_t j = 0; j < H; ++j) {
        double v = (double)bf16_value(xr[j]);
        ss += v * v;
    }
    double var = ss / (double)H;
    return 1.0 / sqrt(var + (double)eps_norm);
}

/* The normalized row y = (x * r) * w in float for a float 1/rms r, then the
 * group quantizer. */
static void rms_apply_row(const uint16_t *xr, const float *w, int64_t H, float r, float *y,
                          uint8_t *q, float *s, float eps, int ue8m0)
{
    for (int64_t j = 0; j < H; ++j)
        y[j] = (bf16_value(xr[j]) * r) * w[j];
    group_quant_row(y, H, q, s, eps, ue8m0);
}

/* rms_norm_per_block_quant: x bf16 [M][H], w fp32 [H] -> q [M][H], s [M][H/128]. */
void orc_rms_norm_per_block_quant(const uint16_t *x, const float *w, int64_t M, int64_t H,
                              float eps_norm, uint8_t *q, float *s, float eps, int ue8m0)
{
    float *y = (float *)malloc((size_t)H * sizeof(float));
    for (int64_t m = 0; m < M; ++m) {
        float r = (float)rms_inv_rms_row(x + m * H, H, eps_norm);
        rms_apply_row(x + m * H, w, H, r, y, q + m * H, s + m * (H / ORC_GROUP), eps, ue8m0);
    }
    free(y);
}

/* The double 1/rms of every row, before the rounding to float (r64 [M]). */
void orc_rms_norm_inv_rms(const uint16_t *x, int64_t M, int64_t H, float eps_norm, double *r64)
{
    for (int64_t m = 0; m < M; ++m)
        r64[m] = rms_inv_rms_row(x + m * H, H, eps_norm);
}

/* rms_norm_per_block_quant with the float 1/rms of every row given (r [M]). */
void orc_rms_norm_apply(const uint16_t *x, const float *w, int64_t M, int64_t H, const float *r,
                        uint8_t *q, float *s, float eps, int ue8m0)
{
    float *y = (float *)malloc((size_t)H * sizeof(float));
    for (int64_t m = 0; m < M; ++m)
        rms_apply_row(x + m * H, w, H, r[m], y, q + m * H, s + m * (H / ORC_GROUP), eps, ue8m0);
    free(y);
}

/* silu(g) * u = g / (1 + e^-g) * u in double, before its rounding to float. */
static double silu_mul_value(uint16_t gb, uint16_t ub)
{
    double g = (double)bf16_value(gb);
    double u = (double)bf16_value(ub);
    return g / (1.0 + exp(-g)) * u;
}

/* silu_and_mul_per_block_quant: x bf16 [M][2I] = [gate | up] -> q [M][I], s [M][I/128]. */
void orc_silu_and_mul_per_block_quant(const uint16_t *x, int64_t M, int64_t I, uint8_t *q, float *s,
                              float eps, int ue8m0)
{
    float *y = (float *)malloc((size_t)I * sizeof(float));
    for (int64_t m = 0; m < M; ++m) {
        const uint16_t *xr = x + m * 2 * I;
        for (int64_t j = 0; j < I; ++j)
            y[j] = (float)silu_mul_value(xr[j], xr[I + j]);
        group_quant_row(y, I, q + m * I, s + m * (I / ORC_GROUP), eps, ue8m0);
    }
    free(y);
}

/* The double silu(g) * u of every element, before the rounding to float
 * (y64 [M][I]). */
void orc_silu_and_mul_values(const uint16_t *x, int64_t M, int64_t I, double *y64)
{
    for (int64_t m = 0; m < M; ++m)
        for (int64_t j = 0; j < I; ++j)
            y64[m * I + j] = silu_mul_value(x[m * 2 * I + j], x[m * 2 * I + I + j]);
}

/* ------------------------------------------------------------------ */
/* 128x128 weight block quantizer                                      */
/* ------------------------------------------------------------------ */

/* w: fp32 [N][K]; q: [N][K]; s: [N/128][K/128].  N, K multiples of 128. */
void orc_weight_block_quant(const float *w, int64_t N, int64_t K,
                            uint8_t *q, float *s, float eps, int ue8m0)
{
    int64_t kb_n = K / ORC_GROUP;
    for (int64_t nb = 0; nb < N / ORC_GROUP; ++nb) {
        for (int64_t kb = 0; kb < kb_n; ++kb) {
            float amax = 0.0f;
            for (int64_t i = 0; i < ORC_GROUP; ++i)
                for (int64_t j = 0; j < ORC_GROUP; ++j) {
                    float a = fabsf(w[(nb * ORC_GROUP + i) * K + kb * ORC_GROUP + j]);
                    if (a > amax)
                        amax = a;
                }
            float sc = orc_scale_from_amax(amax, eps, ue8m0);
            s[nb * kb_n + kb] = sc;
            for (int64_t i = 0; i < ORC_GROUP; ++i)
                for (int64_t j = 0; j < ORC_GROUP; ++j) {
                    int64_t idx = (nb * ORC_GROUP + i) * K + kb * ORC_GROUP + j;
                    q[idx] = quantize_one(w[idx], sc);
                }
        }
    }
}

/* ------------------------------------------------------------------ */
/* blockwise-scaled GEMM, fp64                                         */
/* ------------------------------------------------------------------ */

/* y[r][n] = sum_k (dec(qa[m][k]) * sa[m][k/128]) * (dec(qw[n][k]) * sw[n/128][k/128])
 * for m = rows[r] (or m = r when rows is NULL), summed in increasing k.
 * qa: [M][K], sa: [M][K/128], qw: [N][K], sw: [N/128][K/128], y: [nrows][N].
 * Every output is an independent fixed-order sum, so the row split over
 * threads does not change any result. */
typedef struct {
    const uint8_t *qa;
    const float *sa;
    const uint8_t *qw;
    const float *sw;
    int64_t N, K;
    const int64_t *rows;
    int64_t r0, r1;
    double *y;
} gemm_job;

static void *gemm_worker(void *arg)
{
    gemm_job *j = (gemm_job *)arg;
    double dec[256];
    int64_t kb_n = j->K / ORC_GROUP;
    for (int c = 0; c < 256; ++c)
        dec[c] = orc_e4m3_decode((uint8_t)c);
    for (int64_t r = j->r0; r < j->r1; ++r) {
        int64_t m = j->rows ? j->rows[r] : r;
        const uint8_t *arow = j->qa + m * j->K;
        const float *srow = j->sa + m * kb_n;
        for (int64_t n = 0; n < j->N; ++n) {
            const uint8_t *wrow = j->qw + n * j->K;
            const float *swrow = j->sw + (n / ORC_GROUP) * kb_n;
            double acc = 0.0;
            for (int64_t k = 0; k < j->K; ++k) {
                double a = dec[arow[k]] * (double)srow[k / ORC_GROUP];
                double b = dec[wrow[k]] * (double)swrow[k / ORC_GROUP];
                acc += a * b;
            }
            j->y[r * j->N + n] = acc;
        }
    }
    return NULL;
}

int orc_block_gemm(const uint8_t *qa, const float *sa, const uint8_t *qw,
                   const float *sw, int64_t M, int64_t N, int64_t K,
                   const int64_t *rows, int64_t nrows, double *y, int nthreads)
{
    int64_t total = rows ? nrows : M;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    if (total < nthreads)
        nthreads = total > 0 ? (int)total : 1;
    pthread_t tid[256];
    gemm_job jobs[256];
    int64_t per = (total + nthreads - 1) / nthreads;
    for (int t = 0; t < nthreads; ++t) {
        gemm_job *j = &jobs[t];
        j->qa = qa; j->sa = sa; j->qw = qw; j->sw = sw;
        j->N = N; j->K = K; j->rows = rows; j->y = y;
        j->r0 = t * per;
        j->r1 = (t + 1) * per < total ? (t + 1) * per : total;
        tid[t] = 0;
        if (j->r0 >= j->r1)
            continue;
        if (pthread_create(&tid[t], NULL, gemm_worker, j) != 0) {
            gemm_worker(j);
            tid[t] = 0;
        }
    }
    for (int t = 0; t < nthreads; ++t)
        if (tid[t])
            pthread_join(tid[t], NULL);
    return nthreads;
}

/* scaled_mm with per-token / per-channel scales, fp64:
 * y[r][n] = sum_k (dec(qa[m][k]) * sa[m]) * (dec(qw[n][k]) * sw[n]),
 * m = rows[r] (or r), summed in increasing k.  qa [M][K], sa [M], qw [N][K],
 * sw [N], y [nrows][N]. */
typedef struct {
    const uint8_t *qa;
    const float *sa;
    const uint8_t *qw;
    const float *sw;
    int64_t N, K;
    const int64_t *rows;
    int64_t r0, r1;
    double *y;
} smm_job;

static void *smm_worker(void *arg)
{
    smm_job *j = (smm_job *)arg;
    double dec[256];
    for (int c = 0; c < 256; ++c)
        dec[c] = orc_e4m3_decode((uint8_t)c);
    for (int64_t r = j->r0; r < j->r1; ++r) {
        int64_t m = j->rows ? j->rows[r] : r;
        const uint8_t *arow = j->qa + m * j->K;
        double sa = (double)j->sa[m];
        for (int64_t n = 0; n < j->N; ++n) {
            const uint8_t *wrow = j->qw + n * j->K;
            double sw = (double)j->sw[n];
            double acc = 0.0;
            for (int64_t k = 0; k < j->K; ++k)
                acc += (dec[arow[k]] * sa) * (dec[wrow[k]] * sw);
            j->y[r * j->N + n] = acc;
        }
    }
    return NULL;
}

int orc_scaled_mm(const uint8_t *qa, const float *sa, const uint8_t *qw, const float *sw,
                  int64_t M, int64_t N, int64_t K, const int64_t *rows, int64_t nrows,
                  double *y, int nthreads)
{
    int64_t total = rows ? nrows : M;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    if (total < nthreads)
        nthreads = total > 0 ? (int)total : 1;
    pthread_t tid[256];
    smm_job jobs[256];
    int64_t per = (total + nthreads - 1) / nthreads;
    for (int t = 0; t < nthreads; ++t) {
        smm_job *j = &jobs[t];
        j->qa = qa; j->sa = sa; j->qw = qw; j->sw = sw;
        j->N = N; j->K = K; j->rows = rows; j->y = y;
        j->r0 = t * per;
        j->r1 = (t + 1) * per < total ? (t + 1) * per : total;
        tid[t] = 0;
        if (j->r0 >= j->r1)
            continue;
        if (pthread_create(&tid[t], NULL, smm_worker, j) != 0) {
            smm_worker(j);
            tid[t] = 0;
        }
    }
    for (int t = 0; t < nthreads; ++t)
        if (tid[t])
            pthread_join(tid[t], NULL);
    return nthreads;
}

/* Row-parallel token quantizer over threads. */
typedef struct {
    const uint16_t *x;
    int64_t K, ldx, ldq, m0, m1;
    uint8_t *q;
    float *s;
    float eps;
    int ue8m0;
} tq_job;

static void *tq_worker(void *arg)
{
    tq_job *j = (tq_job *)arg;
    orc_token_quant(j->x + j->m0 * j->ldx, j->m1 - j->m0, j->K, j->ldx,
                    j->q + j->m0 * j->ldq, j->ldq, j->s + j->m0, j->eps, j->ue8m0);
    return NULL;
}

int orc_token_quant_mt(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                       uint8_t *q, int64_t ldq, float *s, float eps, int ue8m0, int nthreads)
{
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    if (M < nthreads)
        nthreads = M > 0 ? (int)M : 1;
    pthread_t tid[256];
    tq_job jobs[256];
    int64_t per = (M + nthreads - 1) / nthreads;
    for (int t = 0; t < nthreads; ++t) {
        tq_job *j = &jobs[t];
        j->x = x; j->K = K; j->ldx = ldx; j->ldq = ldq;
        j->q = q; j->s = s; j->eps = eps; j->ue8m0 = ue8m0;
        j->m0 = t * per;
        j->m1 = (t + 1) * per < M ? (t + 1) * per : M;
        tid[t] = 0;
        if (j->m0 >= j->m1)
            continue;
        if (pthread_create(&tid[t], NULL, tq_worker, j) != 0) {
            tq_worker(j);
            tid[t] = 0;
        }
    }
    for (int t = 0; t < nthreads; ++t)
        if (tid[t])
            pthread_join(tid[t], NULL);
    return nthreads;
}

/* Row-parallel group quantizer over threads (each row independent). */
typedef struct {
    const uint16_t *x;
    int64_t K, ldx, ldq, lds, m0, m1;
    uint8_t *q;
    float *s;
    float eps;
    int ue8m0;
} quant_job;

static void *quant_worker(void *arg)
{
    quant_job *j = (quant_job *)arg;
    orc_group_quant(j->x + j->m0 * j->ldx, j->m1 - j->m0, j->K, j->ldx,
                    j->q + j->m0 * j->ldq, j->ldq, j->s + j->m0 * j->lds,
                    j->lds, j->eps, j->ue8m0);
    return NULL;
}

int orc_group_quant_mt(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                       uint8_t *q, int64_t ldq, float *s, int64_t lds,
                       float eps, int ue8m0, int nthreads)
{
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    if (M < nthreads)
        nthreads = M > 0 ? (int)M : 1;
    pthread_t tid[256];
    quant_job jobs[256];
    int64_t per = (M + nthreads - 1) / nthreads;
    for (int t = 0; t < nthreads; ++t) {
        quant_job *j = &jobs[t];
        j->x = x; j->K = K; j->ldx = ldx; j->ldq = ldq; j->lds = lds;
        j->q = q; j->s = s; j->eps = eps; j->ue8m0 = ue8m0;
        j->m0 = t * per;
        j->m1 = (t + 1) * per < M ? (t + 1) * per : M;
        tid[t] = 0;
        if (j->m0 >= j->m1)
            continue;
        if (pthread_create(&tid[t], NULL, quant_worker, j) != 0) {
            quant_worker(j);
            tid[t] = 0;
        }
    }
    for (int t = 0; t < nthreads; ++t)
        if (tid[t])
            pthread_join(tid[t], NULL);
    return nthreads;
}

/* 128-row bands of W are independent: threads over bands. */
typedef struct {
    const float *w;
    int64_t N, K, nb0, nb1;
    uint8_t *q;
    float *s;
    float eps;
    int ue8m0;
} wq_job;

static void *wq_worker(void *arg)
{
    wq_job *j = (wq_job *)arg;
    int64_t off = j->nb0 * ORC_GROUP;
    orc_weight_block_quant(j->w + off * j->K, (j->nb1 - j->nb0) * ORC_GROUP, j->K,
                           j->q + off * j->K, j->s + j->nb0 * (j->K / ORC_GROUP),
                           j->eps, j->ue8m0);
    return NULL;
}

int orc_weight_block_quant_mt(const float *w, int64_t N, int64_t K, uint8_t *q,
                              float *s, float eps, int ue8m0, int nthreads)
{
    int64_t nbands = N / ORC_GROUP;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    if (nbands < nthreads)
        nthreads = nbands > 0 ? (int)nbands : 1;
    pthread_t tid[256];
    wq_job jobs[256];
    int64_t per = (nbands + nthreads - 1) / nthreads;
    for (int t = 0; t < nthreads; ++t) {
        wq_job *j = &jobs[t];
        j->w = w; j->N = N; j->K = K; j->q = q; j->s = s;
        j->eps = eps; j->ue8m0 = ue8m0;
        j->nb0 = t * per;
        j->nb1 = (t + 1) * per < nbands ? (t + 1) * per : nbands;
        tid[t] = 0;
        if (j->nb0 >= j->nb1)
            continue;
        if (pthread_create(&tid[t], NULL, wq_worker, j) != 0) {
            wq_worker(j);
            tid[t] = 0;
        }
    }
    for (int t = 0; t < nthreads; ++t)
        if (tid[t])
            pthread_join(tid[t], NULL);
    return nthreads;
}

/* Threaded codec over a flat array (used by the exhaustive codec pin). */
typedef struct {
    const float *t;
    uint8_t *q;
    int64_t i0, i1;
} enc_job;

static void *enc_worker(void *arg)
{
    enc_job *j = (enc_job *)arg;
    orc_e4m3_encode_array(j->t + j->i0, j->q + j->i0, j->i1 - j->i0);
    return NULL;
}

int orc_e4m3_encode_array_mt(const float *t, uint8_t *q, int64_t n, int nthreads)
{
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    pthread_t tid[256];
    enc_job jobs[256];
    int64_t per = (n + nthreads - 1) / nthreads;
    for (int i = 0; i < nthreads; ++i) {
        enc_job *j = &jobs[i];
        j->t = t; j->q = q;
        j->i0 = i * per;
        j->i1 = (i + 1) * per < n ? (i + 1) * per : n;
        tid[i] = 0;
        if (j->i0 >= j->i1)
            continue;
        if (pthread_create(&tid[i], NULL, enc_worker, j) != 0) {
            enc_worker(j);
            tid[i] = 0;
        }
    }
    for (int i = 0; i < nthreads; ++i)
        if (tid[i])
            pthread_join(tid[i], NULL);
    return nthreads;
}
