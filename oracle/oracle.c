/*
 * oracle.c -- plain, slow, obviously correct CPU reference for the fused
 * per-token-quantize -> int8 GEMM -> dequant linear layer (W8A8 / W4A8).
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this file's library. It shares no code, header,
 * table or helper with the GPU library, and includes nothing from it.
 *
 * Sources (page title and section; the pages are about the "Cider" project):
 *  [P2] "在Mac上跑大模型，MLX 不是终点" (juejin.cn), section "W8A8 对称量化：Cider 的选择":
 *       per-token symmetric scale = max|x| / 127, x_int8 = round(x / scale) clamped
 *       to [-128, 127]; output = (x_int8 . w_int8) * scale_x * scale_w.
 *       Section "INT8 TensorOps 内核设计": int8 x int8 products accumulate in int32.
 *       Section "三种量化粒度的实现": per-channel = one weight scale per output
 *       channel; per-group = one scale per 64 or 128 elements, dequant becomes a
 *       segmented multiplication.
 *  [P5] Cider README (gitea mirror), section "量化" (quantization table):
 *       weights symmetric INT8 per-channel or per-group (gs = 64/128); W4A8 weights
 *       symmetric INT4 with zero point 8 packed in uint8 (section "模式");
 *       activations symmetric INT8 per token; INT32 accumulation;
 *       output C = C_int32 * s_act * s_weight. Section "说明": weight scales use
 *       the plain min-max method by default.
 *
 * Readings taken where the pages are silent (each is listed with its reason in
 * the design notes of this repository):
 *  - "round" is IEEE round-half-to-even of the correctly rounded fp32 quotient
 *    x / scale (a true fp32 division, not a multiply by 1/scale);
 *  - scales are fp32; scale = max / 127 is one correctly rounded fp32 division;
 *  - a run whose scale is 0 (all-zero row or group) gets scale 0 and codes 0;
 *  - int4: scale = max / 7, codes clamped to [-8, 7], stored as u = q + 8,
 *    two per byte, even k in the low nibble;
 *  - the int8 GEMM is exact integer arithmetic (accumulated here in int64 and
 *    checked to fit in int32);
 *  - dequantization is given twice: in fp64 (the exact value to within fp64
 *    rounding; per-channel (acc * s_x) * s_w, per-group s_x * sum_g s_w[n,g] * acc_g
 *    with acc_g the int32 sum over group g), and in the pages' fp32 arithmetic
 *    (per-channel two fp32 products left to right; per-group one fp32 fused
 *    multiply-add per group in K order, then the token scale), the value an fp16 /
 *    bf16 output is rounded from;
 *  - int4 weights are per group or, with group size 0, per output channel.
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off -fopenmp -shared -fPIC.
 * Parallelism: an OpenMP "parallel for" over independent rows only.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_BAD_ARG 1
#define ORACLE_OVERFLOW 2

/* IEEE binary16 bit pattern -> float, exactly (every half is a float). */
static float half_to_float(uint16_t h)
{
    uint32_t sign = (uint32_t)(h >> 15) & 1u;
    uint32_t expo = (uint32_t)(h >> 10) & 0x1Fu;
    uint32_t mant = (uint32_t)h & 0x3FFu;
    float mag;
    if (expo == 0) {
        /* zero or subnormal: mant * 2^-24 */
        mag = ldexpf((float)mant, -24);
    } else if (expo == 31) {
        mag = mant ? NAN : INFINITY;
    } else {
        /* (1024 + mant) * 2^(expo - 15 - 10) */
        mag = ldexpf((float)(1024u + mant), (int)expo - 25);
    }
    return sign ? -mag : mag;
}

/* bfloat16 bit pattern -> float: the upper 16 bits of a binary32. */
static float bf16_to_float(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/*
 * Symmetric quantization of one run of n values (a token row, a weight row or
 * a weight group) [P2 "W8A8 对称量化"; P5 "量化"]:
 *   a = max |v|;  s = a / qdiv  (fp32 division);
 *   q = clamp(rint(v / s), lo, hi)  (fp32 division, round half to even).
 * Returns s. A zero scale gives all-zero codes.
 */
static float quantize_run_amax(const float *v, int64_t n, float a, float qdiv, int lo, int hi, int8_t *q);

static float quantize_run(const float *v, int64_t n, float qdiv, int lo, int hi, int8_t *q)
{
    float a = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float m = fabsf(v[i]);
        if (m > a) a = m;
    }
    return quantize_run_amax(v, n, a, qdiv, lo, hi, q);
}

/* The steps after the run's magnitude a: s = a / qdiv, q = clamp(rint(v / s), lo, hi). */
static float quantize_run_amax(const float *v, int64_t n, float a, float qdiv, int lo, int hi, int8_t *q)
{
    float s = a / qdiv;
    for (int64_t i = 0; i < n; ++i) {
        if (s == 0.0f) {
            q[i] = 0;
            continue;
        }
        float t = v[i] / s;
        float r = rintf(t); /* default rounding mode: nearest, ties to even */
        if (r < (float)lo) r = (float)lo;
        if (r > (float)hi) r = (float)hi;
        q[i] = (int8_t)r;
    }
    return s;
}

/*
 * Per-token activation quantization [P2 "W8A8 对称量化"; P5 "Metal Kernel 流水线",
 * step quantize_per_token]. x: M rows of K half (or bf16) values with row
 * stride ldx elements. Outputs x_q int8 [M, K] (row stride K) and s_x [M].
 */
int oracle_quantize_per_token(const uint16_t *x, int x_is_bf16, int64_t M, int64_t K,
                              int64_t ldx, int8_t *x_q, float *s_x)
{
    if (M < 0 || K <= 0 || ldx < K) return ORACLE_BAD_ARG;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        float row[K];
        for (int64_t k = 0; k < K; ++k) {
            uint16_t bits = x[m * ldx + k];
            row[k] = x_is_bf16 ? bf16_to_float(bits) : half_to_float(bits);
        }
        s_x[m] = quantize_run(row, K, 127.0f, -128, 127, x_q + m * K);
    }
    return ORACLE_OK;
}

/*
 * Offline weight quantization, min-max [P5 "说明", "量化", "模式"; P2
 * "三种量化粒度的实现"]. W fp32 [N, K] row-major (row n = output channel n).
 *  bits 8, group_size 0    : s_w [N],        w_q int8 [N, K]
 *  bits 8, group_size g>0  : s_w [N, K/g],   w_q int8 [N, K]   (groups along K)
 *  bits 4, group_size g>0  : s_w [N, K/g],   w_q uint8 [N, K/2]; u = q + 8,
 *                            byte j = u[2j] | u[2j+1] << 4 (even k low nibble)
 *  bits 4, group_size 0    : s_w [N],        w_q uint8 [N, K/2]; the per-column int4 of
 *                            P5 "量化" (one scale per output channel), same packing
 */
int oracle_quantize_weight(const float *W, int64_t N, int64_t K, int bits, int group_size,
                           void *w_q, float *s_w)
{
    if (N < 0 || K <= 0) return ORACLE_BAD_ARG;
    if (bits != 8 && bits != 4) return ORACLE_BAD_ARG;
    if (group_size < 0 || (group_size > 0 && K % group_size != 0)) return ORACLE_BAD_ARG;
    if (bits == 4 && (K % 2 != 0 || group_size % 2 != 0)) return ORACLE_BAD_ARG;
    const int64_t run = group_size ? group_size : K;
    const int64_t G = K / run;
    const float qdiv = bits == 8 ? 127.0f : 7.0f;
    const int lo = bits == 8 ? -128 : -8;
    const int hi = bits == 8 ? 127 : 7;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        int8_t codes[K];
        for (int64_t g = 0; g < G; ++g)
            s_w[n * G + g] = quantize_run(W + n * K + g * run, run, qdiv, lo, hi, codes + g * run);
        if (bits == 8) {
            memcpy((int8_t *)w_q + n * K, codes, (size_t)K);
        } else {
            uint8_t *dst = (uint8_t *)w_q + n * (K / 2);
            for (int64_t j = 0; j < K / 2; ++j) {
                unsigned lo_u = (unsigned)(codes[2 * j] + 8);
                unsigned hi_u = (unsigned)(codes[2 * j + 1] + 8);
                dst[j] = (uint8_t)(lo_u | (hi_u << 4));
            }
        }
    }
    return ORACLE_OK;
}

/* int4 packed [N, K/2] -> int8 codes [N, K]: q[2j] = low nibble - 8, q[2j+1] = high - 8. */
int oracle_unpack_int4(const uint8_t *packed, int64_t N, int64_t K, int8_t *w_q)
{
    if (N < 0 || K <= 0 || K % 2 != 0) return ORACLE_BAD_ARG;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t j = 0; j < K / 2; ++j) {
            uint8_t b = packed[n * (K / 2) + j];
            w_q[n * K + 2 * j] = (int8_t)((int)(b & 0x0F) - 8);
            w_q[n * K + 2 * j + 1] = (int8_t)((int)(b >> 4) - 8);
        }
    return ORACLE_OK;
}

/*
 * Integer GEMM [P2 "INT8 TensorOps 内核设计"; P5 "量化" accumulation INT32]:
 *   acc[m, n] = sum_k x_q[m, k] * w_q[n, k]
 * over columns [k0, k0 + kn) (k0 = 0, kn = K for the full product; a group
 * for the per-group path). Exact: int64 accumulation, then checked against
 * the int32 range. Returns ORACLE_OVERFLOW if any sum leaves int32.
 */
static int gemm_i32_range(const int8_t *x_q, const int8_t *w_q, int64_t M, int64_t N,
                          int64_t K, int64_t k0, int64_t kn, int32_t *acc, int64_t acc_stride)
{
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            int64_t sum = 0;
            for (int64_t k = k0; k < k0 + kn; ++k)
                sum += (int64_t)x_q[m * K + k] * (int64_t)w_q[n * K + k];
            if (sum > INT32_MAX || sum < INT32_MIN) bad = 1;
            acc[(m * N + n) * acc_stride] = (int32_t)sum;
        }
    }
    return bad ? ORACLE_OVERFLOW : ORACLE_OK;
}

int oracle_gemm_i32(const int8_t *x_q, const int8_t *w_q, int64_t M, int64_t N, int64_t K,
                    int32_t *acc)
{
    if (M < 0 || N < 0 || K <= 0) return ORACLE_BAD_ARG;
    return gemm_i32_range(x_q, w_q, M, N, K, 0, K, acc, 1);
}

/*
 * Group accumulators acc_g[m, n, g] = sum over k in [g*gs, (g+1)*gs) of
 * x_q[m, k] * w_q[n, k]. Layout [M, N, G].
 */
int oracle_group_acc(const int8_t *x_q, const int8_t *w_q, int64_t M, int64_t N, int64_t K,
                     int group_size, int32_t *acc_g)
{
    if (M < 0 || N < 0 || K <= 0 || group_size <= 0 || K % group_size != 0) return ORACLE_BAD_ARG;
    const int64_t G = K / group_size;
    int rc = ORACLE_OK;
    for (int64_t g = 0; g < G; ++g) {
        int r = gemm_i32_range(x_q, w_q, M, N, K, g * group_size, group_size, acc_g + g, G);
        if (r != ORACLE_OK) rc = r;
    }
    return rc;
}

/*
 * Per-channel dequant [P2 "W8A8 对称量化"; P5 "量化" C = C_int32 * s_act * s_weight],
 * evaluated left to right in fp64: y[m, n] = (acc[m, n] * s_x[m]) * s_w[n].
 */
int oracle_dequant_pc(const int32_t *acc, const float *s_x, const float *s_w, int64_t M,
                      int64_t N, double *y)
{
    if (M < 0 || N < 0) return ORACLE_BAD_ARG;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            y[m * N + n] = ((double)acc[m * N + n] * (double)s_x[m]) * (double)s_w[n];
    return ORACLE_OK;
}

/*
 * Per-group dequant [P2 "三种量化粒度的实现": each group has its own weight scale,
 * so dequant is a segmented multiplication]:
 *   y[m, n] = s_x[m] * sum_g s_w[n, g] * acc_g[m, n, g]      (fp64)
 * Also returns mag[m, n] = |s_x[m]| * sum_g |s_w[n, g] * acc_g| (the size of the
 * terms being summed; an fp32 evaluation of the sum can only be trusted
 * relative to this, not to |y|, when terms cancel).
 */
int oracle_dequant_pg(const int32_t *acc_g, const float *s_x, const float *s_w, int64_t M,
                      int64_t N, int64_t G, double *y, double *mag)
{
    if (M < 0 || N < 0 || G <= 0) return ORACLE_BAD_ARG;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double t = 0.0, a = 0.0;
            for (int64_t g = 0; g < G; ++g) {
                double term = (double)s_w[n * G + g] * (double)acc_g[(m * N + n) * G + g];
                t += term;
                a += fabs(term);
            }
            y[m * N + n] = (double)s_x[m] * t;
            if (mag) mag[m * N + n] = fabs((double)s_x[m]) * a;
        }
    return ORACLE_OK;
}

/*
 * Per-channel dequant in the pages' own precision [P5 "量化": fp32 scales, INT32 accumulation,
 * C = C_int32 * s_act * s_weight, read left to right]: the int32 sum is converted to fp32
 * (round to nearest even), then multiplied by s_x[m] and by s_w[n], each product rounded to
 * fp32 on its own:
 *   y32[m, n] = ((float)acc[m, n] * s_x[m]) * s_w[n]
 * This is the fp32 value an fp16 / bf16 output is rounded from (once, to nearest even).
 */
int oracle_dequant_pc_f32(const int32_t *acc, const float *s_x, const float *s_w, int64_t M, int64_t N,
                          float *y32)
{
    if (M < 0 || N < 0) return ORACLE_BAD_ARG;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            const float a = (float)acc[m * N + n];
            const float t = a * s_x[m];
            y32[m * N + n] = t * s_w[n];
        }
    return ORACLE_OK;
}

/*
 * Per-group dequant in fp32 [P2 "三种量化粒度的实现": per group its own weight scale, so the
 * dequantization is a segmented multiplication; P5 "量化": fp32 scales]. The segments are
 * folded in K order, each with one correctly rounded fused multiply-add, and the token scale
 * is applied last:
 *   t = +0; for g = 0 .. G-1: t = fmaf((float)acc_g[m, n, g], s_w[n, g], t);  y32 = t * s_x[m]
 */
int oracle_dequant_pg_f32(const int32_t *acc_g, const float *s_x, const float *s_w, int64_t M, int64_t N,
                          int64_t G, float *y32)
{
    if (M < 0 || N < 0 || G <= 0) return ORACLE_BAD_ARG;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            float t = 0.0f;
            for (int64_t g = 0; g < G; ++g)
                t = fmaf((float)acc_g[(m * N + n) * G + g], s_w[n * G + g], t);
            y32[m * N + n] = t * s_x[m];
        }
    return ORACLE_OK;
}

/*
 * Decode matrix-vector product with the activations as they are [P5 "Metal Kernel 流水线",
 * decode (M = 1): the int8 matrix-vector kernel dequantizes the weights as it goes and
 * quantizes no activation; P2 "INT8 TensorOps 内核设计", the two paths: seq_len = 1 takes
 * a dedicated int8 matrix-vector kernel]. x: M rows of K half (or bf16) values, row
 * stride ldx elements; w_q int8 [N, K]; s_w fp32 [N] (group_size 0) or [N, K / group_size]:
 *   y[m, n]   = sum_k x[m, k] * (w_q[n, k] * s_w[n, g(k)])           (fp64)
 *   mag[m, n] = sum_k |x[m, k] * w_q[n, k] * s_w[n, g(k)]|
 * with g(k) = k / group_size (0 for per-channel). Every term is exact in fp64 (a half has
 * 11 significant bits, a code 8, a scale 24), so y is the exact value up to the rounding of
 * the fp64 sum.
 */
int oracle_mv(const uint16_t *x, int x_is_bf16, int64_t M, int64_t K, int64_t ldx, const int8_t *w_q,
              const float *s_w, int64_t N, int group_size, double *y, double *mag)
{
    if (M < 0 || N < 0 || K <= 0 || ldx < K || group_size < 0 || (group_size && K % group_size))
        return ORACLE_BAD_ARG;
    const int64_t G = group_size ? K / group_size : 1;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double t = 0.0, a = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const uint16_t h = x[m * ldx + k];
                const double xv = x_is_bf16 ? (double)bf16_to_float(h) : (double)half_to_float(h);
                const double s = (double)s_w[group_size ? n * G + k / group_size : n];
                const double term = xv * ((double)w_q[n * K + k] * s);
                t += term;
                a += fabs(term);
            }
            y[m * N + n] = t;
            if (mag) mag[m * N + n] = a;
        }
    return ORACLE_OK;
}

/*
 * Offline weight quantization with a clipped scale [P5 "说明": besides the default min-max
 * scale, the scale can come from a percentile of the weights, clip_percentile]. For each run
 * (row, or group of group_size along K) the magnitude a is the pct-th percentile of |v|
 * instead of the maximum, read as the usual linear interpolation between order statistics:
 * with u_0 <= ... <= u_{n-1} the sorted magnitudes, h = (pct * (n - 1)) / 100 in fp64,
 * i = floor(h); a = u_{n-1} if i >= n - 1, else a = u_i + (h - i) * (u_{i+1} - u_i) in fp64,
 * rounded once to fp32. Then the min-max steps with that a: s = a / qdiv, codes clamped, so
 * weights beyond the percentile saturate. pct in (0, 100]; pct = 100 is min-max.
 */
static int cmp_float(const void *x, const void *y)
{
    float a = *(const float *)x, b = *(const float *)y;
    return (a > b) - (a < b);
}

int oracle_quantize_weight_clipped(const float *W, int64_t N, int64_t K, int bits, int group_size, float pct,
                                   void *w_q, float *s_w)
{
    if (N < 0 || K <= 0) return ORACLE_BAD_ARG;
    if (bits != 8 && bits != 4) return ORACLE_BAD_ARG;
    if (group_size < 0 || (group_size > 0 && K % group_size != 0)) return ORACLE_BAD_ARG;
    if (bits == 4 && (K % 2 != 0 || group_size % 2 != 0)) return ORACLE_BAD_ARG;
    if (!(pct > 0.0f && pct <= 100.0f)) return ORACLE_BAD_ARG;
    const int64_t run = group_size ? group_size : K;
    const int64_t G = K / run;
    const float qdiv = bits == 8 ? 127.0f : 7.0f;
    const int lo = bits == 8 ? -128 : -8;
    const int hi = bits == 8 ? 127 : 7;
    const double h = ((double)pct * (double)(run - 1)) / 100.0;
    const int64_t i = (int64_t)floor(h);
    const double f = h - (double)i;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        int8_t codes[K];
        float u[run];
        for (int64_t g = 0; g < G; ++g) {
            const float *v = W + n * K + g * run;
            for (int64_t j = 0; j < run; ++j) u[j] = fabsf(v[j]);
            qsort(u, (size_t)run, sizeof(float), cmp_float);
            const float a = i >= run - 1 ? u[run - 1] : (float)((double)u[i] + f * ((double)u[i + 1] - (double)u[i]));
            s_w[n * G + g] = quantize_run_amax(v, run, a, qdiv, lo, hi, codes + g * run);
        }
        if (bits == 8) {
            memcpy((int8_t *)w_q + n * K, codes, (size_t)K);
        } else {
            uint8_t *dst = (uint8_t *)w_q + n * (K / 2);
            for (int64_t j = 0; j < K / 2; ++j) {
                unsigned lo_u = (unsigned)(codes[2 * j] + 8);
                unsigned hi_u = (unsigned)(codes[2 * j + 1] + 8);
                dst[j] = (uint8_t)(lo_u | (hi_u << 4));
            }
        }
    }
    return ORACLE_OK;
}

/*
 * Decode-step attention [P5 "优化 SDPA（解码注意力）": one query token per head (Q_seq = 1),
 * no mask, grouped-query heads sharing a KV head]. q [B, Hq, D]; k, v [B, Hkv, Ncap, D] of
 * which the first N rows per head are used; half or bf16 bit patterns. Query head h reads KV
 * head h / (Hq / Hkv). In fp64:
 *   s_n = scale * sum_d q[d] k[n, d];  p_n = exp(s_n - max s);  o[d] = sum_n p_n v[n, d] / sum_n p_n
 * Also returns per (b, h, d) vmag = sum_n p_n |v[n, d]| / sum_n p_n, and per (b, h)
 * smag = max_n scale * sum_d |q[d] k[n, d]| (the sizes an fp32 evaluation's errors scale with).
 */
int oracle_sdpa_decode(const uint16_t *q, const uint16_t *k, const uint16_t *v, int is_bf16, int64_t B, int64_t Hq,
                       int64_t Hkv, int64_t N, int64_t Ncap, int64_t D, double scale, double *o, double *vmag,
                       double *smag)
{
    if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || N <= 0 || Ncap < N || D <= 0) return ORACLE_BAD_ARG;
    const int64_t G = Hq / Hkv;
#pragma omp parallel for schedule(static)
    for (int64_t bh = 0; bh < B * Hq; ++bh) {
        const int64_t b = bh / Hq, h = bh % Hq, kvh = h / G;
        const uint16_t *qh = q + bh * D;
        const uint16_t *kb = k + (b * Hkv + kvh) * Ncap * D;
        const uint16_t *vb = v + (b * Hkv + kvh) * Ncap * D;
        double *s = (double *)malloc((size_t)N * sizeof(double));
        double mx = -INFINITY, sm = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            double t = 0.0, a = 0.0;
            for (int64_t d = 0; d < D; ++d) {
                const double qv = is_bf16 ? (double)bf16_to_float(qh[d]) : (double)half_to_float(qh[d]);
                const double kv = is_bf16 ? (double)bf16_to_float(kb[n * D + d]) : (double)half_to_float(kb[n * D + d]);
                t += qv * kv;
                a += fabs(qv * kv);
            }
            s[n] = scale * t;
            if (s[n] > mx) mx = s[n];
            if (scale * a > sm) sm = scale * a;
        }
        double l = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            s[n] = exp(s[n] - mx);
            l += s[n];
        }
        for (int64_t d = 0; d < D; ++d) {
            double acc = 0.0, am = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                const double vv = is_bf16 ? (double)bf16_to_float(vb[n * D + d]) : (double)half_to_float(vb[n * D + d]);
                acc += s[n] * vv;
                am += s[n] * fabs(vv);
            }
            o[bh * D + d] = acc / l;
            if (vmag) vmag[bh * D + d] = am / l;
        }
        if (smag) smag[bh] = sm;
        free(s);
    }
    return ORACLE_OK;
}

/*
 * RMSNorm with the per-token quantization folded in: the producer of a linear layer's
 * input emits int8 codes and a per-token scale instead of a normalized half row, so the
 * activation quantization needs no pass of its own [P5 "Metal Kernel 流水线": the layer
 * runs quantize_per_token, then the GEMM, as two dispatches; P2 "W8A8 对称量化": the online
 * quantization must not become the new bottleneck]. The pages name no producer; the one
 * taken is RMSNorm with a per-channel weight g, the norm in front of the q/k/v and
 * gate/up linears of a Qwen3 block:
 *     n[k] = x[k] * g[k] / sqrt(mean_k x[k]^2 + eps).
 * The row factor 1 / sqrt(...) is positive and common to the row, so it cancels in
 * n[k] / (max_k |n[k]| / 127) and moves into the scale:
 *     u[k]  = x[k] * g[k]                 (one fp32 multiply)
 *     x_q, s_u = the symmetric quantization of the run u (as quantize_per_token)
 *     r     = 1 / sqrt(sum_k x[k]^2 / K + eps)   (fp64; every square is exact in fp64)
 *     s_x   = s_u * r                     (fp64, returned for the caller's tolerance)
 * so s_x * x_q[k] approximates n[k] within half a quantization step. x and g: half or bf16
 * bit patterns; x rows of stride ldx elements; outputs x_q [M, K], s_u [M] (fp32) and
 * s_x [M] (fp64).
 */
int oracle_rmsnorm_quantize(const uint16_t *x, int x_is_bf16, const uint16_t *g, int g_is_bf16, double eps,
                            int64_t M, int64_t K, int64_t ldx, int8_t *x_q, float *s_u, double *s_x)
{
    if (M < 0 || K <= 0 || ldx < K || !(eps >= 0.0)) return ORACLE_BAD_ARG;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        float u[K];
        double ss = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const uint16_t xb = x[m * ldx + k];
            const float xv = x_is_bf16 ? bf16_to_float(xb) : half_to_float(xb);
            const float gv = g_is_bf16 ? bf16_to_float(g[k]) : half_to_float(g[k]);
            u[k] = xv * gv;
            ss += (double)xv * (double)xv;
        }
        const float s = quantize_run(u, K, 127.0f, -128, 127, x_q + m * K);
        s_u[m] = s;
        /* an all-zero row has zero codes; its scale is 0 (also when eps = 0) */
        s_x[m] = s == 0.0f ? 0.0 : (double)s * (1.0 / sqrt(ss / (double)K + eps));
    }
    return ORACLE_OK;
}

/*
 * exp in fp32 by a fixed sequence of fp32 operations, the evaluation the SwiGLU producer
 * below specifies (and its GPU kernel follows), so that both sides take the same code
 * decisions. Range reduction after Cody and Waite: x = k ln 2 + r with k = rint(x log2 e),
 * r = x - k ln 2 formed with two fused multiply-adds against ln 2 split into its fp32
 * rounding and the fp32 rounding of the remainder; |r| <= ln 2 / 2 + tiny. e^r is the Taylor
 * polynomial of degree 7 (coefficients 1 / n!, rounded to fp32) by Horner's rule with fused
 * multiply-adds (truncation error below |r|^8 / 8! < 5.3e-9 relative); the result is p * 2^k,
 * 2^k built exactly. The argument is first clamped to [-87, 88], which keeps k in
 * [-126, 127] (2^k a normal number) and the result finite.
 */
static float exp_steps(float x)
{
    const float log2e = 0x1.715476p+0f;   /* log2(e) rounded to fp32 */
    const float ln2_hi = 0x1.62e43p-1f;   /* ln 2 rounded to fp32 */
    const float ln2_lo = -0x1.05c61p-29f; /* ln 2 - ln2_hi rounded to fp32 */
    if (x > 88.0f) x = 88.0f;
    if (x < -87.0f) x = -87.0f;
    const float k = rintf(x * log2e);
    float r = fmaf(-k, ln2_hi, x);
    r = fmaf(-k, ln2_lo, r);
    float p = 1.0f / 5040.0f;
    p = fmaf(p, r, 1.0f / 720.0f);
    p = fmaf(p, r, 1.0f / 120.0f);
    p = fmaf(p, r, 1.0f / 24.0f);
    p = fmaf(p, r, 1.0f / 6.0f);
    p = fmaf(p, r, 0.5f);
    p = fmaf(p, r, 1.0f);
    p = fmaf(p, r, 1.0f);
    uint32_t bits = (uint32_t)((int)k + 127) << 23; /* 2^k, k in [-126, 127] */
    float two_k;
    memcpy(&two_k, &bits, sizeof two_k);
    return p * two_k;
}

/*
 * SwiGLU with the per-token quantization folded in: the producer of the down projection's
 * input writes its int8 codes and per-token scale directly [P5 "Metal Kernel 流水线": the
 * quantization is otherwise its own dispatch before the GEMM; P2 "W8A8 对称量化": the online
 * quantization must not become the bottleneck; P5 "ANE+GPU 异构张量并行", 关键设计选择: the
 * block's input preparation is shared]. The pages name no MLP; the one taken is the gated
 * MLP of a Qwen3 block, whose down projection reads h = silu(gate) * up, gate and up being
 * the two halves of the gate/up projection's output. In fp32:
 *     e = exp_steps(-g);  s = g / (1 + e)  (IEEE division);  h = s * u
 * then the per-token quantization of the run h exactly as quantize_per_token does it (h is
 * never rounded to fp16 / bf16 first). gate / up: M rows of I half or bf16 values with row
 * strides ldg / ldu elements. Outputs x_q [M, I], s_x [M] and, if h is not NULL, h [M, I]
 * (fp32, for the tests).
 */
int oracle_swiglu_quantize(const uint16_t *gate, const uint16_t *up, int is_bf16, int64_t M, int64_t I, int64_t ldg,
                           int64_t ldu, int8_t *x_q, float *s_x, float *h)
{
    if (M < 0 || I <= 0 || ldg < I || ldu < I) return ORACLE_BAD_ARG;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        float row[I];
        for (int64_t i = 0; i < I; ++i) {
            const uint16_t gb = gate[m * ldg + i], ub = up[m * ldu + i];
            const float g = is_bf16 ? bf16_to_float(gb) : half_to_float(gb);
            const float u = is_bf16 ? bf16_to_float(ub) : half_to_float(ub);
            const float e = exp_steps(-g);
            const float s = g / (1.0f + e);
            row[i] = s * u;
            if (h) h[m * I + i] = row[i];
        }
        s_x[m] = quantize_run(row, I, 127.0f, -128, 127, x_q + m * I);
    }
    return ORACLE_OK;
}

/* exp_steps over an array (for the tests' checks of the evaluation itself). */
int oracle_exp_steps(const float *x, int64_t n, float *y)
{
    if (n < 0) return ORACLE_BAD_ARG;
    for (int64_t i = 0; i < n; ++i) y[i] = exp_steps(x[i]);
    return ORACLE_OK;
}
