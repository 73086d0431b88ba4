/*
 * TEST INFRASTRUCTURE ONLY.  A plain, slow, obviously correct CPU definition
 * of the TQ2_0 ternary decode matvec, used to check the GPU library.  Only
 * the tests, the smoke check and the benchmark's CPU-baseline leg may load
 * it; the GPU library never does, and the two share no code.
 *
 * Source of every definition below: the page "BitCPM ternary (1.58-bit)"
 * (coreai-model-zoo knowledge base) for the TQ2_0 format, the pack rule and
 * the block decomposition, and the page "gemma4 wNa8o8 requires int8
 * activations" for the static int8 activation quantizer.  Where the pages
 * leave a step open, the reading taken is stated at the function.
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off -fopenmp -shared -fPIC.
 * No SIMD intrinsics, no blocking: one row at a time, k in ascending order.
 *
 * Byte layout read and written here (our own; the pages fix no interleave):
 *   codes  : uint8  [N][K/4]   element k of row n sits in byte n*(K/4)+k/4
 *                              at bits 2*(k%4) .. 2*(k%4)+1 (LSB first)
 *   scales : uint16 [N][K/256] IEEE binary16 bit patterns, one per block
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define BLOCK 256

/* ---- IEEE binary16 <-> binary32, written from the format definition ---- */

/* Exact value of a binary16 bit pattern (subnormals kept). */
static double half_value(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int f = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);                 /* subnormal: f * 2^-24 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);     /* (1 + f/1024) * 2^(e-15) */
    return sign ? -v : v;
}

float oracle_half_to_float(uint16_t h) { return (float)half_value(h); }

/* Round a non-negative finite float to binary16, nearest, ties to even. */
uint16_t oracle_float_to_half(float xf)
{
    if (isnan(xf)) return 0x7E00;
    uint16_t sign = signbit(xf) ? 0x8000 : 0;
    double a = fabs((double)xf);
    if (a >= 65520.0) return sign | 0x7C00;       /* past the last midpoint */
    if (a < ldexp(1.0, -14)) {                     /* subnormal range */
        double m = nearbyint(a * ldexp(1.0, 24)); /* units of 2^-24, RNE */
        return sign | (uint16_t)m;                 /* m == 1024 is 2^-14 */
    }
    int ex;
    frexp(a, &ex);                                 /* a in [2^(ex-1), 2^ex) */
    int E = ex - 1;
    double m = nearbyint(ldexp(a, 10 - E));       /* in [1024, 2048], RNE */
    if (m == 2048.0) { m = 1024.0; E += 1; }
    if (E + 15 >= 31) return sign | 0x7C00;
    return sign | (uint16_t)(((E + 15) << 10) | ((int)m - 1024));
}

/* ---- unpack one row (field order above) ---- */

static int code_at(const uint8_t *row_codes, int64_t k)
{
    return (row_codes[k >> 2] >> (2 * (k & 3))) & 3;
}

/* Dequantize row n: W[k] = d_b * (q - 1).  Exact in fp32 since the value
 * is one of -d, 0, +d ("BitCPM ternary", TQ2_0 definition). */
static void dequant_row(const uint8_t *codes, const uint16_t *scales,
                        int64_t n, int64_t K, float *out)
{
    const uint8_t *rc = codes + n * (K / 4);
    const uint16_t *rs = scales + n * (K / BLOCK);
    for (int64_t k = 0; k < K; ++k) {
        float d = oracle_half_to_float(rs[k / BLOCK]);
        out[k] = d * (float)(code_at(rc, k) - 1);
    }
}

void oracle_dequant(const uint8_t *codes, const uint16_t *scales,
                    int64_t N, int64_t K, float *W)
{
    for (int64_t n = 0; n < N; ++n) dequant_row(codes, scales, n, K, W + n * K);
}

/* ---- pack ("BitCPM ternary": d = max|W| over the block, code = round(W/d)+1)
 * Readings: d is max|W| rounded to binary16 (nearest, ties to even); codes
 * are taken against that rounded d with IEEE fp32 division, rounded half to
 * even and clamped to [-1, 1]; an all-zero block (d == 0) gets code 1
 * everywhere.  A block holding a non-finite value, or whose max rounds to
 * binary16 infinity, is counted as bad; its bytes are then unspecified. */
int64_t oracle_pack(const float *W, int64_t N, int64_t K,
                    uint8_t *codes, uint16_t *scales)
{
    int64_t bad = 0;
    int64_t BK = K / BLOCK;
    memset(codes, 0, (size_t)(N * (K / 4)));
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t b = 0; b < BK; ++b) {
            const float *w = W + n * K + b * BLOCK;
            float m = 0.0f;
            int nonfinite = 0;
            for (int i = 0; i < BLOCK; ++i) {
                float a = fabsf(w[i]);
                if (!isfinite(a)) nonfinite = 1;
                else if (a > m) m = a;
            }
            uint16_t hb = oracle_float_to_half(m);
            if (nonfinite || hb == 0x7C00) ++bad;
            scales[n * BK + b] = hb;
            float d = oracle_half_to_float(hb);
            uint8_t *rc = codes + n * (K / 4) + b * (BLOCK / 4);
            for (int i = 0; i < BLOCK; ++i) {
                int q = 1;
                if (d != 0.0f && isfinite(d)) {
                    float c = rintf(w[i] / d);
                    if (isnan(c)) c = 0.0f;
                    if (c < -1.0f) c = -1.0f;
                    if (c > 1.0f) c = 1.0f;
                    q = (int)c + 1;
                }
                rc[i >> 2] |= (uint8_t)(q << (2 * (i & 3)));
            }
        }
    }
    return bad;
}

/* ---- fp16-activation matvec: y_n = sum_k W_nk * x_k, the plain definition
 * (the block form on the page is an identity of this sum).  Summed in fp64
 * in ascending k, rounded once to fp32.  Rows are independent. */
void oracle_gemv(const uint8_t *codes, const uint16_t *scales, int64_t N,
                 int64_t K, const uint16_t *x, float *y)
{
    double *xd = (double *)malloc(sizeof(double) * (size_t)K);
    for (int64_t k = 0; k < K; ++k) xd[k] = half_value(x[k]);
#pragma omp parallel
    {
        float *w = (float *)malloc(sizeof(float) * (size_t)K);
#pragma omp for schedule(static)
        for (int64_t n = 0; n < N; ++n) {
            dequant_row(codes, scales, n, K, w);
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) acc += (double)w[k] * xd[k];
            y[n] = (float)acc;
        }
        free(w);
    }
    free(xd);
}

/* ---- static int8 activation quantizer (page "gemma4 wNa8o8 requires int8
 * activations": clamp(round(x/s), -128, 127)).  Readings: x/s is one IEEE
 * fp32 division; round is half to even; the clamp is applied in float before
 * the conversion.  Non-finite x is unspecified (NaN maps to 0 here). */
void oracle_quantize_i8(const uint16_t *x, int64_t K, float s, int8_t *xq)
{
    for (int64_t k = 0; k < K; ++k) {
        float v = oracle_half_to_float(x[k]) / s;
        float r = rintf(v);
        if (isnan(r)) r = 0.0f;
        if (r < -128.0f) r = -128.0f;
        if (r > 127.0f) r = 127.0f;
        xq[k] = (int8_t)r;
    }
}

/* Block partials P_nb = sum_{k in b} xq_k * (q_nk - 1), exact integers. */
void oracle_partials_i8(const uint8_t *codes, int64_t N, int64_t K,
                        const int8_t *xq, int32_t *P)
{
    int64_t BK = K / BLOCK;
    for (int64_t n = 0; n < N; ++n) {
        const uint8_t *rc = codes + n * (K / 4);
        for (int64_t b = 0; b < BK; ++b) {
            int64_t acc = 0;
            for (int64_t k = b * BLOCK; k < (b + 1) * BLOCK; ++k)
                acc += (int64_t)xq[k] * (code_at(rc, k) - 1);
            P[n * BK + b] = (int32_t)acc;
        }
    }
}

/* d * 2^24 as an exact integer, from the binary16 fields. */
static int64_t scale_times_2p24(uint16_t h)
{
    int e = (h >> 10) & 31;
    int64_t f = h & 1023;
    int64_t D = (e == 0) ? f : ((1024 | f) << (e - 1));
    return (h & 0x8000) ? -D : D;
}

/* int8 matvec on pre-quantized activations.  y_n = sum_b d_b * s * P_nb.
 * Reading: the sum is formed exactly, A_n = sum_b (d_b*2^24) * P_nb in int64
 * (exact while K <= 65280), then y_n = fl32((fl64(A_n) * s) * 2^-24).  This
 * makes the result independent of summation order.  `partials` (nullable)
 * receives P as [N][K/256]. */
void oracle_gemv_i8q(const uint8_t *codes, const uint16_t *scales, int64_t N,
                     int64_t K, const int8_t *xq, float s, float *y,
                     int32_t *partials)
{
    int64_t BK = K / BLOCK;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        const uint8_t *rc = codes + n * (K / 4);
        int64_t A = 0;
        for (int64_t b = 0; b < BK; ++b) {
            int64_t P = 0;
            for (int64_t k = b * BLOCK; k < (b + 1) * BLOCK; ++k)
                P += (int64_t)xq[k] * (code_at(rc, k) - 1);
            if (partials) partials[n * BK + b] = (int32_t)P;
            A += scale_times_2p24(scales[n * BK + b]) * P;
        }
        y[n] = (float)(((double)A * (double)s) * 0x1p-24);
    }
}

/* Quantize, then the int8 matvec. */
void oracle_gemv_i8(const uint8_t *codes, const uint16_t *scales, int64_t N,
                    int64_t K, const uint16_t *x, float s, float *y)
{
    int8_t *xq = (int8_t *)malloc((size_t)K);
    oracle_quantize_i8(x, K, s, xq);
    oracle_gemv_i8q(codes, scales, N, K, xq, s, y, NULL);
    free(xq);
}

/* Number of threads the OpenMP loops above run with. */
#ifdef _OPENMP
#include <omp.h>
int oracle_threads(void) { return omp_get_max_threads(); }
void oracle_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
#else
int oracle_threads(void) { return 1; }
void oracle_set_threads(int n) { (void)n; }
#endif

/* ---- output requantization (page "gemma4 wNa8o8 requires int8
 * activations", the recipe paragraph: the int8 matmul's result is
 * requantized to int8 with the output activation scale, then dequantized).
 * Readings as for the input quantizer: one IEEE fp32 division, rint (ties to
 * even), clamp in float; the dequantized value is one fp32 product. */
void oracle_requant_i8(const float *y, int64_t N, float s_out, int8_t *y_q,
                       float *y_deq)
{
    for (int64_t n = 0; n < N; ++n) {
        float r = rintf(y[n] / s_out);
        if (isnan(r)) r = 0.0f;
        if (r < -128.0f) r = -128.0f;
        if (r > 127.0f) r = 127.0f;
        y_q[n] = (int8_t)r;
        if (y_deq) y_deq[n] = r * s_out;
    }
}

/* ---- SiLU(gate) * up in fp64 (reference for the fused MLP epilogue):
 * silu(v) = v / (1 + e^-v). */
void oracle_silu_mul(const float *g, const float *u, int64_t N, double *h)
{
    for (int64_t n = 0; n < N; ++n) {
        double v = (double)g[n];
        h[n] = v / (1.0 + exp(-v)) * (double)u[n];
    }
}

/* ---- several tokens: Y[m] = W X[m] for each token m, the matvec above
 * applied token by token (the page's prefill runs one matvec per token). */
void oracle_gemm(const uint8_t *codes, const uint16_t *scales, int64_t N,
                 int64_t K, const uint16_t *X, int64_t M, float *Y)
{
    for (int64_t m = 0; m < M; ++m) oracle_gemv(codes, scales, N, K, X + m * K, Y + m * N);
}
