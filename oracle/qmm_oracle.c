/*
 * qmm_oracle.c -- plain, slow, obviously correct CPU reference for
 * block-quantized MUL_MAT (decode GEMV and prefill GEMM).
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the
 * benchmark's CPU-baseline leg, never by the GPU library.  Nothing here is
 * shared with the GPU path.  See qmm_oracle.h for the contract of each
 * function and the pages each one follows.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -shared -fPIC.
 * The rounding steps rely on the default IEEE rounding mode (round to
 * nearest, ties to even) for nearbyint(), and on binary32 division being
 * correctly rounded (SSE arithmetic on x86-64, no excess precision).
 */
#include "qmm_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------
 * IEEE-754 binary16 / bfloat16 conversions.
 *
 * Written from the definitions: a finite value is sign * n * 2^e with an
 * integer significand n of p bits (p = 11 for binary16, 8 for bfloat16) and a
 * bounded exponent; below the smallest normal the quantum stays fixed
 * (subnormals).  Conversion from binary32 picks the nearest representable
 * value, ties to the one with an even significand, and overflows to infinity
 * when the rounded magnitude exceeds the largest finite value.  All scaling
 * below is by powers of two in binary64, hence exact, so nearbyint() is the
 * only rounding step.
 * ------------------------------------------------------------------------ */

uint16_t orc_f32_to_f16(float f)
{
    uint32_t bits;
    memcpy(&bits, &f, 4);
    const uint16_t sign = (bits >> 31) ? 0x8000u : 0u;
    if (isnan(f)) return (uint16_t)(sign | 0x7E00u);
    if (isinf(f)) return (uint16_t)(sign | 0x7C00u);
    const double a = fabs((double)f);
    /* Largest finite binary16: 65504 = 2047 * 2^5.  The next step up would be
     * 65536; the tie 65520 goes to the even significand (2048 -> 2^16), which
     * overflows, so everything from 65520 up becomes infinity. */
    if (a >= 65520.0) return (uint16_t)(sign | 0x7C00u);
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: value = n * 2^-24, n in [0, 1024]; n == 1024 is the
         * smallest normal, whose encoding is the same integer. */
        const double n = nearbyint(ldexp(a, 24));
        return (uint16_t)(sign | (uint16_t)n);
    }
    int e;
    frexp(a, &e);            /* a in [2^(e-1), 2^e) */
    int E = e - 1;           /* a in [2^E, 2^(E+1)), E in [-14, 15] */
    double n = nearbyint(ldexp(a, 10 - E)); /* 11-bit significand, in [1024, 2048] */
    if (n == 2048.0) { n = 1024.0; E += 1; }
    return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)(n - 1024.0));
}

float orc_f16_to_f32(uint16_t h)
{
    const int sign = h >> 15;
    const int ex = (h >> 10) & 31;
    const int man = h & 1023;
    double v;
    if (ex == 31) v = man ? NAN : INFINITY;
    else if (ex == 0) v = ldexp((double)man, -24);
    else v = ldexp((double)(1024 + man), ex - 25);
    return (float)(sign ? -v : v);
}

uint16_t orc_f32_to_bf16(float f)
{
    uint32_t bits;
    memcpy(&bits, &f, 4);
    const uint16_t sign = (bits >> 31) ? 0x8000u : 0u;
    if (isnan(f)) return (uint16_t)(sign | 0x7FC0u);
    if (isinf(f)) return (uint16_t)(sign | 0x7F80u);
    const double a = fabs((double)f);
    if (a < ldexp(1.0, -126)) {
        /* subnormal range: value = n * 2^-133, n in [0, 128] */
        const double n = nearbyint(ldexp(a, 133));
        return (uint16_t)(sign | (uint16_t)n);
    }
    int e;
    frexp(a, &e);
    int E = e - 1;                          /* a in [2^E, 2^(E+1)) */
    double n = nearbyint(ldexp(a, 7 - E));  /* 8-bit significand, in [128, 256] */
    if (n == 256.0) { n = 128.0; E += 1; }
    if (E + 127 >= 255) return (uint16_t)(sign | 0x7F80u); /* overflow */
    return (uint16_t)(sign | (uint16_t)((E + 127) << 7) | (uint16_t)(n - 128.0));
}

float orc_bf16_to_f32(uint16_t h)
{
    /* bfloat16 is, by definition, the upper half of a binary32 word. */
    const uint32_t bits = (uint32_t)h << 16;
    float f;
    memcpy(&f, &bits, 4);
    return f;
}

void orc_f32_to_f16_n(const float *src, uint16_t *dst, size_t n)
{
    for (size_t i = 0; i < n; ++i) dst[i] = orc_f32_to_f16(src[i]);
}
void orc_f16_to_f32_n(const uint16_t *src, float *dst, size_t n)
{
    for (size_t i = 0; i < n; ++i) dst[i] = orc_f16_to_f32(src[i]);
}
void orc_f32_to_bf16_n(const float *src, uint16_t *dst, size_t n)
{
    for (size_t i = 0; i < n; ++i) dst[i] = orc_f32_to_bf16(src[i]);
}
void orc_bf16_to_f32_n(const uint16_t *src, float *dst, size_t n)
{
    for (size_t i = 0; i < n; ++i) dst[i] = orc_bf16_to_f32(src[i]);
}

/* ------------------------------------------------------------------------
 * Block quantization (Development Guide §6.1: 32 values share one FP16
 * scale; llama.cpp Guide §2.2: w_i ~= Delta * q_i with Delta taken from the
 * block's largest magnitude).
 *
 * Steps, in binary32:
 *   amax  = max_i |w_i|
 *   s     = amax / 127   (Q8_0)    or   amax / 8   (Q4_0)
 *   s_h   = fp16(s), round to nearest even; d = the value of s_h
 *   d == 0: every code is the zero code (q = 0, nibble = 8)
 *   else    q_i = roundf(w_i / d) (half away from zero), the quotient one
 *           correctly rounded binary32 division by the stored scale;
 *           Q8_0 clamps q to [-127, 127]; Q4_0 stores nibble q + 8 clamped
 *           to [0, 15] (offset binary for q in [-8, 7]).
 * ------------------------------------------------------------------------ */

static float block_amax(const float *w, int n)
{
    float amax = 0.0f;
    for (int i = 0; i < n; ++i) {
        const float v = fabsf(w[i]);
        if (v > amax) amax = v;
    }
    return amax;
}

/* The Q8 steps over a block of n values (scale divisor 127). */
static void quantize_q8(const float *w, int n, uint16_t *scale_bits, int8_t *q)
{
    const float s = block_amax(w, n) / 127.0f;
    const uint16_t h = orc_f32_to_f16(s);
    const float d = orc_f16_to_f32(h);
    *scale_bits = h;
    for (int i = 0; i < n; ++i) {
        if (d == 0.0f) { q[i] = 0; continue; }
        float r = roundf(w[i] / d);
        if (r > 127.0f) r = 127.0f;
        if (r < -127.0f) r = -127.0f;
        q[i] = (int8_t)r;
    }
}

/* The Q4 steps over a block of n values with scale divisor div (8: the
 * offset-binary Q4_0 rule, nibble = clamp(q + 8, 0, 15); 7: the pages'
 * symmetric rule, q clamped to [-8, 7], stored as q + 8 -- the same thing). */
static void quantize_q4(const float *w, int n, float div, uint16_t *scale_bits, uint8_t *nib)
{
    const float s = block_amax(w, n) / div;
    const uint16_t h = orc_f32_to_f16(s);
    const float d = orc_f16_to_f32(h);
    *scale_bits = h;
    for (int i = 0; i < n; ++i) {
        if (d == 0.0f) { nib[i] = 8; continue; }
        float q = roundf(w[i] / d);
        if (q > 7.0f) q = 7.0f;
        if (q < -8.0f) q = -8.0f;
        nib[i] = (uint8_t)(q + 8.0f);
    }
}

void orc_quantize_block_q8_0(const float w[32], uint16_t *scale_bits, int8_t q[32])
{
    quantize_q8(w, 32, scale_bits, q);
}

void orc_quantize_block_q4_0(const float w[32], uint16_t *scale_bits, uint8_t nib[32])
{
    quantize_q4(w, 32, 8.0f, scale_bits, nib);
}

/* The pages' own Q4 rule ("A Complete Guide to llama.cpp and Customization
 * with C++", §2.2): Delta = max|w| / 7, q in [-8, 7]; stored, like Q4_0, as
 * the offset-binary nibble q + 8 with the fp16 Delta. */
void orc_quantize_block_q4_sym7(const float w[32], uint16_t *scale_bits, uint8_t nib[32])
{
    quantize_q4(w, 32, 7.0f, scale_bits, nib);
}

/* 64-weight blocks (same page and section: the block length is usually 32
 * or 64): the same steps over 64 values sharing one fp16 scale. */
void orc_quantize_block_q8_b64(const float w[64], uint16_t *scale_bits, int8_t q[64])
{
    quantize_q8(w, 64, scale_bits, q);
}

void orc_quantize_block_q4_b64(const float w[64], int divisor, uint16_t *scale_bits, uint8_t nib[64])
{
    quantize_q4(w, 64, (float)divisor, scale_bits, nib);
}

/* ------------------------------------------------------------------------
 * Row-planar packing (see qmm_oracle.h).
 * ------------------------------------------------------------------------ */

static size_t align16(size_t v) { return (v + 15u) & ~(size_t)15u; }

static int is_quant(int type)
{
    return type == ORC_Q8_0 || type == ORC_Q4_0 || type == ORC_Q8_B64 || type == ORC_Q4_B64;
}
static int is_q8(int type) { return type == ORC_Q8_0 || type == ORC_Q8_B64; }
/* Weights per block (one fp16 scale each). */
static int64_t block_len(int type) { return (type == ORC_Q8_B64 || type == ORC_Q4_B64) ? 64 : 32; }
/* Bytes of scales before the codes: 2 per block, padded to 16. */
static size_t scale_bytes(int type, int64_t K) { return align16((size_t)(2 * (K / block_len(type)))); }

size_t orc_row_size(int type, int64_t K)
{
    if (K < 0) return 0;
    switch (type) {
    case ORC_F32:  return (size_t)K * 4u;
    case ORC_F16:  return (size_t)K * 2u;
    case ORC_BF16: return (size_t)K * 2u;
    case ORC_Q8_0:
    case ORC_Q8_B64: return scale_bytes(type, K) + align16((size_t)K);
    case ORC_Q4_0:
    case ORC_Q4_B64: return scale_bytes(type, K) + align16((size_t)K / 2u);
    default:       return 0;
    }
}

int orc_quantize_rows(int type, const float *w, int64_t K, int64_t M,
                      uint8_t *dst, size_t pitch)
{
    return orc_quantize_rows_rule(type, ORC_RULE_DEFAULT, w, K, M, dst, pitch);
}

int orc_quantize_rows_rule(int type, int rule, const float *w, int64_t K, int64_t M,
                           uint8_t *dst, size_t pitch)
{
    if (!is_quant(type) || K < 0 || M < 0 || (K % block_len(type)) != 0) return -1;
    if (rule != ORC_RULE_DEFAULT && !(rule == ORC_RULE_Q4_SYM7 && !is_q8(type))) return -1;
    if (pitch < orc_row_size(type, K)) return -1;
    const int64_t bl = block_len(type);
    const int64_t nblk = K / bl;
    const size_t qoff = scale_bytes(type, K);
    for (int64_t m = 0; m < M; ++m) {
        uint8_t *row = dst + (size_t)m * pitch;
        memset(row, 0, orc_row_size(type, K));
        for (int64_t b = 0; b < nblk; ++b) {
            const float *blk = w + (size_t)m * (size_t)K + (size_t)(b * bl);
            uint16_t sb;
            if (is_q8(type)) {
                int8_t q[64];
                quantize_q8(blk, (int)bl, &sb, q);
                memcpy(row + qoff + (size_t)(b * bl), q, (size_t)bl);   /* code k at qoff + k */
            } else {
                uint8_t nib[64];
                quantize_q4(blk, (int)bl, rule == ORC_RULE_Q4_SYM7 ? 7.0f : 8.0f, &sb, nib);
                /* each run of 32 codes packs like a Q4_0 block: byte j of the
                 * run holds code j (low nibble) and code j + 16 (high) */
                for (int64_t h = 0; h < bl / 32; ++h) {
                    uint8_t *qb = row + qoff + (size_t)((b * bl + 32 * h) / 2);
                    for (int j = 0; j < 16; ++j)
                        qb[j] = (uint8_t)(nib[32 * h + j] | (nib[32 * h + j + 16] << 4));
                }
            }
            row[2 * b] = (uint8_t)(sb & 0xFF);
            row[2 * b + 1] = (uint8_t)(sb >> 8);
        }
    }
    return 0;
}

/* One row of W' (the exact dequantized weights, Development Guide §6.2:
 * multiply each unpacked code by the block's scale).  scale * code is exact
 * in binary32: at most 11 + 8 significant bits. */
static void dequantize_row(int type, const uint8_t *row, int64_t K, float *out)
{
    if (type == ORC_F32) {
        memcpy(out, row, (size_t)K * 4u);
        return;
    }
    if (type == ORC_F16 || type == ORC_BF16) {
        for (int64_t k = 0; k < K; ++k) {
            const uint16_t h = (uint16_t)(row[2 * k] | (row[2 * k + 1] << 8));
            out[k] = (type == ORC_F16) ? orc_f16_to_f32(h) : orc_bf16_to_f32(h);
        }
        return;
    }
    const size_t qoff = scale_bytes(type, K);
    const int64_t bl = block_len(type);
    for (int64_t k = 0; k < K; ++k) {
        const int64_t b = k / bl;                       /* the scale's block */
        const uint16_t sb = (uint16_t)(row[2 * b] | (row[2 * b + 1] << 8));
        const float d = orc_f16_to_f32(sb);
        int code;
        if (is_q8(type)) {
            code = (int8_t)row[qoff + (size_t)k];
        } else {
            const int64_t run = k / 32, i = k % 32;     /* 32-code run, position */
            const uint8_t byte = row[qoff + (size_t)run * 16u + (size_t)(i & 15)];
            const int nib = (i < 16) ? (byte & 0x0F) : (byte >> 4);
            code = nib - 8;
        }
        out[k] = d * (float)code;
    }
}

static int valid_weight(int type, int64_t K, size_t pitch)
{
    if (K < 0) return 0;
    if (type != ORC_F32 && type != ORC_F16 && type != ORC_BF16 && !is_quant(type)) return 0;
    if (is_quant(type) && (K % block_len(type)) != 0) return 0;
    return pitch >= orc_row_size(type, K);
}

int orc_dequantize_rows(int type, const uint8_t *src, size_t pitch,
                        int64_t K, int64_t M, float *dst)
{
    if (!valid_weight(type, K, pitch) || M < 0) return -1;
    for (int64_t m = 0; m < M; ++m)
        dequantize_row(type, src + (size_t)m * pitch, K, dst + (size_t)m * (size_t)K);
    return 0;
}

/* ------------------------------------------------------------------------
 * MUL_MAT: the plain definition (No Python! ... §6: C_ij = sum_k A_ik B_kj),
 * with the operands laid out as the ne/nb convention gives them (§4): W is
 * ne = [K, M] (row m contiguous), x is ne = [K, N] (token n contiguous), so
 * y[n][m] = sum_k W'[m][k] x[n][k].  Every product of two binary32 values is
 * exact in binary64; the sum is sequential in binary64.
 * ------------------------------------------------------------------------ */

static float x_value(const void *x, int x_type, int64_t K, int64_t n, int64_t k)
{
    if (x_type == ORC_BF16)
        return orc_bf16_to_f32(((const uint16_t *)x)[n * K + k]);
    return ((const float *)x)[n * K + k];
}

static void dot_row(const float *wrow, const void *x, int x_type, int64_t K, int64_t n,
                    double *y, double *a)
{
    double acc = 0.0, aacc = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        const double p = (double)wrow[k] * (double)x_value(x, x_type, K, n, k);
        acc += p;
        aacc += fabs(p);
    }
    *y = acc;
    *a = aacc;
}

static void row_to_bf16_values(float *row, int64_t K)
{
    for (int64_t k = 0; k < K; ++k) row[k] = orc_bf16_to_f32(orc_f32_to_bf16(row[k]));
}

int orc_mul_mat_rows(int type, const uint8_t *w, size_t pitch, int64_t K, int64_t M,
                     const void *x, int x_type, int64_t N, int w_to_bf16,
                     int64_t m0, int64_t m1, double *y, double *a)
{
    if (!valid_weight(type, K, pitch) || M < 0 || N < 0) return -1;
    if (x_type != ORC_F32 && x_type != ORC_BF16) return -1;
    if (m0 < 0 || m1 > M || m0 > m1) return -1;
    float *wrow = (float *)malloc(sizeof(float) * (size_t)(K > 0 ? K : 1));
    if (!wrow) return -1;
    for (int64_t m = m0; m < m1; ++m) {
        dequantize_row(type, w + (size_t)m * pitch, K, wrow);
        if (w_to_bf16) row_to_bf16_values(wrow, K);
        for (int64_t n = 0; n < N; ++n)
            dot_row(wrow, x, x_type, K, n, &y[n * M + m], &a[n * M + m]);
    }
    free(wrow);
    return 0;
}

int orc_mul_mat_pairs(int type, const uint8_t *w, size_t pitch, int64_t K, int64_t M,
                      const void *x, int x_type, int64_t N, int w_to_bf16,
                      const int64_t *ms, const int64_t *ns, int64_t count,
                      double *y, double *a)
{
    if (!valid_weight(type, K, pitch) || M < 0 || N < 0 || count < 0) return -1;
    if (x_type != ORC_F32 && x_type != ORC_BF16) return -1;
    for (int64_t i = 0; i < count; ++i)
        if (ms[i] < 0 || ms[i] >= M || ns[i] < 0 || ns[i] >= N) return -1;
    float *wrow = (float *)malloc(sizeof(float) * (size_t)(K > 0 ? K : 1));
    if (!wrow) return -1;
    for (int64_t i = 0; i < count; ++i) {
        dequantize_row(type, w + (size_t)ms[i] * pitch, K, wrow);
        if (w_to_bf16) row_to_bf16_values(wrow, K);
        dot_row(wrow, x, x_type, K, ns[i], &y[i], &a[i]);
    }
    free(wrow);
    return 0;
}

/* ---- SwiGLU ------------------------------------------------------------- */

double orc_swish(double z)
{
    /* z * sigma(z); for z far below zero e^{-z} overflows to +inf and the
     * quotient is the correct limit (-0). */
    return z / (1.0 + exp(-z));
}

void orc_swiglu_n(const double *g, const double *u, double *h, size_t n)
{
    for (size_t i = 0; i < n; ++i) h[i] = orc_swish(g[i]) * u[i];
}

/* ---- block-record interchange ---------------------------------------------- */

size_t orc_record_size(int type)
{
    if (type == ORC_Q4_0) return 2 + 16;
    if (type == ORC_Q8_0) return 2 + 32;
    return 0;
}

/* Offset of the codes inside a packed row and the code bytes of one block. */
static int64_t code_offset(int64_t K) { return (K / 16 + 15) / 16 * 16; }
static int64_t block_code_bytes(int type) { return type == ORC_Q4_0 ? 16 : 32; }

int orc_rows_to_records(int type, const uint8_t *rows, size_t pitch, int64_t K, int64_t M,
                        uint8_t *records)
{
    const size_t rec = orc_record_size(type);
    if (rec == 0 || K <= 0 || K % 32 != 0 || M < 0 || pitch < orc_row_size(type, K)) return -1;
    const int64_t nblk = K / 32, cb = block_code_bytes(type), qoff = code_offset(K);
    for (int64_t m = 0; m < M; ++m) {
        const uint8_t *row = rows + (size_t)m * pitch;
        for (int64_t b = 0; b < nblk; ++b) {
            uint8_t *out = records + ((size_t)m * nblk + b) * rec;
            out[0] = row[2 * b];               /* scale, little endian */
            out[1] = row[2 * b + 1];
            for (int64_t i = 0; i < cb; ++i) out[2 + i] = row[qoff + b * cb + i];
        }
    }
    return 0;
}

int orc_records_to_rows(int type, const uint8_t *records, int64_t K, int64_t M,
                        uint8_t *rows, size_t pitch)
{
    const size_t rec = orc_record_size(type);
    if (rec == 0 || K <= 0 || K % 32 != 0 || M < 0 || pitch < orc_row_size(type, K)) return -1;
    const int64_t nblk = K / 32, cb = block_code_bytes(type), qoff = code_offset(K);
    for (int64_t m = 0; m < M; ++m) {
        uint8_t *row = rows + (size_t)m * pitch;
        memset(row, 0, pitch);
        for (int64_t b = 0; b < nblk; ++b) {
            const uint8_t *in = records + ((size_t)m * nblk + b) * rec;
            row[2 * b] = in[0];
            row[2 * b + 1] = in[1];
            for (int64_t i = 0; i < cb; ++i) row[qoff + b * cb + i] = in[2 + i];
        }
    }
    return 0;
}

/* ---- integer-activation MUL_MAT ------------------------------------------- */

/* Integer code i of the b-th run of 32 codes of a packed row: Q8 the int8
 * code, Q4 the nibble minus 8 (the pages' q in [-8, 7]). */
static int block_code(int type, const uint8_t *row, int64_t K, int64_t b, int i)
{
    const size_t qoff = scale_bytes(type, K);
    if (is_q8(type)) return (int8_t)row[qoff + (size_t)b * 32u + (size_t)i];
    const uint8_t byte = row[qoff + (size_t)b * 16u + (size_t)(i & 15)];
    return ((i < 16) ? (byte & 0x0F) : (byte >> 4)) - 8;
}

/* The scale of the b-th run of 32 codes: that of the block holding it. */
static double block_scale(int type, const uint8_t *row, int64_t b)
{
    const int64_t s = b / (block_len(type) / 32);
    return (double)orc_f16_to_f32((uint16_t)(row[2 * s] | (row[2 * s + 1] << 8)));
}

int orc_mul_mat_q8act_rows(int type, const uint8_t *w, size_t pitch, int64_t K, int64_t M,
                           const uint8_t *xq, size_t x_pitch, int64_t N,
                           int64_t m0, int64_t m1, double *y, double *a)
{
    if (!is_quant(type) || K < 0 || K % block_len(type) != 0 || M < 0 || N < 0) return -1;
    if (pitch < orc_row_size(type, K) || x_pitch < orc_row_size(ORC_Q8_0, K)) return -1;
    if (m0 < 0 || m1 > M || m0 > m1) return -1;
    for (int64_t m = m0; m < m1; ++m) {
        const uint8_t *wr = w + (size_t)m * pitch;
        for (int64_t n = 0; n < N; ++n) {
            const uint8_t *xr = xq + (size_t)n * x_pitch;
            double acc = 0.0, aacc = 0.0;
            for (int64_t b = 0; b < K / 32; ++b) {
                int64_t s = 0;
                for (int i = 0; i < 32; ++i)
                    s += (int64_t)block_code(type, wr, K, b, i) * block_code(ORC_Q8_0, xr, K, b, i);
                const double t = block_scale(type, wr, b) * block_scale(ORC_Q8_0, xr, b) * (double)s;
                acc += t;
                aacc += fabs(t);
            }
            y[n * M + m] = acc;
            a[n * M + m] = aacc;
        }
    }
    return 0;
}
