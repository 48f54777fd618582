/*
 * qmm_oracle.h -- plain, slow CPU reference for block-quantized MUL_MAT.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the oracle that the GPU library is
 * checked against.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load it.  It shares no code, header, table or constant
 * with the GPU library (it does not include include/qmm.h) and the GPU library
 * never calls it.
 *
 * Everything here is scalar C with IEEE binary32 arithmetic where the method
 * fixes binary32 (the quantizer) and binary64 accumulation for every dot
 * product.  Built with -O2 -ffp-contract=off and no fast-math.
 *
 * Sources (the pages this follows):
 *  - "No Python! Building an AI Inference Engine Exclusively in C++",
 *    §4 (tensor ne/nb strides) and §6 (the GEMM definition C_ij = sum_k A_ik B_kj).
 *  - "Development Guide for Small AI Models (TinyLLaMA, etc.) Using C++",
 *    §6.1 (Q4_0 block: 32 values, one FP16 scale, 32 four-bit values) and
 *    §6.2 (load, unpack, multiply by the scale, multiply-add with activations).
 *  - "A Complete Guide to llama.cpp and Customization with C++", §2.2
 *    (w_i ~= Delta * q_i per block, Delta from the block's max |w|).
 */
#ifndef QMM_ORACLE_H
#define QMM_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Weight encodings the oracle knows.  Own numbering (not the library's). */
enum {
    ORC_F32 = 0,   /* dense binary32 rows                                   */
    ORC_F16 = 1,   /* dense binary16 rows (bits)                            */
    ORC_BF16 = 2,  /* dense bfloat16 rows (bits)                            */
    ORC_Q8_0 = 3,  /* 32-blocks: fp16 scale + 32 int8 codes                 */
    ORC_Q4_0 = 4,  /* 32-blocks: fp16 scale + 32 offset-binary 4-bit codes  */
    ORC_Q8_B64 = 5,/* 64-blocks: fp16 scale + 64 int8 codes                 */
    ORC_Q4_B64 = 6 /* 64-blocks: fp16 scale + 64 offset-binary 4-bit codes  */
};

/* ---- IEEE conversions, written from the format definitions ---------- */
uint16_t orc_f32_to_f16(float f);        /* round to nearest, ties to even */
float    orc_f16_to_f32(uint16_t h);     /* exact                          */
uint16_t orc_f32_to_bf16(float f);       /* round to nearest, ties to even */
float    orc_bf16_to_f32(uint16_t h);    /* exact                          */

void orc_f32_to_f16_n(const float *src, uint16_t *dst, size_t n);
void orc_f16_to_f32_n(const uint16_t *src, float *dst, size_t n);
void orc_f32_to_bf16_n(const float *src, uint16_t *dst, size_t n);
void orc_bf16_to_f32_n(const uint16_t *src, float *dst, size_t n);

/* ---- one 32-weight block ------------------------------------------- */
/* Q8_0: scale_bits = fp16(amax/127); q_i = clamp(roundf(w_i/scale), -127, 127). */
void orc_quantize_block_q8_0(const float w[32], uint16_t *scale_bits, int8_t q[32]);
/* Q4_0: scale_bits = fp16(amax/8); nib_i = clamp(roundf(w_i/scale) + 8, 0, 15). */
void orc_quantize_block_q4_0(const float w[32], uint16_t *scale_bits, uint8_t nib[32]);

/* The pages' symmetric Q4 rule ("A Complete Guide to llama.cpp and
 * Customization with C++", §2.2: Delta = max|w| / 7, q in [-8, 7]):
 * scale_bits = fp16(amax/7); nib_i = clamp(roundf(w_i/scale), -8, 7) + 8.
 * Same storage (and dequantization) as Q4_0.                               */
void orc_quantize_block_q4_sym7(const float w[32], uint16_t *scale_bits, uint8_t nib[32]);

/* 64-weight blocks ("A Complete Guide to llama.cpp ...", §2.2: the block
 * length is usually 32 or 64): the same steps over 64 values, one fp16
 * scale.  divisor 8 (offset-binary rule) or 7 (the pages' symmetric rule).  */
void orc_quantize_block_q8_b64(const float w[64], uint16_t *scale_bits, int8_t q[64]);
void orc_quantize_block_q4_b64(const float w[64], int divisor, uint16_t *scale_bits, uint8_t nib[64]);

/* Quantization rules of orc_quantize_rows_rule.                            */
enum { ORC_RULE_DEFAULT = 0,   /* Q8_0: amax/127; Q4_0: amax/8 (offset 8) */
       ORC_RULE_Q4_SYM7 = 1 }; /* Q4_0 storage, the pages' amax/7 rule    */

/* ---- packed rows ------------------------------------------------------
 * Row-planar packing of one row of K weights in blocks of B = 32 (Q8_0,
 * Q4_0) or 64 (Q8_B64, Q4_B64) weights (K % B == 0):
 *   bytes [0, 2*K/B)             fp16 scale of block b at offset 2b (little endian)
 *   zero padding up to qoff = align16(2*K/B)
 *   Q8:  byte qoff + k           the int8 code of weight k
 *   Q4:  bytes [qoff + 16r, +16) the r-th run of 32 codes (weights 32r ..
 *        32r+31), byte j = nib_{32r+j} | nib_{32r+j+16} << 4 (a 64-block is
 *        two such runs under one scale)
 *   zero padding up to the row size (a multiple of 16).
 * orc_row_size returns that size (dense types: K * element size).          */
size_t orc_row_size(int type, int64_t K);

/* Quantize M rows of K floats (row m at w + m*K) into dst (row m at
 * dst + m*pitch, pitch >= orc_row_size).  Returns 0, or -1 on bad args.     */
int orc_quantize_rows(int type, const float *w, int64_t K, int64_t M,
                      uint8_t *dst, size_t pitch);

/* The same with an explicit rule (ORC_RULE_Q4_SYM7 only with the Q4 types). */
int orc_quantize_rows_rule(int type, int rule, const float *w, int64_t K, int64_t M,
                           uint8_t *dst, size_t pitch);

/* Expand rows of any weight type to exact binary32 values (M x K, dense).  */
int orc_dequantize_rows(int type, const uint8_t *src, size_t pitch,
                        int64_t K, int64_t M, float *dst);

/* ---- MUL_MAT ----------------------------------------------------------
 * y[n][m] = sum_k W'[m][k] * x[n][k], W' the exactly dequantized weights,
 * accumulated sequentially in binary64; a[n][m] = sum_k |W'[m][k] x[n][k]|.
 * x_type is ORC_F32 (x as floats, row n at x + n*K) or ORC_BF16 (x as bf16
 * bits, row n at x + n*K).  w_to_bf16 != 0 first rounds every W' to bf16
 * (diagnostic variant of the bf16 matrix-core path).  Only rows
 * [m0, m1) are computed; y and a are N x M (row n at + n*M).             */
int orc_mul_mat_rows(int type, const uint8_t *w, size_t pitch, int64_t K, int64_t M,
                     const void *x, int x_type, int64_t N, int w_to_bf16,
                     int64_t m0, int64_t m1, double *y, double *a);

/* Same sum for a list of (m, n) pairs only: y[i], a[i] for pair i.         */
int orc_mul_mat_pairs(int type, const uint8_t *w, size_t pitch, int64_t K, int64_t M,
                      const void *x, int x_type, int64_t N, int w_to_bf16,
                      const int64_t *ms, const int64_t *ns, int64_t count,
                      double *y, double *a);

/* ---- integer-activation MUL_MAT ----------------------------------------
 * "A Complete Guide to llama.cpp and Customization with C++", §2.2: with the
 * activations quantized per block as well, x_i ~= Delta_x * qx_i, the block
 * dot product is y ~= Delta * Delta_x * sum_i q_i qx_i, whose sum is pure
 * integer arithmetic.  Weights: Q8_0 (q = code) or Q4_0 (q = nibble - 8),
 * or their 64-block forms (b then runs over 32-code runs and Delta_w(m,b) is
 * the scale of the 64-block holding run b); activations: Q8_0 rows of the
 * same K (quantized by orc_quantize_rows, the Q8_0 rule).
 * y[n][m] = sum_b Delta_w(m,b) Delta_x(n,b) S_b with the
 * integer S_b = sum_i q_i qx_i exact in int64 and the block terms summed in
 * binary64 (every term is exact there: at most 11 + 11 + 20 bits);
 * a[n][m] = sum_b |Delta_w Delta_x S_b|.  Rows [m0, m1) only.             */
int orc_mul_mat_q8act_rows(int type, const uint8_t *w, size_t pitch, int64_t K, int64_t M,
                           const uint8_t *xq, size_t x_pitch, int64_t N,
                           int64_t m0, int64_t m1, double *y, double *a);

/* ---- block-record interchange ------------------------------------------
 * GGUF-style tensor data: the blocks of a quantized tensor as back-to-back
 * records in row-major order (row 0's K/32 blocks, then row 1's, ...), each
 * record the block's fp16 scale (2 bytes, little endian) followed by its
 * codes: 16 bytes for Q4_0 (byte j = nib_j | nib_{j+16} << 4) or 32 int8
 * bytes for Q8_0.  "Development Guide for Small AI Models (TinyLLaMA, etc.)
 * Using C++", §6.1: one FP16 scale (2 bytes) then 32 4-bit values (16
 * bytes); §3.2: tensor data is an aligned array after the tensor info.      */
size_t orc_record_size(int type);        /* 18 (Q4_0), 34 (Q8_0), else 0 */
/* Packed rows (row m at rows + m*pitch) -> M*K/32 records.  0 or -1.        */
int orc_rows_to_records(int type, const uint8_t *rows, size_t pitch, int64_t K, int64_t M,
                        uint8_t *records);
/* Records -> packed rows, every byte of each row's pitch written (the
 * padding with zeros).  0 or -1.                                            */
int orc_records_to_rows(int type, const uint8_t *records, int64_t K, int64_t M,
                        uint8_t *rows, size_t pitch);

/* ---- SwiGLU epilogue of the fused gate/up projection ------------------
 * "Development Guide for Small AI Models (TinyLLaMA, etc.) Using C++", §4.4:
 * SwiGLU(x) = Swish(x W_gate) (elementwise *) (x W_up), with
 * Swish(z) = z * sigma(z) and sigma(z) = 1 / (1 + e^{-z}).  Binary64.       */
double orc_swish(double z);
/* h[i] = Swish(g[i]) * u[i] for i < n.                                      */
void orc_swiglu_n(const double *g, const double *u, double *h, size_t n);

/* ---- timing (oracle_timing.c): the CPU baseline ------------------------
 * Median wall time (seconds) of `reps` runs of orc_mul_mat_rows over all M
 * rows (x_type as there, w_to_bf16 = 0), the rows split statically into
 * `threads` contiguous ranges on as many POSIX threads; y and a (N x M) as
 * orc_mul_mat_rows fills them.  -1 on bad arguments.                        */
double orc_time_mul_mat(int type, const uint8_t *w, size_t pitch, int64_t K, int64_t M,
                        const void *x, int x_type, int64_t N, int threads, int reps,
                        double *y, double *a);
/* Online CPUs of the host (sysconf), the hardware thread count.            */
int orc_online_cpus(void);

#ifdef __cplusplus
}
#endif
#endif /* QMM_ORACLE_H */
