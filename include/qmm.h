/*
 * qmm.h -- C ABI of libqmm: block-quantized MUL_MAT on AMD Instinct MI355X
 * (gfx950), in its two forms: the decode GEMV (one to eight tokens, fp32
 * activations) and the prefill GEMM (many tokens, bf16 activations).
 *
 * The operation is the weight-by-activation matrix product that the pages
 * single out as the bulk of LLM inference time ("No Python! Building an AI
 * Inference Engine Exclusively in C++", §6; "A Complete Guide to llama.cpp and
 * Customization with C++", §2.1: with one token per step it is a GEMV), over
 * block-quantized weights ("Development Guide for Small AI Models (TinyLLaMA,
 * etc.) Using C++", §6.1-§6.2; "A Complete Guide to llama.cpp ...", §2.2).
 *
 * Tensors follow the pages' ne / nb convention ("No Python! ...", §4):
 * ne[i] is the number of elements along dimension i, nb[i] the distance in
 * BYTES between neighbours along dimension i, and ne[0] is the contiguous
 * dimension.  A matrix with ne = [K, M] therefore holds M rows of K elements,
 * row r starting at data + r * nb[1].
 *
 * MUL_MAT semantics (every entry point below):
 *     W  ne = [K, M]   weights, one row per output feature
 *     x  ne = [K, N]   activations, one row of K per token
 *     y  ne = [M, N]   F32 result, one row of M per token
 *     y[n][m] = sum_k W'[m][k] * x[n][k]
 * where W' is the dequantized weight: Delta_b * code for the block b that
 * holds k (32 weights per block; 64 for the _B64 types).  The contraction runs over ne[0] of both operands (the second
 * operand is the "transposed" one of the pages' tensor_mul_mat, §5 of
 * "No Python! ...").
 *
 * Quantized row layout ("row-planar"; the pages fix the block contents but
 * not the byte order, see the Development Guide §6.1):
 *     bytes [0, 2*K/32)       fp16 scale Delta_b of block b at offset 2b (LE)
 *     zero padding up to qoff = align16(K/16)
 *     Q8_0: bytes [qoff + 32b, +32)  the 32 int8 codes of block b
 *     Q4_0: bytes [qoff + 16b, +16)  block b, byte j = code_j | code_{j+16} << 4,
 *                                    stored codes 0..15 meaning code - 8
 *     zero padding up to qmm_row_size() (a multiple of 16 bytes).
 * The row keeps the 34 (Q8_0) or 18 (Q4_0) bytes per 32 weights of the block
 * records; when K is a multiple of 256 there is no padding at all.
 * 64-weight blocks ("A Complete Guide to llama.cpp ...", §2.2: the block
 * length is usually 32 or 64), types Q8_B64 / Q4_B64, K % 64 == 0: the same
 * row with one fp16 Delta per 64 weights (bytes [0, 2*K/64), codes from
 * qoff = align16(K/32)); the codes are laid out exactly as above, so a
 * 64-block is two consecutive 32-code runs under one Delta.
 *
 * Ownership and errors (all entry points):
 *  - Every buffer is caller-owned DEVICE memory; the library allocates
 *    nothing, keeps no pointer after returning and holds no global state.
 *  - `stream` is a hipStream_t passed as void*; NULL is the default stream.
 *    Work is enqueued asynchronously; nothing synchronizes.
 *  - Arguments are validated on the host before anything is enqueued.  A
 *    non-zero (negative) return means nothing was enqueued and every output
 *    is untouched.  A launch failure returns QMM_ERR_DEVICE; faults during
 *    execution surface at the caller's next synchronization of `stream`.
 *  - Tensors with zero rows or zero tokens are valid and enqueue nothing.
 *    K = 0 yields y = 0.
 *  - Entry points are thread-safe.
 */
#ifndef QMM_H
#define QMM_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define QMM_API __attribute__((visibility("default")))
#else
#define QMM_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* Element / block types.  F16 and BF16 are IEEE binary16 and bfloat16. */
typedef enum {
    QMM_TYPE_F32  = 0,
    QMM_TYPE_F16  = 1,
    QMM_TYPE_BF16 = 2,
    QMM_TYPE_Q8_0 = 3,  /* 32-blocks: fp16 Delta + 32 int8 codes in [-127, 127]   */
    QMM_TYPE_Q4_0 = 4,  /* 32-blocks: fp16 Delta + 32 four-bit codes (value - 8)  */
    QMM_TYPE_Q8_B64 = 5,/* 64-blocks: fp16 Delta + 64 int8 codes in [-127, 127]   */
    QMM_TYPE_Q4_B64 = 6 /* 64-blocks: fp16 Delta + 64 four-bit codes (value - 8)  */
} qmm_type;

typedef enum {
    QMM_OK              = 0,
    QMM_ERR_NULL        = -1,  /* a descriptor or a needed data pointer is NULL      */
    QMM_ERR_TYPE        = -2,  /* type not accepted by this entry point              */
    QMM_ERR_SHAPE       = -3,  /* ne mismatch between operands, K % block, N range   */
    QMM_ERR_LAYOUT      = -4,  /* nb / alignment not supported                       */
    QMM_ERR_ALIAS       = -5,  /* the output overlaps an input                       */
    QMM_ERR_UNSUPPORTED = -6,  /* n_dims > 2, ne[2] or ne[3] != 1, or K*N too large */
    QMM_ERR_DEVICE      = -7,  /* the HIP runtime refused the launch                 */
    QMM_ERR_SCRATCH     = -8   /* more scratch than the static array holds           */
} qmm_status;

/* Tensor descriptor ("No Python! ...", §4: Tensor {n_dims, ne[4], nb[4],
 * type, data}).  Layout rules checked by every entry point:
 *  - n_dims is 1 or 2, ne[2] = ne[3] = 1 (higher dims: QMM_ERR_UNSUPPORTED);
 *  - dense types: nb[0] = element size;  quantized types: nb[0] = 0;
 *  - nb[1] >= qmm_row_size(type, ne[0]); for quantized weights nb[1] % 16 == 0
 *    and data % 16 == 0; F16 weights need nb[1] % 16 == 0 and data % 16 == 0;
 *    F32 activations and outputs need 4-byte alignment of data and nb[1];
 *    BF16 activations of qmm_gemm need 16-byte alignment of data and nb[1];
 *  - quantized ne[0] must be a multiple of 32 (64 for the _B64 types; else
 *    QMM_ERR_SHAPE);
 *  - ne[0] and ne[1] at most 2^48, and the bytes the tensor spans
 *    ((ne[1] - 1) nb[1] + the row size) at most 2^62 and inside the address
 *    space from data on (else QMM_ERR_UNSUPPORTED). */
typedef struct qmm_tensor {
    int32_t  type;     /* qmm_type                          */
    int32_t  n_dims;   /* 1 or 2                            */
    int64_t  ne[4];    /* elements per dimension            */
    uint64_t nb[4];    /* byte stride per dimension         */
    void    *data;     /* device pointer                    */
} qmm_tensor;

/* Bytes of one packed (or dense) row of ne0 elements; 0 for an unknown type
 * or an invalid ne0 (negative, above 2^48, or not a multiple of the block
 * length).
 * A row holds its blocks' contents as the Development Guide for Small AI
 * Models (TinyLLaMA, etc.) Using C++, §6.1 lists them (one fp16 scale per
 * block, then the block's codes), 34 bytes per 32 Q8_0 weights and 18 per
 * 32 Q4_0 weights, with the scales first and each part 16-byte aligned.
 * Q8_0: align16(ne0/16) + align16(ne0);  Q4_0: align16(ne0/16) + align16(ne0/2);
 * Q8_B64: align16(ne0/32) + align16(ne0);  Q4_B64: align16(ne0/32) + align16(ne0/2). */
QMM_API size_t qmm_row_size(int32_t type, int64_t ne0);

/* Quantize F32 rows into Q8_0, Q4_0, Q8_B64 or Q4_B64 rows (load time, once
 * per weight).  src: F32 ne = [K, M];  dst: ne = [K, M], K a multiple of the
 * block length.
 * Per block of 32 (or 64) ("A Complete Guide to llama.cpp ...", §2.2; Development
 * Guide §6.1): amax = max|w|; Delta = fp16(amax / 127) for Q8 or
 * fp16(amax / 8) for Q4 (round to nearest even); code = round(w / Delta)
 * half away from zero, one IEEE binary32 division by the stored Delta;
 * Q8_0 clamps to [-127, 127], Q4_0 stores code + 8 clamped to [0, 15];
 * Delta = 0 gives all-zero codes.  Bit-exact and deterministic.  Inputs must
 * be finite with amax / 127 (Q8_0) or amax / 8 (Q4_0) below 65520. */
QMM_API int qmm_quantize(const qmm_tensor *src_f32, qmm_tensor *dst_q, void *stream);

/* Quantization rules of qmm_quantize_rule. */
typedef enum {
    QMM_QUANT_DEFAULT = 0,   /* the rules of qmm_quantize                          */
    QMM_QUANT_Q4_AMAX7 = 1   /* Q4_0 storage, the pages' symmetric rule (below)    */
} qmm_quant_rule;

/* qmm_quantize with an explicit rule.  QMM_QUANT_Q4_AMAX7 is the rule of
 * "A Complete Guide to llama.cpp and Customization with C++", §2.2
 * (Delta = max|w| / 7, q in [-8, 7]): Delta = fp16(amax / 7) (RNE);
 * q = round(w / Delta) half away from zero by one binary32 division by the
 * stored Delta, clamped to [-8, 7]; stored as the Q4_0 nibble q + 8, so the
 * result is an ordinary Q4_0 (or Q4_B64) tensor (every kernel reads it
 * unchanged) and |W' - w| <= Delta / 2 holds for every weight (no code
 * clamps).  Only for dst type Q4_0 or Q4_B64 (else QMM_ERR_TYPE); an unknown
 * rule returns
 * QMM_ERR_UNSUPPORTED.  Inputs must be finite with amax / 7 below 65520. */
QMM_API int qmm_quantize_rule(const qmm_tensor *src_f32, qmm_tensor *dst_q, int32_t rule, void *stream);

/* Expand Q8_0 / Q4_0 / Q8_B64 / Q4_B64 / F16 rows to F32 (W' = Delta * code, exact in binary32;
 * "Development Guide ...", §6.2 step "Dequantization").
 * src ne = [K, M];  dst: F32 ne = [K, M].  Bit-exact. */
QMM_API int qmm_dequantize(const qmm_tensor *src, qmm_tensor *dst_f32, void *stream);

/* Decode GEMV / skinny GEMM ("A Complete Guide to llama.cpp ...", §2.1: one
 * token per step makes every projection a GEMV; Development Guide §6.2: the
 * codes are unpacked to their signed values and scaled before the
 * multiply-add).
 * w: Q8_0, Q4_0, Q8_B64, Q4_B64 or F16, ne = [K, M];  x: F32 ne = [K, N],
 * 1 <= N <= 8
 * (N > 8: QMM_ERR_SHAPE);  y: F32 ne = [M, N], must not overlap w or x.
 * Each lane keeps its slice of x in registers, which bounds K: the call
 * returns QMM_ERR_UNSUPPORTED when K exceeds 32768 (Q4_0, Q8_0) or 16384
 * (F16), when the row pitch nb[1] of w exceeds 2^28 bytes (loads address
 * a few rows with 32-bit offsets), or when M or the row pitch of x or y (in
 * elements) reaches 2^31.  Tokens are processed in groups that fit
 * the registers (one pass over the weights per group).
 * Weights are read once from HBM and dequantized in registers; binary32
 * multiply-add; the accumulation order is unspecified (results agree with
 * the exact sum within 1e-4 * sum_k |W'[m][k] x[n][k]| + 1e-6 for every
 * output and every input: each product is a signed code times x, so the
 * rounding error is relative to sum |W' x|, never to a larger biased sum).
 * From 5 tokens (from 3 when the call has more than 2048 rows or K above
 * 4096; from 7 when K is above 6144), quantized weights go to the bf16
 * matrix cores instead: signed codes enter exactly, x as two
 * bfloat16 parts (x = hi + lo to 2^-17 relative), products accumulated in
 * binary32, within the same bound.  So do F16 rows whose K is a multiple of
 * 32, from 5 tokens (from 3 with at least 16384 rows or K above 8192): each
 * half enters exactly as two bfloat16 parts, and an infinite weight there
 * gives NaN (not +-Inf) in its row's outputs, since the low part of an
 * activation may be 0. */
/* Integer activations ("A Complete Guide to llama.cpp ...", §2.2: with x
 * quantized per block too, x_i ~= Delta_x qx_i, the block dot product is
 * Delta Delta_x sum_i q_i qx_i, an integer sum): when x is Q8_0 (ne = [K, N],
 * the activations quantized with qmm_quantize, 1 <= N <= 8), w must be
 * quantized (else QMM_ERR_TYPE; with 64-blocks, Delta_w(m,b) below is the
 * scale of the 64-block holding the 32-block b) and
 *   y[n][m] = sum_b Delta_w(m,b) Delta_x(n,b) sum_i q_i qx_i
 * with each block's integer sum exact (int8 dot products into int32) and
 * the block terms summed in binary32 (|y - exact| <= (K/16 + 16) 2^-24
 * sum_b |block term|).  This approximates the fp32-activation product by the
 * quantization of x: |y - sum_k W' x| <= sum_k |W'_k| Delta_x / 2.  K up to
 * 16384 (Q8_0) or 32768 (Q4_0), else QMM_ERR_UNSUPPORTED; tokens go in
 * passes over the weights of up to 8 (fewer for long rows).  Q8_0 weights
 * from 5 tokens with at least 8192 rows or K above 4096 run on the bf16
 * matrix cores, where the codes enter exactly and the block sums are exact
 * too (same arithmetic, same bound). */
QMM_API int qmm_gemv(const qmm_tensor *w, const qmm_tensor *x_f32, qmm_tensor *y_f32, void *stream);

/* Most GEMVs one qmm_gemv_batch call takes. */
#define QMM_GEMV_BATCH_MAX 8

/* One GEMV of a batch: the operands of a qmm_gemv call. */
typedef struct qmm_gemv_item {
    const qmm_tensor *w;
    const qmm_tensor *x_f32;
    qmm_tensor *y_f32;
} qmm_gemv_item;

/* Several independent decode GEMVs in one launch ("A Complete Guide to
 * llama.cpp ...", §2.1: at one token per step the Q, K and V projections are
 * three GEMVs of the same input; "Development Guide ...", §4.4: so are the
 * gate and up projections of the feed-forward block).  Each item follows the
 * rules of qmm_gemv; all items must share the weight type, K and N, and the
 * activation type: F32 for all, or Q8_0 for all (the integer-activation
 * path of qmm_gemv, with its accuracy; a mix is QMM_ERR_TYPE); no output
 * may overlap any operand of any item.  1 <= count <=
 * QMM_GEMV_BATCH_MAX (else QMM_ERR_SHAPE).  Equivalent to count qmm_gemv
 * calls, without the fixed cost of count - 1 kernel launches; the workgroups
 * of the launch are shared among the items in proportion to their rows. */
QMM_API int qmm_gemv_batch(const qmm_gemv_item *items, int32_t count, void *stream);

/* The fused gate/up projection of the feed-forward block with its SwiGLU
 * epilogue ("Development Guide for Small AI Models (TinyLLaMA, etc.) Using
 * C++", §4.4: SwiGLU(x) = Swish(x W_gate) * (x W_up) elementwise, with
 * Swish(z) = z sigma(z) = z / (1 + e^{-z})):
 *   h[n][m] = Swish(sum_k Wg'[m][k] x[n][k]) * sum_k Wu'[m][k] x[n][k].
 * w_gate, w_up: the same type (any qmm_gemv weight type) and ne = [K, M], each with
 * its own row pitch under the rules of qmm_gemv;  x: F32 ne = [K, N],
 * 1 <= N <= 8, or Q8_0 rows (the integer-activation path of qmm_gemv, then
 * the two sums carry that path's accuracy and the weights are quantized);  h: F32 ne = [M, N], overlapping none of w_gate, w_up, x
 * (QMM_ERR_ALIAS).  Different types: QMM_ERR_TYPE; different ne: QMM_ERR_SHAPE.
 * One launch streams both matrices once and writes h only (the two
 * projections are never stored); from 3 fp32 tokens, with quantized weights
 * and K <= 4096, on the bf16 matrix cores.  The two sums carry the accuracy of
 * qmm_gemv; the epilogue runs in binary32 (expf, one division, two
 * products), so |h - h_exact| <= 1.1 e_g (|u| + e_u) + |Swish(g)| e_u
 * + 2^-20 |h| with e_g, e_u the qmm_gemv bounds of the two sums. */
QMM_API int qmm_gemv_swiglu(const qmm_tensor *w_gate, const qmm_tensor *w_up,
                            const qmm_tensor *x_f32, qmm_tensor *h_f32, void *stream);

/* Prefill GEMM ("No Python! ...", §6: C_ij = sum_k A_ik B_kj, with many tokens
 * per step).  w: Q4_0, Q8_0, Q4_B64, Q8_B64 or F16 (F16 with K % 32 == 0, else
 * QMM_ERR_UNSUPPORTED), ne = [K, M];  x: BF16 ne = [K, N], any N >= 0;
 * y: F32 ne = [M, N], must not overlap w or x.  Weight tiles are dequantized
 * (F16: converted) to bfloat16 (round to nearest even) and multiplied on the
 * bf16 matrix cores with binary32 accumulation (results agree with the exact
 * sum of the weights within 1e-2 * sum_k |W'[m][k] x[n][k]| + 1e-5). */
QMM_API int qmm_gemm(const qmm_tensor *w, const qmm_tensor *x_bf16, qmm_tensor *y_f32, void *stream);

/* qmm_gemm with a caller-owned workspace that lets a product with too few
 * output tiles to occupy every compute unit split K ("No Python! ...", §6:
 * C_ij = sum_k A_ik B_kj is a sum over k, so it can be cut into k ranges
 * whose partial sums are added afterwards).  Each range's partial sums go to
 * the workspace; a second kernel on the same stream adds them in range order,
 * so results are deterministic (the same for every call with the same
 * workspace size) and agree with the exact sum within the qmm_gemm bound.
 *
 * qmm_gemm_workspace_size(w, x_bf16): bytes the split that the current
 * device's compute-unit count calls for uses (0 when K is not split, or for
 * NULL descriptors); it depends only on the shapes and the device.
 *
 * qmm_gemm_ws: operands and errors as qmm_gemm.  workspace: device memory,
 * 16-byte aligned (else QMM_ERR_LAYOUT), overlapping none of w, x, y in the
 * bytes the call uses (QMM_ERR_ALIAS); workspace_bytes: its size.  A NULL
 * workspace or a size below the planned one makes the call choose a smaller
 * split that fits, down to none (then it is qmm_gemm).  The workspace is
 * scratch: its contents on entry do not matter, it is written and read by
 * the enqueued kernels, and it must stay allocated, and unused by other
 * work, until they have run.  qmm_gemm is qmm_gemm_ws with no workspace. */
QMM_API size_t qmm_gemm_workspace_size(const qmm_tensor *w, const qmm_tensor *x_bf16);
QMM_API int qmm_gemm_ws(const qmm_tensor *w, const qmm_tensor *x_bf16, qmm_tensor *y_f32, void *workspace,
                        size_t workspace_bytes, void *stream);

/* qmm_gemm_ws for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the split-K workspace is the first workspace_bytes of a static device
 * array of QMM_NOALLOC_SCRATCH_BYTES that the library owns (one per device,
 * held until the process ends), so the call neither allocates nor frees.
 * Same operands, result bits and errors as qmm_gemm_ws with a caller
 * workspace of workspace_bytes; workspace_bytes above
 * QMM_NOALLOC_SCRATCH_BYTES returns QMM_ERR_SCRATCH with nothing enqueued.
 * qmm_gemm_workspace_size(w, x_bf16) gives the full split (at most 16 MiB on
 * a 256-CU device, so it always fits there); 0 runs without a split.
 * Every call on one device shares that device's array: calls that overlap in
 * time on one device (on different streams, or from several host threads
 * without ordering) race on it and give wrong results.  The array needs no
 * clearing: each split writes every partial sum it later reads. */
#define QMM_NOALLOC_SCRATCH_BYTES (16u << 20)
QMM_API int qmm_gemm_noalloc(const qmm_tensor *w, const qmm_tensor *x_bf16, qmm_tensor *y_f32,
                             size_t workspace_bytes, void *stream);

/* Most products one qmm_gemm_batch call takes. */
#define QMM_GEMM_BATCH_MAX 8

/* One product of a GEMM batch: the operands of a qmm_gemm call. */
typedef struct qmm_gemm_item {
    const qmm_tensor *w;
    const qmm_tensor *x_bf16;
    qmm_tensor *y_f32;
} qmm_gemm_item;

/* Several independent prefill GEMMs in one launch (the query, key and value
 * projections of a decoder layer multiply the same tokens: "Development
 * Guide for Small AI Models (TinyLLaMA, etc.) Using C++", §4; so do the gate
 * and up projections of its feed-forward block, §4.4).  Each item follows
 * the rules of qmm_gemm; all items must share the weight type, K and N
 * (else QMM_ERR_TYPE / QMM_ERR_SHAPE), and no output may overlap any operand
 * of any item (QMM_ERR_ALIAS).  1 <= count <= QMM_GEMM_BATCH_MAX (else
 * QMM_ERR_SHAPE).  The items' 128 x 128 output tiles form one grid, so
 * small matrices that would leave most compute units idle on their own
 * share a launch; each output equals, bit for bit, that of qmm_gemm on the
 * same item (K is never split in a batch). */
QMM_API int qmm_gemm_batch(const qmm_gemm_item *items, int32_t count, void *stream);

/* The fused gate/up prefill projection with its SwiGLU epilogue ("Development
 * Guide for Small AI Models (TinyLLaMA, etc.) Using C++", §4.4: SwiGLU(x) =
 * Swish(x W_gate) * (x W_up) elementwise, Swish(z) = z / (1 + e^{-z})):
 *   h[n][m] = Swish(sum_k Wg'[m][k] x[n][k]) * sum_k Wu'[m][k] x[n][k].
 * w_gate, w_up: the same type (any qmm_gemm weight type) and ne = [K, M], each
 * under the rules of qmm_gemm with its own row pitch;  x: BF16 ne = [K, N];
 * h: F32 ne = [M, N], overlapping none of the operands (QMM_ERR_ALIAS).
 * Different types: QMM_ERR_TYPE; different ne: QMM_ERR_SHAPE.  One launch
 * computes both products (each workgroup 64 rows of each matrix times 128
 * tokens) and writes h only.  Each sum carries the accuracy of qmm_gemm; the
 * epilogue runs in binary32 (expf, one division, two products). */
QMM_API int qmm_gemm_swiglu(const qmm_tensor *w_gate, const qmm_tensor *w_up, const qmm_tensor *x_bf16,
                            qmm_tensor *h_f32, void *stream);

/* GGUF-style block records ("Development Guide for Small AI Models (TinyLLaMA,
 * etc.) Using C++", §3.2: a GGUF file's tensor data is an aligned array;
 * §6.1: a Q4_0 block is one FP16 scale (2 bytes) followed by 32 4-bit
 * values (16 bytes)).  A record is the block's fp16 scale (little endian)
 * followed by its codes: 16 bytes for Q4_0 (byte j holds element j in its
 * low nibble and element j + 16 in its high nibble, offset binary: value =
 * scale * (nibble - 8)) or 32 int8 bytes for Q8_0 (value = scale * code).
 * The M * K/32 records of a tensor run back to back in row-major order:
 * row 0's blocks 0 .. K/32 - 1, then row 1's, and so on.
 *
 * qmm_record_size: bytes of one record, 18 (Q4_0) or 34 (Q8_0); 0 for any
 * other type.
 *
 * qmm_records_to_rows: fills the packed rows of dst_q (Q8_0 or Q4_0, ne =
 * [K, M], the layout rules of qmm_quantize) from M * K/32 records at
 * `records` (device memory, 16-byte aligned, caller-owned, not overlapping
 * dst_q).  Every byte of each row's qmm_row_size bytes is written (the gap
 * between the scales and the codes with zeros); bytes past it up to nb[1]
 * are left as they are.  qmm_rows_to_records is the inverse: it writes the
 * M * K/32 records of src_q to `records`.  Both are bit-exact and
 * asynchronous on `stream`.
 * Errors: QMM_ERR_NULL (no tensor, or NULL records for a non-empty tensor),
 * QMM_ERR_TYPE (not Q8_0 / Q4_0: the _B64 types have no GGUF record), QMM_ERR_SHAPE / QMM_ERR_LAYOUT (the tensor
 * rules), QMM_ERR_LAYOUT (records not 16-byte aligned), QMM_ERR_ALIAS
 * (records overlap the rows), QMM_ERR_UNSUPPORTED (M * K/32 >= 2^31).
 * An empty tensor enqueues nothing. */
QMM_API size_t qmm_record_size(int32_t type);
QMM_API int qmm_records_to_rows(const void *records, qmm_tensor *dst_q, void *stream);
QMM_API int qmm_rows_to_records(const qmm_tensor *src_q, void *records, void *stream);

/* ---- Measurement helpers: context for the MUL_MAT figures, not part of
 * the operation.  Inference is bound by memory bandwidth ("No Python!
 * Building an AI Inference Engine Exclusively in C++", §9), so a decode GEMV
 * of B bytes is judged against what one launch can stream of B bytes at all;
 * the matrix-core peak assumes a shader clock, measured here under load. */

/* Streaming read: `workgroups` workgroups of 256 threads read the `bytes`
 * bytes at device address src with 128-bit loads (grid-stride, two batches
 * of four loads per thread in flight) and write one 32-bit xor of what each
 * read to sink[0 .. workgroups-1] (device memory), so that no load can be
 * elided.  bytes: a multiple of 16 below 2^31 (else QMM_ERR_SHAPE /
 * QMM_ERR_UNSUPPORTED); src 16-byte aligned (QMM_ERR_LAYOUT);
 * 1 <= workgroups <= 65536 (QMM_ERR_SHAPE); NULL src (bytes > 0) or sink:
 * QMM_ERR_NULL.  Asynchronous on `stream`. */
QMM_API int qmm_stream_read(const void *src, size_t bytes, uint32_t *sink, int32_t workgroups, void *stream);

/* Shader-clock and matrix-core probe: `workgroups` workgroups of four waves
 * each run `iters` rounds of a chain and write, per wave w, out[2w] = the
 * shader-clock counter's delta (s_memtime) and out[2w+1] = the
 * constant-rate counter's delta (s_memrealtime) over the chain.  The shader
 * clock is out[2w] / out[2w+1] times the constant counter's rate (the
 * device's wall clock rate).  Chains: mode 0, sixteen binary32 FMA chains
 * per lane; mode 1, four bf16 32x32x16 matrix-instruction chains per wave;
 * modes 2-4, the inner loop of a block-quantized GEMM per round: four
 * 32 x 32 output tiles each advanced by one 32-block of K ("A Complete Guide
 * to llama.cpp ...", §2.2: each block's integer dot product is scaled by
 * Delta_w * Delta_x before blocks are added), with bf16 operands and the
 * scale already in the weights (mode 2), or int8 operands and the block's
 * int32 tile converted and scaled on the vector ALUs, by the weight scale
 * only (mode 3) or by the weight and the activation scale (mode 4).  Each
 * round is 4 * 32 * 32 * 32 multiply-adds per wave.  out: device memory of
 * 8 * workgroups uint64 (QMM_ERR_NULL if NULL); 1 <= workgroups <= 65536,
 * iters >= 1, 0 <= mode <= 4 (else QMM_ERR_SHAPE). */
QMM_API int qmm_clock_probe(uint64_t *out, int32_t workgroups, int32_t iters, int32_t mode, void *stream);

/* Rate of the constant-rate counter of the current device in kHz (the HIP
 * device attribute WallClockRate), or QMM_ERR_DEVICE if it cannot be read. */
QMM_API int64_t qmm_wall_clock_khz(void);

/* Static text for a qmm_status value (never NULL).  Every call reports
 * failure as a status code that the caller checks, as the calls of "A
 * Complete Guide to llama.cpp and Customization with C++", §5.2-§5.4 do;
 * nothing is thrown across the ABI. */
QMM_API const char *qmm_strerror(int status);

#ifdef __cplusplus
}
#endif
#endif /* QMM_H */
