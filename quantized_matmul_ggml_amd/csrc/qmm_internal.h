// qmm_internal.h -- declarations shared by the host entry points (qmm_api.cpp)
// and the kernel translation units (*.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/qmm.h"
#include <stddef.h>
#include <stdint.h>

namespace qmm {

// Weight encodings the kernels understand (same values as qmm_type).
enum WType : int { W_F32 = 0, W_F16 = 1, W_BF16 = 2, W_Q8_0 = 3, W_Q4_0 = 4, W_Q8_B64 = 5, W_Q4_B64 = 6 };

// Byte offset of the codes inside a quantized row: the fp16 scales come
// first (K/32 of them, or K/64 with scale_shift 1), padded to 16 bytes.
__host__ __device__ inline int64_t quant_offset(int64_t K, int scale_shift = 0)
{
    return ((K >> (4 + scale_shift)) + 15) / 16 * 16;
}

// Cache policy of the loads that stream weights through a GEMV, each byte
// read once per call: non-temporal ("nt"), so the weights neither displace
// what the next launches reuse from the caches nor linger in them.  On the
// decode step (89 launches, 618 MB) this was 7-9 % faster than the default
// policy.  The prefill GEMM, whose weights four workgroups share through
// the L2, and the matrix-core GEMV's direct-to-LDS loads (5-7 % slower
// this way) keep the default.
constexpr int kStreamLoad = 2;

// Raw buffer resources (kernels): word 3 of the descriptor (32-bit data
// format, no swizzle), and an offset above every buffer size the kernels
// build, whose loads return zeros without touching memory.
constexpr int BUFFER_FLAGS = 0x00020000;
constexpr uint32_t OUT_OF_RANGE = 0x80000000u;

// One weight matrix as the kernels see it: M rows of K weights, row r at
// base + r * pitch (bytes).  type is the code format (W_Q8_0, W_Q4_0 or
// W_F16); the 64-block types arrive as their code format with scale_shift 1
// (one scale per two 32-weight runs: the scale of run c is scale c >> 1).
struct WeightView {
    const uint8_t *base;
    uint64_t pitch;
    int64_t K;
    int64_t M;
    int type;
    int scale_shift = 0;
};

// Activations: N rows of K values, row n at data + n * pitch_elems elements.
struct ActView {
    const void *data;
    uint64_t pitch_elems;
    int64_t N;
};

// Output: N rows of M floats, row n at data + n * pitch_elems.
struct OutView {
    float *data;
    uint64_t pitch_elems;
};

// Launch shape of the GEMV kernel, a pure function of (type, K, M, N).
struct GemvConfig {
    int nt;    // tokens per kernel instance (N rounded up to 1, 2, 4 or 8)
    int ks;    // waves sharing one row (1, 2 or 4)
    int cpl;   // 16-byte code chunks per lane (1, 2, 4 or 8)
    int u;     // rows per wave group per iteration
    int wgw;   // waves per workgroup (4 or 16)
};

// Fills cfg and returns true when the register-resident GEMV supports the
// shape (each lane keeps at most 128 activation floats); false otherwise.
bool gemv_config(int type, int64_t K, int64_t M, int64_t N, GemvConfig *cfg);
// Whether the GEMV kernels can address the operands: loads span a few rows
// with 32-bit buffer offsets, so the weight row pitch is bounded (2^28
// bytes), and row counts and activation / output pitches are 32-bit.
inline bool gemv_supported(const WeightView &w, const ActView &x, const OutView &y)
{
    return w.pitch <= (1ull << 28) && w.M < (1ll << 31) && x.pitch_elems < (1ull << 31) &&
           y.pitch_elems < (1ull << 31);
}

// Launchers (return hipSuccess or the launch error).  Shapes are validated by
// the caller; every launcher accepts M == 0 / N == 0 as a no-op.
// q4_amax7: the pages' symmetric Q4 rule (Delta = amax / 7) instead of amax / 8.
// scale_shift 1: 64-weight blocks (one scale per two 32-code runs).
hipError_t launch_quantize(const float *src, uint64_t src_pitch_elems, int64_t K, int64_t M,
                           uint8_t *dst, uint64_t dst_pitch, int type, hipStream_t stream,
                           bool q4_amax7 = false, int scale_shift = 0);
hipError_t launch_dequantize(const uint8_t *src, uint64_t src_pitch, int64_t K, int64_t M,
                             int type, float *dst, uint64_t dst_pitch_elems, hipStream_t stream,
                             int scale_shift = 0);
hipError_t launch_gemv(const WeightView &w, const ActView &x, const OutView &y,
                       hipStream_t stream);

// Several GEMVs (same weight type, K and token count) in one launch; each
// workgroup serves one of them.  count <= QMM_GEMV_BATCH_MAX.
struct GemvTask {
    WeightView w;
    ActView x;
    OutView y;
};
hipError_t launch_gemv_batch(const GemvTask *tasks, int count, hipStream_t stream);

// The integer-activation GEMV (gemv_i8.hip): w Q4_0 / Q8_0, the N
// activation rows xq Q8_0 of the same K (xq.M = N), y F32.  Supported when
// the plain configuration for (type, K, M, N) uses at most 4 chunks per lane.
bool gemv_i8_supported(int wtype, int64_t K, int64_t M, int64_t N);
hipError_t launch_gemv_i8(const WeightView &w, const WeightView &xq, const OutView &y, int64_t N,
                          hipStream_t stream);
// count (1 .. QMM_GEMV_BATCH_MAX) such GEMVs sharing the weight type, K and
// N in one launch (grid y indexes the items).
hipError_t launch_gemv_i8_batch(const WeightView *w, const WeightView *xq, const OutView *y, int count,
                                int64_t N, hipStream_t stream);
// The fused gate/up SwiGLU projection with Q8_0 activations:
// h[n][m] = Swish(sum of gate block terms) * sum of up block terms.
bool gemv_i8_swiglu_supported(int wtype, int64_t K, int64_t M, int64_t N);
hipError_t launch_gemv_i8_swiglu(const WeightView &wg, const WeightView &wu, const WeightView &xq,
                                 const OutView &h, int64_t N, hipStream_t stream);

// The fused gate/up projection with the SwiGLU epilogue:
// h[n][m] = Swish(sum_k Wg'[m][k] x[n][k]) * sum_k Wu'[m][k] x[n][k].
// wg and wu share the type, K and M.
hipError_t launch_gemv_swiglu(const WeightView &wg, const WeightView &wu, const ActView &x,
                              const OutView &h, hipStream_t stream);

// Which launches the matrix-core kernels take (measured on the decoder's
// shapes, graph-replayed): from 5 tokens every one; at 3 and 4 tokens those
// of more than 2048 rows or of rows over 4096 (5632 x 2048: 5.8 against
// 7.3 us at 3 tokens; 2048 x 5632: 7.5 against 8.2), while 2048 x 2048
// stays on the VALU kernel (3.95 against 4.2 us at 3 tokens), whose cost
// per weight grows with the tokens but whose grid fills the chip at any
// row count.
// Rows over 192 blocks (K > 6144) run on the matrix cores as several
// dependent passes, and the VALU kernel's one launch is faster up to 6
// tokens (2048 x 5632 Q4_0 in two passes: 12.7 / 14.1 us on the VALU kernel
// against 14.3 / 14.8 at 5 / 6 tokens; 16.7 against 15.3 at 8).
inline bool use_matrix_cores(int64_t N, int64_t m_total, int64_t K)
{
    if (K > 6144) return N >= 7;
    if (N >= 5) return true;
    return N >= 3 && (m_total > 2048 || K > 4096);
}

// F16 rows (K a multiple of 32; graph-replayed, µs per launch, VALU kernel
// against matrix cores): from 5 tokens every launch (5632 x 2048: 10.3 / 8.9
// at 5 tokens; 4096 x 4096: 18.0 / 11.5; 4096 x 11008: 80.4 / 38.3); at 3
// and 4 tokens only very tall matrices (32000 x 2048: 32.9 / 28.0) and rows
// over 8192, whose 4-token activation slice no VALU configuration holds in
// registers (4096 x 11008: 50.3 / 37.6); otherwise the VALU kernel
// (11008 x 4096: 19.5 / 25.5; 2048 x 5632: 11.2 / 14.8), which also takes 1
// and 2 tokens everywhere.
inline bool use_matrix_cores_f16(int64_t N, int64_t m_total, int64_t K)
{
    if (N >= 5) return true;
    return N >= 3 && (m_total >= 16384 || K > 8192);
}

// The matrix-core GEMV with register-resident activation fragments
// (gemv_mf.hip): Q4_0 / Q8_0 weights, and F16 rows of whole 32-blocks with
// a pitch that is a multiple of 16; weight pitch <= 2^27; quantized K up to
// 6144 in one launch (F16: 4096), longer rows in passes that add to y.
bool gemv_mf_supported(const GemvTask *tasks, int count);
hipError_t launch_gemv_mf(const GemvTask *tasks, int count, hipStream_t stream);
// The same kernel with Q8_0 weights and Q8_0 activation rows (xq[i]: pitch
// in bytes, a multiple of 16): each block's integer sum exact on the matrix
// cores, the block terms Delta_w Delta_x S summed in binary32.
bool gemv_mf_q8x_supported(const WeightView *w, const WeightView *xq, int count, int64_t N);
// The same kernel on a gate/up pair with the SwiGLU epilogue (one pass over
// K: at most 128 blocks, K <= 4096).
bool gemv_mf_swiglu_supported(const WeightView &wg, const WeightView &wu, const ActView &x);
hipError_t launch_gemv_mf_swiglu(const WeightView &wg, const WeightView &wu, const ActView &x, const OutView &h,
                                 hipStream_t stream);
hipError_t launch_gemv_mf_q8x(const WeightView *w, const WeightView *xq, const OutView *y, int count, int64_t N,
                              hipStream_t stream);
// Measurement kernels (probe.hip): a streaming read of `bytes` (multiple of
// 16, < 2^31) by `workgroups` workgroups of 256 threads, one xor word per
// workgroup into sink; and the clock probe (workgroups x 4 waves, each
// writing its shader-clock and constant-counter deltas to out).
hipError_t launch_stream_read(const void *src, uint64_t bytes, uint32_t *sink, int workgroups, hipStream_t stream);
hipError_t launch_clock_probe(uint64_t *out, int workgroups, int iters, int mode, hipStream_t stream);
// Compute units of the current device (queried once per device; gemm.hip).
int device_cus();
// Device address of the library's static scratch array on the current
// device (QMM_NOALLOC_SCRATCH_BYTES, 256-byte aligned; gemm.hip), looked up
// once per device.
hipError_t static_scratch(void **ptr);
// Grant a kernel more than the default dynamic LDS (once per size; gemm.hip).
hipError_t allow_dynamic_lds(const void *fn, int bytes);

// GGUF-style block records (records.hip): bytes of one record (18 for
// Q4_0, 34 for Q8_0, else 0), and the conversion between w's packed rows and
// M * K/32 back-to-back records at `records` (16-byte aligned device memory):
// records -> rows when to_rows (every byte of each row's row size is
// written, the gap before the codes with zeros), rows -> records otherwise.
// M * K/32 < 2^31.
int record_size(int type);
hipError_t launch_records(const WeightView &w, uint8_t *records, bool to_rows, hipStream_t stream);

// The prefill GEMM (gemm.hip): whether the operand strides fit its 32-bit
// per-tile offsets, and its launcher.
bool gemm_supported(const WeightView &w, const ActView &x);
// How the GEMM splits K: `splits` ranges of `split_steps` K-steps (64 of K)
// each, whose partial sums take ws_bytes of workspace (slab rows of mp = M
// rounded up to 4 floats).  splits == 1 (no workspace) unless the tiles
// leave compute units idle and a split fits in ws_bytes.
struct GemmPlan {
    int splits;
    int split_steps;
    int64_t mp;
    uint64_t ws_bytes;
};
GemmPlan gemm_plan(int64_t M, int64_t K, int64_t N, uint64_t ws_bytes);
// ws (16-byte aligned, ws_bytes long, or NULL) holds the partial sums when K
// is split; a second kernel then adds them into y.
hipError_t launch_gemm(const WeightView &w, const ActView &x, const OutView &y,
                       float *ws, uint64_t ws_bytes, hipStream_t stream);
// count (1 .. QMM_GEMM_BATCH_MAX) products sharing the type, K and N in one
// launch, without a K split; items with no rows own no tiles.
hipError_t launch_gemm_batch(const WeightView *w, const ActView *x, const OutView *y, int count,
                             hipStream_t stream);
// The fused gate/up prefill projection with the SwiGLU epilogue:
// h[n][m] = Swish(sum_k Wg'[m][k] x[n][k]) * sum_k Wu'[m][k] x[n][k]
// (wg and wu share the type, K and M; K is never split).
hipError_t launch_gemm_swiglu(const WeightView &wg, const WeightView &wu, const ActView &x, const OutView &h,
                              hipStream_t stream);

}  // namespace qmm
