// gemm.hip -- prefill GEMM: block-quantized weights x bf16 activations -> fp32.
//
// Y[n][m] = sum_k W'[m][k] * X[n][k] for many tokens at once (No Python!
// Building an AI Inference Engine Exclusively in C++, §6: C_ij = sum_k A_ik B_kj;
// §6.1: tile the matrices, repack tiles so the inner loop reads contiguous
// data, and feed the multiply-add units).  On gfx950 the multiply-add units are
// the bf16 matrix cores: each weight tile is dequantized once per workgroup
// (Development Guide for Small AI Models (TinyLLaMA, etc.) Using C++, §6.2:
// unpack, multiply by the block scale) into LDS as bf16, the activation tile
// is copied to LDS, and v_mfma_f32_32x32x16_bf16 accumulates in fp32.
//
// Tiling: a 256-thread workgroup owns a 128 (tokens) x 128 (weight rows)
// output tile; its four waves each own 64 x 64 (2 x 2 MFMA tiles of 32 x 32).
// K advances 64 (two 32-blocks) per step; LDS is double buffered so each step
// needs one barrier, and the next step's global loads are issued before the
// current step's matrix-core work.  Tokens sit on the MFMA row side so that
// each lane's results run along the contiguous m dimension of Y.
#include "qmm_internal.h"

namespace qmm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128;        // weight rows per tile
constexpr int BN = 128;        // tokens per tile
constexpr int BK = 64;         // K per step (two 32-blocks)
constexpr int LDS_STRIDE = BK + 8;   // bf16 elements per LDS row (+16 B pad)

struct GemmArgs {
    const uint8_t *w;
    uint64_t pitch;
    int64_t M;
    int64_t K;
    int64_t qoff;
    const uint16_t *x;      // bf16 bits, row n at x + n * x_pitch
    uint64_t x_pitch;
    int64_t N;
    float *y;
    uint64_t y_pitch;
};

__device__ inline uint32_t pack_bf16(float lo, float hi)
{
    const __bf16 a = static_cast<__bf16>(lo);
    const __bf16 b = static_cast<__bf16>(hi);
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// Dequantize one 32-block (codes in registers) to 32 bf16 values in k order,
// packed two per dword: out[0..15].
template <int WT>
__device__ inline void dequant_block(const uint4 *q, float d, uint32_t out[16])
{
    if (WT == W_Q4_0) {
        const uint32_t wd[4] = {q[0].x, q[0].y, q[0].z, q[0].w};
        float v[32];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t byte = (wd[i] >> (8 * e)) & 0xFFu;
                v[4 * i + e] = (float)((int)(byte & 0x0Fu) - 8) * d;
                v[16 + 4 * i + e] = (float)((int)(byte >> 4) - 8) * d;
            }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) out[i] = pack_bf16(v[2 * i], v[2 * i + 1]);
    } else {
        const uint32_t wd[8] = {q[0].x, q[0].y, q[0].z, q[0].w, q[1].x, q[1].y, q[1].z, q[1].w};
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int32_t wv = (int32_t)wd[i / 2];
            const int sh = 16 * (i & 1);
            const float a = (float)(int8_t)(wv >> sh) * d;
            const float b = (float)(int8_t)(wv >> (sh + 8)) * d;
            out[i] = pack_bf16(a, b);
        }
    }
}

template <int WT>
__global__ __launch_bounds__(256) void gemm_kernel(const GemmArgs a)
{
    constexpr int QV = (WT == W_Q4_0) ? 1 : 2;    // uint4 loads per block of codes
    __shared__ __attribute__((aligned(16))) uint16_t xs[2][BN * LDS_STRIDE];
    __shared__ __attribute__((aligned(16))) uint16_t ws[2][BM * LDS_STRIDE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave & 1;     // weight-row half of the tile
    const int wn = wave >> 1;    // token half of the tile
    const int64_t m0 = (int64_t)blockIdx.x * BM;
    const int64_t n0 = (int64_t)blockIdx.y * BN;
    const int64_t nblk = a.K / 32;
    const int64_t steps = (a.K + BK - 1) / BK;

    // Loader roles: thread t stages weight row t/2, block t%2 of the step,
    // and token t/2, k-half t%2 of the step.
    const int lrow = tid >> 1;
    const int lhalf = tid & 1;
    int64_t wrow = m0 + lrow;
    wrow = wrow < a.M ? wrow : a.M - 1;
    const uint8_t *wr = a.w + (uint64_t)wrow * a.pitch;
    const int64_t xrow = n0 + lrow;
    const bool xvalid = xrow < a.N;
    const uint16_t *xr = a.x + (uint64_t)(xvalid ? xrow : 0) * a.x_pitch;

    uint4 qreg[QV];
    uint16_t sreg;
    uint4 xreg[4];

    auto load_step = [&](int64_t s) {
        const int64_t b = s * 2 + lhalf;
        if (b < nblk) {
#pragma unroll
            for (int v = 0; v < QV; ++v)
                qreg[v] = *reinterpret_cast<const uint4 *>(wr + a.qoff + b * 16 * QV + 16 * v);
            sreg = *reinterpret_cast<const uint16_t *>(wr + 2 * b);
        } else {
#pragma unroll
            for (int v = 0; v < QV; ++v) qreg[v] = make_uint4(0, 0, 0, 0);
            sreg = 0;
        }
        if (xvalid && b < nblk) {
            const uint4 *src = reinterpret_cast<const uint4 *>(xr + b * 32);
#pragma unroll
            for (int v = 0; v < 4; ++v) xreg[v] = src[v];
        } else {
#pragma unroll
            for (int v = 0; v < 4; ++v) xreg[v] = make_uint4(0, 0, 0, 0);
        }
    };

    auto store_step = [&](int buf) {
        uint32_t deq[16];
        dequant_block<WT>(qreg, (float)__builtin_bit_cast(_Float16, sreg), deq);
        uint4 *wdst = reinterpret_cast<uint4 *>(&ws[buf][lrow * LDS_STRIDE + 32 * lhalf]);
#pragma unroll
        for (int v = 0; v < 4; ++v)
            wdst[v] = make_uint4(deq[4 * v], deq[4 * v + 1], deq[4 * v + 2], deq[4 * v + 3]);
        uint4 *xdst = reinterpret_cast<uint4 *>(&xs[buf][lrow * LDS_STRIDE + 32 * lhalf]);
#pragma unroll
        for (int v = 0; v < 4; ++v) xdst[v] = xreg[v];
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[s][t][r] = 0.0f;

    if (steps > 0) {
        load_step(0);
        store_step(0);
    }
    __syncthreads();

    const int frow = lane & 31;         // row of the MFMA operand this lane feeds
    const int fk = (lane >> 5) * 8;     // its 8-element k group
    for (int64_t s = 0; s < steps; ++s) {
        const int buf = (int)(s & 1);
        if (s + 1 < steps) load_step(s + 1);
#pragma unroll
        for (int kk = 0; kk < BK; kk += 16) {
            bf16x8 af[2], bfr[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const uint4 va = *reinterpret_cast<const uint4 *>(
                    &xs[buf][(wn * 64 + i * 32 + frow) * LDS_STRIDE + kk + fk]);
                af[i] = __builtin_bit_cast(bf16x8, va);
                const uint4 vb = *reinterpret_cast<const uint4 *>(
                    &ws[buf][(wm * 64 + i * 32 + frow) * LDS_STRIDE + kk + fk]);
                bfr[i] = __builtin_bit_cast(bf16x8, vb);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        if (s + 1 < steps) store_step(buf ^ 1);
        __syncthreads();
    }

    // Epilogue: acc[i][j] register r holds token 8*(r/4) + 4*(lane/32) + r%4
    // of sub-tile i and weight row lane%32 of sub-tile j.
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t m = m0 + wm * 64 + j * 32 + (lane & 31);
            if (m >= a.M) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t n = n0 + wn * 64 + i * 32 + 8 * (r / 4) + 4 * (lane >> 5) + (r % 4);
                if (n < a.N) a.y[(uint64_t)n * a.y_pitch + m] = acc[i][j][r];
            }
        }
    }
}

}  // namespace

hipError_t launch_gemm(const WeightView &w, const ActView &x, const OutView &y,
                       hipStream_t stream)
{
    if (w.M == 0 || x.N == 0) return hipSuccess;
    GemmArgs a;
    a.w = w.base;
    a.pitch = w.pitch;
    a.M = w.M;
    a.K = w.K;
    a.qoff = quant_offset(w.K);
    a.x = static_cast<const uint16_t *>(x.data);
    a.x_pitch = x.pitch_elems;
    a.N = x.N;
    a.y = y.data;
    a.y_pitch = y.pitch_elems;
    const dim3 grid((unsigned)((w.M + BM - 1) / BM), (unsigned)((x.N + BN - 1) / BN));
    if (w.type == W_Q4_0)
        hipLaunchKernelGGL(gemm_kernel<W_Q4_0>, grid, dim3(256), 0, stream, a);
    else if (w.type == W_Q8_0)
        hipLaunchKernelGGL(gemm_kernel<W_Q8_0>, grid, dim3(256), 0, stream, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace qmm
