// quant.hip -- load-time Q8_0 / Q4_0 quantization and dequantization on the GPU.
//
// Block rule (A Complete Guide to llama.cpp and Customization with C++, §2.2:
// w_i ~= Delta * q_i with Delta from the block's largest |w|; Development Guide
// for Small AI Models (TinyLLaMA, etc.) Using C++, §6.1: 32 values per block,
// one FP16 scale):
//   amax = max |w_i|;  Delta = fp16_rne(amax / 127) (Q8_0) or fp16_rne(amax / 8) (Q4_0)
//   q_i  = roundf(w_i / Delta)  -- one correctly rounded binary32 division by the
//          stored scale, then round half away from zero;
//   Q8_0 clamps q to [-127, 127]; Q4_0 stores q + 8 clamped to [0, 15].
// The library is built without fast-math, so '/' is the IEEE division and
// the fp16 / bf16 conversions round to nearest even: the codes are bit-exact.
//
// A second Q4 rule is the pages' own (A Complete Guide to llama.cpp ...,
// §2.2: Delta = max|w| / 7, q_i in [-8, 7]): the same steps with 7 as the
// divisor, stored the same way (clamp(q + 8, 0, 15) = clamp(q, -8, 7) + 8).
//
// 64-weight blocks (same page: the block length is usually 32 or 64) take
// the same steps over 64 values; their codes are stored as two runs of 32
// laid out like a 32-block's.
//
// These kernels run once per weight at load time, so they favour clarity:
// one thread per block.
#include "qmm_internal.h"

namespace qmm {
namespace {

__device__ inline uint16_t f32_to_f16_bits(float f)
{
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

__device__ inline float f16_bits_to_f32(uint16_t h)
{
    return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

template <int TYPE, int DIV, int BS>
__global__ __launch_bounds__(256) void quantize_kernel(const float *__restrict__ src,
                                                       uint64_t src_pitch, int64_t K, int64_t M,
                                                       uint8_t *__restrict__ dst, uint64_t dst_pitch)
{
    constexpr int RUNS = BS / 32;          // 32-code runs per block, laid out as in the 32-blocks
    const int64_t nblk = K / BS;
    const int64_t total = M * nblk;
    const int64_t qoff = quant_offset(K, BS == 64 ? 1 : 0);
    const int64_t qbytes = (TYPE == W_Q8_0) ? K : K / 2;
    const int64_t row_bytes = qoff + ((qbytes + 15) / 16) * 16;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = i / nblk;
        const int64_t b = i - r * nblk;
        const float *w = src + r * src_pitch + b * BS;
        float v[BS];
        float amax = 0.0f;
#pragma unroll
        for (int j = 0; j < BS; ++j) {
            v[j] = w[j];
            amax = fmaxf(amax, fabsf(v[j]));
        }
        const float s = amax / (float)DIV;
        const uint16_t sb = f32_to_f16_bits(s);
        const float d = f16_bits_to_f32(sb);
        uint8_t *row = dst + r * dst_pitch;
        *reinterpret_cast<uint16_t *>(row + 2 * b) = sb;
#pragma unroll
        for (int h = 0; h < RUNS; ++h) {
            const float *vr = v + 32 * h;
            const int64_t run = b * RUNS + h;          // 32-code run within the row
            if (TYPE == W_Q8_0) {
                uint32_t words[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) words[j] = 0;
#pragma unroll
                for (int j = 0; j < 32; ++j) {
                    float q = 0.0f;
                    if (d != 0.0f) q = fminf(fmaxf(roundf(vr[j] / d), -127.0f), 127.0f);
                    words[j / 4] |= (uint32_t)(uint8_t)(int8_t)q << (8 * (j % 4));
                }
                uint4 *out = reinterpret_cast<uint4 *>(row + qoff + 32 * run);
                out[0] = make_uint4(words[0], words[1], words[2], words[3]);
                out[1] = make_uint4(words[4], words[5], words[6], words[7]);
            } else {
                uint32_t nib[32];
#pragma unroll
                for (int j = 0; j < 32; ++j) {
                    float q = 8.0f;
                    if (d != 0.0f) q = fminf(fmaxf(roundf(vr[j] / d) + 8.0f, 0.0f), 15.0f);
                    nib[j] = (uint32_t)q;
                }
                uint32_t words[4] = {0, 0, 0, 0};
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    words[j / 4] |= (nib[j] | (nib[j + 16] << 4)) << (8 * (j % 4));
                *reinterpret_cast<uint4 *>(row + qoff + 16 * run) =
                    make_uint4(words[0], words[1], words[2], words[3]);
            }
        }
        if (b == 0) {
            for (int64_t p = 2 * nblk; p < qoff; ++p) row[p] = 0;
            for (int64_t p = qoff + qbytes; p < row_bytes; ++p) row[p] = 0;
        }
    }
}

template <int TYPE, int BS>
__global__ __launch_bounds__(256) void dequantize_kernel(const uint8_t *__restrict__ src,
                                                         uint64_t src_pitch, int64_t K, int64_t M,
                                                         float *__restrict__ dst, uint64_t dst_pitch)
{
    constexpr int RUNS = BS / 32;
    const int64_t nblk = K / BS;
    const int64_t total = M * nblk;
    const int64_t qoff = quant_offset(K, BS == 64 ? 1 : 0);
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = i / nblk;
        const int64_t b = i - r * nblk;
        const uint8_t *row = src + r * src_pitch;
        const float d = f16_bits_to_f32(*reinterpret_cast<const uint16_t *>(row + 2 * b));
#pragma unroll
        for (int h = 0; h < RUNS; ++h) {
            const int64_t run = b * RUNS + h;
            float *out = dst + r * dst_pitch + run * 32;
            if (TYPE == W_Q8_0) {
                const int8_t *q = reinterpret_cast<const int8_t *>(row + qoff + 32 * run);
#pragma unroll
                for (int j = 0; j < 32; ++j) out[j] = d * (float)q[j];
            } else {
                const uint8_t *q = row + qoff + 16 * run;
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    out[j] = d * (float)((int)(q[j] & 0x0F) - 8);
                    out[j + 16] = d * (float)((int)(q[j] >> 4) - 8);
                }
            }
        }
    }
}

__global__ __launch_bounds__(256) void f16_to_f32_kernel(const uint8_t *__restrict__ src,
                                                         uint64_t src_pitch, int64_t K, int64_t M,
                                                         float *__restrict__ dst, uint64_t dst_pitch)
{
    const int64_t total = M * K;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = i / K;
        const int64_t k = i - r * K;
        const uint16_t *row = reinterpret_cast<const uint16_t *>(src + r * src_pitch);
        dst[r * dst_pitch + k] = f16_bits_to_f32(row[k]);
    }
}

unsigned grid_for(int64_t items)
{
    const int64_t blocks = (items + 255) / 256;
    return (unsigned)(blocks < 65536 ? (blocks > 0 ? blocks : 1) : 65536);
}

}  // namespace

hipError_t launch_quantize(const float *src, uint64_t src_pitch_elems, int64_t K, int64_t M,
                           uint8_t *dst, uint64_t dst_pitch, int type, hipStream_t stream,
                           bool q4_amax7, int scale_shift)
{
    const int64_t items = M * (K / (scale_shift ? 64 : 32));
    if (items == 0) return hipSuccess;
    const dim3 grid(grid_for(items)), block(256);
#define QMM_QUANT(T, D, B) hipLaunchKernelGGL((quantize_kernel<T, D, B>), grid, block, 0, stream, \
                                              src, src_pitch_elems, K, M, dst, dst_pitch)
    if (scale_shift == 0) {
        if (type == W_Q8_0) QMM_QUANT(W_Q8_0, 127, 32);
        else if (q4_amax7) QMM_QUANT(W_Q4_0, 7, 32);
        else QMM_QUANT(W_Q4_0, 8, 32);
    } else {
        if (type == W_Q8_0) QMM_QUANT(W_Q8_0, 127, 64);
        else if (q4_amax7) QMM_QUANT(W_Q4_0, 7, 64);
        else QMM_QUANT(W_Q4_0, 8, 64);
    }
#undef QMM_QUANT
    return hipGetLastError();
}

hipError_t launch_dequantize(const uint8_t *src, uint64_t src_pitch, int64_t K, int64_t M,
                             int type, float *dst, uint64_t dst_pitch_elems, hipStream_t stream,
                             int scale_shift)
{
    if (type == W_F16) {
        if (M * K == 0) return hipSuccess;
        hipLaunchKernelGGL(f16_to_f32_kernel, dim3(grid_for(M * K)), dim3(256), 0, stream,
                           src, src_pitch, K, M, dst, dst_pitch_elems);
        return hipGetLastError();
    }
    const int64_t items = M * (K / (scale_shift ? 64 : 32));
    if (items == 0) return hipSuccess;
    const dim3 grid(grid_for(items)), block(256);
    if (type == W_Q8_0) {
        if (scale_shift) hipLaunchKernelGGL((dequantize_kernel<W_Q8_0, 64>), grid, block, 0, stream, src, src_pitch, K, M, dst, dst_pitch_elems);
        else hipLaunchKernelGGL((dequantize_kernel<W_Q8_0, 32>), grid, block, 0, stream, src, src_pitch, K, M, dst, dst_pitch_elems);
    } else {
        if (scale_shift) hipLaunchKernelGGL((dequantize_kernel<W_Q4_0, 64>), grid, block, 0, stream, src, src_pitch, K, M, dst, dst_pitch_elems);
        else hipLaunchKernelGGL((dequantize_kernel<W_Q4_0, 32>), grid, block, 0, stream, src, src_pitch, K, M, dst, dst_pitch_elems);
    }
    return hipGetLastError();
}

}  // namespace qmm
