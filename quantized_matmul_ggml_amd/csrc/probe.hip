// probe.hip -- measurement kernels that give the MUL_MAT figures their
// context: the rate at which one launch can stream a buffer of a given size
// out of HBM (the ceiling a decode GEMV of that many bytes can reach: No
// Python! Building an AI Inference Engine Exclusively in C++, §9, inference
// is bound by memory bandwidth), and the shader clock under load (the clock
// the matrix-core peak assumes).
//
//  * stream_read_kernel: every thread reads 16-byte units with buffer loads,
//    two batches of U loads in flight (the next batch is issued before the
//    current one is consumed), grid-stride over the buffer; each workgroup
//    xor-folds what it read into one word, so no load can be dropped.  The
//    loads carry the GEMVs' weight-streaming cache policy (kStreamLoad), so
//    the ceiling is measured the way the weights are read.
//  * clock_kernel: each wave times a long dependent chain (binary32 FMAs,
//    or bf16 matrix instructions) with the shader-clock counter (s_memtime)
//    and the constant-rate counter (s_memrealtime); the ratio of the two
//    deltas times the constant counter's rate is the shader clock.
#include "qmm_internal.h"

namespace qmm {
namespace {

constexpr int kReadThreads = 256;
constexpr int kReadU = 4;             // 16-byte loads per thread per batch

__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const uint8_t *src, uint32_t bytes,
                                                                    uint32_t *sink)
{
    const __amdgpu_buffer_rsrc_t res = __builtin_amdgcn_make_buffer_rsrc((void *)src, 0, (int)bytes, BUFFER_FLAGS);
    const uint32_t units = bytes / 16;
    const uint32_t stride = gridDim.x * kReadThreads;        // units per batch row
    const uint32_t batch = stride * kReadU;                  // units per batch
    const uint32_t first = blockIdx.x * kReadThreads + threadIdx.x;
    const uint32_t iters = (units + batch - 1) / batch;
    auto load = [&](uint4 (&v)[kReadU], uint32_t it) {
#pragma unroll
        for (int j = 0; j < kReadU; ++j) {
            const uint32_t u = it * batch + (uint32_t)j * stride + first;
            const uint32_t off = u < units ? u * 16u : OUT_OF_RANGE;
            v[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(res, off, 0, kStreamLoad));
        }
    };
    uint4 acc = make_uint4(0, 0, 0, 0);
    uint4 cur[kReadU], nxt[kReadU];
    load(cur, 0);
    for (uint32_t it = 0; it < iters; ++it) {
        load(nxt, it + 1);                                   // past the end: reads nothing
#pragma unroll
        for (int j = 0; j < kReadU; ++j) {
            acc.x ^= cur[j].x;
            acc.y ^= cur[j].y;
            acc.z ^= cur[j].z;
            acc.w ^= cur[j].w;
            cur[j] = nxt[j];
        }
    }
    uint32_t r = acc.x ^ acc.y ^ acc.z ^ acc.w;
    for (int o = 32; o >= 1; o >>= 1) r ^= __shfl_xor(r, o);
    __shared__ uint32_t part[kReadThreads / 64];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = r;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t t = 0;
        for (int w = 0; w < kReadThreads / 64; ++w) t ^= part[w];
        sink[blockIdx.x] = t;
    }
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

// The inner loop of a block-quantized GEMM on the matrix cores, per 32-block
// of K and 32 x 32 output tile, four independent tiles per round:
//  * RESCALE 0: bf16 operands, the block's two v_mfma_f32_32x32x16_bf16
//    accumulating in place (the scale was applied to the weights before the
//    matrix instruction, as in gemm.hip);
//  * RESCALE 1: int8 operands (Q8_0 activations times weight codes), one
//    v_mfma_i32_32x32x32_i8 per block into a fresh int32 tile, which is then
//    converted and added with the block's weight scale (each lane's 16
//    outputs share one weight row, so one scale per lane): 16 conversions
//    and 16 FMAs per lane;
//  * RESCALE 2: the same with each output also multiplied by its token's
//    activation scale (16 different ones per lane), as Q8_0 activations
//    need: 16 more multiplies.
// "A Complete Guide to llama.cpp and Customization with C++", §2.2: the
// integer sum of a block must be scaled by Delta_w * Delta_x before blocks
// are added, which is what the int8 modes pay for on the vector ALUs.
template <int RESCALE>
__device__ inline float block_gemm_chain(int iters, float seed)
{
    constexpr int T = 4;
    f32x16 acc[T] = {};
    bf16x8 va[T], vb[T];
    i32x4 ia[T], ib[T];
    float sx[16];
#pragma unroll
    for (int t = 0; t < T; ++t) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            va[t][i] = (__bf16)(seed * (float)(i + 1 + t));
            vb[t][i] = (__bf16)(seed * (float)((threadIdx.x + t) & 7));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ia[t][i] = (int)(threadIdx.x * 0x01010101u + i + t);
            ib[t][i] = (int)(0x03030303u * (i + 1 + t));
        }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) sx[r] = seed * (float)(r + 1);
    const float sw = seed * 0.25f;
    for (int it = 0; it < iters; ++it) {
        // operands the compiler must treat as new every round (they stand
        // for the next block's fragments), so no matrix instruction is
        // shared between tiles or hoisted out of the loop
#pragma unroll
        for (int t = 0; t < T; ++t) {
            if constexpr (RESCALE == 0) asm volatile("" : "+v"(va[t]), "+v"(vb[t]));
            else asm volatile("" : "+v"(ia[t]), "+v"(ib[t]));
        }
        if constexpr (RESCALE == 0) {
#pragma unroll
            for (int t = 0; t < T; ++t) {
                acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[t], vb[t], acc[t], 0, 0, 0);
                acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vb[t], va[t], acc[t], 0, 0, 0);
            }
        } else {
            i32x16 d[T];
#pragma unroll
            for (int t = 0; t < T; ++t) d[t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ia[t], ib[t], i32x16{}, 0, 0, 0);
#pragma unroll
            for (int t = 0; t < T; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float v = RESCALE == 2 ? (float)d[t][r] * sx[r] : (float)d[t][r];
                    acc[t][r] = fmaf(v, sw, acc[t][r]);
                }
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[t][r];
    return s;
}

// out[2 * wave] = shader-clock delta, out[2 * wave + 1] = constant-counter
// delta over `iters` rounds of the chosen chain (mode 0: 16 independent
// binary32 FMA chains; mode 1: 4 independent bf16 matrix-instruction chains;
// modes 2, 3, 4: block_gemm_chain with RESCALE 0, 1, 2).
__global__ __launch_bounds__(256) void clock_kernel(uint64_t *out, int iters, int mode, float seed)
{
    const int wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    float a[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) a[i] = seed * (float)(threadIdx.x + i);
    f32x16 c[4] = {};
    bf16x8 va, vb;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        va[i] = (__bf16)(seed * (float)(i + 1));
        vb[i] = (__bf16)(seed * (float)(threadIdx.x & 7));
    }
    if (mode >= 2) {
        const uint64_t t0 = __builtin_amdgcn_s_memtime();
        const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
        const float s = mode == 2 ? block_gemm_chain<0>(iters, seed)
                      : mode == 3 ? block_gemm_chain<1>(iters, seed) : block_gemm_chain<2>(iters, seed);
        asm volatile("" ::"v"(s));
        const uint64_t t1 = __builtin_amdgcn_s_memtime();
        const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
        if ((threadIdx.x & 63) == 0) {
            out[2 * wave] = t1 - t0;
            out[2 * wave + 1] = r1 - r0;
        }
        return;
    }
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    if (mode == 0) {
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int i = 0; i < 16; ++i) a[i] = fmaf(a[i], 0.999f, seed);
        }
    } else {
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int i = 0; i < 4; ++i) c[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, vb, c[i], 0, 0, 0);
        }
    }
    // make the chains' results needed before the end stamps
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += a[i] + c[i & 3][i];
    asm volatile("" ::"v"(s));
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    if ((threadIdx.x & 63) == 0) {
        out[2 * wave] = t1 - t0;
        out[2 * wave + 1] = r1 - r0;
    }
}

}  // namespace

hipError_t launch_stream_read(const void *src, uint64_t bytes, uint32_t *sink, int workgroups, hipStream_t stream)
{
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)workgroups), dim3(kReadThreads), 0, stream,
                       static_cast<const uint8_t *>(src), (uint32_t)bytes, sink);
    return hipGetLastError();
}

hipError_t launch_clock_probe(uint64_t *out, int workgroups, int iters, int mode, hipStream_t stream)
{
    hipLaunchKernelGGL(clock_kernel, dim3((unsigned)workgroups), dim3(256), 0, stream, out, iters, mode, 0.5f);
    return hipGetLastError();
}

}  // namespace qmm
