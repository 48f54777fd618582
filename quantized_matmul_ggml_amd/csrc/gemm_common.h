// gemm_common.h -- what the two prefill GEMM kernels share: the launch
// arguments (one product, a batch of products, or a product whose K is split
// into ranges), the workgroup-to-tile mapping, and small bit-level helpers.
// Internal to the library.
#pragma once

#include "qmm_internal.h"

#include <type_traits>

namespace qmm {

constexpr int kMaxGemmItems = QMM_GEMM_BATCH_MAX;

// One product of a launch (several share one launch in a batch): its
// weights, tokens and output, and the first tile index it owns.
struct GemmItem {
    const uint8_t *w;
    uint64_t pitch;
    int64_t M;
    const uint16_t *x;      // bf16 bits, row n at x + n * x_pitch
    uint64_t x_pitch;
    float *y;               // the output, or the first partial-sum slab
    uint64_t y_pitch;
    const uint8_t *w2;      // fused SwiGLU launches: the up projection (w is the gate)
    uint64_t pitch2;
    int tile_begin;
    int pad;
};

struct GemmArgs {
    int64_t K;              // shared by the items, like the type, N and qoff
    int64_t qoff;
    int64_t N;
    int n_tiles;            // token tiles
    int n_splits;           // K ranges per tile (1: the whole K)
    int split_steps;        // K-steps of 64 per range, a multiple of 8
    int n_items;
    uint64_t split_stride;  // floats between the slabs of consecutive ranges
    GemmItem item[kMaxGemmItems];
};

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Round two floats to bf16 (nearest even) in one v_cvt_pk_bf16_f32.
__device__ inline uint32_t pack_bf16(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// (a & m) | c in one VALU op (written out: the compiler splits it, since a
// gfx9 VOP3 takes no literal and c must sit in a register).
__device__ inline uint32_t and_or(uint32_t a, uint32_t m, uint32_t c)
{
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(m), "v"(c));
    return r;
}

__device__ inline float lo_half(uint32_t p) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(p & 0xFFFFu)); }
__device__ inline float hi_half(uint32_t p) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(p >> 16)); }

// Calls f(std::integral_constant<int, 0>{}) .. f(std::integral_constant<int, N-1>{}).
template <int N, int I = 0, class F>
__device__ inline void static_for(F &&f)
{
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<N, I + 1>(f);
    }
}

// The launch-order index of this workgroup.  Workgroups are handed to the
// chip's eight XCDs in turn (workgroup b to XCD b mod 8), each XCD with its
// own L2; renumbering them so that XCD x runs a contiguous run of the
// launch's (tile, range) order lets the token tiles of one weight tile, which
// read the same weight rows, share that XCD's L2.
__device__ inline int xcd_order_index()
{
    const int b = (int)blockIdx.x, nwg = (int)gridDim.x;
    const int x = b % 8, i = b / 8, q = nwg / 8, r = nwg % 8;
    return x * q + (x < r ? x : r) + i;
}

// Register-dequantizing GEMM (gemm_rq.hip) for Q4_0 / Q8_0 codes, with
// 32-weight scales (ss 0) or 64-weight scales (ss 1); sw: the fused gate/up
// pair (w the gate, w2 the up matrix, 64 rows of each per tile).
hipError_t launch_gemm_rq(const GemmArgs &a, unsigned blocks, int type, int ss, bool sw, hipStream_t stream);
bool gemm_rq_handles(int type);

}  // namespace qmm
