// wave_reduce.h -- cross-lane sums of the GEMV kernels (device code only).
//
// A wave of 64 lanes enters with V partial values per lane and leaves with
// the V full sums spread over lanes 32 .. 32+V-1 (a transposed butterfly:
// each exchange halves the set of values a lane carries).  Every exchange is
// a VALU operation (DPP or v_permlane*_swap), none goes through LDS.
#pragma once

#include <hip/hip_runtime.h>

namespace qmm {
namespace {

// The value of a partner lane for the exchange on lane bit B: a lane whose
// index has the same lower bits 0..B-1 and the other value of bit B.  The
// pairing is a bijection, not necessarily an involution, which is all the
// butterfly below needs (every partial value is received exactly once).
// Every exchange stays on the VALU: DPP quad permutations for bits 0 and 1,
// DPP rotations by 4 and 8 lanes within a 16-lane row for bits 2 and 3,
// v_permlane16_swap / v_permlane32_swap for bits 4 and 5.
// A copy of v that the compiler cannot prove equal to v.  A swap whose two
// operands are provably the same value has had the lane-dependent choice
// between its two results folded into one of them (observed with the ROCm
// 7.2 compiler), which is wrong for half of the lanes; distinct operands keep
// the choice.
__device__ inline unsigned opaque_copy(unsigned v)
{
    unsigned r;
    asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "v"(v));
    return r;
}

template <int B>
__device__ inline float partner(float v, int lane)
{
    const int iv = __builtin_bit_cast(int, v);
    if constexpr (B == 0) {
        return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(iv, 0xB1, 0xF, 0xF, true));
    } else if constexpr (B == 1) {
        return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(iv, 0x4E, 0xF, 0xF, true));
    } else if constexpr (B == 2) {
        return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(iv, 0x124, 0xF, 0xF, true));  // row_ror:4
    } else if constexpr (B == 3) {
        return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(iv, 0x128, 0xF, 0xF, true));  // row_ror:8
    } else if constexpr (B == 4) {
        // [0]: odd rows receive the even rows' values; [1]: even rows the odd rows'
        const auto p = __builtin_amdgcn_permlane16_swap((unsigned)iv, opaque_copy((unsigned)iv), false, false);
        return __builtin_bit_cast(float, (lane & 16) ? p[0] : p[1]);
    } else {
        const auto p = __builtin_amdgcn_permlane32_swap((unsigned)iv, opaque_copy((unsigned)iv), false, false);
        return __builtin_bit_cast(float, (lane & 32) ? p[0] : p[1]);
    }
}

// Transposed butterfly over the 64 lanes of a wave.  Every lane enters with
// V partial values; each exchange on lane bit B (from bit 0 up) halves the
// set a lane carries, then the single remaining value is all-reduced over
// the higher bits.  On exit every lane of the upper half (lanes 32..63)
// holds the full wave sum of value value_index<V>(lane), so lanes
// 32 .. 32+V-1 together hold all V sums.
template <int V, int B>
struct WaveReduce {
    static __device__ inline float run(const float *v, int lane)
    {
        constexpr int H = V / 2;
        const bool upper = ((lane >> B) & 1) != 0;
        float keep[H];
#pragma unroll
        for (int i = 0; i < H; ++i) {
            const float send = upper ? v[i] : v[i + H];
            const float mine = upper ? v[i + H] : v[i];
            keep[i] = mine + partner<B>(send, lane);
        }
        return WaveReduce<H, B + 1>::run(keep, lane);
    }
};
// v_permlane32_swap: lanes 32..63 receive the values of lanes 0..31 (a
// VALU exchange, no LDS crossbar).
__device__ inline float lower_half_to_upper(float v)
{
    const unsigned u = __builtin_bit_cast(unsigned, v);
    return __builtin_bit_cast(float, __builtin_amdgcn_permlane32_swap(u, opaque_copy(u), false, false)[0]);
}

template <int B>
struct WaveReduce<1, B> {
    static __device__ inline float run(const float *v, int lane)
    {
        // all-reduce over bits B..4 (the rotations of bits 2 and 3 add the
        // next quad, then the next two, so every lane ends with its row sum)
        float s = v[0];
        if constexpr (B <= 0) s += partner<0>(s, lane);
        if constexpr (B <= 1) s += partner<1>(s, lane);
        if constexpr (B <= 2) s += partner<2>(s, lane);
        if constexpr (B <= 3) s += partner<3>(s, lane);
        if constexpr (B <= 4) s += partner<4>(s, lane);
        s += lower_half_to_upper(s);      // complete in lanes 32..63 only
        return s;
    }
};

// Index of the value a lane holds after WaveReduce<V, 0>: the halving on bit
// b picks the upper half of the remaining indices, so lane bit b is index
// bit log2(V) - 1 - b.
template <int V>
__device__ inline int value_index(int lane)
{
    int idx = 0;
#pragma unroll
    for (int b = 0; (1 << b) < V; ++b) idx = (idx << 1) | ((lane >> b) & 1);
    return idx;
}

constexpr int ilog2(int v) { return v <= 1 ? 0 : 1 + ilog2(v / 2); }
constexpr int pow2_ceil(int v) { return v <= 1 ? 1 : 2 * pow2_ceil((v + 1) / 2); }

}  // namespace
}  // namespace qmm
