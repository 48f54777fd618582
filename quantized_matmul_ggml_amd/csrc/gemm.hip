// gemm.hip -- prefill GEMM: block-quantized weights x bf16 activations -> fp32.
//
// This file holds the launch planning (K split, batches), the split-K slab
// sum, and the producer/consumer kernel below, which serves F16 weights and
// the fused gate/up SwiGLU pair; single Q4_0 / Q8_0 products and their
// batches run on the register-dequantizing kernel of gemm_rq.hip.
//
// Y[n][m] = sum_k W'[m][k] * X[n][k] for many tokens at once (No Python!
// Building an AI Inference Engine Exclusively in C++, §6: C_ij = sum_k A_ik B_kj;
// §6.1: tile the matrices, repack tiles so the inner loop reads contiguous
// data, and feed the multiply-add units).  On gfx950 the multiply-add units are
// the bf16 matrix cores: each weight tile is dequantized once per workgroup
// (Development Guide for Small AI Models (TinyLLaMA, etc.) Using C++, §6.2:
// unpack, multiply by the block scale) into LDS as bf16, and
// v_mfma_f32_32x32x16_bf16 accumulates in fp32.
//
// The workgroup is split by role.  Of its eight waves, four (one per SIMD)
// load the weight and token tiles, dequantize the weights and write both into
// a four-stage LDS ring, two K-steps ahead of use; the other four (again one per SIMD) read operand
// fragments from LDS and issue the matrix instructions.  Each SIMD thus holds
// one wave of each kind, so the dequantization arithmetic of one issues while
// the matrix instructions of the other run.
//
// Tile: 128 weight rows x 128 tokens, K advancing 64 (two 32-blocks) per step;
// each consumer wave owns 64 x 64 of the output (2 x 2 MFMA tiles of 32 x 32).
// Tokens sit on the MFMA row side so that each lane's results run along the
// contiguous m dimension of Y.
//
// Loads go through buffer resources based at the tile's first row and sized
// to the bytes the operands span, so rows and tokens past the end read as
// zero; blocks past the end of K get a zero scale and zero tokens.
//
// One launch serves three callers:
//  * one product, with K optionally split into ranges (a workgroup per tile
//    and range) whose partial sums go to a caller workspace and are added in
//    range order by split_sum_kernel (products with too few tiles for the
//    chip; gemm_plan decides);
//  * a batch of up to QMM_GEMM_BATCH_MAX products sharing type, K and N,
//    whose tiles form one grid (a workgroup finds its item by tile index);
//  * the gate/up pair with the SwiGLU epilogue (SW): 64 rows of each matrix
//    per tile, combined in LDS after the last step.
#include "gemm_common.h"

#include <atomic>
#include <mutex>
#include <type_traits>

namespace qmm {
namespace {


constexpr int BM = 128;                   // weight rows per tile
constexpr int BN = 128;                   // tokens per tile
constexpr int BK = 64;                    // K per step (two 32-blocks)
constexpr int LDS_STRIDE = BK + 8;        // bf16 elements per LDS row (+16 B pad)
constexpr int OPERAND_ELEMS = 128 * LDS_STRIDE;
constexpr int STAGE_ELEMS = 2 * OPERAND_ELEMS;   // weights, then tokens
constexpr int STAGES = 4;
constexpr int X_DEPTH = 4;                // K-steps of token loads in flight
static_assert(X_DEPTH == STAGES, "the consumer loop unrolls over both with one index");
constexpr int SCALE_GROUP_STEPS = 8;      // steps whose scales are staged together
constexpr int SCALE_GROUP_BLOCKS = 2 * SCALE_GROUP_STEPS;
constexpr int W_PAIRS = 4;                // pairs of K-steps of weight codes in flight
static_assert(2 * W_PAIRS == SCALE_GROUP_STEPS, "the producer loop unrolls over both with one index");
constexpr int F16_PAIRS = 2;              // pairs of K-steps of F16 weights in flight (4x the bytes of Q4_0)
constexpr int THREADS = 512;

// One producer lane's share of a K-step: one 32-block of one weight row.
template <int WT>
struct WBlock {
    static constexpr int QV = (WT == W_Q4_0) ? 1 : 2;
    u32x4 q[QV];
    uint16_t s;
};

// Dequantize one 32-block to 32 bf16 values in k order, two per dword.
// (code - offset) * d is exact in fp32 (at most 19 significant bits), so each
// value is the bf16 rounding of the exact product.
//  Q4_0: a nibble n moved to bits 6..9 of a binary16 half whose exponent
//        field is that of 16.0 (0x4C00) reads as 16 + n, so one shift and one
//        and-or make two codes, and v_fma_mix_f32 widens the half inside
//        (16 + n) d - 24 d, exact: 2.5 VALU ops per weight with the packing.
//  Q8_0: likewise from the byte code + 128 under the exponent of 1024.
template <int WT>
__device__ inline void dequant_block(const WBlock<WT> &st, uint32_t out[16])
{
    const float d = (float)__builtin_bit_cast(_Float16, st.s);
    if constexpr (WT == W_Q4_0) {
        const float nd = -24.0f * d;
        const uint32_t m = 0x03C003C0u;
        const uint32_t magic = __builtin_amdgcn_readfirstlane(0x4C004C00u);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t w = st.q[0][i];       // byte j: codes k = 4i + j (low), 16 + 4i + j (high)
            const uint32_t p0 = and_or(w << 6, m, magic);   // k = 4i,      4i + 2
            const uint32_t p1 = and_or(w << 2, m, magic);   // k = 16 + 4i, 16 + 4i + 2
            const uint32_t p2 = and_or(w >> 2, m, magic);   // k = 4i + 1,  4i + 3
            const uint32_t p3 = and_or(w >> 6, m, magic);   // k = 16 + 4i + 1, 16 + 4i + 3
            out[2 * i] = pack_bf16(fmaf(lo_half(p0), d, nd), fmaf(lo_half(p2), d, nd));
            out[2 * i + 1] = pack_bf16(fmaf(hi_half(p0), d, nd), fmaf(hi_half(p2), d, nd));
            out[8 + 2 * i] = pack_bf16(fmaf(lo_half(p1), d, nd), fmaf(lo_half(p3), d, nd));
            out[8 + 2 * i + 1] = pack_bf16(fmaf(hi_half(p1), d, nd), fmaf(hi_half(p3), d, nd));
        }
    } else {
        // Q8_0: code + 128 (sign bit flipped) as the low byte of a binary16
        // half with the exponent field of 1024 (0x6400) reads as 1152 + code
        const float nd = -1152.0f * d;
        const uint32_t magic = __builtin_amdgcn_readfirstlane(0x64006400u);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t u = st.q[i / 4][i % 4] ^ 0x80808080u;
            const uint32_t p0 = and_or(u, 0x00FF00FFu, magic);        // k = 4i, 4i + 2
            const uint32_t p1 = and_or(u >> 8, 0x00FF00FFu, magic);   // k = 4i + 1, 4i + 3
            out[2 * i] = pack_bf16(fmaf(lo_half(p0), d, nd), fmaf(lo_half(p1), d, nd));
            out[2 * i + 1] = pack_bf16(fmaf(hi_half(p0), d, nd), fmaf(hi_half(p1), d, nd));
        }
    }
}

// The fp16 scale of a producer lane's block of step S of a scale group:
// 32-weight block 2S + h of the group, which lane S / 2 of the lane's quad
// (the four lanes sharing a pair of rows) holds in dword S % 2 of row
// use0 ? 0 : 1, half h.  With 64-weight blocks (SS = 1) both halves of step
// S share 64-block S: dword 0 of lane S / 2, half S % 2.  The quad broadcast
// is a DPP move.
template <int S, int SS>
__device__ inline uint16_t group_scale(const uint32_t (&sreg)[2][2], bool use0, int h)
{
    constexpr int ctrl = (S / 2) * 0x55;     // quad_perm [S/2, S/2, S/2, S/2]
    constexpr int dw = SS ? 0 : S % 2;
    const uint32_t v0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)sreg[0][dw], ctrl, 0xF, 0xF, false);
    const uint32_t v1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)sreg[1][dw], ctrl, 0xF, 0xF, false);
    return (uint16_t)((use0 ? v0 : v1) >> (16 * (SS ? S % 2 : h)));
}

// Two fp16 weights (one dword) to two bf16 (nearest even): each half widens
// exactly to fp32, then one v_cvt_pk_bf16_f32.
__device__ inline uint32_t f16x2_to_bf16x2(uint32_t w)
{
    const float lo = (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
    const float hi = (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
    return pack_bf16(lo, hi);
}

// Swish(z) = z * sigma(z) = z / (1 + e^{-z}) in binary32 (for z far below
// zero e^{-z} overflows and the quotient is the limit -0).
__device__ inline float swish(float z)
{
    return z / (1.0f + expf(-z));
}

// SW: the fused gate/up projection with the SwiGLU epilogue ("Development
// Guide for Small AI Models (TinyLLaMA, etc.) Using C++", §4.4): a tile is 64
// rows of the gate matrix (tile rows 0..63) and the same 64 rows of the up
// matrix (tile rows 64..127) times 128 tokens; the consumer waves of the two
// halves meet in LDS after the last step, and h = Swish(gate) * up is stored.
template <int WT, int SS, bool SW>
__global__ __launch_bounds__(THREADS) void gemm_kernel(const GemmArgs a)
{
    static_assert(SS == 0 || WT != W_F16, "64-weight blocks are quantized");
    constexpr int QB = (WT == W_Q4_0) ? 16 : 32;     // code bytes per block (quantized rows)
    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
    // STAGES x [weights BM x LDS_STRIDE | tokens BN x LDS_STRIDE] bf16

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // the division runs on the vector unit; the tile is uniform, so move it
    // back to scalar registers (buffer resources must live there)
    // Workgroup b takes K range b % n_splits of tile b / n_splits: steps
    // s0 .. s0 + steps - 1 of K.  Every offset below is relative to s0, and
    // nblk counts the 32-blocks of K from block 2 s0 on.
    // (in the XCD-contiguous order of xcd_order_index)
    const int wgi = xcd_order_index();
    const int split = __builtin_amdgcn_readfirstlane(wgi % a.n_splits);
    const int btile = __builtin_amdgcn_readfirstlane(wgi / a.n_splits);
    // the item owning the tile: the last whose first tile is not past it
    int item = 0;
    for (int i = 1; i < a.n_items; ++i)
        if (btile >= a.item[i].tile_begin) item = i;
    const GemmItem &itm = a.item[item];
    const uint8_t *const Wp = itm.w;
    const uint64_t pitch = itm.pitch;
    const int64_t M = itm.M;
    const uint16_t *const Xp = itm.x;
    const uint64_t x_pitch = itm.x_pitch;
    const uint64_t y_pitch = itm.y_pitch;
    const int tile = btile - itm.tile_begin;
    const int mt = __builtin_amdgcn_readfirstlane(tile / a.n_tiles);
    const int nt = __builtin_amdgcn_readfirstlane(tile - mt * a.n_tiles);
    const int64_t m0 = (int64_t)mt * (SW ? BM / 2 : BM);   // the tile's first matrix row
    const int64_t n0 = (int64_t)nt * BN;
    const int s0 = split * a.split_steps;
    const int64_t nblk = a.K / 32 - 2 * (int64_t)s0;
    const int all_steps = (int)((a.K + BK - 1) / BK);
    const int steps = all_steps - s0 < a.split_steps ? all_steps - s0 : a.split_steps;
    float *const out = itm.y + (uint64_t)split * a.split_stride;

    // Step p of K sits in LDS stage p % STAGES and is complete at barrier p.
    // It is written between barriers p-2 and p-1 (weights by the producers,
    // tokens by the consumers), two steps ahead of its use: between barriers
    // t and t+1 the consumers read step t into registers and multiply step
    // t-1.  The stage written then, that of step t-2, was read in window t-2
    // and those reads were consumed by the matrix instructions of window
    // t-1.  A wave's wait before barrier t+1 leaves its LDS operations of
    // window t in flight and only requires those of window t-1 to have
    // landed.
    //
    // Every global load covers whole row segments with several lanes per
    // row, so that one instruction touches few cache lines: the vector L1
    // serves about one line per two cycles whatever part of it is used.

    if constexpr (WT == W_F16) {
      if (wave >= 4) {
        // ---------------- producers: F16 weights ----------------
        // Same ring protocol as the quantized producers below; the weights
        // are converted to bf16 instead of dequantized.  A pair of K-steps
        // spans 256 bytes of a row (four 32-blocks); load v of a row covers
        // block v of the pair with 4 lanes of 16 bytes (lane q4 holds
        // k = 8 q4 .. 8 q4 + 7 of the block), so an instruction touches 64
        // contiguous bytes of each of 16 rows.  Each lane serves two rows.
        const int pw = wave - 4;
        const int q4 = lane & 3;
        // fused SwiGLU: producers 2 and 3 serve the up matrix (tile rows 64..127)
        const bool upper = SW && pw >= 2;
        const uint8_t *const Wm = upper ? itm.w2 : Wp;
        const uint64_t pm = upper ? itm.pitch2 : pitch;
        const int lrow = upper ? 64 : 0;          // tile row of the matrix's row m0
        const int64_t rows = M - m0 < (SW ? BM / 2 : BM) ? M - m0 : (SW ? BM / 2 : BM);
        const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(Wm + (uint64_t)m0 * pm), 0,
            (int)(uint32_t)((rows - 1) * pm + 2 * a.K), BUFFER_FLAGS);
        const int wrow0 = 32 * pw + 2 * (lane >> 2);
        const uint32_t roff[2] = {(uint32_t)((wrow0 - lrow) * pm) + 16 * q4 + 128u * s0,
                                  (uint32_t)((wrow0 + 1 - lrow) * pm) + 16 * q4 + 128u * s0};
        uint16_t *fdst0 = lds + wrow0 * LDS_STRIDE + 8 * q4;
        struct FPair { u32x4 q[2][4]; };   // [row wrow0 + i][block v of the pair]
        FPair fr[F16_PAIRS];
        auto load_f = [&](FPair &fp, int pair) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    fp.q[i][v] = __builtin_amdgcn_raw_buffer_load_b128(
                        wres, roff[i] + (uint32_t)pair * 256 + 64 * v, 0, 0);
        };
        // step p = 2 pair + s holds blocks 2 s and 2 s + 1 of the pair, i.e.
        // K-blocks 2 p and 2 p + 1; a block past K is written as zeros (its
        // bytes belong to the next row or to the padding)
        auto produce_f = [&](int p, const FPair &fp) {
            const int s = p & 1;
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int bb = 0; bb < 2; ++bb) {
                    const bool live = 2 * p + bb < nblk;
                    const u32x4 q = fp.q[i][2 * s + bb];
                    u32x4 o;
#pragma unroll
                    for (int d = 0; d < 4; ++d) o[d] = live ? f16x2_to_bf16x2(q[d]) : 0u;
                    *reinterpret_cast<u32x4 *>(fdst0 + (p % STAGES) * STAGE_ELEMS + i * LDS_STRIDE + 32 * bb) = o;
                }
        };
#pragma unroll
        for (int j = 0; j < F16_PAIRS; ++j) {
            load_f(fr[j], j);
            __builtin_amdgcn_sched_barrier(0);
        }
        for (int p0 = 0; p0 < steps; p0 += 2 * F16_PAIRS) {
            static_for<2 * F16_PAIRS>([&](auto U) {
                constexpr int u = decltype(U)::value;
                const int p = p0 + u;
                if (p < steps) produce_f(p, fr[(u / 2) % F16_PAIRS]);
                if (u % 2 == 1) load_f(fr[(u / 2) % F16_PAIRS], p / 2 + F16_PAIRS);
                if (p >= 1 && p < steps) asm volatile("s_waitcnt lgkmcnt(4)\n\ts_barrier" ::: "memory");
            });
        }
        if (steps > 0) asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");   // barrier steps - 1
        if constexpr (SW) {          // the consumers' exchange of the two halves
            asm volatile("s_barrier" ::: "memory");
            asm volatile("s_barrier" ::: "memory");
        }
        return;
      }
    } else {
      if (wave >= 4) {
        // ---------------- producers: quantized weights ----------------
        //  * codes: 4 lanes per row covering two steps (four blocks), 16 rows
        //    per load; of the two loads a lane makes per pair of steps, one
        //    holds a block of the first step and one of the second (the
        //    16-byte chunk order is rotated between them);
        //  * scales: 4 lanes per row pair covering eight steps, handed to the
        //    lane that needs each one with a quad broadcast.
        const int pw = wave - 4;
        const int q4 = lane & 3;
        // fused SwiGLU: producers 2 and 3 serve the up matrix (tile rows 64..127)
        const bool upper = SW && pw >= 2;
        const uint8_t *const Wm = upper ? itm.w2 : Wp;
        const uint64_t pm = upper ? itm.pitch2 : pitch;
        const int lrow = upper ? 64 : 0;          // tile row of the matrix's row m0
        const int64_t rows = M - m0 < (SW ? BM / 2 : BM) ? M - m0 : (SW ? BM / 2 : BM);
        const uint32_t row_bytes = (uint32_t)(a.qoff + (WT == W_Q4_0 ? a.K / 2 : a.K));
        const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(Wm + (uint64_t)m0 * pm), 0,
            (int)(uint32_t)((rows - 1) * pm + row_bytes), BUFFER_FLAGS);

        // code load i of a pair covers rows 32 pw + 2 m + i (m = lane / 4)
        // with chunk (q4 + 2 i) % 4 of the pair's four blocks
        const int wrow0 = 32 * pw + 2 * (lane >> 2);
        uint32_t qoff[2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
            qoff[i] = (uint32_t)((wrow0 + i - lrow) * pm + a.qoff) + ((q4 + 2 * i) & 3) * QB + 2u * QB * s0;
        // step s of a pair uses load i_s = (q4 / 2 == s) ? 0 : 1; within its
        // step the block is half h = q4 % 2
        const int h = q4 & 1;
        const bool first_is_0 = (q4 >> 1) == 0;
        // scale load i covers rows wrow0 + i, blocks 4 q4 .. 4 q4 + 3 of a group
        // (64-blocks: blocks 2 q4, 2 q4 + 1, the group's 8 scales)
        constexpr uint32_t SLANE = SS ? 4 : 8;                  // scale bytes per lane and row
        // (scale bytes of a step: 4, or 2 with 64-blocks; s0 is a whole number of groups)
        const uint32_t s0b = (SS ? 2u : 4u) * s0;
        const uint32_t soff[2] = {(uint32_t)((wrow0 - lrow) * pm) + SLANE * q4 + s0b,
                                  (uint32_t)((wrow0 + 1 - lrow) * pm) + SLANE * q4 + s0b};
        uint16_t *wdst0 = lds + wrow0 * LDS_STRIDE + 32 * h;

        struct WPair { u32x4 q[2][WBlock<WT>::QV]; };
        WPair wr[W_PAIRS];
        uint32_t sreg[2][2], snext[2][2];   // [row wrow0 + i][dword] of a scale group

        auto load_w = [&](WPair &wp, int pair) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int v = 0; v < WBlock<WT>::QV; ++v)
                    wp.q[i][v] = __builtin_amdgcn_raw_buffer_load_b128(
                        wres, qoff[i] + (uint32_t)pair * (4 * QB) + 16 * v, 0, 0);
        };
        auto load_scales = [&](uint32_t (&dst)[2][2], int group) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                if constexpr (SS) {
                    dst[i][0] = __builtin_amdgcn_raw_buffer_load_b32(
                        wres, soff[i] + (uint32_t)group * SCALE_GROUP_BLOCKS, 0, 0);
                    dst[i][1] = 0;
                } else {
                    const auto v = __builtin_amdgcn_raw_buffer_load_b64(
                        wres, soff[i] + (uint32_t)group * (2 * SCALE_GROUP_BLOCKS), 0, 0);
                    dst[i][0] = v[0];
                    dst[i][1] = v[1];
                }
            }
        };
        auto produce = [&](auto S_, int p, const WPair &wp) {
            constexpr int S = decltype(S_)::value;   // p % SCALE_GROUP_STEPS
            const bool use0 = ((S & 1) == 0) == first_is_0;
            const int blk = 2 * p + h;
            WBlock<WT> b;
#pragma unroll
            for (int v = 0; v < WBlock<WT>::QV; ++v) b.q[v] = use0 ? wp.q[0][v] : wp.q[1][v];
            const uint16_t s16 = group_scale<S, SS>(sreg, use0, h);
            b.s = blk < nblk ? s16 : (uint16_t)0;   // past K: zero scale (the codes may be anything)
            uint32_t deq[16];
            dequant_block<WT>(b, deq);
            u32x4 *dst = reinterpret_cast<u32x4 *>(wdst0 + (p % STAGES) * STAGE_ELEMS + (use0 ? 0 : LDS_STRIDE));
#pragma unroll
            for (int v = 0; v < 4; ++v)
                dst[v] = u32x4{deq[4 * v], deq[4 * v + 1], deq[4 * v + 2], deq[4 * v + 3]};
        };

        // Loads are unconditional (those past the end read zeros or unused
        // bytes) so that the number in flight is the same on every path; the
        // scheduling fences keep the initial loads in slot order, which the
        // wait counts inside the loop rely on.
        load_scales(sreg, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < W_PAIRS; ++j) {
            load_w(wr[j], j);
            __builtin_amdgcn_sched_barrier(0);
        }
        // Step p: code pair slot (p / 2) % W_PAIRS, scale group p / SCALE_GROUP_STEPS
        // (loaded at its group's first step one group ahead).  Iteration p
        // writes step p and ends with barrier p - 1, before which only this
        // iteration's four LDS writes may still be in flight.
        for (int p0 = 0; p0 < steps; p0 += SCALE_GROUP_STEPS) {
            static_for<SCALE_GROUP_STEPS>([&](auto U) {
                constexpr int u = decltype(U)::value;
                const int p = p0 + u;
                if (u == 0) load_scales(snext, p / SCALE_GROUP_STEPS + 1);
                if (p < steps) produce(U, p, wr[(u / 2) % W_PAIRS]);
                if (u % 2 == 1) load_w(wr[(u / 2) % W_PAIRS], p / 2 + W_PAIRS);
                if (u == SCALE_GROUP_STEPS - 1) {
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        sreg[i][0] = snext[i][0];
                        sreg[i][1] = snext[i][1];
                    }
                }
                if (p >= 1 && p < steps) asm volatile("s_waitcnt lgkmcnt(4)\n\ts_barrier" ::: "memory");
            });
        }
        if (steps > 0) asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");   // barrier steps - 1
        if constexpr (SW) {          // the consumers' exchange of the two halves
            asm volatile("s_barrier" ::: "memory");
            asm volatile("s_barrier" ::: "memory");
        }
        return;
      }
    }

    // ---------------- consumers: tokens + matrix cores ----------------
    const int c = wave;
    const int wm = c & 1;        // weight-row half of the tile
    const int wn = c >> 1;       // token half of the tile

    // Token staging: wave c loads rows 32 c .. 32 c + 31 of the token tile,
    // 8 lanes per row (a step's 128 bytes), 8 rows per load.
    const int q8 = lane & 7;
    const int64_t toks = a.N - n0 < BN ? a.N - n0 : BN;
    const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(Xp + (uint64_t)n0 * x_pitch), 0,
        (int)(uint32_t)(((toks - 1) * x_pitch + a.K) * 2), BUFFER_FLAGS);
    const int xrow = 32 * c + (lane >> 3);
    const uint32_t xoff = (uint32_t)(xrow * x_pitch * 2) + 16 * q8 + 128u * s0;
    const uint32_t xrow_step = (uint32_t)(8 * x_pitch * 2);
    const int64_t xlim = a.K - 8 * q8 - 64 * (int64_t)s0;   // chunk q8 of step t is in K iff 64 t < xlim
    uint16_t *xdst0 = lds + OPERAND_ELEMS + xrow * LDS_STRIDE + 8 * q8;
    struct XStep { u32x4 v[4]; };
    XStep xr[X_DEPTH];
    auto load_x = [&](XStep &xs, int t) {
        const bool in_k = (int64_t)64 * t < xlim;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            xs.v[i] = __builtin_amdgcn_raw_buffer_load_b128(
                xres, in_k ? xoff + i * xrow_step + (uint32_t)t * 128 : OUT_OF_RANGE, 0, 0);
    };
    auto store_x = [&](const XStep &xs, int t) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<u32x4 *>(xdst0 + (t % STAGES) * STAGE_ELEMS + i * 8 * LDS_STRIDE) = xs.v[i];
    };

    // Fragments: lane (frow, fk) feeds MFMA row frow, k group fk of each
    // 16-deep k chunk.
    const int frow = lane & 31;
    const int fk = (lane >> 5) * 8;
    const int a_off = OPERAND_ELEMS + (wn * 64 + frow) * LDS_STRIDE + fk;   // tokens
    const int b_off = (wm * 64 + frow) * LDS_STRIDE + fk;                   // weights
    auto frag = [&](int stage, int off, int i, int kk) {
        return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(
            lds + stage * STAGE_ELEMS + off + i * 32 * LDS_STRIDE + kk * 16));
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // One set of fragment registers: each is refilled with the next step's
    // fragment right after the last matrix instruction that uses it, so reads
    // and matrix instructions alternate (a burst of reads would fill the LDS
    // command queue and stall the in-order issue of the matrix instructions
    // behind it) and every read has a whole step to land.
    bf16x8 fa[BK / 16][2], fb[BK / 16][2];
    auto read_all = [&](int stage) {
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk)
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                fa[kk][i] = frag(stage, a_off, i, kk);
                fb[kk][i] = frag(stage, b_off, i, kk);
            }
    };
    auto mma = [&](int kk, int i, int j) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[kk][i], fb[kk][j], acc[i][j], 0, 0, 0);
    };
    auto mma_and_read = [&](int stage) {
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            mma(kk, 0, 0);
            mma(kk, 0, 1);
            fa[kk][0] = frag(stage, a_off, 0, kk);
            mma(kk, 1, 0);
            fb[kk][0] = frag(stage, b_off, 0, kk);
            mma(kk, 1, 1);
            fa[kk][1] = frag(stage, a_off, 1, kk);
            fb[kk][1] = frag(stage, b_off, 1, kk);
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // two matrix instructions
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
    };
    auto mma_all = [&]() {
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk)
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) mma(kk, i, j);
    };

    // Tokens of step s are stored in window s-2 from ring slot s % X_DEPTH,
    // which is then refilled with step s + X_DEPTH; steps 0 and 1 are stored
    // before barrier 0.  (The scheduling fences keep the initial loads in
    // slot order.)
#pragma unroll
    for (int j = 0; j < X_DEPTH; ++j) {
        load_x(xr[j], j);
        __builtin_amdgcn_sched_barrier(0);
    }
    // (unconditional, like the loop's loads, so that the wait counts at the
    // loop head see one history; with no steps nothing reads the stages)
    store_x(xr[0], 0);
    load_x(xr[0], X_DEPTH);
    store_x(xr[1], 1);
    load_x(xr[1], X_DEPTH + 1);
    if (steps > 0) asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");   // barrier 0
    store_x(xr[2], 2);
    load_x(xr[2], X_DEPTH + 2);
    read_all(0);
    // Window t >= 1: store the tokens of step t+2, read step t, multiply step
    // t-1.  Before barrier t the stores of window t-2 (tokens of step t) must
    // have landed; the twenty LDS operations of window t-1 may not.
    for (int t0 = 1; t0 < steps; t0 += X_DEPTH) {
        static_for<X_DEPTH>([&](auto U) {
            constexpr int u = decltype(U)::value;
            const int t = t0 + u;                 // t0 % X_DEPTH == 1
            if (t < steps) {
                asm volatile("s_waitcnt lgkmcnt(15)\n\ts_barrier" ::: "memory");
                store_x(xr[(u + 3) % X_DEPTH], t + 2);
                load_x(xr[(u + 3) % X_DEPTH], t + 2 + X_DEPTH);
                mma_and_read((u + 1) % STAGES);
            }
        });
    }
    if (steps > 0) mma_all();

    // Epilogue: acc[i][j] register r holds token 8*(r/4) + 4*(lane/32) + r%4
    // of sub-tile i and weight row lane%32 of sub-tile j.
    if constexpr (SW) {
        // The gate-half (wm = 0) and up-half (wm = 1) consumers of the same
        // tokens (same wn) each finish one token sub-tile: wm = 0 sub-tile
        // 0, wm = 1 sub-tile 1.  Each hands the other the sums it needs
        // through LDS, which no stage uses any more.
        float *xa = reinterpret_cast<float *>(lds) + wn * (2 * 2 * 16 * 64);   // up sums of sub-tile 0
        float *xb = xa + 2 * 16 * 64;                                          // gate sums of sub-tile 1
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");   // every stage read
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                if (wm == 1) xa[(j * 16 + r) * 64 + lane] = acc[0][j][r];
                else xb[(j * 16 + r) * 64 + lane] = acc[1][j][r];
            }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        auto finish = [&](auto I_) {
            constexpr int i = decltype(I_)::value;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int64_t m = m0 + j * 32 + (lane & 31);
                if (m >= M) continue;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t n = n0 + wn * 64 + i * 32 + 8 * (r / 4) + 4 * (lane >> 5) + (r % 4);
                    const float g = i == 0 ? acc[0][j][r] : xb[(j * 16 + r) * 64 + lane];
                    const float u = i == 0 ? xa[(j * 16 + r) * 64 + lane] : acc[1][j][r];
                    if (n < a.N) __builtin_nontemporal_store(swish(g) * u, out + (uint64_t)n * y_pitch + m);
                }
            }
        };
        if (wm == 0) finish(std::integral_constant<int, 0>{});
        else finish(std::integral_constant<int, 1>{});
        return;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t m = m0 + wm * 64 + j * 32 + (lane & 31);
            if (m >= M) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t n = n0 + wn * 64 + i * 32 + 8 * (r / 4) + 4 * (lane >> 5) + (r % 4);
                if (n < a.N) __builtin_nontemporal_store(acc[i][j][r], out + (uint64_t)n * y_pitch + m);   // streaming store: skips filling the L2
            }
        }
    }
}

constexpr size_t LDS_BYTES = (size_t)STAGES * STAGE_ELEMS * sizeof(uint16_t);

template <int WT, int SS, bool SW = false>
hipError_t launch_typed(const GemmArgs &a, unsigned blocks, hipStream_t stream)
{
    const hipError_t attr = allow_dynamic_lds(reinterpret_cast<const void *>(&gemm_kernel<WT, SS, SW>), (int)LDS_BYTES);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((gemm_kernel<WT, SS, SW>), dim3(blocks), dim3(THREADS), LDS_BYTES, stream, a);
    return hipGetLastError();
}

// y[n][m] = sum over s = 0, 1, .., S-1 in that order of slab s's [n][m]:
// the K ranges' partial sums added in a fixed order, so the result does not
// depend on which workgroup finished first.  Slab rows are Mp floats (M
// rounded up to 4), so each thread moves four outputs with 16-byte loads;
// vec_y says whether y's rows allow 16-byte stores too.
__global__ __launch_bounds__(256) void split_sum_kernel(const float *ws, uint64_t slab, int S, int64_t Mp,
                                                        float *y, uint64_t y_pitch, int64_t M, int64_t N,
                                                        int vec_y)
{
    const int64_t quads = Mp / 4;
    const int64_t total = N * quads;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
        const int64_t n = i / quads;
        const int64_t m = (i - n * quads) * 4;
        const float *src = ws + (uint64_t)n * Mp + m;
        float4 acc = *reinterpret_cast<const float4 *>(src);
        for (int s = 1; s < S; ++s) {
            const float4 v = *reinterpret_cast<const float4 *>(src + (uint64_t)s * slab);
            acc.x += v.x;
            acc.y += v.y;
            acc.z += v.z;
            acc.w += v.w;
        }
        float *dst = y + (uint64_t)n * y_pitch + m;
        if (vec_y && m + 4 <= M) {
            *reinterpret_cast<float4 *>(dst) = acc;
        } else {
            if (m < M) dst[0] = acc.x;
            if (m + 1 < M) dst[1] = acc.y;
            if (m + 2 < M) dst[2] = acc.z;
            if (m + 3 < M) dst[3] = acc.w;
        }
    }
}


constexpr int kMinSplitSteps = SCALE_GROUP_STEPS;   // K-steps of the shortest range (512 of K)

}  // namespace

// Compute units of the current device (queried once per device).
int device_cus()
{
    static std::atomic<int> cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
    if (dev < 64) {
        const int c = cus[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    if (dev < 64) cus[dev].store(n, std::memory_order_relaxed);
    return n;
}

GemmPlan gemm_plan(int64_t M, int64_t K, int64_t N, uint64_t ws_bytes)
{
    GemmPlan p;
    const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    const int64_t steps = (K + BK - 1) / BK;
    p.mp = (M + 3) / 4 * 4;
    p.splits = 1;
    p.split_steps = (int)steps;
    p.ws_bytes = 0;
    if (M <= 0 || N <= 0 || steps <= 0) return p;
    // Estimated time (us) of a launch: a fixed part, the K-steps of one range
    // at a per-step cost that grows with the workgroups running at once, and
    // for a split the second launch plus the partial sums written and read
    // back (fitted to timings of this kernel on MI355X over M = 256..5632,
    // K = 2048..5632, N = 128..512; e.g. 2048 x 5632 x 512: 44.8 us whole,
    // 26.7 us in four ranges, while 2048 x 2048 x 512 is fastest whole).
    const int64_t cus = device_cus();
    auto cost = [&](int64_t ranges, int64_t len) {
        const double wgs = (double)(tiles * ranges);
        const double step_us = 0.29 + 0.2 * wgs / 256.0;
        double t = 10.0 + (double)len * step_us;
        if (ranges > 1) t += 2.5 + 0.35e-6 * (double)ranges * (double)N * (double)p.mp * sizeof(float);
        return t;
    };
    double best = cost(1, steps);
    // Ranges are multiples of SCALE_GROUP_STEPS, at least kMinSplitSteps long,
    // and one round of workgroups must still fit the chip.
    for (int64_t s = 2; tiles * s <= cus && steps >= s * kMinSplitSteps; s *= 2) {
        int64_t len = (steps + s - 1) / s;
        len = (len + SCALE_GROUP_STEPS - 1) / SCALE_GROUP_STEPS * SCALE_GROUP_STEPS;
        const int64_t used = (steps + len - 1) / len;
        const uint64_t bytes = (uint64_t)used * (uint64_t)N * (uint64_t)p.mp * sizeof(float);
        if (used < 2 || bytes > ws_bytes) continue;
        const double t = cost(used, len);
        if (t < best) {
            best = t;
            p.splits = (int)used;
            p.split_steps = (int)len;
            p.ws_bytes = bytes;
        }
    }
    return p;
}

bool gemm_supported(const WeightView &w, const ActView &x)
{
    // buffer offsets within one tile are 32-bit
    return (uint64_t)BM * w.pitch < (1ull << 31) && (uint64_t)BN * x.pitch_elems * 2 < (1ull << 31);
}

namespace {

// Launch the GEMM over `count` items (same type, K and N) with `plan`'s K
// split, then the slab sum when K is split (one item only).
hipError_t launch_items(const WeightView *w, const ActView *x, const OutView *y, int count,
                        const GemmPlan &plan, float *ws, hipStream_t stream)
{
    GemmArgs a;
    a.K = w[0].K;
    a.qoff = quant_offset(w[0].K, w[0].scale_shift);
    a.N = x[0].N;
    a.n_tiles = (int)((x[0].N + BN - 1) / BN);
    a.n_splits = plan.splits;
    a.split_steps = plan.split_steps;
    a.n_items = count;
    a.split_stride = plan.splits > 1 ? (uint64_t)x[0].N * (uint64_t)plan.mp : 0;
    int tiles = 0;
    for (int i = 0; i < kMaxGemmItems; ++i) {
        GemmItem &it = a.item[i];
        const int k = i < count ? i : count - 1;      // unused slots repeat the last item
        it.w = w[k].base;
        it.pitch = w[k].pitch;
        it.M = w[k].M;
        it.x = static_cast<const uint16_t *>(x[k].data);
        it.x_pitch = x[k].pitch_elems;
        it.y = plan.splits > 1 ? ws : y[k].data;
        it.y_pitch = plan.splits > 1 ? (uint64_t)plan.mp : y[k].pitch_elems;
        it.w2 = w[k].base;
        it.pitch2 = w[k].pitch;
        it.tile_begin = i < count ? tiles : 0x7FFFFFFF;
        it.pad = 0;
        if (i < count) tiles += (int)((w[k].M + BM - 1) / BM) * a.n_tiles;
    }
    const unsigned blocks = (unsigned)tiles * (unsigned)plan.splits;
    if (blocks == 0) return hipSuccess;
    const WeightView &w0 = w[0];
    hipError_t e = hipErrorInvalidValue;
    // quantized weights: the register-dequantizing kernel (gemm_rq.hip);
    // F16 weights: this file's kernel
    if (gemm_rq_handles(w0.type)) e = launch_gemm_rq(a, blocks, w0.type, w0.scale_shift, false, stream);
    else if (w0.type == W_F16 && !w0.scale_shift) e = launch_typed<W_F16, 0>(a, blocks, stream);
    if (e != hipSuccess || plan.splits == 1) return e;
    const int64_t quads = x[0].N * (plan.mp / 4);
    const int64_t want = (quads + 255) / 256;
    const unsigned grid = (unsigned)(want < 4096 ? want : 4096);
    const int vec_y = ((uintptr_t)y[0].data % 16 == 0 && y[0].pitch_elems % 4 == 0) ? 1 : 0;
    hipLaunchKernelGGL(split_sum_kernel, dim3(grid), dim3(256), 0, stream, (const float *)ws,
                       (uint64_t)a.split_stride, plan.splits, plan.mp, y[0].data, y[0].pitch_elems, w0.M,
                       x[0].N, vec_y);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const WeightView &w, const ActView &x, const OutView &y,
                       float *ws, uint64_t ws_bytes, hipStream_t stream)
{
    if (w.M == 0 || x.N == 0) return hipSuccess;
    const GemmPlan plan = gemm_plan(w.M, w.K, x.N, ws ? ws_bytes : 0);
    return launch_items(&w, &x, &y, 1, plan, ws, stream);
}

hipError_t launch_gemm_swiglu(const WeightView &wg, const WeightView &wu, const ActView &x, const OutView &h,
                              hipStream_t stream)
{
    if (wg.M == 0 || x.N == 0) return hipSuccess;
    GemmArgs a;
    a.K = wg.K;
    a.qoff = quant_offset(wg.K, wg.scale_shift);
    a.N = x.N;
    a.n_tiles = (int)((x.N + BN - 1) / BN);
    a.n_splits = 1;
    a.split_steps = (int)((wg.K + BK - 1) / BK);
    a.n_items = 1;
    a.split_stride = 0;
    for (int i = 0; i < kMaxGemmItems; ++i) {
        GemmItem &it = a.item[i];
        it.w = wg.base;
        it.pitch = wg.pitch;
        it.w2 = wu.base;
        it.pitch2 = wu.pitch;
        it.M = wg.M;
        it.x = static_cast<const uint16_t *>(x.data);
        it.x_pitch = x.pitch_elems;
        it.y = h.data;
        it.y_pitch = h.pitch_elems;
        it.tile_begin = i == 0 ? 0 : 0x7FFFFFFF;
        it.pad = 0;
    }
    const unsigned blocks = (unsigned)((wg.M + BM / 2 - 1) / (BM / 2)) * (unsigned)a.n_tiles;
    if (gemm_rq_handles(wg.type)) return launch_gemm_rq(a, blocks, wg.type, wg.scale_shift, true, stream);
    if (wg.scale_shift) {
        if (wg.type == W_Q4_0) return launch_typed<W_Q4_0, 1, true>(a, blocks, stream);
        if (wg.type == W_Q8_0) return launch_typed<W_Q8_0, 1, true>(a, blocks, stream);
        return hipErrorInvalidValue;
    }
    if (wg.type == W_Q4_0) return launch_typed<W_Q4_0, 0, true>(a, blocks, stream);
    if (wg.type == W_Q8_0) return launch_typed<W_Q8_0, 0, true>(a, blocks, stream);
    if (wg.type == W_F16) return launch_typed<W_F16, 0, true>(a, blocks, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_gemm_batch(const WeightView *w, const ActView *x, const OutView *y, int count,
                             hipStream_t stream)
{
    if (count < 1 || count > kMaxGemmItems) return hipErrorInvalidValue;
    if (x[0].N == 0) return hipSuccess;
    GemmPlan plan;
    plan.splits = 1;
    plan.split_steps = (int)((w[0].K + BK - 1) / BK);
    plan.mp = 0;
    plan.ws_bytes = 0;
    return launch_items(w, x, y, count, plan, nullptr, stream);
}

// Raise a kernel's dynamic-LDS limit once (the attribute persists for the
// process); later launches, including those recorded into graphs, reuse it.
hipError_t allow_dynamic_lds(const void *fn, int bytes)
{
    static std::mutex mu;
    static const void *fns[64];
    static int granted[64];
    static int n = 0;
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < n; ++i)
        if (fns[i] == fn && granted[i] >= bytes) return hipSuccess;
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
    for (int i = 0; i < n; ++i)
        if (fns[i] == fn) { granted[i] = bytes; return hipSuccess; }
    if (n < 64) { fns[n] = fn; granted[n] = bytes; ++n; }
    return hipSuccess;
}

}  // namespace qmm

// ---- scratch memory for callers that cannot allocate ----------------------
//
// The split-K partial sums of qmm_gemm_noalloc live in this array instead of
// a caller workspace.  Every device the library runs on holds its own copy
// until the process ends.  In host code the name is only a stand-in: the
// device address comes from hipGetSymbolAddress, once per device, with that
// device current, and only that address is handed to kernels.
namespace qmm {
namespace {
static __device__ __align__(256) uint8_t scratch[QMM_NOALLOC_SCRATCH_BYTES];
}  // namespace

hipError_t static_scratch(void **ptr)
{
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *addr[kMaxDevices];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

}  // namespace qmm
