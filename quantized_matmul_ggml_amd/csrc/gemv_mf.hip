// gemv_mf.hip -- decode GEMV / skinny GEMM for Q4_0 and Q8_0 weights and up
// to 8 tokens on the bf16 matrix cores: fp32 activations, Q8_0 activations
// (with Q8_0 weights), and the gate/up pair fused with SwiGLU; F16 weights
// with fp32 activations.
//
// Same operation as gemv.hip (y[n][m] = sum_k W'[m][k] x[n][k]), with the
// multiply-adds moved to v_mfma_f32_16x16x32_bf16 (D 16 x 16 += A 16 x 32 *
// B 32 x 16), so that the vector ALUs only unpack codes and apply block scales
// and the cost per weight does not grow with the token count (Development
// Guide for Small AI Models (TinyLLaMA, etc.) Using C++, §6.2: unpack, scale,
// multiply-add; A Complete Guide to llama.cpp and Customization with C++,
// §2.2: the scale factors out of each block's dot product).
//
//  * A (16 x 32): channel i = 2 n + h is token n, h = 0 the bf16 high part of
//    the activations and h = 1 the bf16 low part (x = hi + lo to 2^-17
//    relative, so the products keep the fp32 GEMV's accuracy).  A wave owns
//    a fixed range of NBW blocks of K and keeps their fragments in registers
//    for every row tile it streams: no LDS traffic per matrix instruction.
//  * B (32 x 16): column j is weight row j of a 16-row tile.  Each lane loads
//    16 contiguous bytes of its row (Q4_0: one block of the four a group of
//    lanes covers; Q8_0: half a block of two), 64 bytes per row per
//    instruction, and two cross-lane swaps (v_permlane32_swap, then
//    v_permlane16_swap for Q4_0) regroup them so that the four lane groups of
//    one matrix instruction hold four disjoint 8-code sets of the SAME block.
//    Codes enter as exact signed bf16 integers, so each product is the
//    dequantized code times the activation part and no large biased sum
//    ever has to cancel: Q8_0 bytes are sign-extended and converted; a Q4_0
//    nibble n is moved to the top of a byte with its top bit flipped, which
//    reads as the int8 value 16 (n - 8), and the block scale absorbs the 16.
//  * F16 rows: a lane loads 8 halves of its row, in matrix order.  Each half
//    splits exactly into two bf16 values (the half rounded to bf16, and the
//    remainder, at most 2 significant bits), which go through two matrix
//    instructions into one accumulator: there is no scale.
//  * D (16 x 16): lane (row j, group g) gets channels 4 g .. 4 g + 3, i.e.
//    tokens 2 g and 2 g + 1, of its row for one block, and applies the block
//    scale in one fused multiply-add per token.
//  * The KW waves of a workgroup split K; their partial sums meet in LDS at
//    the end of each tile.  A tile is TR = 16 weight rows, or 8 (columns
//    8..15 then repeat rows 0..7 and are not stored) where 16-row stages
//    would not fit the LDS; the fused SwiGLU tile is 8 gate rows and the 8
//    up rows of the same indices.
//  * Q8_0 activations (XQ) and the SwiGLU epilogue (SW) are described at the
//    kernel.
#include "qmm_internal.h"
#include "wave_reduce.h"

namespace qmm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kTileRows = 16;
constexpr int kMaxMfItems = QMM_GEMV_BATCH_MAX;

template <int WT> struct MfFmt;
// code_scale: the factor between the value a code enters the matrix
// instruction with and its signed code (Q4_0 codes enter as 16 (n - 8)).
// scaled: fp16 block scales follow the codes' section (F16 rows have none).
template <> struct MfFmt<W_Q4_0> { static constexpr int bpg = 4, block_bytes = 16; static constexpr float code_scale = 0.0625f; static constexpr bool scaled = true; };
template <> struct MfFmt<W_Q8_0> { static constexpr int bpg = 2, block_bytes = 32; static constexpr float code_scale = 1.0f; static constexpr bool scaled = true; };
template <> struct MfFmt<W_F16>  { static constexpr int bpg = 1, block_bytes = 64; static constexpr float code_scale = 1.0f; static constexpr bool scaled = false; };

struct alignas(64) MfItem {
    const uint8_t *w;
    const void *x;        // fp32 rows, or Q8_0 rows (whole rows, whatever the pass)
    float *y;
    uint32_t pitch;       // bytes between weight rows
    uint32_t x_pitch;     // between token rows of x: elements (fp32) or bytes (Q8_0)
    uint32_t y_pitch;     // elements between token rows of y
    int32_t M;
    int32_t n_tiles;      // 16-row tiles
    int32_t wg_count;     // workgroups of this item (grid x; grid y indexes the item)
    int32_t pad[2];
};
static_assert(sizeof(MfItem) == 64, "one 64-byte record per item");

struct MfArgs {
    int32_t N;            // tokens of this launch (<= 8)
    int32_t K;            // K of this pass (32 nb); fp32 x points at its first element
    int32_t qoff;         // byte offset of the codes in a row
    int32_t nb;           // 32-blocks of this pass (<= 128; <= 192 in the wide launch)
    int32_t n_items;
    int32_t kb0;          // first block of this pass within the row
    int32_t nb_row;       // 32-blocks per row
    int32_t accumulate;   // add to y (a later pass over K) instead of storing
    int32_t xqoff;        // Q8_0 activations: byte offset of the codes in an x row
    uint32_t pitch2;      // fused SwiGLU: bytes between the up matrix's rows
    const uint8_t *w2;    // fused SwiGLU: the up matrix (item 0's w is the gate)
    int32_t pad[4];
    MfItem item[kMaxMfItems];
};
static_assert(offsetof(MfArgs, item) == 64, "the shared fields fill the first 64 bytes");

// Round two floats to bf16 (nearest even) in one v_cvt_pk_bf16_f32.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ inline uint32_t pack_bf16(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}
__device__ inline float bf16_lo(uint32_t p) { return __builtin_bit_cast(float, p << 16); }
__device__ inline float bf16_hi(uint32_t p) { return __builtin_bit_cast(float, p & 0xFFFF0000u); }

// Byte E of w as a signed int8, converted to float (one SDWA conversion).
template <int E>
__device__ inline float sbyte(uint32_t w)
{
    return (float)(int8_t)(w >> (8 * E));
}

// The k positions (within a block) of the 8 values lane group g feeds to
// one matrix instruction, in register order; A and B use the same list.
//  Q4_0: group g holds dword g of the block (bytes 4g..4g+3; byte s has
//        element 4g+s in its low nibble and 16+4g+s in its high nibble),
//        unpacked as lo(s0) lo(s2) hi(s0) hi(s2) lo(s1) lo(s3) hi(s1) hi(s3).
//  Q8_0: group g holds codes k0(g) .. k0(g)+7 with k0 = 0, 16, 8, 24.
//  F16:  group g holds halves 8g .. 8g+7.

// Swap helpers: [0] is the new first operand, [1] the new second.
__device__ inline void swap32(uint32_t &a, uint32_t &b)
{
    const auto p = __builtin_amdgcn_permlane32_swap(a, b, false, false);
    a = p[0];
    b = p[1];
}
__device__ inline void swap16(uint32_t &a, uint32_t &b)
{
    const auto p = __builtin_amdgcn_permlane16_swap(a, b, false, false);
    a = p[0];
    b = p[1];
}

// A wave's share of one TR-row tile in LDS: the code bytes of its NBW
// blocks of each row (SB = 16 U bytes, U 16-byte units) and their scales
// (SR bytes), as the direct-to-LDS loads deliver them: one load instruction
// moves 64 lanes x 16 contiguous bytes of RPI whole rows; the scales come
// with 4-byte lanes (one fp16 scale per 32 weights, or per 64 with SS = 1).
template <int WT, int NBW, int SS, int TR>
struct MfStage {
    static constexpr int SB = NBW * MfFmt<WT>::block_bytes;
    static constexpr int U = SB / 16;
    static constexpr int RPI = 64 / U;
    static constexpr int NI = TR / RPI;                        // code load instructions
    static constexpr int SR = MfFmt<WT>::scaled ? (2 * NBW) >> SS : 0;
    static constexpr int NS = (TR * SR + 255) / 256;           // scale load instructions
    static constexpr int CODE_BYTES = NI * 1024;
    static constexpr int BYTES = CODE_BYTES + NS * 256;
    static_assert(U >= 4 && U <= 64, "2..16 rows per load instruction");
    static_assert(TR == 8 || TR == 16, "8 or 16 rows per tile");
    static_assert(RPI <= TR, "whole load instructions per tile");
};

// Position (16-byte unit) of unit u of row r inside its row's LDS span: the
// units of 8 rows that lanes read together land in 8 different 128-byte bank
// windows (rows of 128 bytes or more start in the same window; rows of 64
// bytes alternate halves).
template <int U>
__device__ inline int swz(int r, int u)
{
    if constexpr (U >= 8) return u ^ (r & 7);
    else return u ^ ((r >> 1) & 3);
}

// Direct-to-LDS buffer loads, issued as instructions the compiler does not
// see (so it neither reorders LDS reads around them nor adds waits of its
// own); the consumer waits with an explicit vmcnt.  Lane i of one load writes
// its SIZE bytes at lds + SIZE * i.  rsrc is the 4-word buffer resource.
// They keep the default cache policy: with the non-temporal one of the
// other GEMVs (kStreamLoad) this kernel was 5-7 % slower on the LM head at
// 4 and 8 tokens.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ inline i32x4 buffer_words(const void *base, uint32_t bytes)
{
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    return i32x4{(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xFFFFu), (int)bytes, BUFFER_FLAGS};
}
// m0 is the loads' LDS base; no other code in this file uses it.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <int SIZE>
__device__ inline void load_to_lds(const i32x4 &rsrc, uint32_t lds, uint32_t voff)
{
    static_assert(SIZE == 4 || SIZE == 16, "dword or dwordx4");
    if constexpr (SIZE == 16)
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                     :: "s"(lds), "v"(voff), "s"(rsrc) : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                     :: "s"(lds), "v"(voff), "s"(rsrc) : "memory", "m0");
}
#pragma clang diagnostic pop
// Wait until at most N vector memory operations of this wave are pending.
template <int N>
__device__ inline void wait_vm()
{
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// LDS of a workgroup with KW waves and NSTG stages, and the most stages (up
// to MAXD, at least 2) that fit the CU's 160 KiB.
constexpr int kLdsBytes = 160 * 1024;
template <int WT, int KW, int NBW, int SS, int TR, bool SW = false>
constexpr int mf_lds_bytes(int nstg)
{
    return nstg * KW * (SW ? 2 : 1) * MfStage<WT, NBW, SS, TR>::BYTES + 2 * KW * 64 * 2 * 4;
}
template <int WT, int KW, int NBW, int SS, int MAXD, int TR, bool SW = false>
constexpr int mf_stages()
{
    int d = MAXD;
    while (d > 2 && mf_lds_bytes<WT, KW, NBW, SS, TR, SW>(d) > kLdsBytes) --d;
    return d;
}

// Swish(z) = z * sigma(z) = z / (1 + e^{-z}) in binary32; for z far below
// zero e^{-z} overflows and the quotient is the limit -0.
__device__ inline float swish(float z)
{
    return z / (1.0f + expf(-z));
}

// XQ: the activations are Q8_0 rows (A Complete Guide to llama.cpp and
// Customization with C++, §2.2: with x quantized per block, a block's dot
// product is Delta * Delta_x * sum_i q_i qx_i), for Q8_0 weights.  Channel
// 2n then carries token n's int8 codes, exact in bf16, and channel 2n + 1
// zeros; the matrix instruction's sum over one block is the exact integer
// sum_i q_i qx_i (|sum| < 2^19), and each block term is one fused
// multiply-add of the exact product Delta * Delta_x (two 11-bit
// significands) with it.  (Q4_0 weights with Q8_0 activations stay on the
// int8 dot-product kernel, measured faster: their 8 codes per lane and block
// come in two 4-byte runs, two load instructions per block.)
//
// SW: the gate/up pair fused with the SwiGLU epilogue (Development Guide for
// Small AI Models (TinyLLaMA, etc.) Using C++, §4.4: h = Swish(x Wg) * (x Wu)).
// A tile is 8 row indices of both matrices: matrix columns 0..7 are gate
// rows, 8..15 the up rows of the same indices, each half staged like an
// 8-row tile.  After the cross-wave sum, lanes j and j + 8 hold the two sums
// of one output, one DPP rotation apart, and only h is stored.  One pass
// over K (h is not linear in partial sums).
template <int WT, int KW, int NBW, int SS, int MAXD, int TR, bool XQ, bool SW>
__global__ __launch_bounds__(64 * KW) void gemv_mf_kernel(const MfArgs a)
{
    constexpr int NSTG = mf_stages<WT, KW, NBW, SS, MAXD, TR, SW>();
    static_assert(mf_lds_bytes<WT, KW, NBW, SS, TR, SW>(NSTG) <= kLdsBytes, "LDS of one workgroup");
    static_assert(!SW || (TR == 8 && !XQ), "SwiGLU tiles are 8 gate + 8 up rows");
    constexpr int SWF = SW ? 2 : 1;        // matrices staged per tile
    constexpr int BPG = MfFmt<WT>::bpg;
    constexpr int BB = MfFmt<WT>::block_bytes;
    constexpr int NG = NBW / BPG;          // 64-byte groups per row per wave
    static_assert(NBW % BPG == 0, "whole load groups");
    using St = MfStage<WT, NBW, SS, TR>;
    static_assert(NSTG >= 2 && NSTG <= 4, "2 to 4 stages");
    static_assert(!XQ || WT == W_Q8_0, "Q8_0 activations with Q8_0 weights");
    __shared__ float red[2][KW][64][2];
    // one array per stage, so that each wait for a stage's loads counts only
    // the loads issued before them
    __shared__ __attribute__((aligned(16))) uint8_t st0[KW][SWF * St::BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t st1[KW][SWF * St::BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t st2[KW][NSTG > 2 ? SWF * St::BYTES : 16];
    __shared__ __attribute__((aligned(16))) uint8_t st3[KW][NSTG > 3 ? SWF * St::BYTES : 16];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 15;               // A channel / B and D column (weight row)
    const int g = lane >> 4;               // k group / D channel group

    const int item = blockIdx.y;
    const MfItem &itm = a.item[item];
    const uint8_t *const W = itm.w;
    const void *const X = itm.x;
    float *const Y = itm.y;
    const uint32_t pitch = itm.pitch, x_pitch = itm.x_pitch, y_pitch = itm.y_pitch;
    const int M = itm.M, n_tiles = itm.n_tiles, n_wg = itm.wg_count;
    const int N = a.N, K = a.K, qoff = a.qoff, nb = a.nb, kb0 = a.kb0, nb_row = a.nb_row, acc = a.accumulate;
    const int xqoff = a.xqoff;
    const uint8_t *const W2 = a.w2;
    const uint32_t pitch2 = a.pitch2;
    asm volatile("" ::"s"(W), "s"(X), "s"(Y), "s"(pitch), "s"(x_pitch), "s"(y_pitch), "s"(M),
                 "s"(n_tiles), "s"(n_wg), "s"(N), "s"(K), "s"(qoff), "s"(nb), "s"(kb0), "s"(nb_row), "s"(acc),
                 "s"(xqoff), "s"(W2), "s"(pitch2));
    if ((int)blockIdx.x >= n_wg) return;
    const int b_begin = wave * NBW;

    // ---- a tile's share of this wave into one stage: rows past M, and
    // units and scales of blocks past the row, read as zeros ----
    const uint32_t row_bytes = (uint32_t)(qoff + nb_row * BB);
    auto issue_mat = [&](uint32_t base, const uint8_t *Wm, uint32_t pm, int tl) {
        const uint32_t pitch = pm;
        const int r0 = tl * TR;
        const int rows = tl < n_tiles ? (M - r0 < TR ? M - r0 : TR) : 0;
        const i32x4 wres = buffer_words(Wm + (uint64_t)(rows > 0 ? r0 : 0) * pitch,
                                        rows > 0 ? (uint32_t)(rows - 1) * pitch + row_bytes : 0u);
#pragma unroll
        for (int i = 0; i < St::NI; ++i) {
            const int r = i * St::RPI + lane / St::U;
            const int u = swz<St::U>(r, lane % St::U);
            const int blk = b_begin + (16 * u) / BB;
            const uint32_t off = blk < nb ? (uint32_t)r * pitch + (uint32_t)(qoff + BB * (kb0 + b_begin) + 16 * u)
                                          : OUT_OF_RANGE;
            load_to_lds<16>(wres, base + 1024 * i, off);
        }
        if constexpr (St::NS > 0) {
#pragma unroll
        for (int i = 0; i < St::NS; ++i) {
            const int byte = 256 * i + 4 * lane;
            const int r = byte / St::SR, rb = byte % St::SR;
            // scale rb / 2 of the wave's slice is that of 32-block
            // b_begin + (rb / 2 << SS) (kb0 and b_begin are even)
            const uint32_t off = (r < TR && (b_begin >> SS) + rb / 2 < (nb >> SS))
                                     ? (uint32_t)r * pitch + (uint32_t)(2 * ((kb0 + b_begin) >> SS) + rb)
                                     : OUT_OF_RANGE;
            load_to_lds<4>(wres, base + St::CODE_BYTES + 256 * i, off);
        }
        }
    };
    auto issue = [&](auto &stg, int tl) {
        const uint32_t base = (uint32_t)reinterpret_cast<uintptr_t>(&stg[wave][0]);
        issue_mat(base, W, pitch, tl);
        if constexpr (SW) issue_mat(base + St::BYTES, W2, pitch2, tl);
    };

    // the first NSTG-1 tiles are in flight while the activations are set up
    int tile = blockIdx.x;
    issue(st0, tile);
    if constexpr (NSTG > 2) issue(st1, tile + n_wg);
    if constexpr (NSTG > 3) issue(st2, tile + 2 * n_wg);
    __builtin_amdgcn_sched_barrier(0);

    // ---- activation fragments of this wave's blocks; channel j = token
    // j / 2, part j % 2; blocks past the row and tokens past N read zeros ----
    const int tok = j >> 1;
    const bool lo_part = (j & 1) != 0;
    bf16x8 xf[NBW];
    // XQ: the block scales Delta_x of the two tokens whose sums this lane
    // receives (2g and 2g + 1), one fp16 per block, two per dword
    uint32_t dxs[2][XQ ? NBW / 2 : 1];
    if constexpr (!XQ) {
        const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<void *>(X), 0, (int)(((uint32_t)(N - 1) * x_pitch + (uint32_t)K) * 4u), BUFFER_FLAGS);
        const uint32_t xrow = (uint32_t)tok * x_pitch * 4u;
        // The 8 k positions of group g come in two runs of 4 (Q4_0: 4g.. and
        // 16+4g..; Q8_0: k0.. and k0+4..; F16: 8g.. and 8g+4..).  Lanes 2t and 2t+1 (token t, high and
        // low part) need the same 8 values: each loads one run (the even lane
        // run 0), converts it to both parts, and the pair trades the part the
        // other lane feeds with one DPP swap.  That halves the load instructions:
        // a CU's vector-memory path returns about 1 KB per 25 cycles, and with
        // 8 tokens and one tile per workgroup the activations are most of a
        // workgroup's bytes.  All loads first, then the conversions: one round
        // trip, not NBW.
        uint32_t raw[NBW][4];
    #pragma unroll
        for (int t = 0; t < NBW; ++t) {
            const int b = b_begin + t;
            const uint32_t base = (uint32_t)(32 * b) * 4;
            uint32_t o0, o1;
            if constexpr (WT == W_Q4_0) { o0 = base + 16 * g; o1 = base + 64 + 16 * g; }
            else if constexpr (WT == W_F16) { o0 = base + 32 * g; o1 = o0 + 16; }
            else { const int k0 = (g == 0) ? 0 : (g == 1) ? 16 : (g == 2) ? 8 : 24; o0 = base + 4 * k0; o1 = o0 + 16; }
            const bool in = b < nb && tok < N;
            const auto p = __builtin_amdgcn_raw_buffer_load_b128(xres, in ? xrow + (lo_part ? o1 : o0) : OUT_OF_RANGE, 0, 0);
    #pragma unroll
            for (int e = 0; e < 4; ++e) raw[t][e] = p[e];
        }
        __builtin_amdgcn_sched_barrier(0);
    #pragma unroll
        for (int t = 0; t < NBW; ++t) {
            float r[4];
    #pragma unroll
            for (int e = 0; e < 4; ++e) r[e] = __builtin_bit_cast(float, raw[t][e]);
            // the run's two register pairs (Q4_0: elements 0, 2 and 1, 3 of the
            // run, for lo(s0) lo(s2) | hi(s0) hi(s2) ...; Q8_0 and F16: 0, 1
            // and 2, 3)
            float a0, a1, b0, b1;
            if constexpr (WT == W_Q4_0) { a0 = r[0]; a1 = r[2]; b0 = r[1]; b1 = r[3]; }
            else { a0 = r[0]; a1 = r[1]; b0 = r[2]; b1 = r[3]; }
            const uint32_t hiA = pack_bf16(a0, a1), loA = pack_bf16(a0 - bf16_lo(hiA), a1 - bf16_hi(hiA));
            const uint32_t hiB = pack_bf16(b0, b1), loB = pack_bf16(b0 - bf16_lo(hiB), b1 - bf16_hi(hiB));
            const uint32_t keepA = lo_part ? loA : hiA, keepB = lo_part ? loB : hiB;
            const uint32_t sendA = lo_part ? hiA : loA, sendB = lo_part ? hiB : loB;
            // quad_perm [1, 0, 3, 2]: swap with the neighbouring lane
            const uint32_t recvA = (uint32_t)__builtin_amdgcn_mov_dpp((int)sendA, 0xB1, 0xF, 0xF, true);
            const uint32_t recvB = (uint32_t)__builtin_amdgcn_mov_dpp((int)sendB, 0xB1, 0xF, 0xF, true);
            // register order: Q4_0 A(run 0) A(run 1) B(run 0) B(run 1);
            // Q8_0 and F16 A(run 0) B(run 0) A(run 1) B(run 1)
            uint32_t w4[4];
            if constexpr (WT == W_Q4_0) {
                w4[0] = lo_part ? recvA : keepA; w4[1] = lo_part ? keepA : recvA;
                w4[2] = lo_part ? recvB : keepB; w4[3] = lo_part ? keepB : recvB;
            } else {
                w4[0] = lo_part ? recvA : keepA; w4[1] = lo_part ? recvB : keepB;
                w4[2] = lo_part ? keepA : recvA; w4[3] = lo_part ? keepB : recvB;
            }
            xf[t] = __builtin_bit_cast(bf16x8, make_uint4(w4[0], w4[1], w4[2], w4[3]));
        }
    } else {
        // Q8_0 rows: fp16 scales from byte 0, int8 codes from byte xqoff;
        // the pass's first block is kb0
        const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<void *>(X), 0, (int)((uint32_t)(N - 1) * x_pitch + (uint32_t)(xqoff + 32 * nb_row)),
            BUFFER_FLAGS);
        const uint32_t xrow = (uint32_t)tok * x_pitch;
        // the even lane of a token pair loads the 8 codes k0(g) .. k0(g)+7
        // of each block; the odd lane's channel stays zero
        const int k0 = (g == 0) ? 0 : (g == 1) ? 16 : (g == 2) ? 8 : 24;
        uint32_t raw[NBW][2];
#pragma unroll
        for (int t = 0; t < NBW; ++t) {
            const int b = b_begin + t;
            const uint32_t base = xrow + (uint32_t)(xqoff + 32 * (kb0 + b));
            const bool in = b < nb && tok < N && !lo_part;
            const auto v = __builtin_amdgcn_raw_buffer_load_b64(xres, in ? base + k0 : OUT_OF_RANGE, 0, 0);
            raw[t][0] = v[0];
            raw[t][1] = v[1];
        }
        // scales: 2 NBW bytes from block kb0 + b_begin of each token's row
        // (8- or 16-byte aligned: kb0 and b_begin are multiples of NBW)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int tk = 2 * g + h;
            const uint32_t off = (uint32_t)tk * x_pitch + 2u * (uint32_t)(kb0 + b_begin);
            const bool in = tk < N;
            if constexpr (NBW == 4) {
                const auto v = __builtin_amdgcn_raw_buffer_load_b64(xres, in ? off : OUT_OF_RANGE, 0, 0);
                dxs[h][0] = v[0];
                dxs[h][1] = v[1];
            } else {
#pragma unroll
                for (int q = 0; q < NBW / 8; ++q) {
                    const auto v = __builtin_amdgcn_raw_buffer_load_b128(xres, in ? off + 16 * q : OUT_OF_RANGE, 0, 0);
#pragma unroll
                    for (int e = 0; e < 4; ++e) dxs[h][4 * q + e] = v[e];
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        // codes 0..7 of the run in register order, exact in bf16
#pragma unroll
        for (int t = 0; t < NBW; ++t) {
            const uint32_t r0 = raw[t][0], r1 = raw[t][1];
            xf[t] = __builtin_bit_cast(bf16x8, make_uint4(pack_bf16(sbyte<0>(r0), sbyte<1>(r0)),
                                                           pack_bf16(sbyte<2>(r0), sbyte<3>(r0)),
                                                           pack_bf16(sbyte<0>(r1), sbyte<1>(r1)),
                                                           pack_bf16(sbyte<2>(r1), sbyte<3>(r1))));
        }
    }

    // one tile: unpack, matrix products, bias and scales; then the partial
    // sums of the KW waves (K ranges) meet in LDS and wave 0 stores the rows
    auto consume = [&](auto &stg, int tl, int it) {
        // SW: columns 8..15 read the up matrix's half of the stage
        const uint8_t *base = stg[wave] + (SW && j >= 8 ? St::BYTES : 0);
        const int jr = j & (TR - 1);       // the tile row column j reads
        // row j's scales, then its units 4p + g
        uint32_t sc[St::SR >= 4 ? St::SR / 4 : 1];
        if constexpr (St::SR == 4) {
            sc[0] = *reinterpret_cast<const uint32_t *>(base + St::CODE_BYTES + St::SR * jr);
        } else if constexpr (St::SR == 8) {
            const uint2 v = *reinterpret_cast<const uint2 *>(base + St::CODE_BYTES + St::SR * jr);
            sc[0] = v.x;
            sc[1] = v.y;
        } else {
#pragma unroll
            for (int h = 0; h < St::SR / 16; ++h) {
                const uint4 v = *reinterpret_cast<const uint4 *>(base + St::CODE_BYTES + St::SR * jr + 16 * h);
                sc[4 * h] = v.x;
                sc[4 * h + 1] = v.y;
                sc[4 * h + 2] = v.z;
                sc[4 * h + 3] = v.w;
            }
        }
        const uint8_t *rowp = base + (jr / St::RPI) * 1024 + (jr % St::RPI) * St::SB;
        float yp0 = 0.0f, yp1 = 0.0f;
        f32x4 Dh = {0.0f, 0.0f, 0.0f, 0.0f};   // F16: all blocks in one accumulator
#pragma unroll
        for (int p = 0; p < NG; ++p) {
            const uint4 cv = *reinterpret_cast<const uint4 *>(rowp + 16 * swz<St::U>(jr, 4 * p + g));
            if constexpr (WT == W_F16) {
                // halves 8g .. 8g + 7 of block p, already in matrix order.
                // Each finite half f = hi + lo exactly: hi = f rounded to
                // bf16, lo = f - hi (at most 2 significant bits, so exact in
                // bf16).  NaN stays NaN; an infinite half gives lo = NaN, so
                // its row's outputs are NaN (the activations' low parts,
                // often exactly 0, would turn Inf into NaN anyway).
                const uint32_t dw[4] = {cv.x, cv.y, cv.z, cv.w};
                uint32_t hv[4], lv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float f0 = (float)__builtin_bit_cast(_Float16, (uint16_t)(dw[e] & 0xFFFFu));
                    const float f1 = (float)__builtin_bit_cast(_Float16, (uint16_t)(dw[e] >> 16));
                    hv[e] = pack_bf16(f0, f1);
                    lv[e] = pack_bf16(f0 - bf16_lo(hv[e]), f1 - bf16_hi(hv[e]));
                }
                Dh = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf[p], __builtin_bit_cast(bf16x8, make_uint4(hv[0], hv[1], hv[2], hv[3])), Dh, 0, 0, 0);
                Dh = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf[p], __builtin_bit_cast(bf16x8, make_uint4(lv[0], lv[1], lv[2], lv[3])), Dh, 0, 0, 0);
                continue;
            }
            uint32_t d0 = cv.x, d1 = cv.y, d2 = cv.z, d3 = cv.w;
            // regroup: the four lane groups of each matrix instruction hold
            // disjoint code sets of one block
            swap32(d0, d2);
            swap32(d1, d3);
            if constexpr (WT == W_Q4_0) {
                swap16(d0, d1);
                swap16(d2, d3);
            }
#pragma unroll
            for (int t = 0; t < BPG; ++t) {
                uint32_t r[4];
                if constexpr (WT == W_Q4_0) {
                    // byte s of w holds lo(s) and hi(s); with the nibbles'
                    // top bits flipped, each nibble at the top of a byte is
                    // the int8 value 16 (n - 8)
                    const uint32_t w = ((t == 0) ? d0 : (t == 1) ? d1 : (t == 2) ? d2 : d3) ^ 0x88888888u;
                    const uint32_t hn = w & 0xF0F0F0F0u;            // hi(s) of every byte
                    const uint32_t ln = (w << 4) & 0xF0F0F0F0u;     // lo(s) of every byte
                    r[0] = pack_bf16(sbyte<0>(ln), sbyte<2>(ln));   // lo(s0) lo(s2)
                    r[1] = pack_bf16(sbyte<0>(hn), sbyte<2>(hn));   // hi(s0) hi(s2)
                    r[2] = pack_bf16(sbyte<1>(ln), sbyte<3>(ln));   // lo(s1) lo(s3)
                    r[3] = pack_bf16(sbyte<1>(hn), sbyte<3>(hn));   // hi(s1) hi(s3)
                } else {
                    const uint32_t wa = (t == 0) ? d0 : d2;
                    const uint32_t wb = (t == 0) ? d1 : d3;
                    r[0] = pack_bf16(sbyte<0>(wa), sbyte<1>(wa));
                    r[1] = pack_bf16(sbyte<2>(wa), sbyte<3>(wa));
                    r[2] = pack_bf16(sbyte<0>(wb), sbyte<1>(wb));
                    r[3] = pack_bf16(sbyte<2>(wb), sbyte<3>(wb));
                }
                const bf16x8 wf = __builtin_bit_cast(bf16x8, make_uint4(r[0], r[1], r[2], r[3]));
                const f32x4 D = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf[p * BPG + t], wf,
                                                                       f32x4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
                // a block past the row (its codes and activations read as
                // zeros) may pick up a scale from the bytes after the row's
                // scales: weight it by 0
                const int hw = (p * BPG + t) >> SS;             // the block's scale in the slice
                const uint32_t sw = sc[hw / 2];
                const float ds = (float)__builtin_bit_cast(_Float16, (uint16_t)((hw & 1) ? (sw >> 16) : (sw & 0xFFFFu)));
                const bool inb = b_begin + p * BPG + t < nb;
                if constexpr (XQ) {
                    // channels 4g + 1 and 4g + 3 are zero: D[0] and D[2] are
                    // the exact block sums of tokens 2g and 2g + 1
                    const int blk = p * BPG + t;
                    const float dx0 = (float)__builtin_bit_cast(_Float16, (uint16_t)(dxs[0][blk / 2] >> (16 * (blk & 1))));
                    const float dx1 = (float)__builtin_bit_cast(_Float16, (uint16_t)(dxs[1][blk / 2] >> (16 * (blk & 1))));
                    yp0 = fmaf(inb ? ds * dx0 : 0.0f, D[0], yp0);
                    yp1 = fmaf(inb ? ds * dx1 : 0.0f, D[2], yp1);
                } else {
                    const float d = inb ? ds : 0.0f;
                    yp0 = fmaf(d, D[0] + D[1], yp0);
                    yp1 = fmaf(d, D[2] + D[3], yp1);
                }
            }
        }
        if constexpr (WT == W_F16) {
            yp0 = Dh[0] + Dh[1];
            yp1 = Dh[2] + Dh[3];
        }
        float *mine = red[it & 1][wave][lane];
        mine[0] = yp0 * MfFmt<WT>::code_scale;     // a power of two: exact
        mine[1] = yp1 * MfFmt<WT>::code_scale;
        __syncthreads();
        if (wave == 0) {
            float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
            for (int w2 = 0; w2 < KW; ++w2) {
                s0 += red[it & 1][w2][lane][0];
                s1 += red[it & 1][w2][lane][1];
            }
            const int m = tl * TR + j;
            if constexpr (SW) {
                // row_ror:8 within each 16-lane row: lane j reads lane j ^ 8
                const float u0 = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, s0), 0x128, 0xF, 0xF, true));
                const float u1 = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, s1), 0x128, 0xF, 0xF, true));
                if (j < 8 && m < M) {
                    float *y0 = Y + (uint64_t)(2 * g) * y_pitch + m;
                    if (2 * g < N) *y0 = swish(s0) * u0;
                    if (2 * g + 1 < N) *(y0 + y_pitch) = swish(s1) * u1;
                }
            } else if (j < TR && m < M) {
                float *y0 = Y + (uint64_t)(2 * g) * y_pitch + m;
                float *y1 = y0 + y_pitch;
                if (2 * g < N) *y0 = acc ? *y0 + s0 : s0;
                if (2 * g + 1 < N) *y1 = acc ? *y1 + s1 : s1;
            }
        }
    };

    // stage s holds tiles it = s (mod NSTG); before a tile is consumed the
    // tile NSTG-1 steps ahead is issued into the stage the previous step freed.  The
    // steps past the last tile issue loads that read nothing.  The loop bounds
    // are uniform over the workgroup.
    for (int it = 0;; it += NSTG) {
        if (tile >= n_tiles) break;
        if constexpr (NSTG == 2) issue(st1, tile + n_wg);
        else if constexpr (NSTG == 3) issue(st2, tile + 2 * n_wg);
        else issue(st3, tile + 3 * n_wg);
        wait_vm<(NSTG - 1) * SWF * (St::NI + St::NS)>();     // this tile's loads have landed
        consume(st0, tile, it);
        tile += n_wg;
        if (tile >= n_tiles) break;
        issue(st0, tile + (NSTG - 1) * n_wg);
        wait_vm<(NSTG - 1) * SWF * (St::NI + St::NS)>();     // this tile's loads have landed
        consume(st1, tile, it + 1);
        tile += n_wg;
        if constexpr (NSTG > 2) {
            if (tile >= n_tiles) break;
            issue(st1, tile + (NSTG - 1) * n_wg);
            wait_vm<(NSTG - 1) * SWF * (St::NI + St::NS)>();
            consume(st2, tile, it + 2);
            tile += n_wg;
        }
        if constexpr (NSTG > 3) {
            if (tile >= n_tiles) break;
            issue(st2, tile + (NSTG - 1) * n_wg);
            wait_vm<(NSTG - 1) * SWF * (St::NI + St::NS)>();
            consume(st3, tile, it + 3);
            tile += n_wg;
        }
    }
    // no load may still write this workgroup's LDS after it ends
    wait_vm<0>();
}

using MfKernel = void (*)(const MfArgs);

// In the Q8_0-activation and fused SwiGLU kernels eight waves share a tile
// (each one eighth of the pass's K, so that two waves per SIMD hide each
// other's latencies), with NBW = 4, 8 or 16 blocks per wave; the other
// fp32-activation passes take sixteen (kNarrowWaves below).  Three stages
// (measured on eight-wave workgroups at K = 2048 and 5632, 4 and 8
// tokens): a Q4_0 workgroup then needed 63 KB of LDS and two shared a CU,
// 2-4 % faster than one with four stages; Q8_0 with two stages (two
// workgroups per CU) was as fast at 4 tokens and 4 % slower at 8.  (The
// stage count drops to what fits 160 KiB, e.g. two for the wide launch.)
constexpr int kWaves = 8;
// Blocks of K one launch covers (16 per wave); longer rows take several
// launches, the later ones adding to y.
constexpr int kPassBlocks = 16 * kWaves;
constexpr int kStages = 3;

// Q4_0, Q8_0 and F16 passes with fp32 activations (other than the wide
// launch) run as ONE workgroup of sixteen waves x 4 or 8 blocks per CU instead of
// eight-wave workgroups: each CU builds the activation fragments of its K
// once (N K 4 bytes per workgroup, which at 8 tokens outweigh a CU's share
// of the weights on its load path) and keeps sixteen waves in flight.
// Measured (graph-replayed, us at 4 / 8 tokens): the Q4_0 [Wgate Wup] batch
// 2 x 5632 x 2048 7.3 / 7.8 against 8.5 / 9.0 (two eight-wave workgroups
// per CU), [Wq Wk Wv] 4.7 / 4.9 against 5.6 / 5.9; at 5 / 8 tokens Q4_0
// 4096 x 4096 6.4 / 6.7 against 7.4 / 7.9, 11008 x 4096 11.0 / 11.3
// against 12.2 / 12.4, Q8_0 4096 x 4096 7.6 / 7.7 against 8.4 / 8.5, Q8_0
// 5632 x 2048 6.3 / 6.5 against 6.6 / 6.8; two sixteen-wave workgroups per
// CU 9.0 / 9.4 on the gate/up batch; Wo 2048 x 2048 unchanged, the Q8_0
// LM head unchanged at 4 tokens and 1 % slower at 8 (16.6 against 16.5,
// medians of 7).  F16 rows too (3-4 %: 5632 x 2048 at 5 / 8 tokens 8.6 /
// 8.9 against 8.9 / 9.3, 32000 x 2048 27.4 / 27.9 against 28.3 / 28.9); Q8_0
// activations keep eight waves (within 1 %, 16384 x 2048 2 % slower with
// sixteen).  The fused SwiGLU tiles need 8 blocks per wave, so they keep
// eight waves (at one workgroup per CU: 7.8 against 8.2 us at 8 tokens
// with two).
constexpr int kNarrowWaves = 16;

// Rows of 129 to 192 blocks (K = 4128 .. 6144; a down projection's 5632)
// run in ONE launch of twelve waves x 16 blocks instead of two passes.
// Short matrices of such rows give each workgroup one tile, so the passes'
// fixed costs (launch, activation set-up, the last wave's data) are paid
// once.  Measured on 2048 x 5632 (graph-replayed, Q4_0, 8 tokens):
// 7.9 us against 14.2 us in two passes.  A Q4_0 tile keeps 16 rows (two
// 55 KB stages); Q8_0 takes 8-row tiles, since 16 rows x 512 code bytes x
// 12 waves would not fit two stages in the LDS.
constexpr int kWideWaves = 12;
constexpr int kWideBlocks = 16 * kWideWaves;
template <int WT> constexpr int wide_tile_rows() { return WT == W_Q4_0 ? 16 : 8; }

// Blocks per wave for a pass of nb blocks (0 if out of range).
int mf_nbw(int64_t nb)
{
    if (nb <= 0 || nb > kPassBlocks) return 0;
    const int64_t per = (nb + kWaves - 1) / kWaves;
    return per <= 4 ? 4 : per <= 8 ? 8 : 16;
}

// Tile rows of a pass of nb blocks: F16 rows of 8 blocks per wave (512
// bytes per row and wave, sixteen waves) take 8-row tiles, so that two
// stages fit the LDS.
int mf_tile_rows(int type, bool wide, int64_t nb)
{
    if (type == W_F16) return (nb + kNarrowWaves - 1) / kNarrowWaves <= 4 ? kTileRows : 8;
    if (!wide) return kTileRows;
    return type == W_Q4_0 ? wide_tile_rows<W_Q4_0>() : wide_tile_rows<W_Q8_0>();
}

// The eight-wave kernel for (type, NBW, scale shift, activation format)
// and its LDS bytes: Q8_0 weights with Q8_0 activations.
template <int WT, int SS, bool XQ>
MfKernel pick_mf(int nbw, int *lds)
{
    constexpr int D = kStages, T = kTileRows;
    switch (nbw) {
    case 4: *lds = mf_lds_bytes<WT, kWaves, 4, SS, T>(mf_stages<WT, kWaves, 4, SS, D, T>()); return gemv_mf_kernel<WT, kWaves, 4, SS, D, T, XQ, false>;
    case 8: *lds = mf_lds_bytes<WT, kWaves, 8, SS, T>(mf_stages<WT, kWaves, 8, SS, D, T>()); return gemv_mf_kernel<WT, kWaves, 8, SS, D, T, XQ, false>;
    case 16: *lds = mf_lds_bytes<WT, kWaves, 16, SS, T>(mf_stages<WT, kWaves, 16, SS, D, T>()); return gemv_mf_kernel<WT, kWaves, 16, SS, D, T, XQ, false>;
    default: return nullptr;
    }
}
// The twelve-wave kernel of the wide launch.
template <int WT, int SS, bool XQ>
MfKernel pick_wide(int *lds)
{
    constexpr int T = wide_tile_rows<WT>();
    *lds = mf_lds_bytes<WT, kWideWaves, 16, SS, T>(mf_stages<WT, kWideWaves, 16, SS, kStages, T>());
    return gemv_mf_kernel<WT, kWideWaves, 16, SS, kStages, T, XQ, false>;
}
// The sixteen-wave kernel of a pass of nb blocks (4 or 8 per wave).
template <int WT, int SS>
MfKernel pick_narrow(int64_t nb, int *lds)
{
    constexpr int D = kStages, KW = kNarrowWaves;
    constexpr int T4 = kTileRows, T8 = WT == W_F16 ? 8 : kTileRows;   // as mf_tile_rows
    const int64_t per = (nb + KW - 1) / KW;
    if (per <= 4) {
        *lds = mf_lds_bytes<WT, KW, 4, SS, T4>(mf_stages<WT, KW, 4, SS, D, T4>());
        return gemv_mf_kernel<WT, KW, 4, SS, D, T4, false, false>;
    }
    if (per <= 8) {
        *lds = mf_lds_bytes<WT, KW, 8, SS, T8>(mf_stages<WT, KW, 8, SS, D, T8>());
        return gemv_mf_kernel<WT, KW, 8, SS, D, T8, false, false>;
    }
    return nullptr;
}
// The kernel of one pass, its LDS bytes and its waves per workgroup.
template <bool XQ>
MfKernel pick(int type, int ss, bool wide, int64_t nb, int *lds, int *waves)
{
    const int nbw = mf_nbw(nb);
    *waves = wide ? kWideWaves : kWaves;
    if constexpr (!XQ) {
        if (wide && type == W_Q4_0) return ss ? pick_wide<W_Q4_0, 1, false>(lds) : pick_wide<W_Q4_0, 0, false>(lds);
        if (!wide && (type == W_Q4_0 || type == W_Q8_0)) {
            *waves = kNarrowWaves;
            if (type == W_Q4_0) return ss ? pick_narrow<W_Q4_0, 1>(nb, lds) : pick_narrow<W_Q4_0, 0>(nb, lds);
            return ss ? pick_narrow<W_Q8_0, 1>(nb, lds) : pick_narrow<W_Q8_0, 0>(nb, lds);
        }
        if (type == W_F16) {
            if (wide) return nullptr;
            *waves = kNarrowWaves;
            return pick_narrow<W_F16, 0>(nb, lds);
        }
    }
    if (wide && type == W_Q8_0) return ss ? pick_wide<W_Q8_0, 1, XQ>(lds) : pick_wide<W_Q8_0, 0, XQ>(lds);
    if (type == W_Q8_0) return ss ? pick_mf<W_Q8_0, 1, XQ>(nbw, lds) : pick_mf<W_Q8_0, 0, XQ>(nbw, lds);
    return nullptr;
}

// The fused SwiGLU kernel: 8 + 8 row tiles (8-row stages need at most 8
// rows per load instruction, so Q4_0 takes at least 8 blocks per wave).
template <int WT, int SS>
MfKernel pick_sw(int nbw, int *lds)
{
    constexpr int D = kStages;
    if (WT == W_Q4_0 && nbw < 8) nbw = 8;
    switch (nbw) {
    case 4:
        if constexpr (WT == W_Q8_0) {
            *lds = mf_lds_bytes<WT, kWaves, 4, SS, 8, true>(mf_stages<WT, kWaves, 4, SS, D, 8, true>());
            return gemv_mf_kernel<WT, kWaves, 4, SS, D, 8, false, true>;
        }
        return nullptr;
    case 8: *lds = mf_lds_bytes<WT, kWaves, 8, SS, 8, true>(mf_stages<WT, kWaves, 8, SS, D, 8, true>()); return gemv_mf_kernel<WT, kWaves, 8, SS, D, 8, false, true>;
    case 16: *lds = mf_lds_bytes<WT, kWaves, 16, SS, 8, true>(mf_stages<WT, kWaves, 16, SS, D, 8, true>()); return gemv_mf_kernel<WT, kWaves, 16, SS, D, 8, false, true>;
    default: return nullptr;
    }
}

// One item's activations: fp32 rows (pitch in elements) or Q8_0 rows of
// the same K (pitch in bytes).
struct MfSrc {
    const void *base;
    uint64_t pitch;
};

template <bool XQ>
hipError_t launch_mf(const WeightView *w, const MfSrc *x, const OutView *y, int count, int64_t N,
                     hipStream_t stream)
{
    if (count < 1 || count > kMaxMfItems) return hipErrorInvalidValue;
    const int type = w[0].type;
    const int64_t K = w[0].K;
    const int64_t nb_row = K / 32;
    const int ss = w[0].scale_shift;
    const bool wide = type != W_F16 && nb_row > kPassBlocks && nb_row <= kWideBlocks;
    const int64_t pass = wide ? kWideBlocks : kPassBlocks;
    int64_t m_total = 0;
    for (int i = 0; i < count; ++i) m_total += w[i].M;
    if (m_total == 0 || N == 0 || nb_row == 0) return hipSuccess;
    for (int64_t n0 = 0; n0 < N; n0 += 8) {
        // passes over K in stream order: the first stores y, the others add
        for (int64_t kb0 = 0; kb0 < nb_row; kb0 += pass) {
            const int64_t nb = nb_row - kb0 < pass ? nb_row - kb0 : pass;
            const int tr = mf_tile_rows(type, wide, nb);
            int64_t tiles_total = 0;
            for (int i = 0; i < count; ++i) tiles_total += (w[i].M + tr - 1) / tr;
            int lds = kLdsBytes, waves = 0;
            const MfKernel k = pick<XQ>(type, ss, wide, nb, &lds, &waves);
            if (!k) return hipErrorInvalidValue;
            // a workgroup streams several tiles with its activation fragments
            // resident: as many workgroups as the LDS of the 256 CUs holds
            // (one per CU for the sixteen-wave kind)
            const int64_t cap = 256 * (int64_t)(waves == kNarrowWaves ? 1 : kLdsBytes / lds);
            MfArgs a = {};
            a.N = (int32_t)(N - n0 < 8 ? N - n0 : 8);
            a.K = (int32_t)(32 * nb);
            a.qoff = type == W_F16 ? 0 : (int32_t)quant_offset(K, ss);
            a.nb = (int32_t)nb;
            a.kb0 = (int32_t)kb0;
            a.nb_row = (int32_t)nb_row;
            a.accumulate = kb0 > 0;
            a.xqoff = XQ ? (int32_t)quant_offset(K) : 0;
            int32_t wg_max = 0;
            for (int i = 0; i < count; ++i) {
                if (w[i].M == 0) continue;
                MfItem &it = a.item[a.n_items++];
                it.w = w[i].base;
                it.pitch = (uint32_t)w[i].pitch;
                it.M = (int32_t)w[i].M;
                if constexpr (XQ)
                    it.x = static_cast<const uint8_t *>(x[i].base) + (uint64_t)n0 * x[i].pitch;
                else
                    it.x = static_cast<const float *>(x[i].base) + (uint64_t)n0 * x[i].pitch + (uint64_t)32 * kb0;
                it.x_pitch = (uint32_t)x[i].pitch;
                it.y = y[i].data + (uint64_t)n0 * y[i].pitch_elems;
                it.y_pitch = (uint32_t)y[i].pitch_elems;
                it.n_tiles = (int32_t)((w[i].M + tr - 1) / tr);
                int64_t wgs = (int64_t)it.n_tiles * cap / tiles_total;
                if (wgs < 1) wgs = 1;
                if (wgs > it.n_tiles) wgs = it.n_tiles;
                it.wg_count = (int32_t)wgs;
                if (wgs > wg_max) wg_max = (int32_t)wgs;
            }
            hipLaunchKernelGGL(k, dim3((unsigned)wg_max, (unsigned)a.n_items), dim3(64 * waves), 0, stream, a);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

}  // namespace

bool gemv_mf_supported(const GemvTask *tasks, int count)
{
    const int type = tasks[0].w.type;
    const int64_t K = tasks[0].w.K;
    if (!(type == W_Q4_0 || type == W_Q8_0 || type == W_F16) || K % 32 != 0 || K == 0) return false;
    // a 16-row tile is one buffer resource with 32-bit offsets
    // and the activations of up to 8 tokens another (byte offsets < 2^31)
    for (int i = 0; i < count; ++i) {
        const int64_t nt = tasks[i].x.N < 8 ? tasks[i].x.N : 8;
        // rows are read in 16-byte units (the entry points require 16-byte
        // weight pitches; F16 rows are checked here too)
        if (type == W_F16 && tasks[i].w.pitch % 16 != 0) return false;
        if (tasks[i].w.pitch > (1ull << 27) ||
            (nt - 1) * (int64_t)tasks[i].x.pitch_elems + K > (int64_t)1 << 29)
            return false;
    }
    return true;
}

hipError_t launch_gemv_mf(const GemvTask *tasks, int count, hipStream_t stream)
{
    if (count < 1 || count > kMaxMfItems) return hipErrorInvalidValue;
    WeightView w[kMaxMfItems];
    MfSrc x[kMaxMfItems];
    OutView y[kMaxMfItems];
    for (int i = 0; i < count; ++i) {
        w[i] = tasks[i].w;
        x[i] = MfSrc{tasks[i].x.data, tasks[i].x.pitch_elems};
        y[i] = tasks[i].y;
    }
    return launch_mf<false>(w, x, y, count, tasks[0].x.N, stream);
}

bool gemv_mf_swiglu_supported(const WeightView &wg, const WeightView &wu, const ActView &x)
{
    const int type = wg.type;
    const int64_t K = wg.K;
    if (!(type == W_Q4_0 || type == W_Q8_0) || K % 32 != 0 || K == 0 || K / 32 > kPassBlocks) return false;
    if (wu.type != type || wu.K != K || wu.M != wg.M || wu.scale_shift != wg.scale_shift) return false;
    const int64_t nt = x.N < 8 ? x.N : 8;
    return wg.pitch <= (1ull << 27) && wu.pitch <= (1ull << 27) &&
           (nt - 1) * (int64_t)x.pitch_elems + K <= (int64_t)1 << 29 && wg.M < ((int64_t)1 << 30);
}

hipError_t launch_gemv_mf_swiglu(const WeightView &wg, const WeightView &wu, const ActView &x, const OutView &h,
                                 hipStream_t stream)
{
    const int type = wg.type;
    const int64_t K = wg.K, M = wg.M, N = x.N;
    const int64_t nb_row = K / 32;
    if (M == 0 || N == 0) return hipSuccess;
    if (nb_row == 0 || nb_row > kPassBlocks) return hipErrorInvalidValue;
    const int ss = wg.scale_shift;
    int lds = kLdsBytes;
    const int nbw = mf_nbw(nb_row);
    const MfKernel k = type == W_Q4_0 ? (ss ? pick_sw<W_Q4_0, 1>(nbw, &lds) : pick_sw<W_Q4_0, 0>(nbw, &lds))
                     : type == W_Q8_0 ? (ss ? pick_sw<W_Q8_0, 1>(nbw, &lds) : pick_sw<W_Q8_0, 0>(nbw, &lds))
                                      : nullptr;
    if (!k) return hipErrorInvalidValue;
    const int64_t n_tiles = (M + 7) / 8;
    const int64_t cap = 256;     // one workgroup per CU (see kNarrowWaves)
    const int64_t wgs = n_tiles < cap ? n_tiles : cap;
    for (int64_t n0 = 0; n0 < N; n0 += 8) {
        MfArgs a = {};
        a.N = (int32_t)(N - n0 < 8 ? N - n0 : 8);
        a.K = (int32_t)K;
        a.qoff = (int32_t)quant_offset(K, ss);
        a.nb = (int32_t)nb_row;
        a.n_items = 1;
        a.kb0 = 0;
        a.nb_row = (int32_t)nb_row;
        a.accumulate = 0;
        a.w2 = wu.base;
        a.pitch2 = (uint32_t)wu.pitch;
        MfItem &it = a.item[0];
        it.w = wg.base;
        it.pitch = (uint32_t)wg.pitch;
        it.M = (int32_t)M;
        it.x = static_cast<const float *>(x.data) + (uint64_t)n0 * x.pitch_elems;
        it.x_pitch = (uint32_t)x.pitch_elems;
        it.y = h.data + (uint64_t)n0 * h.pitch_elems;
        it.y_pitch = (uint32_t)h.pitch_elems;
        it.n_tiles = (int32_t)n_tiles;
        it.wg_count = (int32_t)wgs;
        hipLaunchKernelGGL(k, dim3((unsigned)wgs, 1u), dim3(64 * kWaves), 0, stream, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

bool gemv_mf_q8x_supported(const WeightView *w, const WeightView *xq, int count, int64_t N)
{
    const int type = w[0].type;
    const int64_t K = w[0].K;
    if (type != W_Q8_0 || K % 32 != 0 || K == 0) return false;
    const int64_t nt = N < 8 ? N : 8;
    for (int i = 0; i < count; ++i) {
        if (w[i].pitch > (1ull << 27) || xq[i].pitch % 16 != 0 ||
            (nt - 1) * (int64_t)xq[i].pitch + quant_offset(K) + K >= (int64_t)1 << 31)
            return false;
    }
    return true;
}

hipError_t launch_gemv_mf_q8x(const WeightView *w, const WeightView *xq, const OutView *y, int count, int64_t N,
                              hipStream_t stream)
{
    if (count < 1 || count > kMaxMfItems) return hipErrorInvalidValue;
    MfSrc x[kMaxMfItems];
    for (int i = 0; i < count; ++i) x[i] = MfSrc{xq[i].base, xq[i].pitch};
    return launch_mf<true>(w, x, y, count, N, stream);
}

}  // namespace qmm
