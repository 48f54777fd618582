// gemm_rq.hip -- prefill GEMM for Q4_0 / Q8_0 weights with the codes
// dequantized in the registers of the waves that multiply them.
//
// Y[n][m] = sum_k W'[m][k] * X[n][k] for a tile of 128 weight rows x 128
// tokens (No Python! Building an AI Inference Engine Exclusively in C++, §6:
// C_ij = sum_k A_ik B_kj; §6.1: tile, pack, feed the multiply-add units).
// Each weight is unpacked to its signed code and multiplied by its block
// scale (Development Guide for Small AI Models (TinyLLaMA, etc.) Using C++,
// §6.2) just before the bf16 matrix instruction that uses it, in the wave
// that issues that instruction; W' is never written to LDS.
//
// Work split (8 waves, two per SIMD; waves g and g + 4 share a SIMD):
//  * row group g = wave % 4 owns tile rows 32 g .. 32 g + 31 for all 128
//    tokens (four 32 x 32 v_mfma_f32_32x32x16_bf16 tiles), so each weight
//    is dequantized once per tile and feeds 128 tokens;
//  * the two waves of a SIMD split every 64-wide K-step by 32-block (wave
//    parity p = wave / 4 takes block 2 t + p of step t) and add their sums
//    at the end, so the SIMD always has a second wave whose unpacking or
//    LDS reads run beside the first one's matrix instructions.
//
// Staging: the token tile (bf16, 128 B per token and step) and the weight
// codes (grouped four steps at a time: 128 B per row for Q4_0, 256 B for
// Q8_0) and scales go from memory to LDS with direct-to-LDS buffer loads,
// D steps ahead, into a ring of D + 1 token stages and two code/scale group
// buffers.  Every 16-byte unit is placed by an XOR of its index with bits of
// its row, so that the rows read together by one LDS instruction fall in
// different banks.  One barrier per step: before it each wave waits for its
// own loads of the step after next; the fragment reads of step t + 1 are
// interleaved with the matrix instructions of step t.
#include "gemm_common.h"

namespace qmm {
namespace {

constexpr int BM = 128;               // weight rows per tile
constexpr int BN = 128;               // tokens per tile
constexpr int THREADS = 512;
constexpr int TOK_BYTES = BN * 128;   // one K-step (64 bf16) of the token tile
constexpr int DT = 4;                 // K-steps of token loads in flight
constexpr int TS = DT + 1;            // token stages
constexpr int GROUP_BYTES = BM * 128; // a code group: 128 bytes of codes per row
constexpr int SGROUP_BYTES = BM * 16; // its scales: 16 bytes per row
constexpr int NB = 4;                 // code / scale group buffers
constexpr int TOK_LOADS = 4;          // per token wave and step (16 KB over waves 4..7)
constexpr int CODE_LOADS = 4;         // per code wave and group (16 KB over waves 0..3)
constexpr int SCALE_LOADS = 2;        // per code wave and group (2 KB)
constexpr int LDS_GROUP_OFF = TS * TOK_BYTES;
constexpr int LDS_SCALE_OFF = LDS_GROUP_OFF + NB * GROUP_BYTES;
constexpr int LDS_BYTES = LDS_SCALE_OFF + NB * SGROUP_BYTES;
static_assert(LDS_BYTES <= 160 * 1024, "one workgroup per CU");
static_assert(LDS_BYTES >= (8 * 2 * 16 * 64 + 8 * 16 * 64) * 4, "the final exchanges reuse the ring");

typedef int i32x4 __attribute__((ext_vector_type(4)));

// A code group is 128 bytes of each tile row: GS K-steps, i.e. 2 GS blocks
// of 16 code bytes (Q4_0, GS = 4) or 32 (Q8_0, GS = 2).  Group g is issued
// in iteration GS g - DC (the first groups before the loop), DC steps ahead
// of its first use; it is last read in iteration GS g + GS - 2, so the
// buffer it shares with group g + NB is free from iteration GS g + GS - 1 on.
template <int WT> struct RqFmt;
template <> struct RqFmt<W_Q4_0> { static constexpr int QB = 16, GS = 4; };
template <> struct RqFmt<W_Q8_0> { static constexpr int QB = 32, GS = 2; };
// F16 rows: 64 bytes per 32 weights, no scales; a group is one K-step
template <> struct RqFmt<W_F16> { static constexpr int QB = 64, GS = 1; };
template <int WT>
struct RqSched {
    static constexpr int QB = RqFmt<WT>::QB;
    static constexpr int GS = RqFmt<WT>::GS;
    static_assert(2 * GS * QB == 128, "a group is 128 bytes of a row");
    static constexpr bool SCALES = WT != W_F16;
    // loads of one group by one code wave
    static constexpr int LOADS = CODE_LOADS + (SCALES ? SCALE_LOADS : 0);
    // group g is issued DC steps ahead of its first step (five for the
    // quantized types, three iterations before its first codes are read;
    // four for F16, whose one-step groups would otherwise need five
    // buffers); it is last read (codes two steps ahead) in iteration
    // GS g + GS - 3
    static constexpr int DC = GS == 1 ? 4 : 5;
    static constexpr int PRO = (DC + GS - 1) / GS;       // groups issued before the loop
    static_assert(PRO <= NB, "the prologue's groups fit the buffers");
    static_assert(NB * GS - DC > GS - 3, "a group buffer is free before the group after next is issued into it");
    // groups the prologue reads (the raw codes of steps 0 and 1)
    static constexpr int PRO_READ = 1 + 1 / GS;
    // loads a code wave may still have in flight at the top of iteration t
    // (t mod GS = u) once the group of step t + 2 has landed: those of the
    // later groups issued by then (iteration GS g - DC <= t - 1)
    static constexpr int pending(int u)
    {
        return LOADS * ((u - 1 + DC) / GS - (u + 2) / GS);
    }
    static_assert(pending(0) >= 0 && pending(GS - 1) >= 0, "the group of step t + 2 is issued before iteration t");
};

__device__ inline i32x4 buffer_rsrc(const void *base, uint32_t bytes)
{
    const uint64_t p = reinterpret_cast<uint64_t>(base);
    return i32x4{(int)(uint32_t)p, (int)((uint32_t)(p >> 32) & 0xFFFFu), (int)bytes, BUFFER_FLAGS};
}

// Direct-to-LDS buffer loads, written as instructions the compiler does not
// see (it neither moves LDS reads across them nor waits for them); lane i of
// one load writes its bytes at lds + size * i.  m0 carries the LDS address.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ inline void lds_load16(const i32x4 &rsrc, uint32_t lds, uint32_t voff)
{
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "s"(lds), "v"(voff), "s"(rsrc) : "memory", "m0");
}
__device__ inline void lds_load4(const i32x4 &rsrc, uint32_t lds, uint32_t voff)
{
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                 :: "s"(lds), "v"(voff), "s"(rsrc) : "memory", "m0");
}
// The same with a scalar byte offset added to the lane's (the buffer's range
// check is applied to the lane offset alone, so soff may only be used where
// lane offset + soff is known to stay inside the buffer).
__device__ inline void lds_load16s(const i32x4 &rsrc, uint32_t lds, uint32_t voff, uint32_t soff)
{
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"(lds), "v"(voff), "s"(rsrc), "s"(soff) : "memory", "m0");
}
__device__ inline void lds_load4s(const i32x4 &rsrc, uint32_t lds, uint32_t voff, uint32_t soff)
{
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
                 :: "s"(lds), "v"(voff), "s"(rsrc), "s"(soff) : "memory", "m0");
}
#pragma clang diagnostic pop
template <int N>
__device__ inline void wait_vm()
{
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// One lane's share of a block: 16 weights of one row, its two halves of the
// block's two 16-deep k chunks (lane half h: k = 8 h .. 8 h + 7 of each
// chunk), as bf16 pairs: b[0..3] chunk 0, b[4..7] chunk 1.  Every value is
// the bf16 rounding (nearest even) of code * Delta, which binary32 holds
// exactly.
//  Q4_0: byte j of the lane's 8 holds the codes of k = 8 h + j (low nibble)
//        and 16 + 8 h + j (high nibble).  A nibble left in place under the
//        binary16 exponent of 1024 (0x6400) reads 1024 + n (low) or 1024 + 16 n
//        (high); v_fma_mix_f32 widens it inside fma(1024 + n, Delta, -1032 Delta)
//        = (n - 8) Delta, or fma(1024 + 16 n, Delta / 16, -72 Delta), both exact.
//  Q8_0: the byte with its sign bit flipped (code + 128) under the same
//        exponent reads 1152 + code; fma(1152 + code, Delta, -1152 Delta).
template <int WT> struct Deq;

// Unpacking in eight parts of a few VALU operations each, so that the parts
// can sit between matrix instructions; part p always writes output p2o[p]
// (parts share the unpacked halves through the struct).
template <>
struct Deq<W_Q4_0> {
    uint32_t w8[2], lo02, lo13, hi02, hi13;
    float d, n0, d16, n1;
    template <int P>
    __device__ inline void part(u32x2 c, uint16_t sbits, bool live, uint32_t (&b)[8])
    {
        // dword 0 of the lane's codes in parts 0..4, dword 1 in parts 4..7
        const uint32_t magic = __builtin_amdgcn_readfirstlane(0x64006400u);
        if constexpr (P == 0) {
            d = live ? (float)__builtin_bit_cast(_Float16, sbits) : 0.0f;
            n0 = -1032.0f * d;
            w8[0] = c[0] >> 8;
        } else if constexpr (P == 1 || P == 5) {
            constexpr int i = P / 4;
            lo02 = and_or(c[i], 0x000F000Fu, magic);
            lo13 = and_or(w8[i], 0x000F000Fu, magic);
            b[2 * i] = pack_bf16(fmaf(lo_half(lo02), d, n0), fmaf(lo_half(lo13), d, n0));
        } else if constexpr (P == 2) {
            b[1] = pack_bf16(fmaf(hi_half(lo02), d, n0), fmaf(hi_half(lo13), d, n0));
            d16 = d * 0.0625f;
            n1 = -72.0f * d;
        } else if constexpr (P == 3) {
            hi02 = and_or(c[0], 0x00F000F0u, magic);
            hi13 = and_or(w8[0], 0x00F000F0u, magic);
            b[4] = pack_bf16(fmaf(lo_half(hi02), d16, n1), fmaf(lo_half(hi13), d16, n1));
        } else if constexpr (P == 4) {
            b[5] = pack_bf16(fmaf(hi_half(hi02), d16, n1), fmaf(hi_half(hi13), d16, n1));
            w8[1] = c[1] >> 8;
        } else if constexpr (P == 6) {
            b[3] = pack_bf16(fmaf(hi_half(lo02), d, n0), fmaf(hi_half(lo13), d, n0));
            hi02 = and_or(c[1], 0x00F000F0u, magic);
            hi13 = and_or(w8[1], 0x00F000F0u, magic);
        } else {                                  // P == 7
            b[6] = pack_bf16(fmaf(lo_half(hi02), d16, n1), fmaf(lo_half(hi13), d16, n1));
            b[7] = pack_bf16(fmaf(hi_half(hi02), d16, n1), fmaf(hi_half(hi13), d16, n1));
        }
    }
};
template <>
struct Deq<W_Q8_0> {
    uint32_t p02, p13;
    float d, n;
    template <int P>
    __device__ inline void part(u32x2 c0, u32x2 c1, uint16_t sbits, bool live, uint32_t (&b)[8])
    {
        // part P: output 4 c + 2 i + e of dword i of chunk c (P = 4 c + 2 i + e)
        const uint32_t magic = __builtin_amdgcn_readfirstlane(0x64006400u);
        constexpr int c = P / 4, i = (P / 2) % 2, e = P % 2;
        if constexpr (P == 0) {
            d = live ? (float)__builtin_bit_cast(_Float16, sbits) : 0.0f;
            n = -1152.0f * d;
        }
        if constexpr (e == 0) {
            const uint32_t w = (c ? c1[i] : c0[i]) ^ 0x80808080u;
            p02 = and_or(w, 0x00FF00FFu, magic);
            p13 = and_or(w >> 8, 0x00FF00FFu, magic);
            b[P] = pack_bf16(fmaf(lo_half(p02), d, n), fmaf(lo_half(p13), d, n));
        } else {
            b[P] = pack_bf16(fmaf(hi_half(p02), d, n), fmaf(hi_half(p13), d, n));
        }
    }
};

// F16: the lane's 16 weights are two runs of 8 halves (k = 8 h .. 8 h + 7 of
// each chunk); each becomes the bf16 rounding (nearest even) of its exact
// binary32 value.  A block past K reads the next row's bytes, which may be
// any halves, Inf and NaN included: it is replaced by zeros.
template <>
struct Deq<W_F16> {
    template <int P>
    __device__ inline void part(u32x4 c0, u32x4 c1, bool live, uint32_t (&b)[8])
    {
        const uint32_t w = P < 4 ? c0[P % 4] : c1[P % 4];
        const uint32_t v = pack_bf16(lo_half(w), hi_half(w));
        b[P] = live ? v : 0u;
    }
};

// A lane's raw weights of one step: codes and scale, or F16 halves.
template <int WT> struct RawOf { u32x2 c0, c1; uint16_t sbits; };
template <> struct RawOf<W_F16> { u32x4 c0, c1; };

// Swish(z) = z * sigma(z) = z / (1 + e^{-z}) in binary32 (for z far below
// zero e^{-z} overflows and the quotient is the limit -0).
__device__ inline float swish(float z)
{
    return z / (1.0f + expf(-z));
}

// BATCH: several products in one launch (a workgroup finds its item by tile
// index); otherwise item 0 only, so that every argument is read in one round
// of scalar loads.
// SW: the fused gate/up projection with the SwiGLU epilogue ("Development
// Guide for Small AI Models (TinyLLaMA, etc.) Using C++", §4.4): a tile is
// 64 rows of the gate matrix (row groups 0, 1) and the same 64 rows of the
// up matrix (row groups 2, 3) times 128 tokens; only h = Swish(gate) * up is
// stored.
template <int WT, int SS, bool BATCH, bool SW>
__global__ __launch_bounds__(THREADS) void gemm_rq_kernel(const GemmArgs a)
{
    using Sc = RqSched<WT>;
    constexpr int QB = Sc::QB, GS = Sc::GS, DC = Sc::DC;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const uint32_t lds0 = (uint32_t)reinterpret_cast<uintptr_t>(lds);

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int rg = wave & 3;          // row group: tile rows 32 rg .. 32 rg + 31
    const int par = wave >> 2;        // block 2 t + par of each step t
    const int h = lane >> 5;
    const bool token_wave = wave >= 4;   // loads the token tile; waves 0..3 load codes and scales

    // Workgroup b takes K range b % n_splits of tile b / n_splits (in the
    // XCD-contiguous order): steps s0 .. s0 + steps - 1 of K.  Offsets below
    // are relative to s0; nblk counts the 32-blocks of K from block 2 s0 on.
    if constexpr (!BATCH) {
        // issue every scalar argument load of a single product at once
        asm volatile("" ::"s"(a.K), "s"(a.qoff), "s"(a.N), "s"(a.n_tiles), "s"(a.n_splits), "s"(a.split_steps),
                     "s"(a.split_stride), "s"(a.item[0].w), "s"(a.item[0].pitch), "s"(a.item[0].M),
                     "s"(a.item[0].x), "s"(a.item[0].x_pitch), "s"(a.item[0].y), "s"(a.item[0].y_pitch),
                     "s"(a.item[0].tile_begin));
    }
    const int wgi = xcd_order_index();
    const int split = __builtin_amdgcn_readfirstlane(wgi % a.n_splits);
    const int btile = __builtin_amdgcn_readfirstlane(wgi / a.n_splits);
    int item = 0;
    if constexpr (BATCH) {
        for (int i = 1; i < a.n_items; ++i)
            if (btile >= a.item[i].tile_begin) item = i;
    }
    const GemmItem &itm = a.item[item];
    const uint64_t pitch = itm.pitch;
    const int64_t M = itm.M;
    const uint64_t x_pitch = itm.x_pitch;
    const uint64_t y_pitch = itm.y_pitch;
    const int tile = btile - itm.tile_begin;
    const int mt = __builtin_amdgcn_readfirstlane(tile / a.n_tiles);
    const int nt = __builtin_amdgcn_readfirstlane(tile - mt * a.n_tiles);
    constexpr int MROWS = SW ? BM / 2 : BM;     // matrix rows per tile
    const int64_t m0 = (int64_t)mt * MROWS;
    const int64_t n0 = (int64_t)nt * BN;
    const int s0 = split * a.split_steps;
    const int64_t nblk = a.K / 32 - 2 * (int64_t)s0;
    const int all_steps = (int)((a.K + 63) / 64);
    const int steps = all_steps - s0 < a.split_steps ? all_steps - s0 : a.split_steps;
    float *const out = itm.y + (uint64_t)split * a.split_stride;

    // ---- loads (token waves) ----
    // Load i of a step covers tokens 8 ti .. 8 ti + 7 (ti = 4 (wave - 4) + i),
    // 8 lanes per token; lane slot e holds the token's 16-byte chunk
    // e ^ ((token >> 1) & 7) of the step.  Tokens past N read zeros (their
    // lane offset is beyond the buffer).  Steps wholly inside K and the range
    // take their step offset as a scalar (no per-lane work); the others
    // check each chunk against K and read zeros past it.
    const int64_t toks = a.N - n0 < BN ? a.N - n0 : BN;
    const i32x4 xres = buffer_rsrc(itm.x + (uint64_t)n0 * x_pitch, (uint32_t)(((toks - 1) * x_pitch + a.K) * 2));
    const int tw = token_wave ? wave - 4 : 0;
    const int64_t kr = a.K - 64 * (int64_t)s0 < 64 * (int64_t)steps ? a.K - 64 * (int64_t)s0 : 64 * (int64_t)steps;
    const int full_steps = (int)(kr / 64);       // steps whose 64 k are all in K and in the range
    uint32_t xoff[TOK_LOADS];
    int xlim[TOK_LOADS];
#pragma unroll
    for (int i = 0; i < TOK_LOADS; ++i) {
        const int tok = 8 * (TOK_LOADS * tw + i) + (lane >> 3);
        const int q = (lane & 7) ^ ((tok >> 1) & 7);
        xoff[i] = (uint32_t)(tok * x_pitch * 2) + 16u * q + 128u * s0;
        xlim[i] = (int)(kr - 8 * q);              // chunk q of step s is in K iff 64 s < xlim
    }
    // FAST: step s is known to be < full_steps
    auto token_load = [&](auto FAST, int i, int s, int stage) {
        const uint32_t dst = lds0 + (uint32_t)(stage * TOK_BYTES) + 1024u * (TOK_LOADS * tw + i);
        if constexpr (decltype(FAST)::value) lds_load16s(xres, dst, xoff[i], 128u * s);
        else lds_load16(xres, dst, 64 * s < xlim[i] ? xoff[i] + 128u * s : OUT_OF_RANGE);
    };

    // ---- loads (code waves) ----
    // Codes: load i covers rows 8 ci .. 8 ci + 7 (ci = 4 wave + i), 8 lanes
    // per row; lane slot e of a row holds its 16-byte unit e ^ ((row >> 1) & 7)
    // of the group.  Scales: 16 bytes per row and group (the group's 2 GS
    // scales, or GS with 64-weight blocks; the rest of the 16 bytes reads
    // zeros), 4 lanes per row, 16 rows per load.  Rows past M read zeros;
    // groups wholly in K and the range take a scalar offset, the last
    // partial one checks each lane, and groups past it read zeros.
    const int64_t rows = M - m0 < MROWS ? M - m0 : MROWS;
    const int64_t qoff = WT == W_F16 ? 0 : a.qoff;  // F16 rows hold no scales
    const uint32_t row_bytes = (uint32_t)(qoff + (a.K / 32) * QB);
    const int cw = token_wave ? 0 : wave;
    // fused SwiGLU: code waves 2, 3 load the up matrix into tile rows 64..127
    const bool upper = SW && cw >= 2;
    const uint8_t *const wm = upper ? itm.w2 : itm.w;
    const uint64_t pm = upper ? itm.pitch2 : pitch;
    const int lrow = upper ? BM / 2 : 0;        // tile row of the matrix's row m0
    const i32x4 wres = buffer_rsrc(wm + (uint64_t)m0 * pm, (uint32_t)((rows - 1) * pm + row_bytes));
    const int64_t nblk_r = nblk < 2 * (int64_t)steps ? nblk : 2 * (int64_t)steps;   // blocks of the range
    const int full_groups = (int)(nblk_r / (2 * GS));
    uint32_t coff[CODE_LOADS];
#pragma unroll
    for (int i = 0; i < CODE_LOADS; ++i) {
        const int row = 8 * (CODE_LOADS * cw + i) + (lane >> 3);
        const int unit = (lane & 7) ^ ((row >> 1) & 7);
        coff[i] = (uint32_t)((row - lrow) * pm + qoff) + (uint32_t)(2 * s0 * QB) + 16u * unit;
    }
    constexpr int SPG = (2 * GS) >> SS;          // scales per row and group
    uint32_t soff[SCALE_LOADS];
    const int sdw = lane & 3;
#pragma unroll
    for (int i = 0; i < SCALE_LOADS; ++i) {
        const int row = 16 * (SCALE_LOADS * cw + i) + (lane >> 2);
        // dwords past the group's scales read zeros in every group
        soff[i] = 2 * sdw < SPG ? (uint32_t)((row - lrow) * pm) + 2u * (uint32_t)((2 * s0) >> SS) + 4u * sdw : OUT_OF_RANGE;
    }
    const int64_t nscales = nblk_r >> SS;        // scales of the range
    // FAST: group g is known to be < full_groups
    auto code_load = [&](auto FAST, int i, int g) {
        const uint32_t dst = lds0 + LDS_GROUP_OFF + (uint32_t)((g % NB) * GROUP_BYTES) + 1024u * (CODE_LOADS * cw + i);
        if constexpr (decltype(FAST)::value) lds_load16s(wres, dst, coff[i], 128u * g);
        else lds_load16(wres, dst, 2 * GS * (int64_t)g < nblk_r ? coff[i] + 128u * g : OUT_OF_RANGE);
    };
    auto scale_load = [&](auto FAST, int i, int g) {
        const uint32_t dst = lds0 + LDS_SCALE_OFF + (uint32_t)((g % NB) * SGROUP_BYTES) + 256u * (SCALE_LOADS * cw + i);
        if constexpr (decltype(FAST)::value) lds_load4s(wres, dst, soff[i], 2u * SPG * g);
        else lds_load4(wres, dst, (int64_t)SPG * g + 2 * sdw < nscales ? soff[i] + 2u * SPG * g : OUT_OF_RANGE);
    };
    auto issue_group = [&](int g) {
#pragma unroll
        for (int i = 0; i < CODE_LOADS; ++i) code_load(std::false_type{}, i, g);
        if constexpr (Sc::SCALES) {
#pragma unroll
            for (int i = 0; i < SCALE_LOADS; ++i) scale_load(std::false_type{}, i, g);
        }
    };

    // ---- LDS reads ----
    // B fragment lane (row rl, half h); A fragment lane (token 32 j + lane % 32, half h).
    const int rl = 32 * rg + (lane & 31);
    // The lane's weights of block bi = 2 u + par: Q4_0 8 bytes of unit bi;
    // Q8_0 8 bytes of each of units 2 bi (chunk 0) and 2 bi + 1 (chunk 1);
    // F16 units 4 bi + h (chunk 0) and 4 bi + 2 + h (chunk 1), whole.
    constexpr int CR = QB == 16 ? 1 : 2;
    uint32_t crd[GS][CR];         // code offsets (within a group buffer) of block 2 u + par
    uint32_t srd[GS];             // scale offsets
#pragma unroll
    for (int u = 0; u < GS; ++u) {
        const int bi = 2 * u + par;
#pragma unroll
        for (int c = 0; c < CR; ++c) {
            const int unit = WT == W_F16 ? 4 * bi + 2 * c + h : (QB / 16) * bi + c;
            crd[u][c] = (uint32_t)(rl * 128 + 16 * (unit ^ ((rl >> 1) & 7)) + (WT == W_F16 ? 0 : 8 * h));
        }
        srd[u] = (uint32_t)(rl * 16 + 2 * (bi >> SS));
    }
    uint32_t trd[4][2];           // token offsets (within a stage) of tile j, chunk c
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int tok = 32 * j + (lane & 31);
            const int q = 4 * par + 2 * c + h;
            trd[j][c] = (uint32_t)(tok * 128 + 16 * (q ^ ((tok >> 1) & 7)));
        }

    f32x16 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
    bf16x8 A[2][4][2];            // token fragments of steps t and t + 1
    uint32_t B[2][8];             // weight fragments of steps t and t + 1
    using Raw = RawOf<WT>;
    Raw R[2];                     // raw codes and scale of steps t + 1 and t + 2 (by step parity)
    Deq<WT> dq;
    const int nblk32 = (int)(nblk < 0x40000000 ? nblk : 0x40000000);

    auto tok_frag = [&](int stage, int j, int c) {
        return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(lds + stage * TOK_BYTES + trd[j][c]));
    };
    // the raw codes and scale of relative step s (static position u = s % GS)
    auto raw_weights = [&](auto U, int s) {
        constexpr int u = decltype(U)::value;
        const int gb = (s / GS) % NB;
        const uint8_t *cg = lds + LDS_GROUP_OFF + gb * GROUP_BYTES;
        Raw r;
        if constexpr (WT == W_F16) {
            r.c0 = *reinterpret_cast<const u32x4 *>(cg + crd[u][0]);
            r.c1 = *reinterpret_cast<const u32x4 *>(cg + crd[u][1]);
        } else {
            r.sbits = *reinterpret_cast<const uint16_t *>(lds + LDS_SCALE_OFF + gb * SGROUP_BYTES + srd[u]);
            r.c0 = *reinterpret_cast<const u32x2 *>(cg + crd[u][0]);
            r.c1 = QB == 32 ? *reinterpret_cast<const u32x2 *>(cg + crd[u][CR - 1]) : r.c0;
        }
        return r;
    };
    // part P of the unpacking of step s from r into b (a block past K gets
    // a zero scale: its codes may be anything)
    auto dequant_part = [&](auto P, const Raw &r, int s, uint32_t (&b)[8]) {
        constexpr int p = decltype(P)::value;
        const bool live = 2 * s + par < nblk32;
        if constexpr (WT == W_Q4_0) dq.template part<p>(r.c0, r.sbits, live, b);
        else if constexpr (WT == W_Q8_0) dq.template part<p>(r.c0, r.c1, r.sbits, live, b);
        else dq.template part<p>(r.c0, r.c1, live, b);
    };
    auto bfrag = [](const uint32_t (&b)[8], int c) {
        return __builtin_bit_cast(bf16x8, u32x4{b[4 * c], b[4 * c + 1], b[4 * c + 2], b[4 * c + 3]});
    };

    // ---- prologue: token steps 0 .. DT-1 and code groups 0 .. PRO-1 in
    // flight; step 0 in registers, the raw codes of step 1 too ----
    if (token_wave) {
#pragma unroll
        for (int s = 0; s < DT; ++s)
#pragma unroll
            for (int i = 0; i < TOK_LOADS; ++i) token_load(std::false_type{}, i, s, s);
        wait_vm<TOK_LOADS * (DT - 1)>();
    } else {
#pragma unroll
        for (int g = 0; g < Sc::PRO; ++g) issue_group(g);
        wait_vm<Sc::LOADS * (Sc::PRO - Sc::PRO_READ)>();
    }
    asm volatile("s_barrier" ::: "memory");
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int c = 0; c < 2; ++c) A[0][j][c] = tok_frag(0, j, c);
    R[0] = raw_weights(std::integral_constant<int, 0>{}, 0);
    R[1] = raw_weights(std::integral_constant<int, 1 % GS>{}, 1);
    static_for<8>([&](auto P) { dequant_part(P, R[0], 0, B[0]); });

    // ---- main loop ----
    // Iteration t multiplies step t (registers) while it reads the token
    // fragments of step t + 1 and the raw codes of step t + 2 from LDS into
    // the other register sets, unpacks step t + 1, and issues this wave's
    // loads: one fragment read, at most one load and an eighth of the
    // unpacking per matrix instruction, so that the two waves of a SIMD keep
    // its matrix core busy while the other one's VALU and LDS work issues.
    // One straight-line copy per load role.
    int rd_stage = 1;             // token stage of step t + 1
    int ld_stage = DT;            // token stage of step t + DT
    // A straight-line copy covers UF iterations, a multiple of GS (the
    // position in the code group is static) and of 2 (so is the register
    // set of each step).
    constexpr int UF = GS % 2 == 0 ? GS : 2 * GS;
    // iterations t0 .. t1 - 1 (t0 a multiple of UF) of one load role, with
    // FAST loads (every load issued wholly in K and the range)
    auto main_loop = [&](auto TW, auto FAST, int t0, int t1) {
        constexpr bool tokw = decltype(TW)::value;
        // the fast runs are whole multiples of UF iterations: no per-step
        // bound check (each one a branch between matrix instructions)
        constexpr bool guard = !decltype(FAST)::value;
        for (; t0 < t1; t0 += UF) {
            static_for<UF>([&](auto U) {
                constexpr int u = decltype(U)::value;
                const int t = t0 + u;
                if (!guard || t < t1) {
                    // this wave's loads for the token stage of step t + 1 and
                    // the code group of step t + 2 have landed; after the
                    // barrier, every wave's have, and the token stage of step
                    // t - 1 and a group buffer last read in iteration t - 1
                    // are free
                    if constexpr (tokw) wait_vm<TOK_LOADS * (DT - 2)>();
                    else wait_vm<Sc::pending(u % GS)>();
                    asm volatile("s_barrier" ::: "memory");
                    constexpr bool group_now = (u + DC) % GS == 0;
                    const int g = (t + DC) / GS;
                    const uint32_t(&bc)[8] = B[u & 1];
                    uint32_t(&bn)[8] = B[(u + 1) & 1];
                    bf16x8(&Ac)[4][2] = A[u & 1];
                    bf16x8(&An)[4][2] = A[(u + 1) & 1];
                    const Raw &rc = R[(u + 1) & 1];       // step t + 1
                    Raw &rn = R[u & 1];                   // step t + 2
                    rn = raw_weights(std::integral_constant<int, (u + 2) % GS>{}, t + 2);
                    __builtin_amdgcn_sched_barrier(0);
                    static_for<8>([&](auto K) {
                        constexpr int k = decltype(K)::value, c = k / 4, j = k % 4;
                        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Ac[j][c], bfrag(bc, c), acc[j], 0, 0, 0);
                        An[j][c] = tok_frag(rd_stage, j, c);
                        if constexpr (tokw) {
                            if constexpr (k < TOK_LOADS) token_load(FAST, k, t + DT, ld_stage);
                        } else if constexpr (group_now) {
                            if constexpr (k < CODE_LOADS) code_load(FAST, k, g);
                            else if constexpr (Sc::SCALES && k < CODE_LOADS + SCALE_LOADS)
                                scale_load(FAST, k - CODE_LOADS, g);
                        }
                        dequant_part(K, rc, t + 1, bn);
                        // keep this order: matrix instruction, its fragment
                        // read, the load, the unpacking share
                        __builtin_amdgcn_sched_barrier(0);
                    });
                    ld_stage = ld_stage + 1 == TS ? 0 : ld_stage + 1;
                    rd_stage = rd_stage + 1 == TS ? 0 : rd_stage + 1;
                }
            });
        }
    };
    // Fast iterations while every load they issue is wholly in K and the
    // range (token waves: step t + DT < full_steps; code waves: group
    // (t + DC) / GS < full_groups), then the rest with per-lane checks.
    if (token_wave) {
        int tf = full_steps - DT;
        tf = tf < 0 ? 0 : (tf > steps ? steps : tf) / UF * UF;
        main_loop(std::true_type{}, std::true_type{}, 0, tf);
        main_loop(std::true_type{}, std::false_type{}, tf, steps);
    } else {
        int tf = GS * full_groups - DC;
        tf = tf < 0 ? 0 : (tf > steps ? steps : tf) / UF * UF;
        main_loop(std::false_type{}, std::true_type{}, 0, tf);
        main_loop(std::false_type{}, std::false_type{}, tf, steps);
    }

    // ---- the two waves of a SIMD add their sums; each stores two token tiles ----
    wait_vm<0>();                 // no load may still write the ring
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    float *xch = reinterpret_cast<float *>(lds);       // [wave][2][16][64]
    const int give = par == 0 ? 2 : 0;
    const int keep = 2 - give;
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int r = 0; r < 16; ++r) xch[((wave * 2 + jj) * 16 + r) * 64 + lane] = acc[give + jj][r];
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const float *other = xch + (wave ^ 4) * 2 * 16 * 64;
    float fin[2][16];             // the sums of token sub-tiles keep, keep + 1
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int r = 0; r < 16; ++r) fin[jj][r] = acc[keep + jj][r] + other[(jj * 16 + r) * 64 + lane];
    auto token = [&](int jj, int r) { return n0 + 32 * (keep + jj) + 8 * (r / 4) + 4 * h + (r % 4); };
    // Outputs go out as streaming (non-temporal) stores: every tile writes
    // its 64 KB at the same moment at the end, and ordinary stores would
    // first fill the L2 with lines that only have to be written back (on
    // the box ~1 us less per 5632 x 2048 x 512 launch; no slower for the
    // partial sums of a K split, which the slab sum reads back next).
    auto store = [&](float *p, float v) { __builtin_nontemporal_store(v, p); };
    if constexpr (SW) {
        // Gate row group g (0, 1) and up row group g + 2 hold the same matrix
        // rows and, for the same parity, the same tokens.  Each hands the
        // other one token sub-tile through LDS and finishes the other one:
        // the gate wave sub-tile keep, the up wave sub-tile keep + 1.
        const bool gate = rg < 2;
        float *sw = reinterpret_cast<float *>(lds) + 8 * 2 * 16 * 64;     // [wave][16][64], after xch
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
        for (int r = 0; r < 16; ++r) sw[(wave * 16 + r) * 64 + lane] = fin[gate ? 1 : 0][r];
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        const float *mate = sw + (wave ^ 2) * 16 * 64;               // row group rg ^ 2, same parity
        const int jj = gate ? 0 : 1;
        const int64_t m = m0 + 32 * (rg & 1) + (lane & 31);
        if (m < M) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float g = gate ? fin[0][r] : mate[r * 64 + lane];
                const float u = gate ? mate[r * 64 + lane] : fin[1][r];
                const int64_t n = token(jj, r);
                if (n < a.N) store(out + (uint64_t)n * y_pitch + m, swish(g) * u);
            }
        }
        return;
    }
    const int64_t m = m0 + rl;
    if (m < M) {
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t n = token(jj, r);
                if (n < a.N) store(out + (uint64_t)n * y_pitch + m, fin[jj][r]);
            }
    }
}

template <int WT, int SS, bool BATCH, bool SW>
hipError_t launch_rq(const GemmArgs &a, unsigned blocks, hipStream_t stream)
{
    constexpr int bytes = LDS_BYTES;
    const hipError_t e = allow_dynamic_lds(reinterpret_cast<const void *>(&gemm_rq_kernel<WT, SS, BATCH, SW>), bytes);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gemm_rq_kernel<WT, SS, BATCH, SW>), dim3(blocks), dim3(THREADS), bytes, stream, a);
    return hipGetLastError();
}
template <int WT, int SS>
hipError_t launch_rq(const GemmArgs &a, unsigned blocks, bool sw, hipStream_t stream)
{
    if (sw) return launch_rq<WT, SS, false, true>(a, blocks, stream);
    return a.n_items > 1 ? launch_rq<WT, SS, true, false>(a, blocks, stream)
                         : launch_rq<WT, SS, false, false>(a, blocks, stream);
}

}  // namespace

bool gemm_rq_handles(int type)
{
    return type == W_Q4_0 || type == W_Q8_0 || type == W_F16;
}

hipError_t launch_gemm_rq(const GemmArgs &a, unsigned blocks, int type, int ss, bool sw, hipStream_t stream)
{
    if (type == W_Q4_0) return ss ? launch_rq<W_Q4_0, 1>(a, blocks, sw, stream) : launch_rq<W_Q4_0, 0>(a, blocks, sw, stream);
    if (type == W_Q8_0) return ss ? launch_rq<W_Q8_0, 1>(a, blocks, sw, stream) : launch_rq<W_Q8_0, 0>(a, blocks, sw, stream);
    if (type == W_F16 && !ss) return launch_rq<W_F16, 0>(a, blocks, sw, stream);
    return hipErrorInvalidValue;
}

}  // namespace qmm
