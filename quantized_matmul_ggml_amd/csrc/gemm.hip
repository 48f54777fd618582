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
// The workgroup is split by role.  Of its eight waves, four (one per SIMD)
// only read LDS and issue matrix-core instructions; the other four (again one
// per SIMD) only load from memory, dequantize and write LDS.  Each SIMD thus
// holds one wave of each kind, so the dequantization arithmetic of one wave
// issues while the other wave's matrix instructions run.  The producers keep
// DEPTH steps of global loads in flight in registers, and LDS holds a ring of
// three K-steps: while the consumers work on step t (and read the first
// fragments of step t+1), the producers fill step t+2.  One barrier per step.
//
// Tile: 128 weight rows x 128 tokens, K advancing 64 (two 32-blocks) per step;
// each consumer wave owns 64 x 64 of the output (2 x 2 MFMA tiles of 32 x 32).
// Tokens sit on the MFMA row side so that each lane's results run along the
// contiguous m dimension of Y.  Loads go through buffer resources based at
// the tile's first row, so rows and tokens past the end read as zero.
#include "qmm_internal.h"

namespace qmm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128;                   // weight rows per tile
constexpr int BN = 128;                   // tokens per tile
constexpr int BK = 64;                    // K per step (two 32-blocks)
constexpr int LDS_STRIDE = BK + 8;        // bf16 elements per LDS row (+16 B pad)
constexpr int OPERAND_ELEMS = 128 * LDS_STRIDE;
constexpr int STAGES = 3;
constexpr int DEPTH = 4;                  // K-steps of global loads in flight
constexpr int THREADS = 512;
constexpr int BUFFER_FLAGS = 0x00020000;  // raw buffer, 32-bit data format

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
    int m_tiles;
    int n_tiles;
    int xcd_chunk;          // tiles per XCD when the tile count divides by 8, else 0
};

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Round two floats to bf16 (nearest even) in one v_cvt_pk_bf16_f32.
__device__ inline uint32_t pack_bf16(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// Byte E of w as a float (v_cvt_f32_ubyteE); written out because the
// compiler otherwise turns mask-then-convert into one bit-field extract per
// value.
template <int E>
__device__ inline float ubyte(uint32_t w)
{
    float r;
    if constexpr (E == 0) asm("v_cvt_f32_ubyte0 %0, %1" : "=v"(r) : "v"(w));
    else if constexpr (E == 1) asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(r) : "v"(w));
    else if constexpr (E == 2) asm("v_cvt_f32_ubyte2 %0, %1" : "=v"(r) : "v"(w));
    else asm("v_cvt_f32_ubyte3 %0, %1" : "=v"(r) : "v"(w));
    return r;
}

// One producer lane's share of a K-step: one 32-block of one weight row
// (codes and scale) and 32 activations of one token.
template <int WT>
struct Stage {
    static constexpr int QV = (WT == W_Q4_0) ? 1 : 2;
    u32x4 q[QV];
    uint16_t s;
    u32x4 x[4];
};

// Dequantize one 32-block to 32 bf16 values in k order, two per dword.
// (code - offset) * d is exact in fp32 (at most 19 significant bits), so each
// value is the bf16 rounding of the exact product.
template <int WT>
__device__ inline void dequant_block(const Stage<WT> &st, uint32_t out[16])
{
    const float d = (float)__builtin_bit_cast(_Float16, st.s);
    if constexpr (WT == W_Q4_0) {
        const float nd = -8.0f * d;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t lo = st.q[0][i] & 0x0F0F0F0Fu;          // codes k = 4i .. 4i+3
            const uint32_t hi = (st.q[0][i] >> 4) & 0x0F0F0F0Fu;   // codes k = 16+4i ..
            out[2 * i] = pack_bf16(fmaf(ubyte<0>(lo), d, nd), fmaf(ubyte<1>(lo), d, nd));
            out[2 * i + 1] = pack_bf16(fmaf(ubyte<2>(lo), d, nd), fmaf(ubyte<3>(lo), d, nd));
            out[8 + 2 * i] = pack_bf16(fmaf(ubyte<0>(hi), d, nd), fmaf(ubyte<1>(hi), d, nd));
            out[8 + 2 * i + 1] = pack_bf16(fmaf(ubyte<2>(hi), d, nd), fmaf(ubyte<3>(hi), d, nd));
        }
    } else {
        const float nd = -128.0f * d;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t u = st.q[i / 4][i % 4] ^ 0x80808080u;   // int8 + 128
            out[2 * i] = pack_bf16(fmaf(ubyte<0>(u), d, nd), fmaf(ubyte<1>(u), d, nd));
            out[2 * i + 1] = pack_bf16(fmaf(ubyte<2>(u), d, nd), fmaf(ubyte<3>(u), d, nd));
        }
    }
}

template <int WT>
__global__ __launch_bounds__(THREADS) void gemm_kernel(const GemmArgs a)
{
    constexpr int QB = (WT == W_Q4_0) ? 16 : 32;     // code bytes per block
    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
    // stage s: weights at lds + s * 2 * OPERAND_ELEMS, tokens right after

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    int tile = blockIdx.x;
    if (a.xcd_chunk) tile = (tile % 8) * a.xcd_chunk + tile / 8;
    // the division runs on the vector unit; the tile is uniform, so move it
    // back to scalar registers (buffer resources must live there)
    const int mt = __builtin_amdgcn_readfirstlane(tile / a.n_tiles);
    const int nt = __builtin_amdgcn_readfirstlane(tile - mt * a.n_tiles);
    const int64_t m0 = (int64_t)mt * BM;
    const int64_t n0 = (int64_t)nt * BN;
    const int64_t nblk = a.K / 32;
    const int steps = (int)((a.K + BK - 1) / BK);

    if (wave >= 4) {
        // ---------------- producers ----------------
        const int p = tid - 256;
        const int prow = p >> 1;           // weight row / token of this lane
        const int phalf = p & 1;           // which 32-block of the step
        const int64_t rows = a.M - m0 < BM ? a.M - m0 : BM;
        const int64_t toks = a.N - n0 < BN ? a.N - n0 : BN;
        // Buffer sizes are the bytes the operands really span, so an offset
        // past them reads zeros without touching memory.  All offsets go in
        // the VGPR operand, which the range check covers.
        const uint32_t row_bytes = (uint32_t)(a.qoff + (WT == W_Q4_0 ? a.K / 2 : a.K));
        const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(a.w + (uint64_t)m0 * a.pitch), 0,
            (int)(uint32_t)((rows - 1) * a.pitch + row_bytes), BUFFER_FLAGS);
        const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(a.x + (uint64_t)n0 * a.x_pitch), 0,
            (int)(uint32_t)(((toks - 1) * a.x_pitch + a.K) * 2), BUFFER_FLAGS);
        constexpr uint32_t OUT_OF_RANGE = 0x80000000u;   // above every buffer size
        const uint32_t qoff = (uint32_t)(prow * a.pitch + a.qoff) + phalf * QB;
        const uint32_t soff = (uint32_t)(prow * a.pitch) + phalf * 2;
        const uint32_t xoff = (uint32_t)(prow * a.x_pitch * 2) + phalf * 64;

        Stage<WT> ring[DEPTH];
        // Blocks past the end of K (the second block of the last step when
        // K/32 is odd) are loaded from an out-of-range offset and so are zero:
        // zero scale, zero activations.
        auto load = [&](Stage<WT> &st, int t) {
            const bool in_k = 2 * t + phalf < nblk;
            const uint32_t oq = in_k ? qoff + (uint32_t)t * (2 * QB) : OUT_OF_RANGE;
            const uint32_t os = in_k ? soff + (uint32_t)t * 4 : OUT_OF_RANGE;
            const uint32_t ox = in_k ? xoff + (uint32_t)t * 128 : OUT_OF_RANGE;
#pragma unroll
            for (int v = 0; v < Stage<WT>::QV; ++v)
                st.q[v] = __builtin_amdgcn_raw_buffer_load_b128(wres, oq + 16 * v, 0, 0);
            st.s = __builtin_amdgcn_raw_buffer_load_b16(wres, os, 0, 0);
#pragma unroll
            for (int v = 0; v < 4; ++v)
                st.x[v] = __builtin_amdgcn_raw_buffer_load_b128(xres, ox + 16 * v, 0, 0);
        };
        auto store = [&](const Stage<WT> &st, int t) {
            uint32_t deq[16];
            dequant_block<WT>(st, deq);
            uint16_t *ws = lds + (t % STAGES) * 2 * OPERAND_ELEMS;
            u32x4 *wdst = reinterpret_cast<u32x4 *>(ws + prow * LDS_STRIDE + 32 * phalf);
#pragma unroll
            for (int v = 0; v < 4; ++v)
                wdst[v] = u32x4{deq[4 * v], deq[4 * v + 1], deq[4 * v + 2], deq[4 * v + 3]};
            u32x4 *xdst = reinterpret_cast<u32x4 *>(ws + OPERAND_ELEMS + prow * LDS_STRIDE + 32 * phalf);
#pragma unroll
            for (int v = 0; v < 4; ++v) xdst[v] = st.x[v];
        };

        // Loads are unconditional (those past the last step read zeros) so
        // that the number in flight is the same on every path and each wait
        // is for one step's loads only.  Step p lives in ring slot p % DEPTH
        // and LDS stage p % STAGES; producing step p (p >= 1) ends with the
        // barrier that releases step p - 1 to the consumers.
#pragma unroll
        for (int j = 0; j < DEPTH; ++j) load(ring[j], j);
        for (int p0 = 0; p0 < steps; p0 += DEPTH) {
#pragma unroll
            for (int u = 0; u < DEPTH; ++u) {
                const int p = p0 + u;
                if (p < steps) store(ring[u], p);
                load(ring[u], p + DEPTH);
                if (p >= 1 && p < steps) __syncthreads();
            }
        }
        // the consumers' last two barriers
        __syncthreads();
        __syncthreads();
        return;
    }

    // ---------------- consumers ----------------
    const int wm = wave & 1;     // weight-row half of the tile
    const int wn = wave >> 1;    // token half of the tile
    const int frow = lane & 31;         // row of the MFMA operand this lane feeds
    const int fk = (lane >> 5) * 8;     // its 8-element k group
    const int a_off = OPERAND_ELEMS + (wn * 64 + frow) * LDS_STRIDE + fk;
    const int b_off = (wm * 64 + frow) * LDS_STRIDE + fk;

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    auto read_frags = [&](int stage, int kk, bf16x8 af[2], bf16x8 bf[2]) {
        const uint16_t *base = lds + stage * 2 * OPERAND_ELEMS + kk * 16;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            af[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(base + a_off + i * 32 * LDS_STRIDE));
            bf[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(base + b_off + i * 32 * LDS_STRIDE));
        }
    };

    __syncthreads();
    bf16x8 af[2][2], bf[2][2];          // [parity of kk][sub-tile]
    if (steps > 0) read_frags(0, 0, af[0], bf[0]);
    int stage = 0;
    for (int t = 0; t < steps; ++t) {
        const int next = stage + 1 == STAGES ? 0 : stage + 1;
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int cur = kk & 1;
            if (kk + 1 < BK / 16)
                read_frags(stage, kk + 1, af[cur ^ 1], bf[cur ^ 1]);
            else if (t + 1 < steps)
                read_frags(next, 0, af[cur ^ 1], bf[cur ^ 1]);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cur][i], bf[cur][j], acc[i][j], 0, 0, 0);
        }
        stage = next;
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

constexpr size_t LDS_BYTES = (size_t)STAGES * 2 * OPERAND_ELEMS * sizeof(uint16_t);

template <int WT>
hipError_t launch_typed(const GemmArgs &a, unsigned tiles, hipStream_t stream)
{
    const hipError_t attr = allow_dynamic_lds(reinterpret_cast<const void *>(&gemm_kernel<WT>), (int)LDS_BYTES);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL(gemm_kernel<WT>, dim3(tiles), dim3(THREADS), LDS_BYTES, stream, a);
    return hipGetLastError();
}

}  // namespace

bool gemm_supported(const WeightView &w, const ActView &x)
{
    // buffer offsets within one tile are 32-bit
    return (uint64_t)BM * w.pitch < (1ull << 31) && (uint64_t)BN * x.pitch_elems * 2 < (1ull << 31);
}

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
    a.m_tiles = (int)((w.M + BM - 1) / BM);
    a.n_tiles = (int)((x.N + BN - 1) / BN);
    const unsigned tiles = (unsigned)a.m_tiles * (unsigned)a.n_tiles;
    // Consecutive tiles share a weight row band; handing each XCD (which
    // receives every eighth workgroup) a contiguous run keeps a band's
    // weights in one L2.
    a.xcd_chunk = tiles % 8 == 0 ? (int)(tiles / 8) : 0;
    if (w.type == W_Q4_0) return launch_typed<W_Q4_0>(a, tiles, stream);
    if (w.type == W_Q8_0) return launch_typed<W_Q8_0>(a, tiles, stream);
    return hipErrorInvalidValue;
}

}  // namespace qmm
