// gemv.hip -- decode GEMV / skinny GEMM over Q4_0, Q8_0 and F16 weight rows.
//
// y[n][m] = sum_k W'[m][k] * x[n][k] for 1 <= N <= 8 tokens of fp32
// activations.  With one token per step every projection is a GEMV and the
// run time is the time to stream the weights from HBM (A Complete Guide to
// llama.cpp and Customization with C++, §2.1; No Python! Building an AI
// Inference Engine Exclusively in C++, §9: read the compressed weights and
// expand them in registers).  The per-weight work follows the Development
// Guide for Small AI Models (TinyLLaMA, etc.) Using C++, §6.2: load the packed
// codes, unpack them with masks and shifts, apply the block scale, multiply-add
// with the activations.
//
// Mapping onto gfx950:
//  * A row's code bytes are cut into 16-byte chunks (one Q4_0 block, half a
//    Q8_0 block, eight F16 weights).  A "wave group" of KS waves (64*KS
//    lanes) owns a row; lane v takes chunks v, v + 64*KS, ... so every load
//    instruction of a wave reads 64 consecutive chunks (1 KiB, 128-bit per
//    lane, fully coalesced).
//  * The activations a lane needs for its chunks are loaded once into VGPRs
//    and reused for every row the wave streams; only weights come from HBM.
//  * Codes are unpacked to their signed values (Q4_0: nibble - 8; Q8_0: the
//    int8 code) before they meet the activations, so every product is an
//    exact dequantized code times x and the accumulation error is relative to
//    sum |code * x|, whatever the codes or activations are.  The block scale
//    is applied once per chunk: sum_i d*q_i*x_i = d*(sum_i q_i*x_i)
//    (A Complete Guide to llama.cpp ..., §2.2: the scale factors out of the
//    block's dot product).
//  * U rows x NT tokens partial sums per lane are reduced across the wave by
//    a transposed butterfly (each exchange halves the set of values a lane
//    carries), then across the KS waves of a group through LDS.
//  * The next row group's loads are issued before the current one is
//    reduced, so each wave keeps U*CPL 128-bit loads in flight.
#include "qmm_internal.h"
#include "wave_reduce.h"

#include <type_traits>

namespace qmm {
namespace {

// Persistent grid: at most 8 four-wave workgroups per CU when a wave owns
// whole rows, 4 when rows span several waves (measured: the larger grid
// helps the former and costs the Q8_0 LM head at 2 and 4 tokens 5-7 %); the
// same number of waves with sixteen-wave workgroups.
inline int max_workgroups(int ks, int wgw) { return (ks == 1 ? 2048 : 1024) * 4 / wgw; }
// Every workgroup stages all K activations of its tokens, so rows longer than
// 4096 take a smaller grid, each workgroup streaming more rows per staging
// (measured on 2048 x 5632 Q4_0: 3 / 4 tokens 10.2 / 11.2 us with the full
// grid, 8.2 / 8.8 us with 512 workgroups, slower again with 384 or 256; at
// one token, graph-replayed: 4096 x 11008 12.5 -> 10.5 us, 4096 x 8192 7.1
// -> 6.7, 8192 x 8192 10.9 -> 10.4, 11008 x 5632 12.4 -> 12.2, 2048 x 5632
// unchanged at 4.2).
inline int max_workgroups(int ks, int wgw, int64_t K)
{
    const int cap = max_workgroups(ks, wgw);
    return (K > 4096 && cap > 512) ? 512 : cap;
}
constexpr int kMaxItems = QMM_GEMV_BATCH_MAX;

// One GEMV of a launch: its weights, activations and outputs.  All items of
// a launch share the weight type, K and the token count.  An item is one
// 64-byte record, and the fields shared by all items sit in the first 64
// bytes of the arguments, so a wave fetches everything it needs in one round
// trip to the kernel arguments (each trip costs a few hundred nanoseconds).
struct alignas(64) GemvItem {
    const uint8_t *w;
    const float *x;
    float *y;
    const uint8_t *w2;    // fused SwiGLU launches: the up projection (w is the gate)
    uint32_t pitch;       // bytes between weight rows (<= 2^28)
    uint32_t pitch2;      // the same for w2
    uint32_t x_pitch;     // elements between token rows of x
    uint32_t y_pitch;     // elements between token rows of y
    int32_t M;
    int32_t n_groups;     // row groups (U rows, or U/2 row indices of each matrix when fused)
    int32_t wg_count;     // workgroups of this item (grid x; grid y indexes the item)
    int32_t iters;        // row-group iterations of each wave group
};
static_assert(sizeof(GemvItem) == 64, "one 64-byte record per item");

struct GemvArgs {
    int32_t N;            // real tokens (<= NT)
    int32_t K;
    int32_t qoff;         // byte offset of the codes inside a row (0 for F16)
    int32_t nchunk;       // 16-byte chunks of codes per row
    int32_t n_items;
    int32_t scale_shift;  // 1: one scale per two 32-weight runs (64-blocks)
    int32_t pad[10];
    GemvItem item[kMaxItems];
};

// (a & m) | c in one VALU op (the compiler would split it: gfx9 VOP3 takes no
// literal operands, so c has to sit in a register).
__device__ inline uint32_t and_or(uint32_t a, uint32_t m, uint32_t c)
{
    uint32_t d;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "s"(m), "v"(c));
    return d;
}

__device__ inline float lo_half(uint32_t p)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(p & 0xFFFFu));
}
__device__ inline float hi_half(uint32_t p)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(p >> 16));
}

// Weights per 16-byte chunk of codes.
template <int WT> struct Fmt;
template <> struct Fmt<W_Q4_0> { static constexpr int wpc = 32; };
template <> struct Fmt<W_Q8_0> { static constexpr int wpc = 16; };
template <> struct Fmt<W_F16>  { static constexpr int wpc = 8; };

// Weight index (within the row) of element i of chunk c, in the order the
// kernel keeps activations: natural k order.
template <int WT>
__device__ inline int64_t chunk_k(int64_t c, int i)
{
    return c * Fmt<WT>::wpc + i;
}

template <int WT>
__device__ inline int64_t chunk_block(int64_t c)
{
    return WT == W_Q4_0 ? c : c / 2;   // Q8_0: two chunks per 32-block
}

// sum_i q_i * x_i over one chunk with the signed codes q_i.
//  Q4_0: byte j of a block holds element j (low nibble) and j+16 (high
//        nibble).  Under the binary16 exponent of 1024 (0x6400) a nibble n
//        left in bits 0..3 of a half reads 1024 + n and one in bits 4..7
//        reads 1024 + 16 n, so two and-ors per dword (and one shift for the
//        odd bytes) place four codes, and one packed binary16 subtraction
//        per pair makes them n - 8 or 16 (n - 8), exactly (small integers).
//        v_fma_mix_f32 widens each half inside the FMA; the 16 (n - 8)
//        products go to their own accumulator, scaled by 1/16 (exact) at
//        the end.
//  Q8_0: each byte is sign-extended and converted (one SDWA conversion).
//  F16:  the halves of each dword feed v_fma_mix_f32 directly.
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
template <int WT>
__device__ inline float chunk_dot(const uint4 q, const float *xv, uint32_t magic)
{
    const uint32_t wd[4] = {q.x, q.y, q.z, q.w};
    float acc = 0.0f;
    if (WT == W_Q4_0) {
        float acc16 = 0.0f;
        const half2_t off1 = {(_Float16)-1032.0f, (_Float16)-1032.0f};
        const half2_t off16 = {(_Float16)-1152.0f, (_Float16)-1152.0f};
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint32_t w = wd[d];
            const uint32_t w8 = w >> 8;
            const half2_t a = __builtin_bit_cast(half2_t, and_or(w, 0x000F000Fu, magic)) + off1;     // elems 4d,      4d+2
            const half2_t b = __builtin_bit_cast(half2_t, and_or(w, 0x00F000F0u, magic)) + off16;    // elems 16+4d,   16+4d+2
            const half2_t c = __builtin_bit_cast(half2_t, and_or(w8, 0x000F000Fu, magic)) + off1;    // elems 4d+1,    4d+3
            const half2_t e = __builtin_bit_cast(half2_t, and_or(w8, 0x00F000F0u, magic)) + off16;   // elems 16+4d+1, 16+4d+3
            acc = fmaf((float)a.x, xv[4 * d], acc);
            acc = fmaf((float)a.y, xv[4 * d + 2], acc);
            acc = fmaf((float)c.x, xv[4 * d + 1], acc);
            acc = fmaf((float)c.y, xv[4 * d + 3], acc);
            acc16 = fmaf((float)b.x, xv[16 + 4 * d], acc16);
            acc16 = fmaf((float)b.y, xv[16 + 4 * d + 2], acc16);
            acc16 = fmaf((float)e.x, xv[16 + 4 * d + 1], acc16);
            acc16 = fmaf((float)e.y, xv[16 + 4 * d + 3], acc16);
        }
        acc = fmaf(acc16, 0.0625f, acc);
    } else if (WT == W_Q8_0) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                acc = fmaf((float)(int8_t)(wd[d] >> (8 * e)), xv[4 * d + e], acc);
        }
    } else {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            acc = fmaf(lo_half(wd[d]), xv[2 * d], acc);
            acc = fmaf(hi_half(wd[d]), xv[2 * d + 1], acc);
        }
    }
    return acc;
}

// Swish(z) = z * sigma(z) = z / (1 + e^{-z}) in binary32; for z far below
// zero e^{-z} overflows and the quotient is the limit -0.
__device__ inline float swish(float z)
{
    return z / (1.0f + expf(-z));
}

// LDS image of one round of activation chunks: lane-local chunk c holds its
// wpc floats at c * (wpc + 4); the 16-byte pad per chunk spreads the
// lane-strided 128-bit reads of the lanes over all banks.
template <int WT>
__host__ __device__ constexpr int lds_chunk_stride() { return Fmt<WT>::wpc + 4; }

// SWIGLU: the fused gate/up projection with the SwiGLU epilogue
// ("Development Guide for Small AI Models (TinyLLaMA, etc.) Using C++",
// §4.4: h = Swish(x W_gate) * (x W_up), Swish(z) = z sigma(z)).  A group then
// covers U/2 row indices of both matrices: group rows u < U/2 come from the
// gate, rows u >= U/2 from the up projection at the same indices, and after
// the reduction each gate sum meets its up sum in a neighbouring lane.
template <int WT, int NT, int KS, int CPL, int U, bool SWIGLU, int WGW>
__global__ __launch_bounds__(64 * WGW) void gemv_kernel(const GemvArgs a)
{
    constexpr int kThreads = 64 * WGW;
    static_assert(!SWIGLU || U % 2 == 0, "a fused group pairs gate and up rows");
    constexpr int RU = SWIGLU ? U / 2 : U;    // row indices per group
    constexpr int WPC = Fmt<WT>::wpc;
    constexpr int SC = lds_chunk_stride<WT>();
    constexpr int G = WGW / KS;               // wave groups per workgroup
    constexpr int VL = 64 * KS;               // lanes per wave group
    constexpr int V = pow2_ceil(U * NT);      // values per lane to reduce
    static_assert(V <= 64, "too many partial sums per lane");
    extern __shared__ __attribute__((aligned(16))) float xs[];
    __shared__ float red[2][WGW][64];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: keeps group indices scalar
    const int grp = wave / KS;
    const int ks = wave % KS;
    const int v = ks * 64 + lane;

    // ---- this workgroup's item: grid y, so the address of its record is
    // known at wave start.  Every field is fetched before the early exit of
    // a short item's surplus workgroups (the empty asm makes them needed
    // there), so the fetches go out together: one round trip. ----
    const int item = blockIdx.y;
    const GemvItem &itm = a.item[item];
    const uint8_t *const W = itm.w;
    const float *const X = itm.x;
    float *const Y = itm.y;
    const uint8_t *const W2 = itm.w2;
    const uint32_t pitch = itm.pitch;
    const uint32_t pitch2 = itm.pitch2;
    const uint32_t x_pitch = itm.x_pitch;
    const uint32_t y_pitch = itm.y_pitch;
    const int M = itm.M;
    const int n_groups = itm.n_groups;
    const int n_wg = itm.wg_count;
    const int iters = itm.iters;
    const int N = a.N;
    const int K = a.K;
    const int qoff = a.qoff;
    const int nchunk = a.nchunk;
    const int sshift = a.scale_shift;
    asm volatile("" ::"s"(W), "s"(X), "s"(Y), "s"(pitch), "s"(x_pitch), "s"(y_pitch), "s"(M),
                 "s"(n_groups), "s"(n_wg), "s"(iters), "s"(N), "s"(K), "s"(qoff), "s"(nchunk), "s"(sshift));
    if constexpr (SWIGLU) asm volatile("" ::"s"(W2), "s"(pitch2));
    if ((int)blockIdx.x >= n_wg) return;
    const int nt_real = N < NT ? N : NT;

    // ---- row loop bookkeeping: every wave of the workgroup runs the same
    // trip count (the KS > 1 reduction uses workgroup barriers) ----
    int g = (int)blockIdx.x * G + grp;
    const int gstep = n_wg * G;

    // ---- weight loads.  Every load is unconditional: a buffer resource
    // spans the rows of one group, and a lane without a chunk (row tail) or a
    // group past the end reads zeros from an out-of-range offset, so the
    // compiler's wait counts follow one fixed sequence of loads and the
    // activation staging below waits for its own loads only. ----
    const int code_bytes = (WT == W_Q4_0) ? K / 2 : (WT == W_Q8_0 ? K : 2 * K);
    const uint32_t row_bytes = (uint32_t)(qoff + code_bytes);
    // F16 rows whose K is not a multiple of 8 end in a partial chunk: its
    // halves inside the row are loaded one by one (the bytes after them may
    // hold anything), the full chunks as usual.
    const bool f16_tail = WT == W_F16 && (K & 7) != 0;
    uint32_t qoffs[CPL], soffs[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int c = v + j * VL;
        const bool full = (WT == W_F16) ? c * 8 + 8 <= K : c < nchunk;
        qoffs[j] = full ? (uint32_t)(qoff + c * 16) : OUT_OF_RANGE;
        soffs[j] = full ? (uint32_t)(2 * (chunk_block<WT>(c) >> sshift)) : OUT_OF_RANGE;
    }
    auto group_rsrc = [&](int gi, const uint8_t *Wm, uint32_t pm) {
        const int r0 = gi * RU;
        const int rows = gi < n_groups ? (M - r0 < RU ? M - r0 : RU) : 0;
        const uint8_t *base = Wm + (uint64_t)(rows > 0 ? r0 : 0) * pm;
        const uint32_t nrec = rows > 0 ? (uint32_t)(rows - 1) * pm + row_bytes : 0u;
        return __builtin_amdgcn_make_buffer_rsrc((void *)base, 0, (int)nrec, BUFFER_FLAGS);
    };
    uint4 q[U][CPL];
    uint16_t sc[U][CPL];
    auto load_group = [&](int gi) {
        const __amdgpu_buffer_rsrc_t res1 = group_rsrc(gi, W, pitch);
        const __amdgpu_buffer_rsrc_t res2 = SWIGLU ? group_rsrc(gi, W2, pitch2) : res1;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool second = SWIGLU && u >= RU;
            const __amdgpu_buffer_rsrc_t res = second ? res2 : res1;
            const uint32_t pu = second ? pitch2 : pitch;
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                const uint32_t ro = (uint32_t)(u % RU) * pu;
                q[u][j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(res, qoffs[j] + ro, 0, kStreamLoad));
                if (WT != W_F16)
                    sc[u][j] = __builtin_amdgcn_raw_buffer_load_b16(res, soffs[j] + ro, 0, kStreamLoad);
            }
        }
        if (f16_tail) {                // uniform; rare: waits for the loads here
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const bool second = SWIGLU && u >= RU;
                const __amdgpu_buffer_rsrc_t res = second ? res2 : res1;
                const uint32_t pu = second ? pitch2 : pitch;
#pragma unroll
                for (int j = 0; j < CPL; ++j) {
                    const uint32_t ro = (uint32_t)(u % RU) * pu;
                    const int c = v + j * VL;
                    const bool partial = c * 8 < K && c * 8 + 8 > K;
                    uint32_t hv[8];
#pragma unroll
                    for (int h = 0; h < 8; ++h) {
                        const uint32_t off = (partial && c * 8 + h < K) ? (uint32_t)(c * 16 + 2 * h) + ro
                                                                          : OUT_OF_RANGE;
                        hv[h] = __builtin_amdgcn_raw_buffer_load_b16(res, off, 0, 0);
                    }
                    q[u][j].x |= hv[0] | (hv[1] << 16);
                    q[u][j].y |= hv[2] | (hv[3] << 16);
                    q[u][j].z |= hv[4] | (hv[5] << 16);
                    q[u][j].w |= hv[6] | (hv[7] << 16);
                }
            }
        }
    };
    // The first staging round's activations are loaded before the first
    // weight loads are issued: staging then waits only for them while the
    // weights stream in.  A thread loads LV consecutive activations at a time
    // (four for quantized rows, whose K is a multiple of 32; one for F16
    // rows, whose K is arbitrary); those at or past K read zeros.
    constexpr int PER = VL * WPC / kThreads;    // activations per thread per round
    constexpr int LV = (WT == W_F16) ? 1 : (PER < 4 ? PER : 4);
    constexpr int NV = PER / LV;
    static_assert(PER % LV == 0, "activation rounds are whole vectors");
    struct XVec { float v[LV]; };
    const uint32_t x_bytes = (uint32_t)K * 4;
    auto load_x_round = [&](XVec (&dst)[NV], int n, int j) {
        const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(X + (uint64_t)n * x_pitch), 0, (int)x_bytes, BUFFER_FLAGS);
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int k = j * VL * WPC + LV * (tid + i * kThreads);
            const uint32_t off = k < K ? (uint32_t)k * 4 : OUT_OF_RANGE;
            if constexpr (LV == 4)
                dst[i] = __builtin_bit_cast(XVec, __builtin_amdgcn_raw_buffer_load_b128(xres, off, 0, 0));
            else if constexpr (LV == 2)
                dst[i] = __builtin_bit_cast(XVec, __builtin_amdgcn_raw_buffer_load_b64(xres, off, 0, 0));
            else
                dst[i] = __builtin_bit_cast(XVec, __builtin_amdgcn_raw_buffer_load_b32(xres, off, 0, 0));
        }
    };
    XVec x0[NV];
    load_x_round(x0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    load_group(g);
    __builtin_amdgcn_sched_barrier(0);

    // ---- activations for this lane's chunks, staged through LDS one (token,
    // chunk round) at a time ----
    float xr[NT][CPL][WPC];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            if (n < nt_real) {                       // uniform over the workgroup
                XVec xv[NV];
                if (n == 0 && j == 0) {
#pragma unroll
                    for (int i = 0; i < NV; ++i) xv[i] = x0[i];
                } else {
                    load_x_round(xv, n, j);
                }
#pragma unroll
                for (int i = 0; i < NV; ++i) {
                    const int e = LV * (tid + i * kThreads);   // element within the round
                    const int cl = e / WPC;
                    *reinterpret_cast<XVec *>(&xs[cl * SC + (e - cl * WPC)]) = xv[i];
                }
                __syncthreads();
                const float4 *src = reinterpret_cast<const float4 *>(&xs[v * SC]);
#pragma unroll
                for (int i = 0; i < WPC / 4; ++i) {
                    const float4 t = src[i];
                    xr[n][j][4 * i] = t.x;
                    xr[n][j][4 * i + 1] = t.y;
                    xr[n][j][4 * i + 2] = t.z;
                    xr[n][j][4 * i + 3] = t.w;
                }
                __syncthreads();
            } else {
#pragma unroll
                for (int i = 0; i < WPC; ++i) xr[n][j][i] = 0.0f;
            }
        }
    }
    const uint32_t magic = 0x64006400u;   // binary16 1024.0 in both halves

    for (int it = 0; it < iters; ++it, g += gstep) {
        uint4 qc[U][CPL];
        uint16_t scc[U][CPL];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int j = 0; j < CPL; ++j) { qc[u][j] = q[u][j]; scc[u][j] = sc[u][j]; }
        load_group(g + gstep);     // past the last group: reads nothing

        float part[V];
#pragma unroll
        for (int i = 0; i < V; ++i) part[i] = 0.0f;
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                const float d = (WT == W_F16)
                                    ? 1.0f
                                    : (float)__builtin_bit_cast(_Float16, scc[u][j]);
#pragma unroll
                for (int n = 0; n < NT; ++n) {
                    const float s = chunk_dot<WT>(qc[u][j], xr[n][j], magic);
                    part[u * NT + n] = fmaf(d, s, part[u * NT + n]);
                }
            }
        }
        const float tot = WaveReduce<V, 0>::run(part, lane);
        const int idx = value_index<V>(lane);
        const bool in_range = g < n_groups;

        const bool owner = lane >= 32 && lane < 32 + V;
        if (KS == 1) {
            if constexpr (SWIGLU) {
                // value idx + V/2 (the up row of gate value idx) sits in the
                // lane whose bit 0 differs: the top index bit is lane bit 0
                const float up = partner<0>(tot, lane);
                if (owner && idx < RU * NT && in_range) {
                    const int u = idx / NT, n = idx % NT;
                    const int r = g * RU + u;
                    if (r < M && n < N) Y[(uint64_t)n * y_pitch + r] = swish(tot) * up;
                }
            } else {
                if (owner && idx < U * NT && in_range) {
                    const int u = idx / NT, n = idx % NT;
                    const int r = g * U + u;
                    if (r < M && n < N) Y[(uint64_t)n * y_pitch + r] = tot;
                }
            }
        } else {
            float *buf = red[it & 1][wave];
            if (owner) buf[idx] = tot;
            __syncthreads();
            if (ks == 0 && lane < RU * NT && in_range) {
                float s = 0.0f;
#pragma unroll
                for (int w2 = 0; w2 < KS; ++w2) s += red[it & 1][grp * KS + w2][lane];
                if constexpr (SWIGLU) {
                    float su = 0.0f;
#pragma unroll
                    for (int w2 = 0; w2 < KS; ++w2) su += red[it & 1][grp * KS + w2][lane + RU * NT];
                    s = swish(s) * su;
                }
                const int u = lane / NT, n = lane % NT;
                const int r = g * RU + u;
                if (r < M && n < N) Y[(uint64_t)n * y_pitch + r] = s;
            }
        }
    }
}

// ---- streaming decode GEMV ------------------------------------------------
//
// The decode shapes (one or two tokens over rows that one wave covers with
// CPL 16-byte chunks per lane) as a grid of a few four-wave workgroups per
// CU, written around what a per-wave timeline of gemv_kernel shows: its math
// waits for the activations, whose loads on a busy CU come back behind
// other waves' weight misses, so the unpacking and multiply-adds bunch up
// after the weight stream instead of riding on it.
//  * The activations are staged once per workgroup, and every wave issues
//    its activation loads before any wave of the workgroup issues a weight
//    load (a barrier between the two, which waits for no data).
//  * Wave w owns the row groups w, w + W, w + 2W, ... (W waves in the grid,
//    at most G groups each) and keeps D groups in flight in a ring of
//    registers, so the math of one group overlaps the transfer of the next
//    D - 1.  The wave's work is straight-line code: every load and every
//    store is issued unconditionally (buffer operations whose out-of-range
//    offsets read zeros or write nothing), only the arithmetic of groups the
//    wave does not own is skipped, so the compiler's wait counts are exact
//    and each group waits for its own loads only.
// Loads, unpacking, the wave reduction and the stores are those of
// gemv_kernel with one wave per row.
template <int WT, int NT, int CPL, int U, int D, int G>
__global__ __launch_bounds__(256) void gemv_stream_kernel(const GemvArgs a)
{
    constexpr int WPC = Fmt<WT>::wpc;
    constexpr int SC = lds_chunk_stride<WT>();
    constexpr int V = pow2_ceil(U * NT);
    constexpr int TOK = 64 * CPL * SC;        // LDS floats per token
    static_assert(V <= 64, "too many partial sums per lane");
    static_assert(D >= 1 && D <= G, "ring depth");
    extern __shared__ __attribute__((aligned(16))) float xs[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int item = blockIdx.y;
    const GemvItem &itm = a.item[item];
    const uint8_t *const W = itm.w;
    const float *const X = itm.x;
    float *const Y = itm.y;
    const uint32_t pitch = itm.pitch;
    const uint32_t x_pitch = itm.x_pitch;
    const uint32_t y_pitch = itm.y_pitch;
    const int M = itm.M;
    const int n_groups = itm.n_groups;
    const int n_wg = itm.wg_count;
    const int N = a.N;
    const int K = a.K;
    const int qoff = a.qoff;
    const int nchunk = a.nchunk;
    const int sshift = a.scale_shift;
    asm volatile("" ::"s"(W), "s"(X), "s"(Y), "s"(pitch), "s"(x_pitch), "s"(y_pitch), "s"(M),
                 "s"(n_groups), "s"(n_wg), "s"(N), "s"(K), "s"(qoff), "s"(nchunk), "s"(sshift));
    if ((int)blockIdx.x >= n_wg) return;
    const int nt_real = N < NT ? N : NT;

    // ---- activation loads: float4 f of token n belongs to chunk 4f / WPC ----
    constexpr int F4 = 64 * CPL * WPC / 4;            // float4s per token the lanes cover
    constexpr int XL = (F4 + 255) / 256;              // per thread
    float4 xv[NT][XL];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(X + (uint64_t)(n < nt_real ? n : 0) * x_pitch), 0, n < nt_real ? K * 4 : 0, BUFFER_FLAGS);
#pragma unroll
        for (int i = 0; i < XL; ++i) {
            const int f = tid + 256 * i;
            const uint32_t off = (f < F4 && 4 * f < K) ? (uint32_t)f * 16u : OUT_OF_RANGE;
            xv[n][i] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(xres, off, 0, 0));
        }
    }
    // every wave's activation loads go out before any weight load
    __builtin_amdgcn_s_barrier();

    // ---- weight ring ----
    const int Wn = n_wg * 4;
    const int g0 = (int)blockIdx.x * 4 + wave;
    const int cnt = g0 < n_groups ? (n_groups - g0 + Wn - 1) / Wn : 0;     // groups this wave owns (<= G)
    const int code_bytes = (WT == W_Q4_0) ? K / 2 : (WT == W_Q8_0 ? K : 2 * K);
    const uint32_t row_bytes = (uint32_t)(qoff + code_bytes);
    uint32_t qoffs[CPL], soffs[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int c = lane + 64 * j;
        const bool full = (WT == W_F16) ? c * 8 + 8 <= K : c < nchunk;
        qoffs[j] = full ? (uint32_t)(qoff + c * 16) : OUT_OF_RANGE;
        soffs[j] = full ? (uint32_t)(2 * (chunk_block<WT>(c) >> sshift)) : OUT_OF_RANGE;
    }
    uint4 q[D][U][CPL];
    uint16_t sc[D][U][CPL];
    auto load = [&](uint4 (&qd)[U][CPL], uint16_t (&sd)[U][CPL], int k) {
        const int r0 = (g0 + k * Wn) * U;
        const int rows = (k < cnt) ? (M - r0 < U ? M - r0 : U) : 0;
        const uint8_t *base = W + (uint64_t)(rows > 0 ? r0 : 0) * pitch;
        const uint32_t nrec = rows > 0 ? (uint32_t)(rows - 1) * pitch + row_bytes : 0u;
        const __amdgpu_buffer_rsrc_t res = __builtin_amdgcn_make_buffer_rsrc((void *)base, 0, (int)nrec, BUFFER_FLAGS);
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                const uint32_t ro = (uint32_t)u * pitch;
                qd[u][j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(res, qoffs[j] + ro, 0, kStreamLoad));
                if (WT != W_F16)
                    sd[u][j] = __builtin_amdgcn_raw_buffer_load_b16(res, soffs[j] + ro, 0, kStreamLoad);
            }
        }
    };
#pragma unroll
    for (int s = 0; s < D; ++s) load(q[s], sc[s], s);

    // ---- stage the activations, then each lane's chunks into registers ----
#pragma unroll
    for (int n = 0; n < NT; ++n) {
#pragma unroll
        for (int i = 0; i < XL; ++i) {
            const int f = tid + 256 * i;
            if (f < F4) {
                const int c = (4 * f) / WPC;
                *reinterpret_cast<float4 *>(&xs[n * TOK + c * SC + (4 * f - c * WPC)]) = xv[n][i];
            }
        }
    }
    __syncthreads();
    float xr[NT][CPL][WPC];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const float4 *src = reinterpret_cast<const float4 *>(&xs[n * TOK + (lane + 64 * j) * SC]);
#pragma unroll
            for (int i = 0; i < WPC / 4; ++i) {
                const float4 t = src[i];
                xr[n][j][4 * i] = t.x;
                xr[n][j][4 * i + 1] = t.y;
                xr[n][j][4 * i + 2] = t.z;
                xr[n][j][4 * i + 3] = t.w;
            }
        }
    }
    const uint32_t magic = 0x64006400u;   // binary16 1024.0 in both halves

    // outputs through a buffer resource over y, so that lanes with nothing to
    // store issue the same store with an out-of-range offset
    const __amdgpu_buffer_rsrc_t yres = __builtin_amdgcn_make_buffer_rsrc(
        (void *)Y, 0, (int)(((uint32_t)(N - 1) * y_pitch + (uint32_t)M) * 4u), BUFFER_FLAGS);
    const int idx = value_index<V>(lane);
    const bool owner = lane >= 32 && lane < 32 + V && idx < U * NT;
    const int own_u = idx / NT, own_n = idx % NT;
#pragma unroll
    for (int k = 0; k < G; ++k) {
        const int s = k % D;
        float tot = 0.0f;
        if (k < cnt) {                                // uniform over the wave
            float part[V];
#pragma unroll
            for (int i = 0; i < V; ++i) part[i] = 0.0f;
#pragma unroll
            for (int u = 0; u < U; ++u) {
#pragma unroll
                for (int j = 0; j < CPL; ++j) {
                    const float d = (WT == W_F16) ? 1.0f : (float)__builtin_bit_cast(_Float16, sc[s][u][j]);
#pragma unroll
                    for (int n = 0; n < NT; ++n) {
                        const float sum = chunk_dot<WT>(q[s][u][j], xr[n][j], magic);
                        part[u * NT + n] = fmaf(d, sum, part[u * NT + n]);
                    }
                }
            }
            tot = WaveReduce<V, 0>::run(part, lane);
        }
        if (k + D < G) load(q[s], sc[s], k + D);       // past this wave's groups: reads nothing
        const int r = (g0 + k * Wn) * U + own_u;
        const bool st = owner && k < cnt && r < M && own_n < N;
        const uint32_t off = st ? ((uint32_t)own_n * y_pitch + (uint32_t)r) * 4u : OUT_OF_RANGE;
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, tot), yres, off, 0, 0);
    }
}

// ---- dispatch -------------------------------------------------------------

using Kernel = void (*)(const GemvArgs);

template <int WT, int NT, int KS, int CPL>
constexpr bool fits()
{
    return CPL * Fmt<WT>::wpc * NT <= 128;
}

// Sixteen-wave workgroups only where a wave owns whole rows of one chunk or
// two per lane of quantized codes (the decode shapes at one or two tokens).
template <int WT, int NT, int KS, int CPL, int U, bool SW>
Kernel pick_w(int wgw)
{
    if (wgw == 4) return gemv_kernel<WT, NT, KS, CPL, U, SW, 4>;
    if constexpr (KS == 1 && CPL <= 2 && NT <= 2 && WT != W_F16)
        if (wgw == 16) return gemv_kernel<WT, NT, KS, CPL, U, SW, 16>;
    return nullptr;
}

template <int WT, int NT, int KS, int CPL>
Kernel pick_u(int u, bool swiglu, int wgw)
{
    if constexpr (!fits<WT, NT, KS, CPL>()) {
        return nullptr;
    } else {
        // Several rows per wave group only while a lane holds few chunks;
        // otherwise the in-flight code registers would spill.
        constexpr int UW = (CPL > 2) ? 1 : (NT <= 1) ? 4 : (NT == 2 ? 2 : 1);
        if (swiglu) {
            // a fused group holds a gate row and an up row per row index
            if (u == 2) return pick_w<WT, NT, KS, CPL, 2, true>(wgw);
            if constexpr (UW == 4)
                if (u == 4) return pick_w<WT, NT, KS, CPL, 4, true>(wgw);
            return nullptr;
        }
        if (u == 1) return pick_w<WT, NT, KS, CPL, 1, false>(wgw);
        if (u == UW) return pick_w<WT, NT, KS, CPL, UW, false>(wgw);
        if constexpr (UW == 4)
            if (u == 2) return pick_w<WT, NT, KS, CPL, 2, false>(wgw);
        return nullptr;
    }
}

template <int WT, int NT, int KS>
Kernel pick_cpl(int cpl, int u, bool swiglu, int wgw)
{
    switch (cpl) {
    case 1: return pick_u<WT, NT, KS, 1>(u, swiglu, wgw);
    case 2: return pick_u<WT, NT, KS, 2>(u, swiglu, wgw);
    case 4: return pick_u<WT, NT, KS, 4>(u, swiglu, wgw);
    case 8: return pick_u<WT, NT, KS, 8>(u, swiglu, wgw);
    default: return nullptr;
    }
}

template <int WT, int NT>
Kernel pick_ks(int ks, int cpl, int u, bool swiglu, int wgw)
{
    switch (ks) {
    case 1: return pick_cpl<WT, NT, 1>(cpl, u, swiglu, wgw);
    case 2: return pick_cpl<WT, NT, 2>(cpl, u, swiglu, wgw);
    case 4: return pick_cpl<WT, NT, 4>(cpl, u, swiglu, wgw);
    default: return nullptr;
    }
}

template <int WT>
Kernel pick_nt(int nt, int ks, int cpl, int u, bool swiglu, int wgw)
{
    switch (nt) {
    case 1: return pick_ks<WT, 1>(ks, cpl, u, swiglu, wgw);
    case 2: return pick_ks<WT, 2>(ks, cpl, u, swiglu, wgw);
    case 4: return pick_ks<WT, 4>(ks, cpl, u, swiglu, wgw);
    case 8: return pick_ks<WT, 8>(ks, cpl, u, swiglu, wgw);
    default: return nullptr;
    }
}

Kernel pick(int wt, const GemvConfig &c, bool swiglu = false)
{
    switch (wt) {
    case W_Q4_0: return pick_nt<W_Q4_0>(c.nt, c.ks, c.cpl, c.u, swiglu, c.wgw);
    case W_Q8_0: return pick_nt<W_Q8_0>(c.nt, c.ks, c.cpl, c.u, swiglu, c.wgw);
    case W_F16:  return pick_nt<W_F16>(c.nt, c.ks, c.cpl, c.u, swiglu, c.wgw);
    default: return nullptr;
    }
}

int weights_per_chunk(int type) { return type == W_Q4_0 ? 32 : type == W_Q8_0 ? 16 : 8; }
int lds_chunk_stride_of(int type) { return weights_per_chunk(type) + 4; }

int64_t chunks_per_row(int type, int64_t K)
{
    const int64_t code_bytes = (type == W_Q4_0) ? K / 2 : (type == W_Q8_0 ? K : 2 * K);
    return (code_bytes + 15) / 16;
}

int round_cpl(int64_t c) { return c <= 1 ? 1 : c == 2 ? 2 : c <= 4 ? 4 : c <= 8 ? 8 : 0; }

}  // namespace

bool gemv_config(int type, int64_t K, int64_t M, int64_t N, GemvConfig *cfg)
{
    if (type != W_Q4_0 && type != W_Q8_0 && type != W_F16) return false;
    if (N < 1 || N > 8 || K < 0 || M < 0) return false;
    GemvConfig c;
    c.nt = N <= 1 ? 1 : N <= 2 ? 2 : N <= 4 ? 4 : 8;
    const int wpc = weights_per_chunk(type);
    const int64_t nchunk = chunks_per_row(type, K);
    c.cpl = 0;
    c.ks = 0;
    // One chunk per lane when a wave group of up to four waves covers the
    // row: the activation slice, and the rounds that stage it through LDS,
    // are then smallest (measured faster for long rows, e.g. K = 5632) ...
    for (int ks : {1, 2, 4}) {
        if (nchunk <= 64 * ks && wpc * c.nt <= 128) {
            c.ks = ks;
            c.cpl = 1;
            break;
        }
    }
    // ... otherwise, for Q4_0 rows, the smallest wave group whose slice fits
    // in registers; for F16 and Q8_0 rows the widest (measured,
    // graph-replayed, 1 / 2 tokens: F16 4096 x 4096 in 7.9 / 9.3 us with
    // four waves of 2 chunks per lane, against 13.4 / 29.8 with one wave of
    // 8; F16 11008 x 4096 in 17.1 / 18.5 against 29.8 / 63.9; F16 2048 x 5632
    // in 7.9 / 9.2 with four waves of 4, against 7.7 / 18.2 with two of 8;
    // Q8_0 4096 x 8192 in 9.7 / 10.8 against 10.8 / 11.8 with one wave of 8
    // and two of 4; Q8_0 2048 x 5632 in 5.6 / 6.9 against 6.0 / 7.6 with two
    // waves of 4.  Q4_0 rows gained or lost up to 3 %).
    if (c.ks == 0) {
        const int order[2][3] = {{1, 2, 4}, {4, 2, 1}};
        for (int ks : order[type != W_Q4_0]) {
            const int cp = round_cpl((nchunk + 64 * ks - 1) / (64 * ks));
            if (cp == 0 || cp * wpc * c.nt > 128) continue;
            c.ks = ks;
            c.cpl = cp;
            break;
        }
    }
    if (c.ks == 0) return false;
    // Rows per wave group: with one wave per row, two rows from 2048 rows up
    // and one below (measured on 256 .. 11264 rows of K = 2048: four rows
    // leave too few waves, one row too little in flight per wave); rows
    // split over several waves take the widest group.
    const int u_wide = c.nt <= 1 ? 4 : (c.nt == 2 ? 2 : 1);
    if (c.ks == 1)
        c.u = c.nt <= 2 ? (M >= 2048 ? 2 : 1) : 1;
    else
        c.u = u_wide;
    // ... widened while the rows alone cannot fill 256 CUs with 8 waves each,
    // as long as no more than a quarter of the lanes is left without a chunk.
    while (c.ks < 4) {
        const int64_t waves = ((M + c.u - 1) / c.u) * c.ks;
        const int nks = c.ks * 2;
        const int64_t need = (nchunk + 64 * nks - 1) / (64 * nks);
        if (waves >= 2048 || 3 * need * 64 * nks > 4 * nchunk) break;
        const int cp = round_cpl(need);
        if (cp == 0 || cp * wpc * c.nt > 128) break;
        c.ks = nks;
        c.cpl = cp;
    }
    if (c.cpl > 2) c.u = 1;
    // F16 and Q8_0 rows of two chunks per lane: two rows per group at one
    // token (F16 4096 x 4096: 7.9 us, against 9.7 with four rows and 8.2
    // with one; Q8_0 2048 x 5632: 5.6, against 5.6 and 6.0)
    if (type != W_Q4_0 && c.cpl == 2 && c.u > 2) c.u = 2;
    c.wgw = 4;
    if (!pick(type, c)) return false;
    *cfg = c;
    return true;
}

// ---- streaming decode GEMV: configuration and launch ------------------------

struct StreamConfig {
    int nt, cpl, u, d, g, wg_per_cu;
};

using StreamKernel = void (*)(const GemvArgs);

template <int WT, int NT, int CPL, int U>
StreamKernel pick_stream_d(int d, int g)
{
    if constexpr (CPL * Fmt<WT>::wpc * NT > 128) {
        return nullptr;
    } else {
        if (d == 4 && g == 4) return gemv_stream_kernel<WT, NT, CPL, U, 4, 4>;
        if (d == 4 && g == 8) return gemv_stream_kernel<WT, NT, CPL, U, 4, 8>;
        return nullptr;
    }
}

template <int WT, int NT>
StreamKernel pick_stream_cu(int cpl, int u, int d, int g)
{
    if (cpl == 1) return u == 1 ? pick_stream_d<WT, NT, 1, 1>(d, g) : u == 2 ? pick_stream_d<WT, NT, 1, 2>(d, g) : nullptr;
    if (cpl == 2) return u == 1 ? pick_stream_d<WT, NT, 2, 1>(d, g) : u == 2 ? pick_stream_d<WT, NT, 2, 2>(d, g) : nullptr;
    if (cpl == 4) return u == 1 ? pick_stream_d<WT, NT, 4, 1>(d, g) : u == 2 ? pick_stream_d<WT, NT, 4, 2>(d, g) : nullptr;
    return nullptr;
}

StreamKernel pick_stream(int type, const StreamConfig &c)
{
    const auto for_type = [&](auto wt) -> StreamKernel {
        constexpr int WT = decltype(wt)::value;
        return c.nt == 1 ? pick_stream_cu<WT, 1>(c.cpl, c.u, c.d, c.g) : c.nt == 2 ? pick_stream_cu<WT, 2>(c.cpl, c.u, c.d, c.g) : nullptr;
    };
    switch (type) {
    case W_Q4_0: return for_type(std::integral_constant<int, W_Q4_0>{});
    case W_Q8_0: return for_type(std::integral_constant<int, W_Q8_0>{});
    case W_F16:  return for_type(std::integral_constant<int, W_F16>{});
    default: return nullptr;
    }
}

// The streaming kernel takes one or two tokens over rows of at most two
// 16-byte chunks per lane (four for F16, whose K must be a multiple of 8),
// as long as the grid of wg_per_cu workgroups per CU covers every row group
// with at most g groups per wave.  It is used where it measured faster than
// gemv_kernel (graph-replayed, weights not cache-resident): F16 rows
// (5632 x 2048: 6.07 against 6.83 us), two tokens (Q4_0 5632 x 2048: 4.19
// against 4.70 us) and Q8_0 matrices of at least 8192 rows at one token (the
// 32000 x 2048 LM head: 14.15 against 14.56 us).  One-token Q4_0 stays on
// gemv_kernel (equal on the gate/up batch, 0.1 us slower alone): both are
// bound by the unpacking and multiply-adds once the first bytes arrive.
bool stream_config(int type, int64_t K, int64_t m_total, int64_t N, StreamConfig *cfg)
{
    if (N < 1 || N > 2 || K <= 0) return false;
    if (type == W_F16 && K % 8 != 0) return false;
    if (N == 1 && !(type == W_F16 || (type == W_Q8_0 && m_total >= 8192))) return false;
    const int64_t cpl = (chunks_per_row(type, K) + 63) / 64;
    StreamConfig c;
    c.nt = (int)N;
    c.cpl = cpl <= 1 ? 1 : cpl <= 2 ? 2 : (type == W_F16 && cpl <= 4) ? 4 : 0;
    if (c.cpl == 0) return false;
    c.u = (N == 1 && type != W_F16) ? 2 : 1;
    c.d = 4;
    c.wg_per_cu = 2;
    const int64_t waves = (int64_t)c.wg_per_cu * device_cus() * 4;
    const int64_t groups = (m_total + c.u - 1) / c.u;
    const int64_t per_wave = (groups + waves - 1) / waves;
    c.g = per_wave <= 4 ? 4 : per_wave <= 8 ? 8 : 0;
    if (c.g == 0) return false;
    if (!pick_stream(type, c)) return false;
    *cfg = c;
    return true;
}

// The stores address y through a buffer resource with 32-bit byte offsets.
bool stream_supported(const GemvTask *tasks, int count)
{
    for (int i = 0; i < count; ++i)
        if ((tasks[i].x.N - 1) * (int64_t)tasks[i].y.pitch_elems + tasks[i].w.M > ((int64_t)1 << 29)) return false;
    return true;
}

hipError_t launch_gemv_stream(const GemvTask *tasks, int count, const StreamConfig &c, hipStream_t stream)
{
    const int type = tasks[0].w.type;
    const int64_t K = tasks[0].w.K;
    const StreamKernel k = pick_stream(type, c);
    if (!k) return hipErrorInvalidValue;
    GemvArgs a = {};
    a.N = (int32_t)tasks[0].x.N;
    a.K = (int32_t)K;
    a.qoff = (type == W_F16) ? 0 : (int32_t)quant_offset(K, tasks[0].w.scale_shift);
    a.nchunk = (int32_t)chunks_per_row(type, K);
    a.scale_shift = tasks[0].w.scale_shift;
    int64_t groups_total = 0;
    for (int i = 0; i < count; ++i) groups_total += (tasks[i].w.M + c.u - 1) / c.u;
    const int64_t budget = (int64_t)c.wg_per_cu * device_cus();
    int32_t wg_max = 0;
    for (int i = 0; i < count; ++i) {
        if (tasks[i].w.M == 0) continue;
        GemvItem &it = a.item[a.n_items++];
        it.w = tasks[i].w.base;
        it.pitch = (uint32_t)tasks[i].w.pitch;
        it.M = (int32_t)tasks[i].w.M;
        it.x = static_cast<const float *>(tasks[i].x.data);
        it.x_pitch = (uint32_t)tasks[i].x.pitch_elems;
        it.y = tasks[i].y.data;
        it.y_pitch = (uint32_t)tasks[i].y.pitch_elems;
        it.n_groups = (int32_t)((tasks[i].w.M + c.u - 1) / c.u);
        // the item's share of the grid, enough waves for at most c.g groups each
        int64_t wgs = (budget * it.n_groups + groups_total - 1) / groups_total;
        const int64_t need = (it.n_groups + 4LL * c.g - 1) / (4LL * c.g);
        if (wgs < need) wgs = need;
        if (wgs > (it.n_groups + 3) / 4) wgs = (it.n_groups + 3) / 4;   // a group per wave at least
        if (wgs < 1) wgs = 1;
        it.wg_count = (int32_t)wgs;
        it.iters = 0;
        if (wgs > wg_max) wg_max = (int32_t)wgs;
    }
    const size_t lds = (size_t)c.nt * 64 * c.cpl * lds_chunk_stride_of(type) * sizeof(float);
    hipLaunchKernelGGL(k, dim3((unsigned)wg_max, (unsigned)a.n_items), dim3(256), lds, stream, a);
    return hipGetLastError();
}

hipError_t launch_gemv_batch(const GemvTask *tasks, int count, hipStream_t stream)
{
    if (count < 1 || count > kMaxItems) return hipErrorInvalidValue;
    const int type = tasks[0].w.type;
    const int64_t K = tasks[0].w.K;
    const int64_t N = tasks[0].x.N;
    int64_t m_total = 0;
    for (int i = 0; i < count; ++i) m_total += tasks[i].w.M;
    if (m_total == 0 || N == 0) return hipSuccess;
    // The matrix-core kernels' cost does not grow with the token count.
    const bool mf = type == W_F16 ? use_matrix_cores_f16(N, m_total, K) : use_matrix_cores(N, m_total, K);
    if (mf && gemv_mf_supported(tasks, count)) return launch_gemv_mf(tasks, count, stream);
    StreamConfig sc;
    if (stream_config(type, K, m_total, N, &sc) && stream_supported(tasks, count))
        return launch_gemv_stream(tasks, count, sc, stream);

    // Tokens are processed in chunks of at most 8; a chunk shrinks (halving)
    // until a register-resident configuration exists for it.
    for (int64_t n0 = 0; n0 < N;) {
        int64_t nb = N - n0 < 8 ? N - n0 : 8;
        GemvConfig c;
        while (!gemv_config(type, K, m_total, nb, &c)) {
            if (nb == 1) return hipErrorInvalidValue;
            nb = nb > 4 ? 4 : nb > 2 ? 2 : 1;
        }
        const Kernel k = pick(type, c);
        const int groups_per_wg = c.wgw / c.ks;
        GemvArgs a = {};
        a.n_items = 0;
        a.N = (int32_t)nb;
        a.K = (int32_t)K;
        a.qoff = (type == W_F16) ? 0 : (int32_t)quant_offset(K, tasks[0].w.scale_shift);
        a.nchunk = (int32_t)chunks_per_row(type, K);
        a.scale_shift = tasks[0].w.scale_shift;
        int64_t need_total = 0;
        int64_t need[kMaxItems];
        for (int i = 0; i < count; ++i) {
            const int64_t groups = (tasks[i].w.M + c.u - 1) / c.u;
            need[i] = (groups + groups_per_wg - 1) / groups_per_wg;
            need_total += need[i];
        }
        int32_t wg_max = 0;
        for (int i = 0; i < count; ++i) {
            if (tasks[i].w.M == 0) continue;
            int64_t wgs = need[i];
            const int wg_cap = max_workgroups(c.ks, c.wgw, K);
            if (need_total > wg_cap) {
                wgs = need[i] * wg_cap / need_total;   // share of the persistent grid
                if (wgs < 1) wgs = 1;
            }
            GemvItem &it = a.item[a.n_items++];
            it.w = tasks[i].w.base;
            it.pitch = (uint32_t)tasks[i].w.pitch;
            it.M = (int32_t)tasks[i].w.M;
            it.x = static_cast<const float *>(tasks[i].x.data) + (uint64_t)n0 * tasks[i].x.pitch_elems;
            it.x_pitch = (uint32_t)tasks[i].x.pitch_elems;
            it.y = tasks[i].y.data + (uint64_t)n0 * tasks[i].y.pitch_elems;
            it.y_pitch = (uint32_t)tasks[i].y.pitch_elems;
            it.n_groups = (int32_t)((tasks[i].w.M + c.u - 1) / c.u);
            it.wg_count = (int32_t)wgs;
            const int64_t per_pass = (int64_t)groups_per_wg * wgs;   // groups one pass of the grid covers
            it.iters = (int32_t)((it.n_groups + per_pass - 1) / per_pass);
            if (wgs > wg_max) wg_max = (int32_t)wgs;
        }
        const int wpc = weights_per_chunk(type);
        const size_t lds = (size_t)64 * c.ks * (wpc + 4) * sizeof(float);
        hipLaunchKernelGGL(k, dim3((unsigned)wg_max, (unsigned)a.n_items), dim3(64 * c.wgw), lds, stream, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        n0 += nb;
    }
    return hipSuccess;
}

hipError_t launch_gemv_swiglu(const WeightView &wg, const WeightView &wu, const ActView &x,
                              const OutView &h, hipStream_t stream)
{
    const int type = wg.type;
    const int64_t K = wg.K, M = wg.M, N = x.N;
    if (M == 0 || N == 0) return hipSuccess;
    // From 3 tokens the matrix-core kernel (2 x 5632 x 2048 Q4_0, graph-
    // replayed, 3 / 8 tokens: 7.8 / 8.2 us against 9.9 / 21.0 us here).
    if (N >= 3 && gemv_mf_swiglu_supported(wg, wu, x)) return launch_gemv_mf_swiglu(wg, wu, x, h, stream);
    for (int64_t n0 = 0; n0 < N;) {
        int64_t nb = N - n0 < 8 ? N - n0 : 8;
        GemvConfig c;
        while (!gemv_config(type, K, 2 * M, nb, &c)) {
            if (nb == 1) return hipErrorInvalidValue;
            nb = nb > 4 ? 4 : nb > 2 ? 2 : 1;
        }
        // The plain configuration for the 2M rows of both matrices; a fused
        // group holds at least one row index of each, and two of each where
        // the plain kernel takes two rows per group (one token, rows that one
        // wave covers, M >= 2048: 2 x 5632 x 2048 Q4_0 5.2 -> 5.05 us).
        if (c.u < 2) c.u = 2;
        if (nb == 1 && c.ks == 1 && c.cpl <= 2 && M >= 2048) c.u = 4;
        const Kernel k = pick(type, c, true);
        if (!k) return hipErrorInvalidValue;
        const int groups_per_wg = c.wgw / c.ks;
        const int ru = c.u / 2;
        GemvArgs a = {};
        a.n_items = 1;
        a.N = (int32_t)nb;
        a.K = (int32_t)K;
        a.qoff = (type == W_F16) ? 0 : (int32_t)quant_offset(K, wg.scale_shift);
        a.nchunk = (int32_t)chunks_per_row(type, K);
        a.scale_shift = wg.scale_shift;
        GemvItem &it = a.item[0];
        it.w = wg.base;
        it.w2 = wu.base;
        it.pitch = (uint32_t)wg.pitch;
        it.pitch2 = (uint32_t)wu.pitch;
        it.M = (int32_t)M;
        it.x = static_cast<const float *>(x.data) + (uint64_t)n0 * x.pitch_elems;
        it.x_pitch = (uint32_t)x.pitch_elems;
        it.y = h.data + (uint64_t)n0 * h.pitch_elems;
        it.y_pitch = (uint32_t)h.pitch_elems;
        it.n_groups = (int32_t)((M + ru - 1) / ru);
        int64_t wgs = (it.n_groups + groups_per_wg - 1) / groups_per_wg;
        if (wgs > max_workgroups(c.ks, c.wgw)) wgs = max_workgroups(c.ks, c.wgw);
        it.wg_count = (int32_t)wgs;
        const int64_t per_pass = (int64_t)groups_per_wg * wgs;
        it.iters = (int32_t)((it.n_groups + per_pass - 1) / per_pass);
        const int wpc = weights_per_chunk(type);
        const size_t lds = (size_t)64 * c.ks * (wpc + 4) * sizeof(float);
        hipLaunchKernelGGL(k, dim3((unsigned)wgs, 1u), dim3(64 * c.wgw), lds, stream, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        n0 += nb;
    }
    return hipSuccess;
}

hipError_t launch_gemv(const WeightView &w, const ActView &x, const OutView &y,
                       hipStream_t stream)
{
    const GemvTask t{w, x, y};
    return launch_gemv_batch(&t, 1, stream);
}

}  // namespace qmm
