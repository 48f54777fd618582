// gemv_i8.hip -- the integer-activation decode GEMV.
//
// A Complete Guide to llama.cpp and Customization with C++, §2.2: when the
// activations are quantized per block as well, x_i ~= Delta_x * qx_i, the
// dot product of a block is y ~= Delta * Delta_x * sum_i q_i qx_i, and the
// sum is integer arithmetic.  Here the activations are Q8_0 rows (quantized
// by qmm_quantize, the weights' Q8_0 rule), the weights Q4_0 (q = nibble - 8)
// or Q8_0, and each block's integer sum is four-way int8 dot products
// (v_dot4c_i32_i8) accumulated exactly in int32; only the per-block term
// Delta * Delta_x * S (Delta * Delta_x is exact in binary32: two 11-bit
// significands) and the sum over blocks round.
//
// The mapping is the one of gemv.hip (16-byte weight chunks, KS waves per
// row, U rows per wave group, the same wave reduction), with two changes:
//  * a lane's activations are its blocks' int8 codes and scales, loaded
//    straight from the Q8_0 rows (32 bytes per Q4_0 block, coalesced across
//    the lanes), with no LDS staging;
//  * a Q4_0 nibble n enters the dot product as the int8 value n (it is below
//    128) and the block sum is corrected by -8 * sum_i qx_i, an integer
//    computed once per activation block.
// Like the fp32 GEMV, a launch takes up to QMM_GEMV_BATCH_MAX items (grid y)
// sharing the persistent grid by rows, or one gate/up pair fused with the
// SwiGLU epilogue (one gate and one up row per group).
#include "qmm_internal.h"
#include "wave_reduce.h"

namespace qmm {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxWorkgroups = 1024;

constexpr int kMaxItems = QMM_GEMV_BATCH_MAX;

// One GEMV of a launch (grid y indexes the items; a batch shares the weight
// type, K and the tokens).
struct alignas(64) I8Item {
    const uint8_t *w;
    const uint8_t *xq;     // Q8_0 rows of the activations
    float *y;
    const uint8_t *w2;     // fused SwiGLU launches: the up projection (w is the gate)
    uint32_t pitch;        // bytes between weight rows
    uint32_t x_pitch;      // bytes between activation rows
    uint32_t y_pitch;      // elements between output rows
    uint32_t pitch2;
    int32_t M;
    int32_t n_groups;      // row groups (U rows, or U/2 row indices of each matrix when fused)
    int32_t wg_count;      // workgroups of this item (the rest of grid x exits)
    int32_t iters;
};
static_assert(sizeof(I8Item) == 64, "one record per item");

struct I8Args {
    int32_t N;
    int32_t K;
    int32_t qoff;          // code offset inside an activation row (Q8_0, 32-blocks)
    int32_t nchunk;        // 16-byte chunks of weight codes per row
    int32_t wqoff;         // code offset inside a weight row (qoff for 32-blocks)
    int32_t scale_shift;   // 1: the weights have one scale per two 32-code runs
    int32_t pad[10];
    I8Item item[kMaxItems];
};

// Per 16-byte chunk of weight codes: Q4_0 one block (32 weights, 8 dwords of
// activation codes), Q8_0 half a block (16 weights, 4 dwords).
template <int WT> struct I8Fmt;
template <> struct I8Fmt<W_Q4_0> { static constexpr int xd = 8; };
template <> struct I8Fmt<W_Q8_0> { static constexpr int xd = 4; };

template <int WT>
__device__ inline int chunk_block(int c) { return WT == W_Q4_0 ? c : c / 2; }

// sum_i w_i qx_i over one chunk, w_i the stored code (Q4_0: nibble 0..15).
// Q4_0 byte j holds elements j (low nibble) and j + 16 (high nibble), so
// dword d of the chunk pairs with activation dwords d and 4 + d.
template <int WT>
__device__ inline int chunk_idot(const uint4 q, const uint32_t *xv)
{
    const uint32_t wd[4] = {q.x, q.y, q.z, q.w};
    int s = 0;
    if constexpr (WT == W_Q4_0) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            s = __builtin_amdgcn_sdot4((int)(wd[d] & 0x0F0F0F0Fu), (int)xv[d], s, false);
            s = __builtin_amdgcn_sdot4((int)((wd[d] >> 4) & 0x0F0F0F0Fu), (int)xv[4 + d], s, false);
        }
    } else {
#pragma unroll
        for (int d = 0; d < 4; ++d) s = __builtin_amdgcn_sdot4((int)wd[d], (int)xv[d], s, false);
    }
    return s;
}

// Swish(z) = z * sigma(z) = z / (1 + e^{-z}) in binary32 (for z far below
// zero e^{-z} overflows and the quotient is the limit -0).
__device__ inline float swish(float z)
{
    return z / (1.0f + expf(-z));
}

// SWIGLU: the fused gate/up projection with the SwiGLU epilogue ("Development
// Guide for Small AI Models (TinyLLaMA, etc.) Using C++", §4.4): a group of U
// rows holds U/2 row indices of the gate matrix (rows u < U/2) and the same
// indices of the up matrix, and h = Swish(gate sum) * up sum is stored.
template <int WT, int NT, int KS, int CPL, int U, bool SWIGLU>
__global__ __launch_bounds__(kThreads) void gemv_i8_kernel(const I8Args a)
{
    static_assert(!SWIGLU || U % 2 == 0, "a fused group pairs gate and up rows");
    constexpr int RU = SWIGLU ? U / 2 : U;    // row indices per group
    constexpr int XD = I8Fmt<WT>::xd;
    constexpr int G = 4 / KS;
    constexpr int VL = 64 * KS;
    constexpr int V = pow2_ceil(U * NT);
    static_assert(V <= 64, "too many partial sums per lane");
    __shared__ float red[2][4][64];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave / KS;
    const int ks = wave % KS;
    const int v = ks * 64 + lane;

    const I8Item &itm = a.item[blockIdx.y];
    const uint8_t *const W = itm.w;
    const uint8_t *const W2 = itm.w2;
    const uint32_t pitch2 = itm.pitch2;
    const uint8_t *const XQ = itm.xq;
    float *const Y = itm.y;
    const uint32_t pitch = itm.pitch, x_pitch = itm.x_pitch, y_pitch = itm.y_pitch;
    const int M = itm.M, n_groups = itm.n_groups, n_wg = itm.wg_count, iters = itm.iters;
    const int N = a.N, K = a.K, qoff = a.qoff, nchunk = a.nchunk;
    if ((int)blockIdx.x >= n_wg) return;     // a shorter item's surplus workgroups
    const int nt_real = N < NT ? N : NT;

    int g = (int)blockIdx.x * G + grp;
    const int gstep = n_wg * G;

    // ---- activations: this lane's blocks, codes and scales, from the Q8_0
    // rows; chunks past the row (and tokens past N) read zeros ----
    const uint32_t x_row_bytes = (uint32_t)(qoff + K);
    uint32_t xc[NT][CPL][XD];
    uint16_t xs[NT][CPL];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(XQ + (uint64_t)(n < nt_real ? n : 0) * x_pitch), 0,
            (int)(n < nt_real ? x_row_bytes : 0u), BUFFER_FLAGS);
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int c = v + j * VL;
            const bool in_row = c < nchunk;
            const int b = chunk_block<WT>(c);
            const uint32_t coff = in_row ? (uint32_t)(qoff + 32 * b + (WT == W_Q8_0 ? 16 * (c & 1) : 0))
                                         : OUT_OF_RANGE;
#pragma unroll
            for (int h = 0; h < XD / 4; ++h) {
                const auto t = __builtin_amdgcn_raw_buffer_load_b128(xr, coff + 16 * h, 0, 0);
#pragma unroll
                for (int e = 0; e < 4; ++e) xc[n][j][4 * h + e] = t[e];
            }
            xs[n][j] = __builtin_amdgcn_raw_buffer_load_b16(xr, in_row ? (uint32_t)(2 * b) : OUT_OF_RANGE, 0, 0);
        }
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- weights: as gemv.hip (buffer resource per row group, unconditional loads) ----
    const int code_bytes = (WT == W_Q4_0) ? K / 2 : K;
    const int wqoff = a.wqoff, sshift = a.scale_shift;
    const uint32_t row_bytes = (uint32_t)(wqoff + code_bytes);
    uint32_t qoffs[CPL], soffs[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int c = v + j * VL;
        const bool in_row = c < nchunk;
        qoffs[j] = in_row ? (uint32_t)(wqoff + 16 * c) : OUT_OF_RANGE;
        soffs[j] = in_row ? (uint32_t)(2 * (chunk_block<WT>(c) >> sshift)) : OUT_OF_RANGE;
    }
    uint4 q[U][CPL];
    uint16_t sc[U][CPL];
    auto group_rsrc = [&](int gi, const uint8_t *Wm, uint32_t pm) {
        const int r0 = gi * RU;
        const int rows = gi < n_groups ? (M - r0 < RU ? M - r0 : RU) : 0;
        return __builtin_amdgcn_make_buffer_rsrc(
            (void *)(Wm + (uint64_t)(rows > 0 ? r0 : 0) * pm), 0,
            (int)(rows > 0 ? (uint32_t)(rows - 1) * pm + row_bytes : 0u), BUFFER_FLAGS);
    };
    auto load_group = [&](int gi) {
        const __amdgpu_buffer_rsrc_t res1 = group_rsrc(gi, W, pitch);
        const __amdgpu_buffer_rsrc_t res2 = SWIGLU ? group_rsrc(gi, W2, pitch2) : res1;
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                const bool second = SWIGLU && u >= RU;
                const __amdgpu_buffer_rsrc_t res = second ? res2 : res1;
                const uint32_t ro = (uint32_t)(u % RU) * (second ? pitch2 : pitch);
                q[u][j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(res, qoffs[j] + ro, 0, kStreamLoad));
                sc[u][j] = __builtin_amdgcn_raw_buffer_load_b16(res, soffs[j] + ro, 0, kStreamLoad);
            }
    };
    load_group(g);
    __builtin_amdgcn_sched_barrier(0);

    // per activation block: its scale as a float and (Q4_0) -8 * sum of its codes
    float dx[NT][CPL];
    int xb[NT][CPL];
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            dx[n][j] = (float)__builtin_bit_cast(_Float16, xs[n][j]);
            int s = 0;
            if constexpr (WT == W_Q4_0) {
#pragma unroll
                for (int d = 0; d < XD; ++d) s = __builtin_amdgcn_sdot4((int)xc[n][j][d], 0x01010101, s, false);
            }
            xb[n][j] = -8 * s;
        }

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
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                const float dw = (float)__builtin_bit_cast(_Float16, scc[u][j]);
#pragma unroll
                for (int n = 0; n < NT; ++n) {
                    const int s = chunk_idot<WT>(qc[u][j], xc[n][j]) + xb[n][j];
                    part[u * NT + n] = fmaf(dw * dx[n][j], (float)s, part[u * NT + n]);
                }
            }
        const float tot = WaveReduce<V, 0>::run(part, lane);
        const int idx = value_index<V>(lane);
        const bool in_range = g < n_groups;
        const bool owner = lane >= 32 && lane < 32 + V;
        if (KS == 1) {
            if constexpr (SWIGLU) {
                // value idx + V/2 (the up sum of gate value idx) sits in the
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

using I8Kernel = void (*)(const I8Args);

template <int WT, int NT, int KS, int CPL>
I8Kernel pick_i8_u(int u)
{
    constexpr int UW = (CPL > 2) ? 1 : (NT <= 1) ? 4 : (NT == 2 ? 2 : 1);
    if (u == 1) return gemv_i8_kernel<WT, NT, KS, CPL, 1, false>;
    if (u == UW) return gemv_i8_kernel<WT, NT, KS, CPL, UW, false>;
    if constexpr (UW == 4)
        if (u == 2) return gemv_i8_kernel<WT, NT, KS, CPL, 2, false>;
    return nullptr;
}

// The fused SwiGLU kernels use two-row groups (one gate, one up row).
template <int WT, int NT, int KS, int CPL>
I8Kernel pick_i8_u_sw(int u)
{
    return u == 2 ? gemv_i8_kernel<WT, NT, KS, CPL, 2, true> : nullptr;
}

template <int WT, int NT, int KS>
I8Kernel pick_i8_cpl(int cpl, int u, bool sw)
{
    switch (cpl) {
    case 1: return sw ? pick_i8_u_sw<WT, NT, KS, 1>(u) : pick_i8_u<WT, NT, KS, 1>(u);
    case 2: return sw ? pick_i8_u_sw<WT, NT, KS, 2>(u) : pick_i8_u<WT, NT, KS, 2>(u);
    case 4: return sw ? pick_i8_u_sw<WT, NT, KS, 4>(u) : pick_i8_u<WT, NT, KS, 4>(u);
    default: return nullptr;
    }
}

template <int WT, int NT>
I8Kernel pick_i8_ks(int ks, int cpl, int u, bool sw)
{
    switch (ks) {
    case 1: return pick_i8_cpl<WT, NT, 1>(cpl, u, sw);
    case 2: return pick_i8_cpl<WT, NT, 2>(cpl, u, sw);
    case 4: return pick_i8_cpl<WT, NT, 4>(cpl, u, sw);
    default: return nullptr;
    }
}

template <int WT>
I8Kernel pick_i8_nt(int nt, int ks, int cpl, int u, bool sw = false)
{
    switch (nt) {
    case 1: return pick_i8_ks<WT, 1>(ks, cpl, u, sw);
    case 2: return pick_i8_ks<WT, 2>(ks, cpl, u, sw);
    case 4: return pick_i8_ks<WT, 4>(ks, cpl, u, sw);
    case 8: return pick_i8_ks<WT, 8>(ks, cpl, u, sw);
    default: return nullptr;
    }
}

}  // namespace

namespace {

// Launch shape: the wave split and chunks per lane of the fp32-activation
// GEMV at one token (a function of the row length only), then as many
// tokens per pass as the activation registers allow (NT * CPL * XD <= 64).
bool i8_config(int wtype, int64_t K, int64_t M, int64_t N, GemvConfig *cfg)
{
    GemvConfig c;
    if (!gemv_config(wtype, K, M, 1, &c) || c.cpl > 4) return false;
    const int xd = (wtype == W_Q4_0) ? 8 : 4;
    int nt = N <= 1 ? 1 : N <= 2 ? 2 : N <= 4 ? 4 : 8;
    while (nt > 1 && nt * c.cpl * xd > 64) nt /= 2;
    if (nt * c.cpl * xd > 64) return false;
    c.nt = nt;
    if (nt >= 4 || c.cpl > 2) c.u = 1;
    else if (nt == 2 && c.u > 2) c.u = 2;
    *cfg = c;
    return true;
}

}  // namespace

namespace {

// count items (or, with w2, one fused gate/up pair: w the gate, w2 the up
// projection) in one launch per pass of up to NT tokens.
hipError_t launch_i8(const WeightView *w, const WeightView *w2, const WeightView *xq, const OutView *y,
                     int count, int64_t N, hipStream_t stream)
{
    if (count < 1 || count > kMaxItems || (w2 && count != 1)) return hipErrorInvalidValue;
    const bool sw = w2 != nullptr;
    int64_t m_total = 0;
    for (int i = 0; i < count; ++i) m_total += w[i].M;
    if (m_total == 0 || N == 0) return hipSuccess;
    // Q8_0 weights from 5 tokens over 8192 rows or more, or rows over 4096,
    // go to the matrix cores, where the codes enter exactly and each block's
    // sum is exact as well (graph-replayed, µs at 5 / 8 tokens: the
    // 32000 x 2048 LM head 16.5 / 16.7 against 20.7 / 21.0 here; 2048 x 5632
    // 8.5 / 8.6 against 13.1 / 13.2; 16384 x 2048 10.2 / 10.3 against 11.8 /
    // 12.5; 8192 x 2048 equal; 2048 x 2048 4.9 / 5.2 against 4.6 / 4.3).
    // This kernel keeps Q4_0 weights (e.g. 11264 x 2048 at 8 tokens: 7.9
    // against 9.6 us) and up to 4 tokens.
    if (!sw && w[0].type == W_Q8_0 && N >= 5 && (m_total >= 8192 || w[0].K > 4096) &&
        use_matrix_cores(N, m_total, w[0].K) && gemv_mf_q8x_supported(w, xq, count, N))
        return launch_gemv_mf_q8x(w, xq, y, count, N, stream);
    const WeightView &w0 = w[0];
    GemvConfig c;
    if (!i8_config(w0.type, w0.K, sw ? 2 * m_total : m_total, N, &c)) return hipErrorInvalidValue;
    if (sw) c.u = 2;                     // one gate and one up row per group
    const int ru = sw ? 1 : c.u;         // row indices per group
    const I8Kernel k = (w0.type == W_Q4_0) ? pick_i8_nt<W_Q4_0>(c.nt, c.ks, c.cpl, c.u, sw)
                                           : pick_i8_nt<W_Q8_0>(c.nt, c.ks, c.cpl, c.u, sw);
    if (!k) return hipErrorInvalidValue;
    const int groups_per_wg = 4 / c.ks;
    I8Args a = {};
    a.K = (int32_t)w0.K;
    a.qoff = (int32_t)quant_offset(w0.K);
    a.wqoff = (int32_t)quant_offset(w0.K, w0.scale_shift);
    a.scale_shift = w0.scale_shift;
    a.nchunk = (int32_t)((w0.type == W_Q4_0 ? w0.K / 2 : w0.K) / 16);
    // the persistent grid's workgroups, shared among the items by rows
    int64_t need[kMaxItems], need_total = 0;
    for (int i = 0; i < count; ++i) {
        const int64_t groups = (w[i].M + ru - 1) / ru;
        need[i] = (groups + groups_per_wg - 1) / groups_per_wg;
        need_total += need[i];
    }
    int64_t grid_x = 1;
    for (int i = 0; i < count; ++i) {
        I8Item &it = a.item[i];
        it.w = w[i].base;
        it.pitch = (uint32_t)w[i].pitch;
        it.w2 = sw ? w2->base : w[i].base;
        it.pitch2 = sw ? (uint32_t)w2->pitch : (uint32_t)w[i].pitch;
        it.x_pitch = (uint32_t)xq[i].pitch;
        it.y_pitch = (uint32_t)y[i].pitch_elems;
        it.M = (int32_t)w[i].M;
        it.n_groups = (int32_t)((w[i].M + ru - 1) / ru);
        int64_t wgs = need[i];
        if (need_total > kMaxWorkgroups) {
            wgs = need[i] * kMaxWorkgroups / need_total;
            if (wgs < 1 && need[i] > 0) wgs = 1;
        }
        it.wg_count = (int32_t)wgs;
        const int64_t per_pass = (int64_t)groups_per_wg * (wgs > 0 ? wgs : 1);
        it.iters = (int32_t)((it.n_groups + per_pass - 1) / per_pass);
        if (wgs > grid_x) grid_x = wgs;
    }
    // tokens in passes of up to NT (one pass over the weights each)
    for (int64_t n0 = 0; n0 < N; n0 += c.nt) {
        for (int i = 0; i < count; ++i) {
            a.item[i].xq = xq[i].base + (uint64_t)n0 * xq[i].pitch;
            a.item[i].y = y[i].data + (uint64_t)n0 * y[i].pitch_elems;
        }
        a.N = (int32_t)(N - n0 < c.nt ? N - n0 : c.nt);
        hipLaunchKernelGGL(k, dim3((unsigned)grid_x, (unsigned)count), dim3(kThreads), 0, stream, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_gemv_i8_batch(const WeightView *w, const WeightView *xq, const OutView *y, int count,
                                int64_t N, hipStream_t stream)
{
    return launch_i8(w, nullptr, xq, y, count, N, stream);
}

hipError_t launch_gemv_i8(const WeightView &w, const WeightView &xq, const OutView &y, int64_t N,
                          hipStream_t stream)
{
    return launch_i8(&w, nullptr, &xq, &y, 1, N, stream);
}

hipError_t launch_gemv_i8_swiglu(const WeightView &wg, const WeightView &wu, const WeightView &xq,
                                 const OutView &h, int64_t N, hipStream_t stream)
{
    return launch_i8(&wg, &wu, &xq, &h, 1, N, stream);
}

bool gemv_i8_swiglu_supported(int wtype, int64_t K, int64_t M, int64_t N)
{
    if (wtype != W_Q4_0 && wtype != W_Q8_0) return false;
    GemvConfig c;
    if (!i8_config(wtype, K, 2 * M, N, &c)) return false;
    return (wtype == W_Q4_0 ? pick_i8_nt<W_Q4_0>(c.nt, c.ks, c.cpl, 2, true)
                            : pick_i8_nt<W_Q8_0>(c.nt, c.ks, c.cpl, 2, true)) != nullptr;
}

bool gemv_i8_supported(int wtype, int64_t K, int64_t M, int64_t N)
{
    if (wtype != W_Q4_0 && wtype != W_Q8_0) return false;
    GemvConfig c;
    if (!i8_config(wtype, K, M, N, &c)) return false;
    return (wtype == W_Q4_0 ? pick_i8_nt<W_Q4_0>(c.nt, c.ks, c.cpl, c.u)
                            : pick_i8_nt<W_Q8_0>(c.nt, c.ks, c.cpl, c.u)) != nullptr;
}

}  // namespace qmm
