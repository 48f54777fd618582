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
//  * Codes are turned into floats with byte conversions; the offset of the
//    codes (8 for Q4_0 nibbles, 128 for Q8_0 bytes after flipping the sign
//    bit) is folded into a per-chunk bias -offset * sum(x) computed once, so a
//    weight costs one conversion and one FMA.  The block scale is applied once
//    per chunk: sum_i d*(c_i - o)*x_i = d*(sum_i c_i*x_i - o*sum_i x_i)
//    (A Complete Guide to llama.cpp ..., §2.2: the scale factors out of the
//    block's dot product).
//  * U rows x NT tokens partial sums per lane are reduced across the wave by
//    a transposed butterfly (each exchange halves the set of values a lane
//    carries), then across the KS waves of a group through LDS.
//  * The next row group's loads are issued before the current one is
//    reduced, so each wave keeps U*CPL 128-bit loads in flight.
#include "qmm_internal.h"

namespace qmm {
namespace {

constexpr int kThreads = 256;  // four wave64 per workgroup

template <int WT> struct Fmt;
template <> struct Fmt<W_Q4_0> { static constexpr int wpc = 32; static constexpr float offset = 8.0f; };
template <> struct Fmt<W_Q8_0> { static constexpr int wpc = 16; static constexpr float offset = 128.0f; };
template <> struct Fmt<W_F16>  { static constexpr int wpc = 8;  static constexpr float offset = 0.0f; };

struct GemvArgs {
    const uint8_t *w;
    uint64_t pitch;       // bytes between weight rows
    int64_t M;
    int64_t K;
    int64_t qoff;         // byte offset of the codes inside a row (0 for F16)
    int64_t nchunk;       // 16-byte chunks of codes per row
    const float *x;
    uint64_t x_pitch;     // elements between token rows of x
    int32_t N;            // real tokens (<= NT)
    float *y;
    uint64_t y_pitch;     // elements between token rows of y
    int64_t n_groups;     // row groups of U rows
};

// Weight index of element i (0..wpc-1) of chunk c, in the order the kernel
// unpacks a chunk: Q4_0 low nibbles of the 16 bytes are elements 0..15 of the
// block, high nibbles elements 16..31 (the packing order of the row layout).
template <int WT>
__device__ inline int64_t chunk_k(int64_t c, int i)
{
    if (WT == W_Q4_0) return c * 32 + i;
    if (WT == W_Q8_0) return c * 16 + i;
    return c * 8 + i;
}

template <int WT>
__device__ inline int64_t chunk_block(int64_t c)
{
    return WT == W_Q4_0 ? c : c / 2;   // Q8_0: two chunks per 32-block
}

// sum_i code_i * x_i for one chunk, starting from the folded bias.
template <int WT>
__device__ inline float chunk_dot(const uint4 q, const float *xv, float acc)
{
    const uint32_t wd[4] = {q.x, q.y, q.z, q.w};
    if (WT == W_Q4_0) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint32_t lo = wd[d] & 0x0F0F0F0Fu;
            const uint32_t hi = (wd[d] >> 4) & 0x0F0F0F0Fu;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc = fmaf((float)((lo >> (8 * e)) & 0xFFu), xv[4 * d + e], acc);
                acc = fmaf((float)((hi >> (8 * e)) & 0xFFu), xv[16 + 4 * d + e], acc);
            }
        }
    } else if (WT == W_Q8_0) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint32_t u = wd[d] ^ 0x80808080u;   // code + 128 in each byte
#pragma unroll
            for (int e = 0; e < 4; ++e)
                acc = fmaf((float)((u >> (8 * e)) & 0xFFu), xv[4 * d + e], acc);
        }
    } else {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const float h0 = (float)__builtin_bit_cast(_Float16, (uint16_t)(wd[d] & 0xFFFFu));
            const float h1 = (float)__builtin_bit_cast(_Float16, (uint16_t)(wd[d] >> 16));
            acc = fmaf(h0, xv[2 * d], acc);
            acc = fmaf(h1, xv[2 * d + 1], acc);
        }
    }
    return acc;
}

// Transposed butterfly over the 64 lanes of a wave.  On entry every lane holds
// V partial values; on exit lane L holds the full wave sum of value
// L >> (6 - log2 V) (and so do the 64/V - 1 lanes that follow it).
template <int V>
struct WaveReduce {
    static __device__ inline float run(const float *v, int lane, int mask)
    {
        constexpr int H = V / 2;
        const bool upper = (lane & mask) != 0;
        float keep[H];
#pragma unroll
        for (int i = 0; i < H; ++i) {
            const float send = upper ? v[i] : v[i + H];
            const float mine = upper ? v[i + H] : v[i];
            keep[i] = mine + __shfl_xor(send, mask, 64);
        }
        return WaveReduce<H>::run(keep, lane, mask >> 1);
    }
};
template <>
struct WaveReduce<1> {
    static __device__ inline float run(const float *v, int, int mask)
    {
        float s = v[0];
        for (int m = mask; m >= 1; m >>= 1) s += __shfl_xor(s, m, 64);
        return s;
    }
};

constexpr int ilog2(int v) { return v <= 1 ? 0 : 1 + ilog2(v / 2); }
constexpr int pow2_ceil(int v) { return v <= 1 ? 1 : 2 * pow2_ceil((v + 1) / 2); }

template <int WT, int NT, int KS, int CPL, int U>
__global__ __launch_bounds__(kThreads) void gemv_kernel(const GemvArgs a)
{
    constexpr int WPC = Fmt<WT>::wpc;
    constexpr int G = 4 / KS;                 // wave groups per workgroup
    constexpr int VL = 64 * KS;               // lanes per wave group
    constexpr int V = pow2_ceil(U * NT);      // values per lane to reduce
    static_assert(V <= 64, "too many partial sums per lane");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int grp = wave / KS;
    const int ks = wave % KS;
    const int v = ks * 64 + lane;

    // ---- activations for this lane's chunks, and the folded code offset ----
    float xr[NT][CPL][WPC];
    float xb[NT][CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int64_t c = v + (int64_t)j * VL;
        const bool ok = c < a.nchunk;
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            float s = 0.0f;
            const bool tok = ok && n < a.N;
            const float *xn = a.x + (uint64_t)n * a.x_pitch;
#pragma unroll
            for (int i = 0; i < WPC; ++i) {
                const int64_t k = chunk_k<WT>(c, i);
                const float val = (tok && k < a.K) ? xn[k] : 0.0f;
                xr[n][j][i] = val;
                s += val;
            }
            xb[n][j] = -Fmt<WT>::offset * s;
        }
    }

    __shared__ float red[2][4][64];

    // ---- row loop: every wave of the workgroup runs the same trip count ----
    const int64_t iters = (a.n_groups + (int64_t)G * gridDim.x - 1) / ((int64_t)G * gridDim.x);
    int64_t g = (int64_t)blockIdx.x * G + grp;
    const int64_t gstep = (int64_t)gridDim.x * G;

    uint4 q[U][CPL];
    uint16_t sc[U][CPL];
    auto load_group = [&](int64_t grp_idx) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            int64_t r = grp_idx * U + u;
            r = r < a.M ? r : a.M - 1;          // tail rows re-read the last row
            const uint8_t *row = a.w + (uint64_t)r * a.pitch;
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                const int64_t c = v + (int64_t)j * VL;
                if (c < a.nchunk) {
                    q[u][j] = *reinterpret_cast<const uint4 *>(row + a.qoff + c * 16);
                    if (WT != W_F16) {
                        sc[u][j] = *reinterpret_cast<const uint16_t *>(row + 2 * chunk_block<WT>(c));
                    } else if (c * 8 + 8 > a.K) {
                        // F16 row tail: the 16-byte chunk runs past K; zero the
                        // halves beyond the row (they may hold anything).
                        const int valid = (int)(a.K - c * 8);
                        uint32_t *wd = reinterpret_cast<uint32_t *>(&q[u][j]);
#pragma unroll
                        for (int h = 0; h < 8; ++h)
                            if (h >= valid) wd[h / 2] &= (h & 1) ? 0x0000FFFFu : 0xFFFF0000u;
                    }
                } else {
                    q[u][j] = make_uint4(0, 0, 0, 0);
                    sc[u][j] = 0;
                }
            }
        }
    };

    if (iters > 0) load_group(g < a.n_groups ? g : a.n_groups - 1);
    for (int64_t it = 0; it < iters; ++it, g += gstep) {
        uint4 qc[U][CPL];
        uint16_t scc[U][CPL];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int j = 0; j < CPL; ++j) { qc[u][j] = q[u][j]; scc[u][j] = sc[u][j]; }
        if (it + 1 < iters) {
            const int64_t gn = g + gstep;
            load_group(gn < a.n_groups ? gn : a.n_groups - 1);
        }

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
                    const float s = chunk_dot<WT>(qc[u][j], xr[n][j], xb[n][j]);
                    part[u * NT + n] = fmaf(d, s, part[u * NT + n]);
                }
            }
        }
        const float tot = WaveReduce<V>::run(part, lane, 32);
        const int idx = lane >> (6 - ilog2(V));
        const bool owner = (lane & ((64 / V) - 1)) == 0;
        const bool in_range = g < a.n_groups;

        if (KS == 1) {
            if (owner && idx < U * NT && in_range) {
                const int u = idx / NT, n = idx % NT;
                const int64_t r = g * U + u;
                if (r < a.M && n < a.N) a.y[(uint64_t)n * a.y_pitch + r] = tot;
            }
        } else {
            float *buf = red[it & 1][wave];
            if (owner) buf[idx] = tot;
            __syncthreads();
            if (ks == 0 && lane < U * NT && in_range) {
                float s = 0.0f;
#pragma unroll
                for (int w2 = 0; w2 < KS; ++w2) s += red[it & 1][grp * KS + w2][lane];
                const int u = lane / NT, n = lane % NT;
                const int64_t r = g * U + u;
                if (r < a.M && n < a.N) a.y[(uint64_t)n * a.y_pitch + r] = s;
            }
        }
    }
}

// ---- dispatch -------------------------------------------------------------

using Kernel = void (*)(const GemvArgs);

template <int WT, int NT, int KS, int CPL>
constexpr bool fits()
{
    return CPL * Fmt<WT>::wpc * NT <= 128;
}

template <int WT, int NT, int KS, int CPL>
Kernel pick_u(int u)
{
    if constexpr (!fits<WT, NT, KS, CPL>()) {
        return nullptr;
    } else {
        // Several rows per wave group only while a lane holds few chunks;
        // otherwise the in-flight code registers would spill.
        constexpr int UW = (CPL > 2) ? 1 : (NT <= 1) ? 4 : (NT == 2 ? 2 : 1);
        if (u == 1) return gemv_kernel<WT, NT, KS, CPL, 1>;
        if (u == UW) return gemv_kernel<WT, NT, KS, CPL, UW>;
        return nullptr;
    }
}

template <int WT, int NT, int KS>
Kernel pick_cpl(int cpl, int u)
{
    switch (cpl) {
    case 1: return pick_u<WT, NT, KS, 1>(u);
    case 2: return pick_u<WT, NT, KS, 2>(u);
    case 4: return pick_u<WT, NT, KS, 4>(u);
    case 8: return pick_u<WT, NT, KS, 8>(u);
    default: return nullptr;
    }
}

template <int WT, int NT>
Kernel pick_ks(int ks, int cpl, int u)
{
    switch (ks) {
    case 1: return pick_cpl<WT, NT, 1>(cpl, u);
    case 2: return pick_cpl<WT, NT, 2>(cpl, u);
    case 4: return pick_cpl<WT, NT, 4>(cpl, u);
    default: return nullptr;
    }
}

template <int WT>
Kernel pick_nt(int nt, int ks, int cpl, int u)
{
    switch (nt) {
    case 1: return pick_ks<WT, 1>(ks, cpl, u);
    case 2: return pick_ks<WT, 2>(ks, cpl, u);
    case 4: return pick_ks<WT, 4>(ks, cpl, u);
    case 8: return pick_ks<WT, 8>(ks, cpl, u);
    default: return nullptr;
    }
}

Kernel pick(int wt, const GemvConfig &c)
{
    switch (wt) {
    case W_Q4_0: return pick_nt<W_Q4_0>(c.nt, c.ks, c.cpl, c.u);
    case W_Q8_0: return pick_nt<W_Q8_0>(c.nt, c.ks, c.cpl, c.u);
    case W_F16:  return pick_nt<W_F16>(c.nt, c.ks, c.cpl, c.u);
    default: return nullptr;
    }
}

int weights_per_chunk(int type) { return type == W_Q4_0 ? 32 : type == W_Q8_0 ? 16 : 8; }

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
    // Short matrices stream one row per wave group so that more waves run.
    const int u_wide = c.nt <= 1 ? 4 : (c.nt == 2 ? 2 : 1);
    c.u = (M < 4096) ? 1 : u_wide;
    c.cpl = 0;
    // Smallest wave group whose activation slice fits in registers ...
    c.ks = 0;
    for (int ks : {1, 2, 4}) {
        const int cp = round_cpl((nchunk + 64 * ks - 1) / (64 * ks));
        if (cp == 0 || cp * wpc * c.nt > 128) continue;
        c.ks = ks;
        c.cpl = cp;
        break;
    }
    if (c.ks == 0) return false;
    // ... widened while the rows alone cannot fill 256 CUs with 8 waves each,
    // as long as at least half of the added lanes get a chunk.
    while (c.ks < 4) {
        const int64_t waves = ((M + c.u - 1) / c.u) * c.ks;
        const int nks = c.ks * 2;
        const int64_t need = (nchunk + 64 * nks - 1) / (64 * nks);
        if (waves >= 2048 || need * 64 * nks > 2 * nchunk) break;
        const int cp = round_cpl(need);
        if (cp == 0 || cp * wpc * c.nt > 128) break;
        c.ks = nks;
        c.cpl = cp;
    }
    if (c.cpl > 2) c.u = 1;
    if (!pick(type, c)) return false;
    *cfg = c;
    return true;
}

hipError_t launch_gemv(const WeightView &w, const ActView &x, const OutView &y,
                       hipStream_t stream)
{
    if (w.M == 0 || x.N == 0) return hipSuccess;
    GemvConfig c;
    if (!gemv_config(w.type, w.K, w.M, x.N, &c)) return hipErrorInvalidValue;
    Kernel k = pick(w.type, c);

    GemvArgs a;
    a.w = w.base;
    a.pitch = w.pitch;
    a.M = w.M;
    a.K = w.K;
    a.qoff = (w.type == W_F16) ? 0 : quant_offset(w.K);
    a.nchunk = chunks_per_row(w.type, w.K);
    a.x = static_cast<const float *>(x.data);
    a.x_pitch = x.pitch_elems;
    a.N = (int32_t)x.N;
    a.y = y.data;
    a.y_pitch = y.pitch_elems;
    a.n_groups = (w.M + c.u - 1) / c.u;
    const int groups_per_wg = 4 / c.ks;
    int64_t wgs = (a.n_groups + groups_per_wg - 1) / groups_per_wg;
    if (wgs > 2048) wgs = 2048;
    hipLaunchKernelGGL(k, dim3((unsigned)wgs), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace qmm
