// gemv_mfma.hip -- decode GEMV / skinny GEMM for Q4_0 and Q8_0 weights on the
// bf16 matrix cores.
//
// Same operation as gemv.hip (y[n][m] = sum_k W'[m][k] x[n][k], 1 <= N <= 8,
// fp32 activations), with the per-weight work moved from the vector ALUs to
// v_mfma_f32_16x16x32_bf16 (16 x 16 output, K = 32 per instruction).  The
// weights are streamed once from HBM as in the VALU kernel; what changes is
// the cost of turning codes into products (Development Guide for Small AI
// Models (TinyLLaMA, etc.) Using C++, §6.2: unpack, scale, multiply-add):
//
//  * B operand (32 x 16): column j = weight row m0 + j; the four 8-element
//    k-groups of a lane hold codes of four different 32-blocks (a "quad" of
//    blocks b0..b0+3).  Codes enter as exact biased bf16 integers: a Q4_0
//    nibble n placed in the low mantissa bits of 0x4300 reads as 128 + n
//    (one shift + one and-or per two codes); a Q8_0 byte with its sign bit
//    flipped reads as code + 128 after an exact byte -> float -> bf16 widening.
//  * A operand (16 x 32): channels i = 4 g + 2 n + h carry, for block b0 + g
//    and token n of a token pair, the bf16 high part (h = 0) or the bf16 low
//    part (h = 1) of the activations, and zero in the k-groups of the other
//    blocks.  x = hi + lo holds x to 2^-17 relative, so the products keep the
//    fp32 GEMV's accuracy.  These fragments are built once per workgroup in LDS.
//  * After the four MFMAs of a quad, lane (j, g) holds the hi and lo sums of
//    block b0 + g for its row and the pair's two tokens; it applies the block
//    scale and removes the code bias there (A Complete Guide to llama.cpp and
//    Customization with C++, §2.2: the scale factors out of each block's dot
//    product): y += d * (D_hi + D_lo - bias * sum_x(block)).
//
// Per 512 weights this costs 7 (Q4_0) or 13 (Q8_0) VALU instructions per
// lane-group plus a quarter of the scale work, against 16 and 18 for the VALU
// kernel, and it does not grow with the number of tokens.
#include "qmm_internal.h"

#include <mutex>

namespace qmm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kMaxWorkgroups = 1024;
constexpr int kRing = 8;          // quads of weight loads in flight per wave

struct MItem {
    const uint8_t *w;
    uint64_t pitch;
    int64_t M;
    const float *x;
    uint64_t x_pitch;
    float *y;
    uint64_t y_pitch;
    int64_t n_tiles;      // 16-row tiles
    int32_t wg_count;     // workgroups of this item (grid x; grid y indexes the item)
    int32_t pad;
};

struct MArgs {
    MItem item[QMM_GEMV_BATCH_MAX];
    int32_t n_items;
    int32_t N;            // real tokens (<= 2 * NP)
    int64_t K;
    int64_t qoff;
    int64_t nblk;         // 32-blocks per row
    int64_t nquad;        // quads of blocks per row
};

template <int WT> struct MFmt;
template <> struct MFmt<W_Q4_0> { static constexpr int block_bytes = 16; static constexpr float bias = 136.0f; };
template <> struct MFmt<W_Q8_0> { static constexpr int block_bytes = 32; static constexpr float bias = 128.0f; };

__device__ inline uint32_t and_or(uint32_t a, uint32_t m, uint32_t c)
{
    uint32_t d;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "s"(m), "v"(c));
    return d;
}

__device__ inline uint16_t bf16_bits(float f)
{
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ inline float bf16_value(uint16_t b)
{
    return __builtin_bit_cast(float, (uint32_t)b << 16);
}

// Position, inside the 8-element k-group of slot t, of element e (0..31) of a
// block, matching the order decode_slot() produces.
//  Q4_0: slot t covers code bytes 4t..4t+3; byte s holds element 4t+s (low
//        nibble) and 16+4t+s (high nibble); the decoded order is
//        lo(s0) lo(s2) hi(s0) hi(s2) lo(s1) lo(s3) hi(s1) hi(s3).
//  Q8_0: slot t covers code bytes 8t..8t+7 in order.
template <int WT>
__device__ inline void slot_of(int e, int &t, int &pos)
{
    if (WT == W_Q4_0) {
        const int hi = e >= 16;
        const int j = hi ? e - 16 : e;
        const int s = j & 3;
        t = j >> 2;
        const int lo_pos[4] = {0, 4, 1, 5};
        const int hi_pos[4] = {2, 6, 3, 7};
        pos = hi ? hi_pos[s] : lo_pos[s];
    } else {
        t = e >> 3;
        pos = e & 7;
    }
}

// The eight biased codes of slot t of a block as bf16.
template <int WT>
__device__ inline bf16x8 decode_slot(const uint4 *q, int t, uint32_t magic)
{
    uint32_t r[4];
    if (WT == W_Q4_0) {
        const uint32_t wd[4] = {q[0].x, q[0].y, q[0].z, q[0].w};
        const uint32_t w = wd[t];
        const uint32_t m = 0x000F000Fu;
        r[0] = and_or(w, m, magic);
        r[1] = and_or(w >> 4, m, magic);
        r[2] = and_or(w >> 8, m, magic);
        r[3] = and_or(w >> 12, m, magic);
    } else {
        const uint32_t wd[8] = {q[0].x, q[0].y, q[0].z, q[0].w, q[1].x, q[1].y, q[1].z, q[1].w};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t u = wd[2 * t + h] ^ 0x80808080u;   // code + 128 per byte
            r[2 * h] = (uint32_t)bf16_bits((float)(u & 0xFFu)) |
                       ((uint32_t)bf16_bits((float)((u >> 8) & 0xFFu)) << 16);
            r[2 * h + 1] = (uint32_t)bf16_bits((float)((u >> 16) & 0xFFu)) |
                           ((uint32_t)bf16_bits((float)(u >> 24)) << 16);
        }
    }
    const uint4 v = make_uint4(r[0], r[1], r[2], r[3]);
    return __builtin_bit_cast(bf16x8, v);
}

// All-reduce over lanes j, j+16, j+32, j+48 (lane bits 4 and 5).
__device__ inline float sum_over_groups(float v)
{
    v += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v),
                                                               0x1F | (0x10 << 10)));
    v += __shfl_xor(v, 32, 64);
    return v;
}

template <int WT, int NP, int KS>
__global__ __launch_bounds__(kThreads) void gemv_mfma_kernel(const MArgs a)
{
    constexpr int BB = MFmt<WT>::block_bytes;
    constexpr int QV = BB / 16;            // uint4 per block of codes
    constexpr int G = 4 / KS;              // tile groups per workgroup
    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
    __shared__ float red[2][4][16][2 * NP];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int grp = wave / KS;
    const int ks = wave % KS;
    const int j = lane & 15;               // row within the tile / A channel
    const int g = lane >> 4;               // block within the quad / k-group

    // The item is grid y, so its descriptor is read in the first round trip
    // to the kernel arguments; a short item's surplus workgroups exit.
    const int item = blockIdx.y;
    if ((int)blockIdx.x >= a.item[item].wg_count) return;
    const uint8_t *const W = a.item[item].w;
    const uint64_t pitch = a.item[item].pitch;
    const int64_t M = a.item[item].M;
    const float *const X = a.item[item].x;
    const uint64_t x_pitch = a.item[item].x_pitch;
    float *const Y = a.item[item].y;
    const uint64_t y_pitch = a.item[item].y_pitch;
    const int64_t n_tiles = a.item[item].n_tiles;
    const int64_t wg = blockIdx.x;
    const int64_t n_wg = a.item[item].wg_count;

    // LDS: A fragments [quad][t][pair][channel][8] bf16, a 16-byte zero
    // block, then the per-(block, token) sums of hi + lo.
    const int64_t a_elems = a.nquad * 4 * NP * 16 * 8;
    uint16_t *const zero16 = lds + a_elems;
    float *const sx = reinterpret_cast<float *>(lds + a_elems + 8);

    // This wave's steps: (tile, quad) pairs, tiles strided over the
    // workgroups, quads strided over the KS waves of a tile group.  Every wave
    // of the workgroup walks tiles_iter tiles (the KS > 1 reduction uses
    // workgroup barriers); tiles past n_tiles load nothing and store nothing.
    const int32_t first_tile = (int32_t)(wg * G + grp);
    const int32_t tile_stride = (int32_t)(n_wg * G);
    const int32_t tiles_iter = (int32_t)((n_tiles + tile_stride - 1) / tile_stride);
    const int32_t quads_mine = (int32_t)((a.nquad - ks + KS - 1) / KS);   // >= 1 (host keeps KS <= nquad)

    uint4 ring[kRing][QV];
    uint16_t ring_sc[kRing];
    int32_t lt = 0, lq = 0;                 // load cursor: tile index, quad index
    auto load_next = [&](int slot) {
        const int32_t tile = first_tile + lt * tile_stride;
        bool done = false;
        if (lt < tiles_iter && tile < n_tiles) {
            int64_t row = (int64_t)tile * 16 + j;
            row = row < M ? row : M - 1;
            const int64_t b = (int64_t)(ks + lq * KS) * 4 + g;
            if (b < a.nblk) {
                const uint8_t *rp = W + (uint64_t)row * pitch;
#pragma unroll
                for (int v = 0; v < QV; ++v)
                    ring[slot][v] = *reinterpret_cast<const uint4 *>(rp + a.qoff + b * BB + 16 * v);
                ring_sc[slot] = *reinterpret_cast<const uint16_t *>(rp + 2 * b);
                done = true;
            }
        }
        if (!done) {
#pragma unroll
            for (int v = 0; v < QV; ++v) ring[slot][v] = make_uint4(0, 0, 0, 0);
            ring_sc[slot] = 0;
        }
        if (++lq == quads_mine) { lq = 0; ++lt; }
    };

#pragma unroll
    for (int i = 0; i < kRing; ++i) load_next(i);

    // ---- build the A fragments and block sums (once per workgroup) ----
    if (tid < 4) reinterpret_cast<uint32_t *>(zero16)[tid] = 0;
    {
        // channels of the blocks past the row's end in the last quad
        const int64_t q_last = a.nquad - 1;
        for (int64_t e = tid; e < (int64_t)4 * NP * 16 * 8; e += kThreads)
            lds[q_last * 4 * NP * 16 * 8 + e] = 0;
    }
    __syncthreads();
    // One task = 4 consecutive activations of one token: coalesced loads,
    // hi/lo split, scatter into the fragment slots; the 8 tasks of a block sit
    // in 8 consecutive lanes and sum their hi + lo with three lane exchanges.
    for (int64_t task0 = 0; task0 < a.nblk * 8 * 2 * NP; task0 += kThreads) {
        const int64_t task = task0 + tid;
        const bool in = task < a.nblk * 8 * 2 * NP;
        const int n = (int)(task / (a.nblk * 8));
        const int64_t r = task - (int64_t)n * a.nblk * 8;
        const int64_t b = r >> 3;
        const int e0 = (int)(r & 7) * 4;
        float s = 0.0f;
        if (in) {
            const bool real = n < a.N;
            const float *xb = X + (uint64_t)(real ? n : 0) * x_pitch + b * 32 + e0;
            const int64_t qd = b >> 2;
            const int gb = (int)(b & 3);
            const int p = n >> 1;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float xv = real ? xb[e] : 0.0f;
                const uint16_t hb = bf16_bits(xv);
                const float hv = bf16_value(hb);
                const uint16_t lb = bf16_bits(xv - hv);
                s += hv + bf16_value(lb);
                int t, pos;
                slot_of<WT>(e0 + e, t, pos);
                const int64_t base = (((qd * 4 + t) * NP + p) * 16 + 4 * gb + 2 * (n & 1)) * 8 + pos;
                lds[base] = hb;
                lds[base + 8] = lb;
            }
        }
        // lanes 8k .. 8k+7 hold one block (kThreads and 8 divide 64)
        s += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, s), 0xB1, 0xF, 0xF, true));
        s += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, s), 0x4E, 0xF, 0xF, true));
        s += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, s), 0x1F | (4 << 10)));
        if (in && e0 == 0) sx[b * 2 * NP + n] = s;
    }
    __syncthreads();

    const bool a_live = (j >> 2) == g;     // this lane's channel belongs to its k-group
    const uint32_t magic = 0x43004300u;    // bf16 128.0 in both halves
    f32x4 acc[NP];
    float yp[NP][2];
#pragma unroll
    for (int p = 0; p < NP; ++p) { yp[p][0] = 0.0f; yp[p][1] = 0.0f; }

    const int32_t total = tiles_iter * quads_mine;
    int32_t ct = 0, cq = 0;                 // compute cursor
    for (int32_t s0 = 0; s0 < total; s0 += kRing) {
#pragma unroll
        for (int i = 0; i < kRing; ++i) {
            if (s0 + i >= total) break;
            const int64_t b = (int64_t)(ks + cq * KS) * 4 + g;
            const int64_t qd = ks + cq * KS;
            // ---- four MFMAs per token pair over the quad ----
#pragma unroll
            for (int p = 0; p < NP; ++p) acc[p] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const bf16x8 bw = decode_slot<WT>(ring[i], t, magic);
#pragma unroll
                for (int p = 0; p < NP; ++p) {
                    const uint16_t *src = a_live ? lds + (((qd * 4 + t) * NP + p) * 16 + j) * 8 : zero16;
                    const bf16x8 ax = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(src));
                    acc[p] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ax, bw, acc[p], 0, 0, 0);
                }
            }
            // ---- block scale and code bias (lane (j, g) owns block b) ----
            const float d = (float)__builtin_bit_cast(_Float16, ring_sc[i]);
            if (b < a.nblk) {
#pragma unroll
                for (int p = 0; p < NP; ++p) {
                    const float2 sxp = *reinterpret_cast<const float2 *>(&sx[b * 2 * NP + 2 * p]);
                    yp[p][0] = fmaf(d, fmaf(-MFmt<WT>::bias, sxp.x, acc[p][0] + acc[p][1]), yp[p][0]);
                    yp[p][1] = fmaf(d, fmaf(-MFmt<WT>::bias, sxp.y, acc[p][2] + acc[p][3]), yp[p][1]);
                }
            }
            load_next(i);
            // ---- end of a tile: reduce over the quads' lanes and waves ----
            if (++cq == quads_mine) {
                const int32_t tile = first_tile + ct * tile_stride;
#pragma unroll
                for (int p = 0; p < NP; ++p) {
                    yp[p][0] = sum_over_groups(yp[p][0]);
                    yp[p][1] = sum_over_groups(yp[p][1]);
                }
                const int64_t m = (int64_t)tile * 16 + j;
                const bool store = tile < n_tiles && m < M;
                if (KS == 1) {
                    if (g == 0 && store) {
#pragma unroll
                        for (int p = 0; p < NP; ++p)
#pragma unroll
                            for (int h = 0; h < 2; ++h)
                                if (2 * p + h < a.N) Y[(uint64_t)(2 * p + h) * y_pitch + m] = yp[p][h];
                    }
                } else {
                    const int rb = ct & 1;
                    if (g == 0) {
#pragma unroll
                        for (int p = 0; p < NP; ++p) {
                            red[rb][wave][j][2 * p] = yp[p][0];
                            red[rb][wave][j][2 * p + 1] = yp[p][1];
                        }
                    }
                    __syncthreads();
                    if (ks == 0 && g == 0 && store) {
#pragma unroll
                        for (int n = 0; n < 2 * NP; ++n) {
                            float v = 0.0f;
#pragma unroll
                            for (int w2 = 0; w2 < KS; ++w2) v += red[rb][grp * KS + w2][j][n];
                            if (n < a.N) Y[(uint64_t)n * y_pitch + m] = v;
                        }
                    }
                }
#pragma unroll
                for (int p = 0; p < NP; ++p) { yp[p][0] = 0.0f; yp[p][1] = 0.0f; }
                cq = 0;
                ++ct;
            }
        }
    }
}

using MKernel = void (*)(const MArgs);

template <int WT, int NP>
MKernel pick_ks(int ks)
{
    switch (ks) {
    case 1: return gemv_mfma_kernel<WT, NP, 1>;
    case 2: return gemv_mfma_kernel<WT, NP, 2>;
    case 4: return gemv_mfma_kernel<WT, NP, 4>;
    default: return nullptr;
    }
}

template <int WT>
MKernel pick_np(int np, int ks)
{
    switch (np) {
    case 1: return pick_ks<WT, 1>(ks);
    case 2: return pick_ks<WT, 2>(ks);
    case 4: return pick_ks<WT, 4>(ks);
    default: return nullptr;
    }
}

MKernel pick_mfma(int type, int np, int ks)
{
    if (type == W_Q4_0) return pick_np<W_Q4_0>(np, ks);
    if (type == W_Q8_0) return pick_np<W_Q8_0>(np, ks);
    return nullptr;
}

size_t mfma_lds_bytes(int64_t K, int np)
{
    const int64_t nblk = K / 32, nquad = (nblk + 3) / 4;
    return (size_t)(nquad * 4 * np * 16 * 8) * 2 + 16 + (size_t)(nblk * 2 * np) * 4;
}

int dynamic_lds_limit()
{
    static int limit = -1;
    if (limit < 0) {
        int dev = 0, v = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
            v = 65536;
        limit = v - (int)(sizeof(float) * 2 * 4 * 16 * 8);   // minus the static reduction buffer
    }
    return limit;
}

// Raise a kernel's dynamic-LDS limit once (the attribute persists for the
// process); later launches, including those recorded into graphs, reuse it.

}  // namespace

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

bool gemv_mfma_supported(int type, int64_t K, int64_t N)
{
    if (type != W_Q4_0 && type != W_Q8_0) return false;
    if (K < 32 || N < 1) return false;
    const int np = N <= 2 ? 1 : N <= 4 ? 2 : 4;
    return (int64_t)mfma_lds_bytes(K, np) <= dynamic_lds_limit();
}

hipError_t launch_gemv_mfma(const GemvTask *tasks, int count, hipStream_t stream)
{
    const int type = tasks[0].w.type;
    const int64_t K = tasks[0].w.K;
    const int64_t N = tasks[0].x.N;
    int64_t tiles_total = 0;
    for (int i = 0; i < count; ++i) tiles_total += (tasks[i].w.M + 15) / 16;
    if (tiles_total == 0 || N == 0) return hipSuccess;
    for (int64_t n0 = 0; n0 < N;) {
        int64_t nb = N - n0 < 8 ? N - n0 : 8;
        int np = nb <= 2 ? 1 : nb <= 4 ? 2 : 4;
        while ((int64_t)mfma_lds_bytes(K, np) > dynamic_lds_limit()) {
            if (np == 1) return hipErrorInvalidValue;
            np /= 2;
            nb = 2 * np;
        }
        // Split the quads of a tile over more waves only while the tiles
        // alone leave CUs short of waves (the LM head's 2000 tiles run 1.4x
        // faster with one wave per tile than with two, measured).
        int ks = tiles_total >= 1024 ? 1 : tiles_total >= 512 ? 2 : 4;
        const int64_t nquad = (K / 32 + 3) / 4;
        while (ks > 1 && ks > nquad) ks /= 2;
        const int groups_per_wg = 4 / ks;
        const MKernel k = pick_mfma(type, np, ks);
        if (!k) return hipErrorInvalidValue;
        MArgs a;
        a.n_items = 0;
        a.N = (int32_t)nb;
        a.K = K;
        a.qoff = quant_offset(K);
        a.nblk = K / 32;
        a.nquad = (a.nblk + 3) / 4;
        int64_t need[QMM_GEMV_BATCH_MAX], need_total = 0;
        for (int i = 0; i < count; ++i) {
            const int64_t t = (tasks[i].w.M + 15) / 16;
            need[i] = (t + groups_per_wg - 1) / groups_per_wg;
            need_total += need[i];
        }
        int32_t wg_max = 0;
        for (int i = 0; i < count; ++i) {
            if (tasks[i].w.M == 0) continue;
            int64_t wgs = need[i];
            if (need_total > kMaxWorkgroups) {
                wgs = need[i] * kMaxWorkgroups / need_total;
                if (wgs < 1) wgs = 1;
            }
            MItem &it = a.item[a.n_items++];
            it.w = tasks[i].w.base;
            it.pitch = tasks[i].w.pitch;
            it.M = tasks[i].w.M;
            it.x = static_cast<const float *>(tasks[i].x.data) + (uint64_t)n0 * tasks[i].x.pitch_elems;
            it.x_pitch = tasks[i].x.pitch_elems;
            it.y = tasks[i].y.data + (uint64_t)n0 * tasks[i].y.pitch_elems;
            it.y_pitch = tasks[i].y.pitch_elems;
            it.n_tiles = (tasks[i].w.M + 15) / 16;
            it.wg_count = (int32_t)wgs;
            it.pad = 0;
            if (wgs > wg_max) wg_max = (int32_t)wgs;
        }
        const size_t lds = mfma_lds_bytes(K, np);
        if (lds > 65536 - sizeof(float) * 2 * 4 * 16 * 8) {
            const hipError_t e = allow_dynamic_lds(reinterpret_cast<const void *>(k), (int)lds);
            if (e != hipSuccess) return e;
        }
        hipLaunchKernelGGL(k, dim3((unsigned)wg_max, (unsigned)a.n_items), dim3(kThreads), lds, stream, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        n0 += nb;
    }
    return hipSuccess;
}

}  // namespace qmm
