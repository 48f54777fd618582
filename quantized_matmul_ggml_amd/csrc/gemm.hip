// gemm.hip -- prefill GEMM: the launch planning (K split, batches), the
// split-K slab sum and the launches of the register-unpacking kernel of
// gemm_rq.hip, which serves every weight type (Q4_0, Q8_0, with 32- or
// 64-weight blocks, and F16).
//
// Y[n][m] = sum_k W'[m][k] * X[n][k] for many tokens at once (No Python!
// Building an AI Inference Engine Exclusively in C++, §6: C_ij = sum_k A_ik B_kj;
// §6.1: tile the matrices and feed the multiply-add units, here the bf16
// matrix cores).  Tiles are 128 weight rows x 128 tokens, K advancing 64
// (two 32-blocks) per step.
//
// One launch serves three callers:
//  * one product, with K optionally split into ranges (a workgroup per tile
//    and range) whose partial sums go to a caller workspace and are added in
//    range order by split_sum_kernel (products with too few tiles for the
//    chip; gemm_plan decides);
//  * a batch of up to QMM_GEMM_BATCH_MAX products sharing type, K and N,
//    whose tiles form one grid (a workgroup finds its item by tile index);
//  * the gate/up pair with the SwiGLU epilogue: 64 rows of each matrix per
//    tile, combined in LDS after the last step.
#include "gemm_common.h"

#include <atomic>
#include <mutex>
#include <type_traits>

namespace qmm {
namespace {

constexpr int BM = 128;                   // weight rows per tile
constexpr int BN = 128;                   // tokens per tile
constexpr int BK = 64;                    // K per step (two 32-blocks)
constexpr int SCALE_GROUP_STEPS = 8;      // K ranges of a split are multiples of this many steps

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
    if (gemm_rq_handles(w0.type)) e = launch_gemm_rq(a, blocks, w0.type, w0.scale_shift, false, stream);
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
