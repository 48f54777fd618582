// host_stubs.cpp -- stand-ins for the kernel launchers of libqmm, so that the
// C-ABI entry points (qmm_api.cpp: argument validation, overlap checks,
// dispatch) can be built for the host alone under AddressSanitizer and
// UndefinedBehaviorSanitizer and driven with fake device addresses.  A stub
// never touches memory: it counts the call and reports success, which is
// what the validation layer sees when a launch is enqueued.
#include "../../quantized_matmul_ggml_amd/csrc/qmm_internal.h"

int g_launches = 0;

extern "C" hipError_t hipGetDevice(int *d)
{
    if (d) *d = 0;
    return hipErrorNoDevice;
}
extern "C" hipError_t hipDeviceGetAttribute(int *v, hipDeviceAttribute_t, int)
{
    if (v) *v = 0;
    return hipErrorNoDevice;
}

namespace qmm {

static hipError_t launched()
{
    ++g_launches;
    return hipSuccess;
}

bool gemv_config(int type, int64_t K, int64_t M, int64_t N, GemvConfig *cfg)
{
    if (type != W_Q4_0 && type != W_Q8_0 && type != W_F16) return false;
    if (N < 1 || N > 8 || K < 0 || M < 0) return false;
    cfg->nt = 1;
    cfg->ks = 1;
    cfg->cpl = 1;
    cfg->u = 1;
    cfg->wgw = 4;
    return true;
}
int record_size(int type) { return type == W_Q4_0 ? 18 : type == W_Q8_0 ? 34 : 0; }
bool gemm_supported(const WeightView &w, const ActView &x)
{
    return 128ull * w.pitch < (1ull << 31) && 128ull * x.pitch_elems * 2 < (1ull << 31);
}
GemmPlan gemm_plan(int64_t M, int64_t K, int64_t N, uint64_t ws_bytes)
{
    GemmPlan p;
    p.splits = 1;
    p.split_steps = (int)((K + 63) / 64);
    p.mp = (M + 3) / 4 * 4;
    p.ws_bytes = 0;
    const uint64_t two = 2ull * (uint64_t)N * (uint64_t)p.mp * 4u;
    if (M > 0 && N > 0 && K >= 1024 && ws_bytes >= two) {
        p.splits = 2;
        p.ws_bytes = two;
    }
    return p;
}
bool gemv_i8_supported(int, int64_t, int64_t, int64_t) { return true; }
bool gemv_i8_swiglu_supported(int, int64_t, int64_t, int64_t) { return true; }
hipError_t static_scratch(void **ptr)
{
    static unsigned char fake[16];
    *ptr = fake;
    return hipSuccess;
}

hipError_t launch_quantize(const float *, uint64_t, int64_t, int64_t, uint8_t *, uint64_t, int, hipStream_t, bool,
                           int) { return launched(); }
hipError_t launch_dequantize(const uint8_t *, uint64_t, int64_t, int64_t, int, float *, uint64_t, hipStream_t,
                             int) { return launched(); }
hipError_t launch_gemv(const WeightView &, const ActView &, const OutView &, hipStream_t) { return launched(); }
hipError_t launch_gemv_batch(const GemvTask *, int, hipStream_t) { return launched(); }
hipError_t launch_gemv_i8(const WeightView &, const WeightView &, const OutView &, int64_t, hipStream_t)
{
    return launched();
}
hipError_t launch_gemv_i8_batch(const WeightView *, const WeightView *, const OutView *, int, int64_t, hipStream_t)
{
    return launched();
}
hipError_t launch_gemv_i8_swiglu(const WeightView &, const WeightView &, const WeightView &, const OutView &, int64_t,
                                 hipStream_t) { return launched(); }
hipError_t launch_gemv_swiglu(const WeightView &, const WeightView &, const ActView &, const OutView &, hipStream_t)
{
    return launched();
}
hipError_t launch_records(const WeightView &, uint8_t *, bool, hipStream_t) { return launched(); }
hipError_t launch_gemm(const WeightView &, const ActView &, const OutView &, float *, uint64_t, hipStream_t)
{
    return launched();
}
hipError_t launch_gemm_batch(const WeightView *, const ActView *, const OutView *, int, hipStream_t)
{
    return launched();
}
hipError_t launch_gemm_swiglu(const WeightView &, const WeightView &, const ActView &, const OutView &, hipStream_t)
{
    return launched();
}
hipError_t launch_stream_read(const void *, uint64_t, uint32_t *, int, hipStream_t) { return launched(); }
hipError_t launch_clock_probe(uint64_t *, int, int, int, hipStream_t) { return launched(); }

}  // namespace qmm
