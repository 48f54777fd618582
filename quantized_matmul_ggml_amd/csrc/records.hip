// records.hip -- GGUF-style block records <-> the library's packed rows.
//
// A quantized tensor in a GGUF file is an aligned array of block records
// (Development Guide for Small AI Models (TinyLLaMA, etc.) Using C++, §3.2:
// tensor data after the tensor info, aligned; §6.1: a block is one FP16
// scale (2 bytes) followed by 32 4-bit values (16 bytes)).  Here a record is
// the block's fp16 scale (little endian) followed by its codes, 16 bytes for
// Q4_0 (byte j = nib_j | nib_{j+16} << 4, as in the packed rows) or 32 int8
// bytes for Q8_0; records run back to back, row-major.  The packed rows put
// a row's scales first and its codes after, each part 16-byte aligned.
//
// Both directions move the same bytes, so they are HBM-bound copies with a
// reshuffle.  A workgroup owns 256 consecutive records: the record side is
// one contiguous span (16-byte aligned, since 256 records are 4608 or 8704
// bytes), moved with 16-byte loads or stores through LDS; the row side is
// one thread per block (a 2-byte scale and 16 or 32 code bytes, the code
// bytes 16-byte aligned).
#include "qmm_internal.h"

namespace qmm {
namespace {

constexpr int kRecThreads = 256;      // records per workgroup

template <int WT> struct Rec;
template <> struct Rec<W_Q4_0> { static constexpr int bytes = 18, code_vecs = 1; };
template <> struct Rec<W_Q8_0> { static constexpr int bytes = 34, code_vecs = 2; };

struct RecArgs {
    uint8_t *records;      // device, 16-byte aligned
    uint8_t *rows;         // device, rows at rows + m * pitch
    uint64_t pitch;
    int32_t K;
    int32_t M;
    int32_t nblk;          // K / 32
    int32_t qoff;          // byte offset of the codes inside a row
    int32_t total;         // M * nblk records
};

// A 16-byte store that streams past the L2 (non-temporal), for the records
// that rows_to_records_kernel writes in whole contiguous spans (2 % faster
// on the box; the scattered 16-byte row stores of the other direction were
// 3 % slower this way and stay ordinary stores).
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
__device__ inline void store16_nt(void *p, uint4 v)
{
    __builtin_nontemporal_store(u32x4v{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4v *>(p));
}

// Records [r0, r0 + n) of the span (n <= 256) staged in LDS: 16-byte pieces
// while whole, 2-byte pieces for the tail that ends the tensor.
template <int WT>
__device__ inline void span_io(uint8_t *lds, uint8_t *rec, int n, bool load)
{
    constexpr int RB = Rec<WT>::bytes;
    const int bytes = n * RB;               // even
    const int vec = bytes / 16;
    for (int i = threadIdx.x; i < vec; i += kRecThreads) {
        if (load)
            *reinterpret_cast<uint4 *>(lds + 16 * i) = *reinterpret_cast<const uint4 *>(rec + 16 * i);
        else
            store16_nt(rec + 16 * i, *reinterpret_cast<const uint4 *>(lds + 16 * i));
    }
    for (int i = 16 * vec / 2 + threadIdx.x; i < bytes / 2; i += kRecThreads) {
        if (load)
            reinterpret_cast<uint16_t *>(lds)[i] = reinterpret_cast<const uint16_t *>(rec)[i];
        else
            reinterpret_cast<uint16_t *>(rec)[i] = reinterpret_cast<const uint16_t *>(lds)[i];
    }
}

// Zero the bytes of a row that belong to no block: the gap between the
// scales and the codes (the codes end exactly at the row size; bytes past it
// up to the pitch are not the tensor's and stay untouched, as qmm_quantize
// leaves them).
__device__ inline void zero_row_gap(uint8_t *row, int nblk, int qoff)
{
    for (int i = 2 * nblk; i < qoff; ++i) row[i] = 0;
}

template <int WT>
__global__ __launch_bounds__(kRecThreads) void records_to_rows_kernel(const RecArgs a)
{
    constexpr int RB = Rec<WT>::bytes;
    constexpr int CB = RB - 2;              // code bytes of a block
    __shared__ __attribute__((aligned(16))) uint8_t lds[kRecThreads * RB];
    const int r0 = blockIdx.x * kRecThreads;
    const int n = a.total - r0 < kRecThreads ? a.total - r0 : kRecThreads;
    span_io<WT>(lds, a.records + (uint64_t)r0 * RB, n, true);
    __syncthreads();
    const int t = threadIdx.x;
    if (t >= n) return;
    const int i = r0 + t;
    const int m = i / a.nblk;
    const int b = i - m * a.nblk;
    uint8_t *row = a.rows + (uint64_t)m * a.pitch;
    const uint16_t *src = reinterpret_cast<const uint16_t *>(lds + t * RB);   // 2-byte aligned
    *reinterpret_cast<uint16_t *>(row + 2 * b) = src[0];
    uint32_t w[CB / 4];
#pragma unroll
    for (int j = 0; j < CB / 4; ++j) w[j] = (uint32_t)src[1 + 2 * j] | ((uint32_t)src[2 + 2 * j] << 16);
    uint4 *dst = reinterpret_cast<uint4 *>(row + a.qoff + CB * b);
#pragma unroll
    for (int v = 0; v < Rec<WT>::code_vecs; ++v)
        dst[v] = make_uint4(w[4 * v], w[4 * v + 1], w[4 * v + 2], w[4 * v + 3]);
    if (b == 0) zero_row_gap(row, a.nblk, a.qoff);
}

template <int WT>
__global__ __launch_bounds__(kRecThreads) void rows_to_records_kernel(const RecArgs a)
{
    constexpr int RB = Rec<WT>::bytes;
    constexpr int CB = RB - 2;
    __shared__ __attribute__((aligned(16))) uint8_t lds[kRecThreads * RB];
    const int r0 = blockIdx.x * kRecThreads;
    const int n = a.total - r0 < kRecThreads ? a.total - r0 : kRecThreads;
    const int t = threadIdx.x;
    if (t < n) {
        const int i = r0 + t;
        const int m = i / a.nblk;
        const int b = i - m * a.nblk;
        const uint8_t *row = a.rows + (uint64_t)m * a.pitch;
        uint16_t *dst = reinterpret_cast<uint16_t *>(lds + t * RB);
        dst[0] = *reinterpret_cast<const uint16_t *>(row + 2 * b);
        const uint4 *src = reinterpret_cast<const uint4 *>(row + a.qoff + CB * b);
#pragma unroll
        for (int v = 0; v < Rec<WT>::code_vecs; ++v) {
            const uint4 q = src[v];
            const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                dst[1 + 8 * v + 2 * j] = (uint16_t)(w[j] & 0xFFFFu);
                dst[2 + 8 * v + 2 * j] = (uint16_t)(w[j] >> 16);
            }
        }
    }
    __syncthreads();
    span_io<WT>(lds, a.records + (uint64_t)r0 * RB, n, false);
}

template <int WT>
hipError_t launch_records(const RecArgs &a, bool to_rows, hipStream_t stream)
{
    const unsigned grid = (unsigned)((a.total + kRecThreads - 1) / kRecThreads);
    if (to_rows)
        hipLaunchKernelGGL(records_to_rows_kernel<WT>, dim3(grid), dim3(kRecThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(rows_to_records_kernel<WT>, dim3(grid), dim3(kRecThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

int record_size(int type) { return type == W_Q4_0 ? 18 : type == W_Q8_0 ? 34 : 0; }

hipError_t launch_records(const WeightView &w, uint8_t *records, bool to_rows, hipStream_t stream)
{
    if (w.M == 0) return hipSuccess;
    RecArgs a;
    a.records = records;
    a.rows = const_cast<uint8_t *>(w.base);
    a.pitch = w.pitch;
    a.K = (int32_t)w.K;
    a.M = (int32_t)w.M;
    a.nblk = (int32_t)(w.K / 32);
    a.qoff = (int32_t)quant_offset(w.K);
    a.total = (int32_t)(w.M * (w.K / 32));
    if (w.type == W_Q4_0) return launch_records<W_Q4_0>(a, to_rows, stream);
    if (w.type == W_Q8_0) return launch_records<W_Q8_0>(a, to_rows, stream);
    return hipErrorInvalidValue;
}

}  // namespace qmm
