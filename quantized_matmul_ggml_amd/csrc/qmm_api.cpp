// qmm_api.cpp -- the C entry points of libqmm: descriptor validation and
// kernel dispatch.  Everything here runs on the host and touches no device
// memory; a call either enqueues its kernels on the caller's stream and
// returns QMM_OK, or returns a negative qmm_status with nothing enqueued.
//
// Descriptor convention: No Python! Building an AI Inference Engine
// Exclusively in C++, §4 (ne = elements per dimension, nb = byte strides,
// ne[0] contiguous).  Operand roles of MUL_MAT: same page, §5 (the result
// takes ne = {a.ne[0], b.ne[1]} with b "transposed") read together with the
// stride definition: W ne = [K, M], x ne = [K, N], y ne = [M, N].
#include "../../include/qmm.h"
#include "qmm_internal.h"

namespace {

using qmm::W_BF16;
using qmm::W_F16;
using qmm::W_F32;
using qmm::W_Q4_0;
using qmm::W_Q8_0;

bool is_quant(int t)
{
    return t == QMM_TYPE_Q8_0 || t == QMM_TYPE_Q4_0 || t == QMM_TYPE_Q8_B64 || t == QMM_TYPE_Q4_B64;
}
bool is_b64(int t) { return t == QMM_TYPE_Q8_B64 || t == QMM_TYPE_Q4_B64; }
// Weights per fp16 scale of a quantized type.
int64_t block_len(int t) { return is_b64(t) ? 64 : 32; }

int64_t elem_size(int t)
{
    switch (t) {
    case QMM_TYPE_F32: return 4;
    case QMM_TYPE_F16: return 2;
    case QMM_TYPE_BF16: return 2;
    default: return 0;
    }
}

// Largest element count per dimension and byte span of one tensor the
// library accepts (far beyond any device memory, and small enough that
// every size computed from them fits 64 bits).
constexpr int64_t kMaxElems = (int64_t)1 << 48;
constexpr uint64_t kMaxSpan = 1ull << 62;

// Shape / layout rules shared by every operand.  `align` is the byte
// alignment required of data and nb[1].
int check_tensor(const qmm_tensor *t, uint64_t align)
{
    if (!t) return QMM_ERR_NULL;
    if (t->type < QMM_TYPE_F32 || t->type > QMM_TYPE_Q4_B64) return QMM_ERR_TYPE;
    if (t->n_dims < 1 || t->n_dims > 4) return QMM_ERR_UNSUPPORTED;
    if (t->n_dims > 2 || t->ne[2] != 1 || t->ne[3] != 1) return QMM_ERR_UNSUPPORTED;
    if (t->ne[0] < 0 || t->ne[1] < 0) return QMM_ERR_SHAPE;
    if (t->ne[0] > kMaxElems || t->ne[1] > kMaxElems) return QMM_ERR_UNSUPPORTED;
    if (t->n_dims == 1 && t->ne[1] != 1) return QMM_ERR_SHAPE;
    if (is_quant(t->type)) {
        if (t->ne[0] % block_len(t->type) != 0) return QMM_ERR_SHAPE;
        if (t->nb[0] != 0) return QMM_ERR_LAYOUT;
    } else if ((int64_t)t->nb[0] != elem_size(t->type)) {
        return QMM_ERR_LAYOUT;
    }
    const uint64_t rs = qmm_row_size(t->type, t->ne[0]);
    if (t->ne[1] > 1 && t->nb[1] < rs) return QMM_ERR_LAYOUT;
    if (t->ne[1] > 1 && t->nb[1] % align != 0) return QMM_ERR_LAYOUT;
    // the bytes the tensor spans must be a range of the address space
    uint64_t span = rs;
    if (t->ne[1] > 1) {
        uint64_t rows;
        if (__builtin_mul_overflow((uint64_t)(t->ne[1] - 1), t->nb[1], &rows) || rows > kMaxSpan)
            return QMM_ERR_UNSUPPORTED;
        span = rows + rs;
    }
    if (span > kMaxSpan || (uintptr_t)t->data > UINTPTR_MAX - span) return QMM_ERR_UNSUPPORTED;
    const bool empty = t->ne[0] == 0 || t->ne[1] == 0;
    if (!t->data && !empty) return QMM_ERR_NULL;
    if ((uintptr_t)t->data % align != 0) return QMM_ERR_LAYOUT;
    return QMM_OK;
}

// Byte range [lo, hi) a 2-D tensor touches.
void extent(const qmm_tensor *t, uintptr_t *lo, uintptr_t *hi)
{
    const uint64_t rs = qmm_row_size(t->type, t->ne[0]);
    *lo = (uintptr_t)t->data;
    *hi = *lo + (t->ne[1] > 0 ? (uint64_t)(t->ne[1] - 1) * t->nb[1] + rs : 0);
}

bool overlaps(const qmm_tensor *a, const qmm_tensor *b)
{
    uintptr_t alo, ahi, blo, bhi;
    extent(a, &alo, &ahi);
    extent(b, &blo, &bhi);
    if (alo == ahi || blo == bhi) return false;
    return alo < bhi && blo < ahi;
}

qmm::WeightView weight_view(const qmm_tensor *w)
{
    qmm::WeightView v;
    v.base = static_cast<const uint8_t *>(w->data);
    v.pitch = w->ne[1] > 1 ? w->nb[1] : qmm_row_size(w->type, w->ne[0]);
    v.K = w->ne[0];
    v.M = w->ne[1];
    // the 64-block types are their code format with one scale per two runs
    v.type = w->type == QMM_TYPE_Q8_B64 ? W_Q8_0 : w->type == QMM_TYPE_Q4_B64 ? W_Q4_0 : w->type;
    v.scale_shift = is_b64(w->type) ? 1 : 0;
    return v;
}

uint64_t pitch_elems(const qmm_tensor *t)
{
    const int64_t es = elem_size(t->type);
    return t->ne[1] > 1 ? t->nb[1] / (uint64_t)es : (uint64_t)t->ne[0];
}

int status_of(hipError_t e) { return e == hipSuccess ? QMM_OK : QMM_ERR_DEVICE; }

// Common checks of MUL_MAT operands.
int check_mul_mat(const qmm_tensor *w, const qmm_tensor *x, const qmm_tensor *y,
                  int x_type, uint64_t x_align)
{
    if (!w || !x || !y) return QMM_ERR_NULL;
    int rc = check_tensor(w, 16);
    if (rc) return rc;
    rc = check_tensor(x, x_align);
    if (rc) return rc;
    rc = check_tensor(y, 4);
    if (rc) return rc;
    if (x->type != x_type || y->type != QMM_TYPE_F32) return QMM_ERR_TYPE;
    if (x->ne[0] != w->ne[0]) return QMM_ERR_SHAPE;
    if (y->ne[0] != w->ne[1] || y->ne[1] != x->ne[1]) return QMM_ERR_SHAPE;
    if (overlaps(y, w) || overlaps(y, x)) return QMM_ERR_ALIAS;
    return QMM_OK;
}

}  // namespace

extern "C" {

size_t qmm_row_size(int32_t type, int64_t ne0)
{
    if (ne0 < 0 || ne0 > kMaxElems) return 0;
    const uint64_t k = (uint64_t)ne0;
    auto a16 = [](uint64_t v) { return (v + 15) / 16 * 16; };
    switch (type) {
    case QMM_TYPE_F32: return k * 4;
    case QMM_TYPE_F16: return k * 2;
    case QMM_TYPE_BF16: return k * 2;
    case QMM_TYPE_Q8_0: return (k % 32) ? 0 : a16(k / 16) + a16(k);
    case QMM_TYPE_Q4_0: return (k % 32) ? 0 : a16(k / 16) + a16(k / 2);
    case QMM_TYPE_Q8_B64: return (k % 64) ? 0 : a16(k / 32) + a16(k);
    case QMM_TYPE_Q4_B64: return (k % 64) ? 0 : a16(k / 32) + a16(k / 2);
    default: return 0;
    }
}

int qmm_quantize(const qmm_tensor *src, qmm_tensor *dst, void *stream)
{
    return qmm_quantize_rule(src, dst, QMM_QUANT_DEFAULT, stream);
}

int qmm_quantize_rule(const qmm_tensor *src, qmm_tensor *dst, int32_t rule, void *stream)
{
    if (rule != QMM_QUANT_DEFAULT && rule != QMM_QUANT_Q4_AMAX7) return QMM_ERR_UNSUPPORTED;
    if (!src || !dst) return QMM_ERR_NULL;
    int rc = check_tensor(src, 4);
    if (rc) return rc;
    rc = check_tensor(dst, 16);
    if (rc) return rc;
    if (src->type != QMM_TYPE_F32 || !is_quant(dst->type)) return QMM_ERR_TYPE;
    if (src->ne[0] != dst->ne[0] || src->ne[1] != dst->ne[1]) return QMM_ERR_SHAPE;
    if (src->ne[0] % block_len(dst->type) != 0) return QMM_ERR_SHAPE;
    if (overlaps(dst, src)) return QMM_ERR_ALIAS;
    if (rule == QMM_QUANT_Q4_AMAX7 && dst->type != QMM_TYPE_Q4_0 && dst->type != QMM_TYPE_Q4_B64)
        return QMM_ERR_TYPE;
    const qmm::WeightView d = weight_view(dst);
    return status_of(qmm::launch_quantize(static_cast<const float *>(src->data), pitch_elems(src),
                                          src->ne[0], src->ne[1],
                                          static_cast<uint8_t *>(dst->data), d.pitch, d.type,
                                          static_cast<hipStream_t>(stream),
                                          rule == QMM_QUANT_Q4_AMAX7, d.scale_shift));
}

int qmm_dequantize(const qmm_tensor *src, qmm_tensor *dst, void *stream)
{
    if (!src || !dst) return QMM_ERR_NULL;
    int rc = check_tensor(src, 16);
    if (rc) return rc;
    rc = check_tensor(dst, 4);
    if (rc) return rc;
    if (!(is_quant(src->type) || src->type == QMM_TYPE_F16) || dst->type != QMM_TYPE_F32)
        return QMM_ERR_TYPE;
    if (src->ne[0] != dst->ne[0] || src->ne[1] != dst->ne[1]) return QMM_ERR_SHAPE;
    if (overlaps(dst, src)) return QMM_ERR_ALIAS;
    const qmm::WeightView s = weight_view(src);
    return status_of(qmm::launch_dequantize(s.base, s.pitch, s.K, s.M, s.type,
                                            static_cast<float *>(dst->data), pitch_elems(dst),
                                            static_cast<hipStream_t>(stream), s.scale_shift));
}

int qmm_gemv(const qmm_tensor *w, const qmm_tensor *x, qmm_tensor *y, void *stream)
{
    if (x && x->type == QMM_TYPE_Q8_0) {
        // the integer-activation path ("A Complete Guide to llama.cpp ...", §2.2)
        int rc = check_mul_mat(w, x, y, QMM_TYPE_Q8_0, 16);
        if (rc) return rc;
        if (!is_quant(w->type)) return QMM_ERR_TYPE;
        if (x->ne[1] > 8) return QMM_ERR_SHAPE;
        if (x->ne[1] == 0 || w->ne[1] == 0) return QMM_OK;
        const qmm::WeightView wv = weight_view(w), xv = weight_view(x);
        if (!qmm::gemv_i8_supported(wv.type, w->ne[0], w->ne[1], x->ne[1])) return QMM_ERR_UNSUPPORTED;
        qmm::OutView yv{static_cast<float *>(y->data), pitch_elems(y)};
        if (wv.pitch > (1ull << 28) || xv.pitch > (1ull << 28) || wv.M >= (1ll << 31) ||
            yv.pitch_elems >= (1ull << 31))
            return QMM_ERR_UNSUPPORTED;
        return status_of(qmm::launch_gemv_i8(wv, xv, yv, x->ne[1], static_cast<hipStream_t>(stream)));
    }
    int rc = check_mul_mat(w, x, y, QMM_TYPE_F32, 4);
    if (rc) return rc;
    if (!(is_quant(w->type) || w->type == QMM_TYPE_F16)) return QMM_ERR_TYPE;
    if (x->ne[1] > 8) return QMM_ERR_SHAPE;
    if (x->ne[1] == 0 || w->ne[1] == 0) return QMM_OK;
    // The activation slice of every lane lives in registers (at most 128
    // floats per lane), which bounds K; tokens are split into chunks that fit.
    qmm::GemvConfig cfg;
    if (!qmm::gemv_config(weight_view(w).type, w->ne[0], w->ne[1], 1, &cfg)) return QMM_ERR_UNSUPPORTED;
    qmm::ActView xv{x->data, pitch_elems(x), x->ne[1]};
    qmm::OutView yv{static_cast<float *>(y->data), pitch_elems(y)};
    if (!qmm::gemv_supported(weight_view(w), xv, yv)) return QMM_ERR_UNSUPPORTED;
    return status_of(qmm::launch_gemv(weight_view(w), xv, yv, static_cast<hipStream_t>(stream)));
}

int qmm_gemv_batch(const qmm_gemv_item *items, int32_t count, void *stream)
{
    if (!items) return QMM_ERR_NULL;
    if (count < 1 || count > QMM_GEMV_BATCH_MAX) return QMM_ERR_SHAPE;
    if (!items[0].x_f32) return QMM_ERR_NULL;
    // Q8_0 activations in the first item select the integer-activation path
    // for the whole batch ("A Complete Guide to llama.cpp ...", §2.2)
    const bool i8 = items[0].x_f32->type == QMM_TYPE_Q8_0;
    qmm::GemvTask tasks[QMM_GEMV_BATCH_MAX];
    for (int i = 0; i < count; ++i) {           // every item on its own first
        const qmm_tensor *w = items[i].w, *x = items[i].x_f32, *y = items[i].y_f32;
        int rc = i8 ? check_mul_mat(w, x, y, QMM_TYPE_Q8_0, 16) : check_mul_mat(w, x, y, QMM_TYPE_F32, 4);
        if (rc) return rc;
        if (i8 ? !is_quant(w->type) : !(is_quant(w->type) || w->type == QMM_TYPE_F16)) return QMM_ERR_TYPE;
        if (x->ne[1] > 8) return QMM_ERR_SHAPE;
        if (i > 0) {
            const qmm_tensor *w0 = items[0].w, *x0 = items[0].x_f32;
            if (w->type != w0->type) return QMM_ERR_TYPE;
            if (w->ne[0] != w0->ne[0] || x->ne[1] != x0->ne[1]) return QMM_ERR_SHAPE;
        }
    }
    for (int i = 0; i < count; ++i) {           // then outputs against every operand
        const qmm_tensor *w = items[i].w, *x = items[i].x_f32, *y = items[i].y_f32;
        for (int j = 0; j < count; ++j) {
            if (j == i) continue;
            if (overlaps(y, items[j].w) || overlaps(y, items[j].x_f32) || overlaps(y, items[j].y_f32))
                return QMM_ERR_ALIAS;
        }
        tasks[i].w = weight_view(w);
        tasks[i].x = qmm::ActView{x->data, pitch_elems(x), x->ne[1]};
        tasks[i].y = qmm::OutView{static_cast<float *>(y->data), pitch_elems(y)};
        if (!i8 && !qmm::gemv_supported(tasks[i].w, tasks[i].x, tasks[i].y)) return QMM_ERR_UNSUPPORTED;
    }
    int64_t m_total = 0;
    for (int i = 0; i < count; ++i) m_total += items[i].w->ne[1];
    const int64_t N = items[0].x_f32->ne[1];
    if (m_total == 0 || N == 0) return QMM_OK;
    if (i8) {
        qmm::WeightView wv[QMM_GEMV_BATCH_MAX], xv[QMM_GEMV_BATCH_MAX];
        qmm::OutView yv[QMM_GEMV_BATCH_MAX];
        for (int i = 0; i < count; ++i) {
            wv[i] = tasks[i].w;
            xv[i] = weight_view(items[i].x_f32);
            yv[i] = tasks[i].y;
            if (wv[i].pitch > (1ull << 28) || xv[i].pitch > (1ull << 28) || wv[i].M >= (1ll << 31) ||
                yv[i].pitch_elems >= (1ull << 31))
                return QMM_ERR_UNSUPPORTED;
        }
        if (!qmm::gemv_i8_supported(wv[0].type, items[0].w->ne[0], m_total, N)) return QMM_ERR_UNSUPPORTED;
        return status_of(qmm::launch_gemv_i8_batch(wv, xv, yv, count, N, static_cast<hipStream_t>(stream)));
    }
    qmm::GemvConfig cfg;
    if (!qmm::gemv_config(tasks[0].w.type, items[0].w->ne[0], m_total, 1, &cfg))
        return QMM_ERR_UNSUPPORTED;
    return status_of(qmm::launch_gemv_batch(tasks, count, static_cast<hipStream_t>(stream)));
}

int qmm_gemv_swiglu(const qmm_tensor *w_gate, const qmm_tensor *w_up, const qmm_tensor *x,
                    qmm_tensor *h, void *stream)
{
    if (x && x->type == QMM_TYPE_Q8_0) {
        // the integer-activation path ("A Complete Guide to llama.cpp ...", §2.2)
        int rc = check_mul_mat(w_gate, x, h, QMM_TYPE_Q8_0, 16);
        if (rc) return rc;
        rc = check_mul_mat(w_up, x, h, QMM_TYPE_Q8_0, 16);
        if (rc) return rc;
        if (!is_quant(w_gate->type)) return QMM_ERR_TYPE;
        if (w_up->type != w_gate->type) return QMM_ERR_TYPE;
        if (w_up->ne[0] != w_gate->ne[0] || w_up->ne[1] != w_gate->ne[1]) return QMM_ERR_SHAPE;
        if (x->ne[1] > 8) return QMM_ERR_SHAPE;
        if (x->ne[1] == 0 || w_gate->ne[1] == 0) return QMM_OK;
        const qmm::WeightView gv = weight_view(w_gate), uv = weight_view(w_up), xv = weight_view(x);
        qmm::OutView hv{static_cast<float *>(h->data), pitch_elems(h)};
        if (!qmm::gemv_i8_swiglu_supported(gv.type, w_gate->ne[0], w_gate->ne[1], x->ne[1]))
            return QMM_ERR_UNSUPPORTED;
        if (gv.pitch > (1ull << 28) || uv.pitch > (1ull << 28) || xv.pitch > (1ull << 28) ||
            gv.M >= (1ll << 31) || hv.pitch_elems >= (1ull << 31))
            return QMM_ERR_UNSUPPORTED;
        return status_of(qmm::launch_gemv_i8_swiglu(gv, uv, xv, hv, x->ne[1], static_cast<hipStream_t>(stream)));
    }
    int rc = check_mul_mat(w_gate, x, h, QMM_TYPE_F32, 4);
    if (rc) return rc;
    rc = check_mul_mat(w_up, x, h, QMM_TYPE_F32, 4);
    if (rc) return rc;
    if (!(is_quant(w_gate->type) || w_gate->type == QMM_TYPE_F16)) return QMM_ERR_TYPE;
    if (w_up->type != w_gate->type) return QMM_ERR_TYPE;
    if (w_up->ne[0] != w_gate->ne[0] || w_up->ne[1] != w_gate->ne[1]) return QMM_ERR_SHAPE;
    if (x->ne[1] > 8) return QMM_ERR_SHAPE;
    if (x->ne[1] == 0 || w_gate->ne[1] == 0) return QMM_OK;
    qmm::GemvConfig cfg;
    if (!qmm::gemv_config(weight_view(w_gate).type, w_gate->ne[0], 2 * w_gate->ne[1], 1, &cfg))
        return QMM_ERR_UNSUPPORTED;
    qmm::ActView xv{x->data, pitch_elems(x), x->ne[1]};
    qmm::OutView hv{static_cast<float *>(h->data), pitch_elems(h)};
    const qmm::WeightView gv = weight_view(w_gate), uv = weight_view(w_up);
    if (!qmm::gemv_supported(gv, xv, hv) || !qmm::gemv_supported(uv, xv, hv)) return QMM_ERR_UNSUPPORTED;
    return status_of(qmm::launch_gemv_swiglu(gv, uv, xv, hv, static_cast<hipStream_t>(stream)));
}

size_t qmm_record_size(int32_t type)
{
    return (size_t)qmm::record_size(type);
}

namespace {

// Shared validation of the record conversions; on success *bytes is the
// size of the record array.
int check_records(const qmm_tensor *q, const void *records, uint64_t *bytes)
{
    int rc = check_tensor(q, 16);
    if (rc) return rc;
    if (q->type != QMM_TYPE_Q8_0 && q->type != QMM_TYPE_Q4_0) return QMM_ERR_TYPE;
    int64_t blocks;
    if (__builtin_mul_overflow(q->ne[1], q->ne[0] / 32, &blocks) || blocks >= (1ll << 31))
        return QMM_ERR_UNSUPPORTED;
    *bytes = (uint64_t)blocks * (uint64_t)qmm::record_size(q->type);
    if (*bytes == 0) return QMM_OK;
    if (!records) return QMM_ERR_NULL;
    if ((uintptr_t)records % 16 != 0) return QMM_ERR_LAYOUT;
    uintptr_t lo, hi;
    extent(q, &lo, &hi);
    const uintptr_t r = (uintptr_t)records;
    if (r < hi && lo < r + *bytes) return QMM_ERR_ALIAS;
    return QMM_OK;
}

}  // namespace

int qmm_records_to_rows(const void *records, qmm_tensor *dst, void *stream)
{
    uint64_t bytes = 0;
    const int rc = check_records(dst, records, &bytes);
    if (rc || bytes == 0) return rc;
    return status_of(qmm::launch_records(weight_view(dst), static_cast<uint8_t *>(const_cast<void *>(records)),
                                         true, static_cast<hipStream_t>(stream)));
}

int qmm_rows_to_records(const qmm_tensor *src, void *records, void *stream)
{
    uint64_t bytes = 0;
    const int rc = check_records(src, records, &bytes);
    if (rc || bytes == 0) return rc;
    return status_of(qmm::launch_records(weight_view(src), static_cast<uint8_t *>(records), false,
                                         static_cast<hipStream_t>(stream)));
}

namespace {

int check_gemm(const qmm_tensor *w, const qmm_tensor *x, const qmm_tensor *y)
{
    const int rc = check_mul_mat(w, x, y, QMM_TYPE_BF16, 16);
    if (rc) return rc;
    if (!(is_quant(w->type) || w->type == QMM_TYPE_F16)) return QMM_ERR_TYPE;
    // the GEMM stages F16 rows in whole 32-weight blocks
    if (w->type == QMM_TYPE_F16 && w->ne[0] % 32 != 0) return QMM_ERR_UNSUPPORTED;
    if (w->ne[1] == 0 || x->ne[1] == 0) return QMM_OK;
    qmm::ActView xv{x->data, pitch_elems(x), x->ne[1]};
    if (!qmm::gemm_supported(weight_view(w), xv)) return QMM_ERR_UNSUPPORTED;
    return QMM_OK;
}

bool range_overlaps(uintptr_t lo, uintptr_t hi, const qmm_tensor *t)
{
    uintptr_t tlo, thi;
    extent(t, &tlo, &thi);
    if (lo == hi || tlo == thi) return false;
    return lo < thi && tlo < hi;
}

}  // namespace

int qmm_gemm(const qmm_tensor *w, const qmm_tensor *x, qmm_tensor *y, void *stream)
{
    return qmm_gemm_ws(w, x, y, nullptr, 0, stream);
}

size_t qmm_gemm_workspace_size(const qmm_tensor *w, const qmm_tensor *x)
{
    // 0 for operands qmm_gemm_ws would refuse by type or shape
    if (!w || !x) return 0;
    if (check_tensor(w, 16) || check_tensor(x, 16)) return 0;
    if (!(is_quant(w->type) || w->type == QMM_TYPE_F16) || x->type != QMM_TYPE_BF16) return 0;
    if (w->ne[0] != x->ne[0]) return 0;
    return (size_t)qmm::gemm_plan(w->ne[1], w->ne[0], x->ne[1], ~0ull).ws_bytes;
}

int qmm_gemm_batch(const qmm_gemm_item *items, int32_t count, void *stream)
{
    if (!items) return QMM_ERR_NULL;
    if (count < 1 || count > QMM_GEMM_BATCH_MAX) return QMM_ERR_SHAPE;
    qmm::WeightView wv[QMM_GEMM_BATCH_MAX];
    qmm::ActView xv[QMM_GEMM_BATCH_MAX];
    qmm::OutView yv[QMM_GEMM_BATCH_MAX];
    for (int i = 0; i < count; ++i) {           // every item on its own first
        const qmm_tensor *w = items[i].w, *x = items[i].x_bf16, *y = items[i].y_f32;
        const int rc = check_gemm(w, x, y);
        if (rc) return rc;
        if (i > 0) {
            const qmm_tensor *w0 = items[0].w, *x0 = items[0].x_bf16;
            if (w->type != w0->type) return QMM_ERR_TYPE;
            if (w->ne[0] != w0->ne[0] || x->ne[1] != x0->ne[1]) return QMM_ERR_SHAPE;
        }
    }
    for (int i = 0; i < count; ++i) {           // then outputs against every operand
        const qmm_tensor *w = items[i].w, *x = items[i].x_bf16, *y = items[i].y_f32;
        for (int j = 0; j < count; ++j) {
            if (j == i) continue;
            if (overlaps(y, items[j].w) || overlaps(y, items[j].x_bf16) || overlaps(y, items[j].y_f32))
                return QMM_ERR_ALIAS;
        }
        wv[i] = weight_view(w);
        xv[i] = qmm::ActView{x->data, pitch_elems(x), x->ne[1]};
        yv[i] = qmm::OutView{static_cast<float *>(y->data), pitch_elems(y)};
    }
    return status_of(qmm::launch_gemm_batch(wv, xv, yv, count, static_cast<hipStream_t>(stream)));
}

int qmm_gemm_swiglu(const qmm_tensor *w_gate, const qmm_tensor *w_up, const qmm_tensor *x, qmm_tensor *h,
                    void *stream)
{
    int rc = check_gemm(w_gate, x, h);
    if (rc) return rc;
    rc = check_gemm(w_up, x, h);
    if (rc) return rc;
    if (w_up->type != w_gate->type) return QMM_ERR_TYPE;
    if (w_up->ne[0] != w_gate->ne[0] || w_up->ne[1] != w_gate->ne[1]) return QMM_ERR_SHAPE;
    if (w_gate->ne[1] == 0 || x->ne[1] == 0) return QMM_OK;
    qmm::ActView xv{x->data, pitch_elems(x), x->ne[1]};
    qmm::OutView hv{static_cast<float *>(h->data), pitch_elems(h)};
    return status_of(qmm::launch_gemm_swiglu(weight_view(w_gate), weight_view(w_up), xv, hv,
                                             static_cast<hipStream_t>(stream)));
}

int qmm_gemm_ws(const qmm_tensor *w, const qmm_tensor *x, qmm_tensor *y, void *workspace,
                size_t workspace_bytes, void *stream)
{
    const int rc = check_gemm(w, x, y);
    if (rc) return rc;
    if (w->ne[1] == 0 || x->ne[1] == 0) return QMM_OK;
    if (!workspace) workspace_bytes = 0;
    if (workspace_bytes) {
        if ((uintptr_t)workspace % 16 != 0) return QMM_ERR_LAYOUT;
        const uint64_t used = qmm::gemm_plan(w->ne[1], w->ne[0], x->ne[1], workspace_bytes).ws_bytes;
        const uintptr_t lo = (uintptr_t)workspace;
        if (range_overlaps(lo, lo + used, w) || range_overlaps(lo, lo + used, x) ||
            range_overlaps(lo, lo + used, y))
            return QMM_ERR_ALIAS;
    }
    qmm::ActView xv{x->data, pitch_elems(x), x->ne[1]};
    qmm::OutView yv{static_cast<float *>(y->data), pitch_elems(y)};
    return status_of(qmm::launch_gemm(weight_view(w), xv, yv, static_cast<float *>(workspace),
                                      workspace_bytes, static_cast<hipStream_t>(stream)));
}

int qmm_gemm_noalloc(const qmm_tensor *w, const qmm_tensor *x, qmm_tensor *y, size_t workspace_bytes,
                     void *stream)
{
    const int rc = check_gemm(w, x, y);
    if (rc) return rc;
    if (workspace_bytes > QMM_NOALLOC_SCRATCH_BYTES) return QMM_ERR_SCRATCH;
    if (w->ne[1] == 0 || x->ne[1] == 0) return QMM_OK;
    void *ws = nullptr;
    if (workspace_bytes && qmm::static_scratch(&ws) != hipSuccess) return QMM_ERR_DEVICE;
    qmm::ActView xv{x->data, pitch_elems(x), x->ne[1]};
    qmm::OutView yv{static_cast<float *>(y->data), pitch_elems(y)};
    return status_of(qmm::launch_gemm(weight_view(w), xv, yv, static_cast<float *>(ws), workspace_bytes,
                                      static_cast<hipStream_t>(stream)));
}

int qmm_stream_read(const void *src, size_t bytes, uint32_t *sink, int32_t workgroups, void *stream)
{
    if (!sink || (bytes > 0 && !src)) return QMM_ERR_NULL;
    if (bytes % 16 != 0 || workgroups < 1 || workgroups > 65536) return QMM_ERR_SHAPE;
    if (bytes >= (1ull << 31)) return QMM_ERR_UNSUPPORTED;
    if ((uintptr_t)src % 16 != 0) return QMM_ERR_LAYOUT;
    return status_of(qmm::launch_stream_read(src, bytes, sink, workgroups, static_cast<hipStream_t>(stream)));
}

int qmm_clock_probe(uint64_t *out, int32_t workgroups, int32_t iters, int32_t mode, void *stream)
{
    if (!out) return QMM_ERR_NULL;
    if (workgroups < 1 || workgroups > 65536 || iters < 1 || mode < 0 || mode > 4) return QMM_ERR_SHAPE;
    return status_of(qmm::launch_clock_probe(out, workgroups, iters, mode, static_cast<hipStream_t>(stream)));
}

int64_t qmm_wall_clock_khz(void)
{
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess) return QMM_ERR_DEVICE;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0)
        return QMM_ERR_DEVICE;
    return khz;
}

const char *qmm_strerror(int status)
{
    switch (status) {
    case QMM_OK: return "success";
    case QMM_ERR_NULL: return "a descriptor or data pointer is NULL";
    case QMM_ERR_TYPE: return "operand type not accepted by this entry point";
    case QMM_ERR_SHAPE: return "operand shapes do not match (or K not a multiple of the block length, or N out of range)";
    case QMM_ERR_LAYOUT: return "unsupported strides or alignment";
    case QMM_ERR_ALIAS: return "the output overlaps an input";
    case QMM_ERR_UNSUPPORTED: return "unsupported tensor rank or size";
    case QMM_ERR_DEVICE: return "the HIP runtime refused the launch";
    case QMM_ERR_SCRATCH: return "the call needs more scratch memory than the library's static array holds";
    default: return "unknown qmm status";
    }
}

}  // extern "C"
