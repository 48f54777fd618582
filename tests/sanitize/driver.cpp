// driver.cpp -- drives the C-ABI validation layer (qmm_api.cpp, with the
// kernel launchers stubbed out) and the CPU oracle under AddressSanitizer and
// UndefinedBehaviorSanitizer: every entry point with a deterministic stream
// of well-formed and malformed descriptors over fake device addresses (the
// host layer validates them and never dereferences them), and every oracle
// routine on small seeded inputs.  Exits 0 when every call returned, with no
// sanitizer report (reports abort the process).
#include "../../include/qmm.h"
#include "../../oracle/qmm_oracle.h"

#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <initializer_list>

extern int g_launches;

namespace {

uint64_t state = 0x9E3779B97F4A7C15ull;
uint64_t next()
{
    state ^= state << 13;
    state ^= state >> 7;
    state ^= state << 17;
    return state;
}
template <class T, size_t N> T pick(const T (&v)[N]) { return v[next() % N]; }

qmm_tensor random_tensor()
{
    static const int32_t types[] = {-1, 0, 1, 2, 3, 4, 5, 6, 7, 3, 4, 0, 2};
    static const int32_t dims[] = {0, 1, 2, 2, 2, 3, 5};
    static const int64_t ne0s[] = {-32, -1, 0, 1, 7, 31, 32, 33, 64, 96, 160, 2048, 5632, 32768, 1ll << 40,
                                   INT64_MAX};
    static const int64_t ne1s[] = {-1, 0, 1, 2, 3, 8, 9, 512, 32000, 1ll << 31, INT64_MAX};
    static const uint64_t nbs[] = {0, 1, 2, 3, 4, 16, 48, 64, 1152, 2176, 4096, 8192, 1ull << 40, UINT64_MAX};
    static const uintptr_t ptrs[] = {0, 0x100000000ull, 0x100000010ull, 0x100000001ull, 0x200000000ull,
                                     0x100000800ull, UINTPTR_MAX - 15};
    qmm_tensor t;
    memset(&t, 0, sizeof(t));
    t.type = pick(types);
    t.n_dims = pick(dims);
    t.ne[0] = pick(ne0s);
    t.ne[1] = pick(ne1s);
    t.ne[2] = (next() % 8) ? 1 : (int64_t)(next() % 3);
    t.ne[3] = (next() % 8) ? 1 : 2;
    const size_t rs = qmm_row_size(t.type, t.ne[0] > 0 ? t.ne[0] : 0);
    t.nb[0] = (next() % 2) ? (uint64_t)(t.type == 0 ? 4 : t.type == 1 || t.type == 2 ? 2 : 0) : pick(nbs);
    t.nb[1] = (next() % 2) ? (uint64_t)rs + 16 * (next() % 3) : pick(nbs);
    t.nb[2] = pick(nbs);
    t.nb[3] = pick(nbs);
    t.data = (void *)pick(ptrs);
    return t;
}

// A well-formed descriptor at a fake device address, rows nb1 apart.
qmm_tensor tensor2(int32_t type, int64_t ne0, int64_t ne1, uintptr_t addr, uint64_t pad = 0)
{
    qmm_tensor t;
    memset(&t, 0, sizeof(t));
    t.type = type;
    t.n_dims = 2;
    t.ne[0] = ne0;
    t.ne[1] = ne1;
    t.ne[2] = t.ne[3] = 1;
    t.nb[0] = type == QMM_TYPE_F32 ? 4 : (type == QMM_TYPE_F16 || type == QMM_TYPE_BF16) ? 2 : 0;
    t.nb[1] = qmm_row_size(type, ne0) + pad;
    t.nb[2] = t.nb[3] = t.nb[1] * (uint64_t)(ne1 > 0 ? ne1 : 1);
    t.data = (void *)addr;
    return t;
}

void fuzz_entry_points(int rounds)
{
    for (int r = 0; r < rounds; ++r) {
        qmm_tensor a = random_tensor(), b = random_tensor(), c = random_tensor(), d = random_tensor();
        const bool nul = next() % 16 == 0;
        qmm_quantize(nul ? nullptr : &a, &b, nullptr);
        qmm_quantize_rule(&a, &b, (int32_t)(next() % 3), nullptr);
        qmm_dequantize(&a, nul ? nullptr : &b, nullptr);
        qmm_gemv(&a, &b, &c, nullptr);
        qmm_gemv_swiglu(&a, &b, &c, &d, nullptr);
        qmm_gemm(&a, &b, &c, nullptr);
        qmm_gemm_ws(&a, &b, &c, (void *)0x300000000ull, (size_t)(next() % (64u << 20)), nullptr);
        qmm_gemm_noalloc(&a, &b, &c, (size_t)(next() % (32u << 20)), nullptr);
        qmm_gemm_workspace_size(&a, &b);
        qmm_gemm_swiglu(&a, &b, &c, &d, nullptr);
        qmm_records_to_rows((const void *)0x400000000ull, &a, nullptr);
        qmm_rows_to_records(&a, (void *)(0x400000000ull + (next() % 2) * 8), nullptr);
        qmm_gemv_item gi[QMM_GEMV_BATCH_MAX + 1];
        qmm_gemm_item mi[QMM_GEMM_BATCH_MAX + 1];
        qmm_tensor pool[3 * (QMM_GEMV_BATCH_MAX + 1)];
        const int count = (int)(next() % (QMM_GEMV_BATCH_MAX + 3)) - 1;
        for (int i = 0; i < QMM_GEMV_BATCH_MAX + 1; ++i) {
            pool[3 * i] = random_tensor();
            pool[3 * i + 1] = random_tensor();
            pool[3 * i + 2] = random_tensor();
            gi[i] = qmm_gemv_item{&pool[3 * i], &pool[3 * i + 1], (next() % 16) ? &pool[3 * i + 2] : nullptr};
            mi[i] = qmm_gemm_item{&pool[3 * i], &pool[3 * i + 1], &pool[3 * i + 2]};
        }
        qmm_gemv_batch((next() % 32) ? gi : nullptr, count, nullptr);
        qmm_gemm_batch(mi, count, nullptr);
        qmm_stream_read((const void *)pick((const uintptr_t[]){0, 0x100000000ull, 0x100000004ull}),
                        (size_t)(next() % 4096), (uint32_t *)0x500000000ull, (int32_t)(next() % 70000) - 10, nullptr);
        qmm_clock_probe((next() % 8) ? (uint64_t *)0x600000000ull : nullptr, (int32_t)(next() % 300) - 5,
                        (int32_t)(next() % 10) - 2, (int32_t)(next() % 7) - 1, nullptr);
        qmm_strerror((int)(next() % 20) - 12);
    }
}

int expect(int got, int want, const char *what)
{
    if (got != want) {
        fprintf(stderr, "%s: status %d, expected %d\n", what, got, want);
        return 1;
    }
    return 0;
}

int well_formed_calls()
{
    int bad = 0;
    const uintptr_t W = 0x100000000ull, X = 0x200000000ull, Y = 0x300000000ull, Z = 0x380000000ull;
    qmm_tensor w = tensor2(QMM_TYPE_Q4_0, 2048, 5632, W), x = tensor2(QMM_TYPE_F32, 2048, 1, X);
    qmm_tensor y = tensor2(QMM_TYPE_F32, 5632, 1, Y), f32w = tensor2(QMM_TYPE_F32, 2048, 5632, X);
    qmm_tensor xb = tensor2(QMM_TYPE_BF16, 2048, 512, X), yb = tensor2(QMM_TYPE_F32, 5632, 512, Y);
    const int before = g_launches;
    bad += expect(qmm_quantize(&f32w, &w, nullptr), QMM_OK, "quantize");
    bad += expect(qmm_dequantize(&w, &f32w, nullptr), QMM_OK, "dequantize");
    bad += expect(qmm_gemv(&w, &x, &y, nullptr), QMM_OK, "gemv");
    qmm_tensor wu = tensor2(QMM_TYPE_Q4_0, 2048, 5632, Z);
    bad += expect(qmm_gemv_swiglu(&w, &wu, &x, &y, nullptr), QMM_OK, "gemv_swiglu");
    bad += expect(qmm_gemm(&w, &xb, &yb, nullptr), QMM_OK, "gemm");
    bad += expect(qmm_gemm_noalloc(&w, &xb, &yb, 1u << 20, nullptr), QMM_OK, "gemm_noalloc");
    bad += expect(qmm_gemm_noalloc(&w, &xb, &yb, QMM_NOALLOC_SCRATCH_BYTES + 16, nullptr), QMM_ERR_SCRATCH,
                  "gemm_noalloc too big");
    bad += expect(qmm_rows_to_records(&w, (void *)0x700000000ull, nullptr), QMM_OK, "rows_to_records");
    qmm_tensor yo = tensor2(QMM_TYPE_F32, 5632, 1, W + 64);     // overlaps w
    bad += expect(qmm_gemv(&w, &x, &yo, nullptr), QMM_ERR_ALIAS, "gemv alias");
    qmm_tensor xn = tensor2(QMM_TYPE_F32, 2048, 9, X);
    bad += expect(qmm_gemv(&w, &xn, &y, nullptr), QMM_ERR_SHAPE, "gemv N=9");
    if (g_launches - before != 7) {
        fprintf(stderr, "expected 7 stub launches, saw %d\n", g_launches - before);
        ++bad;
    }
    for (int t = -2; t < 10; ++t)
        for (int64_t k : {-64ll, -1ll, 0ll, 1ll, 31ll, 32ll, 33ll, 64ll, 96ll, 2048ll, 5632ll, 1ll << 40})
            (void)qmm_row_size(t, k);
    return bad;
}

int oracle_paths()
{
    int bad = 0;
    // conversions: every binary16 / bfloat16 pattern, and a spread of binary32 ones
    for (uint32_t h = 0; h < 65536; ++h) {
        const float f = orc_f16_to_f32((uint16_t)h);
        if (f == f && orc_f32_to_f16(f) != (uint16_t)h) ++bad;
        (void)orc_bf16_to_f32((uint16_t)h);
    }
    for (uint32_t i = 0; i < 1u << 20; ++i) {
        const uint32_t u = (uint32_t)next();
        float f;
        memcpy(&f, &u, 4);
        (void)orc_f32_to_f16(f);
        (void)orc_f32_to_bf16(f);
    }
    // rows of every quantized type, odd row counts and padded pitches
    const int64_t K = 192, M = 5, N = 3;
    float *w = (float *)malloc(sizeof(float) * K * M);
    float *xf = (float *)malloc(sizeof(float) * K * N);
    for (int64_t i = 0; i < K * M; ++i) w[i] = (float)((int64_t)(next() % 2001) - 1000) * 1e-3f;
    for (int64_t i = 0; i < K * M; i += 37) w[i] = 0.0f;
    for (int64_t i = 0; i < K * N; ++i) xf[i] = (float)((int64_t)(next() % 2001) - 1000) * 1e-2f;
    uint16_t *xb = (uint16_t *)malloc(2 * K * N);
    orc_f32_to_bf16_n(xf, xb, (size_t)(K * N));
    double *y = (double *)malloc(sizeof(double) * M * N), *a = (double *)malloc(sizeof(double) * M * N);
    for (int type : {ORC_Q8_0, ORC_Q4_0, ORC_Q8_B64, ORC_Q4_B64}) {
        for (int rule : {ORC_RULE_DEFAULT, ORC_RULE_Q4_SYM7}) {
            if (rule == ORC_RULE_Q4_SYM7 && !(type == ORC_Q4_0 || type == ORC_Q4_B64)) continue;
            const size_t pitch = orc_row_size(type, K) + 32;
            uint8_t *rows = (uint8_t *)calloc(M, pitch);
            float *deq = (float *)malloc(sizeof(float) * K * M);
            bad += orc_quantize_rows_rule(type, rule, w, K, M, rows, pitch) != 0;
            bad += orc_dequantize_rows(type, rows, pitch, K, M, deq) != 0;
            bad += orc_mul_mat_rows(type, rows, pitch, K, M, xf, ORC_F32, N, 0, 0, M, y, a) != 0;
            bad += orc_mul_mat_rows(type, rows, pitch, K, M, xb, ORC_BF16, N, 1, 1, M - 1, y, a) != 0;
            const int64_t ms[3] = {0, M - 1, 2}, ns[3] = {N - 1, 0, 1};
            bad += orc_mul_mat_pairs(type, rows, pitch, K, M, xf, ORC_F32, N, 0, ms, ns, 3, y, a) != 0;
            // activations as Q8_0 rows for the integer path
            const size_t xp = orc_row_size(ORC_Q8_0, K);
            uint8_t *xq = (uint8_t *)calloc(N, xp);
            bad += orc_quantize_rows(ORC_Q8_0, xf, K, N, xq, xp) != 0;
            bad += orc_mul_mat_q8act_rows(type, rows, pitch, K, M, xq, xp, N, 0, M, y, a) != 0;
            if (orc_record_size(type)) {
                uint8_t *rec = (uint8_t *)malloc(orc_record_size(type) * (K / 32) * M);
                uint8_t *back = (uint8_t *)calloc(M, pitch);
                bad += orc_rows_to_records(type, rows, pitch, K, M, rec) != 0;
                bad += orc_records_to_rows(type, rec, K, M, back, pitch) != 0;
                for (int64_t m = 0; m < M; ++m) bad += memcmp(rows + m * pitch, back + m * pitch, orc_row_size(type, K)) != 0;
                free(rec);
                free(back);
            }
            free(xq);
            free(rows);
            free(deq);
        }
    }
    // the F16 weights and the plain definition on an F32 matrix
    const size_t p16 = orc_row_size(ORC_F16, K);
    uint16_t *w16 = (uint16_t *)malloc(p16 * M);
    orc_f32_to_f16_n(w, w16, (size_t)(K * M));
    bad += orc_mul_mat_rows(ORC_F16, (const uint8_t *)w16, p16, K, M, xf, ORC_F32, N, 0, 0, M, y, a) != 0;
    bad += orc_mul_mat_rows(ORC_F32, (const uint8_t *)w, 4 * K, K, M, xf, ORC_F32, N, 0, 0, M, y, a) != 0;
    double g[4] = {-1000.0, -1.5, 0.0, 40.0}, u[4] = {1.0, 2.0, 3.0, 4.0}, h[4];
    orc_swiglu_n(g, u, h, 4);
    bad += !(isfinite(h[0]) && isfinite(h[3]));
    // rejected arguments
    bad += orc_mul_mat_rows(ORC_Q4_0, nullptr, 0, 33, 1, xf, ORC_F32, 1, 0, 0, 1, y, a) == 0;
    bad += orc_quantize_rows(99, w, K, M, nullptr, 0) == 0;
    free(w16);
    free(w);
    free(xf);
    free(xb);
    free(y);
    free(a);
    return bad;
}

}  // namespace

int main()
{
    int bad = well_formed_calls();
    fuzz_entry_points(20000);
    bad += oracle_paths();
    printf("sanitized host layer and oracle: %d failure(s), %d stub launches\n", bad, g_launches);
    return bad ? 1 : 0;
}
