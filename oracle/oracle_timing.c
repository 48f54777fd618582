/* oracle_timing.c -- wall-clock timing of the oracle's MUL_MAT, for the CPU
 * baseline that the GPU figures are reported beside.
 *
 * TEST INFRASTRUCTURE ONLY (like the rest of oracle/): only the tests,
 * smoke() and the benchmark's CPU leg call it.  It times the oracle as it
 * stands: orc_mul_mat_rows (plain scalar C, binary64 accumulation), with the
 * output rows split statically into `threads` contiguous ranges, one POSIX
 * thread per range (rows are independent, so nothing else is shared).  It
 * adds no arithmetic of its own. */
#define _GNU_SOURCE
#include "qmm_oracle.h"

#include <pthread.h>
#include <stdlib.h>
#include <time.h>
#include <unistd.h>

typedef struct {
    int type;
    const uint8_t *w;
    size_t pitch;
    int64_t K, M;
    const void *x;
    int x_type;
    int64_t N;
    int64_t m0, m1;
    double *y, *a;
    int rc;
} job_t;

static void *run_job(void *p)
{
    job_t *j = (job_t *)p;
    j->rc = orc_mul_mat_rows(j->type, j->w, j->pitch, j->K, j->M, j->x, j->x_type, j->N, 0,
                             j->m0, j->m1, j->y, j->a);
    return NULL;
}

static double now_s(void)
{
    struct timespec t;
    clock_gettime(CLOCK_MONOTONIC, &t);
    return (double)t.tv_sec + 1e-9 * (double)t.tv_nsec;
}

static int cmp_double(const void *a, const void *b)
{
    const double x = *(const double *)a, y = *(const double *)b;
    return (x > y) - (x < y);
}

int orc_online_cpus(void)
{
    const long n = sysconf(_SC_NPROCESSORS_ONLN);
    return n > 0 ? (int)n : 1;
}

double orc_time_mul_mat(int type, const uint8_t *w, size_t pitch, int64_t K, int64_t M,
                        const void *x, int x_type, int64_t N, int threads, int reps,
                        double *y, double *a)
{
    if (threads < 1 || reps < 1 || reps > 64 || M < 0) return -1.0;
    if (threads > M && M > 0) threads = (int)M;
    job_t *jobs = (job_t *)calloc((size_t)threads, sizeof(job_t));
    pthread_t *tid = (pthread_t *)calloc((size_t)threads, sizeof(pthread_t));
    double times[64];
    if (!jobs || !tid) {
        free(jobs);
        free(tid);
        return -1.0;
    }
    int bad = 0;
    for (int r = 0; r < reps && !bad; ++r) {
        const double t0 = now_s();
        for (int t = 0; t < threads; ++t) {
            job_t *j = &jobs[t];
            j->type = type;
            j->w = w;
            j->pitch = pitch;
            j->K = K;
            j->M = M;
            j->x = x;
            j->x_type = x_type;
            j->N = N;
            j->m0 = M * t / threads;
            j->m1 = M * (t + 1) / threads;
            j->y = y;
            j->a = a;
            j->rc = 0;
            if (threads == 1) run_job(j);
            else if (pthread_create(&tid[t], NULL, run_job, j) != 0) bad = 1;
        }
        if (threads > 1)
            for (int t = 0; t < threads; ++t) pthread_join(tid[t], NULL);
        times[r] = now_s() - t0;
        for (int t = 0; t < threads; ++t) bad |= jobs[t].rc != 0;
    }
    free(jobs);
    free(tid);
    if (bad) return -1.0;
    qsort(times, (size_t)reps, sizeof(double), cmp_double);
    return times[reps / 2];
}
