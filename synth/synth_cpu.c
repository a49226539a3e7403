/*
 * synth_cpu.c -- host build of the seeded input generator (see
 * synth_core.h).  Fills whole ranges or gathers single elements by index,
 * split over a few POSIX threads.  It draws inputs only.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>

#include "synth_core.h"

/* Standard normal CDF through libm's erfc. */
static double normal_cdf(double z) { return 0.5 * erfc(-z / sqrt(2.0)); }

/* table[i] = the standard normal quantile at p = (i + 1/2) / SYN_TABLE_SIZE,
 * found by bisection on the CDF (monotone, so 200 halvings of [-40, 40]
 * reach the double nearest the root). */
void syn_table(double *table) {
    for (int i = 0; i < SYN_TABLE_SIZE; ++i) {
        double p = ((double)i + 0.5) / (double)SYN_TABLE_SIZE;
        double lo = -40.0, hi = 40.0;
        for (int it = 0; it < 200; ++it) {
            double mid = 0.5 * (lo + hi);
            if (mid == lo || mid == hi) break;
            if (normal_cdf(mid) < p) lo = mid; else hi = mid;
        }
        table[i] = 0.5 * (lo + hi);
    }
}

typedef struct {
    int kind;
    uint64_t key;
    int64_t start;      /* first element index (fill) */
    const int64_t *idx; /* element indices (gather), or NULL */
    int64_t lo, hi;     /* this worker's output range */
    double sigma;
    uint32_t thr;
    double mul;
    const double *table;
    void *out;
} job_t;

static void emit(const job_t *jb, int64_t o, uint64_t j) {
    double v = syn_value(jb->table, syn_bits(jb->key, j), jb->sigma, jb->thr, jb->mul);
    float f = (float)v;
    if (jb->kind == SYN_F32)
        ((float *)jb->out)[o] = f;
    else if (jb->kind == SYN_BF16)
        ((uint16_t *)jb->out)[o] = syn_trunc_bf16(f);
    else
        ((uint16_t *)jb->out)[o] = syn_trunc_f16(f);
}

static void *worker(void *arg) {
    const job_t *jb = (const job_t *)arg;
    if (jb->idx) {
        for (int64_t o = jb->lo; o < jb->hi; ++o) emit(jb, o, (uint64_t)jb->idx[o]);
    } else {
        for (int64_t o = jb->lo; o < jb->hi; ++o) emit(jb, o, (uint64_t)(jb->start + o));
    }
    return 0;
}

static int run(job_t base, int64_t count, int nthreads) {
    if (count <= 0) return 0;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 64) nthreads = 64;
    if ((int64_t)nthreads > count / 4096 + 1) nthreads = (int)(count / 4096 + 1);
    pthread_t th[64];
    job_t jobs[64];
    int64_t per = (count + nthreads - 1) / nthreads;
    int started = 0, rc = 0;
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = base;
        jobs[t].lo = (int64_t)t * per;
        jobs[t].hi = jobs[t].lo + per < count ? jobs[t].lo + per : count;
        if (jobs[t].lo >= jobs[t].hi) break;
        if (t == 0) continue; /* this thread runs job 0 itself */
        if (pthread_create(&th[t], 0, worker, &jobs[t]) != 0) { rc = -1; break; }
        started = t;
    }
    worker(&jobs[0]);
    for (int t = 1; t <= started; ++t) pthread_join(th[t], 0);
    return rc;
}

/* out[o] = value of element (start + o), o in [0, count) */
int syn_fill(int kind, uint64_t seed, uint64_t tag, int64_t start, int64_t count,
             double sigma, uint32_t thr, double mul, const double *table, void *out,
             int nthreads) {
    job_t b = {kind, syn_key(seed, tag), start, 0, 0, 0, sigma, thr, mul, table, out};
    return run(b, count, nthreads);
}

/* out[o] = value of element idx[o], o in [0, count) */
int syn_gather(int kind, uint64_t seed, uint64_t tag, const int64_t *idx, int64_t count,
               double sigma, uint32_t thr, double mul, const double *table, void *out,
               int nthreads) {
    job_t b = {kind, syn_key(seed, tag), 0, idx, 0, 0, sigma, thr, mul, table, out};
    return run(b, count, nthreads);
}
