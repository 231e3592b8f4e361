/*
 * sampler.c -- seeded, counter-based random inputs for the tests and the
 * benchmark. Holds none of the decode method's arithmetic: it only draws
 * bytes from a categorical distribution the caller tabulates, and uniform
 * 53-bit doubles.
 *
 * Generator: the i-th output (i = 0, 1, ...) of SplitMix64 seeded with `key`
 * (Steele, Lea and Flood, "Fast splittable pseudorandom number generators",
 * OOPSLA 2014; the 64-bit finaliser constants as published with the
 * reference SplitMix64 generator): z = key + (i + 1) * 0x9E3779B97F4A7C15,
 * then z ^= z >> 30, z *= 0xBF58476D1CE4E5B9, z ^= z >> 27,
 * z *= 0x94D049BB133111EB, z ^= z >> 31. Being a function of (key, i), any
 * index can be regenerated on its own, and a stream can be filled by many
 * threads in any split with identical results.
 */
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>

static inline uint64_t sm64(uint64_t key, uint64_t i) {
    uint64_t z = key + (i + 1) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

uint64_t synth_u64(uint64_t key, uint64_t i) { return sm64(key, i); }

/* out[i] = 64-bit outputs for indices start .. start+n-1 */
void synth_fill_u64(uint64_t key, uint64_t start, uint64_t n, uint64_t *out) {
    for (uint64_t i = 0; i < n; i++) out[i] = sm64(key, start + i);
}

typedef struct {
    uint64_t key, start, lo, hi;
    const uint8_t *cat_sym;
    const uint64_t *cat_thr;
    int ncat;
    uint8_t *out;
} cat_job;

/* Category of u: the first c with u < thr[c]; the last category takes the rest.
 * Categories are listed most probable first, so the scan is short. */
static void *cat_run(void *arg) {
    cat_job *jb = arg;
    const uint64_t *thr = jb->cat_thr;
    const uint8_t *sym = jb->cat_sym;
    int last = jb->ncat - 1;
    for (uint64_t i = jb->lo; i < jb->hi; i++) {
        uint64_t u = sm64(jb->key, jb->start + i);
        int c = 0;
        while (c < last && u >= thr[c]) c++;
        jb->out[i] = sym[c];
    }
    return NULL;
}

/* Draw n bytes for stream indices start .. start+n-1 with nthreads threads. */
int synth_categorical(uint64_t key, uint64_t start, uint64_t n, const uint8_t *cat_sym,
                      const uint64_t *cat_thr, int ncat, uint8_t *out, int nthreads) {
    if (ncat < 1) return -1;
    if (nthreads < 1) nthreads = 1;
    if ((uint64_t)nthreads > n) nthreads = n ? (int)n : 1;
    cat_job *jobs = calloc((size_t)nthreads, sizeof(cat_job));
    pthread_t *tid = calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !tid) {
        free(jobs);
        free(tid);
        return -1;
    }
    for (int t = 0; t < nthreads; t++)
        jobs[t] = (cat_job){key, start, n * t / nthreads, n * (t + 1) / nthreads,
                            cat_sym, cat_thr, ncat, out};
    for (int t = 1; t < nthreads; t++) pthread_create(&tid[t], NULL, cat_run, &jobs[t]);
    cat_run(&jobs[0]);
    for (int t = 1; t < nthreads; t++) pthread_join(tid[t], NULL);
    free(jobs);
    free(tid);
    return 0;
}
