/*
 * Exhaustive check of the oracle's rANS step pair over every coder state.
 *
 * For each x in [lo, hi) (inside [2^16, 2^32)): y = D(x) with the oracle's
 * decode step for the symbol owning slot x mod 4096. Then the oracle's encode
 * step must give x back:
 *   - if y >= 2^16 (no renormalisation word in decode), encoding y emits no word;
 *   - if y < 2^16 (decode reads a word w), encoding y * 2^16 + w must emit
 *     exactly w, for w in {0, 1, 0x8000, 0xFFFF, low half of x}.
 * Also y >= 16 * f (the closed-form bound that makes one word enough).
 * The step functions are the oracle's own, looked up with dlsym; this file
 * only enumerates states and compares.
 */
#include <dlfcn.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>

typedef int (*enc_fn)(uint32_t *, uint32_t, uint32_t, uint16_t *);
typedef int (*dec_fn)(uint32_t *, uint32_t, uint32_t);

typedef struct {
    enc_fn enc;
    dec_fn dec;
    const uint16_t *freq;
    uint32_t cum[257];
    uint8_t owner[4096];
    uint64_t lo, hi, fails;
} job_t;

static void *run(void *arg) {
    job_t *j = arg;
    uint64_t fails = 0;
    for (uint64_t xx = j->lo; xx < j->hi; xx++) {
        uint32_t x = (uint32_t)xx;
        uint8_t s = j->owner[x & 4095u];
        uint32_t f = j->freq[s], c = j->cum[s];
        uint32_t y = x;
        int need = j->dec(&y, f, c);
        if ((uint64_t)y < 16ull * f) fails++;
        if (!need) {
            uint32_t z = y;
            uint16_t w = 0;
            int e = j->enc(&z, f, c, &w);
            if (e || z != x) fails++;
        } else {
            uint16_t ws[5] = {0, 1, 0x8000, 0xFFFF, (uint16_t)(x * 2654435761u >> 16)};
            for (int k = 0; k < 5; k++) {
                uint32_t z = (y << 16) | ws[k];
                uint16_t w = 0;
                int e = j->enc(&z, f, c, &w);
                if (!e || w != ws[k] || z != x) fails++;
            }
        }
    }
    j->fails = fails;
    return NULL;
}

/* Returns the number of failing states, or UINT64_MAX on a setup error. */
uint64_t bijection_failures(const char *oracle_path, const uint16_t freq[256], uint64_t lo,
                            uint64_t hi, int nthreads) {
    void *h = dlopen(oracle_path, RTLD_NOW | RTLD_LOCAL);
    if (!h) return UINT64_MAX;
    enc_fn enc = (enc_fn)dlsym(h, "or_encode_step");
    dec_fn dec = (dec_fn)dlsym(h, "or_decode_step");
    if (!enc || !dec) return UINT64_MAX;
    if (nthreads < 1) nthreads = 1;
    job_t *jobs = calloc((size_t)nthreads, sizeof(job_t));
    pthread_t *tid = calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !tid) return UINT64_MAX;
    uint32_t cum[257];
    cum[0] = 0;
    for (int s = 0; s < 256; s++) cum[s + 1] = cum[s] + freq[s];
    if (cum[256] != 4096) return UINT64_MAX;
    for (int t = 0; t < nthreads; t++) {
        jobs[t].enc = enc;
        jobs[t].dec = dec;
        jobs[t].freq = freq;
        for (int s = 0; s < 257; s++) jobs[t].cum[s] = cum[s];
        for (int s = 0; s < 256; s++)
            for (uint32_t k = cum[s]; k < cum[s + 1]; k++) jobs[t].owner[k] = (uint8_t)s;
        jobs[t].lo = lo + (hi - lo) * t / nthreads;
        jobs[t].hi = lo + (hi - lo) * (t + 1) / nthreads;
    }
    for (int t = 1; t < nthreads; t++) pthread_create(&tid[t], NULL, run, &jobs[t]);
    run(&jobs[0]);
    uint64_t fails = jobs[0].fails;
    for (int t = 1; t < nthreads; t++) {
        pthread_join(tid[t], NULL);
        fails += jobs[t].fails;
    }
    free(jobs);
    free(tid);
    return fails;
}
