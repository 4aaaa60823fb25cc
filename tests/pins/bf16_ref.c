/* Exhaustive check of an fp32 -> bf16 rounding function against an independent
 * reference: pick the nearer of the two bf16 neighbours by exact long-double
 * distance, ties to the even pattern, overflow past the largest finite value
 * (by at least half a unit in the last place) to infinity.  Test helper only. */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

typedef uint16_t (*rnd_fn)(float);

static long double bfval(uint16_t b) {
    int e = (b >> 7) & 0xFF, m = b & 0x7F;
    long double v = (e == 0) ? ldexpl((long double)m, -133) : ldexpl((long double)(128 + m), e - 134);
    return (b & 0x8000) ? -v : v;
}

static uint16_t reference(uint32_t u) {
    float f;
    memcpy(&f, &u, 4);
    uint16_t lo = (uint16_t)(u >> 16);
    if ((u & 0xFFFFu) == 0) return lo;
    if ((u & 0x7F800000u) == 0x7F800000u) return lo; /* inf exactly handled above; NaN checked separately */
    uint16_t hi = (uint16_t)(lo + 1);
    long double x = (long double)f, dl = fabsl(x - bfval(lo)), dh = fabsl(bfval(hi) - x);
    if (dl < dh) return lo;
    if (dh < dl) return hi;
    return (lo & 1) ? hi : lo;
}

typedef struct { rnd_fn f; uint64_t b, e, bad; uint32_t first; } job;

static void* run(void* p) {
    job* j = (job*)p;
    for (uint64_t i = j->b; i < j->e; ++i) {
        uint32_t u = (uint32_t)i;
        float x;
        memcpy(&x, &u, 4);
        uint16_t got = j->f(x);
        if (x != x) {
            if (((got & 0x7F80) != 0x7F80) || !(got & 0x7F) || ((got ^ (u >> 16)) & 0x8000)) { if (!j->bad++) j->first = u; }
            continue;
        }
        if (got != reference(u)) { if (!j->bad++) j->first = u; }
    }
    return 0;
}

/* Returns the number of mismatching patterns in [begin, end); *first gets the first one. */
uint64_t check_range(rnd_fn f, uint64_t begin, uint64_t end, int nthreads, uint32_t* first) {
    pthread_t th[64];
    job jobs[64];
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 64) nthreads = 64;
    uint64_t per = (end - begin + nthreads - 1) / nthreads, bad = 0;
    *first = 0;
    for (int t = 0; t < nthreads; ++t) {
        jobs[t].f = f; jobs[t].b = begin + per * t; jobs[t].e = jobs[t].b + per; jobs[t].bad = 0; jobs[t].first = 0;
        if (jobs[t].b > end) jobs[t].b = end;
        if (jobs[t].e > end) jobs[t].e = end;
        pthread_create(&th[t], 0, run, &jobs[t]);
    }
    for (int t = 0; t < nthreads; ++t) {
        pthread_join(th[t], 0);
        if (jobs[t].bad && !bad) *first = jobs[t].first;
        bad += jobs[t].bad;
    }
    return bad;
}
